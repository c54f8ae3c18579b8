"""The C ABI on the host: the library loads, exports what include/bsa.h
declares, sizes its workspace, and rejects every bad argument before touching
the GPU (these calls return before any HIP call, so they run without one)."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_attention_39_amd as bsa
from block_sparse_attention_39_amd._lib import Desc, lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = open(os.path.join(ROOT, "include", "bsa.h")).read()

OK, NULL, SHAPE, UNSUP, ALIGN, WS, LAUNCH, ARG = 0, -1, -2, -3, -4, -5, -6, -7
FAKE = 1 << 20  # a non-NULL, 16-byte aligned address that is never dereferenced


def declared_functions():
    return sorted(set(re.findall(r"^\s*(?:bsa_status|const char \*|int)\s*\**\s*(bsa_\w+)\s*\(", HEADER, re.M)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert names == sorted(bsa.EXPORTS)
    L = lib()
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings():
    m = re.search(r"#define BSA_VERSION (\d+)", HEADER)
    assert lib().bsa_version() == int(m.group(1))
    for code in (OK, NULL, SHAPE, UNSUP, ALIGN, WS, LAUNCH, ARG):
        assert lib().bsa_status_string(code)
    assert lib().bsa_status_string(123) == b"unknown status"


def test_header_limits_match_binding():
    m = re.search(r"#define BSA_MAX_VIDEO_TILES (\d+)", HEADER)
    assert int(m.group(1)) == bsa.MAX_VIDEO_TILES


def cfg(**kw):
    base = dict(batch=2, heads=3, head_dim=128, grid=(8, 8, 12), keep_tiles=5)
    base.update(kw)
    grid = base.pop("grid")
    return bsa.make_desc(base.pop("batch"), base.pop("heads"), base.pop("head_dim"), grid, base.pop("keep_tiles"),
                         **base)


def ws_size(d):
    n = ctypes.c_size_t(0)
    st = lib().bsa_workspace_size(ctypes.byref(d), ctypes.byref(n))
    return st, n.value


def test_workspace_size_formula():
    d = bsa.make_desc(2, 24, 128, (32, 48, 80), 480)
    st, n = ws_size(d)
    assert st == OK
    pooled = 2 * 24 * 1920 * 128 * 4          # float means of Q, and of K
    split = 2 * 24 * 1920 * 128 * 2 * 2       # their bf16 hi/lo pairs (1,920 rows: whole 16-row blocks)
    norms = 2 * 24 * 1920 * 4                 # their norms
    select_scratch = 256 * 8 * 1920 * 8       # the selection's fallback scratch: one row per wave of the grid
    fwd = (8 * 64 + 4) * 4                    # block-group progress counters and statistics of the forward
    al = lambda x: (x + 255) // 256 * 256
    assert n == 2 * pooled + 2 * split + 2 * norms + select_scratch + al(fwd)
    # no score matrix: the workspace is a few percent of one input tensor's size per head
    assert n < 2 * 24 * 122880 * 128 * 2 // 5
    assert bsa.forward_stats_offset(d) == n - al(fwd) + 8 * 64 * 4
    # dynamic mode also covers the per-(batch, region, head) statistic
    dd = bsa.make_desc(2, 24, 128, (32, 48, 80), 480, dynamic=True)
    assert ws_size(dd)[1] >= 2 * 240 * 24 * 3 * 8
    # no video: nothing to plan, only the forward's counters
    assert ws_size(bsa.make_desc(1, 2, 64, (0, 0, 0), 0, n_prefix=128)) == (OK, al(fwd))


@pytest.mark.parametrize("kw,expect", [
    (dict(head_dim=96), UNSUP),
    (dict(head_dim=32), UNSUP),
    (dict(grid=(8, 8, 10)), SHAPE),              # not divisible by the 4x4x4 tile
    (dict(keep_tiles=0), SHAPE),
    (dict(keep_tiles=13), SHAPE),                # 12 video tiles
    (dict(n_prefix=100), SHAPE),
    (dict(tile=(4, 4, 2)), SHAPE),               # 32 tokens
    (dict(tile=(0, 8, 8)), SHAPE),
    (dict(scale=float("nan")), ARG),
    (dict(scale=0.0), ARG),
    (dict(scale=-1.0), ARG),
    (dict(batch=-1), SHAPE),
    (dict(dynamic=True), SHAPE),                 # dynamic grid must be a multiple of 8
    (dict(dynamic=True, grid=(8, 8, 16), tau=-0.5), ARG),
])
def test_descriptor_errors(kw, expect):
    d = cfg(**kw)
    assert ws_size(d)[0] == expect
    L = lib()
    assert L.bsa_forward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == expect
    assert L.bsa_plan(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == expect
    assert L.bsa_permute(ctypes.byref(d), 1, None, FAKE, None, FAKE, FAKE, None, 0, None) == expect


def test_bad_tile_mode_and_op():
    d = cfg()
    d.tile_mode = 7
    assert ws_size(d)[0] == ARG
    d = cfg()
    assert lib().bsa_permute(ctypes.byref(d), 10, None, FAKE, None, FAKE, FAKE, None, 0, None) == ARG
    assert lib().bsa_permute(ctypes.byref(d), -1, None, FAKE, None, FAKE, FAKE, None, 0, None) == ARG


def test_null_pointers():
    L = lib()
    assert L.bsa_workspace_size(None, ctypes.byref(ctypes.c_size_t())) == NULL
    d = cfg()
    assert L.bsa_workspace_size(ctypes.byref(d), None) == NULL
    assert L.bsa_forward(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == NULL
    for i in range(5):
        args = [FAKE] * 5
        args[i] = None
        assert L.bsa_forward(ctypes.byref(d), *args, None, None, 0, None) == NULL
    assert L.bsa_plan(ctypes.byref(d), None, FAKE, FAKE, FAKE, 1 << 40, None) == NULL
    assert L.bsa_plan(ctypes.byref(d), FAKE, FAKE, None, FAKE, 1 << 40, None) == NULL
    assert L.bsa_permute(ctypes.byref(d), 0, None, None, None, None, None, None, 0, None) == NULL
    assert L.bsa_permute(ctypes.byref(d), 1, None, None, None, FAKE, FAKE, None, 0, None) == NULL
    assert L.bsa_permute(ctypes.byref(d), 2, None, FAKE, None, None, FAKE, None, 0, None) == NULL
    dd = cfg(dynamic=True, grid=(8, 8, 16))
    assert L.bsa_permute(ctypes.byref(dd), 0, None, FAKE, FAKE, None, None, FAKE, 1 << 40, None) == NULL
    assert L.bsa_permute(ctypes.byref(dd), 0, FAKE, FAKE, None, None, None, FAKE, 1 << 40, None) == NULL


def test_alignment_and_workspace_errors():
    L = lib()
    d = cfg()
    bad = FAKE + 8
    assert L.bsa_forward(ctypes.byref(d), bad, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == ALIGN
    assert L.bsa_forward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE + 2, FAKE, None, None, 0, None) == ALIGN
    assert L.bsa_forward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 1, None, 0, None) == ALIGN
    st, need = ws_size(d)
    assert L.bsa_forward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, need - 1, None) == WS
    assert L.bsa_forward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE + 16, need, None) == ALIGN
    st, need = ws_size(d)
    assert L.bsa_plan(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, need - 1, None) == WS
    assert L.bsa_plan(ctypes.byref(d), FAKE, FAKE, FAKE, None, need, None) == WS
    assert L.bsa_plan(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE + 16, need, None) == ALIGN
    assert L.bsa_permute(ctypes.byref(d), 1, None, FAKE, None, bad, FAKE, None, 0, None) == ALIGN
    assert L.bsa_permute(ctypes.byref(d), 0, None, FAKE + 1, None, None, None, None, 0, None) == ALIGN


def test_too_many_tiles_for_plan():
    # 8,320 tiles > the plan limit; permute and forward accept it
    d = bsa.make_desc(1, 1, 64, (16, 128, 260), 10)
    assert lib().bsa_plan(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == UNSUP


def test_too_many_tiles_for_forward():
    # prefix + video tiles above BSA_MAX_TILES: forward refuses before touching anything
    m = re.search(r"#define BSA_MAX_TILES (\d+)", HEADER)
    assert int(m.group(1)) == bsa._lib.MAX_TILES
    d = bsa.make_desc(1, 1, 64, (16, 128, 260), 10, n_prefix=64 * (bsa._lib.MAX_TILES - 8320 + 1))
    assert lib().bsa_forward(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == UNSUP
    d = bsa.make_desc(1, 1, 64, (16, 128, 260), 10, n_prefix=64 * (bsa._lib.MAX_TILES - 8320))
    assert lib().bsa_forward(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == NULL


def test_permute_ops_match_header():
    for name, val in (("BUILD", bsa.PERM_BUILD), ("GATHER", bsa.PERM_GATHER), ("SCATTER", bsa.PERM_SCATTER),
                      ("GATHER_KF", bsa.PERM_GATHER_KF), ("GATHER_VF", bsa.PERM_GATHER_VF),
                      ("GATHER_POOL", bsa.PERM_GATHER_POOL), ("GATHER_KF_POOL", bsa.PERM_GATHER_KF_POOL),
                      ("TILED_TO_KF", bsa.PERM_TILED_TO_KF), ("TILED_TO_VF", bsa.PERM_TILED_TO_VF),
                      ("POOL", bsa.PERM_POOL)):
        m = re.search(r"BSA_PERM_%s = (\d+)" % name, HEADER)
        assert m and int(m.group(1)) == val
    d = cfg()
    L = lib()
    for op in (bsa.PERM_GATHER_KF, bsa.PERM_GATHER_VF, bsa.PERM_GATHER_POOL, bsa.PERM_GATHER_KF_POOL,
               bsa.PERM_TILED_TO_KF, bsa.PERM_TILED_TO_VF):
        # accepted ops: a missing source is reported as such
        assert L.bsa_permute(ctypes.byref(d), op, None, FAKE, None, None, FAKE, None, 0, None) == NULL
        assert L.bsa_permute(ctypes.byref(d), op, None, FAKE, None, FAKE + 8, FAKE, None, 0, None) == ALIGN
    # the pooling gathers write into the workspace: it must be there and large enough
    st, need = ws_size(d)
    for op in (bsa.PERM_GATHER_POOL, bsa.PERM_GATHER_KF_POOL):
        assert L.bsa_permute(ctypes.byref(d), op, None, FAKE, None, FAKE, FAKE, None, 0, None) == WS
        assert L.bsa_permute(ctypes.byref(d), op, None, FAKE, None, FAKE, FAKE, FAKE, need - 1, None) == WS
        assert L.bsa_permute(ctypes.byref(d), op, None, FAKE, None, FAKE, FAKE, FAKE + 16, need, None) == ALIGN
        assert L.bsa_permute(ctypes.byref(d), op, None, None, None, FAKE, FAKE, FAKE, need, None) == NULL
    # the pooling alone reads raster Q through perm into the workspace; no destination
    P = bsa.PERM_POOL
    assert L.bsa_permute(ctypes.byref(d), P, None, FAKE, None, None, None, FAKE, need, None) == NULL
    assert L.bsa_permute(ctypes.byref(d), P, None, None, None, FAKE, None, FAKE, need, None) == NULL
    assert L.bsa_permute(ctypes.byref(d), P, None, FAKE, None, FAKE + 8, None, FAKE, need, None) == ALIGN
    assert L.bsa_permute(ctypes.byref(d), P, None, FAKE + 2, None, FAKE, None, FAKE, need, None) == ALIGN
    assert L.bsa_permute(ctypes.byref(d), P, None, FAKE, None, FAKE, None, None, 0, None) == WS
    assert L.bsa_permute(ctypes.byref(d), P, None, FAKE, None, FAKE, None, FAKE, need - 1, None) == WS
    assert L.bsa_permute(ctypes.byref(d), P, None, FAKE, None, FAKE, None, FAKE + 16, need, None) == ALIGN
    # no video: nothing to pool
    dp = bsa.make_desc(1, 2, 128, (0, 0, 0), 0, n_prefix=128)
    assert L.bsa_permute(ctypes.byref(dp), P, None, None, None, None, None, None, 0, None) == 0
    # the tiled -> fragment conversions need no permutation
    for op in (bsa.PERM_TILED_TO_KF, bsa.PERM_TILED_TO_VF):
        assert L.bsa_permute(ctypes.byref(d), op, None, None, None, FAKE, None, None, 0, None) == NULL


def test_select_host_checks():
    """bsa_select: the kept lists and a full workspace are required; sizes and
    alignment are checked before anything is enqueued."""
    L = lib()
    d = cfg()
    st, need = ws_size(d)
    assert L.bsa_select(None, FAKE, FAKE, need, None) == NULL
    assert L.bsa_select(ctypes.byref(d), None, FAKE, need, None) == NULL
    assert L.bsa_select(ctypes.byref(d), FAKE + 2, FAKE, need, None) == ALIGN
    assert L.bsa_select(ctypes.byref(d), FAKE, None, need, None) == WS
    assert L.bsa_select(ctypes.byref(d), FAKE, FAKE, need - 1, None) == WS
    assert L.bsa_select(ctypes.byref(d), FAKE, FAKE + 16, need, None) == ALIGN
    big = bsa.make_desc(1, 1, 64, (16, 128, 260), 10)   # 8,320 tiles > the plan limit
    assert L.bsa_select(ctypes.byref(big), FAKE, FAKE, 1 << 40, None) == UNSUP
    for e in (cfg(batch=0), bsa.make_desc(1, 2, 64, (0, 0, 0), 0)):
        assert L.bsa_select(ctypes.byref(e), None, None, 0, None) == OK
    n = ctypes.c_size_t(0)
    assert L.bsa_forward_stats_offset(None, ctypes.byref(n)) == NULL
    assert L.bsa_forward_stats_offset(ctypes.byref(d), None) == NULL
    assert L.bsa_forward_stats_offset(ctypes.byref(d), ctypes.byref(n)) == OK
    assert n.value % 4 == 0 and n.value + 8 <= need


def test_empty_problems_are_no_ops():
    L = lib()
    for d in (cfg(batch=0), cfg(heads=0), bsa.make_desc(1, 2, 64, (0, 0, 0), 0)):
        # nothing to do: success without touching any pointer or the GPU
        assert L.bsa_forward(ctypes.byref(d), None, None, None, None, None, None, None, 0, None) == OK
        assert L.bsa_plan(ctypes.byref(d), None, None, None, None, 0, None) == OK
        assert L.bsa_permute(ctypes.byref(d), 1, None, None, None, None, None, None, 0, None) == OK


def test_binding_refuses_host_tensors():
    import torch
    d = cfg()
    x = torch.zeros(16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        bsa.forward(d, x, x, x, x.view(torch.int32), x)


def test_desc_layout_matches_header():
    # field order and size of bsa_desc
    fields = re.search(r"typedef struct bsa_desc \{(.*?)\} bsa_desc;", HEADER, re.S).group(1)
    names = re.findall(r"(?:int32_t|float)\s+(\w+);", fields)
    assert names == [n for n, _ in Desc._fields_]
    assert ctypes.sizeof(Desc) == 4 * len(names)
    assert np.dtype(np.int32).itemsize == 4


def test_padded_mode_host_checks():
    """Ragged grids (BSA_TILE_STATIC_PADDED): the mode constant matches the
    header; the workspace is sized on the padded tile count; the tile must
    still be 64 tokens; the backward takes a ragged grid (a missing tensor is
    reported as such); structured lists count on the rounded-up tile grid."""
    m = re.search(r"BSA_TILE_STATIC_PADDED = (\d+)", HEADER)
    assert m and int(m.group(1)) == bsa.TILE_STATIC_PADDED
    L = lib()
    d = bsa.make_desc(2, 24, 128, (31, 45, 80), 480, padded=True)   # 32 x 48 x 80 tiles after padding
    assert bsa.video_slots(d) == 32 * 48 * 80
    assert ws_size(d) == ws_size(bsa.make_desc(2, 24, 128, (32, 48, 80), 480))
    # the same grid in the plain static mode is not a whole number of tiles
    assert ws_size(bsa.make_desc(2, 24, 128, (31, 45, 80), 480))[0] == SHAPE
    assert ws_size(bsa.make_desc(1, 1, 64, (5, 6, 7), 3, padded=True, tile=(4, 4, 2)))[0] == SHAPE
    assert ws_size(bsa.make_desc(1, 1, 64, (5, 6, 7), 9, padded=True))[0] == SHAPE   # 8 tiles
    n = ctypes.c_size_t(0)
    assert L.bsa_backward_workspace_size(ctypes.byref(d), ctypes.byref(n)) == OK
    assert L.bsa_backward(ctypes.byref(d), *([None] * 11), None, 0, None) == NULL
    # padded mode on a grid that divides: the plain static problem
    dp = bsa.make_desc(1, 2, 64, (8, 8, 12), 5, padded=True)
    assert bsa.video_slots(dp) == 768 and ws_size(dp) == ws_size(bsa.make_desc(1, 2, 64, (8, 8, 12), 5))
    # structured lists over the 2 x 2 x 2 tile grid of a 5 x 6 x 7 grid
    import oracle
    ds = bsa.make_desc(1, 2, 64, (5, 6, 7), 3, padded=True)
    mask = (ctypes.c_int32 * 2)(bsa.MASK_SPATIAL, bsa.MASK_TEMPORAL)
    e = ctypes.c_int64(0)
    assert L.bsa_structured_entries(ctypes.byref(ds), mask, 0, 0, ctypes.byref(e)) == OK
    rp, _ = oracle.plan_structured((2, 2, 2), [0, 1], 0, 0, 1)
    assert e.value == rp[-1]


def test_backward_stats_offset():
    """The backward's statistics sit at the end of either backward workspace,
    after the 2 KB of round counters: the last 16 bytes of the 256-byte
    aligned region of (8 * 64 + 4) ints.  Host-only."""
    L = lib()
    d = cfg()                                   # 2 x 3 heads, 12 video tiles, k = 5
    off, n = ctypes.c_size_t(0), ctypes.c_size_t(0)
    region = (8 * 64 + 4) * 4
    al = lambda x: (x + 255) // 256 * 256
    assert L.bsa_backward_workspace_size(ctypes.byref(d), ctypes.byref(n)) == OK
    assert L.bsa_backward_stats_offset(ctypes.byref(d), 0, ctypes.byref(off)) == OK
    assert off.value == n.value - al(region) + 8 * 64 * 4
    assert L.bsa_backward_csr_workspace_size(ctypes.byref(d), 1000, ctypes.byref(n)) == OK
    assert L.bsa_backward_stats_offset(ctypes.byref(d), 1000, ctypes.byref(off)) == OK
    assert off.value == n.value - al(region) + 8 * 64 * 4
    assert L.bsa_backward_stats_offset(ctypes.byref(d), -1, ctypes.byref(off)) == SHAPE
    assert L.bsa_backward_stats_offset(ctypes.byref(d), 0, None) == NULL


def test_backward_csr_host_checks():
    """bsa_backward_csr: workspace sized on the CSR column count; missing
    lists, an empty column array and a short workspace are refused before
    anything is enqueued."""
    L = lib()
    d = cfg()                                   # 2 x 3 heads, 12 video tiles, k = 5
    n = ctypes.c_size_t(0)
    assert L.bsa_backward_csr_workspace_size(ctypes.byref(d), 100, ctypes.byref(n)) == OK
    small = n.value
    assert L.bsa_backward_csr_workspace_size(ctypes.byref(d), 1000, ctypes.byref(n)) == OK
    assert n.value - small == (1000 * 4 + 255) // 256 * 256 - (100 * 4 + 255) // 256 * 256
    assert L.bsa_backward_csr_workspace_size(ctypes.byref(d), -1, ctypes.byref(n)) == SHAPE
    # with the fixed-keep count the two backward workspaces agree
    fixed = ctypes.c_size_t(0)
    assert L.bsa_backward_workspace_size(ctypes.byref(d), ctypes.byref(fixed)) == OK
    assert L.bsa_backward_csr_workspace_size(ctypes.byref(d), 2 * 3 * 12 * 5, ctypes.byref(n)) == OK
    assert n.value == fixed.value
    ptrs = [FAKE] * 8                           # q k v o d_o lse perm | row_ptr col
    assert L.bsa_backward_csr(ctypes.byref(d), *ptrs[:7], None, FAKE, 100, FAKE, FAKE, FAKE, FAKE, small,
                              None) == NULL
    assert L.bsa_backward_csr(ctypes.byref(d), *ptrs[:7], FAKE, None, 100, FAKE, FAKE, FAKE, FAKE, small,
                              None) == NULL
    assert L.bsa_backward_csr(ctypes.byref(d), *ptrs[:7], FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, small,
                              None) == SHAPE
    assert L.bsa_backward_csr(ctypes.byref(d), *ptrs[:7], FAKE + 4, FAKE, 100, FAKE, FAKE, FAKE, FAKE, small,
                              None) == ALIGN
    assert L.bsa_backward_csr(ctypes.byref(d), *ptrs[:7], FAKE, FAKE, 100, FAKE, FAKE, FAKE, FAKE, small - 1,
                              None) == WS


def test_forward_raster_host_checks():
    """bsa_forward_raster's argument checks (host only, nothing launched):
    the tensors and perm are required (perm not without video), aligned, the
    workspace optional but whole and aligned, and the tile limit is
    bsa_forward's."""
    L = lib()
    d = cfg()
    F = L.bsa_forward_raster
    # q, perm, k, v, block_idx, o
    for i in range(6):
        args = [FAKE] * 6
        args[i] = None
        assert F(ctypes.byref(d), *args, None, None, 0, None) == NULL
    assert F(None, *([FAKE] * 6), None, None, 0, None) == NULL
    assert F(ctypes.byref(d), FAKE + 8, *([FAKE] * 5), None, None, 0, None) == ALIGN
    assert F(ctypes.byref(d), FAKE, FAKE + 2, *([FAKE] * 4), None, None, 0, None) == ALIGN
    assert F(ctypes.byref(d), *([FAKE] * 5), FAKE + 8, None, None, 0, None) == ALIGN
    assert F(ctypes.byref(d), *([FAKE] * 6), FAKE + 1, None, 0, None) == ALIGN
    st, need = ws_size(d)
    assert F(ctypes.byref(d), *([FAKE] * 6), None, FAKE, need - 1, None) == WS
    assert F(ctypes.byref(d), *([FAKE] * 6), None, FAKE + 16, need, None) == ALIGN
    # prefix only: the tensors are still required
    dp = bsa.make_desc(1, 2, 128, (0, 0, 0), 0, n_prefix=128)
    assert F(ctypes.byref(dp), None, None, FAKE, FAKE, None, FAKE, None, None, 0, None) == NULL
    # too many tiles, as bsa_forward
    big = bsa.make_desc(1, 1, 64, (16, 128, 260), 10, n_prefix=64 * (bsa._lib.MAX_TILES - 8320 + 1))
    assert F(ctypes.byref(big), *([FAKE] * 6), None, None, 0, None) == UNSUP
    # empty problems are no-ops
    assert F(ctypes.byref(bsa.make_desc(0, 2, 128, (8, 8, 8), 2)), *([None] * 6), None, None, 0, None) == 0


def test_overlapping_output_is_rejected():
    """An output whose byte range meets an input of the same call is refused
    on the host (BSA_ERR_ARG), before anything is enqueued: forward (tiled,
    raster, CSR) and the permutation copies."""
    L = lib()
    d = cfg()
    B, H, D = d.batch, d.heads, d.head_dim
    n_tot = d.n_prefix + d.grid_t * d.grid_h * d.grid_w
    tiled = B * H * n_tot * D * 2
    far = FAKE + 4 * tiled + (1 << 20)  # a second region clear of the first
    far -= far % 256
    # forward: o inside q, o just past q (allowed: ranges touch but do not meet)
    assert L.bsa_forward(ctypes.byref(d), FAKE, far, far + 2 * tiled, FAKE, FAKE + tiled - 256, None, None, 0,
                         None) == ARG
    st = L.bsa_forward(ctypes.byref(d), FAKE, far, far + 2 * tiled, FAKE, FAKE, None, None, 0, None)
    assert st == ARG  # in place
    # o overlapping k_frag
    assert L.bsa_forward(ctypes.byref(d), FAKE, far, far + 2 * tiled, FAKE, far + 256, None, None, 0, None) == ARG
    # raster: o_raster on q_raster
    F = L.bsa_forward_raster
    assert F(ctypes.byref(d), FAKE, FAKE, far, far + 2 * tiled, FAKE, FAKE, None, None, 0, None) == ARG
    # CSR forward
    assert L.bsa_forward_csr(ctypes.byref(d), FAKE, far, far + 2 * tiled, FAKE, FAKE, 1, FAKE, None, None, 0,
                             None) == ARG
    # permute: gather in place, scatter in place, tiled -> fragment in place
    for op in (bsa.PERM_GATHER, bsa.PERM_GATHER_KF, bsa.PERM_GATHER_VF, bsa.PERM_SCATTER, bsa.PERM_TILED_TO_KF,
               bsa.PERM_TILED_TO_VF):
        assert L.bsa_permute(ctypes.byref(d), op, None, FAKE, None, FAKE, FAKE + 256, None, 0, None) == ARG, op


def test_overlaps_of_lse_lists_and_gradients_are_rejected():
    """The forward's lse may meet neither an input nor O, and O not the kept
    lists or the permutation; the backward's three gradients may meet
    neither each other, an input nor the workspace (BSA_ERR_ARG, nothing
    enqueued).  Every other argument lies in a region of its own."""
    L = lib()
    d = cfg()
    B, H, D = d.batch, d.heads, d.head_dim
    n_tot = d.n_prefix + d.grid_t * d.grid_h * d.grid_w
    tiled = B * H * n_tot * D * 2
    step = 8 * tiled + (1 << 20)
    step -= step % 4096
    R = [FAKE + i * step for i in range(16)]  # disjoint regions
    q, k, v, idx, o, lse, perm = R[0], R[1], R[2], R[3], R[4], R[5], R[6]
    # forward, tiled: lse on q, lse on o, o on the kept lists
    F = L.bsa_forward
    assert F(ctypes.byref(d), q, k, v, idx, o, q + 256, None, 0, None) == ARG
    assert F(ctypes.byref(d), q, k, v, idx, o, o + 512, None, 0, None) == ARG
    assert F(ctypes.byref(d), q, k, v, idx, idx + 16, lse, None, 0, None) == ARG
    # raster: o on the permutation, lse on k
    G = L.bsa_forward_raster
    assert G(ctypes.byref(d), q, perm, k, v, idx, perm, lse, None, 0, None) == ARG
    assert G(ctypes.byref(d), q, perm, k, v, idx, o, k, None, 0, None) == ARG
    # CSR: o on the row pointers
    rp, col = R[7], R[8]
    assert L.bsa_forward_csr(ctypes.byref(d), q, k, v, rp, col, 5, rp, lse, None, 0, None) == ARG
    # backward
    n = ctypes.c_size_t(0)
    assert L.bsa_backward_workspace_size(ctypes.byref(d), ctypes.byref(n)) == OK
    ws = R[9]
    d_o, dq, dk, dv = R[10], R[11], R[12], R[13]
    Bw = L.bsa_backward
    args = lambda dq_, dk_, dv_: (ctypes.byref(d), q, k, v, o, d_o, lse, perm, idx, dq_, dk_, dv_, ws, n.value, None)
    assert Bw(*args(dq, dq + 256, dv)) == ARG      # dq and dk meet
    assert Bw(*args(dq, dk, ws + 4096)) == ARG     # dv inside the workspace
    assert Bw(*args(d_o, dk, dv)) == ARG           # dq on dO
    assert Bw(*args(dq, perm, dv)) == ARG          # dk on the permutation
    assert Bw(*args(dq, dk, lse)) == ARG           # dv on the lse


def test_keep_from_sparsity():
    """The sparsity -> kept-tiles helper against the pages' worked figures:
    sparsity 0.75 keeps 480 of 1,920 key tiles per query tile (Prism page,
    section on Prism's block-sparse attention); 0.9375 (the CLI default the
    same page names) keeps 120; rounding to nearest, clamped to [1, n]; and
    calls under the 12,288-token minimum of the ComfyUI node ("倍速で回した一晩",
    section "같은 방식을 직접 해보려면") stay dense."""
    assert bsa.keep_tiles_for(0.75, 1920) == 480
    assert bsa.keep_tiles_for(0.9375, 1920) == 120
    assert bsa.keep_tiles_for(0.9, 1920) == 192 and bsa.keep_tiles_for(0.95, 1920) == 96
    assert bsa.keep_tiles_for(0.93, 1920) == 134  # 134.4 rounds down
    assert bsa.keep_tiles_for(0.0, 32) == 32 and bsa.keep_tiles_for(1.0, 32) == 1
    assert bsa.keep_tiles_for(0.99, 32) == 1      # never zero tiles
    assert bsa.keep_tiles_for(0.75, 1512) == 378  # the prefix workload's video tiles
    assert bsa.keep_tiles_for(0.75, 0) == 0
    for bad in (-0.1, 1.5, float("nan")):
        with pytest.raises(ValueError):
            bsa.keep_tiles_for(bad, 100)
    assert bsa.DENSE_BELOW_TOKENS == 12288
    assert bsa.keep_for_call(0.75, 32, 2048) == 32            # small call: dense
    assert bsa.keep_for_call(0.75, 1920, 122880) == 480
    assert bsa.keep_for_call(0.75, 192, 12288) == 48          # at the minimum: sparse
    assert bsa.keep_for_call(0.75, 192, 12288, dense_below=0) == 48


def test_csr_select_and_raster_forward_host_checks():
    """bsa_select_csr (the CSR selection from the means in the workspace) and
    bsa_forward_csr_raster reject bad arguments on the host."""
    L = lib()
    d = cfg()
    st, need = ws_size(d)
    n_entries = ctypes.c_int64()
    assert L.bsa_csr_entries(ctypes.byref(d), None, ctypes.byref(n_entries)) == OK
    E = n_entries.value
    S_ = L.bsa_select_csr
    assert S_(ctypes.byref(d), None, None, None, FAKE, E, FAKE, need, None) == NULL        # row_ptr
    assert S_(ctypes.byref(d), None, None, FAKE, None, E, FAKE, need, None) == NULL        # col_idx
    assert S_(ctypes.byref(d), None, None, FAKE, FAKE, E - 1, FAKE, need, None) == SHAPE   # too few entries
    assert S_(ctypes.byref(d), None, None, FAKE, FAKE, E, None, 0, None) == WS
    assert S_(ctypes.byref(d), None, None, FAKE, FAKE, E, FAKE, need - 1, None) == WS
    assert S_(ctypes.byref(d), None, None, FAKE + 4, FAKE, E, FAKE, need, None) == ALIGN
    F = L.bsa_forward_csr_raster
    # q, perm, k, v, row_ptr, col_idx
    for i in range(6):
        args = [FAKE] * 6
        args[i] = None
        assert F(ctypes.byref(d), *args, E, FAKE, None, None, 0, None) == NULL, i
    assert F(ctypes.byref(d), *([FAKE] * 6), E, None, None, None, 0, None) == NULL        # o
    assert F(ctypes.byref(d), *([FAKE] * 6), 0, FAKE, None, None, 0, None) == SHAPE       # no entries
    assert F(ctypes.byref(d), FAKE, FAKE + 2, *([FAKE] * 4), E, FAKE, None, None, 0, None) == ALIGN
    assert F(ctypes.byref(d), *([FAKE] * 6), E, FAKE, None, FAKE, need - 1, None) == WS
    assert F(ctypes.byref(d), *([FAKE] * 6), E, FAKE, None, None, 0, None) == ARG         # o on q
