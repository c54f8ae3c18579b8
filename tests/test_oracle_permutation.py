"""Pins of the oracle's tile numbering, permutation, gather and scatter.

Each check compares the oracle with an independent statement of the same fact
(a closed-form inverse, numpy fancy indexing, a bijection count) or with the
counts printed on the Prism speed-ablation page (tests/golden/pages_counts.json).
"""
import json
import os

import numpy as np
import pytest

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_counts.json")))


def raster_coords(grid):
    T, H, W = grid
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    return t.reshape(-1), h.reshape(-1), w.reshape(-1)


@pytest.mark.parametrize("grid,tile", [((8, 16, 16), (4, 4, 4)), ((8, 8, 12), (4, 4, 4)),
                                       ((4, 8, 16), (2, 4, 8)), ((16, 4, 4), (16, 2, 2)),
                                       ((2, 4, 32), (2, 2, 16))])
def test_static_perm_matches_closed_form_inverse(orc, grid, tile):
    T, H, W = grid
    tt, th, tw = tile
    perm = orc.perm_static(grid, tile)
    t, h, w = raster_coords(grid)
    tile_id = ((t // tt) * (H // th) + h // th) * (W // tw) + w // tw
    offset = ((t % tt) * th + h % th) * tw + w % tw
    slot = tile_id * 64 + offset
    expect = np.empty(T * H * W, np.int64)
    expect[slot] = np.arange(T * H * W)
    np.testing.assert_array_equal(perm, expect)
    assert np.array_equal(np.sort(perm), np.arange(T * H * W))  # bijection


def test_static_perm_rejects_non_divisible(orc):
    with pytest.raises(ValueError):
        orc.perm_static((8, 8, 10), (4, 4, 4))
    with pytest.raises(ValueError):
        orc.perm_static((8, 8, 8), (4, 4, 2))  # 32 tokens, not 64


def test_pages_tile_count(orc):
    grid = tuple(GOLD["grid_twh"])
    perm = orc.perm_static(grid, tuple(GOLD["default_block"]))
    n_tokens = perm.size
    assert abs(n_tokens - GOLD["tokens_approx"]) / GOLD["tokens_approx"] < 0.01
    assert n_tokens // GOLD["tokens_per_block"] == GOLD["key_blocks_per_query_block"]


def _rand_raster(rng, B, Ntot, H, D):
    return rng.integers(0, 65536, size=(B, Ntot, H, D), dtype=np.uint16)


@pytest.mark.parametrize("n_prefix", [0, 128])
def test_gather_is_fancy_index_and_scatter_inverts(orc, n_prefix):
    rng = np.random.default_rng(5)
    grid = (8, 8, 12)
    B, H, D = 2, 3, 16
    Nv = 8 * 8 * 12
    x = _rand_raster(rng, B, n_prefix + Nv, H, D)
    perm = orc.perm_static(grid)
    t = orc.gather(x, perm, n_prefix)
    src = np.concatenate([np.arange(n_prefix), n_prefix + perm])
    expect = x[:, src].transpose(0, 2, 1, 3)
    np.testing.assert_array_equal(t, expect)
    back = orc.scatter(t, perm, n_prefix)
    np.testing.assert_array_equal(back, x)


def test_gather_identity_perm_is_transpose(orc):
    rng = np.random.default_rng(6)
    x = _rand_raster(rng, 1, 64 * 4, 2, 8)
    perm = np.arange(64 * 4, dtype=np.int32)
    np.testing.assert_array_equal(orc.gather(x, perm, 0), x.transpose(0, 2, 1, 3))


# ----------------------------------------------------------------- dynamic ----

def _check_dynamic_tiles(orc, shape, grid):
    """Every tile is an axis-aligned box of its region's shape; region slots
    cover exactly that region (or the region pair) ; the map is a bijection."""
    T, H, W = grid
    RT, RH, RW = T // 8, H // 8, W // 8
    perm = orc.perm_dynamic(shape, grid)
    B = shape.shape[0]
    for b in range(B):
        p = perm[b]
        assert np.array_equal(np.sort(p), np.arange(T * H * W))
        t, h, w = p // (H * W), (p // W) % H, p % W
        for r in range(RT * RH * RW):
            sid = int(shape[b, r])
            ext = orc.shape_extent(sid)
            rt, rh, rw = r // (RH * RW), (r // RW) % RH, r % RW
            for s in range(r * 8, r * 8 + 8):
                sl = slice(s * 64, s * 64 + 64)
                tt, hh, ww = t[sl], h[sl], w[sl]
                spans = (tt.max() - tt.min() + 1, hh.max() - hh.min() + 1, ww.max() - ww.min() + 1)
                assert spans == ext, (r, s, spans, ext)
                # aligned to the shape inside the region
                assert tt.min() % ext[0] == 0 and hh.min() % ext[1] == 0 and ww.min() % ext[2] == 0
                # raster order inside the tile
                key = (tt * H + hh) * W + ww
                assert np.all(np.diff(key) > 0)
            if sid < 7:
                sl = slice(r * 512, r * 512 + 512)
                assert t[sl].min() == rt * 8 and t[sl].max() == rt * 8 + 7
                assert h[sl].min() == rh * 8 and h[sl].max() == rh * 8 + 7
                assert w[sl].min() == rw * 8 and w[sl].max() == rw * 8 + 7
    return perm


def test_dynamic_all_default_equals_static_tiles(orc):
    grid = (16, 8, 24)
    R = 2 * 1 * 3
    shape = np.zeros((2, R), np.uint8)
    perm = _check_dynamic_tiles(orc, shape, grid)
    stat = orc.perm_static(grid)
    # same set of tiles, numbered region-major instead of grid raster
    dyn_tiles = {tuple(sorted(perm[0][i * 64:(i + 1) * 64])) for i in range(perm.shape[1] // 64)}
    st_tiles = {tuple(sorted(stat[i * 64:(i + 1) * 64])) for i in range(stat.size // 64)}
    assert dyn_tiles == st_tiles


def test_dynamic_mixed_shapes_and_pairs(orc):
    grid = (16, 16, 32)  # regions 2 x 2 x 4
    RT, RH, RW = 2, 2, 4
    rng = np.random.default_rng(7)
    shape = rng.integers(0, 7, size=(2, RT * RH * RW)).astype(np.uint8)
    # batch 0: one w-pair (regions 0,1) and one t-pair (regions 2 and 2 + RH*RW)
    shape[0, 0] = shape[0, 1] = 7
    shape[0, 2] = shape[0, 2 + RH * RW] = 8
    # batch 1: all w-pairs
    shape[1, :] = 7
    _check_dynamic_tiles(orc, shape, grid)
    # pairs: slots of both regions together cover exactly the 8x8x16 (or 16x8x8) union
    perm = orc.perm_dynamic(shape, grid)
    p = perm[0][0:16 * 64]
    T, H, W = grid
    t, h, w = p // (H * W), (p // W) % H, p % W
    assert (t.min(), t.max(), h.min(), h.max(), w.min(), w.max()) == (0, 7, 0, 7, 0, 15)


def test_dynamic_rejects_unpaired_long_shape(orc):
    grid = (8, 8, 16)
    shape = np.array([[7, 0]], np.uint8)
    with pytest.raises(ValueError):
        orc.perm_dynamic(shape, grid)
