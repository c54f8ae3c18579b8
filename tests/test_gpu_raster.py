"""The raster-I/O path: bsa_permute(POOL) for Q's tile means and
bsa_forward_raster, which reads Q and writes O in the raster layout itself.

* Against the tiled path (gather, select, forward, scatter) on every small
  parity workload and every ragged grid: Q's means, the kept lists, the
  output and the lse equal bit for bit, with the raster output first filled
  with a NaN pattern so that a row the kernel failed to write shows; the same
  for the one-block-per-tile launch (no workspace).
* Against the oracle on its own: the raster output, gathered into tile order
  by the oracle, within the output tolerance of the oracle's attention, and
  Q's means bit-exact against the oracle's pooling of the oracle's gather.
* Variable keep (bsa_select_csr from the pooled means, bsa_forward_csr_raster)
  and structured lists against the tiled CSR path, bit for bit.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_39_amd as bsa
import oracle
import synthetic as S
from parity import DeviceRun, check_output, desc_for, to_bits
from test_gpu_padded import CASES as PADDED_CASES
from test_gpu_parity import CASES as PARITY_CASES

pytestmark = pytest.mark.gpu

NAN_BITS = 0x7FC1  # a quiet NaN in bf16


def raster_run(wl, g, grouped=True):
    """The raster path on the inputs of DeviceRun g, into a NaN-filled output."""
    att = bsa.BlockSparseAttention(g.desc, with_lse=True, grouped=grouped)
    out = torch.full_like(g.q.view(torch.int16), NAN_BITS).view(torch.bfloat16)
    att(g.q, g.k, g.v, out)
    torch.cuda.synchronize()
    return att, out


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))


CASES = PARITY_CASES + PADDED_CASES


@pytest.mark.parametrize("wl", CASES, ids=[c.name for c in CASES])
def test_raster_path_equals_tiled_path(wl):
    print(f"\n[case] {wl}", flush=True)
    q, k, v = S.qkv(wl)
    g = DeviceRun(wl, q, k, v).run()
    for grouped in (True, False):
        att, out = raster_run(wl, g, grouped)
        n = wl.n_video_slots
        assert same_bits(att.perm[:, :n], g.att.perm[:, :n])
        if wl.n_video:
            gq, gk = g.pooled()
            rq, rk = bsa.pooled_views(g.desc, att.workspace)
            assert np.array_equal(rq.cpu().numpy(), gq) and np.array_equal(rk.cpu().numpy(), gk)
            assert same_bits(att.block_idx, g.att.block_idx)
        assert same_bits(out, g.out), f"raster output differs (grouped={grouped})"
        assert torch.equal(att.lse, g.att.lse)
        print(f"[raster] grouped={grouped}: output, lse, lists and means equal", flush=True)


ORACLE_CASES = [PARITY_CASES[1], PARITY_CASES[3], PARITY_CASES[10], PADDED_CASES[0], PADDED_CASES[1]]


@pytest.mark.parametrize("wl", ORACLE_CASES, ids=[c.name for c in ORACLE_CASES])
def test_raster_path_matches_oracle(wl):
    print(f"\n[case] {wl}", flush=True)
    q, k, v = S.qkv(wl)
    g = DeviceRun(wl, q, k, v)  # inputs and descriptor only
    att, out = raster_run(wl, g)
    npf, scale = wl.n_prefix, float(np.float32(wl.scale))
    perm = att.perm.cpu().numpy()[:, :wl.n_video_slots]
    if wl.padded:
        p1 = oracle.perm_static_padded(wl.grid, wl.tile)
        assert np.array_equal(perm, np.broadcast_to(p1, perm.shape))
        gat = lambda x: oracle.gather_padded(x, p1, npf)
        pool = lambda x: oracle.pool_padded(x, p1, npf)
        real = oracle.key_real(p1, npf)
    else:
        if not wl.dynamic:
            assert np.array_equal(perm, np.broadcast_to(oracle.perm_static(wl.grid, wl.tile), perm.shape))
        gat = lambda x: oracle.gather(x, perm, npf)
        pool = lambda x: oracle.pool(x, npf)
        real = None
    qt, kt, vt = gat(q), gat(k), gat(v)
    o_t = gat(to_bits(out))  # the raster output in tile order (zeros in padding slots)
    rq, _ = bsa.pooled_views(g.desc, att.workspace)
    assert np.array_equal(rq.cpu().numpy(), pool(qt))
    gidx = att.block_idx.cpu().numpy()[:, :, :wl.n_video_tiles, :wl.keep_tiles]
    nqt = wl.n_tiled_tokens // 64
    tiles = np.arange(nqt, dtype=np.int32)
    if nqt > 32:
        tiles = np.sort(np.random.default_rng(wl.seed).choice(nqt, size=32, replace=False)).astype(np.int32)
    worst = 0.0
    for b in range(wl.batch):
        for h in range(wl.heads):
            if real is None:
                ref, _ = oracle.attention(qt[b, h], kt[b, h], vt[b, h], npf, gidx[b, h], scale, tiles)
            else:
                ref, _ = oracle.attention_padded(qt[b, h], kt[b, h], vt[b, h], npf, gidx[b, h], real, scale, tiles)
            got = o_t[b, h].reshape(nqt, 64, wl.head_dim)[tiles]
            if real is not None:  # padding query rows are not outputs
                rows = real.reshape(nqt, 64)[tiles].astype(bool)
                got, ref = got[rows], ref.reshape(got.shape)[rows]
            mx, _ = check_output(got, ref, f"b{b} h{h}")
            worst = max(worst, mx)
    print(f"[raster] worst max|err| {worst:.3e} against the oracle", flush=True)


# ---- variable keep and structured lists through the raster-I/O calls --------
CSR_CASES = [
    (S.Workload("csr_rows", 2, 2, 128, (8, 8, 16), 6, seed=22), [6, 11], (-1, 13)),
    (S.Workload("csr_prefix_d64", 1, 3, 64, (8, 8, 12), 4, seed=23, n_prefix=128), [4, 1, 7], None),
    (S.Workload("csr_pad", 1, 2, 128, (7, 9, 13), 5, seed=24, padded=True), [5, 2], (0, 4)),
    (S.Workload("csr_dynamic", 1, 2, 128, (16, 16, 16), 6, seed=25, dynamic=True, recipe="field"), [6, 20], None),
]


@pytest.mark.parametrize("wl,keep_h,rows_range", CSR_CASES, ids=[c[0].name for c in CSR_CASES])
def test_csr_raster_equals_tiled(wl, keep_h, rows_range):
    """Per-head (and per-row) keeps: the means left by POOL and GATHER_KF_POOL
    and bsa_select_csr give bsa_plan_csr's row pointers and lists, and
    bsa_forward_csr_raster gives bsa_forward_csr followed by the scatter, bit
    for bit (output first filled with NaN), lse included; grouped and plain."""
    print(f"\n[case] {wl} keep_per_head={keep_h} rows={rows_range}", flush=True)
    q, k, v = S.qkv(wl)
    g = DeviceRun(wl, q, k, v).run()
    d, a = g.desc, g.att
    n = wl.n_video_tiles
    kr = None
    if rows_range is not None:
        rng = np.random.default_rng(wl.seed + 100)
        kr = torch.from_numpy(rng.integers(rows_range[0], rows_range[1] + 1,
                                           size=(wl.batch, wl.heads, n)).astype(np.int32)).cuda()
    rows = wl.batch * wl.heads * n
    entries = bsa.csr_entries(d, keep_h)
    rp_t = torch.full((rows + 1,), -7, dtype=torch.int64, device="cuda")
    col_t = torch.full((entries,), -7, dtype=torch.int32, device="cuda")
    bsa.plan_csr(d, a.q_t, a.k_f, rp_t, col_t, a.workspace, keep_per_head=keep_h, keep_rows=kr)
    o_t = torch.empty_like(a.q_t)
    lse_t = torch.empty_like(a.lse)
    bsa.forward_csr(d, a.q_t, a.k_f, a.v_f, rp_t, col_t, o_t, lse_t, workspace=a.workspace)
    ref = torch.empty_like(g.q)
    bsa.scatter(d, o_t, ref, a.perm)
    # the raster-I/O path on a fresh set of buffers
    r = bsa.BlockSparseAttention(d, with_lse=True)
    r.build(g.q)
    r.pool_qk(g.q, g.k)
    r.gather_v(g.v)
    rp_r = torch.full_like(rp_t, -7)
    col_r = torch.full_like(col_t, -7)
    bsa.select_csr(d, rp_r, col_r, r.workspace, keep_per_head=keep_h, keep_rows=kr)
    torch.cuda.synchronize()
    assert torch.equal(rp_r, rp_t)
    assert torch.equal(col_r[:int(rp_t[-1])], col_t[:int(rp_t[-1])])
    for ws in (r.workspace, None):
        out = torch.full_like(g.q.view(torch.int16), NAN_BITS).view(torch.bfloat16)
        lse = torch.full_like(lse_t, 7.0)
        bsa.forward_csr_raster(d, g.q, r.perm, r.k_f, r.v_f, rp_r, col_r, out, lse, workspace=ws)
        torch.cuda.synchronize()
        assert same_bits(out, ref), f"raster CSR output differs (workspace={ws is not None})"
        assert torch.equal(lse, lse_t)
    print("[raster CSR] lists, output and lse equal the tiled path's", flush=True)


@pytest.mark.parametrize("wl,mask,rt,rs", [
    (S.Workload("st_prefix", 2, 3, 128, (8, 8, 16), 4, seed=32, n_prefix=128), [1, 0, 1], 0, 2),
    (S.Workload("st_shape_d64", 1, 2, 64, (16, 8, 8), 4, seed=33, tile=(8, 2, 4)), [0, 1], 1, 0),
], ids=["st_prefix", "st_shape_d64"])
def test_structured_raster_equals_tiled(wl, mask, rt, rs):
    """Structured lists need no pooling: the K and V gathers and
    bsa_forward_csr_raster give bsa_forward_csr followed by the scatter, bit
    for bit."""
    print(f"\n[case] {wl} mask={mask} radii=({rt}, {rs})", flush=True)
    q, k, v = S.qkv(wl)
    g = DeviceRun(wl, q, k, v).run()
    d, a = g.desc, g.att
    rows = wl.batch * wl.heads * wl.n_video_tiles
    row_ptr = torch.empty(rows + 1, dtype=torch.int64, device="cuda")
    col = torch.empty(bsa.structured_entries(d, mask, rt, rs), dtype=torch.int32, device="cuda")
    bsa.plan_structured(d, mask, rt, rs, row_ptr, col)
    o_t = torch.empty_like(a.q_t)
    lse_t = torch.empty_like(a.lse)
    bsa.forward_csr(d, a.q_t, a.k_f, a.v_f, row_ptr, col, o_t, lse_t, workspace=a.workspace)
    ref = torch.empty_like(g.q)
    bsa.scatter(d, o_t, ref, a.perm)
    out = torch.full_like(g.q.view(torch.int16), NAN_BITS).view(torch.bfloat16)
    lse = torch.empty_like(lse_t)
    bsa.forward_csr_raster(d, g.q, a.perm, a.k_f, a.v_f, row_ptr, col, out, lse, workspace=a.workspace)
    torch.cuda.synchronize()
    assert same_bits(out, ref) and torch.equal(lse, lse_t)
