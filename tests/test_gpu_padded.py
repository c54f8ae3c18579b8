"""GPU parity of ragged grids (BSA_TILE_STATIC_PADDED): a video grid that is
not a whole number of static tiles, covered by the tile grid rounded up.

* permutation (-1 in padding slots), gathers (zeros there), scatter: bit-exact;
* tile means over the real tokens only: bit-exact;
* kept tiles: the selection rules of the other parity tests;
* attention over the real keys only (boundary tiles masked), on the real
  query rows, with the forward's output and lse tolerances;
* on a grid that divides, padded mode is the plain static path bit for bit;
* dQ, dK, dV on the raster rows against the oracle's gradients of the padded
  forward, with the backward's tolerances (small cases in full, the 720p clip
  on sampled tiles).
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_39_amd as bsa
import oracle
import synthetic as S
from parity import (DeviceRun, attending_tiles, bits_to_f64, check_lse, check_output, check_selection, kfrag_layout,
                    oracle_lse_delta_rows, to_bits, to_dev,
                    vfrag_layout)

pytestmark = pytest.mark.gpu

W = S.Workload
CASES = [
    # tile (0,0,0) full, every other tile a boundary tile; one t-layer of 16 real keys per tile
    W("pad_5x6x7", 2, 2, 128, (5, 6, 7), 5, seed=41, n_prefix=64, padded=True),
    W("pad_d64", 1, 3, 64, (9, 13, 10), 7, seed=42, padded=True),
    W("pad_tile2x4x8", 1, 2, 128, (7, 9, 20), 4, seed=43, tile=(2, 4, 8), padded=True),
    W("pad_keep_all", 1, 2, 128, (6, 5, 9), 12, seed=44, n_prefix=128, padded=True),
    W("pad_k1_d64", 2, 1, 64, (13, 7, 6), 1, seed=45, padded=True),
    W("pad_many", 1, 1, 128, (30, 21, 43), 37, seed=46, padded=True),
]


def check_padded_path(wl, g, q, k, v, qtiles=None, bh=None):
    npf, scale = wl.n_prefix, float(np.float32(wl.scale))
    B, H, D = wl.batch, wl.heads, wl.head_dim
    p1 = oracle.perm_static_padded(wl.grid, wl.tile)
    perm = np.ascontiguousarray(np.broadcast_to(p1, (B, p1.size)))
    assert np.array_equal(g.perm(), perm)
    nqt = wl.n_tiled_tokens // 64
    real = oracle.key_real(p1, npf)
    o_t = to_bits(g.att.o_t)
    lse = g.att.lse.cpu().numpy()
    gq, gk = g.pooled()
    gidx = g.block_idx()
    pairs = bh if bh is not None else [(b, h) for b in range(B) for h in range(H)]
    worst = 0.0
    for b, h in pairs:
        sl = lambda x: np.ascontiguousarray(x[b:b + 1, :, h:h + 1])
        qt, kt, vt = (oracle.gather_padded(sl(x), p1, npf) for x in (q, k, v))
        assert np.array_equal(to_bits(g.att.q_t[b:b + 1, h:h + 1]), qt)
        assert np.array_equal(to_bits(g.att.k_f[b:b + 1, h:h + 1]).reshape(-1), kfrag_layout(kt).reshape(-1))
        assert np.array_equal(to_bits(g.att.v_f[b:b + 1, h:h + 1]).reshape(-1), vfrag_layout(vt).reshape(-1))
        qp, kp = oracle.pool_padded(qt, p1, npf), oracle.pool_padded(kt, p1, npf)
        assert np.array_equal(gq[b:b + 1, h:h + 1], qp) and np.array_equal(gk[b:b + 1, h:h + 1], kp)
        n_exact, n_near, n_gamma = check_selection(gidx[b:b + 1, h:h + 1], qp, kp, wl.keep_tiles)
        tiles = np.arange(nqt, dtype=np.int32) if qtiles is None else qtiles
        ref, ref_lse = oracle.attention_padded(qt[0, 0], kt[0, 0], vt[0, 0], npf, gidx[b, h], real, scale, tiles)
        rows = real.reshape(nqt, 64)[tiles].astype(bool)  # real query rows of the sampled tiles
        got = o_t[b, h].reshape(nqt, 64, D)[tiles]
        mx, mean = check_output(got[rows], ref[rows], f"b{b} h{h}")
        worst = max(worst, mx)
        check_lse(lse[b, h].reshape(nqt, 64)[tiles][rows], ref_lse[rows],
                  qt[0, 0].reshape(nqt, 64, D)[tiles][rows], kt[0, 0], scale, f"lse b{b} h{h}")
        print(f"[b{b} h{h}] plan exact {n_exact} near {n_near}; attention max|err| {mx:.2e} mean {mean:.2e}",
              flush=True)
    return perm, worst


@pytest.mark.parametrize("wl", CASES, ids=[c.name for c in CASES])
def test_padded_path_matches_oracle(wl):
    print(f"\n[case] {wl} slots {wl.n_video_slots} tiles {wl.n_video_tiles}", flush=True)
    q, k, v = S.qkv(wl)
    g = DeviceRun(wl, q, k, v).run()
    perm, worst = check_padded_path(wl, g, q, k, v)
    # scatter: the real rows back to raster order, padding slots dropped
    ref_out = oracle.scatter_padded(to_bits(g.att.o_t), perm, wl.n_prefix, wl.n_video)
    assert np.array_equal(to_bits(g.out), ref_out)
    print(f"[forward] worst max|err| {worst:.3e}", flush=True)


def test_padded_mode_on_divisible_grid_is_static_path():
    base = W("pad_div", 2, 2, 128, (8, 8, 12), 5, seed=47, n_prefix=64)
    q, k, v = S.qkv(base)
    g1 = DeviceRun(base, q, k, v).run()
    g2 = DeviceRun(W("pad_div", 2, 2, 128, (8, 8, 12), 5, seed=47, n_prefix=64, padded=True), q, k, v).run()
    assert np.array_equal(g1.perm(), g2.perm())
    assert np.array_equal(g1.block_idx(), g2.block_idx())
    assert np.array_equal(to_bits(g1.out), to_bits(g2.out))
    assert np.array_equal(g1.att.lse.cpu().numpy(), g2.att.lse.cpu().numpy())


def test_prism720p_ragged_sampled():
    """The 720p clip's real latent grid, 31 x 45 x 80 tokens (batch 2, 24
    heads, head_dim 128), padded to the 32 x 48 x 80 tile grid (1,920 tiles,
    keep 480): permutation in full; gathers, means, lists and attention on
    sampled (batch, head) slices and query tiles, boundary tiles among them."""
    wl = S.WORKLOADS["prism720p_ragged"]
    print(f"\n[case] {wl}", flush=True)
    q, k, v = S.qkv(wl)
    g = DeviceRun(wl, q, k, v).run()
    nqt = wl.n_tiled_tokens // 64
    rng = np.random.default_rng(91)
    # tiles of the last t-layer and last h-row are boundary tiles (31 = 7*4 + 3, 45 = 11*4 + 1)
    boundary = np.array([1919, 1900, 1500, 79 + 80 * 11], np.int32)
    tiles = np.unique(np.concatenate([boundary, rng.choice(nqt, size=12, replace=False)])).astype(np.int32)
    check_padded_path(wl, g, q, k, v, qtiles=tiles, bh=[(0, 0), (1, 13)])
    del g
    torch.cuda.empty_cache()


# ---- gradients on ragged grids ---------------------------------------------------

BWD_CASES = [
    W("bpad_5x6x7", 2, 2, 128, (5, 6, 7), 5, seed=51, n_prefix=64, padded=True),
    W("bpad_d64", 1, 3, 64, (9, 13, 10), 7, seed=52, padded=True),
    W("bpad_tile2x4x8", 1, 2, 128, (7, 9, 20), 4, seed=53, tile=(2, 4, 8), padded=True),
    W("bpad_keep_all", 1, 1, 128, (6, 5, 9), 12, seed=54, n_prefix=128, padded=True),
]


def raster_to_tiled_rows(perm1, npf):
    """tiled slot of every raster row (prefix first), for one batch element"""
    real_slots = np.nonzero(perm1 >= 0)[0]
    src = np.empty(npf + real_slots.size, np.int64)
    src[:npf] = np.arange(npf)
    src[npf + perm1[real_slots]] = npf + real_slots
    return src


def check_grad(got, ref, what):
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    ref_mx, ref_mean = float(np.abs(ref).max()), float(np.abs(ref).mean())
    print(f"[{what}] max|err| {mx:.3e} (ref max {ref_mx:.3e}), mean|err| {mean:.3e} (ref mean {ref_mean:.3e})",
          flush=True)
    assert np.isfinite(got).all(), what
    assert mx <= 2e-2 * ref_mx + 1e-6, what
    assert mean <= 1e-2 * ref_mean + 1e-7, what


def run_padded_backward(wl):
    q, k, v = S.qkv(wl)
    do = S.tensor(wl, "do")
    g = DeviceRun(wl, q, k, v).run()
    dq, dk, dv = (torch.empty_like(g.q) for _ in range(3))
    ws = torch.empty(max(bsa.backward_workspace_size(g.desc), 256), dtype=torch.uint8, device="cuda")
    bsa.backward(g.desc, g.q, g.k, g.v, g.out, to_dev(do), g.att.lse, g.att.perm, g.att.block_idx, dq, dk, dv, ws)
    torch.cuda.synchronize()
    return (q, k, v, do), g, (dq, dk, dv)


@pytest.mark.parametrize("wl", BWD_CASES, ids=[c.name for c in BWD_CASES])
def test_padded_backward_matches_oracle(wl):
    """dQ, dK, dV on the raster rows against the oracle's gradients of the
    padded forward (real keys, real queries), with the GPU's selection."""
    print(f"\n[case] {wl}", flush=True)
    (q, k, v, do), g, grads = run_padded_backward(wl)
    npf, scale = wl.n_prefix, float(np.float32(wl.scale))
    p1 = oracle.perm_static_padded(wl.grid, wl.tile)
    tiled = [oracle.gather_padded(x, p1, npf) for x in (q, k, v, do)]
    real = np.broadcast_to(oracle.key_real(p1, npf), (wl.batch, npf + p1.size))
    ref = oracle.backward_full_padded(*tiled, npf, g.block_idx(), real, scale)
    src = raster_to_tiled_rows(p1, npf)
    for name, dev, r in zip(("dq", "dk", "dv"), grads, ref):
        got = bits_to_f64(to_bits(dev))                      # raster [B, Nras, H, D]
        check_grad(got, r[:, :, src].transpose(0, 2, 1, 3), name)


def test_prism720p_ragged_backward_sampled():
    """Full size (31 x 45 x 80 padded to 32 x 48 x 80, batch 2, 24 heads,
    head_dim 128, keep 480): dQ of sampled query tiles entirely from the
    oracle; dK, dV of sampled key tiles also entirely from the oracle (its
    forward on the query tiles that attend them, about 480 per key tile, for
    their lse and Delta = dO . O).  Boundary tiles among the samples."""
    wl = S.WORKLOADS["prism720p_ragged"]
    print(f"\n[case] {wl}", flush=True)
    (q, k, v, do), g, grads = run_padded_backward(wl)
    npf, scale = wl.n_prefix, float(np.float32(wl.scale))
    p1 = oracle.perm_static_padded(wl.grid, wl.tile)
    real = oracle.key_real(p1, npf)
    nqt = wl.n_tiled_tokens // 64
    gidx = g.block_idx()
    lse_gpu = g.att.lse.cpu().numpy()
    for b, h in [(0, 5), (1, 22)]:
        sl = lambda x: np.ascontiguousarray(x[b:b + 1, :, h:h + 1])
        qt, kt, vt, dot = (oracle.gather_padded(sl(x), p1, npf)[0, 0] for x in (q, k, v, do))
        gt = [bits_to_f64(oracle.gather_padded(to_bits(x[b:b + 1, :, h:h + 1]), p1, npf)[0, 0])
              .reshape(nqt, 64, wl.head_dim) for x in grads]
        rows = real.reshape(nqt, 64).astype(bool)
        qtiles = np.array([5, 1919, 1900, 959], np.int32)   # 1919, 1900, 959: boundary tiles
        o_ref, lse_ref = oracle.attention_padded(qt, kt, vt, npf, gidx[b, h], real, scale, qtiles)
        lse = np.zeros(wl.n_tiled_tokens)
        delta = np.zeros(wl.n_tiled_tokens)
        qrows = (qtiles[:, None] * 64 + np.arange(64)).reshape(-1)
        lse[qrows] = lse_ref.reshape(-1)
        delta[qrows] = (o_ref.reshape(-1, wl.head_dim) * bits_to_f64(dot)[qrows]).sum(1)
        ref_dq = oracle.backward_dq_padded(qt, kt, vt, dot, lse, delta, npf, gidx[b, h], real, scale, qtiles)
        check_grad(gt[0][qtiles][rows[qtiles]], ref_dq[rows[qtiles]], f"dq b{b} h{h}")
        ktiles = np.array([1919, 1000], np.int32)
        need = attending_tiles(ktiles, wl.n_prefix_tiles, wl.n_video_tiles, idx=gidx[b, h])
        lse_all, delta_all, rr = oracle_lse_delta_rows(
            lambda t: oracle.attention_padded(qt, kt, vt, npf, gidx[b, h], real, scale, t), need, dot,
            wl.n_tiled_tokens, wl.head_dim)
        lrows = rows[need].reshape(-1)   # the real query rows among them
        check_lse(lse_gpu[b, h].reshape(nqt, 64)[need].reshape(-1)[lrows], lse_all[rr][lrows],
                  qt.reshape(nqt, 64, -1)[need].reshape(-1, wl.head_dim)[lrows], kt, scale,
                  f"lse b{b} h{h} (extra check)")
        ref_dk, ref_dv = oracle.backward_dkdv_padded(qt, kt, vt, dot, lse_all, delta_all, npf, gidx[b, h], real,
                                                     scale, ktiles)
        check_grad(gt[1][ktiles][rows[ktiles]], ref_dk[rows[ktiles]], f"dk b{b} h{h}")
        check_grad(gt[2][ktiles][rows[ktiles]], ref_dv[rows[ktiles]], f"dv b{b} h{h}")
    del g, grads
    torch.cuda.empty_cache()


def test_padded_csr_and_structured_lists():
    """Ragged grid with CSR lists (per-head keeps) and with structured lists
    (spatial radius 0, temporal radius 2 on a 2 x 3 x 3 tile grid): the CSR
    forward against the oracle's masked CSR attention on the real rows, and
    the CSR backward against the oracle's masked gradients (each head's rows
    have one length, so they are fixed-keep lists for the oracle)."""
    wl = W("pad_csr", 1, 2, 128, (7, 9, 10), 5, seed=48, n_prefix=64, padded=True)
    q, k, v = S.qkv(wl)
    do = S.tensor(wl, "do")
    g = DeviceRun(wl, q, k, v).run()
    a, d = g.att, g.desc
    npf, scale, D = wl.n_prefix, float(np.float32(wl.scale)), wl.head_dim
    p1 = oracle.perm_static_padded(wl.grid, wl.tile)
    real = oracle.key_real(p1, npf)
    tiled = [oracle.gather_padded(x, p1, npf) for x in (q, k, v, do)]
    qt, kt, vt, dot = tiled
    n = wl.n_video_tiles
    nqt = wl.n_tiled_tokens // 64
    rows_real = real.reshape(nqt, 64).astype(bool)
    tiles = np.arange(nqt, dtype=np.int32)
    src = raster_to_tiled_rows(p1, npf)
    lists = {}
    row_ptr = torch.empty(wl.batch * wl.heads * n + 1, dtype=torch.int64, device="cuda")
    col = torch.empty(bsa.csr_entries(d, [5, 2]), dtype=torch.int32, device="cuda")
    bsa.plan_csr(d, a.q_t, a.k_f, row_ptr, col, a.workspace, keep_per_head=[5, 2])
    lists["csr"] = (row_ptr, col)
    mask = [bsa.MASK_SPATIAL, bsa.MASK_TEMPORAL]
    rp2 = torch.empty_like(row_ptr)
    col2 = torch.empty(bsa.structured_entries(d, mask, 0, 2), dtype=torch.int32, device="cuda")
    bsa.plan_structured(d, mask, 0, 2, rp2, col2)  # full rows: one length per head
    lists["structured"] = (rp2, col2)
    for name, (rp, cl) in lists.items():
        print(f"\n[case] {wl} {name} lists", flush=True)
        o_t = torch.empty_like(a.q_t)
        lse = torch.empty_like(a.lse)
        bsa.forward_csr(d, a.q_t, a.k_f, a.v_f, rp, cl, o_t, lse, workspace=a.workspace)
        out = torch.empty_like(g.q)
        bsa.scatter(d, o_t, out, a.perm)
        dq, dk, dv = (torch.empty_like(g.q) for _ in range(3))
        ws = torch.empty(bsa.backward_csr_workspace_size(d, cl.numel()), dtype=torch.uint8, device="cuda")
        bsa.backward_csr(d, g.q, g.k, g.v, out, to_dev(do), lse, a.perm, rp, cl, dq, dk, dv, ws)
        torch.cuda.synchronize()
        rp_h, cl_h = rp.cpu().numpy(), cl.cpu().numpy()
        o_bits, lse_h = to_bits(o_t), lse.cpu().numpy()
        for h in range(wl.heads):
            r0 = h * n
            rph = rp_h[r0:r0 + n + 1] - rp_h[r0]
            clh = cl_h[rp_h[r0]:rp_h[r0 + n]]
            ref, ref_lse = oracle.attention_padded_csr(qt[0, h], kt[0, h], vt[0, h], npf, rph, clh, real, scale,
                                                       tiles)
            check_output(o_bits[0, h].reshape(nqt, 64, D)[rows_real], ref[rows_real], f"{name} h{h}")
            check_lse(lse_h[0, h].reshape(nqt, 64)[rows_real], ref_lse[rows_real],
                      qt[0, h].reshape(nqt, 64, D)[rows_real], kt[0, h], scale, f"{name} lse h{h}")
        grads_ref = padded_csr_gradients(qt, kt, vt, dot, npf, rp_h, cl_h, real, scale, wl.heads, n)
        for gname, dev, r in zip(("dq", "dk", "dv"), (dq, dk, dv), grads_ref):
            check_grad(bits_to_f64(to_bits(dev)), r[:, :, src].transpose(0, 2, 1, 3), f"{name} {gname}")
    del g
    torch.cuda.empty_cache()


def padded_csr_gradients(qt, kt, vt, dot, npf, row_ptr, col, real, scale, H, n):
    """The oracle's masked gradients over CSR lists whose rows are of one
    length per head (per-head keeps, or structured rules that keep full
    rows): each head's rows are a fixed-keep list."""
    B, _, Ntot, D = qt.shape
    out = [np.zeros((B, H, Ntot, D)) for _ in range(3)]
    for h in range(H):
        r0 = h * n
        lens = np.diff(row_ptr[r0:r0 + n + 1])
        assert (lens == lens[0]).all()
        idx = col[row_ptr[r0]:row_ptr[r0 + n]].reshape(n, int(lens[0]))
        g = oracle.backward_full_padded(qt[:, h:h + 1], kt[:, h:h + 1], vt[:, h:h + 1], dot[:, h:h + 1], npf,
                                        idx[None, None], real[None], scale)
        for o, x in zip(out, g):
            o[:, h] = x[:, 0]
    return out
