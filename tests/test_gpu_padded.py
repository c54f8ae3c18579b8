"""GPU parity of ragged grids (BSA_TILE_STATIC_PADDED): a video grid that is
not a whole number of static tiles, covered by the tile grid rounded up.

* permutation (-1 in padding slots), gathers (zeros there), scatter: bit-exact;
* tile means over the real tokens only: bit-exact;
* kept tiles: the selection rules of the other parity tests;
* attention over the real keys only (boundary tiles masked), on the real
  query rows, with the forward's output and lse tolerances;
* on a grid that divides, padded mode is the plain static path bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from parity import GpuRun, check_lse, check_output, check_selection, kfrag_layout, to_bits, vfrag_layout

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
        n_exact, n_near = check_selection(gidx[b:b + 1, h:h + 1], qp, kp, wl.keep_tiles)
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
    g = GpuRun(wl, q, k, v).run()
    perm, worst = check_padded_path(wl, g, q, k, v)
    # scatter: the real rows back to raster order, padding slots dropped
    ref_out = oracle.scatter_padded(to_bits(g.att.o_t), perm, wl.n_prefix, wl.n_video)
    assert np.array_equal(to_bits(g.out), ref_out)
    print(f"[forward] worst max|err| {worst:.3e}", flush=True)


def test_padded_mode_on_divisible_grid_is_static_path():
    base = W("pad_div", 2, 2, 128, (8, 8, 12), 5, seed=47, n_prefix=64)
    q, k, v = S.qkv(base)
    g1 = GpuRun(base, q, k, v).run()
    g2 = GpuRun(W("pad_div", 2, 2, 128, (8, 8, 12), 5, seed=47, n_prefix=64, padded=True), q, k, v).run()
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
    g = GpuRun(wl, q, k, v).run()
    nqt = wl.n_tiled_tokens // 64
    rng = np.random.default_rng(91)
    # tiles of the last t-layer and last h-row are boundary tiles (31 = 7*4 + 3, 45 = 11*4 + 1)
    boundary = np.array([1919, 1900, 1500, 79 + 80 * 11], np.int32)
    tiles = np.unique(np.concatenate([boundary, rng.choice(nqt, size=12, replace=False)])).astype(np.int32)
    check_padded_path(wl, g, q, k, v, qtiles=tiles, bh=[(0, 0), (1, 13)])
    del g
    torch.cuda.empty_cache()
