"""Pins of the oracle's ragged-grid path: a video grid that is not a whole
number of static tiles, covered by the tile grid rounded up, its boundary
tiles partly padding (Sparse VideoGen page, section on theoretical and
physical sparsity: full, boundary and empty tiles; Prism page, section on the
quadratic cost: the 720p grid counts padding tokens).

* Permutation: equal to the tile order built by numpy from the padded raster
  index grid (pad with -1, split every axis into tiles, tile axes first); the
  plain static permutation when the grid divides.
* Gather / scatter: padding slots are zeros; the round trip is the identity.
* Tile means: the mean over real tokens (numpy, float64), unchanged by any
  value written into padding slots; the plain means for full tiles.
* Attention: torch's float64 scaled_dot_product_attention under an explicit
  mask (kept tiles and prefix, real keys only); unchanged by padding-slot
  contents; identical to the CSR attention without padding.  With every tile
  kept, the whole path (gather, attention, scatter) is dense attention over
  the real tokens in raster order.
* Gradients: torch autograd of the same masked fp64 attention (loss = sum of
  O * dO, dO zero on padding rows); zero dK, dV on padding key rows; real
  rows unchanged by padding-slot contents; with every tile kept, autograd of
  dense attention over the real tokens in raster order.
"""
import numpy as np
import pytest
import torch

from synthetic import bf16_bits_to_f32, to_bf16_bits

GRIDS = [((5, 6, 7), (4, 4, 4)), ((9, 4, 13), (2, 4, 8)), ((3, 17, 2), (16, 2, 2)), ((8, 8, 8), (4, 4, 4))]


def _numpy_perm(grid, tile):
    T, H, W = grid
    tt, th, tw = tile
    Tp, Hp, Wp = (-(-g // t) * t for g, t in zip(grid, tile))
    idx = np.pad(np.arange(T * H * W, dtype=np.int32).reshape(T, H, W), ((0, Tp - T), (0, Hp - H), (0, Wp - W)),
                 constant_values=-1)
    x = idx.reshape(Tp // tt, tt, Hp // th, th, Wp // tw, tw).transpose(0, 2, 4, 1, 3, 5)
    return x.reshape(-1)


@pytest.mark.parametrize("grid,tile", GRIDS)
def test_perm_matches_numpy_tiling(orc, grid, tile):
    p = orc.perm_static_padded(grid, tile)
    assert np.array_equal(p, _numpy_perm(grid, tile))
    real = p[p >= 0]
    assert np.array_equal(np.sort(real), np.arange(np.prod(grid)))
    if all(g % t == 0 for g, t in zip(grid, tile)):
        assert np.array_equal(p, orc.perm_static(grid, tile))


def _rand_bits(rng, shape, scale=1.0):
    return to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * scale)


def test_gather_scatter_round_trip(orc):
    rng = np.random.default_rng(81)
    grid, tile, npf, B, H, D = (5, 6, 7), (4, 4, 4), 64, 2, 3, 16
    nr = int(np.prod(grid))
    x = _rand_bits(rng, (B, npf + nr, H, D))
    p = orc.perm_static_padded(grid, tile)
    t = orc.gather_padded(x, p, npf)
    assert t.shape == (B, H, npf + p.size, D)
    pad_rows = npf + np.nonzero(p < 0)[0]
    assert not t[:, :, pad_rows].any()
    real_slots = np.nonzero(p >= 0)[0]
    assert np.array_equal(t[:, :, npf + real_slots], x[:, npf + p[real_slots]].transpose(0, 2, 1, 3))
    assert np.array_equal(orc.scatter_padded(t, p, npf, nr), x)
    # a divisible grid: the plain gather
    p8 = orc.perm_static_padded((8, 8, 8), tile)
    x8 = _rand_bits(rng, (1, 512, 2, 8))
    assert np.array_equal(orc.gather_padded(x8, p8, 0), orc.gather(x8, orc.perm_static((8, 8, 8), tile), 0))


def test_pool_real_tokens_only(orc):
    rng = np.random.default_rng(82)
    grid, tile, npf, B, H, D = (5, 6, 7), (4, 4, 4), 128, 2, 2, 8
    x = _rand_bits(rng, (B, npf + int(np.prod(grid)), H, D), 2.0)
    p = orc.perm_static_padded(grid, tile)
    t = orc.gather_padded(x, p, npf)
    got = orc.pool_padded(t, p, npf)
    nvt = p.size // 64
    vals = bf16_bits_to_f32(t[:, :, npf:]).astype(np.float64).reshape(B, H, nvt, 64, D)
    real = (p >= 0).reshape(nvt, 64)
    ref = np.stack([vals[:, :, i][:, :, real[i]].mean(axis=2) for i in range(nvt)], axis=2).astype(np.float32)
    assert np.array_equal(got, ref)
    # padding-slot contents do not matter
    t2 = t.copy()
    t2[:, :, npf + np.nonzero(p < 0)[0]] = _rand_bits(rng, (B, H, int((p < 0).sum()), D), 50.0)
    assert np.array_equal(orc.pool_padded(t2, p, npf), got)
    # full tiles: the plain 64-token mean
    full = np.nonzero(real.all(axis=1))[0]
    assert full.size > 0
    assert np.array_equal(got[:, :, full], orc.pool(t, npf)[:, :, full])


def _f64(bits):
    return torch.from_numpy(bf16_bits_to_f32(bits).astype(np.float64))


def _mask(npf, nvt, row_ptr, col, real):
    N = npf + nvt * 64
    m = np.zeros((N, N), bool)
    m[:npf, :] = True
    m[npf:, :npf] = True
    for i in range(nvt):
        for j in col[row_ptr[i]:row_ptr[i + 1]]:
            m[npf + i * 64: npf + (i + 1) * 64, npf + j * 64: npf + (j + 1) * 64] = True
    return m & real.astype(bool)[None, :]


@pytest.mark.parametrize("grid,tile,npf,D", [((5, 6, 7), (4, 4, 4), 64, 16), ((9, 4, 13), (2, 4, 8), 0, 8)])
def test_attention_matches_masked_sdpa(orc, grid, tile, npf, D):
    rng = np.random.default_rng(83 + D)
    p = orc.perm_static_padded(grid, tile)
    nvt = p.size // 64
    N = npf + p.size
    q, k, v = (orc.gather_padded(_rand_bits(rng, (1, npf + int(np.prod(grid)), 1, D), 1.5), p, npf)[0, 0]
               for _ in range(3))
    lens = rng.integers(1, nvt + 1, size=nvt)
    row_ptr = np.zeros(nvt + 1, np.int64)
    row_ptr[1:] = np.cumsum(lens)
    col = np.concatenate([np.sort(rng.choice(nvt, size=n, replace=False)) for n in lens]).astype(np.int32)
    real = orc.key_real(p, npf)
    scale = 0.3
    tiles = np.arange(N // 64, dtype=np.int32)
    out, lse = orc.attention_padded_csr(q, k, v, npf, row_ptr, col, real, scale, tiles)
    m = torch.from_numpy(_mask(npf, nvt, row_ptr, col, real))
    qq, kk, vv = (_f64(x)[None, None] for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=m[None, None], scale=scale)[0, 0]
    np.testing.assert_allclose(out.reshape(N, D), ref.numpy(), rtol=0, atol=1e-12)
    logits = (_f64(q) @ _f64(k).T) * scale
    ref_lse = torch.logsumexp(logits.masked_fill(~m, -np.inf), 1).numpy()
    np.testing.assert_allclose(lse.reshape(N), ref_lse, rtol=0, atol=1e-12)
    # padding-slot contents of K and V do not matter
    pad = npf + np.nonzero(p < 0)[0]
    k2, v2 = k.copy(), v.copy()
    k2[pad] = _rand_bits(rng, (pad.size, D), 30.0)
    v2[pad] = _rand_bits(rng, (pad.size, D), 30.0)
    out2, lse2 = orc.attention_padded_csr(q, k2, v2, npf, row_ptr, col, real, scale, tiles)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_attention_without_padding_is_csr(orc):
    rng = np.random.default_rng(84)
    D, npf, nvt = 16, 64, 5
    N = npf + nvt * 64
    q, k, v = (_rand_bits(rng, (N, D)) for _ in range(3))
    lens = rng.integers(1, nvt + 1, size=nvt)
    row_ptr = np.zeros(nvt + 1, np.int64)
    row_ptr[1:] = np.cumsum(lens)
    col = np.concatenate([np.sort(rng.choice(nvt, size=n, replace=False)) for n in lens]).astype(np.int32)
    tiles = np.arange(N // 64, dtype=np.int32)
    o1, l1 = orc.attention_csr(q, k, v, npf, row_ptr, col, 0.25, tiles)
    o2, l2 = orc.attention_padded_csr(q, k, v, npf, row_ptr, col, np.ones(N, np.uint8), 0.25, tiles)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_all_tiles_kept_is_dense_attention_on_real_tokens(orc):
    rng = np.random.default_rng(85)
    grid, tile, npf, D = (6, 5, 9), (4, 4, 4), 64, 16
    nr = int(np.prod(grid))
    x = [_rand_bits(rng, (1, npf + nr, 1, D), 1.5) for _ in range(3)]
    p = orc.perm_static_padded(grid, tile)
    nvt = p.size // 64
    qt, kt, vt = (orc.gather_padded(a, p, npf)[0, 0] for a in x)
    idx = np.tile(np.arange(nvt, dtype=np.int32), (nvt, 1))
    out, _ = orc.attention_padded(qt, kt, vt, npf, idx, orc.key_real(p, npf), 0.25,
                                  np.arange((npf + p.size) // 64, dtype=np.int32))
    # back to raster order through the permutation (real slots only)
    o_ras = np.zeros((npf + nr, D))
    o_t = out.reshape(npf + p.size, D)
    o_ras[:npf] = o_t[:npf]
    real_slots = np.nonzero(p >= 0)[0]
    o_ras[npf + p[real_slots]] = o_t[npf + real_slots]
    qq, kk, vv = (_f64(a[0, :, 0])[None, None] for a in x)
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=0.25)[0, 0]
    np.testing.assert_allclose(o_ras, ref.numpy(), rtol=0, atol=1e-12)


# ---- gradients on a ragged grid ------------------------------------------------

def _autograd(q, k, v, do, mask, scale):
    qq, kk, vv = (_f64(x).requires_grad_(True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(qq[None, None], kk[None, None], vv[None, None],
                                                           attn_mask=None if mask is None else
                                                           torch.from_numpy(mask)[None, None], scale=scale)[0, 0]
    (out * _f64(do)).sum().backward()
    return qq.grad.numpy(), kk.grad.numpy(), vv.grad.numpy()


@pytest.mark.parametrize("grid,tile,npf,D,keep", [((5, 6, 7), (4, 4, 4), 64, 16, 3), ((9, 4, 13), (2, 4, 8), 0, 8, 2)])
def test_gradients_match_masked_autograd(orc, grid, tile, npf, D, keep):
    """Kept lists and real keys as an explicit token mask on the tiled order;
    dO is zero on padding rows (they carry no loss), as the gathered dO is."""
    rng = np.random.default_rng(86 + D)
    p = orc.perm_static_padded(grid, tile)
    nvt = p.size // 64
    nr = int(np.prod(grid))
    q, k, v, do = (orc.gather_padded(_rand_bits(rng, (1, npf + nr, 1, D), 1.5), p, npf)[0, 0] for _ in range(4))
    idx = np.stack([np.sort(rng.choice(nvt, size=keep, replace=False)) for _ in range(nvt)]).astype(np.int32)
    real = orc.key_real(p, npf)
    scale = 0.3
    dq, dk, dv = (x[0, 0] for x in orc.backward_full_padded(q[None, None], k[None, None], v[None, None],
                                                             do[None, None], npf, idx[None, None], real[None], scale))
    row_ptr = np.arange(nvt + 1, dtype=np.int64) * keep
    m = _mask(npf, nvt, row_ptr, idx.reshape(-1), real)
    rq, rk, rv = _autograd(q, k, v, do, m, scale)
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)
    assert not dk[real == 0].any() and not dv[real == 0].any()
    # padding-slot contents of Q, K, V do not change the real rows' gradients
    pad = np.nonzero(real == 0)[0]
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for x in (q2, k2, v2):
        x[pad] = _rand_bits(rng, (pad.size, D), 20.0)
    g2 = [x[0, 0] for x in orc.backward_full_padded(q2[None, None], k2[None, None], v2[None, None], do[None, None],
                                                    npf, idx[None, None], real[None], scale)]
    r = real == 1
    for a, b in zip((dq, dk, dv), g2):
        assert np.array_equal(a[r], b[r])


def test_all_tiles_kept_gradients_are_dense_autograd_on_real_tokens(orc):
    rng = np.random.default_rng(87)
    grid, tile, npf, D = (6, 5, 9), (4, 4, 4), 64, 16
    nr = int(np.prod(grid))
    x = [_rand_bits(rng, (1, npf + nr, 1, D), 1.5) for _ in range(4)]
    p = orc.perm_static_padded(grid, tile)
    nvt = p.size // 64
    qt, kt, vt, dt = (orc.gather_padded(a, p, npf) for a in x)
    idx = np.tile(np.arange(nvt, dtype=np.int32), (nvt, 1))
    grads = orc.backward_full_padded(qt, kt, vt, dt, npf, idx[None, None], orc.key_real(p, npf)[None], 0.25)
    ref = _autograd(*(a[0, :, 0] for a in x), None, 0.25)
    real_slots = np.nonzero(p >= 0)[0]
    for g, r in zip(grads, ref):
        back = np.zeros((npf + nr, D))
        back[:npf] = g[0, 0, :npf]
        back[npf + p[real_slots]] = g[0, 0, npf + real_slots]
        np.testing.assert_allclose(back, r, rtol=0, atol=1e-11)
