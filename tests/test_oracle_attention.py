"""Pins of the oracle's attention over kept tiles.

* k = n reduces to dense softmax attention: checked against torch's
  scaled_dot_product_attention in float64 on the CPU (a library routine the
  oracle does not use).
* Brute force on tiny grids: an explicit token-by-token boolean mask built from
  the selection (prefix rows dense, video rows see the prefix and their kept
  tiles -- Ref2VA VSA page, section on conditioning tokens) through the same
  library routine.
* Closed forms: constant V gives constant output; k = 1 with V constant per
  tile gives that tile's constant.
"""
import numpy as np
import pytest
import torch

from synthetic import bf16_bits_to_f32, to_bf16_bits


def _rand_tiled(rng, n_tok, D, scale=1.0):
    return to_bf16_bits(rng.standard_normal((n_tok, D)).astype(np.float32) * scale)


def _f64(x):
    return torch.from_numpy(bf16_bits_to_f32(x).astype(np.float64))


def _sdpa(q, k, v, scale, mask=None):
    qq, kk, vv = (t.unsqueeze(0).unsqueeze(0) for t in (q, k, v))
    m = None if mask is None else torch.from_numpy(mask).unsqueeze(0).unsqueeze(0)
    return torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=m, scale=scale)[0, 0]


@pytest.mark.parametrize("D,npf,nvt", [(8, 0, 6), (64, 128, 5), (128, 64, 3)])
def test_k_equals_n_is_dense_attention(orc, D, npf, nvt):
    rng = np.random.default_rng(D + npf)
    N = npf + nvt * 64
    q, k, v = (_rand_tiled(rng, N, D) for _ in range(3))
    idx = np.tile(np.arange(nvt, dtype=np.int32), (nvt, 1))
    scale = 1.0 / np.sqrt(D)
    out, lse = orc.attention(q, k, v, npf, idx, scale, np.arange(N // 64, dtype=np.int32))
    ref = _sdpa(_f64(q), _f64(k), _f64(v), scale).numpy()
    np.testing.assert_allclose(out.reshape(N, D), ref, rtol=0, atol=1e-12)
    logits = (_f64(q) @ _f64(k).T) * scale
    np.testing.assert_allclose(lse.reshape(N), torch.logsumexp(logits, 1).numpy(), rtol=0, atol=1e-12)


def _mask_from_selection(npf, nvt, idx):
    N = npf + nvt * 64
    m = np.zeros((N, N), bool)
    m[:npf, :] = True                     # prefix queries: dense
    m[npf:, :npf] = True                  # every video query sees the prefix
    for i in range(nvt):
        rows = slice(npf + i * 64, npf + (i + 1) * 64)
        for j in idx[i]:
            m[rows, npf + j * 64: npf + (j + 1) * 64] = True
    return m


@pytest.mark.parametrize("D,npf,nvt,k", [(8, 0, 8, 3), (64, 0, 8, 1), (16, 128, 6, 2), (64, 64, 5, 4)])
def test_brute_force_masked_attention(orc, D, npf, nvt, k):
    rng = np.random.default_rng(100 + D + k)
    N = npf + nvt * 64
    q, kx, v = (_rand_tiled(rng, N, D, 2.0) for _ in range(3))
    idx = np.stack([np.sort(rng.choice(nvt, size=k, replace=False)) for _ in range(nvt)]).astype(np.int32)
    scale = 0.3
    out, lse = orc.attention(q, kx, v, npf, idx, scale, np.arange(N // 64, dtype=np.int32))
    mask = _mask_from_selection(npf, nvt, idx)
    ref = _sdpa(_f64(q), _f64(kx), _f64(v), scale, mask).numpy()
    np.testing.assert_allclose(out.reshape(N, D), ref, rtol=0, atol=1e-12)
    logits = (_f64(q) @ _f64(kx).T).numpy() * scale
    logits[~mask] = -np.inf
    np.testing.assert_allclose(lse.reshape(N), torch.logsumexp(torch.from_numpy(logits), 1).numpy(),
                               rtol=0, atol=1e-12)


def test_query_tile_subset(orc):
    rng = np.random.default_rng(9)
    D, npf, nvt, k = 16, 64, 4, 2
    N = npf + nvt * 64
    q, kx, v = (_rand_tiled(rng, N, D) for _ in range(3))
    idx = np.array([[0, 1], [1, 3], [0, 2], [2, 3]], np.int32)
    full, _ = orc.attention(q, kx, v, npf, idx, 0.25, np.arange(5, dtype=np.int32))
    sub, _ = orc.attention(q, kx, v, npf, idx, 0.25, np.array([3, 0], np.int32))
    np.testing.assert_array_equal(sub[0], full[3])
    np.testing.assert_array_equal(sub[1], full[0])


def test_constant_v_gives_constant_output(orc):
    rng = np.random.default_rng(10)
    D, npf, nvt, k = 32, 64, 5, 2
    N = npf + nvt * 64
    q, kx = (_rand_tiled(rng, N, D, 3.0) for _ in range(2))
    v = to_bf16_bits(np.full((N, D), -1.25, np.float32))
    idx = np.stack([np.sort(rng.choice(nvt, size=k, replace=False)) for _ in range(nvt)]).astype(np.int32)
    out, _ = orc.attention(q, kx, v, npf, idx, 0.2, np.arange(N // 64, dtype=np.int32))
    np.testing.assert_allclose(out, -1.25, rtol=0, atol=1e-13)


def test_single_kept_tile_with_tilewise_constant_v(orc):
    rng = np.random.default_rng(12)
    D, nvt = 16, 6
    N = nvt * 64
    q, kx = (_rand_tiled(rng, N, D, 3.0) for _ in range(2))
    const = np.arange(nvt, dtype=np.float32) * 0.5 - 1.0
    v = to_bf16_bits(np.repeat(const, 64)[:, None] * np.ones((1, D), np.float32))
    idx = rng.integers(0, nvt, size=(nvt, 1)).astype(np.int32)
    out, _ = orc.attention(q, kx, v, 0, idx, 0.2, np.arange(nvt, dtype=np.int32))
    for i in range(nvt):
        np.testing.assert_allclose(out[i], const[idx[i, 0]], rtol=0, atol=1e-13)


def test_end_to_end_reference_dense_limit(orc):
    """The whole raster -> raster path at k = n equals dense attention on the
    raster sequence: permutation, pooling and selection then cancel out."""
    import synthetic as S
    wl = S.Workload("t", 1, 2, 16, (4, 8, 8), 4, seed=2, n_prefix=64)
    q, k, v = S.qkv(wl)
    res = orc.reference(q, k, v, grid=wl.grid, n_prefix=wl.n_prefix, k=wl.n_video_tiles, scale=0.25)
    for h in range(wl.heads):
        ref = _sdpa(_f64(q[0, :, h]), _f64(k[0, :, h]), _f64(v[0, :, h]), 0.25).numpy()
        np.testing.assert_allclose(res["o"][0, :, h], ref, rtol=0, atol=1e-12)
