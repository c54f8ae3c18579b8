"""Pins of the oracle's gradients of attention over kept tiles.

The gradients are the plain derivative of the function the oracle's forward
computes.  They are pinned against:

* torch autograd through scaled_dot_product_attention in float64 on the CPU
  (a library routine the oracle does not use): dense (k = n) and with an
  explicit token-by-token boolean mask built from the selection (prefix rows
  dense, video rows see the prefix and their kept tiles -- Ref2VA VSA page,
  section on conditioning tokens);
* invariants that hold for any inputs: the weights of every query add up to 1,
  so the dV rows add up to the sum of the dO rows, and each query's dS row adds
  up to 0, so the dK rows add up to 0;
* a closed form: constant V leaves dQ and dK at 0.
"""
import numpy as np
import pytest
import torch

from synthetic import bf16_bits_to_f32, to_bf16_bits


def _rand(rng, n_tok, D, scale=1.0):
    return to_bf16_bits(rng.standard_normal((n_tok, D)).astype(np.float32) * scale)


def _f64(x):
    return torch.from_numpy(bf16_bits_to_f32(x).astype(np.float64))


def _mask_from_selection(npf, nvt, idx):
    N = npf + nvt * 64
    m = np.zeros((N, N), bool)
    m[:npf, :] = True
    m[npf:, :npf] = True
    for i in range(nvt):
        rows = slice(npf + i * 64, npf + (i + 1) * 64)
        for j in idx[i]:
            m[rows, npf + j * 64: npf + (j + 1) * 64] = True
    return m


def _autograd(q, k, v, do, scale, mask=None):
    qq, kk, vv = (_f64(x).requires_grad_(True) for x in (q, k, v))
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qq[None, None], kk[None, None], vv[None, None],
                                                         attn_mask=m, scale=scale)[0, 0]
    o.backward(_f64(do))
    return qq.grad.numpy(), kk.grad.numpy(), vv.grad.numpy()


def _oracle_grads(orc, q, k, v, do, npf, idx, scale):
    N, D = q.shape
    dq, dk, dv = orc.backward_full(q[None, None], k[None, None], v[None, None], do[None, None], npf,
                                   None if idx is None else idx[None, None], scale)
    return dq[0, 0], dk[0, 0], dv[0, 0]


@pytest.mark.parametrize("D,npf,nvt", [(8, 0, 4), (64, 128, 3)])
def test_k_equals_n_is_dense_backward(orc, D, npf, nvt):
    rng = np.random.default_rng(200 + D)
    N = npf + nvt * 64
    q, k, v, do = (_rand(rng, N, D) for _ in range(4))
    idx = np.tile(np.arange(nvt, dtype=np.int32), (nvt, 1))
    scale = 1.0 / np.sqrt(D)
    got = _oracle_grads(orc, q, k, v, do, npf, idx, scale)
    ref = _autograd(q, k, v, do, scale)
    for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-12, err_msg=name)


@pytest.mark.parametrize("D,npf,nvt,k", [(8, 0, 6, 2), (16, 64, 5, 3), (64, 0, 4, 1)])
def test_brute_force_masked_backward(orc, D, npf, nvt, k):
    rng = np.random.default_rng(300 + D + k)
    N = npf + nvt * 64
    q, kx, v, do = (_rand(rng, N, D, 1.5) for _ in range(4))
    idx = np.stack([np.sort(rng.choice(nvt, size=k, replace=False)) for _ in range(nvt)]).astype(np.int32)
    scale = 0.3
    got = _oracle_grads(orc, q, kx, v, do, npf, idx, scale)
    ref = _autograd(q, kx, v, do, scale, _mask_from_selection(npf, nvt, idx))
    for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-11, err_msg=name)


def test_gradient_sums(orc):
    rng = np.random.default_rng(41)
    D, npf, nvt, k = 16, 64, 6, 2
    N = npf + nvt * 64
    q, kx, v, do = (_rand(rng, N, D) for _ in range(4))
    idx = np.stack([np.sort(rng.choice(nvt, size=k, replace=False)) for _ in range(nvt)]).astype(np.int32)
    dq, dk, dv = _oracle_grads(orc, q, kx, v, do, npf, idx, 0.25)
    np.testing.assert_allclose(dv.sum(0), bf16_bits_to_f32(do).astype(np.float64).sum(0), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dk.sum(0), 0.0, rtol=0, atol=1e-10)


def test_constant_v_leaves_dq_dk_zero(orc):
    rng = np.random.default_rng(42)
    D, npf, nvt, k = 8, 0, 5, 2
    N = nvt * 64
    q, kx, do = (_rand(rng, N, D) for _ in range(3))
    v = np.tile(to_bf16_bits(rng.standard_normal((1, D)).astype(np.float32)), (N, 1))
    idx = np.stack([np.sort(rng.choice(nvt, size=k, replace=False)) for _ in range(nvt)]).astype(np.int32)
    dq, dk, dv = _oracle_grads(orc, q, kx, v, do, npf, idx, 0.5)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    assert np.abs(dv).max() > 1e-3


def test_sampled_tiles_match_full(orc):
    rng = np.random.default_rng(43)
    D, npf, nvt, k = 16, 128, 5, 3
    N = npf + nvt * 64
    q, kx, v, do = (_rand(rng, N, D) for _ in range(4))
    idx = np.stack([np.sort(rng.choice(nvt, size=k, replace=False)) for _ in range(nvt)]).astype(np.int32)
    scale = 0.25
    dq, dk, dv = _oracle_grads(orc, q, kx, v, do, npf, idx, scale)
    lse, delta = orc.lse_delta(q, kx, v, do, npf, idx, scale)
    _, lse_fwd = orc.attention(q, kx, v, npf, idx, scale, np.arange(N // 64, dtype=np.int32))
    np.testing.assert_array_equal(lse, lse_fwd.reshape(N))
    tiles = np.array([4, 0, 6], np.int32)
    sq = orc.backward_dq(q, kx, v, do, lse, delta, npf, idx, scale, tiles)
    sk, sv = orc.backward_dkdv(q, kx, v, do, lse, delta, npf, idx, scale, tiles)
    for a, t in enumerate(tiles):
        rows = slice(t * 64, (t + 1) * 64)
        np.testing.assert_array_equal(sq[a], dq[rows])
        np.testing.assert_array_equal(sk[a], dk[rows])
        np.testing.assert_array_equal(sv[a], dv[rows])
