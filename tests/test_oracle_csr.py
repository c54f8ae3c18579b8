"""Pins of the oracle's variable-keep path (kept lists of their own length per
query tile, in CSR form).

* Attention: with every row of the same length it is the fixed-keep
  attention, bit for bit; with rows of different lengths it equals torch's
  scaled_dot_product_attention in float64 under an explicit token-by-token
  mask built from the lists (prefix rows dense, video rows see the prefix and
  their kept tiles -- Ref2VA VSA page, section on conditioning tokens).
* Gradients: uniform rows give the fixed-keep gradients bit for bit; rows of
  different lengths match torch autograd through the masked fp64 attention.
* Selection: each row holds the k_row tiles a stable descending sort of its
  exact float64 scores puts first (lowest tile number first among equal
  scores -- the reading of the tie rule), ascending; the counts are the
  per-head keeps clamped by the per-row keeps; a row's list for a smaller
  count is a subset of its list for a larger one.
"""
import numpy as np
import pytest
import torch

from synthetic import bf16_bits_to_f32, to_bf16_bits


def _rand(rng, n_tok, D, scale=1.0):
    return to_bf16_bits(rng.standard_normal((n_tok, D)).astype(np.float32) * scale)


def _f64(x):
    return torch.from_numpy(bf16_bits_to_f32(x).astype(np.float64))


def _csr_mask(npf, nvt, row_ptr, col):
    N = npf + nvt * 64
    m = np.zeros((N, N), bool)
    m[:npf, :] = True
    m[npf:, :npf] = True
    for i in range(nvt):
        rows = slice(npf + i * 64, npf + (i + 1) * 64)
        for j in col[row_ptr[i]:row_ptr[i + 1]]:
            m[rows, npf + j * 64: npf + (j + 1) * 64] = True
    return m


def test_uniform_rows_equal_fixed_keep(orc):
    rng = np.random.default_rng(71)
    D, npf, nvt, k = 16, 64, 6, 3
    N = npf + nvt * 64
    q, kx, v = (_rand(rng, N, D) for _ in range(3))
    idx = np.stack([np.sort(rng.choice(nvt, size=k, replace=False)) for _ in range(nvt)]).astype(np.int32)
    row_ptr = np.arange(nvt + 1, dtype=np.int64) * k
    tiles = np.arange(N // 64, dtype=np.int32)
    o1, l1 = orc.attention(q, kx, v, npf, idx, 0.3, tiles)
    o2, l2 = orc.attention_csr(q, kx, v, npf, row_ptr, idx.reshape(-1), 0.3, tiles)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("D,npf,nvt", [(8, 0, 7), (64, 128, 5)])
def test_variable_rows_match_masked_dense(orc, D, npf, nvt):
    rng = np.random.default_rng(72 + D)
    N = npf + nvt * 64
    q, kx, v = (_rand(rng, N, D, 1.5) for _ in range(3))
    lens = rng.integers(1, nvt + 1, size=nvt)
    row_ptr = np.zeros(nvt + 1, np.int64)
    row_ptr[1:] = np.cumsum(lens)
    col = np.concatenate([np.sort(rng.choice(nvt, size=n, replace=False)) for n in lens]).astype(np.int32)
    scale = 0.25
    out, lse = orc.attention_csr(q, kx, v, npf, row_ptr, col, scale, np.arange(N // 64, dtype=np.int32))
    m = torch.from_numpy(_csr_mask(npf, nvt, row_ptr, col))
    qq, kk, vv = (_f64(x)[None, None] for x in (q, kx, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=m[None, None], scale=scale)[0, 0]
    np.testing.assert_allclose(out.reshape(N, D), ref.numpy(), rtol=0, atol=1e-12)
    logits = (_f64(q) @ _f64(kx).T) * scale
    ref_lse = torch.logsumexp(logits.masked_fill(~m, -np.inf), 1).numpy()
    np.testing.assert_allclose(lse.reshape(N), ref_lse, rtol=0, atol=1e-12)


def _brute_lists(qp, kp, lens):
    """Per row, the first k_row tiles of a stable descending sort of the
    float64 scores (lower tile number first among equal scores), ascending."""
    B, H, n, _ = qp.shape
    out = []
    for b in range(B):
        for h in range(H):
            s = qp[b, h].astype(np.float64) @ kp[b, h].astype(np.float64).T
            for i in range(n):
                order = np.lexsort((np.arange(n), -s[i]))
                out.append(np.sort(order[:lens[b, h, i]]))
    return out


def test_selection_counts_and_sets(orc):
    rng = np.random.default_rng(73)
    B, H, n, D = 2, 3, 12, 8
    qp = rng.standard_normal((B, H, n, D)).astype(np.float32)
    kp = rng.standard_normal((B, H, n, D)).astype(np.float32)
    keep_h = [5, 1, 12]
    keep_rows = rng.integers(-2, 14, size=(B, H, n))
    row_ptr, col = orc.plan_csr(qp, kp, keep_h, keep_rows)
    lens = np.minimum(np.maximum(keep_rows, 1), np.array(keep_h)[None, :, None])
    assert np.array_equal(np.diff(row_ptr), lens.reshape(-1))
    got = [col[row_ptr[r]:row_ptr[r + 1]] for r in range(B * H * n)]
    for g, e in zip(got, _brute_lists(qp, kp, lens)):
        assert np.array_equal(g, e)


def test_selection_ties_and_nesting(orc):
    # all-equal scores: every row keeps tiles 0..k-1 (the tie rule)
    B, H, n, D = 1, 2, 9, 4
    qp = np.ones((B, H, n, D), np.float32)
    kp = np.ones((B, H, n, D), np.float32)
    row_ptr, col = orc.plan_csr(qp, kp, [4, 7])
    for r in range(B * H * n):
        assert np.array_equal(col[row_ptr[r]:row_ptr[r + 1]], np.arange(row_ptr[r + 1] - row_ptr[r]))
    # nesting: a smaller count keeps a subset of a larger one's tiles
    rng = np.random.default_rng(74)
    qp = rng.standard_normal((1, 1, 16, 8)).astype(np.float32)
    kp = rng.standard_normal((1, 1, 16, 8)).astype(np.float32)
    lists = {}
    for k in (1, 4, 9, 16):
        rp, c = orc.plan_csr(qp, kp, [k])
        lists[k] = [set(c[rp[i]:rp[i + 1]]) for i in range(16)]
    for a, b in ((1, 4), (4, 9), (9, 16)):
        assert all(x <= y for x, y in zip(lists[a], lists[b]))


# ---- gradients over CSR lists ---------------------------------------------------

def test_csr_gradients_uniform_rows_equal_fixed_keep(orc):
    rng = np.random.default_rng(75)
    B, H, D, npf, nvt, k = 1, 2, 16, 64, 5, 3
    N = npf + nvt * 64
    q, kx, v, do = (_rand(rng, B * H * N, D).reshape(B, H, N, D) for _ in range(4))
    idx = np.stack([np.stack([np.sort(rng.choice(nvt, size=k, replace=False)) for _ in range(nvt)])
                    for _ in range(B * H)]).reshape(B, H, nvt, k).astype(np.int32)
    row_ptr = np.arange(B * H * nvt + 1, dtype=np.int64) * k
    g1 = orc.backward_full(q, kx, v, do, npf, idx, 0.3)
    g2 = orc.backward_full_csr(q, kx, v, do, npf, row_ptr, idx.reshape(-1), 0.3)
    for a, b in zip(g1, g2):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("D,npf,nvt", [(8, 0, 6), (16, 128, 4)])
def test_csr_gradients_match_masked_autograd(orc, D, npf, nvt):
    """Rows of different lengths: torch autograd through fp64 SDPA under the
    token mask of the lists, loss = sum of O * dO."""
    rng = np.random.default_rng(76 + D)
    N = npf + nvt * 64
    q, kx, v, do = (_rand(rng, N, D, 1.5) for _ in range(4))
    lens = rng.integers(1, nvt + 1, size=nvt)
    row_ptr = np.zeros(nvt + 1, np.int64)
    row_ptr[1:] = np.cumsum(lens)
    col = np.concatenate([np.sort(rng.choice(nvt, size=n, replace=False)) for n in lens]).astype(np.int32)
    scale = 0.25
    got = orc.backward_full_csr(q[None, None], kx[None, None], v[None, None], do[None, None], npf, row_ptr, col,
                                scale)
    m = torch.from_numpy(_csr_mask(npf, nvt, row_ptr, col))
    qq, kk, vv = (_f64(x).requires_grad_(True) for x in (q, kx, v))
    out = torch.nn.functional.scaled_dot_product_attention(qq[None, None], kk[None, None], vv[None, None],
                                                           attn_mask=m[None, None], scale=scale)[0, 0]
    (out * _f64(do)).sum().backward()
    for g, r in zip(got, (qq.grad, kk.grad, vv.grad)):
        np.testing.assert_allclose(g[0, 0], r.numpy(), rtol=0, atol=1e-11)
