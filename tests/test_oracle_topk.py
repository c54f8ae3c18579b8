"""Pins of the oracle's pooled score and per-row top-k (Prism speed-ablation
page: per query block keep the (1 - sparsity) most relevant key blocks)."""
import json
import os

import numpy as np
import pytest

from synthetic import keep_from_sparsity

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_counts.json")))


def test_pages_keep_count():
    n = GOLD["key_blocks_per_query_block"]
    assert keep_from_sparsity(n, GOLD["sparsity"]) == GOLD["kept_key_blocks"]
    k93 = keep_from_sparsity(n, GOLD["high_sparsity"])
    assert abs(100.0 * k93 / n - GOLD["high_sparsity_keep_percent_approx"]) < 0.5


def test_planted_ranking(orc):
    # q = u, k_j = j * eps * u: s_j = j * eps * |u|^2, so the top k are the last k
    n, D, k = 40, 16, 7
    u = np.linspace(0.5, 1.5, D).astype(np.float32)
    qp = np.broadcast_to(u, (1, 1, n, D)).copy()
    kp = (np.arange(n, dtype=np.float32)[:, None] * np.float32(0.01) * u)[None, None]
    idx, s_k, s_k1, _ = orc.topk(qp, kp, k)
    for i in range(n):
        np.testing.assert_array_equal(idx[0, 0, i], np.arange(n - k, n))
    assert np.all(s_k > s_k1)


def test_all_equal_scores_take_lowest_indices(orc):
    n, D, k = 33, 8, 5
    qp = np.ones((2, 1, n, D), np.float32)
    kp = np.full((2, 1, n, D), 0.25, np.float32)
    idx, s_k, s_k1, _ = orc.topk(qp, kp, k)
    assert np.all(idx == np.arange(k))
    assert np.all(s_k == s_k1)


def test_tie_straddling_the_boundary(orc):
    # scores 9, 8, 1, 5, 0, 0, 0, 0, 5, 0: j=3 and j=8 tie at 5.
    sc = np.array([9, 8, 1, 5, 0, 0, 0, 0, 5, 0], np.float32)
    n = sc.size
    qp = np.ones((1, 1, n, 1), np.float32)
    kp = sc.reshape(1, 1, n, 1)
    idx4, _, _, _ = orc.topk(qp, kp, 4)       # both tied tiles fit
    np.testing.assert_array_equal(idx4[0, 0, 0], [0, 1, 3, 8])
    idx3, s_k, s_k1, _ = orc.topk(qp, kp, 3)  # the tie is split: lower index wins
    np.testing.assert_array_equal(idx3[0, 0, 0], [0, 1, 3])
    assert s_k[0, 0, 0] == s_k1[0, 0, 0] == 5.0


@pytest.mark.parametrize("n,k", [(37, 1), (37, 9), (64, 16), (100, 100), (130, 33)])
def test_matches_exhaustive_sort(orc, n, k):
    rng = np.random.default_rng(n * 1000 + k)
    B, H, D = 2, 2, 24
    qp = rng.standard_normal((B, H, n, D)).astype(np.float32)
    kp = rng.standard_normal((B, H, n, D)).astype(np.float32)
    idx, s_k, s_k1, mag = orc.topk(qp, kp, k)
    for b in range(B):
        for h in range(H):
            s = qp[b, h].astype(np.float64) @ kp[b, h].astype(np.float64).T
            for i in range(n):
                order = sorted(range(n), key=lambda j: (-s[i, j], j))
                assert list(idx[b, h, i]) == sorted(order[:k])
                assert s_k[b, h, i] == pytest.approx(s[i, order[k - 1]], rel=1e-12, abs=1e-12)
                if k < n:
                    assert s_k1[b, h, i] == pytest.approx(s[i, order[k]], rel=1e-12, abs=1e-12)
                else:
                    assert np.isnan(s_k1[b, h, i])
                absum = np.abs(qp[b, h, i].astype(np.float64) * kp[b, h].astype(np.float64)).sum(1)
                m = max(absum[order[t]] for t in range(k - 1, min(k + 1, n)))
                assert mag[b, h, i] == pytest.approx(m, rel=1e-12)


def test_rows_subset_and_shape_invariants(orc):
    rng = np.random.default_rng(3)
    n, D, k = 50, 8, 12
    qp = rng.standard_normal((1, 2, n, D)).astype(np.float32)
    kp = rng.standard_normal((1, 2, n, D)).astype(np.float32)
    full, *_ = orc.topk(qp, kp, k)
    rows = np.array([49, 0, 17], np.int32)
    sub, *_ = orc.topk(qp, kp, k, rows=rows)
    np.testing.assert_array_equal(sub, full[:, :, rows])
    for row in full.reshape(-1, k):
        assert len(set(row.tolist())) == k and np.all(np.diff(row) > 0)
        assert row.min() >= 0 and row.max() < n


def test_rejects_bad_k(orc):
    qp = np.zeros((1, 1, 4, 2), np.float32)
    with pytest.raises(ValueError):
        orc.topk(qp, qp, 0)
    with pytest.raises(ValueError):
        orc.topk(qp, qp, 5)
