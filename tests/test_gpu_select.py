"""GPU tests of the selection (bsa_plan, bsa_select) beyond random workloads.

* The tile means taken inside the Q and K gathers (bsa_permute GATHER_POOL /
  GATHER_KF_POOL, then bsa_select) equal bsa_plan's own pooling, and give the
  same lists and output, bit for bit.
* Rows whose float scores cannot be ordered: channels of +/-2^20 cancel, so
  float partial sums lose everything below about 0.06, while the true scores
  differ by as little as the small channels make them.  The selection must
  still be exactly the oracle's top k of the double scores.  With more than
  64 tiles every key falls in the re-scored band and the radix-select path
  over double keys runs; with fewer, the in-register ranking.
* Rows of all-equal scores keep the lowest tile numbers, through both paths.
* The same adversarial rows through the CSR planner with per-head keeps.
* A caller holding K and V in the tiled layout: TILED_TO_KF / TILED_TO_VF give
  exactly the fragment layouts the raster gathers write.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_39_amd as bsa
import oracle
import synthetic as S
from parity import DeviceRun, check_output, check_selection, desc_for, to_bits, to_dev

pytestmark = pytest.mark.gpu

W = S.Workload
CASES = [
    S.WORKLOADS["tiny"],
    W("ragged", 2, 3, 128, (8, 8, 12), 5, seed=11),
    W("prefix_d64", 2, 2, 64, (4, 8, 24), 2, seed=13, n_prefix=192),
    W("pad_5x6x7", 2, 2, 128, (5, 6, 7), 5, seed=41, n_prefix=64, padded=True),
    W("dynamic", 2, 2, 128, (16, 16, 32), 6, seed=18, dynamic=True, recipe="field"),
    W("many_tiles", 1, 1, 64, (16, 32, 40), 77, seed=21),
]


@pytest.mark.parametrize("wl", CASES, ids=[c.name for c in CASES])
def test_pooling_gathers_equal_plan(wl):
    print(f"\n[case] {wl}", flush=True)
    q, k, v = S.qkv(wl)
    fused = DeviceRun(wl, q, k, v).run()
    means = [x.copy() for x in fused.pooled()]
    idx, out = fused.block_idx().copy(), to_bits(fused.out).copy()
    q_t, k_f = to_bits(fused.att.q_t).copy(), to_bits(fused.att.k_f).copy()
    plain = DeviceRun(wl, q, k, v)
    plain.att.pool_in_gather = False
    plain.run()
    for a, b in zip(means, plain.pooled()):
        assert np.array_equal(a, b)
    assert np.array_equal(q_t, to_bits(plain.att.q_t)) and np.array_equal(k_f, to_bits(plain.att.k_f))
    assert np.array_equal(idx, plain.block_idx())
    assert np.array_equal(out, to_bits(plain.out))


def cancelling_inputs(wl, equal_head: bool):
    """Raster Q, K, V (bf16 bits) whose tiles are constant per tile: Q tiles
    are all ones; K tile j of head 0 holds 2^20 in the first channel, -2^20 in
    the last, sigma(j)/16 (sigma a seeded permutation) in the second and small
    random values in the others; head 1 (equal_head) has the same K vector in
    every tile."""
    rng = np.random.default_rng(wl.seed)
    n, D, B, H = wl.n_video_tiles, wl.head_dim, wl.batch, wl.heads
    perm = oracle.perm_static(wl.grid)
    kt = np.zeros((H, n, D), np.float32)
    sigma = rng.permutation(n)
    kt[:, :, 2:D - 1] = rng.standard_normal((H, n, D - 3)) / 256.0
    kt[:, :, 0] = 2.0 ** 20
    kt[:, :, D - 1] = -2.0 ** 20
    kt[:, :, 1] = sigma / 16.0
    if equal_head:
        kt[1] = kt[1, 0]
    kt = S.bf16_bits_to_f32(S.to_bf16_bits(kt))
    tok_tile = np.arange(wl.n_video) // 64
    qr = np.ones((B, wl.n_video, H, D), np.float32)
    kr = np.empty((B, wl.n_video, H, D), np.float32)
    kr[:, perm] = kt[:, tok_tile].transpose(1, 0, 2)[None]
    vr = rng.standard_normal((B, wl.n_video, H, D)).astype(np.float32)
    return S.to_bf16_bits(qr), S.to_bf16_bits(kr), S.to_bf16_bits(vr)


@pytest.mark.parametrize("wl", [W("cancel80", 1, 2, 128, (8, 16, 40), 37, seed=51),
                                W("cancel16", 1, 2, 128, (8, 8, 16), 5, seed=52),
                                W("cancel80_d64", 1, 2, 64, (8, 16, 40), 61, seed=53)],
                         ids=["radix_path", "ranking_path", "d64"])
def test_cancelling_channels_select_exactly(wl):
    print(f"\n[case] {wl}", flush=True)
    q, k, v = cancelling_inputs(wl, equal_head=True)
    g = DeviceRun(wl, q, k, v).run()
    perm = oracle.perm_static(wl.grid)[None]
    qt, kt = oracle.gather(q, perm, 0), oracle.gather(k, perm, 0)
    qp, kp = oracle.pool(qt, 0), oracle.pool(kt, 0)
    gq, gk = g.pooled()
    assert np.array_equal(gq, qp) and np.array_equal(gk, kp)
    # a selection from float scores alone would not do: a float sum in channel
    # order carries 2^20 past every small channel and is off by more than the
    # gaps between scores
    s64 = qp[0, 0].astype(np.float64) @ kp[0, 0].astype(np.float64).T
    s32 = np.add.accumulate(qp[0, 0][:, None, :] * kp[0, 0][None, :, :], axis=-1, dtype=np.float32)[..., -1]
    assert np.abs(s32.astype(np.float64) - s64).max() > np.diff(np.sort(s64[0])).min()
    idx = g.block_idx()
    n_clear, n_near, n_gamma = check_selection(idx, qp, kp, wl.keep_tiles)
    print(f"[plan] rows {n_clear} clear, {n_near} near ties, {n_gamma} in the float band", flush=True)
    assert np.all(idx[0, 1] == np.arange(wl.keep_tiles))  # equal scores: the lowest tile numbers
    # the CSR planner on the same rows, per-head keeps
    desc = desc_for(wl)
    keep_h = [wl.keep_tiles, max(1, wl.keep_tiles // 3)]
    rows = wl.batch * wl.heads * wl.n_video_tiles
    row_ptr = torch.empty(rows + 1, dtype=torch.int64, device="cuda")
    col = torch.empty(bsa.csr_entries(desc, keep_h), dtype=torch.int32, device="cuda")
    bsa.plan_csr(desc, g.att.q_t, g.att.k_f, row_ptr, col, g.att.workspace, keep_per_head=keep_h)
    torch.cuda.synchronize()
    rp, cl = row_ptr.cpu().numpy(), col.cpu().numpy()
    for h, kh in enumerate(keep_h):
        o_rp, o_col = oracle.plan_csr(qp[:, h:h + 1], kp[:, h:h + 1], [kh])
        n = wl.n_video_tiles
        got = cl[rp[h * n]:rp[(h + 1) * n]]
        assert np.array_equal(np.diff(rp[h * n:(h + 1) * n + 1]), np.diff(o_rp))
        assert np.array_equal(got, o_col), f"head {h}"


def test_equal_scores_everywhere_fallback():
    """Every score of every row equal (Q == 0): more than 64 members per row,
    so the double radix select runs on every row; lists are 0..k-1."""
    wl = W("zeros", 1, 2, 64, (8, 16, 40), 23, seed=54)
    q, k, v = S.qkv(wl)
    q = np.zeros_like(q)
    g = DeviceRun(wl, q, k, v).run()
    assert np.all(g.block_idx() == np.arange(23))


def test_tiled_inputs_convert_to_fragment_layouts():
    """TILED_TO_KF / TILED_TO_VF of tiled K and V equal the fragment layouts
    the raster gathers write; the path driven from tiled K and V gives the
    same lists and output bit for bit."""
    wl = W("tiled_in", 2, 3, 128, (8, 8, 12), 5, seed=61, n_prefix=64)
    q, k, v = S.qkv(wl)
    g = DeviceRun(wl, q, k, v).run()
    desc, att = g.desc, g.att
    k_t, v_t = torch.empty_like(att.q_t), torch.empty_like(att.q_t)
    bsa.gather(desc, g.k, k_t, att.perm)
    bsa.gather(desc, g.v, v_t, att.perm)
    k_f, v_f = torch.empty_like(att.k_f), torch.empty_like(att.v_f)
    bsa.tiled_to_kf(desc, k_t, k_f)
    bsa.tiled_to_vf(desc, v_t, v_f)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(k_f), to_bits(att.k_f))
    assert np.array_equal(to_bits(v_f), to_bits(att.v_f))
    idx = torch.empty_like(att.block_idx)
    o_t = torch.empty_like(att.o_t)
    bsa.plan(desc, att.q_t, k_f, idx, att.workspace)
    bsa.forward(desc, att.q_t, k_f, v_f, idx, o_t, workspace=att.workspace)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), att.block_idx.cpu().numpy())
    assert np.array_equal(to_bits(o_t), to_bits(att.o_t))


def test_forward_stats_count_rounds():
    """The grouped forward records its rounds; on an idle GPU with one block
    per CU no round's start wait gives up."""
    wl = W("stats", 2, 4, 128, (16, 16, 32), 12, seed=62)
    q, k, v = S.qkv(wl)
    g = DeviceRun(wl, q, k, v).run()
    gave_up, rounds = bsa.forward_stats(g.desc, g.att.workspace)
    print(f"[stats] rounds {rounds}, waits that gave up {gave_up}", flush=True)
    assert rounds >= wl.batch * wl.heads * wl.n_video_tiles // 256
    assert gave_up == 0


@pytest.mark.parametrize("grid,keep", [((32, 48, 96), 301), ((32, 64, 160), 640), ((32, 64, 256), 300)],
                         ids=["n2304", "n5120", "n8192_max"])
def test_large_tile_counts(grid, keep):
    """More video tiles than 16 rows of scores fit in LDS: 8 rows per item
    (2,304 tiles) and 4 rows per item (5,120 tiles, and the largest video
    tile count the library accepts, 8,192); lists against the oracle on every
    row, including the pooled means."""
    wl = W(f"n{grid}", 1, 1, 64, grid, keep, seed=71)
    print(f"\n[case] {wl}", flush=True)
    q, k, v = S.qkv(wl)
    desc = desc_for(wl)
    att = bsa.BlockSparseAttention(desc)
    qd, kd = to_dev(q), to_dev(k)
    att.build(qd)
    att.gather_qk(qd, kd)
    att.plan()
    torch.cuda.synchronize()
    perm = oracle.perm_static(wl.grid)[None]
    qt, kt = oracle.gather(q, perm, 0), oracle.gather(k, perm, 0)
    qp, kp = oracle.pool(qt, 0), oracle.pool(kt, 0)
    gq, gk = bsa.pooled_views(desc, att.workspace)
    assert np.array_equal(gq.cpu().numpy(), qp) and np.array_equal(gk.cpu().numpy(), kp)
    n_clear, n_near, n_gamma = check_selection(att.block_idx.cpu().numpy(), qp, kp, keep)
    print(f"[plan] rows {n_clear} clear, {n_near} near ties, {n_gamma} in the float band", flush=True)


def test_maximum_total_tiles_whole_path():
    """The most tiles per (batch, head) the library accepts: 8,192 prefix
    tiles and 8,192 video tiles (16,384, a million tokens).  Permutation,
    gathers and scatter are bit-exact on every row; the lists against the
    oracle on every row; attention of a prefix query tile (every key) and a
    video query tile (the prefix plus its kept tiles) against the oracle; the
    raster-I/O path equal to the tiled one bit for bit."""
    wl = W("max_tiles", 1, 1, 64, (32, 64, 256), 16, seed=72, n_prefix=8192 * 64)
    print(f"\n[case] {wl}", flush=True)
    assert wl.n_tokens // 64 == bsa.MAX_VIDEO_TILES * 2 and wl.n_video_tiles == bsa.MAX_VIDEO_TILES
    q, k, v = S.qkv(wl)
    g = DeviceRun(wl, q, k, v).run()
    perm = oracle.perm_static(wl.grid)[None]
    assert np.array_equal(g.perm(), perm)
    npf = wl.n_prefix
    qt, kt, vt = (oracle.gather(x, perm, npf) for x in (q, k, v))
    assert np.array_equal(to_bits(g.att.q_t).reshape(qt.shape), qt)
    qp, kp = oracle.pool(qt, npf), oracle.pool(kt, npf)
    gq, gk = g.pooled()
    assert np.array_equal(gq, qp) and np.array_equal(gk, kp)
    idx = g.block_idx()
    n_clear, n_near, n_gamma = check_selection(idx, qp, kp, wl.keep_tiles)
    print(f"[plan] rows {n_clear} clear, {n_near} near ties, {n_gamma} in the float band", flush=True)
    tiles = np.array([3, wl.n_prefix_tiles + 4321], dtype=np.int32)
    ref, _ = oracle.attention(qt[0, 0], kt[0, 0], vt[0, 0], npf, idx[0, 0], float(np.float32(wl.scale)), tiles)
    got = to_bits(g.att.o_t[0, 0]).reshape(-1, 64, wl.head_dim)[tiles]
    mx, mean = check_output(got, ref, "max tiles")
    print(f"[forward] max|err| {mx:.2e} mean {mean:.2e}", flush=True)
    sc = oracle.scatter(to_bits(g.att.o_t), perm, npf)
    assert np.array_equal(to_bits(g.out), sc)
    # the raster-I/O path at the same size (raster rows past 2^19 and slot
    # numbers up to 2^20 - 1): the same output and lse bit for bit
    att = bsa.BlockSparseAttention(g.desc, with_lse=True)
    out = torch.full_like(g.q.view(torch.int16), 0x7FC1).view(torch.bfloat16)
    att(g.q, g.k, g.v, out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), g.out.view(torch.int16))
    assert torch.equal(att.lse, g.att.lse)
