"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times, on sampled outputs the oracle computes one by one:

* Prism-scale 720p: grid 32x48x80 (122,880 tokens, 1,920 tiles), batch 2,
  24 heads, head_dim 128, 480 kept tiles, and the keep sweep 192/120/96;
* dynamic tile shapes on the same grid;
* dense prefix of 2,048 tokens before a 24x48x84 video grid (1,512 tiles),
  378 kept video tiles.

Permutation and shape maps are compared in full, and at 720p the pooled means
and kept lists of every row of every (batch, head); gather, attention and
scatter on sampled (batch, head) pairs and query tiles.  The raster-I/O path
that the benchmark times (Q's means alone, bsa_forward_raster) is compared
with the tiled path in full, bit for bit, on the 720p, dynamic and prefix
workloads.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_39_amd as bsa
import oracle
import synthetic as S
from parity import DeviceRun, bits_to_f64, check_lse, gamma, check_output, check_selection, kfrag_layout, to_bits, vfrag_layout

pytestmark = pytest.mark.gpu

SAMPLE_BH = [(0, 0), (1, 23), (0, 13)]
N_QTILES = 24


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), as float64: float32 first
    is exact enough here (the float64 values come from the oracle's sums and
    double rounding through float32 moves a result by at most one bf16 ulp
    only at exact float32 midpoints, which the comparison below tolerates)."""
    return S.bf16_bits_to_f32(S.to_bf16_bits(x.astype(np.float32))).astype(np.float64)


def weight_rounding_bound(qt, kt, vt, npf, idx, tiles, o_ref, scale):
    """Per output element, a bound on |o_gpu - o| before the output's own
    rounding.  o = sum_j w_j v_j / sum_j w_j; the kernel uses weights
    w_j (1 + d_j) with |d_j| <= 2^-8 (bf16 keeps 8 significant bits) + 2 eps (eps: the float
    logit error, scale * gamma_D * |q| * max_j |k_j|, through exp; the common
    part cancels in the normalisation), in the numerator and the normaliser
    alike, so |o_gpu - o| <= max|d| / (1 - max|d|) * max_j |v_j - o| over the
    query's keys; float accumulation adds a few float ulps of max |v|."""
    D = qt.shape[-1]
    kmax = np.linalg.norm(bits_to_f64(kt), axis=-1).max()
    qf = bits_to_f64(qt)
    vf = bits_to_f64(vt)
    npt = npf // 64
    out = np.empty_like(o_ref)
    for n, i in enumerate(tiles):
        if i < npt:
            keys = np.arange(vf.shape[0])
        else:
            vid = idx[i - npt]
            keys = np.concatenate([np.arange(npf), (npf + vid[:, None] * 64 + np.arange(64)).reshape(-1)])
        vk = vf[keys]
        vmax, vmin = vk.max(0), vk.min(0)
        o = o_ref[n]
        spread = np.maximum(vmax[None, :] - o, o - vmin[None, :])
        qn = np.linalg.norm(qf[i * 64:(i + 1) * 64], axis=-1)
        d = 2.0 ** -8 + 2.0 * scale * gamma(D) * qn * kmax * 1.01
        out[n] = (d / (1.0 - d))[:, None] * spread + 8 * 2.0 ** -24 * np.abs(vk).max()
    return out


def check_against_rounded(got, ref, qt, kt, vt, npf, idx, tiles, scale, what):
    """The GPU's bf16 output against the oracle's output rounded to bf16 (ties
    to even), which separates the output's own rounding (up to half an ulp:
    2^-6 for |o| in [4, 8)) from the error of the computation.  Each result
    must lie within the rounding of both sides plus the computation's bound,
    and most must equal the rounded oracle bit for bit."""
    ref_r = bf16_round(ref)
    gotf = bits_to_f64(got)
    rerr = np.abs(gotf - ref_r)
    rnd = np.abs(ref_r - ref)
    comp = weight_rounding_bound(qt, kt, vt, npf, idx, tiles, ref, scale)
    # half an ulp on each side, at the largest magnitude either can reach
    mag = np.maximum(np.abs(ref) + comp, 2.0 ** -126)
    ulp = 2.0 ** (np.floor(np.log2(mag)) - 7)
    equal = gotf == ref_r
    print(f"[forward {what}] against the oracle rounded to bf16: max|err| {rerr.max():.2e} mean {rerr.mean():.2e}; "
          f"the rounding alone: max {rnd.max():.2e} mean {rnd.mean():.2e}; bf16 results equal "
          f"{float(equal.mean()):.4f}; computation bound: max {comp.max():.2e} mean {comp.mean():.2e}; "
          f"worst use of the bound {float(((rerr - ulp) / comp).max()):.2f}; max |o| {float(np.abs(ref).max()):.2f}",
          flush=True)
    assert np.all(rerr <= ulp + comp), what
    # the rounding dominates: most results are the oracle's own rounded value
    # and the mean distance to it is well under the mean rounding error
    assert equal.mean() >= 0.8, what
    assert rerr.mean() < 0.5 * rnd.mean(), what


def check_sampled(g: DeviceRun, q, k, v, perm, keep=None, sample_bh=SAMPLE_BH, vs_rounded=False):
    """vs_rounded: also compare with the oracle's output rounded to bf16."""
    wl = g.wl
    keep = keep or wl.keep_tiles
    npf = wl.n_prefix
    scale = float(np.float32(wl.scale))
    gq, gk = g.pooled()
    gidx = g.att.block_idx.cpu().numpy()[:, :, :wl.n_video_tiles, :keep]
    o_t = g.att.o_t
    out = g.out
    lse = g.att.lse
    rng = np.random.default_rng(wl.seed + keep)
    nqt = wl.n_tokens // 64
    for b, h in sample_bh:
        h = min(h, wl.heads - 1)
        sl = lambda x: np.ascontiguousarray(x[b:b + 1, :, h:h + 1])
        qt, kt, vt = (oracle.gather(sl(x), perm[b:b + 1], npf) for x in (q, k, v))
        for ref, dev in ((qt, g.att.q_t), (kfrag_layout(kt), g.att.k_f), (vfrag_layout(vt), g.att.v_f)):
            assert np.array_equal(to_bits(dev[b, h]).reshape(ref.shape[2:]), ref[0, 0])
        qp, kp = oracle.pool(qt, npf), oracle.pool(kt, npf)
        assert np.array_equal(gq[b, h], qp[0, 0]) and np.array_equal(gk[b, h], kp[0, 0])
        n_exact, n_near, n_gamma = check_selection(gidx[b:b + 1, h:h + 1], qp, kp, keep)
        print(f"[plan b{b} h{h}] exact rows {n_exact}, near ties {n_near}", flush=True)
        # attention on sampled query tiles, prefix tiles included when present
        tiles = rng.choice(nqt, size=N_QTILES, replace=False)
        if wl.n_prefix_tiles:
            tiles[:2] = [0, wl.n_prefix_tiles - 1]
        tiles = np.sort(tiles).astype(np.int32)
        ref, ref_lse = oracle.attention(qt[0, 0], kt[0, 0], vt[0, 0], npf, gidx[b, h], scale, tiles)
        got = to_bits(o_t[b, h]).reshape(nqt, 64, wl.head_dim)[tiles]
        mx, mean = check_output(got, ref, f"b{b} h{h}")
        print(f"[forward b{b} h{h}] max|err| {mx:.2e} mean {mean:.2e}", flush=True)
        if vs_rounded:
            check_against_rounded(got, ref, qt[0, 0], kt[0, 0], vt[0, 0], npf, gidx[b, h], tiles, scale, f"b{b} h{h}")
        got_lse = lse[b, h].cpu().numpy().reshape(nqt, 64)[tiles]
        check_lse(got_lse, ref_lse, qt[0, 0].reshape(nqt, 64, -1)[tiles], kt[0, 0], scale, f"lse b{b} h{h}")
        # scatter back, exact
        sc = oracle.scatter(to_bits(o_t[b:b + 1, h:h + 1]), perm[b:b + 1], npf)
        assert np.array_equal(to_bits(out[b, :, h]), sc[0, :, 0])


def assert_raster_io_equals_tiled(g: DeviceRun):
    """The raster-I/O path on g's inputs (bsa_permute(POOL), the pooling K
    gather, the V gather beside the selection, bsa_forward_raster; grouped
    launch): Q's means, every kept list, the whole raster output and the lse
    equal the tiled path's bit for bit, the output first filled with NaN so
    that a row left unwritten shows."""
    att = bsa.BlockSparseAttention(g.desc, with_lse=True)
    assert att.raster_io
    out = torch.full_like(g.q.view(torch.int16), 0x7FC1).view(torch.bfloat16)
    att(g.q, g.k, g.v, out)
    torch.cuda.synchronize()
    assert torch.equal(att.block_idx, g.att.block_idx)
    rq, rk = bsa.pooled_views(g.desc, att.workspace)
    tq, tk = bsa.pooled_views(g.desc, g.att.workspace)
    assert torch.equal(rq, tq) and torch.equal(rk, tk)
    assert torch.equal(out.view(torch.int16), g.out.view(torch.int16))
    assert torch.equal(att.lse, g.att.lse)
    print("[raster I/O] means, lists, output and lse equal the tiled path's", flush=True)
    del att, out


@pytest.fixture(scope="module")
def prism():
    wl = S.WORKLOADS["prism720p"]
    print(f"\n[case] {wl}", flush=True)
    q, k, v = S.qkv(wl)
    g = DeviceRun(wl, q, k, v).run()
    yield wl, q, k, v, g
    del g
    torch.cuda.empty_cache()


def test_prism720p_sampled(prism):
    wl, q, k, v, g = prism
    perm = np.ascontiguousarray(np.broadcast_to(oracle.perm_static(wl.grid), (wl.batch, wl.n_video)))
    assert np.array_equal(g.perm(), perm)
    check_sampled(g, q, k, v, perm)
    # determinism of the whole path at full size
    first = to_bits(g.out)
    g.run()
    assert np.array_equal(first, to_bits(g.out))


def test_prism720p_raster_io(prism):
    wl, q, k, v, g = prism
    assert_raster_io_equals_tiled(g)


def test_prism720p_plan_every_row(prism):
    """The plan at full size on every (batch, head): pooled means of every tile
    bit-exact, kept lists of every row exact: the contract's rows (k-th /
    (k+1)-th relative gap at least 1e-4) and the near ties as well."""
    wl, q, k, v, g = prism
    npf = wl.n_prefix
    perm = np.ascontiguousarray(np.broadcast_to(oracle.perm_static(wl.grid), (wl.batch, wl.n_video)))
    gq, gk = g.pooled()
    gidx = g.block_idx()
    n_exact = n_near = n_gamma = 0
    for b in range(wl.batch):
        for h in range(wl.heads):
            sl = lambda x: np.ascontiguousarray(x[b:b + 1, :, h:h + 1])
            qt, kt = (oracle.gather(sl(x), perm[b:b + 1], npf) for x in (q, k))
            qp, kp = oracle.pool(qt, npf), oracle.pool(kt, npf)
            assert np.array_equal(gq[b, h], qp[0, 0]) and np.array_equal(gk[b, h], kp[0, 0]), f"b{b} h{h}"
            e, n, gb = check_selection(gidx[b:b + 1, h:h + 1], qp, kp, wl.keep_tiles)
            n_exact += e
            n_near += n
            n_gamma += gb
    print(f"[plan, every row] rows outside the 1e-4 band {n_exact}, near-tie rows {n_near} (exact too), "
          f"rows within the float rounding band {n_gamma} (exact too)", flush=True)
    assert n_exact + n_near == wl.batch * wl.heads * wl.n_video_tiles


@pytest.mark.parametrize("keep", [192, 120, 96])
def test_prism720p_keep_sweep_sampled(prism, keep):
    wl, q, k, v, _ = prism
    wk = wl.with_keep(keep)
    print(f"\n[case] {wk}", flush=True)
    g = DeviceRun(wk, q, k, v).run()
    perm = np.ascontiguousarray(np.broadcast_to(oracle.perm_static(wl.grid), (wl.batch, wl.n_video)))
    check_sampled(g, q, k, v, perm, sample_bh=[(1, 5)])
    del g
    torch.cuda.empty_cache()


def test_prefix_sampled():
    wl = S.WORKLOADS["prefix"]
    print(f"\n[case] {wl}", flush=True)
    q, k, v = S.qkv(wl)
    g = DeviceRun(wl, q, k, v).run()
    perm = np.ascontiguousarray(np.broadcast_to(oracle.perm_static(wl.grid), (wl.batch, wl.n_video)))
    assert np.array_equal(g.perm(), perm)
    check_sampled(g, q, k, v, perm, sample_bh=[(0, 0), (0, 17)])
    assert_raster_io_equals_tiled(g)
    del g
    torch.cuda.empty_cache()


def test_dynamic_sampled():
    wl = S.WORKLOADS["prism720p_dynamic"]
    print(f"\n[case] {wl}", flush=True)
    q, k, v = S.qkv(wl)
    g = DeviceRun(wl, q, k, v).run()
    st = oracle.shape_stats(q, wl.n_prefix, wl.grid)
    shape_o, near = oracle.shape_choose(st, wl.grid, float(np.float32(wl.tau)))
    gs = g.shape_map()
    clear = near == 0
    assert np.array_equal(gs[clear], shape_o[clear])
    hist = np.bincount(gs.reshape(-1), minlength=9)
    print(f"[shapes] histogram {hist.tolist()}, near-threshold regions {int((~clear).sum())}", flush=True)
    assert (hist > 0).sum() >= 4
    perm = oracle.perm_dynamic(gs, wl.grid)
    assert np.array_equal(g.perm(), perm)
    check_sampled(g, q, k, v, perm, sample_bh=[(0, 3), (1, 20)], vs_rounded=True)
    assert_raster_io_equals_tiled(g)
    del g
    torch.cuda.empty_cache()
