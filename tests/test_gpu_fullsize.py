"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times, on sampled outputs the oracle computes one by one:

* Prism-scale 720p: grid 32x48x80 (122,880 tokens, 1,920 tiles), batch 2,
  24 heads, head_dim 128, 480 kept tiles, and the keep sweep 192/120/96;
* dynamic tile shapes on the same grid;
* dense prefix of 2,048 tokens before a 24x48x84 video grid (1,512 tiles),
  378 kept video tiles.

Permutation and shape maps are compared in full, and at 720p the pooled means
and kept lists of every row of every (batch, head); gather, attention and
scatter on sampled (batch, head) pairs and query tiles.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from parity import GpuRun, check_lse, check_output, check_selection, kfrag_layout, to_bits, vfrag_layout

pytestmark = pytest.mark.gpu

SAMPLE_BH = [(0, 0), (1, 23), (0, 13)]
N_QTILES = 24


def check_sampled(g: GpuRun, q, k, v, perm, keep=None, sample_bh=SAMPLE_BH):
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
        n_exact, n_near = check_selection(gidx[b:b + 1, h:h + 1], qp, kp, keep)
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
        got_lse = lse[b, h].cpu().numpy().reshape(nqt, 64)[tiles]
        check_lse(got_lse, ref_lse, qt[0, 0].reshape(nqt, 64, -1)[tiles], kt[0, 0], scale, f"lse b{b} h{h}")
        # scatter back, exact
        sc = oracle.scatter(to_bits(o_t[b:b + 1, h:h + 1]), perm[b:b + 1], npf)
        assert np.array_equal(to_bits(out[b, :, h]), sc[0, :, 0])


@pytest.fixture(scope="module")
def prism():
    wl = S.WORKLOADS["prism720p"]
    print(f"\n[case] {wl}", flush=True)
    q, k, v = S.qkv(wl)
    g = GpuRun(wl, q, k, v).run()
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


def test_prism720p_plan_every_row(prism):
    """The plan at full size on every (batch, head): pooled means of every tile
    bit-exact, kept lists of every row exact outside near ties (a valid top-k
    within the band on near ties)."""
    wl, q, k, v, g = prism
    npf = wl.n_prefix
    perm = np.ascontiguousarray(np.broadcast_to(oracle.perm_static(wl.grid), (wl.batch, wl.n_video)))
    gq, gk = g.pooled()
    gidx = g.block_idx()
    n_exact = n_near = 0
    for b in range(wl.batch):
        for h in range(wl.heads):
            sl = lambda x: np.ascontiguousarray(x[b:b + 1, :, h:h + 1])
            qt, kt = (oracle.gather(sl(x), perm[b:b + 1], npf) for x in (q, k))
            qp, kp = oracle.pool(qt, npf), oracle.pool(kt, npf)
            assert np.array_equal(gq[b, h], qp[0, 0]) and np.array_equal(gk[b, h], kp[0, 0]), f"b{b} h{h}"
            e, n = check_selection(gidx[b:b + 1, h:h + 1], qp, kp, wl.keep_tiles)
            n_exact += e
            n_near += n
    print(f"[plan, every row] exact rows {n_exact}, near-tie rows {n_near}", flush=True)
    assert n_exact + n_near == wl.batch * wl.heads * wl.n_video_tiles


@pytest.mark.parametrize("keep", [192, 120, 96])
def test_prism720p_keep_sweep_sampled(prism, keep):
    wl, q, k, v, _ = prism
    wk = wl.with_keep(keep)
    print(f"\n[case] {wk}", flush=True)
    g = GpuRun(wk, q, k, v).run()
    perm = np.ascontiguousarray(np.broadcast_to(oracle.perm_static(wl.grid), (wl.batch, wl.n_video)))
    check_sampled(g, q, k, v, perm, sample_bh=[(1, 5)])
    del g
    torch.cuda.empty_cache()


def test_prefix_sampled():
    wl = S.WORKLOADS["prefix"]
    print(f"\n[case] {wl}", flush=True)
    q, k, v = S.qkv(wl)
    g = GpuRun(wl, q, k, v).run()
    perm = np.ascontiguousarray(np.broadcast_to(oracle.perm_static(wl.grid), (wl.batch, wl.n_video)))
    assert np.array_equal(g.perm(), perm)
    check_sampled(g, q, k, v, perm, sample_bh=[(0, 0), (0, 17)])
    del g
    torch.cuda.empty_cache()


def test_dynamic_sampled():
    wl = S.WORKLOADS["prism720p_dynamic"]
    print(f"\n[case] {wl}", flush=True)
    q, k, v = S.qkv(wl)
    g = GpuRun(wl, q, k, v).run()
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
    check_sampled(g, q, k, v, perm, sample_bh=[(0, 3), (1, 20)])
    del g
    torch.cuda.empty_cache()
