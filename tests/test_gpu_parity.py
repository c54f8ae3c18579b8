"""GPU parity of every step of the path against the CPU oracle, on small
workloads the oracle finishes in seconds: several tiles, ragged tile counts
(not multiples of the 64-lane or 256-thread blocking), odd k, k = 1, k = n,
head dims 64 and 128, non-default static tile shapes, a dense prefix, a
prefix with no video at all, and dynamic tile shapes."""
import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from parity import DeviceRun, bits_to_f64, check_lse, check_output, check_selection, kfrag_layout, to_bits, vfrag_layout

pytestmark = pytest.mark.gpu

W = S.Workload
CASES = [
    S.WORKLOADS["tiny"],
    W("ragged", 2, 3, 128, (8, 8, 12), 5, seed=11),
    W("prefix128", 1, 2, 128, (8, 8, 16), 3, seed=12, n_prefix=128),
    W("prefix_d64", 2, 2, 64, (4, 8, 24), 2, seed=13, n_prefix=192),
    W("dense_k_eq_n", 1, 2, 128, (8, 8, 8), 8, seed=14),
    W("k1_d64", 1, 3, 64, (8, 8, 12), 1, seed=15),
    W("tile2x4x8", 1, 2, 128, (8, 16, 16), 4, seed=16, tile=(2, 4, 8)),
    W("tile16x2x2", 1, 1, 64, (16, 4, 8), 3, seed=20, tile=(16, 2, 2)),
    W("prefix_only", 1, 2, 128, (0, 0, 0), 0, seed=17, n_prefix=256),
    W("many_tiles", 1, 1, 64, (16, 32, 40), 77, seed=21),
    W("dynamic", 2, 2, 128, (16, 16, 32), 6, seed=18, dynamic=True, recipe="field"),
    W("dynamic_prefix_d64", 1, 2, 64, (16, 16, 16), 4, seed=19, dynamic=True, recipe="field", n_prefix=64),
]


def reference_perm(wl, q, g):
    B = wl.batch
    if wl.n_video == 0:
        return np.zeros((B, 0), np.int32), None
    if not wl.dynamic:
        return np.ascontiguousarray(np.broadcast_to(oracle.perm_static(wl.grid, wl.tile), (B, wl.n_video))), None
    st = oracle.shape_stats(q, wl.n_prefix, wl.grid)
    shape_o, near = oracle.shape_choose(st, wl.grid, float(np.float32(wl.tau)))
    gs = g.shape_map()
    clear = near == 0
    assert np.array_equal(gs[clear], shape_o[clear]), "shape choice differs away from a threshold"
    # near-threshold regions: follow the GPU's (valid) choice
    return oracle.perm_dynamic(gs, wl.grid), shape_o


@pytest.mark.parametrize("wl", CASES, ids=[c.name for c in CASES])
def test_path_matches_oracle(wl):
    print(f"\n[case] {wl}", flush=True)
    q, k, v = S.qkv(wl)
    g = DeviceRun(wl, q, k, v).run()
    npf, scale = wl.n_prefix, float(np.float32(wl.scale))

    # permutation
    perm, _ = reference_perm(wl, q, g)
    if wl.n_video:
        assert np.array_equal(g.perm(), perm)

    # gather: exact copies
    qt, kt, vt = (oracle.gather(x, perm, npf) for x in (q, k, v))
    for ref, dev in ((qt, g.att.q_t), (kfrag_layout(kt), g.att.k_f), (vfrag_layout(vt), g.att.v_f)):
        assert np.array_equal(to_bits(dev).reshape(ref.shape), ref)

    # plan: pooled means bit-exact, kept tiles exact outside near ties
    if wl.n_video:
        qp, kp = oracle.pool(qt, npf), oracle.pool(kt, npf)
        gq, gk = g.pooled()
        assert np.array_equal(gq, qp) and np.array_equal(gk, kp)
        gidx = g.block_idx()
        n_exact, n_near, n_gamma = check_selection(gidx, qp, kp, wl.keep_tiles)
        print(f"[plan] rows exact {n_exact}, near ties {n_near}", flush=True)
    else:
        gidx = np.zeros((wl.batch, wl.heads, 0, 0), np.int32)

    # forward, against the oracle run with the GPU's selection
    o_t = to_bits(g.att.o_t)
    lse = g.att.lse.cpu().numpy()
    nqt = wl.n_tokens // 64
    rng = np.random.default_rng(wl.seed)
    tiles = np.arange(nqt, dtype=np.int32)
    if nqt > 64:
        tiles = np.sort(rng.choice(nqt, size=64, replace=False)).astype(np.int32)
    worst = 0.0
    for b in range(wl.batch):
        for h in range(wl.heads):
            ref, ref_lse = oracle.attention(qt[b, h], kt[b, h], vt[b, h], npf, gidx[b, h], scale, tiles)
            got = o_t[b, h].reshape(nqt, 64, wl.head_dim)[tiles]
            mx, _ = check_output(got, ref, f"b{b} h{h}")
            worst = max(worst, mx)
            check_lse(lse[b, h].reshape(nqt, 64)[tiles], ref_lse, qt[b, h].reshape(nqt, 64, -1)[tiles], kt[b, h],
                      scale, f"lse b{b} h{h}")
    print(f"[forward] worst max|err| {worst:.3e}", flush=True)

    # scatter: exact copies back to raster order
    assert np.array_equal(to_bits(g.out), oracle.scatter(o_t, perm, npf))


def test_outputs_are_deterministic():
    wl = W("det", 2, 2, 128, (8, 8, 16), 5, seed=31, n_prefix=64)
    q, k, v = S.qkv(wl)
    g = DeviceRun(wl, q, k, v).run()
    first = (to_bits(g.out).copy(), g.block_idx().copy())
    g.run()
    assert np.array_equal(first[0], to_bits(g.out))
    assert np.array_equal(first[1], g.block_idx())


def test_planted_selection_and_ties_on_gpu():
    """Planted rankings through the whole plan: tiles whose pooled keys grow
    along a common direction rank by index (the top k are the last k); equal
    pooled keys keep the lowest indices."""
    wl = W("planted", 1, 2, 64, (8, 8, 16), 5, seed=0)
    n, D = wl.n_video_tiles, wl.head_dim
    u = np.linspace(0.5, 1.5, D).astype(np.float32)
    perm = oracle.perm_static(wl.grid)
    qt = np.broadcast_to(u, (1, 2, wl.n_video, D)).astype(np.float32).copy()
    kt = np.empty((1, 2, wl.n_video, D), np.float32)
    tile_of_slot = np.arange(wl.n_video) // 64
    kt[0, 0] = (tile_of_slot[:, None] * 0.25 * u[None, :])   # head 0: strictly increasing scores
    kt[0, 1] = 0.5 * u[None, :]                              # head 1: every score equal
    # back to raster order so that the GPU gather produces exactly these tiles
    qr = np.empty((1, wl.n_video, 2, D), np.float32)
    kr = np.empty_like(qr)
    qr[0, perm] = qt[0].transpose(1, 0, 2)
    kr[0, perm] = kt[0].transpose(1, 0, 2)
    q, k = S.to_bf16_bits(qr), S.to_bf16_bits(kr)
    v = S.to_bf16_bits(np.ones_like(qr))
    g = DeviceRun(wl, q, k, v).run()
    idx = g.block_idx()
    assert np.all(idx[0, 0] == np.arange(n - 5, n))
    assert np.all(idx[0, 1] == np.arange(5))
    # V == 1 everywhere: the output is exactly 1
    assert np.all(bits_to_f64(to_bits(g.out)) == 1.0)


def test_large_logits_stay_finite():
    """Scores far above the rescale margin (row maxima growing along the key
    list) must neither overflow nor lose the normalisation."""
    wl = W("big", 1, 1, 128, (8, 8, 8), 8, seed=5)
    q, k, v = S.qkv(wl)
    qf = S.bf16_bits_to_f32(q) * 6.0
    kf = S.bf16_bits_to_f32(k) * 6.0
    q, k = S.to_bf16_bits(qf), S.to_bf16_bits(kf)
    g = DeviceRun(wl, q, k, v).run()
    perm = oracle.perm_static(wl.grid)
    qt, kt, vt = (oracle.gather(x, perm, 0) for x in (q, k, v))
    ref, _ = oracle.attention(qt[0, 0], kt[0, 0], vt[0, 0], 0, g.block_idx()[0, 0], float(np.float32(wl.scale)),
                              np.arange(8, dtype=np.int32))
    got = to_bits(g.att.o_t)[0, 0].reshape(8, 64, 128)
    assert np.isfinite(bits_to_f64(got)).all()
    check_output(got, ref, "large logits")
    torch.cuda.synchronize()


@pytest.mark.parametrize("wl", [CASES[1], CASES[2], CASES[9]], ids=["ragged", "prefix128", "many_tiles"])
def test_grouped_and_plain_launch_agree(wl):
    """The grouped persistent launch (workspace given) only changes the order
    in which query tiles are scheduled: outputs are bit-identical to one block
    per query tile."""
    q, k, v = S.qkv(wl)
    g = DeviceRun(wl, q, k, v).run()
    grouped = to_bits(g.att.o_t).copy(), g.att.lse.cpu().numpy().copy()
    g.att.grouped = False
    g.run()
    assert np.array_equal(grouped[0], to_bits(g.att.o_t))
    assert np.array_equal(grouped[1], g.att.lse.cpu().numpy())


@pytest.mark.parametrize("growing", [True, False], ids=["growing", "shrinking"])
def test_rescale_path_with_steep_logits(growing):
    """Logits that change by ~50 (base 2) from one key tile to the next: with
    growing logits nearly every slice of every wave overflows the running
    reference and takes the rescale path; with shrinking ones the later
    weights underflow to zero.  Both must match the exact fp64 oracle."""
    wl = W("steep", 1, 2, 128, (8, 8, 16), 16, seed=41)
    n, D = wl.n_video_tiles, wl.head_dim
    perm = oracle.perm_static(wl.grid)
    rng = np.random.default_rng(41)
    qt = (1.0 + 0.1 * rng.standard_normal((1, 2, wl.n_video, D))).astype(np.float32)
    tile_of_slot = np.arange(wl.n_video) // 64
    ramp = 3.0 * (tile_of_slot if growing else (n - 1 - tile_of_slot))
    kt = (ramp[None, None, :, None] + 0.1 * rng.standard_normal((1, 2, wl.n_video, D))).astype(np.float32)
    vt = rng.standard_normal((1, 2, wl.n_video, D)).astype(np.float32)
    # back to raster order so that the GPU gather produces exactly these tiles
    def raster(x):
        r = np.empty((1, wl.n_video, 2, D), np.float32)
        r[0, perm] = x[0].transpose(1, 0, 2)
        return S.to_bf16_bits(r)
    q, k, v = raster(qt), raster(kt), raster(vt)
    g = DeviceRun(wl, q, k, v).run()
    idx = g.block_idx()
    assert np.all(idx == np.arange(n))  # k = n: every tile kept
    qg, kg, vg = (oracle.gather(x, perm, 0) for x in (q, k, v))
    got = to_bits(g.att.o_t)
    lse = g.att.lse.cpu().numpy()
    for h in range(2):
        ref, ref_lse = oracle.attention(qg[0, h], kg[0, h], vg[0, h], 0, idx[0, h], float(np.float32(wl.scale)),
                                        np.arange(n, dtype=np.int32))
        check_output(got[0, h].reshape(n, 64, D), ref, f"h{h}")
        check_lse(lse[0, h].reshape(n, 64), ref_lse, qg[0, h].reshape(n, 64, D), kg[0, h], float(np.float32(wl.scale)),
                  f"lse h{h}")


def test_overlapped_call_equals_sequential_steps():
    """BlockSparseAttention.__call__ gathers V on a side stream beside the
    plan; the result equals the step-by-step path bit for bit, call after
    call (the side stream's work is ordered before the forward each time)."""
    wl = W("overlap", 2, 3, 128, (8, 16, 16), 6, seed=33, n_prefix=64)
    q, k, v = S.qkv(wl)
    g = DeviceRun(wl, q, k, v).run()
    ref = to_bits(g.out).copy()
    for it in range(3):
        out = g.att(g.q, g.k, g.v)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(out), ref), f"call {it}"
