"""GPU parity of the backward (dQ, dK, dV) against the CPU oracle's fp64
gradients, on small workloads the oracle finishes in seconds: several tiles,
ragged tile counts, k = 1, k = n, head dims 64 and 128, a dense prefix, a
prefix with no video, and dynamic tile shapes.

The forward runs first on the GPU (its selection, output and lse are checked
by the forward parity tests); the backward gets the raster inputs, the GPU's
output, a seeded dO and the forward's lse.  The oracle differentiates the same
function exactly, with the GPU's selection.

Tolerance, per gradient tensor: max |err| <= 2e-2 * max |ref| and
mean |err| <= 1e-2 * mean |ref|.  The kernel rounds P and dS to bf16 (relative
at most 2^-8: 8 significant bits) before their products and each gradient to
bf16 at the end (2^-8), and its Delta uses the bf16-rounded forward output;
summed over many terms of mixed sign these stay a small multiple of 2^-8 of
the tensor's scale.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_39_amd as bsa
import oracle
import synthetic as S
from parity import DeviceRun, bits_to_f64, to_bits, to_dev

pytestmark = pytest.mark.gpu

W = S.Workload
CASES = [
    S.WORKLOADS["tiny"],
    W("ragged", 2, 3, 128, (8, 8, 12), 5, seed=11),
    W("prefix128", 1, 2, 128, (8, 8, 16), 3, seed=12, n_prefix=128),
    W("prefix_d64", 2, 2, 64, (4, 8, 24), 2, seed=13, n_prefix=192),
    W("dense_k_eq_n", 1, 2, 128, (8, 8, 8), 8, seed=14),
    W("k1_d64", 1, 3, 64, (8, 8, 12), 1, seed=15),
    W("prefix_only", 1, 2, 128, (0, 0, 0), 0, seed=17, n_prefix=256),
    W("dynamic", 1, 2, 128, (16, 16, 16), 6, seed=18, dynamic=True, recipe="field"),
]
RTOL_MAX = 2e-2
RTOL_MEAN = 1e-2


def run_backward(wl):
    q, k, v = S.qkv(wl)
    do = S.tensor(wl, "do")
    g = DeviceRun(wl, q, k, v).run()
    dO = to_dev(do)
    dq, dk, dv = (torch.empty_like(g.q) for _ in range(3))
    ws = torch.empty(max(bsa.backward_workspace_size(g.desc), 256), dtype=torch.uint8, device="cuda")
    bsa.backward(g.desc, g.q, g.k, g.v, g.out, dO, g.att.lse, g.att.perm, g.att.block_idx, dq, dk, dv, ws)
    torch.cuda.synchronize()
    g.bwd_ws = ws
    return (q, k, v, do), g, (dq, dk, dv)


def check_grad(got, ref, what):
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    ref_mx, ref_mean = float(np.abs(ref).max()), float(np.abs(ref).mean())
    print(f"[{what}] max|err| {mx:.3e} (ref max {ref_mx:.3e}), mean|err| {mean:.3e} (ref mean {ref_mean:.3e})",
          flush=True)
    assert np.isfinite(got).all(), what
    assert mx <= RTOL_MAX * ref_mx + 1e-6, f"{what}: max {mx:.3e} vs {RTOL_MAX} x {ref_mx:.3e}"
    assert mean <= RTOL_MEAN * ref_mean + 1e-7, f"{what}: mean {mean:.3e} vs {RTOL_MEAN} x {ref_mean:.3e}"


@pytest.mark.parametrize("wl", CASES, ids=[c.name for c in CASES])
def test_backward_matches_oracle(wl):
    print(f"\n[case] {wl}", flush=True)
    (q, k, v, do), g, grads = run_backward(wl)
    npf, scale = wl.n_prefix, float(np.float32(wl.scale))
    perm = g.perm()
    qt, kt, vt, dot = (oracle.gather(x, perm, npf) for x in (q, k, v, do))
    gidx = g.block_idx() if wl.n_video else None
    ref = oracle.backward_full(qt, kt, vt, dot, npf, gidx, scale)
    for name, dev, r in zip(("dq", "dk", "dv"), grads, ref):
        got = bits_to_f64(oracle.gather(to_bits(dev), perm, npf))
        check_grad(got, r, name)


def test_backward_is_deterministic():
    wl = W("det", 1, 2, 128, (8, 8, 16), 5, seed=31, n_prefix=64)
    _, _, a = run_backward(wl)
    _, _, b = run_backward(wl)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_backward_stats_count_rounds():
    """The grouped dQ and dK/dV launches record one block round per query
    tile and per key tile (prefix tiles included); on an idle GPU with one
    block per CU no round's start wait gives up."""
    wl = W("bstats", 2, 4, 128, (16, 16, 32), 12, seed=63, n_prefix=128)
    _, g, _ = run_backward(wl)
    dq_gave_up, dq_rounds, kv_gave_up, kv_rounds = bsa.backward_stats(g.desc, g.bwd_ws)
    tiles = wl.batch * wl.heads * (wl.n_prefix_tiles + wl.n_video_tiles)
    print(f"[stats] dQ rounds {dq_rounds} (gave up {dq_gave_up}), dK/dV rounds {kv_rounds} (gave up {kv_gave_up})",
          flush=True)
    assert dq_rounds == tiles and kv_rounds == tiles
    assert dq_gave_up == 0 and kv_gave_up == 0


def test_autograd_attention_matches_direct_calls():
    """bsa.attention as a torch autograd function: its output and the
    gradients that loss.backward() produces equal the raster forward and
    bsa_backward called directly, bit for bit; two calls through one
    BlockSparseAttention before either backward each keep their own
    selection and lse."""
    wl = W("autograd", 1, 2, 128, (8, 8, 16), 4, seed=91, n_prefix=64)
    desc = bsa.make_desc(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.keep_tiles, scale=wl.scale,
                         n_prefix=wl.n_prefix)
    att = bsa.BlockSparseAttention(desc)
    inputs = []
    for seed in (91, 92):
        wk = W("autograd", 1, 2, 128, (8, 8, 16), 4, seed=seed, n_prefix=64)
        q, k, v = S.qkv(wk)
        inputs.append(([to_dev(x).requires_grad_() for x in (q, k, v)], to_dev(S.tensor(wk, "do"))))
    outs = [bsa.attention(*qkv, att) for qkv, _ in inputs]
    for out, (_, do) in zip(outs, inputs):
        (out.float() * do.float()).sum().backward()
    torch.cuda.synchronize()
    ws = torch.empty(bsa.backward_workspace_size(desc), dtype=torch.uint8, device="cuda")
    for out, (qkv, do) in zip(outs, inputs):
        q, k, v = (x.detach() for x in qkv)
        ref = bsa.BlockSparseAttention(desc, with_lse=True)
        o2 = ref(q, k, v)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        bsa.backward(desc, q, k, v, o2, do, ref.lse, ref.perm, ref.block_idx, dq, dk, dv, ws)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(out.detach()), to_bits(o2))
        for got, want in zip((x.grad for x in qkv), (dq, dk, dv)):
            assert np.array_equal(to_bits(got), to_bits(want))
