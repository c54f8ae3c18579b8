"""GPU parity of the backward at the full Prism-scale 720p size (grid 32x48x80,
122,880 tokens, batch 2, 24 heads, head_dim 128, 480 kept tiles), in the
launch configuration the benchmark times, on sampled tiles the oracle
computes one by one:

* dQ of sampled query tiles: entirely from the oracle (its lse and output of
  those tiles give Delta), with the GPU's selection;
* dK and dV of sampled key tiles: also entirely from the oracle.  A key
  tile collects from the query tiles that keep it (about 480 each); the
  oracle's forward runs on exactly those query tiles for their lse and
  Delta = dO . O.  The GPU forward's lse on the same rows is compared with
  the oracle's as an extra check.

Tolerance as at the small sizes: max |err| <= 2e-2 * max |ref| and
mean |err| <= 1e-2 * mean |ref| over the sampled tiles of a tensor.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_39_amd as bsa
import oracle
import synthetic as S
from parity import DeviceRun, attending_tiles, bits_to_f64, check_lse, oracle_lse_delta_rows, to_bits, to_dev

pytestmark = pytest.mark.gpu

RTOL_MAX = 2e-2
RTOL_MEAN = 1e-2
SAMPLE_BH = [(0, 0), (1, 17)]
N_QTILES = 6
N_KTILES = 2


def check(got, ref, what):
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    ref_mx, ref_mean = float(np.abs(ref).max()), float(np.abs(ref).mean())
    print(f"[{what}] max|err| {mx:.3e} (ref max {ref_mx:.3e}), mean|err| {mean:.3e} (ref mean {ref_mean:.3e})",
          flush=True)
    assert np.isfinite(got).all(), what
    assert mx <= RTOL_MAX * ref_mx + 1e-6, what
    assert mean <= RTOL_MEAN * ref_mean + 1e-7, what


def test_prism720p_backward_sampled():
    wl = S.WORKLOADS["prism720p"]
    print(f"\n[case] {wl}", flush=True)
    q, k, v = S.qkv(wl)
    do = S.tensor(wl, "do")
    g = DeviceRun(wl, q, k, v).run()
    dO = to_dev(do)
    dq, dk, dv = (torch.empty_like(g.q) for _ in range(3))
    ws = torch.empty(bsa.backward_workspace_size(g.desc), dtype=torch.uint8, device="cuda")
    bsa.backward(g.desc, g.q, g.k, g.v, g.out, dO, g.att.lse, g.att.perm, g.att.block_idx, dq, dk, dv, ws)
    torch.cuda.synchronize()
    print("[gpu] backward done", flush=True)

    npf, scale = wl.n_prefix, float(np.float32(wl.scale))
    perm = g.perm()
    nqt = wl.n_tokens // 64
    gidx = g.att.block_idx.cpu().numpy()[:, :, :wl.n_video_tiles, :wl.keep_tiles]
    lse_gpu = g.att.lse.cpu().numpy()
    rng = np.random.default_rng(wl.seed + 7)
    for b, h in SAMPLE_BH:
        sl = lambda x: np.ascontiguousarray(x[b:b + 1, :, h:h + 1])
        qt, kt, vt, dot = (oracle.gather(sl(x), perm[b:b + 1], npf)[0, 0] for x in (q, k, v, do))
        grads = [bits_to_f64(oracle.gather(to_bits(x[b:b + 1, :, h:h + 1]), perm[b:b + 1], npf)[0, 0])
                 .reshape(nqt, 64, wl.head_dim) for x in (dq, dk, dv)]

        # dQ: lse and Delta of the sampled rows from the oracle's own forward
        qtiles = np.sort(rng.choice(nqt, size=N_QTILES, replace=False)).astype(np.int32)
        o_ref, lse_ref = oracle.attention(qt, kt, vt, npf, gidx[b, h], scale, qtiles)
        lse = np.zeros(wl.n_tokens)
        delta = np.zeros(wl.n_tokens)
        rows = (qtiles[:, None] * 64 + np.arange(64)).reshape(-1)
        lse[rows] = lse_ref.reshape(-1)
        delta[rows] = (o_ref.reshape(-1, wl.head_dim) * bits_to_f64(dot)[rows]).sum(1)
        ref_dq = oracle.backward_dq(qt, kt, vt, dot, lse, delta, npf, gidx[b, h], scale, qtiles)
        check(grads[0][qtiles], ref_dq, f"dq b{b} h{h} tiles {qtiles.tolist()}")

        # dK, dV: lse and Delta of every query tile that attends a sampled key
        # tile, from the oracle's forward on those tiles
        ktiles = np.sort(rng.choice(nqt, size=N_KTILES, replace=False)).astype(np.int32)
        need = attending_tiles(ktiles, wl.n_prefix_tiles, wl.n_video_tiles, idx=gidx[b, h])
        lse_all, delta_all, rows = oracle_lse_delta_rows(
            lambda t: oracle.attention(qt, kt, vt, npf, gidx[b, h], scale, t), need, dot, wl.n_tokens,
            wl.head_dim)
        print(f"[dk/dv b{b} h{h}] oracle forward on the {need.size} query tiles that attend {ktiles.tolist()}",
              flush=True)
        check_lse(lse_gpu[b, h].reshape(nqt, 64)[need], lse_all[rows].reshape(-1, 64),
                  qt.reshape(nqt, 64, -1)[need], kt, scale, f"lse b{b} h{h} (extra check)")
        ref_dk, ref_dv = oracle.backward_dkdv(qt, kt, vt, dot, lse_all, delta_all, npf, gidx[b, h], scale,
                                              ktiles)
        check(grads[1][ktiles], ref_dk, f"dk b{b} h{h} tiles {ktiles.tolist()}")
        check(grads[2][ktiles], ref_dv, f"dv b{b} h{h} tiles {ktiles.tolist()}")
    del g, dq, dk, dv, ws
    torch.cuda.empty_cache()
