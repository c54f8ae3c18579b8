"""Seeded random small problems through the whole path (permutation, plan,
forward, scatter, backward) against the oracle: head dim 64 or 128, any of
the nine 64-token tile shapes, grids that are or are not whole numbers of
tiles (padded mode), with or without a dense prefix, one or two batch
elements and up to three heads, keep from 1 to every tile.  The rules are
those of the other parity tests: permutation, gathers, means and scatter
bit-exact, lists exact outside near ties, attention and gradients within the
forward's and the backward's tolerances; the raster-I/O path (Q's means
alone, bsa_forward_raster) equal to the tiled one bit for bit."""
import numpy as np
import pytest
import torch

import block_sparse_attention_39_amd as bsa
import oracle
import synthetic as S
from parity import (DeviceRun, bits_to_f64, check_lse, check_output, check_selection, kfrag_layout, to_bits, to_dev,
                    vfrag_layout)

pytestmark = pytest.mark.gpu

TILES = [(4, 4, 4), (2, 4, 8), (2, 8, 4), (8, 4, 2), (4, 2, 8), (4, 8, 2), (8, 2, 4), (2, 2, 16), (16, 2, 2)]


def random_workload(seed):
    rng = np.random.default_rng(1000 + seed)
    tile = TILES[rng.integers(len(TILES))]
    while True:
        grid = tuple(int(rng.integers(1, 3 * t + 1)) for t in tile)
        slots = int(np.prod([-(-g // t) * t for g, t in zip(grid, tile)]))
        if slots <= 64 * 40:
            break
    nvt = slots // 64
    padded = any(g % t for g, t in zip(grid, tile)) or bool(rng.integers(2))
    return S.Workload(f"rand{seed}", int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.choice([64, 128])),
                      grid, int(rng.integers(1, nvt + 1)), seed=2000 + seed, n_prefix=int(rng.choice([0, 64, 128])),
                      tile=tile, padded=padded)


def check_grad(got, ref, what):
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    ref_mx, ref_mean = float(np.abs(ref).max()), float(np.abs(ref).mean())
    print(f"[{what}] max|err| {mx:.3e} (ref max {ref_mx:.3e})", flush=True)
    assert np.isfinite(got).all(), what
    assert mx <= 2e-2 * ref_mx + 1e-6 and mean <= 1e-2 * ref_mean + 1e-7, what


@pytest.mark.parametrize("seed", range(12))
def test_random_problem(seed):
    wl = random_workload(seed)
    print(f"\n[case] {wl} slots {wl.n_video_slots}", flush=True)
    q, k, v = S.qkv(wl)
    do = S.tensor(wl, "do")
    g = DeviceRun(wl, q, k, v).run()
    npf, scale, D = wl.n_prefix, float(np.float32(wl.scale)), wl.head_dim
    p1 = oracle.perm_static_padded(wl.grid, wl.tile)
    perm = np.ascontiguousarray(np.broadcast_to(p1, (wl.batch, p1.size)))
    assert np.array_equal(g.perm(), perm)
    tiled = [oracle.gather_padded(x, p1, npf) for x in (q, k, v, do)]
    qt, kt, vt, dot = tiled
    assert np.array_equal(to_bits(g.att.q_t), qt)
    assert np.array_equal(to_bits(g.att.k_f).reshape(-1), kfrag_layout(kt).reshape(-1))
    assert np.array_equal(to_bits(g.att.v_f).reshape(-1), vfrag_layout(vt).reshape(-1))
    qp, kp = oracle.pool_padded(qt, p1, npf), oracle.pool_padded(kt, p1, npf)
    gq, gk = g.pooled()
    assert np.array_equal(gq, qp) and np.array_equal(gk, kp)
    gidx = g.block_idx()
    check_selection(gidx, qp, kp, wl.keep_tiles)
    real = oracle.key_real(p1, npf)
    nqt = wl.n_tiled_tokens // 64
    tiles = np.arange(nqt, dtype=np.int32)
    rows = real.reshape(nqt, 64).astype(bool)
    o_t, lse = to_bits(g.att.o_t), g.att.lse.cpu().numpy()
    for b in range(wl.batch):
        for h in range(wl.heads):
            ref, ref_lse = oracle.attention_padded(qt[b, h], kt[b, h], vt[b, h], npf, gidx[b, h], real, scale, tiles)
            check_output(o_t[b, h].reshape(nqt, 64, D)[rows], ref[rows], f"b{b} h{h}")
            check_lse(lse[b, h].reshape(nqt, 64)[rows], ref_lse[rows], qt[b, h].reshape(nqt, 64, D)[rows],
                      kt[b, h], scale, f"lse b{b} h{h}")
    assert np.array_equal(to_bits(g.out), oracle.scatter_padded(o_t, p1, npf, wl.n_video))
    # the raster-I/O path: the same means, lists, output and lse bit for bit
    ra = bsa.BlockSparseAttention(g.desc, with_lse=True)
    rout = torch.full_like(g.q.view(torch.int16), 0x7FC1).view(torch.bfloat16)
    ra(g.q, g.k, g.v, rout)
    torch.cuda.synchronize()
    rq, rk = bsa.pooled_views(g.desc, ra.workspace)
    assert np.array_equal(rq.cpu().numpy(), gq) and np.array_equal(rk.cpu().numpy(), gk)
    assert torch.equal(ra.block_idx, g.att.block_idx)
    assert torch.equal(rout.view(torch.int16), g.out.view(torch.int16)) and torch.equal(ra.lse, g.att.lse)
    # gradients
    dq, dk, dv = (torch.empty_like(g.q) for _ in range(3))
    ws = torch.empty(max(bsa.backward_workspace_size(g.desc), 256), dtype=torch.uint8, device="cuda")
    bsa.backward(g.desc, g.q, g.k, g.v, g.out, to_dev(do), g.att.lse, g.att.perm, g.att.block_idx, dq, dk, dv, ws)
    torch.cuda.synchronize()
    ref = oracle.backward_full_padded(qt, kt, vt, dot, npf, gidx, np.broadcast_to(real, (wl.batch, real.size)),
                                      scale)
    real_slots = np.nonzero(p1 >= 0)[0]
    src = np.empty(npf + real_slots.size, np.int64)
    src[:npf] = np.arange(npf)
    src[npf + p1[real_slots]] = npf + real_slots
    for name, dev, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_grad(bits_to_f64(to_bits(dev)), r[:, :, src].transpose(0, 2, 1, 3), name)
