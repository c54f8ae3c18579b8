"""The raster-I/O path: bsa_permute(POOL) for Q's tile means and
bsa_forward_raster, which reads Q and writes O in the raster layout itself.

* Against the tiled path (gather, select, forward, scatter) on every small
  parity workload and every ragged grid: Q's means, the kept lists, the
  output and the lse equal bit for bit, with the raster output first filled
  with a NaN pattern so that a row the kernel failed to write shows; the same
  for the one-block-per-tile launch (no workspace).
* Against the oracle on its own: the raster output, gathered into tile order
  by the oracle, within the output tolerance of the oracle's attention, and
  Q's means bit-exact against the oracle's pooling of the oracle's gather.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_39_amd as bsa
import oracle
import synthetic as S
from parity import GpuRun, check_output, desc_for, to_bits
from test_gpu_padded import CASES as PADDED_CASES
from test_gpu_parity import CASES as PARITY_CASES

pytestmark = pytest.mark.gpu

NAN_BITS = 0x7FC1  # a quiet NaN in bf16


def raster_run(wl, g, grouped=True):
    """The raster path on the inputs of GpuRun g, into a NaN-filled output."""
    att = bsa.BlockSparseAttention(g.desc, with_lse=True, grouped=grouped)
    out = torch.full_like(g.q.view(torch.int16), NAN_BITS).view(torch.bfloat16)
    att(g.q, g.k, g.v, out)
    torch.cuda.synchronize()
    return att, out


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))


CASES = PARITY_CASES + PADDED_CASES


@pytest.mark.parametrize("wl", CASES, ids=[c.name for c in CASES])
def test_raster_path_equals_tiled_path(wl):
    print(f"\n[case] {wl}", flush=True)
    q, k, v = S.qkv(wl)
    g = GpuRun(wl, q, k, v).run()
    for grouped in (True, False):
        att, out = raster_run(wl, g, grouped)
        n = wl.n_video_slots
        assert same_bits(att.perm[:, :n], g.att.perm[:, :n])
        if wl.n_video:
            gq, gk = g.pooled()
            rq, rk = bsa.pooled_views(g.desc, att.workspace)
            assert np.array_equal(rq.cpu().numpy(), gq) and np.array_equal(rk.cpu().numpy(), gk)
            assert same_bits(att.block_idx, g.att.block_idx)
        assert same_bits(out, g.out), f"raster output differs (grouped={grouped})"
        assert torch.equal(att.lse, g.att.lse)
        print(f"[raster] grouped={grouped}: output, lse, lists and means equal", flush=True)


ORACLE_CASES = [PARITY_CASES[1], PARITY_CASES[3], PARITY_CASES[10], PADDED_CASES[0], PADDED_CASES[1]]


@pytest.mark.parametrize("wl", ORACLE_CASES, ids=[c.name for c in ORACLE_CASES])
def test_raster_path_matches_oracle(wl):
    print(f"\n[case] {wl}", flush=True)
    q, k, v = S.qkv(wl)
    g = GpuRun(wl, q, k, v)  # inputs and descriptor only
    att, out = raster_run(wl, g)
    npf, scale = wl.n_prefix, float(np.float32(wl.scale))
    perm = att.perm.cpu().numpy()[:, :wl.n_video_slots]
    if wl.padded:
        p1 = oracle.perm_static_padded(wl.grid, wl.tile)
        assert np.array_equal(perm, np.broadcast_to(p1, perm.shape))
        gat = lambda x: oracle.gather_padded(x, p1, npf)
        pool = lambda x: oracle.pool_padded(x, p1, npf)
        real = oracle.key_real(p1, npf)
    else:
        if not wl.dynamic:
            assert np.array_equal(perm, np.broadcast_to(oracle.perm_static(wl.grid, wl.tile), perm.shape))
        gat = lambda x: oracle.gather(x, perm, npf)
        pool = lambda x: oracle.pool(x, npf)
        real = None
    qt, kt, vt = gat(q), gat(k), gat(v)
    o_t = gat(to_bits(out))  # the raster output in tile order (zeros in padding slots)
    rq, _ = bsa.pooled_views(g.desc, att.workspace)
    assert np.array_equal(rq.cpu().numpy(), pool(qt))
    gidx = att.block_idx.cpu().numpy()[:, :, :wl.n_video_tiles, :wl.keep_tiles]
    nqt = wl.n_tiled_tokens // 64
    tiles = np.arange(nqt, dtype=np.int32)
    if nqt > 32:
        tiles = np.sort(np.random.default_rng(wl.seed).choice(nqt, size=32, replace=False)).astype(np.int32)
    worst = 0.0
    for b in range(wl.batch):
        for h in range(wl.heads):
            if real is None:
                ref, _ = oracle.attention(qt[b, h], kt[b, h], vt[b, h], npf, gidx[b, h], scale, tiles)
            else:
                ref, _ = oracle.attention_padded(qt[b, h], kt[b, h], vt[b, h], npf, gidx[b, h], real, scale, tiles)
            got = o_t[b, h].reshape(nqt, 64, wl.head_dim)[tiles]
            if real is not None:  # padding query rows are not outputs
                rows = real.reshape(nqt, 64)[tiles].astype(bool)
                got, ref = got[rows], ref.reshape(got.shape)[rows]
            mx, _ = check_output(got, ref, f"b{b} h{h}")
            worst = max(worst, mx)
    print(f"[raster] worst max|err| {worst:.3e} against the oracle", flush=True)
