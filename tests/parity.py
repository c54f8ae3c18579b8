"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare it with the CPU oracle.

Comparison rules:
* permutation, gather, scatter: bit-exact;
* pooled tile means: bit-exact (both sides sum the 64 bf16 values exactly and
  round once to float);
* kept tile indices: bit-exact on every row whose k-th / (k+1)-th score gap is
  at least 1e-4 of the larger of the two scores (the contract); rows below
  that are near ties, counted apart.  The selection kernel promises more (the
  exact top k of the double scores summed in channel order, as the oracle
  sums them), so near-tie rows are compared exactly too.  Rows whose gap lies
  within twice the rounding bound of a D-term float dot product,
  gamma_D * sum_d |qbar_d kbar_jd| (gamma_D = D u / (1 - D u), u = 2^-24), are
  the ones a float-only selection could get wrong; they are counted as well;
* attention output: max |err| <= 2e-2 and mean |err| <= 2e-3 against the fp64
  oracle run with the GPU's own selection (identical to the oracle's on every
  row that is not a near tie);
* log-sum-exp: per query |err| <= 2^-8 (the bf16 rounding of the weights moves
  the normaliser by at most 2^-8 relative: bf16 keeps 8 significant bits, and
  |log(1 + x)| <= |x| for x >= 0, 1.004 |x| just below 0, covered by the
  second term's slack) + 2 * scale * gamma_D * |q| max_j |k_j|
  (float accumulation of the logits).
"""
from __future__ import annotations

import numpy as np
import torch

import block_sparse_attention_39_amd as bsa
import oracle
import synthetic as S

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
REL_TIE = 1e-4


def to_dev(x_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bits_to_f64(b: np.ndarray) -> np.ndarray:
    return S.bf16_bits_to_f32(b).astype(np.float64)


def desc_for(wl: S.Workload):
    return bsa.make_desc(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.keep_tiles, scale=wl.scale,
                         n_prefix=wl.n_prefix, dynamic=wl.dynamic, tile=wl.tile, tau=wl.tau, padded=wl.padded)


class DeviceRun:
    """The whole path on the GPU, every intermediate kept for inspection."""

    def __init__(self, wl: S.Workload, q, k, v, with_lse=True):
        self.wl = wl
        self.desc = desc_for(wl)
        self.att = bsa.BlockSparseAttention(self.desc, with_lse=with_lse)
        self.q, self.k, self.v = (to_dev(x) for x in (q, k, v))
        self.out = torch.empty_like(self.q)

    def run(self):
        a = self.att
        a.build(self.q)
        a.gather_qkv(self.q, self.k, self.v)
        a.plan()
        a.forward()
        a.scatter_out(self.out)
        torch.cuda.synchronize()
        return self

    def perm(self):
        return self.att.perm.cpu().numpy()[:, :self.wl.n_video_slots]

    def shape_map(self):
        return None if self.att.shape_map is None else self.att.shape_map.cpu().numpy()

    def pooled(self):
        qb, kb = bsa.pooled_views(self.desc, self.att.workspace)
        return qb.cpu().numpy(), kb.cpu().numpy()

    def block_idx(self):
        return self.att.block_idx.cpu().numpy()[:, :, :self.wl.n_video_tiles, :self.wl.keep_tiles]


def _swap23(m: np.ndarray) -> np.ndarray:
    return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1)


def kfrag_layout(x_tiled: np.ndarray) -> np.ndarray:
    """Tiled [B, H, Ntot, D] -> the K-fragment layout [B, H, Ntot/64, 2, D/16, 64, 8]
    as the C header defines it: element [t][kh][s][l][e] is channel
    16 s + 8 (l // 32) + e of token 32 kh + swap23(l % 32) of tile t."""
    B, H, N, D = x_tiled.shape
    t = x_tiled.reshape(B, H, N // 64, 64, D)
    kh = np.arange(2)[:, None, None, None]
    s = np.arange(D // 16)[None, :, None, None]
    lane = np.arange(64)[None, None, :, None]
    e = np.arange(8)[None, None, None, :]
    tok = 32 * kh + _swap23(lane % 32) + 0 * s + 0 * e
    ch = 16 * s + 8 * (lane // 32) + e + 0 * kh
    return np.ascontiguousarray(t[:, :, :, tok, ch])


def vfrag_layout(x_tiled: np.ndarray) -> np.ndarray:
    """Tiled [B, H, Ntot, D] -> the V-fragment layout [B, H, Ntot/64, 2, D/32, 2, 64, 8]:
    element [t][kh][i][c][l][e] is channel 32 i + l % 32 of token
    32 kh + 16 c + 8 (l // 32) + e of tile t."""
    B, H, N, D = x_tiled.shape
    t = x_tiled.reshape(B, H, N // 64, 64, D)
    kh = np.arange(2)[:, None, None, None, None]
    i = np.arange(D // 32)[None, :, None, None, None]
    c = np.arange(2)[None, None, :, None, None]
    lane = np.arange(64)[None, None, None, :, None]
    e = np.arange(8)[None, None, None, None, :]
    tok = 32 * kh + 16 * c + 8 * (lane // 32) + e + 0 * i
    ch = 32 * i + lane % 32 + 0 * kh + 0 * c + 0 * e
    return np.ascontiguousarray(t[:, :, :, tok, ch])


def gamma(n: int) -> float:
    u = 2.0 ** -24
    return n * u / (1.0 - n * u)


def near_tie_rows(s_k, s_k1):
    """The contract's near ties: k-th and (k+1)-th scores closer than 1e-4 of
    the larger of the two, or both zero.  k = n has no (k+1)-th score."""
    gap = s_k - s_k1
    denom = np.maximum(np.abs(s_k), np.abs(s_k1))
    flag = (denom == 0) | (gap < REL_TIE * denom)
    return np.where(np.isnan(s_k1), False, flag)


def gamma_band_rows(s_k, s_k1, mag, D):
    """Rows whose gap is within twice the float dot product's rounding bound
    (where a selection from float scores alone could differ)."""
    flag = (s_k - s_k1) <= 2.0 * gamma(D) * mag
    return np.where(np.isnan(s_k1), False, flag)


def check_selection(gpu_idx, qp, kp, k, rows=None):
    """Compare GPU block_idx (rows of one (b, h) or all) with the oracle's.

    qp, kp: pooled float32 [B,H,n,D] (the oracle's); gpu_idx: [B,H,nrows,k].
    Returns (rows outside the near-tie band, near-tie rows, float-band rows);
    every row is compared exactly."""
    o_idx, s_k, s_k1, mag = oracle.topk(qp, kp, k, rows=rows)
    D = qp.shape[-1]
    near = near_tie_rows(s_k, s_k1)
    clear = ~near
    assert np.array_equal(gpu_idx[clear], o_idx[clear]), "kept tiles differ on a row without a near tie"
    # the kernel's own promise: the exact double top k on near-tie rows too
    assert np.array_equal(gpu_idx[near], o_idx[near]), "kept tiles differ on a near-tie row"
    return int(clear.sum()), int(near.sum()), int(gamma_band_rows(s_k, s_k1, mag, D).sum())


def lse_bound(q_tiles_bits, k_bits, scale):
    """Per-query bound on |lse_gpu - lse_oracle|; q_tiles_bits [nq, 64, D],
    k_bits [Ntot, D] (all keys of the head)."""
    D = q_tiles_bits.shape[-1]
    qn = np.linalg.norm(bits_to_f64(q_tiles_bits), axis=-1)
    kmax = np.linalg.norm(bits_to_f64(k_bits), axis=-1).max()
    return 2.0 ** -8 + 2.0 * scale * gamma(D) * qn * kmax


def check_lse(lse_gpu, lse_ref, q_tiles_bits, k_bits, scale, what="lse"):
    err = np.abs(lse_gpu.astype(np.float64) - lse_ref)
    bound = lse_bound(q_tiles_bits, k_bits, scale)
    assert np.all(err <= bound), f"{what}: worst excess {float((err - bound).max()):.3e}"
    return float(err.max())


def check_output(o_gpu_bits, o_ref, what="output"):
    err = np.abs(bits_to_f64(o_gpu_bits) - o_ref)
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{what}: max {mx:.3e} mean {mean:.3e}"
    return mx, mean


def attending_tiles(ktiles, n_prefix_tiles, nvt, row_ptr=None, col=None, idx=None):
    """Tiled query tile numbers whose key set holds any of the tiled key tiles
    ``ktiles``: every prefix query tile, and the video query tiles whose kept
    list (fixed keep ``idx [nvt, k]``, or CSR ``row_ptr``/``col``) holds a
    sampled video key tile (a sampled prefix key tile is attended by all)."""
    kt = np.asarray(ktiles)
    if np.any(kt < n_prefix_tiles):
        return np.arange(n_prefix_tiles + nvt, dtype=np.int32)
    kv = kt - n_prefix_tiles
    if idx is not None:
        hit = np.isin(idx, kv).any(axis=1)
    else:
        hit = np.array([np.isin(col[row_ptr[i]:row_ptr[i + 1]], kv).any() for i in range(nvt)])
    vid = n_prefix_tiles + np.nonzero(hit)[0]
    return np.concatenate([np.arange(n_prefix_tiles), vid]).astype(np.int32)


def oracle_lse_delta_rows(attention, qtiles, dot_bits, n_rows, D):
    """lse and Delta = dO . O of the query tiles ``qtiles`` from the oracle's
    own forward (``attention(qtiles) -> (o, lse)``), as float64 arrays over all
    ``n_rows`` tiled rows (zero elsewhere: the oracle's dK/dV read only the
    rows of queries that attend the sampled key tiles)."""
    o_ref, lse_ref = attention(np.asarray(qtiles, np.int32))
    lse = np.zeros(n_rows)
    delta = np.zeros(n_rows)
    rows = (np.asarray(qtiles)[:, None] * 64 + np.arange(64)).reshape(-1)
    lse[rows] = lse_ref.reshape(-1)
    delta[rows] = (o_ref.reshape(-1, D) * bits_to_f64(dot_bits)[rows]).sum(1)
    return lse, delta, rows
