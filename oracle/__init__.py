"""CPU oracle for block-sparse video self-attention -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It wraps ``liboracle.so`` (plain C, double precision,
OpenMP) built from ``bsa_oracle.c`` in this folder; it shares no code with the
GPU library and the GPU library never imports it.

Each wrapper marshals numpy arrays into the C routine of the same name; the
arithmetic, and the citation of the page passage each step follows, live in
``bsa_oracle.c``.  bf16 tensors travel as ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "bsa_oracle.c")

TILE = 64
# extents (t, h, w) of the nine 64-token shapes, by shape id
SHAPE_NAMES = ["4x4x4", "2x4x8", "2x8x4", "8x4x2", "4x2x8", "4x8x2", "8x2x4", "2x2x16", "16x2x2"]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-std=c11", "-Wall", "-shared", "-fPIC",
               "-o", tmp, SRC_PATH, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.orc_perm_static.argtypes = [i32, i32, i32, i32, i32, i32, P]
        L.orc_perm_static.restype = i32
        L.orc_shape_extent.argtypes = [i32, i32]
        L.orc_shape_extent.restype = i32
        L.orc_shape_stats.argtypes = [P, i32, i32, i32, i32, i32, i32, i32, P]
        L.orc_shape_stats.restype = None
        L.orc_shape_choose.argtypes = [P, i32, i32, i32, i32, f64, f64, P, P]
        L.orc_shape_choose.restype = None
        L.orc_perm_dynamic.argtypes = [P, i32, i32, i32, i32, P]
        L.orc_perm_dynamic.restype = i32
        L.orc_gather.argtypes = [P, P, i32, i32, i64, i32, i32, P]
        L.orc_gather.restype = None
        L.orc_scatter.argtypes = [P, P, i32, i32, i64, i32, i32, P]
        L.orc_scatter.restype = None
        L.orc_pool.argtypes = [P, i32, i32, i32, i32, i32, P]
        L.orc_pool.restype = None
        L.orc_topk.argtypes = [P, P, i32, i32, i32, i32, i32, P, i32, P, P, P, P]
        L.orc_topk.restype = None
        L.orc_attention.argtypes = [P, P, P, i32, i32, i32, i32, P, f64, P, i32, P, P]
        L.orc_attention.restype = None
        L.orc_attention_csr.argtypes = [P, P, P, i32, i32, i32, P, P, f64, P, i32, P, P]
        L.orc_attention_csr.restype = None
        L.orc_attention_lse_delta.argtypes = [P, P, P, P, i32, i32, i32, i32, P, f64, P, P]
        L.orc_attention_lse_delta.restype = None
        L.orc_attention_backward_dq.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, P, f64, P, i32, P]
        L.orc_attention_backward_dq.restype = None
        L.orc_attention_backward_dkdv.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, P, f64, P, i32, P, P]
        L.orc_attention_backward_dkdv.restype = None
        L.orc_perm_static_padded.argtypes = [i32, i32, i32, i32, i32, i32, P]
        L.orc_perm_static_padded.restype = i32
        L.orc_gather_padded.argtypes = [P, P, i32, i32, i64, i64, i32, i32, P]
        L.orc_gather_padded.restype = None
        L.orc_scatter_padded.argtypes = [P, P, i32, i32, i64, i64, i32, i32, P]
        L.orc_scatter_padded.restype = None
        L.orc_pool_padded.argtypes = [P, P, i32, i32, i32, i32, i32, P]
        L.orc_pool_padded.restype = None
        L.orc_attention_padded.argtypes = [P, P, P, i32, i32, i32, P, P, P, f64, P, i32, P, P]
        L.orc_attention_padded.restype = None
        L.orc_attention_lse_delta_padded.argtypes = [P, P, P, P, i32, i32, i32, i32, P, P, f64, P, P]
        L.orc_attention_lse_delta_padded.restype = None
        L.orc_attention_backward_dq_padded.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, P, P, f64, P, i32, P]
        L.orc_attention_backward_dq_padded.restype = None
        L.orc_attention_backward_dkdv_padded.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, P, P, f64, P, i32, P,
                                                          P]
        L.orc_attention_backward_dkdv_padded.restype = None
        L.orc_attention_lse_delta_csr.argtypes = [P, P, P, P, i32, i32, i32, P, P, f64, P, P]
        L.orc_attention_lse_delta_csr.restype = None
        L.orc_attention_backward_dq_csr.argtypes = [P, P, P, P, P, P, i32, i32, i32, P, P, f64, P, i32, P]
        L.orc_attention_backward_dq_csr.restype = None
        L.orc_attention_backward_dkdv_csr.argtypes = [P, P, P, P, P, P, i32, i32, i32, P, P, f64, P, i32, P, P]
        L.orc_attention_backward_dkdv_csr.restype = None
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def perm_static(grid, tile=(4, 4, 4)) -> np.ndarray:
    """Tiled video slot -> raster video index for static tiles, ``int32 [T*H*W]``."""
    T, Hg, W = grid
    out = np.empty(T * Hg * W, np.int32)
    if lib().orc_perm_static(T, Hg, W, *tile, _ptr(out)) != 0:
        raise ValueError("grid not divisible by the tile, or tile is not 64 tokens")
    return out


def shape_extent(shape_id: int):
    return tuple(lib().orc_shape_extent(shape_id, a) for a in range(3))


def shape_stats(q_raster: np.ndarray, n_prefix: int, grid) -> np.ndarray:
    """Mean |delta Q| along (t, h, w) per 8x8x8 region, ``float64 [B, R, 3]``."""
    q = _c(q_raster, np.uint16)
    B, Ntot, H, D = q.shape
    T, Hg, W = grid
    assert Ntot == n_prefix + T * Hg * W
    R = (T // 8) * (Hg // 8) * (W // 8)
    out = np.empty((B, R, 3), np.float64)
    lib().orc_shape_stats(_ptr(q), B, n_prefix, T, Hg, W, H, D, _ptr(out))
    return out


def shape_choose(stats: np.ndarray, grid, tau: float, rel_eps: float = 1e-4):
    """Shape id per region (``uint8 [B, R]``) and near-threshold flags."""
    st = _c(stats, np.float64)
    B, R, _ = st.shape
    T, Hg, W = grid
    shape = np.empty((B, R), np.uint8)
    near = np.empty((B, R), np.uint8)
    lib().orc_shape_choose(_ptr(st), B, T, Hg, W, float(tau), float(rel_eps), _ptr(shape), _ptr(near))
    return shape, near


def perm_dynamic(shape: np.ndarray, grid) -> np.ndarray:
    """Tiled video slot -> raster video index per batch, ``int32 [B, T*H*W]``."""
    sh = _c(shape, np.uint8)
    B = sh.shape[0]
    T, Hg, W = grid
    out = np.empty((B, T * Hg * W), np.int32)
    if lib().orc_perm_dynamic(_ptr(sh), B, T, Hg, W, _ptr(out)) != 0:
        raise ValueError("invalid shape map")
    return out


def _perm_b(perm, B, Nv):
    p = _c(perm, np.int32)
    if p.ndim == 1:
        p = np.ascontiguousarray(np.broadcast_to(p, (B, Nv)))
    assert p.shape == (B, Nv)
    return p


def gather(x_raster: np.ndarray, perm: np.ndarray, n_prefix: int) -> np.ndarray:
    """Raster ``[B, Ntot, H, D]`` -> tiled ``[B, H, Ntot, D]`` (exact copies)."""
    x = _c(x_raster, np.uint16)
    B, Ntot, H, D = x.shape
    Nv = Ntot - n_prefix
    p = _perm_b(perm, B, Nv)
    out = np.empty((B, H, Ntot, D), np.uint16)
    lib().orc_gather(_ptr(x), _ptr(p), B, n_prefix, Nv, H, D, _ptr(out))
    return out


def scatter(x_tiled: np.ndarray, perm: np.ndarray, n_prefix: int) -> np.ndarray:
    """Tiled ``[B, H, Ntot, D]`` -> raster ``[B, Ntot, H, D]`` (exact copies)."""
    x = _c(x_tiled, np.uint16)
    B, H, Ntot, D = x.shape
    Nv = Ntot - n_prefix
    p = _perm_b(perm, B, Nv)
    out = np.empty((B, Ntot, H, D), np.uint16)
    lib().orc_scatter(_ptr(x), _ptr(p), B, n_prefix, Nv, H, D, _ptr(out))
    return out


def pool(x_tiled: np.ndarray, n_prefix: int) -> np.ndarray:
    """Per video tile mean of the 64 tokens, ``float32 [B, H, nvt, D]``."""
    x = _c(x_tiled, np.uint16)
    B, H, Ntot, D = x.shape
    nvt = (Ntot - n_prefix) // TILE
    out = np.empty((B, H, nvt, D), np.float32)
    lib().orc_pool(_ptr(x), B, H, n_prefix, nvt, D, _ptr(out))
    return out


def topk(qp: np.ndarray, kp: np.ndarray, k: int, rows=None):
    """Kept video key tiles per query tile.

    Returns ``(idx int32 [B,H,nrows,k] ascending, s_k, s_k1, mag)``; the last
    three are ``float64 [B,H,nrows]`` (k-th score, (k+1)-th score or NaN,
    larger sum of |products| of those two entries)."""
    q = _c(qp, np.float32)
    kk = _c(kp, np.float32)
    B, H, n, D = q.shape
    if not 1 <= k <= n:
        raise ValueError("k out of range")
    r = None if rows is None else _c(rows, np.int32)
    nrows = n if r is None else r.shape[0]
    idx = np.empty((B, H, nrows, k), np.int32)
    s_k = np.empty((B, H, nrows), np.float64)
    s_k1 = np.empty((B, H, nrows), np.float64)
    mag = np.empty((B, H, nrows), np.float64)
    lib().orc_topk(_ptr(q), _ptr(kk), B, H, n, D, k, _ptr(r), nrows, _ptr(idx), _ptr(s_k),
                   _ptr(s_k1), _ptr(mag))
    return idx, s_k, s_k1, mag


def attention(q_bh, k_bh, v_bh, n_prefix: int, idx_bh, scale: float, qtiles):
    """Exact double-precision attention for one (b,h) slice of tiled tensors.

    ``q_bh, k_bh, v_bh``: ``uint16 [Ntot, D]``; ``idx_bh``: ``int32 [nvt, k]``
    (may be empty when there are no video tiles); ``qtiles``: tiled query tile
    numbers.  Returns ``(out float64 [nq, 64, D], lse float64 [nq, 64])``."""
    q = _c(q_bh, np.uint16)
    kx = _c(k_bh, np.uint16)
    v = _c(v_bh, np.uint16)
    Ntot, D = q.shape
    nvt = (Ntot - n_prefix) // TILE
    ix = _c(idx_bh, np.int32)
    k = ix.shape[1] if ix.ndim == 2 else 0
    qt = _c(qtiles, np.int32)
    nq = qt.shape[0]
    out = np.empty((nq, TILE, D), np.float64)
    lse = np.empty((nq, TILE), np.float64)
    lib().orc_attention(_ptr(q), _ptr(kx), _ptr(v), n_prefix, nvt, D, k, _ptr(ix), float(scale),
                        _ptr(qt), nq, _ptr(out), _ptr(lse))
    return out, lse


def attention_csr(q_bh, k_bh, v_bh, n_prefix: int, row_ptr_bh, col, scale: float, qtiles):
    """As ``attention``, with video query tile i keeping the video tiles
    ``col[row_ptr_bh[i]:row_ptr_bh[i+1]]`` (variable keep, CSR lists).
    ``row_ptr_bh``: int64 ``[nvt + 1]`` into ``col`` (int32)."""
    q = _c(q_bh, np.uint16)
    kx = _c(k_bh, np.uint16)
    v = _c(v_bh, np.uint16)
    Ntot, D = q.shape
    nvt = (Ntot - n_prefix) // TILE
    rp = _c(row_ptr_bh, np.int64)
    cl = _c(col, np.int32) if len(col) else np.zeros(1, np.int32)
    qt = _c(qtiles, np.int32)
    nq = qt.shape[0]
    out = np.empty((nq, TILE, D), np.float64)
    lse = np.empty((nq, TILE), np.float64)
    lib().orc_attention_csr(_ptr(q), _ptr(kx), _ptr(v), n_prefix, nvt, D, _ptr(rp), _ptr(cl), float(scale),
                            _ptr(qt), nq, _ptr(out), _ptr(lse))
    return out, lse


def plan_csr(qp, kp, keep_per_head, keep_rows=None):
    """Variable-keep selection from pooled ``qp, kp`` (float32 ``[B,H,nvt,D]``):
    row (b,h,i) keeps ``min(max(keep_rows[b,h,i], 1), keep_per_head[h])`` tiles
    (``keep_per_head[h]`` without ``keep_rows``), chosen by the same rule as
    ``topk``.  Returns ``(row_ptr int64 [B*H*nvt + 1], col int32)`` with rows in
    (b, h, i) order."""
    B, H, n, _ = qp.shape
    lens = np.empty((B, H, n), np.int64)
    for h in range(H):
        lens[:, h, :] = keep_per_head[h]
    if keep_rows is not None:
        lens = np.minimum(np.maximum(np.asarray(keep_rows, np.int64), 1), lens)
    row_ptr = np.zeros(B * H * n + 1, np.int64)
    row_ptr[1:] = np.cumsum(lens.reshape(-1))
    col = np.empty(int(row_ptr[-1]), np.int32)
    for b in range(B):
        for h in range(H):
            for k in np.unique(lens[b, h]):
                rows = np.nonzero(lens[b, h] == k)[0].astype(np.int32)
                idx = topk(qp[b:b + 1, h:h + 1], kp[b:b + 1, h:h + 1], int(k), rows)[0]
                for a, i in enumerate(rows):
                    r = (b * H + h) * n + i
                    col[row_ptr[r]:row_ptr[r + 1]] = idx[0, 0, a]
    return row_ptr, col


def plan_structured(tile_grid, head_mask, radius_t: int, radius_hw: int, batch: int):
    """Structured kept lists (Sparse VideoGen page, section on its key idea:
    spatial heads look within nearby frames, temporal heads follow a position
    across frames).  ``tile_grid`` = (Tt, Th, Tw) tiles; video tile (t, h, w)
    is number (t*Th + h)*Tw + w.  For head h, query tile (ti, hi, wi) keeps
    every tile with |t - ti| <= radius_t (head_mask 0, spatial) or with
    |h - hi| <= radius_hw and |w - wi| <= radius_hw (1, temporal), ascending.
    Returns ``(row_ptr int64 [batch*H*nvt + 1], col int32)``, rows in (b, h, i)
    order."""
    Tt, Th, Tw = tile_grid
    nvt = Tt * Th * Tw
    lists = {}
    for kind in (0, 1):
        rows = []
        for i in range(nvt):
            ti, hi, wi = i // (Th * Tw), (i // Tw) % Th, i % Tw
            keep = []
            for j in range(nvt):
                tj, hj, wj = j // (Th * Tw), (j // Tw) % Th, j % Tw
                if kind == 0:
                    ok = abs(tj - ti) <= radius_t
                else:
                    ok = abs(hj - hi) <= radius_hw and abs(wj - wi) <= radius_hw
                if ok:
                    keep.append(j)
            rows.append(np.array(keep, np.int32))
        lists[kind] = rows
    all_rows = [lists[int(m)][i] for _ in range(batch) for m in head_mask for i in range(nvt)]
    row_ptr = np.zeros(len(all_rows) + 1, np.int64)
    row_ptr[1:] = np.cumsum([len(r) for r in all_rows])
    col = np.concatenate(all_rows).astype(np.int32) if all_rows else np.zeros(0, np.int32)
    return row_ptr, col


def plan(q_tiled, k_tiled, n_prefix: int, k: int):
    """Pool Q and K, score and select: ``(qp, kp, idx, s_k, s_k1, mag)``."""
    qp = pool(q_tiled, n_prefix)
    kp = pool(k_tiled, n_prefix)
    idx, s_k, s_k1, mag = topk(qp, kp, k)
    return qp, kp, idx, s_k, s_k1, mag


def forward_full(q_tiled, k_tiled, v_tiled, n_prefix: int, idx, scale: float):
    """Attention output for every query tile of every (b,h): ``float64 [B,H,Ntot,D]``."""
    B, H, Ntot, D = q_tiled.shape
    nqt = Ntot // TILE
    out = np.empty((B, H, Ntot, D), np.float64)
    lse = np.empty((B, H, Ntot), np.float64)
    tiles = np.arange(nqt, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            ix = idx[b, h] if idx is not None else np.zeros((0, 0), np.int32)
            o, l = attention(q_tiled[b, h], k_tiled[b, h], v_tiled[b, h], n_prefix, ix, scale, tiles)
            out[b, h] = o.reshape(Ntot, D)
            lse[b, h] = l.reshape(Ntot)
    return out, lse


def reference(q_raster, k_raster, v_raster, *, grid, n_prefix: int, k: int, scale: float,
              tile=(4, 4, 4), dynamic: bool = False, tau: float = 0.10):
    """The whole path on raster inputs; returns a dict with every intermediate.

    Output ``o`` is raster ``float64 [B, Ntot, H, D]``."""
    B = q_raster.shape[0]
    res = {}
    if dynamic:
        st = shape_stats(q_raster, n_prefix, grid)
        shape, near = shape_choose(st, grid, tau)
        perm = perm_dynamic(shape, grid)
        res.update(stats=st, shape=shape, shape_near=near)
    else:
        perm = np.ascontiguousarray(np.broadcast_to(perm_static(grid, tile), (B, grid[0] * grid[1] * grid[2])))
    qt = gather(q_raster, perm, n_prefix)
    kt = gather(k_raster, perm, n_prefix)
    vt = gather(v_raster, perm, n_prefix)
    qp, kp, idx, s_k, s_k1, mag = plan(qt, kt, n_prefix, k)
    o_t, lse = forward_full(qt, kt, vt, n_prefix, idx, scale)
    # scatter the float64 output back to raster order
    Bq, H, Ntot, D = o_t.shape
    o = np.empty((Bq, Ntot, H, D), np.float64)
    for b in range(Bq):
        src = np.empty(Ntot, np.int64)
        src[:n_prefix] = np.arange(n_prefix)
        src[n_prefix:] = n_prefix + perm[b]
        o[b, src] = o_t[b].transpose(1, 0, 2)
    res.update(perm=perm, q_tiled=qt, k_tiled=kt, v_tiled=vt, qp=qp, kp=kp, idx=idx, s_k=s_k,
               s_k1=s_k1, mag=mag, o_tiled=o_t, lse=lse, o=o)
    return res


def _bh_args(q_bh, k_bh, v_bh, do_bh, n_prefix, idx_bh):
    q, kx, v, do = (_c(x, np.uint16) for x in (q_bh, k_bh, v_bh, do_bh))
    Ntot, D = q.shape
    nvt = (Ntot - n_prefix) // TILE
    ix = _c(idx_bh, np.int32) if idx_bh is not None else np.zeros((0, 0), np.int32)
    k = ix.shape[1] if ix.ndim == 2 else 0
    return q, kx, v, do, Ntot, D, nvt, ix, k


def lse_delta(q_bh, k_bh, v_bh, do_bh, n_prefix: int, idx_bh, scale: float):
    """lse and Delta = dO . O of every query token of one (b,h) (tiled order):
    ``(lse, delta)``, float64 ``[Ntot]`` each."""
    q, kx, v, do, Ntot, D, nvt, ix, k = _bh_args(q_bh, k_bh, v_bh, do_bh, n_prefix, idx_bh)
    lse = np.empty(Ntot, np.float64)
    delta = np.empty(Ntot, np.float64)
    lib().orc_attention_lse_delta(_ptr(q), _ptr(kx), _ptr(v), _ptr(do), n_prefix, nvt, D, k, _ptr(ix),
                                  float(scale), _ptr(lse), _ptr(delta))
    return lse, delta


def backward_dq(q_bh, k_bh, v_bh, do_bh, lse, delta, n_prefix: int, idx_bh, scale: float, qtiles):
    """dQ of the query tiles ``qtiles`` of one (b,h): float64 ``[nq, 64, D]``."""
    q, kx, v, do, Ntot, D, nvt, ix, k = _bh_args(q_bh, k_bh, v_bh, do_bh, n_prefix, idx_bh)
    qt = _c(qtiles, np.int32)
    out = np.empty((qt.shape[0], TILE, D), np.float64)
    lib().orc_attention_backward_dq(_ptr(q), _ptr(kx), _ptr(v), _ptr(do), _ptr(_c(lse, np.float64)),
                                    _ptr(_c(delta, np.float64)), n_prefix, nvt, D, k, _ptr(ix), float(scale),
                                    _ptr(qt), qt.shape[0], _ptr(out))
    return out


def backward_dkdv(q_bh, k_bh, v_bh, do_bh, lse, delta, n_prefix: int, idx_bh, scale: float, ktiles):
    """dK and dV of the key tiles ``ktiles`` of one (b,h): two float64 ``[nk, 64, D]``."""
    q, kx, v, do, Ntot, D, nvt, ix, k = _bh_args(q_bh, k_bh, v_bh, do_bh, n_prefix, idx_bh)
    kt = _c(ktiles, np.int32)
    dk = np.empty((kt.shape[0], TILE, D), np.float64)
    dv = np.empty((kt.shape[0], TILE, D), np.float64)
    lib().orc_attention_backward_dkdv(_ptr(q), _ptr(kx), _ptr(v), _ptr(do), _ptr(_c(lse, np.float64)),
                                      _ptr(_c(delta, np.float64)), n_prefix, nvt, D, k, _ptr(ix), float(scale),
                                      _ptr(kt), kt.shape[0], _ptr(dk), _ptr(dv))
    return dk, dv


def backward_full(q_tiled, k_tiled, v_tiled, do_tiled, n_prefix: int, idx, scale: float):
    """Gradients of every (b,h), tiled order: ``(dq, dk, dv)`` float64 ``[B,H,Ntot,D]``."""
    B, H, Ntot, D = q_tiled.shape
    tiles = np.arange(Ntot // TILE, dtype=np.int32)
    dq = np.empty((B, H, Ntot, D), np.float64)
    dk = np.empty_like(dq)
    dv = np.empty_like(dq)
    for b in range(B):
        for h in range(H):
            ix = idx[b, h] if idx is not None else None
            args = (q_tiled[b, h], k_tiled[b, h], v_tiled[b, h], do_tiled[b, h])
            lse, delta = lse_delta(*args, n_prefix, ix, scale)
            dq[b, h] = backward_dq(*args, lse, delta, n_prefix, ix, scale, tiles).reshape(Ntot, D)
            gk, gv = backward_dkdv(*args, lse, delta, n_prefix, ix, scale, tiles)
            dk[b, h] = gk.reshape(Ntot, D)
            dv[b, h] = gv.reshape(Ntot, D)
    return dq, dk, dv


# ---- ragged grids: static tiles over the grid rounded up to whole tiles ------

def padded_slots(grid, tile=(4, 4, 4)) -> int:
    """Video slots of the tiled order: every axis rounded up to whole tiles."""
    return int(np.prod([-(-g // t) * t for g, t in zip(grid, tile)]))


def perm_static_padded(grid, tile=(4, 4, 4)) -> np.ndarray:
    """Tiled video slot -> raster video index, -1 for a padding slot,
    ``int32 [padded_slots]``."""
    T, Hg, W = grid
    out = np.empty(padded_slots(grid, tile), np.int32)
    if lib().orc_perm_static_padded(T, Hg, W, *tile, _ptr(out)) != 0:
        raise ValueError("tile is not 64 tokens")
    return out


def gather_padded(x_raster: np.ndarray, perm: np.ndarray, n_prefix: int) -> np.ndarray:
    """Raster ``[B, n_prefix + Nras, H, D]`` -> tiled ``[B, H, n_prefix + Nslots, D]``
    (``Nslots`` = perm's length; zeros in padding slots)."""
    x = _c(x_raster, np.uint16)
    B, Nr, H, D = x.shape
    Ns = perm.shape[-1]
    p = _perm_b(perm, B, Ns)
    out = np.empty((B, H, n_prefix + Ns, D), np.uint16)
    lib().orc_gather_padded(_ptr(x), _ptr(p), B, n_prefix, Nr - n_prefix, Ns, H, D, _ptr(out))
    return out


def scatter_padded(x_tiled: np.ndarray, perm: np.ndarray, n_prefix: int, n_raster_video: int) -> np.ndarray:
    """Tiled ``[B, H, n_prefix + Nslots, D]`` -> raster ``[B, n_prefix + n_raster_video, H, D]``
    (padding slots dropped)."""
    x = _c(x_tiled, np.uint16)
    B, H, Nt, D = x.shape
    Ns = Nt - n_prefix
    p = _perm_b(perm, B, Ns)
    out = np.zeros((B, n_prefix + n_raster_video, H, D), np.uint16)
    lib().orc_scatter_padded(_ptr(x), _ptr(p), B, n_prefix, n_raster_video, Ns, H, D, _ptr(out))
    return out


def pool_padded(x_tiled: np.ndarray, perm: np.ndarray, n_prefix: int) -> np.ndarray:
    """Per video tile mean over its real tokens, ``float32 [B, H, nvt, D]``."""
    x = _c(x_tiled, np.uint16)
    B, H, Ntot, D = x.shape
    nvt = (Ntot - n_prefix) // TILE
    p = _perm_b(perm, B, nvt * TILE)
    out = np.empty((B, H, nvt, D), np.float32)
    lib().orc_pool_padded(_ptr(x), _ptr(p), B, H, n_prefix, nvt, D, _ptr(out))
    return out


def key_real(perm_b: np.ndarray, n_prefix: int) -> np.ndarray:
    """uint8 [n_prefix + Nslots]: 1 for a real token of the tiled order
    (prefix and perm >= 0), 0 for a padding slot."""
    return np.concatenate([np.ones(n_prefix, np.uint8), (np.asarray(perm_b) >= 0).astype(np.uint8)])


def attention_padded_csr(q_bh, k_bh, v_bh, n_prefix: int, row_ptr_bh, col, real, scale: float, qtiles):
    """As ``attention_csr``, with only the real keys (``real`` from ``key_real``)."""
    q = _c(q_bh, np.uint16)
    kx = _c(k_bh, np.uint16)
    v = _c(v_bh, np.uint16)
    Ntot, D = q.shape
    nvt = (Ntot - n_prefix) // TILE
    rp = _c(row_ptr_bh, np.int64)
    cl = _c(col, np.int32) if len(col) else np.zeros(1, np.int32)
    kr = _c(real, np.uint8)
    assert kr.shape == (Ntot,)
    qt = _c(qtiles, np.int32)
    nq = qt.shape[0]
    out = np.empty((nq, TILE, D), np.float64)
    lse = np.empty((nq, TILE), np.float64)
    lib().orc_attention_padded(_ptr(q), _ptr(kx), _ptr(v), n_prefix, nvt, D, _ptr(rp), _ptr(cl), _ptr(kr),
                               float(scale), _ptr(qt), nq, _ptr(out), _ptr(lse))
    return out, lse


def attention_padded(q_bh, k_bh, v_bh, n_prefix: int, idx_bh, real, scale: float, qtiles):
    """As ``attention`` (fixed keep, ``idx_bh [nvt, k]``), with only the real keys."""
    ix = _c(idx_bh, np.int32)
    nvt, k = ix.shape
    row_ptr = np.arange(nvt + 1, dtype=np.int64) * k
    return attention_padded_csr(q_bh, k_bh, v_bh, n_prefix, row_ptr, ix.reshape(-1), real, scale, qtiles)


def lse_delta_padded(q_bh, k_bh, v_bh, do_bh, n_prefix: int, idx_bh, real, scale: float):
    """As ``lse_delta`` on a ragged grid (real keys only)."""
    q, kx, v, do, Ntot, D, nvt, ix, k = _bh_args(q_bh, k_bh, v_bh, do_bh, n_prefix, idx_bh)
    kr = _c(real, np.uint8)
    assert kr.shape == (Ntot,)
    lse = np.empty(Ntot, np.float64)
    delta = np.empty(Ntot, np.float64)
    lib().orc_attention_lse_delta_padded(_ptr(q), _ptr(kx), _ptr(v), _ptr(do), n_prefix, nvt, D, k, _ptr(ix),
                                         _ptr(kr), float(scale), _ptr(lse), _ptr(delta))
    return lse, delta


def backward_dq_padded(q_bh, k_bh, v_bh, do_bh, lse, delta, n_prefix: int, idx_bh, real, scale: float, qtiles):
    """As ``backward_dq`` on a ragged grid (real keys only)."""
    q, kx, v, do, Ntot, D, nvt, ix, k = _bh_args(q_bh, k_bh, v_bh, do_bh, n_prefix, idx_bh)
    kr = _c(real, np.uint8)
    qt = _c(qtiles, np.int32)
    out = np.empty((qt.shape[0], TILE, D), np.float64)
    lib().orc_attention_backward_dq_padded(_ptr(q), _ptr(kx), _ptr(v), _ptr(do), _ptr(_c(lse, np.float64)),
                                           _ptr(_c(delta, np.float64)), n_prefix, nvt, D, k, _ptr(ix), _ptr(kr),
                                           float(scale), _ptr(qt), qt.shape[0], _ptr(out))
    return out


def backward_dkdv_padded(q_bh, k_bh, v_bh, do_bh, lse, delta, n_prefix: int, idx_bh, real, scale: float, ktiles):
    """As ``backward_dkdv`` on a ragged grid: real keys, real queries; padding
    key rows are zero."""
    q, kx, v, do, Ntot, D, nvt, ix, k = _bh_args(q_bh, k_bh, v_bh, do_bh, n_prefix, idx_bh)
    kr = _c(real, np.uint8)
    kt = _c(ktiles, np.int32)
    dk = np.empty((kt.shape[0], TILE, D), np.float64)
    dv = np.empty((kt.shape[0], TILE, D), np.float64)
    lib().orc_attention_backward_dkdv_padded(_ptr(q), _ptr(kx), _ptr(v), _ptr(do), _ptr(_c(lse, np.float64)),
                                             _ptr(_c(delta, np.float64)), n_prefix, nvt, D, k, _ptr(ix), _ptr(kr),
                                             float(scale), _ptr(kt), kt.shape[0], _ptr(dk), _ptr(dv))
    return dk, dv


def backward_full_padded(q_tiled, k_tiled, v_tiled, do_tiled, n_prefix: int, idx, real, scale: float):
    """Gradients of every (b,h) on a ragged grid, tiled order (padding rows
    of dK, dV zero): ``(dq, dk, dv)`` float64 ``[B,H,Ntot,D]``.  ``real``:
    ``key_real`` of each batch element, ``[B, Ntot]``."""
    B, H, Ntot, D = q_tiled.shape
    tiles = np.arange(Ntot // TILE, dtype=np.int32)
    dq = np.empty((B, H, Ntot, D), np.float64)
    dk = np.empty_like(dq)
    dv = np.empty_like(dq)
    for b in range(B):
        for h in range(H):
            ix = idx[b, h] if idx is not None else None
            args = (q_tiled[b, h], k_tiled[b, h], v_tiled[b, h], do_tiled[b, h])
            lse, delta = lse_delta_padded(*args, n_prefix, ix, real[b], scale)
            dq[b, h] = backward_dq_padded(*args, lse, delta, n_prefix, ix, real[b], scale, tiles).reshape(Ntot, D)
            g_k, g_v = backward_dkdv_padded(*args, lse, delta, n_prefix, ix, real[b], scale, tiles)
            dk[b, h] = g_k.reshape(Ntot, D)
            dv[b, h] = g_v.reshape(Ntot, D)
    return dq, dk, dv


# ---- gradients over CSR kept lists -------------------------------------------------

def _csr_args(q_bh, k_bh, v_bh, do_bh, n_prefix, row_ptr_bh, col):
    q, kx, v, do = (_c(x, np.uint16) for x in (q_bh, k_bh, v_bh, do_bh))
    Ntot, D = q.shape
    nvt = (Ntot - n_prefix) // TILE
    rp = _c(row_ptr_bh, np.int64) if nvt else np.zeros(1, np.int64)
    cl = _c(col, np.int32) if len(col) else np.zeros(1, np.int32)
    return q, kx, v, do, Ntot, D, nvt, rp, cl


def lse_delta_csr(q_bh, k_bh, v_bh, do_bh, n_prefix: int, row_ptr_bh, col, scale: float):
    """As ``lse_delta`` over CSR lists of one (b,h) (``row_ptr_bh`` ``[nvt + 1]``
    into ``col``)."""
    q, kx, v, do, Ntot, D, nvt, rp, cl = _csr_args(q_bh, k_bh, v_bh, do_bh, n_prefix, row_ptr_bh, col)
    lse = np.empty(Ntot, np.float64)
    delta = np.empty(Ntot, np.float64)
    lib().orc_attention_lse_delta_csr(_ptr(q), _ptr(kx), _ptr(v), _ptr(do), n_prefix, nvt, D, _ptr(rp), _ptr(cl),
                                      float(scale), _ptr(lse), _ptr(delta))
    return lse, delta


def backward_dq_csr(q_bh, k_bh, v_bh, do_bh, lse, delta, n_prefix: int, row_ptr_bh, col, scale: float, qtiles):
    """As ``backward_dq`` over CSR lists of one (b,h)."""
    q, kx, v, do, Ntot, D, nvt, rp, cl = _csr_args(q_bh, k_bh, v_bh, do_bh, n_prefix, row_ptr_bh, col)
    qt = _c(qtiles, np.int32)
    out = np.empty((qt.shape[0], TILE, D), np.float64)
    lib().orc_attention_backward_dq_csr(_ptr(q), _ptr(kx), _ptr(v), _ptr(do), _ptr(_c(lse, np.float64)),
                                        _ptr(_c(delta, np.float64)), n_prefix, nvt, D, _ptr(rp), _ptr(cl),
                                        float(scale), _ptr(qt), qt.shape[0], _ptr(out))
    return out


def backward_dkdv_csr(q_bh, k_bh, v_bh, do_bh, lse, delta, n_prefix: int, row_ptr_bh, col, scale: float, ktiles):
    """As ``backward_dkdv`` over CSR lists of one (b,h)."""
    q, kx, v, do, Ntot, D, nvt, rp, cl = _csr_args(q_bh, k_bh, v_bh, do_bh, n_prefix, row_ptr_bh, col)
    kt = _c(ktiles, np.int32)
    dk = np.empty((kt.shape[0], TILE, D), np.float64)
    dv = np.empty((kt.shape[0], TILE, D), np.float64)
    lib().orc_attention_backward_dkdv_csr(_ptr(q), _ptr(kx), _ptr(v), _ptr(do), _ptr(_c(lse, np.float64)),
                                          _ptr(_c(delta, np.float64)), n_prefix, nvt, D, _ptr(rp), _ptr(cl),
                                          float(scale), _ptr(kt), kt.shape[0], _ptr(dk), _ptr(dv))
    return dk, dv


def backward_full_csr(q_tiled, k_tiled, v_tiled, do_tiled, n_prefix: int, row_ptr, col, scale: float):
    """Gradients of every (b,h) over CSR lists (``row_ptr`` int64 ``[B*H*nvt + 1]``
    and ``col`` as ``plan_csr`` returns them), tiled order: ``(dq, dk, dv)``
    float64 ``[B,H,Ntot,D]``."""
    B, H, Ntot, D = q_tiled.shape
    nvt = (Ntot - n_prefix) // TILE
    tiles = np.arange(Ntot // TILE, dtype=np.int32)
    dq = np.empty((B, H, Ntot, D), np.float64)
    dk = np.empty_like(dq)
    dv = np.empty_like(dq)
    for b in range(B):
        for h in range(H):
            r0 = (b * H + h) * nvt
            if nvt:
                rp = np.asarray(row_ptr[r0:r0 + nvt + 1], np.int64) - row_ptr[r0]
                cl = col[row_ptr[r0]:row_ptr[r0 + nvt]]
            else:
                rp, cl = np.zeros(1, np.int64), np.zeros(0, np.int32)
            args = (q_tiled[b, h], k_tiled[b, h], v_tiled[b, h], do_tiled[b, h])
            lse, delta = lse_delta_csr(*args, n_prefix, rp, cl, scale)
            dq[b, h] = backward_dq_csr(*args, lse, delta, n_prefix, rp, cl, scale, tiles).reshape(Ntot, D)
            g_k, g_v = backward_dkdv_csr(*args, lse, delta, n_prefix, rp, cl, scale, tiles)
            dk[b, h] = g_k.reshape(Ntot, D)
            dv[b, h] = g_v.reshape(Ntot, D)
    return dq, dk, dv
