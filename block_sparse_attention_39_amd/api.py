"""Python binding of the C ABI: argument marshalling only.

Tensors are torch tensors on the GPU (torch provides device memory and the
stream); every function passes raw device pointers to libbsa.so and raises
``BsaError`` on a non-zero status.  All compute runs in the library's HIP
kernels.
"""
from __future__ import annotations

import ctypes
import math

import torch

from ._lib import (PERM_BUILD, PERM_GATHER, PERM_GATHER_KF, PERM_GATHER_KF_POOL, PERM_GATHER_POOL, PERM_GATHER_VF,
                   PERM_POOL, PERM_SCATTER, PERM_TILED_TO_KF, PERM_TILED_TO_VF, TILE_DYNAMIC, TILE_STATIC, TILE_STATIC_PADDED,
                   BsaError, Desc, lib)


def make_desc(batch: int, heads: int, head_dim: int, grid, keep_tiles: int, *, scale: float | None = None,
              n_prefix: int = 0, dynamic: bool = False, tile=(4, 4, 4), tau: float = 0.10,
              padded: bool = False) -> Desc:
    """``padded``: a ragged grid, rounded up to whole static tiles."""
    T, H, W = grid
    mode = TILE_DYNAMIC if dynamic else (TILE_STATIC_PADDED if padded else TILE_STATIC)
    return Desc(batch, heads, head_dim, T, H, W, n_prefix, mode, tile[0], tile[1], tile[2], keep_tiles,
                1.0 / math.sqrt(head_dim) if scale is None else scale, tau)


def keep_tiles_for(sparsity: float, n_video_tiles: int) -> int:
    """Kept key tiles per query tile for a sparsity s in [0, 1]: the (1 - s)
    share of the n video tiles, rounded to nearest, at least one and at most
    all of them ("Prism / Kandinsky 6 speed ablation" page, section on Prism's
    block-sparse attention: s = 0.75 keeps a quarter of the key blocks, 480 of
    1,920 per query block).  The C interface takes the integer count."""
    s = float(sparsity)
    if not 0.0 <= s <= 1.0:
        raise ValueError(f"sparsity {sparsity} outside [0, 1]")
    n = int(n_video_tiles)
    if n <= 0:
        return 0
    return min(max(int(math.floor((1.0 - s) * n + 0.5)), 1), n)


# Below this many tokens a call stays dense ("倍速で回した一晩" page, section
# "같은 방식을 직접 해보려면": the sparse attention node leaves calls with
# fewer tokens than its minimum, 12,288 there, dense).
DENSE_BELOW_TOKENS = 12288


def keep_for_call(sparsity: float, n_video_tiles: int, n_tokens: int,
                  dense_below: int = DENSE_BELOW_TOKENS) -> int:
    """keep_tiles_for, except that a call with fewer than ``dense_below``
    tokens keeps every tile (k = n runs the same kernels densely)."""
    if n_tokens < dense_below:
        return max(int(n_video_tiles), 0)
    return keep_tiles_for(sparsity, n_video_tiles)


def video_slots(desc: Desc) -> int:
    """Video tokens of the tiled layouts: the grid, or for a ragged grid the
    grid rounded up to whole tiles."""
    T, H, W = desc.grid_t, desc.grid_h, desc.grid_w
    if desc.tile_mode != TILE_STATIC_PADDED:
        return T * H * W
    tt, th, tw = desc.tile_t, desc.tile_h, desc.tile_w
    return -(-T // tt) * tt * (-(-H // th) * th) * (-(-W // tw) * tw)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must live in GPU memory (libbsa has no CPU path)")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status: int, where: str):
    if status != 0:
        raise BsaError(status, where)


def workspace_size(desc: Desc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().bsa_workspace_size(ctypes.byref(desc), ctypes.byref(n)), "bsa_workspace_size")
    return n.value


def permute_build(desc: Desc, perm, shape_map=None, q_raster=None, workspace=None, stream=None):
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().bsa_permute(ctypes.byref(desc), PERM_BUILD, _ptr(q_raster), _ptr(perm), _ptr(shape_map), None, None,
                             _ptr(workspace), ws, _stream(stream)), "bsa_permute(BUILD)")


def gather(desc: Desc, src, dst, perm, stream=None):
    _check(lib().bsa_permute(ctypes.byref(desc), PERM_GATHER, None, _ptr(perm), None, _ptr(src), _ptr(dst), None, 0,
                             _stream(stream)), "bsa_permute(GATHER)")


def gather_kf(desc: Desc, src, dst, perm, stream=None):
    """Raster K -> the K-fragment layout (the tiled order, each 64-token tile in
    the attention kernel's operand order; same size as the tiled layout)."""
    _check(lib().bsa_permute(ctypes.byref(desc), PERM_GATHER_KF, None, _ptr(perm), None, _ptr(src), _ptr(dst), None,
                             0, _stream(stream)), "bsa_permute(GATHER_KF)")


def gather_vf(desc: Desc, src, dst, perm, stream=None):
    """Raster V -> the V-fragment layout (same size as the tiled layout)."""
    _check(lib().bsa_permute(ctypes.byref(desc), PERM_GATHER_VF, None, _ptr(perm), None, _ptr(src), _ptr(dst), None,
                             0, _stream(stream)), "bsa_permute(GATHER_VF)")


def _ws(workspace):
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def gather_pool(desc: Desc, src, dst, perm, workspace, stream=None):
    """Raster Q -> tiled, with the tile means of Q written into the workspace."""
    _check(lib().bsa_permute(ctypes.byref(desc), PERM_GATHER_POOL, None, _ptr(perm), None, _ptr(src), _ptr(dst),
                             _ptr(workspace), _ws(workspace), _stream(stream)), "bsa_permute(GATHER_POOL)")


def gather_kf_pool(desc: Desc, src, dst, perm, workspace, stream=None):
    """Raster K -> the K-fragment layout, with the tile means of K written into
    the workspace."""
    _check(lib().bsa_permute(ctypes.byref(desc), PERM_GATHER_KF_POOL, None, _ptr(perm), None, _ptr(src), _ptr(dst),
                             _ptr(workspace), _ws(workspace), _stream(stream)), "bsa_permute(GATHER_KF_POOL)")


def pool(desc: Desc, src, perm, workspace, stream=None):
    """The tile means of raster Q alone (no tiled copy) into the workspace, as
    gather_pool writes them: for forward_raster, which reads raster Q."""
    _check(lib().bsa_permute(ctypes.byref(desc), PERM_POOL, None, _ptr(perm), None, _ptr(src), None,
                             _ptr(workspace), _ws(workspace), _stream(stream)), "bsa_permute(POOL)")


def tiled_to_kf(desc: Desc, src, dst, stream=None):
    """Tiled K -> the K-fragment layout."""
    _check(lib().bsa_permute(ctypes.byref(desc), PERM_TILED_TO_KF, None, None, None, _ptr(src), _ptr(dst), None, 0,
                             _stream(stream)), "bsa_permute(TILED_TO_KF)")


def tiled_to_vf(desc: Desc, src, dst, stream=None):
    """Tiled V -> the V-fragment layout."""
    _check(lib().bsa_permute(ctypes.byref(desc), PERM_TILED_TO_VF, None, None, None, _ptr(src), _ptr(dst), None, 0,
                             _stream(stream)), "bsa_permute(TILED_TO_VF)")


def scatter(desc: Desc, src, dst, perm, stream=None):
    _check(lib().bsa_permute(ctypes.byref(desc), PERM_SCATTER, None, _ptr(perm), None, _ptr(src), _ptr(dst), None, 0,
                             _stream(stream)), "bsa_permute(SCATTER)")


def plan(desc: Desc, q_tiled, k_frag, block_idx, workspace, stream=None):
    ws = workspace.numel() * workspace.element_size()
    _check(lib().bsa_plan(ctypes.byref(desc), _ptr(q_tiled), _ptr(k_frag), _ptr(block_idx), _ptr(workspace), ws,
                          _stream(stream)), "bsa_plan")


def select(desc: Desc, block_idx, workspace, stream=None):
    """Scores and top-k from the tile means already in the workspace (written
    by gather_pool / gather_kf_pool or an earlier plan)."""
    _check(lib().bsa_select(ctypes.byref(desc), _ptr(block_idx), _ptr(workspace), _ws(workspace), _stream(stream)),
           "bsa_select")


def forward_stats_offset(desc: Desc) -> int:
    """Byte offset in the workspace of the forward's int32 statistics: rounds
    whose start wait gave up, rounds started (of the last grouped call)."""
    n = ctypes.c_size_t(0)
    _check(lib().bsa_forward_stats_offset(ctypes.byref(desc), ctypes.byref(n)), "bsa_forward_stats_offset")
    return n.value


def forward_stats(desc: Desc, workspace):
    """(rounds whose start wait gave up, rounds started) of the last grouped
    forward call on this workspace (a device read: synchronises the stream)."""
    off = forward_stats_offset(desc)
    v = workspace.view(torch.uint8)[off:off + 8].view(torch.int32).cpu().tolist()
    return int(v[0]), int(v[1])


def forward(desc: Desc, q_tiled, k_frag, v_frag, block_idx, o_tiled, lse=None, workspace=None, stream=None):
    """``k_frag`` / ``v_frag`` are K and V in the fragment layouts written by
    gather_kf / gather_vf.  With ``workspace`` the video query tiles run as the
    grouped persistent grid."""
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().bsa_forward(ctypes.byref(desc), _ptr(q_tiled), _ptr(k_frag), _ptr(v_frag), _ptr(block_idx),
                             _ptr(o_tiled), _ptr(lse), _ptr(workspace), ws, _stream(stream)), "bsa_forward")


def forward_raster(desc: Desc, q_raster, perm, k_frag, v_frag, block_idx, o_raster, lse=None, workspace=None,
                   stream=None):
    """forward with Q read from and O written to the raster layout through
    ``perm`` (the same values as gather, forward and scatter)."""
    _check(lib().bsa_forward_raster(ctypes.byref(desc), _ptr(q_raster), _ptr(perm), _ptr(k_frag), _ptr(v_frag),
                                    _ptr(block_idx), _ptr(o_raster), _ptr(lse), _ptr(workspace), _ws(workspace),
                                    _stream(stream)), "bsa_forward_raster")


def forward_noalloc(desc: Desc, q_tiled, k_frag, v_frag, block_idx, o_tiled, lse=None, stream=None):
    """bsa_forward's grouped launch without a workspace: for callers that
    cannot allocate device memory (the library keeps its round counters in a
    static per-GPU array; calls that overlap on one GPU race)."""
    _check(lib().bsa_forward_noalloc(ctypes.byref(desc), _ptr(q_tiled), _ptr(k_frag), _ptr(v_frag), _ptr(block_idx),
                                     _ptr(o_tiled), _ptr(lse), _stream(stream)), "bsa_forward_noalloc")


def _keep_heads(desc: Desc, keep_per_head):
    """Host int32 array of the per-head keep counts (or None)."""
    if keep_per_head is None:
        return None, None
    arr = (ctypes.c_int32 * len(keep_per_head))(*[int(x) for x in keep_per_head])
    if len(keep_per_head) != desc.heads:
        raise ValueError("keep_per_head needs one count per head")
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def csr_entries(desc: Desc, keep_per_head=None) -> int:
    """Entries the CSR column array needs: B * nVT * sum of the per-head keeps."""
    _, kp = _keep_heads(desc, keep_per_head)
    n = ctypes.c_int64(0)
    _check(lib().bsa_csr_entries(ctypes.byref(desc), kp, ctypes.byref(n)), "bsa_csr_entries")
    return n.value


def plan_csr(desc: Desc, q_tiled, k_frag, row_ptr, col_idx, workspace, keep_per_head=None, keep_rows=None,
             stream=None):
    """Variable-keep selection: ``row_ptr`` int64 ``[B*H*nVT + 1]`` and ``col_idx``
    int32 (at least csr_entries() entries) on the device; ``keep_per_head`` a
    host sequence of H counts, ``keep_rows`` an optional device int32
    ``[B, H, nVT]`` tensor of per-row counts (clamped to 1..keep_per_head[h])."""
    arr, kp = _keep_heads(desc, keep_per_head)
    ws = workspace.numel() * workspace.element_size()
    _check(lib().bsa_plan_csr(ctypes.byref(desc), _ptr(q_tiled), _ptr(k_frag), kp, _ptr(keep_rows), _ptr(row_ptr),
                              _ptr(col_idx), col_idx.numel(), _ptr(workspace), ws, _stream(stream)), "bsa_plan_csr")
    del arr


def select_csr(desc: Desc, row_ptr, col_idx, workspace, keep_per_head=None, keep_rows=None, stream=None):
    """plan_csr's row pointers and selection alone, from the tile means the
    pooling permutes (pool / gather_pool, gather_kf_pool) left in the
    workspace."""
    arr, kp = _keep_heads(desc, keep_per_head)
    _check(lib().bsa_select_csr(ctypes.byref(desc), kp, _ptr(keep_rows), _ptr(row_ptr), _ptr(col_idx),
                                col_idx.numel(), _ptr(workspace), _ws(workspace), _stream(stream)), "bsa_select_csr")
    del arr


def forward_csr_raster(desc: Desc, q_raster, perm, k_frag, v_frag, row_ptr, col_idx, o_raster, lse=None,
                       workspace=None, stream=None):
    """forward_csr with Q read from and O written to the raster layout through
    ``perm`` (the same values as gather, forward_csr and scatter)."""
    _check(lib().bsa_forward_csr_raster(ctypes.byref(desc), _ptr(q_raster), _ptr(perm), _ptr(k_frag), _ptr(v_frag),
                                        _ptr(row_ptr), _ptr(col_idx), col_idx.numel(), _ptr(o_raster), _ptr(lse),
                                        _ptr(workspace), _ws(workspace), _stream(stream)), "bsa_forward_csr_raster")


def forward_csr(desc: Desc, q_tiled, k_frag, v_frag, row_ptr, col_idx, o_tiled, lse=None, workspace=None,
                stream=None):
    """bsa_forward with the kept lists in CSR form (from plan_csr)."""
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().bsa_forward_csr(ctypes.byref(desc), _ptr(q_tiled), _ptr(k_frag), _ptr(v_frag), _ptr(row_ptr),
                                 _ptr(col_idx), col_idx.numel(), _ptr(o_tiled), _ptr(lse), _ptr(workspace), ws,
                                 _stream(stream)), "bsa_forward_csr")


def _head_mask(desc: Desc, head_mask):
    if len(head_mask) != desc.heads:
        raise ValueError("head_mask needs one entry per head")
    arr = (ctypes.c_int32 * len(head_mask))(*[int(x) for x in head_mask])
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def structured_entries(desc: Desc, head_mask, radius_t: int, radius_hw: int) -> int:
    """Entries of the structured CSR lists (MASK_SPATIAL / MASK_TEMPORAL per head)."""
    arr, hp = _head_mask(desc, head_mask)
    n = ctypes.c_int64(0)
    _check(lib().bsa_structured_entries(ctypes.byref(desc), hp, int(radius_t), int(radius_hw), ctypes.byref(n)),
           "bsa_structured_entries")
    return n.value


def plan_structured(desc: Desc, head_mask, radius_t: int, radius_hw: int, row_ptr, col_idx, stream=None):
    """Structured lists: spatial heads keep the tiles within radius_t tile-frames,
    temporal heads the tiles within radius_hw in h and w at every time; CSR
    output for forward_csr."""
    arr, hp = _head_mask(desc, head_mask)
    _check(lib().bsa_plan_structured(ctypes.byref(desc), hp, int(radius_t), int(radius_hw), _ptr(row_ptr),
                                     _ptr(col_idx), col_idx.numel(), _stream(stream)), "bsa_plan_structured")


def backward_workspace_size(desc: Desc) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().bsa_backward_workspace_size(ctypes.byref(desc), ctypes.byref(n)), "bsa_backward_workspace_size")
    return n.value


def backward(desc: Desc, q, k, v, o, d_o, lse, perm, block_idx, dq, dk, dv, workspace, stream=None):
    """Gradients of the forward: raster bf16 ``q, k, v, o, d_o`` ``[B, Ntot, H, D]``,
    the forward's ``lse`` ``[B, H, Ntot]`` (tiled order), ``perm`` and ``block_idx``
    -> raster bf16 ``dq, dk, dv``."""
    ws = workspace.numel() * workspace.element_size()
    _check(lib().bsa_backward(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse),
                              _ptr(perm), _ptr(block_idx), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws,
                              _stream(stream)), "bsa_backward")


def backward_stats_offset(desc: Desc, col_entries: int = 0) -> int:
    """Byte offset in the backward workspace (col_entries 0: the fixed-keep
    one; else the CSR one of that many columns) of int32 stats[4]."""
    n = ctypes.c_size_t(0)
    _check(lib().bsa_backward_stats_offset(ctypes.byref(desc), int(col_entries), ctypes.byref(n)),
           "bsa_backward_stats_offset")
    return n.value


def backward_stats(desc: Desc, workspace, col_entries: int = 0):
    """(dQ waits that gave up, dQ rounds, dK/dV waits that gave up, dK/dV
    rounds) of the last backward call on this workspace (a device read:
    synchronises the stream)."""
    off = backward_stats_offset(desc, col_entries)
    return tuple(int(x) for x in workspace.view(torch.uint8)[off:off + 16].view(torch.int32).cpu().tolist())


def backward_csr_workspace_size(desc: Desc, col_entries: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().bsa_backward_csr_workspace_size(ctypes.byref(desc), int(col_entries), ctypes.byref(n)),
           "bsa_backward_csr_workspace_size")
    return n.value


def backward_csr(desc: Desc, q, k, v, o, d_o, lse, perm, row_ptr, col_idx, dq, dk, dv, workspace, stream=None):
    """As ``backward``, over the CSR lists of ``plan_csr`` / ``plan_structured``."""
    ws = workspace.numel() * workspace.element_size()
    _check(lib().bsa_backward_csr(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(d_o), _ptr(lse),
                                  _ptr(perm), _ptr(row_ptr), _ptr(col_idx), col_idx.numel(), _ptr(dq), _ptr(dk),
                                  _ptr(dv), _ptr(workspace), ws, _stream(stream)), "bsa_backward_csr")


def pooled_views(desc: Desc, workspace):
    """(qbar, kbar) float views of the workspace after bsa_plan ([B, H, nVT, D])."""
    B, H, D = desc.batch, desc.heads, desc.head_dim
    nvt = video_slots(desc) // 64
    n = B * H * nvt * D
    pooled_bytes = (n * 4 + 255) // 256 * 256
    f = workspace.view(torch.uint8)
    q = f[:n * 4].view(torch.float32).view(B, H, nvt, D)
    k = f[pooled_bytes:pooled_bytes + n * 4].view(torch.float32).view(B, H, nvt, D)
    return q, k


class BlockSparseAttention:
    """Owns the device buffers of one problem size and runs the whole path:
    permutation (build, gather Q/K/V), plan, forward and the output scatter.

    ``__call__(q, k, v)`` takes raster bf16 tensors ``[B, Ntot, H, D]`` on the
    GPU and returns the raster output.  Buffers are allocated once, through
    torch: the fragment-layout K and V, the lists and the workspace in the
    constructor, the tiled Q and O (``q_t``, ``o_t``) on first use.  With
    ``overlap`` the V gather runs on a side stream (default priority) while the
    plan runs on the caller's stream: the plan does not read V, and the forward
    waits for both.  With ``pool_in_gather`` (default) the Q and K gathers also
    take the tile means (bsa_permute GATHER_POOL / GATHER_KF_POOL) and the plan
    is bsa_select; otherwise plain gathers and bsa_plan, which reads Q and K
    again.  With ``raster_io`` (default; needs ``pool_in_gather``) ``__call__``
    skips the tiled Q and O: Q's means come from bsa_permute(POOL) and
    bsa_forward_raster reads raster Q and writes raster O itself."""

    def __init__(self, desc: Desc, device="cuda", with_lse: bool = False, grouped: bool = True,
                 overlap: bool = True, pool_in_gather: bool = True, raster_io: bool = True):
        self.desc = desc
        B, H, D = desc.batch, desc.heads, desc.head_dim
        self.device = device
        self.n_video = video_slots(desc)  # tiled video tokens (padding slots included)
        self.n_tot = desc.n_prefix + self.n_video
        self.nvt = self.n_video // 64
        self.dynamic = desc.tile_mode == TILE_DYNAMIC
        bf = torch.bfloat16
        self.perm = torch.empty((B, max(self.n_video, 1)), dtype=torch.int32, device=device)
        regions = (desc.grid_t // 8) * (desc.grid_h // 8) * (desc.grid_w // 8)
        self.shape_map = torch.empty((B, max(regions, 1)), dtype=torch.uint8, device=device) if self.dynamic else None
        # k_f, v_f: the fragment layouts (the size of the tiled layout)
        self.k_f, self.v_f = (torch.empty((B, H, self.n_tot, D), dtype=bf, device=device) for _ in range(2))
        self._q_t = self._o_t = None
        self.block_idx = torch.empty((B, H, max(self.nvt, 1), max(desc.keep_tiles, 1)), dtype=torch.int32,
                                     device=device)
        self.workspace = torch.empty(max(workspace_size(desc), 256), dtype=torch.uint8, device=device)
        self.lse = torch.empty((B, H, self.n_tot), dtype=torch.float32, device=device) if with_lse else None
        self.grouped = grouped
        self.pool_in_gather = pool_in_gather
        self.raster_io = raster_io and pool_in_gather
        self.side = torch.cuda.Stream(device=device) if overlap else None

    def _tiled(self):
        d = self.desc
        return torch.empty((d.batch, d.heads, self.n_tot, d.head_dim), dtype=torch.bfloat16, device=self.device)

    @property
    def q_t(self):
        """Tiled Q [B, H, Ntot, D] (allocated on first use)."""
        if self._q_t is None:
            self._q_t = self._tiled()
        return self._q_t

    @property
    def o_t(self):
        """Tiled O [B, H, Ntot, D] (allocated on first use)."""
        if self._o_t is None:
            self._o_t = self._tiled()
        return self._o_t

    def build(self, q, stream=None):
        permute_build(self.desc, self.perm, self.shape_map, q if self.dynamic else None, self.workspace, stream)

    def gather_qkv(self, q, k, v, stream=None):
        self.gather_qk(q, k, stream)
        self.gather_v(v, stream)

    def gather_qk(self, q, k, stream=None):
        if self.pool_in_gather:
            gather_pool(self.desc, q, self.q_t, self.perm, self.workspace, stream)
            gather_kf_pool(self.desc, k, self.k_f, self.perm, self.workspace, stream)
        else:
            gather(self.desc, q, self.q_t, self.perm, stream)
            gather_kf(self.desc, k, self.k_f, self.perm, stream)

    def pool_qk(self, q, k, stream=None):
        """The raster-I/O path's first step: Q's tile means (no tiled copy) and
        the K gather with K's means."""
        pool(self.desc, q, self.perm, self.workspace, stream)
        gather_kf_pool(self.desc, k, self.k_f, self.perm, self.workspace, stream)

    def gather_v(self, v, stream=None):
        gather_vf(self.desc, v, self.v_f, self.perm, stream)

    def gather_v_and_plan(self, v, stream=None):
        """The V gather and the plan, overlapped on the side stream when there
        is one and ``stream`` is a torch stream or None."""
        if self.side is None or not (stream is None or isinstance(stream, torch.cuda.Stream)):
            self.gather_v(v, stream)
            self.plan(stream)
            return
        cur = torch.cuda.current_stream() if stream is None else stream
        self.side.wait_stream(cur)
        self.gather_v(v, self.side)
        self.plan(cur)
        cur.wait_stream(self.side)

    def plan(self, stream=None):
        if self.pool_in_gather:
            select(self.desc, self.block_idx, self.workspace, stream)
        else:
            plan(self.desc, self.q_t, self.k_f, self.block_idx, self.workspace, stream)

    def forward(self, stream=None):
        forward(self.desc, self.q_t, self.k_f, self.v_f, self.block_idx, self.o_t, self.lse,
                self.workspace if self.grouped else None, stream)

    def backward_workspace(self):
        """The bsa_backward workspace for this problem size (allocated on first use)."""
        if getattr(self, "_bwd_ws", None) is None:
            self._bwd_ws = torch.empty(backward_workspace_size(self.desc), dtype=torch.uint8, device=self.device)
        return self._bwd_ws

    def forward_raster(self, q, out, stream=None):
        """The forward from raster Q straight into raster ``out``."""
        forward_raster(self.desc, q, self.perm, self.k_f, self.v_f, self.block_idx, out, self.lse,
                       self.workspace if self.grouped else None, stream)

    def scatter_out(self, out, stream=None):
        scatter(self.desc, self.o_t, out, self.perm, stream)

    def __call__(self, q, k, v, out=None, stream=None):
        if out is None:
            out = torch.empty_like(q)
        self.build(q, stream)
        if self.raster_io:
            self.pool_qk(q, k, stream)
            self.gather_v_and_plan(v, stream)
            self.forward_raster(q, out, stream)
            return out
        self.gather_qk(q, k, stream)
        self.gather_v_and_plan(v, stream)
        self.forward(stream)
        self.scatter_out(out, stream)
        return out


class _Attention(torch.autograd.Function):
    """The op as a differentiable torch function: forward through the raster
    path of a BlockSparseAttention, backward through bsa_backward with the
    forward's own permutation, kept lists and lse (the selection is held
    fixed: the gradient is that of exact attention over the kept tiles)."""

    @staticmethod
    def forward(ctx, q, k, v, att):
        out = torch.empty_like(q)
        att(q, k, v, out)
        # this call's permutation, lists and lse: the next call through the
        # same object overwrites its buffers
        ctx.save_for_backward(q, k, v, out, att.perm.clone(), att.block_idx.clone(), att.lse.clone())
        ctx.att = att
        return out

    @staticmethod
    def backward(ctx, d_o):
        q, k, v, out, perm, block_idx, lse = ctx.saved_tensors
        att = ctx.att
        d_o = d_o.to(torch.bfloat16).contiguous()
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        backward(att.desc, q, k, v, out, d_o, lse, perm, block_idx, dq, dk, dv, att.backward_workspace())
        return dq, dk, dv, None


def attention(q, k, v, att: "BlockSparseAttention"):
    """Block-sparse attention of raster bf16 ``q, k, v`` ``[B, Ntot, H, D]`` (on
    the GPU, contiguous) as a differentiable operation: returns the raster
    output; its gradient runs bsa_backward with this call's own selection.
    ``att`` owns the buffers for ``q``'s size (``BlockSparseAttention(desc)``);
    one object can serve several calls (layers), each saving its lists."""
    if att.lse is None:
        att.lse = torch.empty((att.desc.batch, att.desc.heads, att.n_tot), dtype=torch.float32, device=q.device)
    return _Attention.apply(q, k, v, att)
