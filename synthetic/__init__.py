"""Seeded synthetic inputs for block-sparse video attention.

Shared by the tests, the benchmark and the smoke check, and by both the GPU
path and the CPU oracle.  It only draws random numbers and rounds them to bf16:
no step of the attention method lives here.

Every value is reproducible from ``(seed, tensor, b, h)``: each (batch, head)
slice of each tensor comes from its own numpy PCG64 stream, so a slice can be
regenerated alone (full-size parity checks sample a few heads) and a whole
tensor can be generated on several threads with identical bytes.

Recipes (the workloads of the design notes):

* ``offsets``: element = N(0,1) + an offset vector ~ N(0, 0.5^2) per
  (batch, head, tensor, tile) shared by the tile's 64 tokens.  Video tiles are
  the static 4x4x4 tiles of the grid; prefix tiles are 64-token runs.
* ``field``: a smooth spatio-temporal field plus N(0,1) noise whose dominant
  axis drifts across the grid, so per-region shape choices vary:
  A*[a_t sin(2 pi t/L + p1) + a_h sin(2 pi h/L + p2) + a_w sin(2 pi w/L + p3)]
  with a_t = sin^2(pi w/W), a_h = sin^2(pi t/T), a_w = sin^2(pi h/H) and
  phases p per (tensor, head, channel) ~ U[0, 2 pi).
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TENSOR_ID = {"q": 0, "k": 1, "v": 2, "do": 3}  # "do": the output gradient of a backward pass


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    grid: tuple            # (T, H, W) video tokens
    keep_tiles: int        # kept video key tiles per video query tile
    seed: int
    n_prefix: int = 0      # dense conditioning tokens stored before the video
    dynamic: bool = False  # dynamic tile shapes per 8x8x8 region
    recipe: str = "offsets"
    tile: tuple = (4, 4, 4)
    tau: float = 0.10
    field_amp: float = 2.0
    field_period: float = 4.0
    padded: bool = False   # ragged grid: static tiles over the grid rounded up

    @property
    def n_video(self) -> int:
        """Video tokens of the raster tensors (the real grid)."""
        T, H, W = self.grid
        return T * H * W

    @property
    def n_tokens(self) -> int:
        """Tokens of the raster tensors."""
        return self.n_prefix + self.n_video

    @property
    def n_video_slots(self) -> int:
        """Video tokens of the tiled order: the grid, or with ``padded`` the
        grid rounded up to whole tiles on every axis."""
        if not self.padded:
            return self.n_video
        return int(np.prod([-(-g // t) * t for g, t in zip(self.grid, self.tile)]))

    @property
    def n_tiled_tokens(self) -> int:
        return self.n_prefix + self.n_video_slots

    @property
    def n_video_tiles(self) -> int:
        return self.n_video_slots // 64

    @property
    def n_prefix_tiles(self) -> int:
        return self.n_prefix // 64

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def with_keep(self, k: int) -> "Workload":
        return dataclasses.replace(self, keep_tiles=k, name=f"{self.name}_k{k}")

    def effective_flops(self) -> float:
        """4 * B * H * D * sum over query tokens of the keys it attends to
        (two matrix products over the kept tiles and the prefix only).  On a
        ragged grid every tile counts whole (padding slots included), as the
        kernels compute them."""
        keys_prefix_q = self.n_tiled_tokens                     # prefix queries: dense
        keys_video_q = self.n_prefix + self.keep_tiles * 64     # video queries
        pairs = self.n_prefix * keys_prefix_q + self.n_video_slots * keys_video_q
        return 4.0 * self.batch * self.heads * self.head_dim * pairs


def keep_from_sparsity(n_tiles: int, sparsity: float) -> int:
    """k = round((1 - s) * n), clamped to [1, n] (1,920 tiles at s = 0.75 -> 480)."""
    k = int(math.floor((1.0 - sparsity) * n_tiles + 0.5))
    return max(1, min(n_tiles, k))


# The workloads of the design notes.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 64, (8, 16, 16), 8, seed=0),
    "prism720p": Workload("prism720p", 2, 24, 128, (32, 48, 80), 480, seed=1),
    "prism720p_dynamic": Workload("prism720p_dynamic", 2, 24, 128, (32, 48, 80), 480, seed=3,
                                  dynamic=True, recipe="field"),
    "prefix": Workload("prefix", 1, 24, 128, (24, 48, 84), 378, seed=4, n_prefix=2048),
    # 121 frames of 720p through a 4x temporal / 16x spatial latent: 31 x 45 x 80
    # tokens, padded to the 32 x 48 x 80 tile grid (1,920 tiles)
    "prism720p_ragged": Workload("prism720p_ragged", 2, 24, 128, (31, 45, 80), 480, seed=5, padded=True),
}
KEEP_SWEEP = (480, 192, 120, 96)   # 25 %, 10 %, 6.25 %, 5 % of 1,920 tiles


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _ceil4(n: int) -> int:
    return (n + 3) // 4


def _video_static_tile_of_token(grid) -> np.ndarray:
    """4x4x4 box index of every video token (boxes may be partial at the edges)."""
    T, H, W = grid
    t = np.arange(T)[:, None, None] // 4
    h = np.arange(H)[None, :, None] // 4
    w = np.arange(W)[None, None, :] // 4
    return ((t * _ceil4(H) + h) * _ceil4(W) + w).reshape(-1)


def slice_bh(wl: Workload, tensor: str, b: int, h: int) -> np.ndarray:
    """One (batch, head) slice in raster token order, bf16 bits ``[Ntot, D]``."""
    tid = TENSOR_ID[tensor]
    D = wl.head_dim
    rng = np.random.default_rng([wl.seed, tid, b, h, 0])
    x = rng.standard_normal((wl.n_tokens, D), dtype=np.float32)
    if wl.recipe == "offsets":
        T, H, W = wl.grid
        n_vt_static = _ceil4(T) * _ceil4(H) * _ceil4(W)
        npt = wl.n_prefix // 64
        orng = np.random.default_rng([wl.seed, tid, b, h, 1])
        off = (0.5 * orng.standard_normal((npt + n_vt_static, D), dtype=np.float32)).astype(np.float32)
        tile_of = np.concatenate([np.arange(wl.n_prefix) // 64, npt + _video_static_tile_of_token(wl.grid)])
        x += off[tile_of]
    elif wl.recipe == "field":
        T, H, W = wl.grid
        prng = np.random.default_rng([wl.seed, tid, h, 2])
        ph = prng.uniform(0.0, 2.0 * np.pi, size=(3, D)).astype(np.float64)
        t = np.arange(T, dtype=np.float64)[:, None, None]
        hh = np.arange(H, dtype=np.float64)[None, :, None]
        w = np.arange(W, dtype=np.float64)[None, None, :]
        a_t = np.sin(np.pi * w / W) ** 2
        a_h = np.sin(np.pi * t / T) ** 2
        a_w = np.sin(np.pi * hh / H) ** 2
        L = wl.field_period
        s_t = np.sin(2 * np.pi * t[..., None] / L + ph[0])   # [T,1,1,D]
        s_h = np.sin(2 * np.pi * hh[..., None] / L + ph[1])  # [1,H,1,D]
        s_w = np.sin(2 * np.pi * w[..., None] / L + ph[2])   # [1,1,W,D]
        field = wl.field_amp * (a_t[..., None] * s_t + a_h[..., None] * s_h + a_w[..., None] * s_w)
        field = field.astype(np.float32)
        x[wl.n_prefix:] += field.reshape(-1, D)
    else:
        raise ValueError(wl.recipe)
    return to_bf16_bits(x)


def tensor(wl: Workload, name: str, threads: int | None = None) -> np.ndarray:
    """A whole raster tensor ``uint16 [B, Ntot, H, D]`` (bf16 bits)."""
    out = np.empty((wl.batch, wl.n_tokens, wl.heads, wl.head_dim), np.uint16)

    def fill(bh):
        b, h = divmod(bh, wl.heads)
        out[b, :, h, :] = slice_bh(wl, name, b, h)

    n = wl.batch * wl.heads
    threads = threads or min(16, os.cpu_count() or 1)
    if n == 1 or threads == 1:
        for bh in range(n):
            fill(bh)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(n)))
    return out


def qkv(wl: Workload, threads: int | None = None):
    return tuple(tensor(wl, n, threads) for n in ("q", "k", "v"))
