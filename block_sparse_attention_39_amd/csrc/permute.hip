// Token permutation between raster order and tile order.
//
// Tokens are regrouped so that every 64-token tile is contiguous per head
// ("Sparse VideoGen TPU 최적화 ..." page, section "실무에서 배울 최적화 기준": token
// permutation makes a sparsity pattern's tiles contiguous, and its cost is
// measured on its own).  The copy is a pure HBM-bound gather: each block moves
// one tile of 64 tokens for every head, reading 256-byte head rows of the
// raster layout and writing 16 KB contiguous runs per head in the tiled layout.
#include "bsa_kernels.h"

namespace bsa {
namespace {

// Static tile order: tile id = raster index in the tile grid (t slowest),
// tokens raster inside the tile ("Prism / Kandinsky 6 speed ablation" page,
// section on Prism: the default 64-token tile is 4x4x4).  The tile grid covers
// T x Hg x W rounded up to whole tiles; a slot past the grid on some axis is
// padding and gets -1.
__global__ void perm_static_kernel(int T, int Hg, int W, int tt, int th, int tw, int64_t n_video, int B,
                                   int32_t* __restrict__ perm) {
    const int64_t total = n_video * B;
    const int nbh = (Hg + th - 1) / th, nbw = (W + tw - 1) / tw;
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
         g += (int64_t)gridDim.x * blockDim.x) {
        const int64_t p = g % n_video;
        const int64_t tile = p / kTile;
        const int r = (int)(p % kTile);
        const int64_t a = tile / ((int64_t)nbh * nbw);
        const int bb = (int)((tile / nbw) % nbh);
        const int cc = (int)(tile % nbw);
        const int x = r / (th * tw), y = (r / tw) % th, z = r % tw;
        const int64_t t = a * tt + x;
        const int h = bb * th + y, w = cc * tw + z;
        perm[g] = (t < T && h < Hg && w < W) ? (int32_t)((t * Hg + h) * W + w) : -1;
    }
}

// x, or zeros when t < 0 (a padding slot), by a bit mask rather than a
// select, so that the load is not moved under a branch: the row loads of a
// thread stay unconditional and in flight together.
// kPad false: a grid of whole tiles, no padding slot and no masking.
template <bool kPad>
__device__ inline uint4 zero_if_padding(uint4 x, int64_t t) {
    if (!kPad) return x;
    const uint32_t m = ~(uint32_t)(t >> 63);  // t < 0: 0; else all ones
    return make_uint4(x.x & m, x.y & m, x.z & m, x.w & m);
}
template <bool kPad>
__device__ inline int64_t row_or_zero(int64_t t) { return kPad ? max(t, (int64_t)0) : t; }

// Raster row (prefix first) of tiled slot p, or -1 for a padding slot (kPad:
// a ragged grid).  A video value outside the raster's n_ras - n_prefix rows
// is clamped into them (below 0 to row 0 without padding), so that a corrupt
// perm cannot address outside the tensors.
template <bool kPad>
__device__ inline int64_t slot_token(const int32_t* __restrict__ perm, int b, int64_t n_video, int n_prefix,
                                     int64_t n_ras, int64_t p) {
    if (p < n_prefix) return p;
    const int32_t v = perm[(int64_t)b * n_video + (p - n_prefix)];
    if (kPad && v < 0) return -1;
    return n_prefix + min(max((int64_t)v, (int64_t)0), n_ras - n_prefix - 1);
}

// One block per (batch, 64-token tile of the tiled order); 256 threads.
// Work item = (head, token in tile, 16-byte chunk), chunk fastest, so a wave
// writes (gather) or reads (scatter) contiguous 256-byte head rows of the
// tiled tensor and touches 256-byte head rows of the raster tensor.
// n_tot: tiled rows (padding slots included); n_ras: raster rows.  Gather
// writes zeros to padding slots, scatter skips them.
template <bool kToRaster, bool kPad>
__global__ __launch_bounds__(256) void permute_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                           const int32_t* __restrict__ perm, int H, int C,
                                                           int n_prefix, int64_t n_video, int64_t n_tot,
                                                           int64_t n_ras) {
    __shared__ int64_t tok[kTile];
    const int b = blockIdx.y;
    const int64_t p0 = (int64_t)blockIdx.x * kTile;
    if (threadIdx.x < kTile) tok[threadIdx.x] = slot_token<kPad>(perm, b, n_video, n_prefix, n_ras, p0 + threadIdx.x);
    __syncthreads();
    const int items = kTile * H * C;
#pragma unroll 4
    for (int it = threadIdx.x; it < items; it += 256) {
        const int c = it % C;
        const int pl = (it / C) % kTile;
        const int h = it / (C * kTile);
        const int64_t tiled = (((int64_t)b * H + h) * n_tot + p0 + pl) * C + c;
        const int64_t t = tok[pl];
        // a padding slot (t < 0) reads a valid row and writes zeros
        const int64_t raster = (((int64_t)b * n_ras + row_or_zero<kPad>(t)) * H + h) * C + c;
        if (kToRaster) {
            if (!kPad || t >= 0) dst[raster] = src[tiled];
        } else {
            dst[tiled] = zero_if_padding<kPad>(src[raster], t);
        }
    }
}

// One 16-byte chunk (channels 8 cc .. +7) of token row t of head h: from the
// raster layout (t: raster row, < 0 for a padding slot, read as zeros) or,
// with kTiled, from the tiled layout (t: tiled row).
template <bool kTiled, bool kPad>
__device__ inline uint4 src_chunk(const uint4* __restrict__ src, int b, int h, int H, int C, int cc, int64_t t,
                                  int64_t n_ras, int64_t n_tot) {
    if (kTiled) return src[(((int64_t)b * H + h) * n_tot + t) * C + cc];
    return zero_if_padding<kPad>(src[(((int64_t)b * n_ras + row_or_zero<kPad>(t)) * H + h) * C + cc], t);
}

// Raster K -> K-fragment layout [B][H][tile][kh][s][lane][8]: chunk
// (kh, s, lane) of a tile holds channels 16 s + 8 (lane / 32) .. +7 of the
// tile's token 32 kh + swap23(lane % 32) (bits 2 and 3 exchanged), i.e. the
// A operand of v_mfma_f32_32x32x16_bf16 for the S^T = K Q^T products of the
// attention kernel.  One block per (batch, tile); work item = (head, chunk),
// chunk fastest, so a wave writes 1 KB contiguous and reads 32-byte runs of
// the tile's raster rows.  kTiled: the source is the tiled layout instead.
__device__ inline int swap23(int m) { return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <bool kPad, bool kTiled = false>
__global__ __launch_bounds__(256) void gather_kf_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        const int32_t* __restrict__ perm, int H, int C,
                                                        int n_prefix, int64_t n_video, int64_t n_tot,
                                                        int64_t n_ras) {
    __shared__ int64_t tok[kTile];
    const int b = blockIdx.y;
    const int64_t tile = blockIdx.x;
    const int64_t p0 = tile * kTile;
    const int64_t n_tiles = n_tot / kTile;
    if (threadIdx.x < kTile)
        tok[threadIdx.x] = kTiled ? p0 + threadIdx.x : slot_token<kPad>(perm, b, n_video, n_prefix, n_ras, p0 + threadIdx.x);
    __syncthreads();
    const int SD = C / 2;
    const int per_head = kTile * C;
    const int items = H * per_head;
#pragma unroll 4
    for (int it = threadIdx.x; it < items; it += 256) {
        const int q = it % per_head, h = it / per_head;
        const int lane = q & 63, s = (q >> 6) % SD, kh = (q >> 6) / SD;
        const int r = 32 * kh + swap23(lane & 31);
        const int cc = 2 * s + (lane >> 5);
        dst[(((int64_t)b * H + h) * n_tiles + tile) * per_head + q] =
            src_chunk<kTiled, kPad>(src, b, h, H, C, cc, tok[r], n_ras, n_tot);
    }
}

// Raster V -> V-fragment layout [B][H][tile][kh][i][c][lane][8]: chunk
// (kh, i, c, lane) of a tile holds channel 32 i + lane % 32 of the tile's
// tokens 32 kh + 16 c + 8 (lane / 32) .. +7, i.e. the A operand of the
// O^T = V^T P^T products.  One block per (batch, tile); work item = (head,
// group of 8 tokens, 8-channel chunk): a thread reads 8 token rows of 16 bytes
// (256-byte head rows across a wave), transposes the 8 x 8 block of bf16
// values in registers and writes 8 chunks for 8 consecutive lanes (128 bytes
// contiguous).  kTiled: the source is the tiled layout instead.
__device__ inline uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ inline uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }
__device__ inline uint32_t word_of(const uint4& v, int w) { return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w; }

template <bool kPad, bool kTiled = false>
__global__ __launch_bounds__(256) void gather_vf_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        const int32_t* __restrict__ perm, int H, int C,
                                                        int n_prefix, int64_t n_video, int64_t n_tot,
                                                        int64_t n_ras) {
    __shared__ int64_t tok[kTile];
    const int b = blockIdx.y;
    const int64_t tile = blockIdx.x;
    const int64_t p0 = tile * kTile;
    const int64_t n_tiles = n_tot / kTile;
    if (threadIdx.x < kTile)
        tok[threadIdx.x] = kTiled ? p0 + threadIdx.x : slot_token<kPad>(perm, b, n_video, n_prefix, n_ras, p0 + threadIdx.x);
    __syncthreads();
    const int OD = C / 4;  // 32-channel blocks
    const int items = H * 8 * C;
    for (int it = threadIdx.x; it < items; it += 256) {
        const int dc = it % C;
        const int g = (it / C) % 8;
        const int h = it / (8 * C);
        uint4 r0, r1, r2, r3, r4, r5, r6, r7;
        auto row = [&](int i) { return src_chunk<kTiled, kPad>(src, b, h, H, C, dc, tok[8 * g + i], n_ras, n_tot); };
        r0 = row(0); r1 = row(1); r2 = row(2); r3 = row(3);
        r4 = row(4); r5 = row(5); r6 = row(6); r7 = row(7);
        // tokens 8 g .. 8 g + 7 = 32 kh + 16 c + 8 hf + e; channels 8 dc + e'
        // = 32 i + 8 (dc % 4) + e' -> lane 32 hf + 8 (dc % 4) + e'
        const int kh = g >> 2, c = (g >> 1) & 1, hf = g & 1, i = dc >> 2;
        uint4* out = dst + (((int64_t)b * H + h) * n_tiles + tile) * (kTile * C) +
                     ((kh * OD + i) * 2 + c) * 64 + 32 * hf + 8 * (dc & 3);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int w = e >> 1;
            uint4 o;
            if (e & 1) {
                o.x = hi_pair(word_of(r0, w), word_of(r1, w));
                o.y = hi_pair(word_of(r2, w), word_of(r3, w));
                o.z = hi_pair(word_of(r4, w), word_of(r5, w));
                o.w = hi_pair(word_of(r6, w), word_of(r7, w));
            } else {
                o.x = lo_pair(word_of(r0, w), word_of(r1, w));
                o.y = lo_pair(word_of(r2, w), word_of(r3, w));
                o.z = lo_pair(word_of(r4, w), word_of(r5, w));
                o.w = lo_pair(word_of(r6, w), word_of(r7, w));
            }
            out[e] = o;
        }
    }
}

// ---- the backward's gathers: two layouts from one read ---------------------
// Position of chunk (token pl, 16-byte chunk c) of a tile in the K-fragment
// layout: chunk (kh, s, lane) holds channels 16 s + 8 (lane / 32) .. +7 of
// token 32 kh + swap23(lane % 32), and swap23 is its own inverse.
__device__ inline int kfrag_pos(int pl, int c, int SD) {
    return ((pl >> 5) * SD + (c >> 1)) * 64 + 32 * (c & 1) + swap23(pl & 31);
}

// Raster -> tiled and K-fragment layouts (Q, dO), each written 1 KB per wave
// store.  One block of 4 waves per (batch, tile); a pass takes two heads, wave
// w the token half w % 2 (32 tokens: K-fragment half kh) of head 2 p + w / 2.
// A wave loads its rows as the plain gather does (lane = (token, 16-byte
// chunk), chunk fastest: 1 KB of 256-byte head rows per load), stores them to
// the tiled layout and into its own 8 KB of LDS (chunk c of token r at
// c ^ (r % C): conflict-free both ways), then writes its half of the
// K-fragment tile from there, 1 KB per store.  No wave reads another's rows.
// kDelta (dO): the same chunk of O is read and the C lanes of a token add up
// their products into Delta, with the row's lse forms beside it.
template <bool kPad, bool kDelta>
__global__ __launch_bounds__(256) void gather_kf_tiled_kernel(const uint4* __restrict__ src,
                                                              uint4* __restrict__ dst_kf, uint4* __restrict__ dst_t,
                                                              const int32_t* __restrict__ perm, int H, int C,
                                                              int n_prefix, int64_t n_video, int64_t n_tot,
                                                              int64_t n_ras, DeltaOut dl) {
    __shared__ int64_t tok[kTile];
    __shared__ uint4 stage[4][32 * 16];  // per wave: 32 tokens x up to 16 chunks
    const int b = blockIdx.y;
    const int64_t tile = blockIdx.x, p0 = tile * kTile, n_tiles = n_tot / kTile;
    if (threadIdx.x < kTile) tok[threadIdx.x] = slot_token<kPad>(perm, b, n_video, n_prefix, n_ras, p0 + threadIdx.x);
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, kh = wave & 1;
    const int SD = C / 2, tpi = 64 / C;  // tpi: tokens per wave load
    const int c = lane % C, ts = lane / C;
    uint4* st = stage[wave];
    for (int hp = 0; hp < H; hp += 2) {
        const int h = hp + (wave >> 1);
        if (h < H) {
            const int64_t bh = (int64_t)b * H + h;
            uint4* dt = dst_t + (bh * n_tot + p0) * C;
#pragma unroll
            for (int i = 0; i < 32 / tpi; ++i) {
                const int r = i * tpi + ts, pl = 32 * kh + r;  // r: token within the half
                const int64_t t = tok[pl];
                const uint4 x = src_chunk<false, kPad>(src, b, h, H, C, c, t, n_ras, n_tot);
                dt[pl * C + c] = x;
                st[r * C + (c ^ (r % C))] = x;
                if (kDelta) {
                    const uint4 y = src_chunk<false, kPad>((const uint4*)dl.o, b, h, H, C, c, t, n_ras, n_tot);
                    float d = 0.f;  // a padding row reads zeros: Delta 0
                    const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        d = fmaf(__uint_as_float(ys[w] << 16), __uint_as_float(xs[w] << 16), d);
                        d = fmaf(__uint_as_float(ys[w] & 0xffff0000u), __uint_as_float(xs[w] & 0xffff0000u), d);
                    }
                    for (int o = 1; o < C; o <<= 1) d += __shfl_xor(d, o);
                    if (c == 0) {
                        const int64_t rr = bh * n_tot + p0 + pl;
                        dl.delta[rr] = d;
                        dl.ndelta[rr] = -d;
                        if (t >= 0) {
                            dl.lse2[rr] = dl.lse[rr] * 1.4426950408889634f;
                            dl.nlse[rr] = -dl.lse[rr] / dl.scale;
                        } else {  // a padding row carries no loss: every weight of it is exactly 0
                            dl.lse2[rr] = __builtin_inff();
                            dl.nlse[rr] = -__builtin_inff();
                        }
                    }
                }
            }
        }
        __syncthreads();  // the stage is complete (and the tok reads done)
        if (h < H) {
            const int64_t bh = (int64_t)b * H + h;
            // K-fragment half kh: chunk (kh, s, lane) = channels 16 s + 8 (lane / 32)
            // of token 32 kh + swap23(lane % 32)
            uint4* dk = dst_kf + (bh * n_tiles + tile) * (kTile * C) + kh * SD * 64 + lane;
            const int r = swap23(lane & 31);
#pragma unroll 4
            for (int s2 = 0; s2 < SD; ++s2) {
                const int cc = 2 * s2 + (lane >> 5);
                dk[s2 * 64] = st[r * C + (cc ^ (r % C))];
            }
        }
        __syncthreads();  // before the next pass overwrites the stage
    }
}

// Raster -> K-fragment and V-fragment layouts (K), each written 128 bytes or
// more per lane group.  The V-fragment gather's mapping: a thread reads 8
// token rows of one 16-byte chunk and writes their 8 x 8 transpose; a wave
// covers 32 tokens (D = 128: two waves per head, wave = K-fragment half) or
// all 64 (D = 64).  It also puts the chunks into its own LDS (chunk c of its
// token r at c ^ (r % C)) and then writes its K-fragment chunks from there,
// 1 KB per store.  No wave reads another's rows.
template <bool kPad>
__global__ __launch_bounds__(256) void gather_kf_vf_kernel(const uint4* __restrict__ src,
                                                           uint4* __restrict__ dst_kf, uint4* __restrict__ dst_vf,
                                                           const int32_t* __restrict__ perm, int H, int C,
                                                           int n_prefix, int64_t n_video, int64_t n_tot,
                                                           int64_t n_ras) {
    __shared__ int64_t tok[kTile];
    __shared__ uint4 stage[4][512];  // per wave: 32 tokens x 16 chunks, or 64 x 8
    const int b = blockIdx.y;
    const int64_t tile = blockIdx.x, p0 = tile * kTile, n_tiles = n_tot / kTile;
    if (threadIdx.x < kTile) tok[threadIdx.x] = slot_token<kPad>(perm, b, n_video, n_prefix, n_ras, p0 + threadIdx.x);
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int OD = C / 4, SD = C / 2;
    const int halves = C == 16 ? 1 : 2;  // K-fragment halves a wave holds
    const int items = H * 8 * C;
    uint4* st = stage[wave];
    for (int base = 0; base < items; base += 256) {
        const int it = base + threadIdx.x;
        const int h = it / (8 * C);  // uniform over a wave (8 C is a multiple of 64)
        const bool on = it < items;
        const int dc = it % C, g = (it / C) % 8;
        const int g0 = ((base + wave * 64) / C) % 8;  // the wave's first token group
        const int kh0 = g0 >> 2;
        if (on) {
            uint4 rw[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                rw[i] = src_chunk<false, kPad>(src, b, h, H, C, dc, tok[8 * g + i], n_ras, n_tot);
            const int64_t tbase = (((int64_t)b * H + h) * n_tiles + tile) * (kTile * C);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 8 * (g - g0) + i;  // token within the wave's range
                st[r * C + (dc ^ (r % C))] = rw[i];
            }
            const int kh = g >> 2, c = (g >> 1) & 1, hf = g & 1, ib = dc >> 2;
            uint4* out = dst_vf + tbase + ((kh * OD + ib) * 2 + c) * 64 + 32 * hf + 8 * (dc & 3);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int w = e >> 1;
                uint4 o;
                if (e & 1) {
                    o.x = hi_pair(word_of(rw[0], w), word_of(rw[1], w));
                    o.y = hi_pair(word_of(rw[2], w), word_of(rw[3], w));
                    o.z = hi_pair(word_of(rw[4], w), word_of(rw[5], w));
                    o.w = hi_pair(word_of(rw[6], w), word_of(rw[7], w));
                } else {
                    o.x = lo_pair(word_of(rw[0], w), word_of(rw[1], w));
                    o.y = lo_pair(word_of(rw[2], w), word_of(rw[3], w));
                    o.z = lo_pair(word_of(rw[4], w), word_of(rw[5], w));
                    o.w = lo_pair(word_of(rw[6], w), word_of(rw[7], w));
                }
                out[e] = o;
            }
        }
        __syncthreads();  // the stage is complete
        if (on) {
            const int64_t tbase = (((int64_t)b * H + h) * n_tiles + tile) * (kTile * C);
            for (int hh = 0; hh < halves; ++hh) {
                const int kh = kh0 + hh;
                const int r = 32 * hh + swap23(lane & 31);
                uint4* dk = dst_kf + tbase + kh * SD * 64 + lane;
#pragma unroll 4
                for (int s2 = 0; s2 < SD; ++s2) {
                    const int cc = 2 * s2 + (lane >> 5);
                    dk[s2 * 64] = st[r * C + (cc ^ (r % C))];
                }
            }
        }
        __syncthreads();  // before the next pass overwrites the stage
    }
}

// Q gather with pooling.  One block of 256 threads per (batch, 64-token
// tile); wave w takes heads w, w + 4, ...  Lane l takes chunk c = l % C (16
// bytes) and token offset ts = l / C of a head, so one wave load reads the
// head rows (256 bytes for D = 128) of 64 / C tokens and one wave store writes
// those 64 / C consecutive tokens of the tiled layout, 1 KB contiguous.  A
// lane moves tokens ts, ts + 64/C, ... of its chunk and, for a video tile,
// adds them up in double (exact unless a tile's values span more than 2^39 in
// magnitude), so the means cost no second read of the tensor.  The lanes of a
// chunk fold their sums (shuffles over the high lane bits); the C lanes with
// ts = 0 store the chunk's means and fold the sum of their squares for the
// norm.
template <bool kPad>
__global__ __launch_bounds__(256) void gather_pool_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                          const int32_t* __restrict__ perm, int H, int C,
                                                          int n_prefix, int64_t n_video, int64_t n_tot,
                                                          int64_t n_ras, PoolOut po) {
    constexpr int U = 4;  // loads in flight per lane
    __shared__ int64_t tok[kTile];
    __shared__ int real;
    const int b = blockIdx.y;
    const int64_t p0 = (int64_t)blockIdx.x * kTile;
    if (threadIdx.x < kTile) {
        const int64_t t = slot_token<kPad>(perm, b, n_video, n_prefix, n_ras, p0 + threadIdx.x);
        tok[threadIdx.x] = t;
        const int nr = __popcll(__ballot(t >= 0));
        if (threadIdx.x == 0) real = nr;
    }
    __syncthreads();
    const bool pool = p0 >= n_prefix;
    const int nvt = (int)(n_video / kTile);
    const int64_t vt = (p0 - n_prefix) / kTile;
    const double count = kPad ? (double)real : (double)kTile;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = lane % C, ts = lane / C, tpw = 64 / C;  // tpw: tokens per wave access
    for (int h = wave; h < H; h += 4) {
        const int64_t bh = (int64_t)b * H + h;
        uint4* dh = dst + (bh * n_tot + p0) * C + c;
        double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int pl0 = 0; pl0 < kTile; pl0 += U * tpw) {
            uint4 x[U];
#pragma unroll
            for (int u = 0; u < U; ++u)
                x[u] = src_chunk<false, kPad>(src, b, h, H, C, c, tok[pl0 + ts + tpw * u], n_ras, n_tot);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                dh[(int64_t)(pl0 + ts + tpw * u) * C] = x[u];
                if (pool) {
                    acc[0] += (double)__uint_as_float(x[u].x << 16);
                    acc[1] += (double)__uint_as_float(x[u].x & 0xffff0000u);
                    acc[2] += (double)__uint_as_float(x[u].y << 16);
                    acc[3] += (double)__uint_as_float(x[u].y & 0xffff0000u);
                    acc[4] += (double)__uint_as_float(x[u].z << 16);
                    acc[5] += (double)__uint_as_float(x[u].z & 0xffff0000u);
                    acc[6] += (double)__uint_as_float(x[u].w << 16);
                    acc[7] += (double)__uint_as_float(x[u].w & 0xffff0000u);
                }
            }
        }
        if (pool) {
            for (int o = C; o < 64; o <<= 1)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o);
            float sq = 0.f;
            if (ts == 0) {
                float m[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) m[e] = (float)(acc[e] / count);
                sq = store_pooled8(po, bh, nvt, 8 * C, vt, c, m);
            }
            for (int o = 1; o < C; o <<= 1) sq += __shfl_xor(sq, o);
            if (lane == 0) po.norm[bh * nvt + vt] = sqrtf(sq);
        }
    }
}

// K gather with pooling, its stores in 256-byte runs.  One block of 256
// threads per (batch, tile).  Lane l of a wave takes token offset tq = l % 16
// and chunk group cg = l / 16; the C / 4 waves of a head cover its C chunks
// (c = 4 (wave mod C/4) + cg), and 16 / C heads go per pass.  A lane moves
// tokens tq, tq + 16, tq + 32, tq + 48 of its chunk: one 16-byte load from the
// token's raster row and one store into the K-fragment layout each, where the
// 16 lanes of a chunk (16 consecutive tokens, which swap23 keeps within their
// aligned group of 16) write 256 contiguous bytes.  The lane adds its 4 values
// in double, the 16 lanes of a chunk fold theirs (shuffles over the low four
// lane bits), the chunk's lane tq = 0 stores the means, and the squares for the
// norm are folded over the head's chunks through LDS in a fixed order.
template <bool kPad>
__global__ __launch_bounds__(256) void gather_kf_pool_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                             const int32_t* __restrict__ perm, int H, int C,
                                                             int n_prefix, int64_t n_video, int64_t n_tot,
                                                             int64_t n_ras, PoolOut po) {
    __shared__ int64_t tok[kTile];
    __shared__ int real;
    __shared__ float sqp[4];
    const int b = blockIdx.y;
    const int64_t tile = blockIdx.x, p0 = tile * kTile;
    if (threadIdx.x < kTile) {
        const int64_t t = slot_token<kPad>(perm, b, n_video, n_prefix, n_ras, p0 + threadIdx.x);
        tok[threadIdx.x] = t;
        const int nr = __popcll(__ballot(t >= 0));
        if (threadIdx.x == 0) real = nr;
    }
    __syncthreads();
    const bool pool = p0 >= n_prefix;
    const int nvt = (int)(n_video / kTile);
    const int64_t vt = (p0 - n_prefix) / kTile;
    const double count = kPad ? (double)real : (double)kTile;
    const int64_t n_tiles = n_tot / kTile;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tq = lane & 15, cg = lane >> 4;
    const int wph = C / 4, hpp = 4 / wph;  // waves per head, heads per pass
    const int hl = wave / wph;
    const int c = 4 * (wave % wph) + cg;
    for (int h0 = 0; h0 < H; h0 += hpp) {
        const int h = h0 + hl;
        float sq = 0.f;
        if (h < H) {
            uint4 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u] = src_chunk<false, kPad>(src, b, h, H, C, c, tok[tq + 16 * u], n_ras, n_tot);
            uint4* dh = dst + (((int64_t)b * H + h) * n_tiles + tile) * (kTile * C) + (c >> 1) * 64 + 32 * (c & 1);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int pl = tq + 16 * u;
                dh[(pl >> 5) * (C / 2) * 64 + swap23(pl & 31)] = x[u];
            }
            if (pool) {
                double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    acc[0] += (double)__uint_as_float(x[u].x << 16);
                    acc[1] += (double)__uint_as_float(x[u].x & 0xffff0000u);
                    acc[2] += (double)__uint_as_float(x[u].y << 16);
                    acc[3] += (double)__uint_as_float(x[u].y & 0xffff0000u);
                    acc[4] += (double)__uint_as_float(x[u].z << 16);
                    acc[5] += (double)__uint_as_float(x[u].z & 0xffff0000u);
                    acc[6] += (double)__uint_as_float(x[u].w << 16);
                    acc[7] += (double)__uint_as_float(x[u].w & 0xffff0000u);
                }
#pragma unroll
                for (int o = 1; o < 16; o <<= 1)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o);
                if (tq == 0) {
                    float m[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) m[e] = (float)(acc[e] / count);
                    sq = store_pooled8(po, (int64_t)b * H + h, nvt, 8 * C, vt, c, m);
                }
            }
        }
        if (pool) {
            sq += __shfl_xor(sq, 16);
            sq += __shfl_xor(sq, 32);
            __syncthreads();  // the previous pass has read sqp
            if (lane == 0) sqp[wave] = sq;
            __syncthreads();
            if (h < H && lane == 0 && wave % wph == 0) {
                float t = 0.f;
                for (int w2 = 0; w2 < wph; ++w2) t += sqp[wave + w2];
                po.norm[((int64_t)b * H + h) * nvt + vt] = sqrtf(t);
            }
        }
    }
}

// Q's means alone (no copy), for the forward that reads raster Q itself.  One
// block per (batch, video tile); thread = (head, 16-byte chunk), chunk
// fastest, so a wave load reads one token's rows of 64 / C heads, 1 KB
// contiguous.  A thread adds up its chunk over the tile's 64 tokens in double,
// eight loads in flight, in token order, and stores the means as the gather
// does.
template <bool kPad>
__global__ __launch_bounds__(1024) void pool_raster_kernel(const uint4* __restrict__ src,
                                                           const int32_t* __restrict__ perm, int H, int C,
                                                           int n_prefix, int64_t n_video, int64_t n_ras, PoolOut po) {
    constexpr int U = 8;  // loads in flight per thread
    __shared__ int64_t tok[kTile];
    __shared__ int real;
    const int b = blockIdx.y;
    const int64_t vt = blockIdx.x, p0 = n_prefix + vt * kTile;
    if (threadIdx.x < kTile) {
        const int64_t t = slot_token<kPad>(perm, b, n_video, n_prefix, n_ras, p0 + threadIdx.x);
        tok[threadIdx.x] = t;
        const int nr = __popcll(__ballot(t >= 0));
        if (threadIdx.x == 0) real = nr;
    }
    __syncthreads();
    const int nvt = (int)(n_video / kTile);
    const double count = kPad ? (double)real : (double)kTile;
    for (int pr = threadIdx.x; pr < H * C; pr += blockDim.x) {
        const int h = pr / C, c = pr % C;
        double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int pl0 = 0; pl0 < kTile; pl0 += U) {
            uint4 x[U];
#pragma unroll
            for (int e = 0; e < U; ++e) x[e] = src_chunk<false, kPad>(src, b, h, H, C, c, tok[pl0 + e], n_ras, 0);
#pragma unroll
            for (int e = 0; e < U; ++e) {
                acc[0] += (double)__uint_as_float(x[e].x << 16);
                acc[1] += (double)__uint_as_float(x[e].x & 0xffff0000u);
                acc[2] += (double)__uint_as_float(x[e].y << 16);
                acc[3] += (double)__uint_as_float(x[e].y & 0xffff0000u);
                acc[4] += (double)__uint_as_float(x[e].z << 16);
                acc[5] += (double)__uint_as_float(x[e].z & 0xffff0000u);
                acc[6] += (double)__uint_as_float(x[e].w << 16);
                acc[7] += (double)__uint_as_float(x[e].w & 0xffff0000u);
            }
        }
        float m[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) m[e] = (float)(acc[e] / count);
        const int64_t bh = (int64_t)b * H + h;
        float sq = store_pooled8(po, bh, nvt, 8 * C, vt, c, m);
        for (int o = 1; o < C; o <<= 1) sq += __shfl_xor(sq, o);
        if (c == 0) po.norm[bh * nvt + vt] = sqrtf(sq);
    }
}

}  // namespace

hipError_t launch_gather_pool(bool kfrag, const uint16_t* src, uint16_t* dst, const int32_t* perm, int B, int H,
                              int D, int n_prefix, int64_t n_video, const PoolOut& po, hipStream_t s,
                              int64_t n_raster_video) {
    const int64_t n_tot = n_prefix + n_video;
    const int64_t n_ras = n_prefix + (n_raster_video < 0 ? n_video : n_raster_video);
    if (B == 0 || H == 0 || n_tot == 0) return hipSuccess;
    const dim3 grid((unsigned)(n_tot / kTile), (unsigned)B);
    const int C = D / 8;
    const bool pad = n_ras != n_tot;
    if (kfrag) {
        auto kernel = pad ? gather_kf_pool_kernel<true> : gather_kf_pool_kernel<false>;
        hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, (const uint4*)src, (uint4*)dst, perm, H, C, n_prefix,
                           n_video, n_tot, n_ras, po);
        return hipGetLastError();
    }
    auto kernel = pad ? gather_pool_kernel<true> : gather_pool_kernel<false>;
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, (const uint4*)src, (uint4*)dst, perm, H, C, n_prefix,
                       n_video, n_tot, n_ras, po);
    return hipGetLastError();
}

hipError_t launch_gather_kf_tiled(const uint16_t* src, uint16_t* dst_kf, uint16_t* dst_t, const int32_t* perm, int B,
                                  int H, int D, int n_prefix, int64_t n_video, hipStream_t s, int64_t n_raster_video,
                                  const DeltaOut* dl) {
    const int64_t n_tot = n_prefix + n_video;
    const int64_t n_ras = n_prefix + (n_raster_video < 0 ? n_video : n_raster_video);
    if (B == 0 || H == 0 || n_tot == 0) return hipSuccess;
    const dim3 grid((unsigned)(n_tot / kTile), (unsigned)B);
    const bool pad = n_ras != n_tot;
    const DeltaOut d = dl ? *dl : DeltaOut{};
    auto kernel = dl ? (pad ? gather_kf_tiled_kernel<true, true> : gather_kf_tiled_kernel<false, true>)
                     : (pad ? gather_kf_tiled_kernel<true, false> : gather_kf_tiled_kernel<false, false>);
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, (const uint4*)src, (uint4*)dst_kf, (uint4*)dst_t, perm, H, D / 8,
                       n_prefix, n_video, n_tot, n_ras, d);
    return hipGetLastError();
}

hipError_t launch_gather_kf_vf(const uint16_t* src, uint16_t* dst_kf, uint16_t* dst_vf, const int32_t* perm, int B,
                               int H, int D, int n_prefix, int64_t n_video, hipStream_t s, int64_t n_raster_video) {
    const int64_t n_tot = n_prefix + n_video;
    const int64_t n_ras = n_prefix + (n_raster_video < 0 ? n_video : n_raster_video);
    if (B == 0 || H == 0 || n_tot == 0) return hipSuccess;
    const dim3 grid((unsigned)(n_tot / kTile), (unsigned)B);
    auto kernel = n_ras != n_tot ? gather_kf_vf_kernel<true> : gather_kf_vf_kernel<false>;
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, (const uint4*)src, (uint4*)dst_kf, (uint4*)dst_vf, perm, H,
                       D / 8, n_prefix, n_video, n_tot, n_ras);
    return hipGetLastError();
}

hipError_t launch_pool_raster(const uint16_t* src, const int32_t* perm, int B, int H, int D, int n_prefix,
                              int64_t n_video, const PoolOut& po, hipStream_t s, int64_t n_raster_video) {
    const int64_t n_tot = n_prefix + n_video;
    const int64_t n_ras = n_prefix + (n_raster_video < 0 ? n_video : n_raster_video);
    if (B == 0 || H == 0 || n_video == 0) return hipSuccess;
    const dim3 grid((unsigned)(n_video / kTile), (unsigned)B);
    const int pairs = H * (D / 8);
    const int threads = pairs >= 1024 ? 1024 : (pairs + 63) / 64 * 64;
    auto kernel = n_ras != n_tot ? pool_raster_kernel<true> : pool_raster_kernel<false>;
    hipLaunchKernelGGL(kernel, grid, dim3(threads), 0, s, (const uint4*)src, perm, H, D / 8, n_prefix, n_video,
                       n_ras, po);
    return hipGetLastError();
}

hipError_t launch_tiled_to_frag(bool kfrag, const uint16_t* src, uint16_t* dst, int B, int H, int D, int64_t n_tot,
                                hipStream_t s) {
    if (B == 0 || H == 0 || n_tot == 0) return hipSuccess;
    const dim3 grid((unsigned)(n_tot / kTile), (unsigned)B);
    if (kfrag)
        hipLaunchKernelGGL((gather_kf_kernel<false, true>), grid, dim3(256), 0, s, (const uint4*)src, (uint4*)dst,
                           (const int32_t*)nullptr, H, D / 8, 0, n_tot, n_tot, n_tot);
    else
        hipLaunchKernelGGL((gather_vf_kernel<false, true>), grid, dim3(256), 0, s, (const uint4*)src, (uint4*)dst,
                           (const int32_t*)nullptr, H, D / 8, 0, n_tot, n_tot, n_tot);
    return hipGetLastError();
}

hipError_t launch_gather_kf(const uint16_t* src, uint16_t* dst, const int32_t* perm, int B, int H, int D,
                            int n_prefix, int64_t n_video, hipStream_t s, int64_t n_raster_video) {
    const int64_t n_tot = n_prefix + n_video;
    const int64_t n_ras = n_prefix + (n_raster_video < 0 ? n_video : n_raster_video);
    if (B == 0 || H == 0 || n_tot == 0) return hipSuccess;
    const dim3 grid((unsigned)(n_tot / kTile), (unsigned)B);
    if (n_ras != n_tot)  // a ragged grid: padding slots
        hipLaunchKernelGGL(gather_kf_kernel<true>, grid, dim3(256), 0, s, (const uint4*)src, (uint4*)dst, perm, H,
                           D / 8, n_prefix, n_video, n_tot, n_ras);
    else
        hipLaunchKernelGGL(gather_kf_kernel<false>, grid, dim3(256), 0, s, (const uint4*)src, (uint4*)dst, perm, H,
                           D / 8, n_prefix, n_video, n_tot, n_ras);
    return hipGetLastError();
}

hipError_t launch_gather_vf(const uint16_t* src, uint16_t* dst, const int32_t* perm, int B, int H, int D,
                            int n_prefix, int64_t n_video, hipStream_t s, int64_t n_raster_video) {
    const int64_t n_tot = n_prefix + n_video;
    const int64_t n_ras = n_prefix + (n_raster_video < 0 ? n_video : n_raster_video);
    if (B == 0 || H == 0 || n_tot == 0) return hipSuccess;
    const dim3 grid((unsigned)(n_tot / kTile), (unsigned)B);
    if (n_ras != n_tot)
        hipLaunchKernelGGL(gather_vf_kernel<true>, grid, dim3(256), 0, s, (const uint4*)src, (uint4*)dst, perm, H,
                           D / 8, n_prefix, n_video, n_tot, n_ras);
    else
        hipLaunchKernelGGL(gather_vf_kernel<false>, grid, dim3(256), 0, s, (const uint4*)src, (uint4*)dst, perm, H,
                           D / 8, n_prefix, n_video, n_tot, n_ras);
    return hipGetLastError();
}

hipError_t launch_perm_static(int B, int T, int Hg, int W, int tt, int th, int tw, int32_t* perm,
                              hipStream_t s) {
    const int64_t n_video = (int64_t)((T + tt - 1) / tt * tt) * ((Hg + th - 1) / th * th) * ((W + tw - 1) / tw * tw);
    const int64_t total = n_video * B;
    if (total == 0) return hipSuccess;
    const int threads = 256;
    const int64_t want = (total + threads - 1) / threads;
    const int blocks = (int)(want < 65536 ? want : 65536);
    hipLaunchKernelGGL(perm_static_kernel, dim3(blocks), dim3(threads), 0, s, T, Hg, W, tt, th, tw, n_video, B,
                       perm);
    return hipGetLastError();
}

hipError_t launch_permute_copy(bool to_raster, const uint16_t* src, uint16_t* dst, const int32_t* perm, int B,
                               int H, int D, int n_prefix, int64_t n_video, hipStream_t s, int64_t n_raster_video) {
    const int64_t n_tot = n_prefix + n_video;
    const int64_t n_ras = n_prefix + (n_raster_video < 0 ? n_video : n_raster_video);
    if (B == 0 || H == 0 || n_tot == 0) return hipSuccess;
    const dim3 grid((unsigned)(n_tot / kTile), (unsigned)B);
    const int C = D / 8;
    const bool pad = n_ras != n_tot;
    auto kernel = to_raster ? (pad ? permute_copy_kernel<true, true> : permute_copy_kernel<true, false>)
                            : (pad ? permute_copy_kernel<false, true> : permute_copy_kernel<false, false>);
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, (const uint4*)src, (uint4*)dst, perm, H, C, n_prefix, n_video,
                       n_tot, n_ras);
    return hipGetLastError();
}

}  // namespace bsa
