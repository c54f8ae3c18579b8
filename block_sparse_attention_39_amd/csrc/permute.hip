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

// raster token of tiled slot p (prefix first), or -1 for a padding slot
__device__ inline int64_t slot_token(const int32_t* __restrict__ perm, int b, int64_t n_video, int n_prefix,
                                     int64_t p) {
    if (p < n_prefix) return p;
    const int32_t v = perm[(int64_t)b * n_video + (p - n_prefix)];
    return v < 0 ? -1 : n_prefix + v;
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
    if (threadIdx.x < kTile) tok[threadIdx.x] = slot_token(perm, b, n_video, n_prefix, p0 + threadIdx.x);
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

// Raster K -> K-fragment layout [B][H][tile][kh][s][lane][8]: chunk
// (kh, s, lane) of a tile holds channels 16 s + 8 (lane / 32) .. +7 of the
// tile's token 32 kh + swap23(lane % 32) (bits 2 and 3 exchanged), i.e. the
// A operand of v_mfma_f32_32x32x16_bf16 for the S^T = K Q^T products of the
// attention kernel.  One block per (batch, tile); work item = (head, chunk),
// chunk fastest, so a wave writes 1 KB contiguous and reads 32-byte runs of
// the tile's raster rows.
__device__ inline int swap23(int m) { return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <bool kPad>
__global__ __launch_bounds__(256) void gather_kf_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        const int32_t* __restrict__ perm, int H, int C,
                                                        int n_prefix, int64_t n_video, int64_t n_tot,
                                                        int64_t n_ras) {
    __shared__ int64_t tok[kTile];
    const int b = blockIdx.y;
    const int64_t tile = blockIdx.x;
    const int64_t p0 = tile * kTile;
    const int64_t n_tiles = n_tot / kTile;
    if (threadIdx.x < kTile) tok[threadIdx.x] = slot_token(perm, b, n_video, n_prefix, p0 + threadIdx.x);
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
        const int64_t t = tok[r];
        dst[(((int64_t)b * H + h) * n_tiles + tile) * per_head + q] =
            zero_if_padding<kPad>(src[(((int64_t)b * n_ras + row_or_zero<kPad>(t)) * H + h) * C + cc], t);
    }
}

// Raster V -> V-fragment layout [B][H][tile][kh][i][c][lane][8]: chunk
// (kh, i, c, lane) of a tile holds channel 32 i + lane % 32 of the tile's
// tokens 32 kh + 16 c + 8 (lane / 32) .. +7, i.e. the A operand of the
// O^T = V^T P^T products.  One block per (batch, tile); work item = (head,
// group of 8 tokens, 8-channel chunk): a thread reads 8 token rows of 16 bytes
// (256-byte head rows across a wave), transposes the 8 x 8 block of bf16
// values in registers and writes 8 chunks for 8 consecutive lanes (128 bytes
// contiguous).
__device__ inline uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ inline uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }
__device__ inline uint32_t word_of(const uint4& v, int w) { return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w; }

template <bool kPad>
__global__ __launch_bounds__(256) void gather_vf_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        const int32_t* __restrict__ perm, int H, int C,
                                                        int n_prefix, int64_t n_video, int64_t n_tot,
                                                        int64_t n_ras) {
    __shared__ int64_t tok[kTile];
    const int b = blockIdx.y;
    const int64_t tile = blockIdx.x;
    const int64_t p0 = tile * kTile;
    const int64_t n_tiles = n_tot / kTile;
    if (threadIdx.x < kTile) tok[threadIdx.x] = slot_token(perm, b, n_video, n_prefix, p0 + threadIdx.x);
    __syncthreads();
    const int OD = C / 4;  // 32-channel blocks
    const int items = H * 8 * C;
    for (int it = threadIdx.x; it < items; it += 256) {
        const int dc = it % C;
        const int g = (it / C) % 8;
        const int h = it / (8 * C);
        uint4 r0, r1, r2, r3, r4, r5, r6, r7;
        auto row = [&](int i) {
            const int64_t t = tok[8 * g + i];
            return zero_if_padding<kPad>(src[(((int64_t)b * n_ras + row_or_zero<kPad>(t)) * H + h) * C + dc], t);
        };
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

}  // namespace

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
