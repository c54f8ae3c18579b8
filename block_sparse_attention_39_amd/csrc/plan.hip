// Tile selection: pooling, pooled scores and per-row top-k.
//
// "Prism / Kandinsky 6 speed ablation" page, section "같은 계산량 안에서 볼 곳을
// 고르는 Prism": a tile's relevance is judged from the mean of its 64 tokens, and
// each query tile keeps the (1 - sparsity) best key tiles.  The score is the dot
// product of the pooled query and key vectors; equal scores go to the lower key
// tile number; kept lists are written in ascending order.
//
// pool   : HBM-bound read of Q (tiled) and K (K-fragment layout) once; one
//          wave per tile, 16-byte loads, double accumulation (exact for bf16
//          inputs), one rounding to float, cross-lane reduction with shuffles.
// scores : float GEMM per (batch, head) of the pooled vectors, 64x64 output
//          blocks through LDS.
// topk   : one block per row; 8-bit radix select on the order-preserving
//          integer image of the float scores (4 passes, LDS histogram), then an
//          index-ordered compaction that takes every score above the threshold
//          and the lowest-numbered ties.
#include "bsa_kernels.h"

namespace bsa {
namespace {

__device__ inline float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// ---------------------------------------------------------------- pooling --
// Block = 4 waves, one tile per wave; the first B*H*nvt tiles are Q's (tiled
// layout), the next ones K's (K-fragment layout).  Sums are exact in double
// (64 bf16 values), so the order of summation does not matter.
//  Q: lane l reads chunk c = l % C of rows r = l / C + i * (64 / C); the wave
//     then folds the 64 / C lanes that share c.
//  K: chunk (kh, s, lane) holds channels 16 s + 8 (lane / 32) .. +7 of token
//     32 kh + swap23(lane % 32); lane l takes channel group (s, hf) =
//     (l / LPG / 2, l / LPG % 2) and 64 / LPG of the tile's tokens, then the
//     LPG lanes of a group fold their sums.
__device__ inline void acc8(double (&acc)[8], const uint4& x) {
    acc[0] += (double)bf_lo(x.x);
    acc[1] += (double)bf_hi(x.x);
    acc[2] += (double)bf_lo(x.y);
    acc[3] += (double)bf_hi(x.y);
    acc[4] += (double)bf_lo(x.z);
    acc[5] += (double)bf_hi(x.z);
    acc[6] += (double)bf_lo(x.w);
    acc[7] += (double)bf_hi(x.w);
}

// the exact sums divided by the tile's token count, rounded once to float
__device__ inline void store_mean8(float* dst, const double (&acc)[8], double count) {
    float4 lo, hi;
    lo.x = (float)(acc[0] / count);
    lo.y = (float)(acc[1] / count);
    lo.z = (float)(acc[2] / count);
    lo.w = (float)(acc[3] / count);
    hi.x = (float)(acc[4] / count);
    hi.y = (float)(acc[5] / count);
    hi.z = (float)(acc[6] / count);
    hi.w = (float)(acc[7] / count);
    ((float4*)dst)[0] = lo;
    ((float4*)dst)[1] = hi;
}

// real tokens of video tile i (64 without padding)
__device__ inline int tile_count(const PadGeo& g, int64_t i) {
    if (g.T == 0) return kTile;
    const int wi = (int)(i % g.Tw), hi = (int)((i / g.Tw) % g.Th), ti = (int)(i / ((int64_t)g.Tw * g.Th));
    return min(g.tt, g.T - ti * g.tt) * min(g.th, g.Hg - hi * g.th) * min(g.tw, g.W - wi * g.tw);
}

template <int D>
__global__ __launch_bounds__(256) void pool_kernel(const uint4* __restrict__ q, const uint4* __restrict__ k,
                                                   float* __restrict__ qbar, float* __restrict__ kbar, int BH,
                                                   int n_prefix, int nvt, PadGeo pad) {
    constexpr int C = D / 8;         // 16-byte chunks per row
    constexpr int SD = D / 16;       // K-fragment steps
    constexpr int LPG = 64 / (2 * SD);  // lanes per channel group (K)
    constexpr int TPL = kTile / LPG;    // tokens per lane (K)
    const int lane = threadIdx.x & 63;
    const int64_t tiles_per_tensor = (int64_t)BH * nvt;
    const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (g >= 2 * tiles_per_tensor) return;
    const bool is_k = g >= tiles_per_tensor;
    const int64_t t = is_k ? g - tiles_per_tensor : g;
    const int64_t bh = t / nvt, i = t % nvt;
    const int64_t n_tot = n_prefix + (int64_t)nvt * kTile;
    const uint4* src = (is_k ? k : q) + ((bh * n_tot + n_prefix + i * kTile) * C);
    const double count = (double)tile_count(pad, i);  // padding tokens are zeros in the tiled tensors
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (!is_k) {
        constexpr int RPI = 64 / C;  // rows covered by one wave-wide load
        const int c = lane % C, r0 = lane / C;
        uint4 x[kTile / RPI];  // every load in flight before the first sum
#pragma unroll
        for (int it = 0; it < kTile / RPI; ++it) x[it] = src[(r0 + it * RPI) * C + c];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int it = 0; it < kTile / RPI; ++it) acc8(acc, x[it]);
#pragma unroll
        for (int o = C; o < 64; o <<= 1)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o);
        if (lane < C) store_mean8(qbar + t * D + 8 * lane, acc, count);
    } else {
        const int grp = lane / LPG, part = lane % LPG;
        const int s = grp >> 1, hf = grp & 1;
        uint4 x[TPL];
#pragma unroll
        for (int u = 0; u < TPL; ++u) {
            const int tok = part * TPL + u;  // 32 kh + m
            const int kh = tok >> 5, m = tok & 31;
            x[u] = src[(kh * SD + s) * 64 + 32 * hf + m];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < TPL; ++u) acc8(acc, x[u]);
#pragma unroll
        for (int o = 1; o < LPG; o <<= 1)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o);
        if (part == 0) store_mean8(kbar + t * D + 16 * s + 8 * hf, acc, count);
    }
}

// ----------------------------------------------------------------- scores --
// S[bh][i][j] = sum_d A[bh][i][d] B[bh][j][d], float.  Block = 256 threads,
// 64x64 output block; thread (ty, tx) computes rows 4ty..4ty+3, cols 4tx..4tx+3.
// Operands are staged transposed in LDS ([d][row]) in slabs of 32 channels.
__global__ __launch_bounds__(256) void scores_kernel(const float* __restrict__ A, const float* __restrict__ Bm,
                                                     float* __restrict__ S, int n, int D) {
    constexpr int KS = 32;
    __shared__ float4 As[KS][16 + 1];
    __shared__ float4 Bs[KS][16 + 1];
    const int bh = blockIdx.z;
    const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    const float* Ab = A + (int64_t)bh * n * D;
    const float* Bb = Bm + (int64_t)bh * n * D;
    float acc[4][4] = {};
    for (int d0 = 0; d0 < D; d0 += KS) {
        // load 64 rows x 32 channels of A and B: 2048 floats each, 8 per thread
        for (int e = threadIdx.x; e < 64 * KS; e += 256) {
            const int row = e / KS, dd = e % KS;
            const float a = (i0 + row < n) ? Ab[(int64_t)(i0 + row) * D + d0 + dd] : 0.f;
            const float b = (j0 + row < n) ? Bb[(int64_t)(j0 + row) * D + d0 + dd] : 0.f;
            reinterpret_cast<float*>(&As[dd][row >> 2])[row & 3] = a;
            reinterpret_cast<float*>(&Bs[dd][row >> 2])[row & 3] = b;
        }
        __syncthreads();
#pragma unroll 8
        for (int dd = 0; dd < KS; ++dd) {
            const float4 a = As[dd][ty];
            const float4 b = Bs[dd][tx];
            const float av[4] = {a.x, a.y, a.z, a.w};
            const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(av[u], bv[v], acc[u][v]);
        }
        __syncthreads();
    }
    float* Sb = S + (int64_t)bh * n * n;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = i0 + 4 * ty + u;
        if (i >= n) continue;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int j = j0 + 4 * tx + v;
            if (j < n) Sb[(int64_t)i * n + j] = acc[u][v];
        }
    }
}

// ------------------------------------------------------------------ top-k --
// Order-preserving unsigned image of a float (larger float -> larger key);
// -0 is folded onto +0 so that equal scores give equal keys.
__device__ inline uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive scan over a block of 256 threads (4 waves); returns the inclusive
// prefix and writes the block total to *total.
__device__ inline int block_scan_256(int x, int* wsum, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int v = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(v, o);
        if (lane >= o) v += y;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
    return v + before;
}

// One block per row of scores.  Fixed keep: k per row, written at row * k.
// Variable keep (row_ptr not null): row r0 + row keeps row_ptr[r + 1] -
// row_ptr[r] tiles, written at row_ptr[r].
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ S, int32_t* __restrict__ idx, int n,
                                                   int k_fixed, const int64_t* __restrict__ row_ptr, int64_t r0) {
    extern __shared__ uint32_t keys[];  // [n]
    __shared__ int hist[256];
    __shared__ int wsum[4];
    __shared__ int sel_digit, sel_above;
    const int64_t row = blockIdx.x;
    const float* s = S + row * n;
    int k = k_fixed;
    int32_t* out = idx + row * k_fixed;
    if (row_ptr) {
        const int64_t beg = row_ptr[r0 + row];
        k = (int)(row_ptr[r0 + row + 1] - beg);
        out = idx + beg;
    }
    for (int j = threadIdx.x; j < n; j += 256) keys[j] = order_key(s[j]);
    uint32_t prefix = 0, mask = 0;
    int need = k;  // how many of the keys matching `prefix` are still to take
    for (int shift = 24; shift >= 0; shift -= 8) {
        hist[threadIdx.x] = 0;
        __syncthreads();
        for (int j = threadIdx.x; j < n; j += 256) {
            const uint32_t key = keys[j];
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
        }
        __syncthreads();
        // counts from the top digit down: thread t holds digit 255 - t
        const int cnt = hist[255 - threadIdx.x];
        int tot;
        const int incl = block_scan_256(cnt, wsum, &tot);
        const int excl = incl - cnt;
        if (excl < need && incl >= need) {
            sel_digit = 255 - threadIdx.x;
            sel_above = excl;
        }
        __syncthreads();
        need -= sel_above;
        prefix |= (uint32_t)sel_digit << shift;
        mask |= 255u << shift;
        __syncthreads();
    }
    // prefix is now the key of the k-th largest score; `need` of the keys equal
    // to it are taken, lowest index first.  Each thread owns a contiguous run
    // of indices, so two block scans (ties before the run, selected entries
    // before the run) place its selections in ascending order.
    const uint32_t thr = prefix;
    const int per = (n + 255) / 256;
    const int j_lo = min((int)threadIdx.x * per, n), j_hi = min(j_lo + per, n);
    int my_above = 0, my_ties = 0;
    for (int j = j_lo; j < j_hi; ++j) {
        const uint32_t key = keys[j];
        my_above += key > thr;
        my_ties += key == thr;
    }
    int tot;
    const int ties_before = block_scan_256(my_ties, wsum, &tot) - my_ties;
    const int my_take = my_above + min(max(need - ties_before, 0), my_ties);
    int pos = block_scan_256(my_take, wsum, &tot) - my_take;
    int tie_rank = ties_before;
    for (int j = j_lo; j < j_hi; ++j) {
        const uint32_t key = keys[j];
        const bool tie = key == thr;
        if (key > thr || (tie && tie_rank < need)) out[pos++] = j;
        tie_rank += tie;
    }
}

// Row pointers from per-row lengths: row_ptr is the exclusive prefix sum of
// len(r) over rows 0..rows-1.  One block of 1,024 threads: each sums a
// contiguous run of rows, the runs are scanned in LDS, then written.
template <typename Len>
__device__ void rowptr_scan(int64_t rows, Len len, int64_t* __restrict__ row_ptr) {
    __shared__ int64_t part[1024];
    const int64_t per = (rows + 1023) / 1024;
    const int64_t r_lo = min((int64_t)threadIdx.x * per, rows), r_hi = min(r_lo + per, rows);
    int64_t sum = 0;
    for (int64_t r = r_lo; r < r_hi; ++r) sum += len(r);
    part[threadIdx.x] = sum;
    __syncthreads();
    // inclusive scan of the 1024 partial sums (Hillis-Steele in LDS)
    for (int o = 1; o < 1024; o <<= 1) {
        const int64_t add = threadIdx.x >= (unsigned)o ? part[threadIdx.x - o] : 0;
        __syncthreads();
        part[threadIdx.x] += add;
        __syncthreads();
    }
    int64_t run = part[threadIdx.x] - sum;
    for (int64_t r = r_lo; r < r_hi; ++r) {
        row_ptr[r] = run;
        run += len(r);
    }
    if (threadIdx.x == 1023) row_ptr[rows] = part[1023];
}

// Variable keep: row (bh, i) keeps keep_rows[bh][i] clamped to [1, keep_h[h]]
// tiles (keep_h[h] without keep_rows).
__global__ __launch_bounds__(1024) void csr_rowptr_kernel(CsrKeep kh, const int32_t* __restrict__ keep_rows,
                                                          int BH, int H, int nvt, int64_t* __restrict__ row_ptr) {
    auto len = [&](int64_t r) -> int64_t {
        const int cap = kh.k[(int)((r / nvt) % H)];
        return keep_rows ? (int64_t)min(max(keep_rows[r], 1), cap) : (int64_t)cap;
    };
    rowptr_scan((int64_t)BH * nvt, len, row_ptr);
}

// Structured lists: the box of key tiles a query tile keeps, in tile-grid
// coordinates (raster tile order: tile (t, h, w) is number (t*Th + h)*Tw + w).
// A spatial head keeps every tile within rt tile-frames of the query tile's;
// a temporal head keeps, at every time, the tiles within rs in h and in w of
// the query tile's position.
struct TileBox {
    int t0, t1, h0, h1, w0, w1;  // inclusive
    __device__ int64_t count() const { return (int64_t)(t1 - t0 + 1) * (h1 - h0 + 1) * (w1 - w0 + 1); }
};
__device__ inline TileBox struct_box(const StructRule& sr, int kind, int i) {
    const int wi = i % sr.Tw, hi = (i / sr.Tw) % sr.Th, ti = i / (sr.Tw * sr.Th);
    TileBox b;
    if (kind == BSA_MASK_SPATIAL) {
        b = {max(ti - sr.rt, 0), min(ti + sr.rt, sr.Tt - 1), 0, sr.Th - 1, 0, sr.Tw - 1};
    } else {
        b = {0, sr.Tt - 1, max(hi - sr.rs, 0), min(hi + sr.rs, sr.Th - 1), max(wi - sr.rs, 0),
             min(wi + sr.rs, sr.Tw - 1)};
    }
    return b;
}

__global__ __launch_bounds__(1024) void struct_rowptr_kernel(StructRule sr, int BH, int H,
                                                             int64_t* __restrict__ row_ptr) {
    const int nvt = sr.Tt * sr.Th * sr.Tw;
    auto len = [&](int64_t r) -> int64_t {
        return struct_box(sr, sr.kind[(int)((r / nvt) % H)], (int)(r % nvt)).count();
    };
    rowptr_scan((int64_t)BH * nvt, len, row_ptr);
}

// One 64-thread block per row writes the row's box of tiles, ascending.
__global__ __launch_bounds__(64) void struct_fill_kernel(StructRule sr, int H, const int64_t* __restrict__ row_ptr,
                                                         int32_t* __restrict__ col) {
    const int nvt = sr.Tt * sr.Th * sr.Tw;
    const int64_t r = blockIdx.x;
    const TileBox b = struct_box(sr, sr.kind[(int)((r / nvt) % H)], (int)(r % nvt));
    const int nh = b.h1 - b.h0 + 1, nw = b.w1 - b.w0 + 1;
    const int64_t n = b.count(), beg = row_ptr[r];
    for (int64_t e = threadIdx.x; e < n; e += 64) {
        const int w = b.w0 + (int)(e % nw), h = b.h0 + (int)((e / nw) % nh), t = b.t0 + (int)(e / ((int64_t)nw * nh));
        col[beg + e] = (t * sr.Th + h) * sr.Tw + w;
    }
}

}  // namespace

hipError_t launch_csr_rowptr(const CsrKeep& kh, const int32_t* keep_rows, int BH, int H, int nvt, int64_t* row_ptr,
                             hipStream_t s) {
    hipLaunchKernelGGL(csr_rowptr_kernel, dim3(1), dim3(1024), 0, s, kh, keep_rows, BH, H, nvt, row_ptr);
    return hipGetLastError();
}

hipError_t launch_structured(const StructRule& sr, int BH, int H, int64_t* row_ptr, int32_t* col, hipStream_t s) {
    const int64_t rows = (int64_t)BH * sr.Tt * sr.Th * sr.Tw;
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(struct_rowptr_kernel, dim3(1), dim3(1024), 0, s, sr, BH, H, row_ptr);
    hipLaunchKernelGGL(struct_fill_kernel, dim3((unsigned)rows), dim3(64), 0, s, sr, H, (const int64_t*)row_ptr, col);
    return hipGetLastError();
}

hipError_t launch_pool(const uint16_t* q_tiled, const uint16_t* k_frag, float* qbar, float* kbar, int BH,
                       int n_prefix, int nvt, int D, hipStream_t s, const PadGeo& pad) {
    const int64_t tiles = 2LL * BH * nvt;
    if (tiles == 0) return hipSuccess;
    const dim3 grid((unsigned)((tiles + 3) / 4));
    if (D == 128)
        hipLaunchKernelGGL(pool_kernel<128>, grid, dim3(256), 0, s, (const uint4*)q_tiled, (const uint4*)k_frag,
                           qbar, kbar, BH, n_prefix, nvt, pad);
    else
        hipLaunchKernelGGL(pool_kernel<64>, grid, dim3(256), 0, s, (const uint4*)q_tiled, (const uint4*)k_frag,
                           qbar, kbar, BH, n_prefix, nvt, pad);
    return hipGetLastError();
}

hipError_t launch_scores(const float* qbar, const float* kbar, float* scores, int BH, int n, int D,
                         hipStream_t s) {
    if (BH == 0 || n == 0) return hipSuccess;
    const dim3 grid((unsigned)((n + 63) / 64), (unsigned)((n + 63) / 64), (unsigned)BH);
    hipLaunchKernelGGL(scores_kernel, grid, dim3(256), 0, s, qbar, kbar, scores, n, D);
    return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int32_t* idx, int rows, int n, int k, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)rows), dim3(256), (size_t)n * sizeof(uint32_t), s, scores, idx,
                       n, k, (const int64_t*)nullptr, (int64_t)0);
    return hipGetLastError();
}

hipError_t launch_topk_csr(const float* scores, int32_t* col_idx, const int64_t* row_ptr, int64_t row0, int rows,
                           int n, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)rows), dim3(256), (size_t)n * sizeof(uint32_t), s, scores,
                       col_idx, n, 0, row_ptr, row0);
    return hipGetLastError();
}

}  // namespace bsa
