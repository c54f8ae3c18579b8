// Sparse flash-style attention forward over the kept tiles, bf16 MFMA on gfx950.
//
// What is computed ("Prism / Kandinsky 6 speed ablation" page, section on
// Prism's block-sparse attention; "Sparse VideoGen TPU 최적화 ..." page, section
// "이론적 sparsity와 물리적 sparsity의 차이"; "RTX 4090에서 5초 영상 72초: Ref2VA
// VSA" page, section "조건 토큰은 왜 다르게 다루나"): every video query tile
// attends exactly to the tokens of its kept key tiles plus the whole dense
// prefix; prefix query tiles attend to every token.  Skipped tiles are never
// touched and kept tiles are computed whole, with no element mask.
//
// One query tile (64 tokens) is processed by one block of 4 waves:
//   wave w = (qh, kh): queries 32*qh .. +31 of the tile, keys 32*kh .. +31 of
//   every key tile.  Each wave keeps its own online softmax for its key half;
//   the two halves are merged once at the end.
//   S^T = K Q^T and O^T = V^T P^T with v_mfma_f32_32x32x16_bf16, so that in
//   every accumulator a lane holds a single query (lane % 32): the softmax row
//   state is per lane, the row max needs one cross-half exchange
//   (v_permlane32_swap), and rescaling O is a per-lane multiply.
//   The K rows feeding S^T are read in an order that swaps the middle two
//   4-row groups of every 16; the S^T accumulator then hands each lane-half the
//   scores of 8 consecutive keys, which is exactly the P^T operand layout, so
//   V^T (stored transposed per tile by the gather) is read in natural order.
//   K and V^T tiles are 16 KB contiguous copies; they stream through two LDS
//   buffers: while the MFMAs work on tile j, the global loads of tile j+1 are
//   in flight in registers; they land in the other buffer and one barrier per
//   tile hands it over.  LDS rows are padded by 16 bytes (no bank conflicts for
//   the 16-row MFMA operand reads), so every LDS address is a per-lane base
//   plus a compile-time offset; the loop is unrolled by two for the buffers.
//   All K and V^T operand reads of a tile are issued before its first MFMA.
//   The softmax works in base 2 (scale * log2 e folded into one FMA) and
//   rescales the accumulators only when a row maximum grows by more than
//   2^8, which is exact (the same reference maximum is used for O and for the
//   normaliser).  The normaliser adds up the same bf16-rounded weights that
//   enter the MFMA (v_dot2 with ones), so each output is a convex combination
//   of V rows.
//
// Two launch forms:
//   * plain: one block per query tile (prefix query tiles first: they are the
//     long, dense ones);
//   * grouped (video query tiles, when a workspace is given): a persistent grid
//     of 8 groups of blocks, block b in group b % 8 (the XCD that the hardware
//     dispatches it to, so a group shares one L2).  A group works through 64
//     consecutive query tiles at a time, and its blocks sweep the key tiles in
//     ascending order in near lock-step: each block publishes the 64-tile key
//     chunk it is loading and may run at most one chunk ahead of the slowest
//     block of its group (two chunks of K and V are 4 MB, the size of an XCD's
//     L2).  Every key tile is then fetched into the group's L2
//     once and read there by the ~quarter of the group's blocks that kept it,
//     instead of once per block.  The waits are bounded (a block never waits
//     more than a few tens of microseconds per chunk), so the kernel finishes
//     even if blocks of a group are not resident together; the fences only
//     shape the schedule, results do not depend on them.
#include <climits>

#include "bsa_kernels.h"

namespace bsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16-byte chunk (native vector, not HIP's uint4)

constexpr float kRescaleLog2 = 8.0f;
// s_waitcnt immediate: vmcnt(0), expcnt and lgkmcnt left alone (gfx9 encoding)
constexpr int kWaitVm0 = 0x0F70;
constexpr int kGroups = 8;        // block groups of the grouped launch (one per XCD)
constexpr int kMaxGroupSize = 64; // blocks per group the fence can track (one per lane)
#ifndef BSA_FENCE_CHUNK
#define BSA_FENCE_CHUNK 64
#endif
constexpr int kChunk = BSA_FENCE_CHUNK;  // key tiles per fence chunk
constexpr int kMaxSpin = 400;            // bounded wait per fence (x s_sleep 2)

template <int D>
struct Cfg {
    static constexpr int C = D / 8;                // 16-byte chunks in a K row
    static constexpr int KB = kTile * D * 2;       // K tile in LDS (16 KB for D = 128)
    static constexpr int VB = D * kTile * 2;       // V^T tile in LDS
    static constexpr int BUF = KB + VB;            // one LDS stage
    static constexpr int NK = kTile * C / 256;     // DMA instructions per wave for a K tile (and for V^T)
    static constexpr int SD = D / 16;              // MFMA steps over d for S^T
    static constexpr int OD = D / 32;              // 32-row d blocks of O^T
};

// LDS layout of a stage: the K tile as 64 rows of D bf16 and the V^T tile as D
// rows of 64 bf16, unpadded, with the 16-byte chunks of every row permuted by
// an XOR so that the 16 rows read by half a wave hit 16 different bank groups:
//   K row r (C chunks):    physical chunk = c ^ kswz(r)
//   V^T row d (8 chunks):  physical chunk = c ^ ((d >> 1) & 7)
template <int D>
__device__ inline int kswz(int r) {
    return Cfg<D>::C == 16 ? (r & 15) : ((r >> 1) & 7);
}
__device__ inline int vswz(int d) { return (d >> 1) & 7; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Copy one key tile (K: 64 x D, V^T: D x 64, both contiguous in HBM) into an
// LDS stage with direct-to-LDS loads: every wave-wide instruction fills 1 KB
// of LDS, lane L the 16 bytes at offset 16 L; the lane fetches whichever
// global chunk belongs there under the XOR layout.  No registers are staged;
// completion is waited for with vmcnt before the stage is handed over.
template <int D>
__device__ inline void dma_tile(const uint8_t* __restrict__ kt, const uint8_t* __restrict__ vt, uint8_t* stage,
                                int wave, int lane) {
    constexpr int C = Cfg<D>::C;
#pragma unroll
    for (int n = 0; n < Cfg<D>::NK; ++n) {
        const int blk = n * 4 + wave;           // 1 KB block of the K region
        const int p = blk * 64 + lane;          // 16-byte slot
        const int r = p / C;
        const int c = (p % C) ^ kswz<D>(r);
        __builtin_amdgcn_global_load_lds((const void*)(kt + (r * C + c) * 16), (lds_ptr_t)(stage + blk * 1024),
                                         16, 0, 0);
    }
#pragma unroll
    for (int n = 0; n < Cfg<D>::NK; ++n) {
        const int blk = n * 4 + wave;
        const int p = blk * 64 + lane;
        const int d = p / 8;
        const int c = (p % 8) ^ vswz(d);
        __builtin_amdgcn_global_load_lds((const void*)(vt + (d * 8 + c) * 16),
                                         (lds_ptr_t)(stage + Cfg<D>::KB + blk * 1024), 16, 0, 0);
    }
}

// max of x over lane l and lane l ^ 32
__device__ inline float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(x, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

// Progress of the blocks of one group (grouped launch only).
struct Fence {
    int* prog;   // this group's progress slots, one per block, or null (no fencing)
    int n;       // blocks in the group
    int slot;    // this block's slot
    int base;    // sequence number of chunk 0 for the current query tile
};

// Wave 0 waits until every other block of the group has reached chunk
// sequence number seq - 1 (bounded), then publishes seq.  (A block whose kept
// tiles skip whole chunks jumps ahead; its own slot is left out of the test.)
// The caller's next barrier holds the other waves.  Relaxed device-scope
// atomics: the progress values only steer the schedule.
__device__ inline void fence_enter(const Fence& f, int seq, int wave, int lane) {
    if (wave != 0) return;
    for (int spin = 0; spin < kMaxSpin; ++spin) {
        int v = INT_MAX;
        if (lane < f.n && lane != f.slot)
            v = __hip_atomic_load(f.prog + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
        if (v >= seq - 1) break;
        __builtin_amdgcn_s_sleep(2);
    }
    if (lane == 0) __hip_atomic_store(f.prog + f.slot, seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One query tile, all four waves of the block.  `vi` < 0 marks a prefix
// (dense) query tile.  With FENCED the block follows its group's key chunks.
template <int D, bool FENCED>
__device__ __attribute__((always_inline)) inline void attend_tile(const ForwardArgs& a, uint8_t* st0, uint8_t* st1,
                                                                  int64_t bh, int qt, int vi, Fence fence) {
    using CF = Cfg<D>;
    constexpr int SD = CF::SD, OD = CF::OD;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int qh = wave & 1, kh = wave >> 1;
    const int lr = lane & 31, hf = lane >> 5;

    const bool dense = vi < 0;
    const int n_iter = dense ? a.npt + a.nvt : a.npt + a.keep;
    const int32_t* idx_row = dense ? nullptr : a.idx + (bh * a.nvt + vi) * a.keep;
    const int n_tiles = a.npt + a.nvt;
    const int64_t n_tot = (int64_t)n_tiles * kTile;
    const uint8_t* kb = (const uint8_t*)(a.k + bh * n_tot * D);
    const uint8_t* vb = (const uint8_t*)(a.vt + bh * n_tot * D);
    constexpr int TB = kTile * D * 2;  // bytes per tile
    // kept-tile numbers are clamped into range so a corrupt list cannot
    // address outside the tensors
    auto tile_of = [&](int j) -> int {
        if (dense || j < a.npt) return j;
        const int t = idx_row[j - a.npt];
        return a.npt + min(max(t, 0), a.nvt - 1);
    };

    // Per-lane LDS byte offsets inside a stage.  S^T operand: K row
    // R = 32*kh + (16-row group) + swapped position, logical chunk 2*s + hf;
    // under the XOR layout the address of step s is koff ^ (s << 5).
    const int r16 = lr & 15;
    const int rsw = (r16 & 3) | ((r16 & 4) << 1) | ((r16 & 8) >> 1);
    const int R = 32 * kh + (lr & 16) + rsw;
    const int koff = R * (D * 2) + ((hf ^ (kswz<D>(R) & 1)) << 4) + ((kswz<D>(R) >> 1) << 5);
    // O^T operand: V^T row 32*i + lr, logical chunk 4*kh + 2*c + hf; the
    // address is (voff ^ (c << 5)) + i * 32 rows
    const int vy = vswz(lr);
    const int voff = Cfg<D>::KB + lr * (kTile * 2) + (((4 * kh + hf) ^ vy) << 4);

    // Q^T operand: lane holds query 32*qh + lr, channels 16*s + 8*hf .. +7
    bf16x8 qf[SD];
    {
        const uint16_t* qrow = a.q + (bh * n_tot + (int64_t)qt * kTile + 32 * qh + lr) * D;
#pragma unroll
        for (int s = 0; s < SD; ++s) qf[s] = *(const bf16x8*)(qrow + 16 * s + 8 * hf);
    }

    f32x16 acc_o[OD];
#pragma unroll
    for (int i = 0; i < OD; ++i) acc_o[i] = f32x16{};
    float m_ref = -1e30f;  // reference maximum (base-2 logits) of this lane's query
    float l_sum = 0.f;     // this lane's share of the normaliser
    const float c2 = a.scale_log2;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    int chunk = -1;  // key chunk of the most recently requested tile (grouped launch)
    auto follow = [&](int j) {
        if constexpr (FENCED) {
            const int c = tile_of(j) / kChunk;
            if (c != chunk) {
                chunk = c;
                fence_enter(fence, fence.base + c, wave, lane);
            }
        }
    };

    __syncthreads();  // the previous query tile of this block may still read LDS
    follow(0);
    if (n_iter > 1) follow(1);
    __syncthreads();
    {
        const int t0 = tile_of(0);
        dma_tile<D>(kb + (int64_t)t0 * TB, vb + (int64_t)t0 * TB, st0, wave, lane);
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
    __syncthreads();

    // one tile per inner step: compute on buffer `cur`, prefetch the next tile
    // into the other one; the inner loop is unrolled so `cur` is a constant
    for (int j0 = 0; j0 < n_iter; j0 += 2) {
#pragma unroll
        for (int cur = 0; cur < 2; ++cur) {
            const int j = j0 + cur;
            if (j < n_iter) {
                const bool more = j + 1 < n_iter;
                uint8_t* const st = cur ? st1 : st0;  // this tile's stage
                uint8_t* const nx = cur ? st0 : st1;  // the next tile's stage
                if (more) {
                    const int tn = tile_of(j + 1);
                    dma_tile<D>(kb + (int64_t)tn * TB, vb + (int64_t)tn * TB, nx, wave, lane);
                }

                // every operand read of the tile up front
                bf16x8 kf[SD], vf[2 * OD];
#pragma unroll
                for (int s = 0; s < SD; ++s) kf[s] = *(const bf16x8*)(st + (koff ^ (s << 5)));
#pragma unroll
                for (int i = 0; i < OD; ++i)
#pragma unroll
                    for (int c = 0; c < 2; ++c)
                        vf[2 * i + c] = *(const bf16x8*)(st + (voff ^ (c << 5)) + i * 32 * (kTile * 2));

                // S^T (32 keys x 32 queries) = K Q^T
                f32x16 s_acc = f32x16{};
#pragma unroll
                for (int s = 0; s < SD; ++s)
                    s_acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], s_acc, 0, 0, 0);

                // online softmax in base 2; after the K-row swap, lane-half hf
                // holds keys 32*kh + 16*c + 8*hf + e at s_acc[8*c + e].  The
                // maximum is taken on the raw scores (the scale is positive).
                float smax = s_acc[0];
#pragma unroll
                for (int r = 1; r < 16; ++r) smax = fmaxf(smax, s_acc[r]);
                const float mt = pair_max(smax) * c2;
                if (__any(mt > m_ref + kRescaleLog2)) {
                    const float m_new = fmaxf(m_ref, mt);
                    const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
                    m_ref = m_new;
                    l_sum *= alpha;
#pragma unroll
                    for (int i = 0; i < OD; ++i)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc_o[i][r] *= alpha;
                }
                const float neg_m = -m_ref;
                bf16x8 pf16[2];
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const f32x2 p = {__builtin_amdgcn_exp2f(fmaf(s_acc[r], c2, neg_m)),
                                     __builtin_amdgcn_exp2f(fmaf(s_acc[r + 1], c2, neg_m))};
                    const bf16x2 pb = __builtin_convertvector(p, bf16x2);
                    l_sum = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, l_sum, false);
                    pf16[r >> 3][r & 7] = pb[0];
                    pf16[r >> 3][(r & 7) + 1] = pb[1];
                }

                // O^T (D x 32 queries) += V^T[:, keys of this wave] P^T
#pragma unroll
                for (int i = 0; i < OD; ++i)
#pragma unroll
                    for (int c = 0; c < 2; ++c)
                        acc_o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[2 * i + c], pf16[c], acc_o[i], 0, 0, 0);

                if (more) __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's part of the next tile landed
                if (j + 2 < n_iter) follow(j + 2);  // the tile requested at the start of the next step
                __syncthreads();
            }
        }
    }

    // ---- merge the two key halves of every query, normalise, store --------
    float* comb = (float*)st0;                       // [2 qh][OD*16][64 lanes]
    float* comb_m = (float*)st1;                     // [2 qh][64]
    float* comb_l = comb_m + 2 * 64;                 // [2 qh][64]
    uint16_t* stage = (uint16_t*)(comb_l + 2 * 64);  // [64][D + 8]
    constexpr int SROW = D + 8;
    const float l_tot = l_sum + __shfl_xor(l_sum, 32);
    if (kh == 1) {
#pragma unroll
        for (int i = 0; i < OD; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) comb[((qh * OD + i) * 16 + r) * 64 + lane] = acc_o[i][r];
        comb_m[qh * 64 + lane] = m_ref;
        comb_l[qh * 64 + lane] = l_tot;
    }
    __syncthreads();
    if (kh == 0) {
        const float m1 = comb_m[qh * 64 + lane], l1 = comb_l[qh * 64 + lane];
        const float mm = fmaxf(m_ref, m1);
        const float a0 = __builtin_amdgcn_exp2f(m_ref - mm), a1 = __builtin_amdgcn_exp2f(m1 - mm);
        const float L = l_tot * a0 + l1 * a1;
        const float inv = 1.0f / L;
        const int qrow = 32 * qh + lr;
#pragma unroll
        for (int i = 0; i < OD; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                uint16_t h4[4];
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int r = jj * 4 + ii;
                    const float o = (acc_o[i][r] * a0 + comb[((qh * OD + i) * 16 + r) * 64 + lane] * a1) * inv;
                    h4[ii] = __builtin_bit_cast(uint16_t, (__bf16)o);
                }
                const int d0 = 32 * i + 8 * jj + 4 * hf;
                uint2 pk;
                pk.x = (uint32_t)h4[0] | ((uint32_t)h4[1] << 16);
                pk.y = (uint32_t)h4[2] | ((uint32_t)h4[3] << 16);
                *(uint2*)(stage + qrow * SROW + d0) = pk;
            }
        if (a.lse && hf == 0)
            a.lse[bh * n_tot + (int64_t)qt * kTile + qrow] = (mm + __log2f(L)) * 0.69314718055994531f;
    }
    __syncthreads();
    {
        constexpr int C = CF::C;
        uint16_t* orow = a.o + (bh * n_tot + (int64_t)qt * kTile) * D;
#pragma unroll
        for (int i = 0; i < CF::NK; ++i) {
            const int q = tid + 256 * i;
            const int r = q / C, c = q % C;
            *(u32x4*)(orow + r * D + c * 8) = *(const u32x4*)(stage + r * SROW + c * 8);
        }
    }
}

// Plain launch: block g handles query tile g of [prefix tiles of every (b,h)]
// followed by [video tiles of every (b,h)], starting at tile `first`.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void
sparse_fwd_kernel(ForwardArgs a, int64_t first) {
    __shared__ __attribute__((aligned(1024))) uint8_t st0[Cfg<D>::BUF];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[Cfg<D>::BUF];
    const int64_t g = first + blockIdx.x;
    const int64_t n_pref = (int64_t)a.BH * a.npt;
    if (g < n_pref) {
        attend_tile<D, false>(a, st0, st1, g / a.npt, (int)(g % a.npt), -1, Fence{});
    } else {
        const int64_t gv = g - n_pref;
        const int vi = (int)(gv % a.nvt);
        attend_tile<D, false>(a, st0, st1, gv / a.nvt, a.npt + vi, vi, Fence{});
    }
}

// Grouped persistent launch over the video query tiles: block b belongs to
// group b % 8; round r of group g covers video query tiles
// [(r*8 + g)*S, (r*8 + g + 1)*S) of the flattened (b, h, tile) order.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void
sparse_fwd_grouped_kernel(ForwardArgs a, int* progress) {
    __shared__ __attribute__((aligned(1024))) uint8_t st0[Cfg<D>::BUF];
    __shared__ __attribute__((aligned(1024))) uint8_t st1[Cfg<D>::BUF];
    const int group = blockIdx.x % kGroups, slot = blockIdx.x / kGroups;
    const int S = gridDim.x / kGroups;
    const int64_t n_items = (int64_t)a.BH * a.nvt;
    const int n_chunks = (a.npt + a.nvt + kChunk - 1) / kChunk;
    Fence f{progress + group * kMaxGroupSize, S, slot, 0};
    for (int64_t r = 0;; ++r) {
        const int64_t item = (r * kGroups + group) * S + slot;
        if (item >= n_items) break;
        f.base = (int)(r * n_chunks);
        attend_tile<D, true>(a, st0, st1, item / a.nvt, a.npt + (int)(item % a.nvt), (int)(item % a.nvt), f);
    }
    // done: never hold the rest of the group back
    if (threadIdx.x == 0) __hip_atomic_store(f.prog + slot, INT_MAX, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void clear_progress_kernel(int* progress, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) progress[i] = 0;
}

template <int D>
hipError_t launch_forward_d(const ForwardArgs& a, int* progress, hipStream_t s) {
    const int64_t n_pref = (int64_t)a.BH * a.npt;
    const int64_t n_vid = (int64_t)a.BH * a.nvt;
    if (!progress) {
        if (n_pref + n_vid > 0)
            hipLaunchKernelGGL(sparse_fwd_kernel<D>, dim3((unsigned)(n_pref + n_vid)), dim3(256), 0, s, a,
                               (int64_t)0);
        return hipGetLastError();
    }
    if (n_pref > 0) hipLaunchKernelGGL(sparse_fwd_kernel<D>, dim3((unsigned)n_pref), dim3(256), 0, s, a, (int64_t)0);
    if (n_vid == 0) return hipGetLastError();
    // persistent grid: the blocks that fit at once, a multiple of the group
    // count, at most kMaxGroupSize per group, and no more than the work
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, sparse_fwd_grouped_kernel<D>, 256, 0);
    if (e != hipSuccess) return e;
    int64_t grid = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
    grid = grid / kGroups * kGroups;
    if (grid > (int64_t)kGroups * kMaxGroupSize) grid = (int64_t)kGroups * kMaxGroupSize;
    const int64_t need = (n_vid + kGroups - 1) / kGroups * kGroups;
    if (grid > need) grid = need;
    if (grid < kGroups) grid = kGroups;
    hipLaunchKernelGGL(clear_progress_kernel, dim3(1), dim3(512), 0, s, progress, kGroups * kMaxGroupSize);
    hipLaunchKernelGGL(sparse_fwd_grouped_kernel<D>, dim3((unsigned)grid), dim3(256), 0, s, a, progress);
    return hipGetLastError();
}

}  // namespace

size_t forward_workspace_bytes() { return (size_t)kGroups * kMaxGroupSize * sizeof(int); }

hipError_t launch_forward(const ForwardArgs& a, int D, int* progress, hipStream_t s) {
    if ((int64_t)a.BH * (a.npt + a.nvt) == 0) return hipSuccess;
    return D == 128 ? launch_forward_d<128>(a, progress, s) : launch_forward_d<64>(a, progress, s);
}

}  // namespace bsa
