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
// One query tile (64 tokens) is processed by one block of 4 waves, one wave
// per SIMD.  Every wave works on all 64 queries and takes a 32-key slice of
// every other key tile of the list: wave w = (par, kh) handles list positions
// par, par + 2, ... and keys 32*kh .. +31 of each.  Each wave keeps its own
// online softmax; the four partial results are merged once per query tile
// through LDS.
//   S^T = K Q^T and O^T = V^T P^T with v_mfma_f32_32x32x16_bf16: in every
//   accumulator a lane holds a single query (lane % 32) so the softmax state is
//   per lane and the row maximum needs one cross-half exchange.
//   K and V are stored in HBM in the MFMA fragment order (K-fragment and
//   V-fragment layouts of the C interface): every wave-wide 16-byte load reads
//   1 KB contiguous and lands exactly in the operand registers, so K and V
//   need no LDS; the Q^T fragments of the query tile are staged once in LDS
//   and read from there once per tile into registers (64 per lane for D = 128).
//   Each wave, one per SIMD, is software pipelined over its slices n; a
//   step is two windows of MFMA slots, one per query half h:
//     window 0: O[1] += V(n-1) P(n-1)[1], S(n)[1] = K(n) Q^T[1], beside the
//               softmax of S(n)[0] -> P(n)[0];
//     window 1: O[0] += V(n) P(n)[0], S(n+1)[0] = K(n+1) Q^T[0], beside the
//               softmax of S(n)[1] -> P(n)[1];
//   with the loads of V(n+1) and K(n+2) in the S slots.  The MFMAs and the
//   softmax instructions are issued alternately in a fixed order, since a
//   single wave has no other wave on its SIMD to overlap with: one pair of
//   weights per MFMA, its three stages (scaled logit, exp2, bf16 pair) in
//   consecutive slots so that no instruction waits on the one before it.
//   The softmax works in base 2 (scale * log2 e folded into one FMA).  Weights
//   are taken against a running reference maximum and the accumulators are
//   rescaled only when a slice's weights add up to more than 2^60 (exact: the
//   same reference is used for O and for the normaliser).  The normaliser
//   adds up the same bf16-rounded weights that enter the MFMA (v_dot2 with
//   ones), so each output is a convex combination of V rows.
//
// Two launch forms:
//   * plain: one block per query tile (prefix query tiles first: they are the
//     long, dense ones);
//   * grouped (video query tiles, when a workspace is given): a persistent grid
//     of 8 groups of blocks, block b in group b % 8 (the XCD that the hardware
//     dispatches it to, so a group shares one L2).  Round r of a group covers
//     consecutive query tiles of one (batch, head); the blocks of a group start
//     each round together (bounded wait) and, having equal work, sweep the key
//     tiles in ascending order in near lock-step, so a key tile is fetched into
//     the group's L2 once and read there by every block that kept it.  The
//     waits only shape the schedule; results do not depend on them.
#include <climits>
#include <mutex>

#include "bsa_kernels.h"

namespace bsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A slice's weights are computed against the current reference maximum
// without looking for the slice's own maximum; only when they add up to more
// than 2^60 (some logit above the reference by ~60 in base 2, or the first
// slice, whose reference is -1e30) is the true maximum taken, O and the
// normaliser rescaled and the weights recomputed.  Weights up to 2^60 are exact
// in float and bf16 and leave O and the normaliser far from overflow.
constexpr float kOverflowSum = 1.152921504606846976e18f;  // 2^60
constexpr int kGroups = 8;         // block groups of the grouped launch (one per XCD)
constexpr int kMaxGroupSize = 64;  // blocks per group the start-of-round wait can track
constexpr int kMaxSpin = 2000;     // bounded wait per round (x s_sleep 2)
constexpr int kStatInts = 4;       // after the counters: rounds whose wait gave up, rounds started
constexpr int kMaxListTiles = BSA_MAX_TILES;  // key tiles one query tile can visit (prefix + video)

template <int D>
struct Cfg {
    static constexpr int SD = D / 16;          // S^T MFMA steps over d = 1 KB loads of a K slice
    static constexpr int OD = D / 32;          // 32-row d blocks of O^T
    static constexpr int NV = 2 * OD;          // 1 KB loads of a V slice
    static constexpr int TB = kTile * D * 2;   // bytes of a K (or V) tile
    static constexpr int SLICE = TB / 2;       // bytes of one 32-key half of a tile
    static constexpr int MROW = D + 4;         // merge row stride in floats
    static constexpr int MERGE = 4 * 64 * MROW;          // floats: one [64][MROW] area per wave
    static constexpr int MERGE_ALL = MERGE + 2 * 4 * 64;   // + row maxima and sums per wave
    // during the main loop the same LDS holds the tile list and the Q^T
    // operand fragments ([2 query halves][SD][64 lanes][16 bytes])
    static constexpr int QFRAG = 2 * SD * 64 * 4;          // floats
    static constexpr int LOOP_ALL = kMaxListTiles + QFRAG;
    static constexpr int LDS_FLOATS = MERGE_ALL > LOOP_ALL ? MERGE_ALL : LOOP_ALL;
    // raster Q and O: the raster row of each of the tile's 64 tokens, past
    // both areas (written at staging, read by the epilogue's stores)
    static constexpr int ROWS = LDS_FLOATS;
    // ragged grid: the 8 boundary classes' 64-bit masks of real keys, written
    // once per block, after the rows
    static constexpr int PTAB = LDS_FLOATS + kTile;
    template <bool kRas, bool kPad>
    static constexpr int lds_floats() { return LDS_FLOATS + (kRas || kPad ? kTile : 0) + (kPad ? 16 : 0); }
};

// max of x over lane l and lane l ^ 32
__device__ inline float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(x, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

// K or V of one (batch, head) as a buffer resource: the loads then take one
// fixed lane offset in a vector register and the tile's offset in a scalar
// one (no 64-bit address arithmetic per load).  Its size is the (batch, head)'s
// whole range, so every load of a valid tile is in bounds.
constexpr int kBufWord3 = 0x00020000;
__device__ inline __amdgpu_buffer_rsrc_t head_rsrc(const void* base, int64_t bh, int n_tiles, int tb) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)base + bh * (int64_t)n_tiles * tb), 0,
                                             n_tiles * tb, kBufWord3);
}
__device__ inline bf16x8 frag_load(__amdgpu_buffer_rsrc_t rs, int lane_ofs, int ofs) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, lane_ofs, ofs, 0));
}
template <int N>
__device__ __attribute__((always_inline)) inline void load_frags(bf16x8 (&dst)[N], __amdgpu_buffer_rsrc_t rs,
                                                                 int lane_ofs, int ofs) {
#pragma unroll
    for (int s = 0; s < N; ++s) dst[s] = frag_load(rs, lane_ofs, ofs + s * 1024);
}

// The rare path of the overflow test: the slice's true maximum (over the
// lane pair that shares a query) becomes the reference, the accumulators of
// the query half and its normaliser are rescaled, and the slice's weights are
// recomputed.
template <int OD>
__device__ __attribute__((always_inline)) inline void rescale_slice(const f32x16& sv, float c2, float vmask,
                                                                    float& m_ref, float& l_sum, f32x16 (&acc)[OD][2],
                                                                    int qb, bf16x8 (&pf)[2], float& lrun,
                                                                    bf16x2 ones) {
    float m = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
#pragma unroll
    for (int e = 3; e < 15; e += 2) m = fmaxf(fmaxf(m, sv[e]), sv[e + 1]);
    m = fmaxf(m, sv[15]);
    const float m_new = fmaxf(m_ref, pair_max(m) * c2 + vmask);
    const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
    m_ref = m_new;
    l_sum *= alpha;
#pragma unroll
    for (int i = 0; i < OD; ++i) acc[i][qb] *= alpha;
    const float nm = vmask - m_new;
    float l = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
        const f32x2 pp = {__builtin_amdgcn_exp2f(fmaf(sv[r], c2, nm)), __builtin_amdgcn_exp2f(fmaf(sv[r + 1], c2, nm))};
        const bf16x2 pb = __builtin_convertvector(pp, bf16x2);
        l = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, l, false);
        pf[r >> 3][r & 7] = pb[0];
        pf[r >> 3][(r & 7) + 1] = pb[1];
    }
    lrun = l;
}

// A query tile of the flattened work: (batch * heads + head, query tile
// number counting the prefix tiles first, video tile number or -1 for a
// prefix tile).
struct Item {
    int64_t bh;
    int qt;
    int vi;
};

template <int D>
struct Regs {
    static constexpr int QPT = 2 * Cfg<D>::SD * 64 / 256;  // Q^T fragment chunks per thread
};
constexpr int kListPre = 4;  // kept-list entries per thread fetched ahead of a tile

// This wave's identity inside the block (the wave index is uniform).
struct Wave {
    int tid, wave, lane, par, kh, lr, hf;
    __device__ Wave() {
        tid = threadIdx.x;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        lane = tid & 63;
        par = wave >> 1;
        kh = wave & 1;
        lr = lane & 31;
        hf = lane >> 5;
    }
};

typedef const __attribute__((address_space(4))) int64_t const_i64;

// Start and length of the kept list of video query tile vi of (batch, head)
// bh: fixed keep, or the CSR row (read through the scalar cache), clamped to
// [0, col_entries) and to 1..nvt entries so that a corrupt row cannot address
// outside the lists.
__device__ inline int64_t row_begin(const ForwardArgs& a, int64_t bh, int vi) {
    const int64_t r = bh * a.nvt + vi;
    if (!a.row_ptr) return r * a.keep;
    return min(max(((const_i64*)a.row_ptr)[r], (int64_t)0), a.col_entries - 1);
}
__device__ inline int row_len(const ForwardArgs& a, int64_t bh, int vi) {
    if (!a.row_ptr) return a.keep;
    const int64_t b = row_begin(a, bh, vi);
    const int64_t e = min(((const_i64*)a.row_ptr)[bh * a.nvt + vi + 1], a.col_entries);
    return (int)min(max(e - b, (int64_t)1), (int64_t)a.nvt);
}

__device__ inline int list_len(const ForwardArgs& a, const Item& it) {
    return it.vi < 0 ? a.npt + a.nvt : a.npt + row_len(a, it.bh, it.vi);
}

// The kept-list value behind list position j of a video query tile (read
// from global memory; positions of the prefix read entry 0).
__device__ inline int list_raw(const ForwardArgs& a, const Item& it, int j) {
    if (it.vi < 0) return 0;  // prefix query tile: no list (and `idx` may be null)
    return a.idx[row_begin(a, it.bh, it.vi) + min(max(j - a.npt, 0), row_len(a, it.bh, it.vi) - 1)];
}

// Tile number of list position j given its raw kept-list value: prefix
// tiles first (and every tile for a prefix query tile), kept video tiles
// clamped into range so a corrupt list cannot address outside the tensors.
__device__ inline int list_tile(const ForwardArgs& a, const Item& it, int j, int raw) {
    return (it.vi < 0 || j < a.npt) ? j : a.npt + min(max(raw, 0), a.nvt - 1);
}

// Raster Q and O: the raster row (inside its batch element) of token `tok` of
// query tile `it`.  Prefix tokens keep their positions; a video slot maps
// through perm, and a padding slot gives -1.
__device__ inline int raster_row(const ForwardArgs& a, const Item& it, int tok) {
    const int p = it.qt * kTile + tok, np = a.npt * kTile;
    if (p < np) return p;
    const int v = a.perm[(int64_t)((int)it.bh / a.H) * (a.nvt * kTile) + (p - np)];
    // a value past the raster rows is clamped into them (a corrupt perm cannot
    // address outside Q or O)
    return v < 0 ? -1 : np + min(v, (int)(a.n_ras - np) - 1);
}

// Raster Q and O: offset of (batch, head) bh's token row 0, in elements;
// token row r of that head sits r * H * D further on.  bh < 2^31 (the
// descriptor checks bound B * H * tiles), so the split is 32-bit.
template <int D>
__device__ inline int64_t raster_head(const ForwardArgs& a, int64_t bh) {
    const int b = (int)bh / a.H, h = (int)bh - b * a.H;
    return ((int64_t)b * a.n_ras * a.H + h) * D;
}

// Issue the loads a query tile starts with: this wave's K and V fragments of
// its first slice and the K fragments of its second (tiles t0, t1), this
// thread's chunks of the tile's Q^T fragments and its first kept-list entries.
// kRas: Q is raster; lane l's `rowq` is the raster row of the tile's token l.
template <int D, bool kRas>
__device__ __attribute__((always_inline)) inline void fetch_first(const ForwardArgs& a, const Item& it, int t0, int t1,
                                                                  const Wave& w, bf16x8 (&kf)[2][Cfg<D>::SD],
                                                                  bf16x8 (&vf)[2][Cfg<D>::NV],
                                                                  u32x4 (&qpre)[Regs<D>::QPT], int (&lpre)[kListPre],
                                                                  int rowq) {
    using CF = Cfg<D>;
    constexpr int SD = CF::SD, TB = CF::TB;
    const int n_tiles = a.npt + a.nvt;
    const int64_t n_tot = (int64_t)n_tiles * kTile;
    const __amdgpu_buffer_rsrc_t krs = head_rsrc(a.k, it.bh, n_tiles, TB), vrs = head_rsrc(a.v, it.bh, n_tiles, TB);
    const int lofs = w.kh * CF::SLICE + w.lane * 16;
    load_frags(kf[0], krs, lofs, t0 * TB);
    load_frags(vf[0], vrs, lofs, t0 * TB);
    load_frags(kf[1], krs, lofs, t1 * TB);
    // Q^T operand fragment (query half qb, step s) of chunk f: lane holds
    // query 32*qb + lr, channels 16*s + 8*hf .. +7
    if constexpr (kRas) {
        // token row r of this (batch, head) at qh + r * H * D; a padding
        // slot loads row 0 and is zeroed
        const uint16_t* qh = a.q + raster_head<D>(a, it.bh);
#pragma unroll
        for (int u = 0; u < Regs<D>::QPT; ++u) {
            const int f = w.tid + 256 * u;
            const int fl = f & 63, fs = (f >> 6) % SD, fq = f / (64 * SD);
            const int r = __shfl(rowq, 32 * fq + (fl & 31));
            const u32x4 x = *(const u32x4*)(qh + (int64_t)max(r, 0) * a.H * D + 16 * fs + 8 * (fl >> 5));
            qpre[u] = r < 0 ? u32x4{} : x;
        }
    } else {
#pragma unroll
        for (int u = 0; u < Regs<D>::QPT; ++u) {
            const int f = w.tid + 256 * u;
            const int fl = f & 63, fs = (f >> 6) % SD, fq = f / (64 * SD);
            const uint16_t* src =
                a.q + (it.bh * n_tot + (int64_t)it.qt * kTile + 32 * fq + (fl & 31)) * D + 16 * fs + 8 * (fl >> 5);
            qpre[u] = *(const u32x4*)src;
        }
    }
#pragma unroll
    for (int u = 0; u < kListPre; ++u) lpre[u] = 0;
    if (it.vi >= 0) {
        const int32_t* row = a.idx + row_begin(a, it.bh, it.vi);
        const int len = row_len(a, it.bh, it.vi);
#pragma unroll
        for (int u = 0; u < kListPre; ++u) {
            const int e = w.tid + 256 * u;
            if (e < len) lpre[u] = row[e];
        }
    }
}

// One query tile, all four waves of the block, given the loads fetch_first
// issued for it.  With `has_next`, the first loads of the block's next tile
// `nx` are issued before this tile's epilogue, so that their latency overlaps
// it.  `vi` < 0 marks a prefix (dense) query tile.  kPad: a ragged grid, whose
// boundary key tiles have padding keys to mask.  kRas: raster Q and O; `rowq`
// holds this tile's raster rows (lane l: token l) on entry and the next
// tile's on exit.
template <int D, bool kPad, bool kRas>
__device__ __attribute__((always_inline)) inline void run_tile(const ForwardArgs& a, float* lds, const Item& it,
                                                               bool has_next, const Item& nx, const Wave& w,
                                                               bf16x8 (&kf)[2][Cfg<D>::SD],
                                                               bf16x8 (&vf)[2][Cfg<D>::NV],
                                                               u32x4 (&qpre)[Regs<D>::QPT],
                                                               int (&lpre)[kListPre], int& rowq) {
    using CF = Cfg<D>;
    constexpr int SD = CF::SD, OD = CF::OD, NV = CF::NV, TB = CF::TB;
    const int tid = w.tid, wave = w.wave, lane = w.lane, par = w.par, kh = w.kh, lr = w.lr, hf = w.hf;
    const int64_t bh = it.bh;
    const int qt = it.qt;
    const bool dense = it.vi < 0;
    const int n_iter = list_len(a, it);
    const int n_tiles = a.npt + a.nvt;
    const int64_t n_tot = (int64_t)n_tiles * kTile;
    int* list = (int*)lds;                            // key tile of every list position
    uint8_t* qlds = (uint8_t*)(lds + kMaxListTiles);  // Q^T fragments

    // ---- stage the tile in LDS: its key-tile list and Q^T fragments ------
    __syncthreads();  // the previous query tile's epilogue is done with LDS
    if (dense) {
        for (int j = tid; j < n_iter; j += 256) list[j] = j | (kPad && j >= a.npt ? pad_class(a.pad, j - a.npt) : 0);
    } else {
        const int32_t* row = a.idx + row_begin(a, bh, it.vi);
        const int len = n_iter - a.npt;
        for (int j = tid; j < a.npt; j += 256) list[j] = j;
#pragma unroll
        for (int u = 0; u < kListPre; ++u) {
            const int e = tid + 256 * u;
            if (e < len) {
                const int vt = min(max(lpre[u], 0), a.nvt - 1);
                list[a.npt + e] = (a.npt + vt) | (kPad ? pad_class(a.pad, vt) : 0);
            }
        }
        for (int e = tid + 256 * kListPre; e < len; e += 256) {
            const int vt = min(max(row[e], 0), a.nvt - 1);
            list[a.npt + e] = (a.npt + vt) | (kPad ? pad_class(a.pad, vt) : 0);
        }
    }
#pragma unroll
    for (int u = 0; u < Regs<D>::QPT; ++u) *(u32x4*)(qlds + (tid + 256 * u) * 16) = qpre[u];
    if (kRas && tid < kTile) ((int*)(lds + CF::ROWS))[tid] = rowq;
    __syncthreads();
    // raster Q and O: the next tile's raster rows, read now and used by its
    // first loads in this tile's epilogue
    if (kRas && has_next) rowq = raster_row(a, nx, lane);

    // the next tile's first two tile numbers for this wave, read now from
    // global memory and used after the main loop
    int n_iter_nx = 0, nraw0 = 0, nraw1 = 0;
    if (has_next) {
        n_iter_nx = list_len(a, nx);
        nraw0 = list_raw(a, nx, min(par, n_iter_nx - 1));
        nraw1 = list_raw(a, nx, min(par + 2, n_iter_nx - 1));
    }

    const int my_n = (n_iter - par + 1) >> 1;  // slices of this wave
    // tile of this wave's slice n; positions past the end repeat the last one
    // (their weights are forced to zero)
#define TILE_AT(n_) __builtin_amdgcn_readfirstlane(list[min(par + 2 * (n_), n_iter - 1)] & (kPad ? kTileBits : -1))
#define CLASSED_AT(n_) (kPad ? __builtin_amdgcn_readfirstlane(list[min(par + 2 * (n_), n_iter - 1)]) : 0)

    const __amdgpu_buffer_rsrc_t krs = head_rsrc(a.k, bh, n_tiles, TB), vrs = head_rsrc(a.v, bh, n_tiles, TB);
    const int lofs = kh * CF::SLICE + lane * 16;

    f32x16 sacc[2];   // S^T per query half: S(n)[0] and S(n)[1] in turn
    bf16x8 pf[2][2];  // P^T per query half, by 16-key half
    f32x16 acc[OD][2];
#pragma unroll
    for (int i = 0; i < OD; ++i) acc[i][0] = acc[i][1] = f32x16{};
    float m_ref[2] = {-1e30f, -1e30f};  // reference maxima (base-2 logits) of this lane's two queries
    float l_sum[2] = {0.f, 0.f};        // this lane's share of the normalisers
    const float c2 = a.scale_log2;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    // K(0), V(0), K(1) are in flight (fetch_first).  S(0)[0] now; the first
    // step's products with P(-1)[1] = 0 and V(-1) = 0 add nothing.
#pragma unroll
    for (int s = 0; s < NV; ++s) vf[1][s] = bf16x8{};
    pf[1][0] = pf[1][1] = bf16x8{};
    sacc[0] = f32x16{};
#pragma unroll
    for (int s = 0; s < SD; ++s)
        sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0][s], *(const bf16x8*)(qlds + (s * 64 + lane) * 16),
                                                          sacc[0], 0, 0, 0);
    // Q^T fragments of both query halves held in registers for the whole tile
    bf16x8 qreg[2][SD];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int s = 0; s < SD; ++s) qreg[h2][s] = *(const bf16x8*)(qlds + lane * 16 + (h2 * SD + s) * 1024);
    int t_v = TILE_AT(1);       // tile whose V is loaded next
    int t_k_next = TILE_AT(2);  // tile whose K is loaded next
    int t_s = CLASSED_AT(0);    // ragged grid: slice n's list entry, with its boundary class
    int t_s_next = CLASSED_AT(1);
    // ragged grid: the class table of real-key masks, and this lane's
    // real-key bits of slice n + 1 (boundary slices only), read a step ahead
    const uint64_t* ptab = (const uint64_t*)(lds + CF::PTAB);
    auto slice_bits = [&](int ts) -> uint32_t {
        return (kPad && (ts >> 16)) ? real_key_bits(ptab[ts >> 16], kh, hf) : 0xffffu;
    };
    uint32_t mb_next = kPad ? slice_bits(t_s) : 0xffffu;

    for (int n0 = 0; n0 <= my_n; n0 += 2) {
#pragma unroll
        for (int B = 0; B < 2; ++B) {
            const int n = n0 + B;
            const int t_k = t_k_next;  // K(n+2) and, one step later, V(n+2)
            // the tile after it, read from LDS now and used at the end of the
            // step (no wait for the read inside the step)
            const int t_after = list[min(par + 2 * (n + 3), n_iter - 1)] & (kPad ? kTileBits : -1);
            const int t_s_after = kPad ? list[min(par + 2 * (n + 2), n_iter - 1)] : 0;
            const int kofs = t_k * TB, vofs = t_v * TB;

            // One step is two windows of 2*OD + SD MFMA slots (16 for
            // D = 128), one per query half h of the softmax:
            //   window 0: O[1] += V(n-1) P(n-1)[1];  S(n)[1] = K(n) Q^T[1]
            //             (+ V(n+1) loads);  softmax of S(n)[0] -> P(n)[0]
            //   window 1: O[0] += V(n) P(n)[0];      S(n+1)[0] = K(n+1) Q^T[0]
            //             (+ K(n+2) loads);  softmax of S(n)[1] -> P(n)[1]
            // so the softmax of a half runs beside products that neither
            // write its scores nor read its weights, and P needs one buffer.
            // The weights of a half go through three stages, a pair of
            // elements at a time: scaled logit (FMA), exp2, and bf16 pair
            // with the normaliser's dot product.  A pair's stages sit in
            // consecutive slots, so no instruction waits on the one before
            // it and the single wave of the SIMD keeps the matrix core busy.
            // A scheduling fence after every slot holds this order; the Q^T
            // fragments stay in registers for the whole tile.
            // After the K-row order of the fragment layout, lane-half hf holds
            // keys 16*c + 8*hf + e of the slice at S[8*c + e].  Slices past
            // the end get -inf added to their logits (no branch).
            const float vmask = n < my_n ? 0.f : -INFINITY;
            constexpr int NPV = 2 * OD;           // PV slots of a window
            constexpr int W = NPV + SD;           // slots of a window
            constexpr int PPS = (8 + W - 4) / (W - 3);  // weight pairs per stage slot: 1 (D = 128), 2 (D = 64)
            constexpr int NSA = 8 / PPS;          // stage slots of a window
            constexpr int GSUM = NSA + 3;         // slot of the normaliser's dot products
            static_assert(NV == SD && NSA * PPS == 8 && GSUM < W, "window layout");
            float lrun[2];
            // a boundary slice: this lane's real-key bits, for both halves
            const uint32_t mb_s = mb_next;
            if (kPad) mb_next = slice_bits(t_s_next);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // h = 0: PV of query half 1 and S of half 1 (this slice);
                // h = 1: PV of half 0 and S of half 0 (next slice)
                const int pq = 1 - h, sq = 1 - h;
                const float neg_m = vmask - m_ref[h];
                // a slice of a boundary tile: its padding keys out
                if (kPad && (t_s >> 16)) {
                    uint32_t mb = mb_s;
                    asm volatile("" : "+v"(mb));  // per half: the 16 element masks are not kept live
                    mask_keys_by_bits(mb, sacc[h]);
                }
                float xa[8][2], xe[8][2];
#pragma unroll
                for (int g = 0; g < W; ++g) {
                    if (g < NPV) {
                        const int c = g / OD, i = g % OD;
                        // h = 0: V(n-1) in vf[B^1]; h = 1: V(n) in vf[B]
                        acc[i][pq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[B ^ 1 ^ h][2 * i + c], pf[pq][c],
                                                                             acc[i][pq], 0, 0, 0);
                        asm volatile("" ::"v"(acc[i][pq][0]));  // keeps the MFMA in its slot
                    } else {
                        const int st = g - NPV;
                        // h = 0: K(n) in kf[B]; h = 1: K(n+1) in kf[B^1]
                        sacc[sq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[B ^ h][st], qreg[sq][st],
                                                                           st == 0 ? f32x16{} : sacc[sq], 0, 0, 0);
                        asm volatile("" ::"v"(sacc[sq][0]));
                        if (h == 0)
                            vf[B ^ 1][st] = frag_load(vrs, lofs, vofs + st * 1024);  // V(n+1)
                        else
                            kf[B][st] = frag_load(krs, lofs, kofs + st * 1024);      // K(n+2)
                    }
                    // stage 1 (pairs of stage slot g-1): scaled logits of S(n)[h]
                    if (g >= 1 && g - 1 < NSA) {
#pragma unroll
                        for (int u = 0; u < PPS; ++u) {
                            const int p = (g - 1) * PPS + u, r = 2 * p;
                            xa[p][0] = fmaf(sacc[h][r], c2, neg_m);
                            xa[p][1] = fmaf(sacc[h][r + 1], c2, neg_m);
                            asm volatile("" : "+v"(xa[p][0]), "+v"(xa[p][1]));
                        }
                    }
                    // stage 2 (pairs of stage slot g-2): exp2
                    if (g >= 2 && g - 2 < NSA) {
#pragma unroll
                        for (int u = 0; u < PPS; ++u) {
                            const int p = (g - 2) * PPS + u;
                            xe[p][0] = __builtin_amdgcn_exp2f(xa[p][0]);
                            xe[p][1] = __builtin_amdgcn_exp2f(xa[p][1]);
                            asm volatile("" : "+v"(xe[p][0]), "+v"(xe[p][1]));
                        }
                    }
                    // stage 3 (pairs of stage slot g-3): the bf16 pair into P^T
                    if (g >= 3 && g - 3 < NSA) {
#pragma unroll
                        for (int u = 0; u < PPS; ++u) {
                            const int p = (g - 3) * PPS + u, r = 2 * p;
                            const f32x2 pp = {xe[p][0], xe[p][1]};
                            const bf16x2 pb = __builtin_convertvector(pp, bf16x2);
                            pf[h][r >> 3][r & 7] = pb[0];
                            pf[h][r >> 3][(r & 7) + 1] = pb[1];
                            asm volatile("" : "+v"(pf[h][r >> 3]));
                        }
                    }
                    // the normaliser: the same bf16 weights that enter the
                    // MFMA, added up by v_dot2 with ones.  v_dot2 waits for the
                    // matrix core to drain, so the eight of a half go together
                    // in one slot (one wait, not eight).
                    if (g == GSUM) {
                        float l0 = 0.f, l1 = 0.f;
#pragma unroll
                        for (int p = 0; p < 8; ++p) {
                            const int r = 2 * p;
                            const bf16x2 pb = {pf[h][r >> 3][r & 7], pf[h][r >> 3][(r & 7) + 1]};
                            if (p & 1)
                                l1 = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, l1, false);
                            else
                                l0 = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, l0, false);
                        }
                        lrun[h] = l0 + l1;
                        asm volatile("" : "+v"(lrun[h]));
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                // Overflow test of half h before its weights are used (rare:
                // the slice's true maximum becomes the reference, O of the
                // half, all of whose products are issued, and the normaliser
                // are rescaled and the weights recomputed).  The anchor keeps
                // the weights ahead of the branch.
                asm volatile("" : "+v"(pf[h][0]), "+v"(pf[h][1]), "+v"(lrun[h]));
                int big = __builtin_amdgcn_readfirstlane((int)__any(!(lrun[h] <= kOverflowSum)));
                asm("" : "+s"(big));
                if (big) rescale_slice<OD>(sacc[h], c2, vmask, m_ref[h], l_sum[h], acc, h, pf[h], lrun[h], ones);
                l_sum[h] += lrun[h];
            }

            t_v = t_k;
            t_k_next = __builtin_amdgcn_readfirstlane(t_after);
            if (kPad) {
                t_s = t_s_next;
                t_s_next = __builtin_amdgcn_readfirstlane(t_s_after);

            }
        }
    }
#undef TILE_AT
#undef CLASSED_AT


    // ---- the next tile's first loads, in flight during this epilogue ------
    if (has_next) {
        const int t0 = list_tile(a, nx, min(par, n_iter_nx - 1), __builtin_amdgcn_readfirstlane(nraw0));
        const int t1 = list_tile(a, nx, min(par + 2, n_iter_nx - 1), __builtin_amdgcn_readfirstlane(nraw1));
        fetch_first<D, kRas>(a, nx, t0, t1, w, kf, vf, qpre, lpre, rowq);
    }

    // ---- merge the four partial results of every query, normalise, store --
    float* merge = lds;                       // [4 waves][64 queries][MROW]
    float* mrow = lds + CF::MERGE;            // [4 waves][64] maxima
    float* lrow = mrow + 4 * 64;              // [4 waves][64] sums
    __syncthreads();  // every wave is done with the kept list
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float lt = l_sum[qb] + __shfl_xor(l_sum[qb], 32);
        if (hf == 0) {
            mrow[wave * 64 + 32 * qb + lr] = m_ref[qb];
            lrow[wave * 64 + 32 * qb + lr] = lt;
        }
    }
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int q = 32 * qb + lr;
        float M = mrow[q];
#pragma unroll
        for (int w = 1; w < 4; ++w) M = fmaxf(M, mrow[w * 64 + q]);
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) L += lrow[w * 64 + q] * __builtin_amdgcn_exp2f(mrow[w * 64 + q] - M);
        const float f = __builtin_amdgcn_exp2f(m_ref[qb] - M) / L;
        float* dst = merge + (wave * 64 + q) * CF::MROW + 4 * hf;
#pragma unroll
        for (int i = 0; i < OD; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 v = {acc[i][qb][4 * j] * f, acc[i][qb][4 * j + 1] * f, acc[i][qb][4 * j + 2] * f,
                                 acc[i][qb][4 * j + 3] * f};
                *(f32x4*)(dst + 32 * i + 8 * j) = v;
            }
        if (a.lse && wave == 0 && hf == 0)
            a.lse[bh * n_tot + (int64_t)qt * kTile + q] = (M + __log2f(L)) * 0.69314718055994531f;
    }
    __syncthreads();
    {
        constexpr int C = D / 8;
        uint16_t* orow = a.o + (bh * n_tot + (int64_t)qt * kTile) * D;
        // raster O: token row r of this (batch, head) at oh + r * H * D
        uint16_t* oh = kRas ? a.o + raster_head<D>(a, bh) : nullptr;
        const int* rows = (const int*)(lds + CF::ROWS);
#pragma unroll
        for (int u = 0; u < kTile * C / 256; ++u) {
            const int cidx = tid + 256 * u;
            const int r = cidx / C, c = cidx % C;
            f32x4 s0 = *(const f32x4*)(merge + r * CF::MROW + 8 * c);
            f32x4 s1 = *(const f32x4*)(merge + r * CF::MROW + 8 * c + 4);
#pragma unroll
            for (int w = 1; w < 4; ++w) {
                s0 += *(const f32x4*)(merge + (w * 64 + r) * CF::MROW + 8 * c);
                s1 += *(const f32x4*)(merge + (w * 64 + r) * CF::MROW + 8 * c + 4);
            }
            u32x4 pk;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const bf16x2 lo = __builtin_convertvector((f32x2){s0[2 * e], s0[2 * e + 1]}, bf16x2);
                const bf16x2 hi = __builtin_convertvector((f32x2){s1[2 * e], s1[2 * e + 1]}, bf16x2);
                pk[e] = __builtin_bit_cast(uint32_t, lo);
                pk[2 + e] = __builtin_bit_cast(uint32_t, hi);
            }
            if constexpr (kRas) {
                const int row = rows[r];  // -1: a padding slot, not stored
                if (row >= 0) *(u32x4*)(oh + (int64_t)row * a.H * D + 8 * c) = pk;
            } else {
                *(u32x4*)(orow + r * D + 8 * c) = pk;
            }
        }
    }
}

// Ragged grid: the boundary classes' masks of real keys into LDS (read after
// the first tile's staging barrier), so that a slice's mask is an LDS read
// instead of a dynamically indexed kernel argument.
template <int D>
__device__ inline void write_pad_table(const ForwardArgs& a, float* lds) {
    if (threadIdx.x < 8) {
        uint64_t v = 0;
#pragma unroll
        for (int c = 0; c < 8; ++c)
            if ((int)threadIdx.x == c) v = a.pad.real[c];
        ((uint64_t*)(lds + Cfg<D>::PTAB))[threadIdx.x] = v;
    }
}

// The first loads of a block's first tile (nothing to overlap them with).
template <int D, bool kRas>
__device__ __attribute__((always_inline)) inline void fetch_first_direct(const ForwardArgs& a, const Item& it,
                                                                         const Wave& w,
                                                                         bf16x8 (&kf)[2][Cfg<D>::SD],
                                                                         bf16x8 (&vf)[2][Cfg<D>::NV],
                                                                         u32x4 (&qpre)[Regs<D>::QPT],
                                                                         int (&lpre)[kListPre], int& rowq) {
    const int n = list_len(a, it);
    const int j0 = min(w.par, n - 1), j1 = min(w.par + 2, n - 1);
    const int t0 = list_tile(a, it, j0, __builtin_amdgcn_readfirstlane(list_raw(a, it, j0)));
    const int t1 = list_tile(a, it, j1, __builtin_amdgcn_readfirstlane(list_raw(a, it, j1)));
    if (kRas) rowq = raster_row(a, it, w.lane);
    fetch_first<D, kRas>(a, it, t0, t1, w, kf, vf, qpre, lpre, rowq);
}

// Plain launch: block g handles query tile g of [prefix tiles of every (b,h)]
// followed by [video tiles of every (b,h)], starting at tile `first`.
template <int D, bool kPad, bool kRas>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void
sparse_fwd_kernel(ForwardArgs a, int64_t first) {
    __shared__ __attribute__((aligned(16))) float lds[Cfg<D>::template lds_floats<kRas, kPad>()];
    const int64_t g = first + blockIdx.x;
    const int64_t n_pref = (int64_t)a.BH * a.npt;
    Item it;
    if (g < n_pref) {
        it = Item{g / a.npt, (int)(g % a.npt), -1};
    } else {
        const int64_t gv = g - n_pref;
        const int vi = (int)(gv % a.nvt);
        it = Item{gv / a.nvt, a.npt + vi, vi};
    }
    const Wave w;
    if (kPad) write_pad_table<D>(a, lds);
    bf16x8 kf[2][Cfg<D>::SD], vf[2][Cfg<D>::NV];
    u32x4 qpre[Regs<D>::QPT];
    int lpre[kListPre];
    int rowq = 0;
    fetch_first_direct<D, kRas>(a, it, w, kf, vf, qpre, lpre, rowq);
    run_tile<D, kPad, kRas>(a, lds, it, false, it, w, kf, vf, qpre, lpre, rowq);
}

// Grouped persistent launch over the video query tiles: block b belongs to
// group b % 8; round r of group g covers video query tiles
// [(r*8 + g)*S, (r*8 + g + 1)*S) of the flattened (b, h, tile) order.
template <int D, bool kPad, bool kRas>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void
sparse_fwd_grouped_kernel(ForwardArgs a, int* progress, int* stats) {
    __shared__ __attribute__((aligned(16))) float lds[Cfg<D>::template lds_floats<kRas, kPad>()];
    const int group = blockIdx.x % kGroups, slot = blockIdx.x / kGroups;
    const int S = gridDim.x / kGroups;
    const int64_t n_items = (int64_t)a.BH * a.nvt;
    int* prog = progress + group * kMaxGroupSize;
    auto item_of = [&](int64_t r) -> int64_t { return (r * kGroups + group) * S + slot; };
    auto make = [&](int64_t item) -> Item {
        return Item{item / a.nvt, a.npt + (int)(item % a.nvt), (int)(item % a.nvt)};
    };
    const Wave w;
    if (kPad) write_pad_table<D>(a, lds);
    bf16x8 kf[2][Cfg<D>::SD], vf[2][Cfg<D>::NV];
    u32x4 qpre[Regs<D>::QPT];
    int lpre[kListPre];
    int rowq = 0;
    if (item_of(0) < n_items) {
        Item cur = make(item_of(0));
        fetch_first_direct<D, kRas>(a, cur, w, kf, vf, qpre, lpre, rowq);
        for (int64_t r = 0;; ++r) {
            // publish the round, then wait (bounded) until every block of the
            // group has started it; the barrier at the start of the tile holds
            // the other waves
            if (threadIdx.x < 64) {
                const int lane = threadIdx.x;
                if (lane == 0) __hip_atomic_store(prog + slot, (int)r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                bool met = false;
                for (int spin = 0; spin < kMaxSpin; ++spin) {
                    int v = INT_MAX;
                    if (lane < S) v = __hip_atomic_load(prog + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
                    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
                    if (v >= (int)r) {
                        met = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
                // statistics: rounds started, and rounds whose wait gave up
                if (lane == 0) {
                    __hip_atomic_fetch_add(stats + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (!met) __hip_atomic_fetch_add(stats, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            const bool has_next = item_of(r + 1) < n_items;
            const Item nx = has_next ? make(item_of(r + 1)) : cur;
            run_tile<D, kPad, kRas>(a, lds, cur, has_next, nx, w, kf, vf, qpre, lpre, rowq);
            if (!has_next) break;
            cur = nx;
        }
    }
    // done: never hold the rest of the group back
    if (threadIdx.x == 0) __hip_atomic_store(prog + slot, INT_MAX, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void clear_progress_kernel(int* progress, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) progress[i] = 0;
}

template <int D, bool kPad, bool kRas>
hipError_t launch_forward_d(const ForwardArgs& a, int* progress, hipStream_t s) {
    const int64_t n_pref = (int64_t)a.BH * a.npt;
    const int64_t n_vid = (int64_t)a.BH * a.nvt;
    if (!progress) {
        if (n_pref + n_vid > 0)
            hipLaunchKernelGGL((sparse_fwd_kernel<D, kPad, kRas>), dim3((unsigned)(n_pref + n_vid)), dim3(256), 0, s, a,
                               (int64_t)0);
        return hipGetLastError();
    }
    if (n_pref > 0) hipLaunchKernelGGL((sparse_fwd_kernel<D, kPad, kRas>), dim3((unsigned)n_pref), dim3(256), 0, s, a, (int64_t)0);
    if (n_vid == 0) return hipGetLastError();
    // persistent grid: the blocks that fit at once, a multiple of the group
    // count, at most kMaxGroupSize per group, and no more than the work
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, sparse_fwd_grouped_kernel<D, kPad, kRas>, 256, 0);
    if (e != hipSuccess) return e;
    int64_t grid = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
    grid = grid / kGroups * kGroups;
    if (grid > (int64_t)kGroups * kMaxGroupSize) grid = (int64_t)kGroups * kMaxGroupSize;
    const int64_t need = (n_vid + kGroups - 1) / kGroups * kGroups;
    if (grid > need) grid = need;
    if (grid < kGroups) grid = kGroups;
    int* stats = progress + kGroups * kMaxGroupSize;
    hipLaunchKernelGGL(clear_progress_kernel, dim3(1), dim3(512), 0, s, progress, kGroups * kMaxGroupSize + kStatInts);
    hipLaunchKernelGGL((sparse_fwd_grouped_kernel<D, kPad, kRas>), dim3((unsigned)grid), dim3(256), 0, s, a, progress,
                       stats);
    return hipGetLastError();
}

}  // namespace

// ---- the forward without a caller workspace ---------------------------------
// For callers that cannot allocate device memory: the grouped launch's round
// counters and statistics live in this file-scope array, one copy per GPU,
// instead of in a workspace.  On the host its name is only a stand-in for the
// device array; kernels get the device address that hipGetSymbolAddress
// returns, looked up once per device with that device current.  The clear
// kernel zeroes it at the start of every call; calls that overlap on one GPU
// share it and race.
constexpr int kScratchInts = 1024;  // 4 KB
static __device__ __align__(256) int scratch[kScratchInts];
static_assert(kGroups * kMaxGroupSize + kStatInts <= kScratchInts, "grouped-launch counters exceed the scratch array");

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device of stream s (the current device
// for the null stream).
hipError_t scratch_pointer(hipStream_t s, int** out) {
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    dev = cur;
    if (s) {
        e = hipStreamGetDevice(s, &dev);
        if (e != hipSuccess) return e;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = static_cast<int*>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}
}  // namespace

size_t forward_scratch_bytes() { return sizeof(scratch); }

size_t forward_workspace_bytes() { return (size_t)(kGroups * kMaxGroupSize + kStatInts) * sizeof(int); }
size_t forward_stats_offset() { return (size_t)kGroups * kMaxGroupSize * sizeof(int); }

namespace {
template <bool kRas>
hipError_t launch_forward_r(const ForwardArgs& a, int D, int* progress, hipStream_t s) {
    if (a.pad.T != 0)
        return D == 128 ? launch_forward_d<128, true, kRas>(a, progress, s)
                        : launch_forward_d<64, true, kRas>(a, progress, s);
    return D == 128 ? launch_forward_d<128, false, kRas>(a, progress, s)
                    : launch_forward_d<64, false, kRas>(a, progress, s);
}
}  // namespace

hipError_t launch_forward(const ForwardArgs& a, int D, int* progress, hipStream_t s) {
    if ((int64_t)a.BH * (a.npt + a.nvt) == 0) return hipSuccess;
    return a.raster ? launch_forward_r<true>(a, D, progress, s) : launch_forward_r<false>(a, D, progress, s);
}

hipError_t launch_forward_noalloc(const ForwardArgs& a, int D, hipStream_t s) {
    if ((int64_t)a.BH * (a.npt + a.nvt) == 0) return hipSuccess;
    int* p = nullptr;
    const hipError_t e = scratch_pointer(s, &p);
    if (e != hipSuccess) return e;
    return launch_forward(a, D, p, s);
}

}  // namespace bsa
