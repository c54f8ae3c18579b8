// Gradients of the kept-tile attention (dQ, dK, dV), bf16 MFMA on gfx950.
//
// What is differentiated: the function the forward computes ("Prism /
// Kandinsky 6 speed ablation" page, section on Prism's block-sparse
// attention, where the same sparsity also speeds up training; "Ref2VA VSA"
// page, section on conditioning tokens, for the dense prefix).  For query q
// with key set S_q, P_qj = exp(scale q.k_j - lse_q):
//   Delta_q = dO_q . O_q,  dP_qj = dO_q . v_j,  dS_qj = P_qj (dP_qj - Delta_q),
//   dQ_q = scale sum_j dS_qj k_j,  dK_j = scale sum_q dS_qj q_q,
//   dV_j = sum_q P_qj dO_q.
// P is recomputed from the forward's lse (no per-slice maximum is needed:
// every exponent is at most 0).
//
// Work split (one block of 4 waves, one wave per SIMD, per tile):
//   * dQ: one block per query tile, over its kept key tiles (the forward's
//     list).  Wave (par, kh) takes list positions par, par + 2, ... and the
//     32-key half kh of each; every wave holds all 64 queries.  Per slice:
//       S^T = K Q^T,  dP^T = V dO^T,  dS^T = P^T (dP^T - Delta),
//       dQ^T += K^T dS^T.
//   * dK, dV: one block per key tile, over the query tiles that attend it (the
//     prefix query tiles, and the video query tiles whose list holds the key
//     tile: the transposed lists).  Wave (par, kh) takes list positions par,
//     par + 2, ... and holds its 32-key half; per slice, for each 32-query half:
//       S = Q K^T,  dP = dO V^T,  dS = P (dP - Delta),
//       dV^T += dO^T P,  dK^T += Q^T dS.
//   All products are v_mfma_f32_32x32x16_bf16 with the operands in the
//   fragment layouts of the C interface (kfrag: rows of 32 tokens by 16
//   channels; vfrag: 32 channels by 16 tokens), loaded straight into
//   registers, 1 KB per wave-wide load; the stationary operand of a block is
//   staged once in LDS.  The swap23 token order of the kfrag layout makes the
//   accumulator rows a lane holds exactly the tokens it must supply as the
//   next product's B operand, so P and dS go from accumulator to operand with
//   a bf16 cast only.  The four waves' partial sums are added once per tile in
//   LDS and written in raster order through the permutation.
#include <climits>

#include "bsa_kernels.h"

namespace bsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxListTilesB = BSA_MAX_TILES;

template <int D>
struct BCfg {
    static constexpr int SD = D / 16;         // kfrag loads (1 KB) of a 32-token half
    static constexpr int OD = D / 32;         // 32-channel blocks
    static constexpr int NV = 2 * OD;         // vfrag loads of a 32-token half
    static constexpr int TB = kTile * D * 2;  // bytes of a tile in a fragment layout
    static constexpr int HALF = TB / 2;       // bytes of a 32-token half
    static constexpr int MROW = D + 4;        // merge row stride in floats
    // stationary fragments: two operands x two 32-token halves x SD x 1 KB
    static constexpr int STAT_FLOATS = 2 * 2 * SD * 256;
    static constexpr int LOOP_FLOATS = kMaxListTilesB + STAT_FLOATS;
    static constexpr int MERGE_FLOATS = 4 * 64 * MROW;
    static constexpr int LDS_FLOATS = LOOP_FLOATS > MERGE_FLOATS ? LOOP_FLOATS : MERGE_FLOATS;
};

// token index l % 32 of a kfrag row (bits 2 and 3 exchanged)
__device__ inline int swap23(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// raster token of tiled row `row` of batch b, or -1 for a padding slot
__device__ inline int64_t raster_token(const BackwardArgs& a, int b, int64_t row) {
    if (row < a.npf) return row;
    const int32_t v = a.perm[(int64_t)b * (a.n_tot - a.npf) + (row - a.npf)];
    // a value past the raster rows is clamped into them (a corrupt perm cannot
    // address outside the gradients)
    return v < 0 ? -1 : a.npf + min((int64_t)v, a.n_ras - a.npf - 1);
}

// one (batch, head) row of D bf16 channels, raster layout
__device__ inline uint16_t* raster_row(uint16_t* base, const BackwardArgs& a, int64_t bh, int64_t tok, int D) {
    const int b = (int)bh / a.H, h = (int)bh % a.H;  // bh < B*H <= INT32_MAX
    return base + (((int64_t)b * a.n_ras + tok) * a.H + h) * D;
}

// ---- kept lists -------------------------------------------------------------
// First entry in idx and length of the kept list of video query tile row r =
// bh * nvt + i: the fixed stride, or the CSR row clamped as the forward
// clamps it (inside [0, col_entries), 1..nvt entries), so that both passes
// see the same key sets.
__device__ inline int64_t kept_begin(const BackwardArgs& a, int64_t r) {
    if (!a.row_ptr) return r * a.keep;
    return min(max(a.row_ptr[r], (int64_t)0), a.col_entries - 1);
}
__device__ inline int kept_len(const BackwardArgs& a, int64_t r) {
    if (!a.row_ptr) return a.keep;
    const int64_t e = min(a.row_ptr[r + 1], a.col_entries);
    return (int)min(max(e - kept_begin(a, r), (int64_t)1), (int64_t)a.nvt);
}

// ---- transposed lists: for each video key tile, the video query tiles that
// kept it, ascending --------------------------------------------------------
// The query tiles in chunks of 64: mask[bh][chunk][j] has bit q set when video
// query tile 64*chunk + q kept video key tile j.  One block per (bh, chunk)
// ORs its 64 kept lists into LDS (a wave per query tile, lanes over its
// entries), then writes the chunk's nvt words.
__global__ __launch_bounds__(256) void bwd_mask_kernel(BackwardArgs a) {
    extern __shared__ unsigned long long mw[];  // [nvt]
    const int64_t bh = blockIdx.x / a.mchunks;
    const int chunk = (int)(blockIdx.x % a.mchunks);
    for (int j = threadIdx.x; j < a.nvt; j += 256) mw[j] = 0ull;
    __syncthreads();
    const int q0 = chunk * 64, nq = min(64, a.nvt - q0);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int q = wave; q < nq; q += 4) {
        const int64_t r = bh * a.nvt + q0 + q;
        const int32_t* ix = a.idx + kept_begin(a, r);
        const int len = kept_len(a, r);
        for (int t = lane; t < len; t += 64) atomicOr(&mw[min(max(ix[t], 0), a.nvt - 1)], 1ull << q);
    }
    __syncthreads();
    unsigned long long* out = a.mask + (bh * a.mchunks + chunk) * a.nvt;
    for (int j = threadIdx.x; j < a.nvt; j += 256) out[j] = mw[j];
}

// cnt[bh][j] = number of video query tiles that kept j
__global__ __launch_bounds__(256) void bwd_tcount_kernel(BackwardArgs a) {
    const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;  // bh * nvt + j
    if (r >= (int64_t)a.BH * a.nvt) return;
    const int64_t bh = r / a.nvt;
    const int j = (int)(r % a.nvt);
    const unsigned long long* m = a.mask + bh * a.mchunks * a.nvt + j;
    int c = 0;
    for (int ch = 0; ch < a.mchunks; ++ch) c += __popcll(m[(int64_t)ch * a.nvt]);
    a.cnt[r] = c;
}

// rowp[0..BH*nvt]: exclusive prefix sums of the counts over (bh, j), one
// block walking the counts 1,024 at a time: a shuffle scan per wave, the 16
// wave totals through LDS, and a running carry
__global__ __launch_bounds__(1024) void bwd_tscan_kernel(BackwardArgs a) {
    __shared__ int wsum[16];
    const int64_t n = (int64_t)a.BH * a.nvt;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    int64_t carry = 0;
    for (int64_t base = 0; base < n; base += 1024) {
        const int64_t j = base + t;
        const int v = j < n ? a.cnt[j] : 0;  // each at most nvt: a tile's sum fits in int
        int x = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(x, o);
            if (lane >= o) x += y;
        }
        if (lane == 63) wsum[wave] = x;
        __syncthreads();
        int below = 0, total = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            const int sw = wsum[w];
            below += w < wave ? sw : 0;
            total += sw;
        }
        if (j < n) a.rowp[j] = carry + below + x - v;
        carry += total;
        __syncthreads();  // wsum is rewritten by the next tile
    }
    if (t == 0) a.rowp[n] = carry;
}

// tlist[rowp[bh][j] ..]: the video query tiles that kept j, ascending.  A wave
// per (bh, j) walks the chunk words in order; lane q writes query tile
// 64*chunk + q at its rank among the word's set bits.
__global__ __launch_bounds__(256) void bwd_tfill_kernel(BackwardArgs a) {
    const int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;  // bh * nvt + j (whole waves)
    if (r >= (int64_t)a.BH * a.nvt) return;
    const int lane = threadIdx.x & 63;
    const int64_t bh = r / a.nvt;
    const int j = (int)(r % a.nvt);
    const unsigned long long* m = a.mask + bh * a.mchunks * a.nvt + j;
    const unsigned long long below = (1ull << lane) - 1ull;
    int64_t o = a.rowp[r];
    for (int ch = 0; ch < a.mchunks; ++ch) {
        const unsigned long long w = m[(int64_t)ch * a.nvt];
        if ((w >> lane) & 1ull) {
            const int64_t p = o + __popcll(w & below);
            if (p < a.tcap) a.tlist[p] = ch * 64 + lane;  // a list past the capacity is cut (malformed CSR only)
        }
        o += __popcll(w);
    }
}

// ---- shared pieces of the two gradient kernels -----------------------------
struct WaveId {
    int tid, wave, lane, par, kh, lr, hf;
    __device__ WaveId() {
        tid = threadIdx.x;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        lane = tid & 63;
        par = wave >> 1;
        kh = wave & 1;
        lr = lane & 31;
        hf = lane >> 5;
    }
};

template <int N>
__device__ __attribute__((always_inline)) inline void load_n(bf16x8 (&dst)[N], const uint8_t* base) {
#pragma unroll
    for (int s = 0; s < N; ++s) dst[s] = *(const bf16x8*)(base + s * 1024);
}
// One (batch, head)'s tiles of a fragment-layout tensor as a buffer resource:
// loads take a fixed lane offset and the tile's offset in a scalar register.
__device__ inline __amdgpu_buffer_rsrc_t head_rsrc(const void* base, int64_t bh, int n_tiles, int tb) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)base + bh * (int64_t)n_tiles * tb), 0,
                                             n_tiles * tb, 0x00020000);
}
__device__ inline bf16x8 frag_load(__amdgpu_buffer_rsrc_t rs, int lane_ofs, int ofs) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, lane_ofs, ofs, 0));
}

// bf16 pair of accumulator elements r, r + 1 into a B-operand fragment pair
__device__ inline void put_pair(bf16x8 (&f)[2], int r, float x, float y) {
    const bf16x2 pb = __builtin_convertvector((f32x2){x, y}, bf16x2);
    f[r >> 3][r & 7] = pb[0];
    f[r >> 3][(r & 7) + 1] = pb[1];
}

// Adds the four waves' 32x32 fragments of a [64 rows][D] result through LDS
// and writes it, times `mul`, as bf16 rows of the raster output.  acc[i][g]:
// rows 32*i + (accumulator row) of the channels, column = token
// 32*g + swap23(lr) for the given token-half owner map.  `own` gives, per wave
// w, the token half (0/1) whose columns it holds in acc[.][0] (and 1 - own in
// acc[.][1] when it holds both halves: both = true).
template <int D>
__device__ __attribute__((always_inline)) inline void merge_store(float* lds, const f32x16 (&acc)[D / 32][2],
                                                                  bool both, const WaveId& w, float mul,
                                                                  const BackwardArgs& a, int64_t bh, int tile,
                                                                  uint16_t* out) {
    constexpr int OD = D / 32, MROW = BCfg<D>::MROW;
    float* merge = lds;  // [4 waves][64 tokens][MROW]
    __syncthreads();     // everyone is done with the loop's LDS
    {
        float* mine = merge + w.wave * 64 * MROW;
        // zero this wave's area when it holds only one half
        if (!both)
            for (int u = w.lane; u < 64 * MROW; u += 64) mine[u] = 0.f;
        const int ng = both ? 2 : 1;
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            if (g >= ng) break;
            const int half = both ? g : w.kh;
            const int tok = 32 * half + swap23(w.lr);
#pragma unroll
            for (int i = 0; i < OD; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 v = {acc[i][g][4 * j], acc[i][g][4 * j + 1], acc[i][g][4 * j + 2], acc[i][g][4 * j + 3]};
                    *(f32x4*)(mine + tok * MROW + 32 * i + 8 * j + 4 * w.hf) = v;
                }
        }
    }
    __syncthreads();
    constexpr int C = D / 8;
    const int b = (int)(bh / a.H);
#pragma unroll
    for (int u = 0; u < kTile * C / 256; ++u) {
        const int cidx = w.tid + 256 * u;
        const int r = cidx / C, c = cidx % C;
        f32x4 s0 = *(const f32x4*)(merge + r * MROW + 8 * c);
        f32x4 s1 = *(const f32x4*)(merge + r * MROW + 8 * c + 4);
#pragma unroll
        for (int q = 1; q < 4; ++q) {
            s0 += *(const f32x4*)(merge + (q * 64 + r) * MROW + 8 * c);
            s1 += *(const f32x4*)(merge + (q * 64 + r) * MROW + 8 * c + 4);
        }
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const bf16x2 lo = __builtin_convertvector((f32x2){s0[2 * e] * mul, s0[2 * e + 1] * mul}, bf16x2);
            const bf16x2 hi = __builtin_convertvector((f32x2){s1[2 * e] * mul, s1[2 * e + 1] * mul}, bf16x2);
            pk[e] = __builtin_bit_cast(uint32_t, lo);
            pk[2 + e] = __builtin_bit_cast(uint32_t, hi);
        }
        const int64_t tok = raster_token(a, b, (int64_t)tile * kTile + r);
        if (tok >= 0) *(u32x4*)(raster_row(out, a, bh, tok, D) + 8 * c) = pk;
    }
}

// ---- dQ ---------------------------------------------------------------------
// Software pipelined like the forward: a step over slice n is two windows of
// 2*OD + SD + SD MFMA slots, one per query half h of the elementwise work:
//   window 0: dQ^T[1] += K^T(n-1) dS^T(n-1)[1], S(n)[1] = K(n) Q^T[1],
//             dP(n)[1] = V(n) dO^T[1];  beside them dS^T(n)[0] and the loads
//             of K^T(n+1);
//   window 1: dQ^T[0] += K^T(n) dS^T(n)[0], S(n+1)[0], dP(n+1)[0]; beside
//             them dS^T(n)[1] and the loads of K(n+2), V(n+2).
// A half's dS^T never shares a window with the products that overwrite its
// scores or read it, so it needs one buffer.  Its pairs of elements go
// through three stages in consecutive slots: P = exp2(S c - lse), then
// P (dP - Delta), then the bf16 cast.  kPad: a ragged grid; the padding keys
// of boundary key tiles get -inf logits, so their dS is exactly 0 (their K
// rows are zero, and 0 * inf must not arise).
template <int D, bool kPad>
__device__ __attribute__((always_inline)) inline void dq_tile(const BackwardArgs& a, float* lds, int64_t bh, int qt,
                                                              const WaveId& w) {
    using CF = BCfg<D>;
    constexpr int SD = CF::SD, OD = CF::OD, NV = CF::NV, TB = CF::TB;
    const int n_tiles = a.npt + a.nvt;
    const bool dense = qt < a.npt;
    const int64_t krow = bh * a.nvt + (qt - a.npt);  // kept-list row of a video query tile
    const int n_iter = dense ? n_tiles : a.npt + kept_len(a, krow);
    int* list = (int*)lds;
    uint8_t* qlds = (uint8_t*)(lds + kMaxListTilesB);   // Q^T fragments [2][SD][64][16 B]
    uint8_t* glds = qlds + 2 * SD * 1024;                // dO^T fragments, same layout

    // ---- stage: the key-tile list and the stationary Q^T, dO^T ---------------
    __syncthreads();  // the previous tile's epilogue is done with LDS
    if (dense) {
        for (int j = w.tid; j < n_iter; j += 256) list[j] = j | (kPad && j >= a.npt ? pad_class(a.pad, j - a.npt) : 0);
    } else {
        const int32_t* row = a.idx + kept_begin(a, krow);
        for (int j = w.tid; j < a.npt; j += 256) list[j] = j;
        for (int e = w.tid; e < n_iter - a.npt; e += 256) {
            const int vt = min(max(row[e], 0), a.nvt - 1);
            list[a.npt + e] = (a.npt + vt) | (kPad ? pad_class(a.pad, vt) : 0);
        }
    }
    {
        const uint8_t* qsrc = (const uint8_t*)a.q_kf + (bh * n_tiles + qt) * (int64_t)TB;
        const uint8_t* gsrc = (const uint8_t*)a.do_kf + (bh * n_tiles + qt) * (int64_t)TB;
        for (int u = w.tid; u < TB / 16; u += 256) {
            *(u32x4*)(qlds + u * 16) = *(const u32x4*)(qsrc + u * 16);
            *(u32x4*)(glds + u * 16) = *(const u32x4*)(gsrc + u * 16);
        }
    }
    __syncthreads();

    // this lane's queries: 32*qb + swap23(lr) (the Q^T column order of kfrag)
    float lse2[2], dlt[2];
    {
        const int64_t base = bh * (int64_t)a.n_tot + (int64_t)qt * kTile;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            lse2[qb] = a.lse2[base + 32 * qb + swap23(w.lr)];
            dlt[qb] = a.delta[base + 32 * qb + swap23(w.lr)];
        }
    }
    const float c2 = a.scale_log2;
    const int par = w.par, lane = w.lane;
    const int my_n = (n_iter - par + 1) >> 1;
    const uint8_t* kkb = (const uint8_t*)a.k_kf + bh * (int64_t)n_tiles * TB + w.kh * CF::HALF + lane * 16;
    const uint8_t* vkb = (const uint8_t*)a.v_kf + bh * (int64_t)n_tiles * TB + w.kh * CF::HALF + lane * 16;
    const uint8_t* kvb = (const uint8_t*)a.k_vf + bh * (int64_t)n_tiles * TB + w.kh * CF::HALF + lane * 16;
    const __amdgpu_buffer_rsrc_t kkr = head_rsrc(a.k_kf, bh, n_tiles, TB), vkr = head_rsrc(a.v_kf, bh, n_tiles, TB),
                                 kvr = head_rsrc(a.k_vf, bh, n_tiles, TB);
    const int lofs = w.kh * CF::HALF + lane * 16;
#define TILE_AT(n_) __builtin_amdgcn_readfirstlane(list[min(par + 2 * (n_), n_iter - 1)] & (kPad ? kTileBits : -1))
#define CLASSED_AT(n_) (kPad ? __builtin_amdgcn_readfirstlane(list[min(par + 2 * (n_), n_iter - 1)]) : 0)

    f32x16 acc[OD][2];
#pragma unroll
    for (int i = 0; i < OD; ++i) acc[i][0] = acc[i][1] = f32x16{};
    f32x16 sacc[2], dpacc[2];
    bf16x8 dsf[2][2];
    bf16x8 kk[2][SD], vk[2][SD], kv[2][NV];
    {
        const int t0 = TILE_AT(0), t1 = TILE_AT(1);
        load_n(kk[0], kkb + (int64_t)t0 * TB);
        load_n(vk[0], vkb + (int64_t)t0 * TB);
        load_n(kv[0], kvb + (int64_t)t0 * TB);
        load_n(kk[1], kkb + (int64_t)t1 * TB);
        load_n(vk[1], vkb + (int64_t)t1 * TB);
    }
    // slice -1: K^T = 0 and dS^T[1] = 0 (the first window's dQ products add nothing)
#pragma unroll
    for (int f = 0; f < NV; ++f) kv[1][f] = bf16x8{};
    dsf[1][0] = dsf[1][1] = bf16x8{};
    // S(0)[0], dP(0)[0]
    sacc[0] = dpacc[0] = f32x16{};
#pragma unroll
    for (int st = 0; st < SD; ++st) {
        sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk[0][st], *(const bf16x8*)(qlds + (st * 64 + lane) * 16),
                                                          sacc[0], 0, 0, 0);
        dpacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vk[0][st], *(const bf16x8*)(glds + (st * 64 + lane) * 16),
                                                           dpacc[0], 0, 0, 0);
    }
    int t_v = TILE_AT(1);       // tile whose K^T fragments are loaded next
    int t_k_next = TILE_AT(2);  // tile whose K, V fragments are loaded next
    int t_s = CLASSED_AT(0);    // ragged grid: slice n's list entry, with its boundary class
    int t_s_next = CLASSED_AT(1);

    constexpr int NS = 2 * SD;         // S and dP slots of a window
    constexpr int W = NS + 2 * OD;     // slots of a window
    constexpr int QLEAD = 4;           // LDS read lead of the Q^T / dO^T fragments, in slots
    constexpr int NG = W / 3;          // stage groups of a window
    constexpr int PPG = 8 / NG;        // pairs of elements per stage group: 1 (D = 128), 2 (D = 64)
    static_assert(NG * PPG == 8 && 2 * OD >= QLEAD && 2 * OD + NV <= W && 2 * SD <= W, "window layout");
    int qoff = lane * 16;
    bf16x8 qf[NS];

    for (int n0 = 0; n0 <= my_n; n0 += 2) {
#pragma unroll
        for (int B = 0; B < 2; ++B) {
            const int n = n0 + B;
            const int t_k = t_k_next;
            const int t_after = list[min(par + 2 * (n + 3), n_iter - 1)] & (kPad ? kTileBits : -1);
            const int t_s_after = kPad ? list[min(par + 2 * (n + 2), n_iter - 1)] : 0;
            const int kofs = t_k * TB, kvofs = t_v * TB;
            const float vmask = n < my_n ? 0.f : -INFINITY;
            asm("" : "+v"(qoff) : "s"(n));  // opaque: keeps the LDS reads in the loop
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // h = 0: S, dP of half 1 (slice n), dQ of half 1 (slice n-1);
                // h = 1: S, dP of half 0 (slice n+1), dQ of half 0 (slice n)
                const int sq = 1 - h, pq = 1 - h;
                const float neg = vmask - lse2[h];
                // a slice of a boundary tile: its padding keys out
                if (kPad && (t_s >> 16)) mask_padding_keys(a.pad.real[t_s >> 16], w.kh, w.hf, sacc[h]);
                float xe[8][2];
#pragma unroll
                for (int g = 0; g < W; ++g) {
                    // the Q^T / dO^T fragment of S/dP slot u, QLEAD slots ahead
                    {
                        const int u = g + QLEAD - 2 * OD;
                        if (u >= 0 && u < NS)
                            qf[u] = *(const bf16x8*)((u < SD ? qlds : glds) + qoff + (sq * SD + u % SD) * 1024);
                    }
                    if (g < 2 * OD) {
                        const int c = g / OD, i = g % OD;
                        acc[i][pq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv[B ^ 1 ^ h][2 * i + c], dsf[pq][c],
                                                                             acc[i][pq], 0, 0, 0);
                        asm volatile("" ::"v"(acc[i][pq][0]));
                    } else if (g < 2 * OD + SD) {
                        const int st = g - 2 * OD;
                        sacc[sq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk[B ^ h][st], qf[st],
                                                                           st == 0 ? f32x16{} : sacc[sq], 0, 0, 0);
                        asm volatile("" ::"v"(sacc[sq][0]));
                    } else {
                        const int st = g - 2 * OD - SD;
                        dpacc[sq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vk[B ^ h][st], qf[SD + st],
                                                                            st == 0 ? f32x16{} : dpacc[sq], 0, 0, 0);
                        asm volatile("" ::"v"(dpacc[sq][0]));
                    }
                    // window 0: K^T(n+1) once its buffer's dQ products are issued;
                    // window 1: K(n+2), V(n+2); one fragment per slot
                    if (h == 0) {
                        const int f = g - 2 * OD;
                        if (f >= 0 && f < NV) kv[B ^ 1][f] = frag_load(kvr, lofs, kvofs + f * 1024);
                    } else {
                        if (g < SD) kk[B][g] = frag_load(kkr, lofs, kofs + g * 1024);
                        if (g >= SD && g < 2 * SD) vk[B][g - SD] = frag_load(vkr, lofs, kofs + (g - SD) * 1024);
                    }
                    // dS^T of half h, stage group q = g / 3
                    const int q = g / 3, stg = g % 3;
                    if (q < NG) {
#pragma unroll
                        for (int u = 0; u < PPG; ++u) {
                            const int p = q * PPG + u, r = 2 * p;
                            if (stg == 0) {
                                xe[p][0] = __builtin_amdgcn_exp2f(fmaf(sacc[h][r], c2, neg));
                                xe[p][1] = __builtin_amdgcn_exp2f(fmaf(sacc[h][r + 1], c2, neg));
                                asm volatile("" : "+v"(xe[p][0]), "+v"(xe[p][1]));
                            } else if (stg == 1) {
                                xe[p][0] *= dpacc[h][r] - dlt[h];
                                xe[p][1] *= dpacc[h][r + 1] - dlt[h];
                                asm volatile("" : "+v"(xe[p][0]), "+v"(xe[p][1]));
                            } else {
                                put_pair(dsf[h], r, xe[p][0], xe[p][1]);
                                asm volatile("" : "+v"(dsf[h][r >> 3]));
                            }
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
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
    merge_store<D>(lds, acc, true, w, a.scale, a, bh, qt, a.dq);
}

// ---- dK, dV -----------------------------------------------------------------
// One block of 8 waves per key tile walks the query tiles that attend it.  The
// waves form two quads; quad p takes the walk's tiles p, p + 2, p + 4, ... and
// wave (p, qh, kh) of it query half qh of those tiles against key half kh.
// Two waves share each SIMD, so that the vector, scalar and LDS instructions
// of one issue while the other's matrix products run.  Each wave keeps the K
// fragments of its key half in registers and reads V's from LDS (the key
// tile's V, 16 KB for D = 128, staged once per key tile), and accumulates its
// own partial dK^T and dV^T; the four partials of a key half are summed once
// per key tile.
//
// Each query tile's Q and dO rows (tiled layout, 2 x 16 KB for D = 128) and
// its 64 values of -lse / scale and -Delta are copied into LDS once, by direct
// loads, one step ahead into the quad's other stage.  In LDS the rows are kept
// whole with their 16-byte chunks XOR-swizzled by the row, so that both
// operand shapes read without bank conflicts:
//   * S = Q K^T and dP = dO V^T take Q and dO as A operands of 32 rows by 16
//     channels: one 16-byte read per lane;
//   * dV^T += dO^T P and dK^T += Q^T dS take dO^T and Q^T, 32 channels by 16
//     rows: two transposing reads (ds_read_b64_tr_b16) per lane, each giving a
//     lane 4 consecutive rows of its channel.
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef const __attribute__((address_space(4))) int32_t const_i32;

// s_waitcnt immediate for vmcnt(n), expcnt and lgkmcnt left alone (gfx9 encoding)
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// a block barrier that does not wait for the direct-to-LDS loads in flight
// (the waits before it are explicit); the empty asm keeps memory accesses on
// their side of it
__device__ __attribute__((always_inline)) inline void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// an int32 read through the scalar data cache (uniform address, data written
// by an earlier launch), so that waiting for it does not wait for the vector
// memory loads in flight
typedef const __attribute__((address_space(4))) int64_t const_i64;
__device__ inline int scalar_load(const int32_t* p) { return *(const_i32*)p; }
__device__ inline int64_t scalar_load(const int64_t* p) { return *(const_i64*)p; }

constexpr int kDkdvThreads = 512;

template <int D>
struct DkdvLds {
    static constexpr int C = D / 8;                          // 16-byte chunks of a row
    static constexpr int ROWS = kTile * D * 2;               // bytes of one tensor's rows
    static constexpr int STAGE = 2 * ROWS + 512;             // Q rows, dO rows, -lse / scale, -Delta
    static constexpr int VB = kTile * D * 2;                 // the key tile's V (K-fragment layout)
    static constexpr int MERGE = kTile * BCfg<D>::MROW * 4;  // [64][MROW] floats, over the stages
    static constexpr int BYTES = VB + 4 * STAGE;             // V, then stages (buffer, quad)
    static constexpr int OPS = C / 2 + 1;                    // direct loads per wave per tile
    static_assert(4 * STAGE >= MERGE, "merge block must fit in the stages");
};

// wave (p, qh, kh) of the dK/dV block
struct DkdvWave {
    int tid, wave, lane, quad, qw, qh, kh, lr, hf;
    __device__ DkdvWave() {
        tid = threadIdx.x;
        wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        lane = tid & 63;
        quad = wave >> 2;
        qw = wave & 3;  // wave within the quad
        qh = (wave >> 1) & 1;
        kh = wave & 1;
        lr = lane & 31;
        hf = lane >> 5;
    }
};

// Position of 16-byte chunk c of row r in LDS: c ^ rswz(r).  LDS serves 64
// banks of 4 bytes a cycle: 16 lanes of a 16-byte read or 32 lanes of an
// 8-byte read.  rswz makes both operand reads of a stage conflict-free:
//   * 16 lanes reading one chunk position of 16 distinct rows (rows
//     swap23(0..15) + 16*m): rswz is a bijection on the bits that tell those
//     rows apart within a bank row (all four low bits when a row is 256 bytes,
//     bits 1..3 when two 128-byte rows share a bank row);
//   * 32 lanes of a transposing read covering chunks 4*i .. 4*i + 3 of 4
//     consecutive rows: the row's two low bits (D = 128; its bit 1 for D = 64,
//     whose row parity picks the bank half) move the 4-chunk block.
template <int D>
__device__ inline int rswz(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Word 3 of a raw buffer resource (gfx9 family): 32-bit data format, no
// swizzle; with stride 0 a lane's offset is checked against num_records.
constexpr int kBufWord3 = 0x00020000;

// Copies query tile tq's Q and dO rows (swizzled) and its -lse / scale and
// -Delta into one LDS stage by direct buffer-to-LDS loads, shared by the four
// waves of a quad: OPS = C / 2 + 1 loads per wave, which the caller issues one
// at a time (op(k), k < OPS) spread over a step, so that they enter the memory
// pipeline gradually.  Buffer loads rather than global ones: the compiler
// treats a global load into LDS as a flat access and then makes every LDS wait
// a full one.
template <int D>
struct QueryTileLoad {
    using L = DkdvLds<D>;
    static constexpr int C = L::C;
    __amdgpu_buffer_rsrc_t rs[2], rl;
    uint8_t* stage;
    int qw, lane;
    __device__ __attribute__((always_inline)) QueryTileLoad(const BackwardArgs& a, int64_t bh, int tq, uint8_t* st,
                                                            const DkdvWave& w)
        : stage(st), qw(w.qw), lane(w.lane) {
        const int64_t row0 = bh * a.n_tot + (int64_t)tq * kTile;
        rs[0] = __builtin_amdgcn_make_buffer_rsrc((void*)(a.q_t + row0 * D), 0, L::ROWS, kBufWord3);
        rs[1] = __builtin_amdgcn_make_buffer_rsrc((void*)(a.do_t + row0 * D), 0, L::ROWS, kBufWord3);
        // -lse / scale and -Delta: wave qw copies 32 of the 128 values
        const float* g = (qw < 2 ? a.nlse : a.ndelta) + row0 + 32 * (qw & 1);
        rl = __builtin_amdgcn_make_buffer_rsrc((void*)g, 0, 32 * 4, kBufWord3);
    }
    __device__ __attribute__((always_inline)) void op(int k) const {
        if (k < C / 2) {
            const int u = k / (C / 4), n = k % (C / 4);
            const int blk = n * 4 + qw;     // 1 KB block of the region
            const int p = blk * 64 + lane;  // its 16-byte slot
            const int r = p / C;
            const int c = (p % C) ^ rswz<D>(r);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[u], (lds_ptr_t)(stage + u * L::ROWS + blk * 1024), 16,
                                                     (r * C + c) * 16, 0, 0, 0);
        } else if (lane < 32) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_ptr_t)(stage + 2 * L::ROWS + qw * 128), 4, lane * 4, 0,
                                                     0, 0);
        }
    }
};

// Sums the four partial dK^T (or dV^T) of each key half of key tile `tile` in
// one [64 keys][MROW] float block of LDS, in a fixed order, and writes it,
// times `mul`, as bf16 rows of the raster output.
template <int D>
__device__ __attribute__((always_inline)) inline void merge_partials(float* lds, const f32x16 (&acc)[D / 32],
                                                                     const DkdvWave& w, float mul,
                                                                     const BackwardArgs& a, int64_t bh, int tile,
                                                                     uint16_t* out) {
    constexpr int OD = D / 32, MROW = BCfg<D>::MROW, C = D / 8;
    const int tok = 32 * w.kh + swap23(w.lr);
    float* mine = lds + tok * MROW + 4 * w.hf;
    const int order = 2 * w.quad + w.qh;  // 3 stores, 2, 1, 0 add in turn
    block_barrier();                      // the previous user of the block is done
#pragma unroll
    for (int turn = 3; turn >= 0; --turn) {
        if (order == turn) {
#pragma unroll
            for (int i = 0; i < OD; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    f32x4* p = (f32x4*)(mine + 32 * i + 8 * j);
                    const f32x4 v = {acc[i][4 * j], acc[i][4 * j + 1], acc[i][4 * j + 2], acc[i][4 * j + 3]};
                    *p = turn == 3 ? v : *p + v;
                }
        }
        __syncthreads();
    }
    const int b = (int)(bh / a.H);
#pragma unroll
    for (int u = 0; u < kTile * C / kDkdvThreads; ++u) {
        const int cidx = w.tid + kDkdvThreads * u;
        const int r = cidx / C, c = cidx % C;
        const f32x4 s0 = *(const f32x4*)(lds + r * MROW + 8 * c);
        const f32x4 s1 = *(const f32x4*)(lds + r * MROW + 8 * c + 4);
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const bf16x2 lo = __builtin_convertvector((f32x2){s0[2 * e] * mul, s0[2 * e + 1] * mul}, bf16x2);
            const bf16x2 hi = __builtin_convertvector((f32x2){s1[2 * e] * mul, s1[2 * e + 1] * mul}, bf16x2);
            pk[e] = __builtin_bit_cast(uint32_t, lo);
            pk[2 + e] = __builtin_bit_cast(uint32_t, hi);
        }
        const int64_t tk = raster_token(a, b, (int64_t)tile * kTile + r);
        if (tk >= 0) *(u32x4*)(raster_row(out, a, bh, tk, D) + 8 * c) = pk;
    }
}

// Per-lane constants of the dK/dV walk (see dkdv_tile).
struct DkdvLane {
    int qa, tb;  // LDS offsets of the two operand shapes
};

// One query tile of the dK/dV walk for one wave: the tile's Q and dO rows,
// -lse / scale and -Delta are in LDS at `st`, the key tile's V at `vl`; when
// `nx` is not null the quad's next tile is loaded into it first.  The
// pointers are declared not to alias: the compiler then leaves the reads of
// `st` and `vl` free of waits for the loads into `nx` (the caller waits for
// those explicitly before their stage is read).
template <int D>
__device__ __attribute__((always_inline)) inline void dkdv_step(
    const BackwardArgs& a, const uint8_t* __restrict__ st, const uint8_t* __restrict__ vl,
    uint8_t* __restrict__ nx, int64_t bh, int tq_next, const DkdvWave& w, const DkdvLane& ln,
    const bf16x8 (&kreg)[D / 16], f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32]) {
    using L = DkdvLds<D>;
    constexpr int SD = D / 16, OD = D / 32, NV = 2 * OD, C = L::C;
    const float c2 = a.scale_log2;
    const int qh = w.qh;
    // the quad's next tile: one load in each of the first OPS slots
    const QueryTileLoad<D> ld(a, bh, tq_next, nx, w);
    // fresh copies of the lane offsets for this step, so that the offsets
    // derived from them are formed where they are used
    int qa_s = ln.qa, tb_s = ln.tb;
    asm volatile("" : "+v"(qa_s), "+v"(tb_s));
    // S and dP start from -lse / scale and -Delta of their rows (accumulator
    // element r = 8*c + e is row 32*qh + 16*c + 8*hf + e), so that the
    // weights are exp2(c2 * S) and dS = P * dP
    const float* init_row = (const float*)(st + 2 * L::ROWS) + 32 * qh + 8 * w.hf;
    f32x16 sc, dp;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const f32x4 x = *(const f32x4*)(init_row + 16 * c + 4 * h);
            const f32x4 y = *(const f32x4*)(init_row + 64 + 16 * c + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sc[8 * c + 4 * h + e] = x[e];
                dp[8 * c + 4 * h + e] = y[e];
            }
        }
    // 2*SD + 2*NV MFMA slots: S (SD), dP (SD), dV (NV), dK (NV); the A
    // operand of slot g (and V's fragment for a dP slot) is read from LDS
    // LEAD slots ahead
    constexpr int NSL = 2 * SD + 2 * NV, LEAD = 3;
    const uint8_t* vh = vl + w.kh * (L::VB / 2) + w.lane * 16;
    auto a_read = [&](int g) -> bf16x8 {
        if (g < 2 * SD) {
            const int s2 = g % SD;
            return *(const bf16x8*)(st + (g < SD ? 0 : L::ROWS) + (qa_s ^ (32 * s2)));
        }
        // dV (dO^T) then dK (Q^T), fragment i of query block c = j / OD
        const int j = (g - 2 * SD) % NV, i = j % OD, c = j / OD;
        const uint8_t* base = st + (g < 2 * SD + NV ? L::ROWS : 0);
        v4i16 h[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
            h[h2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4i16*)(base + (tb_s ^ (64 * i) ^ (16 * h2)) + (16 * c + 4 * h2) * C * 16));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // The elementwise work is spread over the MFMA slots, one pair q of
    // accumulator elements (2q, 2q + 1) at a time: its weights during the dP
    // products (S is complete two slots after its last product), its dS during
    // the dV products (likewise for dP); pairs 0..3 fill the first query block
    // (c = 0) before the products that read it.
    constexpr int PW = SD >= 8 ? 8 : SD - 2;
    auto p_slot = [](int q) { return SD + 2 + q * PW / 8; };
    auto ds_slot = [](int q) { return 2 * SD + 2 + q * PW / 8; };
    bf16x8 af[NSL], vf[SD];
#pragma unroll
    for (int g = 0; g < LEAD; ++g) af[g] = a_read(g);
    bf16x8 pf[2], dsf[2];
    float pw[16];  // weights P of the elements
#pragma unroll
    for (int g = 0; g < NSL; ++g) {
        if (g + LEAD < NSL) af[g + LEAD] = a_read(g + LEAD);
        if (g + LEAD >= SD && g + LEAD < 2 * SD) vf[g + LEAD - SD] = *(const bf16x8*)(vh + (g + LEAD - SD) * 1024);
        if (nx && g < L::OPS) ld.op(g);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = 2 * q;
            if (g == p_slot(q)) {
                pw[r] = __builtin_amdgcn_exp2f(sc[r] * c2);
                pw[r + 1] = __builtin_amdgcn_exp2f(sc[r + 1] * c2);
                put_pair(pf, r, pw[r], pw[r + 1]);
            }
            if (g == ds_slot(q)) put_pair(dsf, r, pw[r] * dp[r], pw[r + 1] * dp[r + 1]);
        }
        if (g < SD) {
            sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[g], kreg[g], sc, 0, 0, 0);
        } else if (g < 2 * SD) {
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[g], vf[g - SD], dp, 0, 0, 0);
        } else {
            const int j = (g - 2 * SD) % NV, i = j % OD, c = j / OD;
            if (g < 2 * SD + NV)
                dv[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[g], pf[c], dv[i], 0, 0, 0);
            else
                dk[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[g], dsf[c], dk[i], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int D>
__device__ __attribute__((always_inline)) inline void dkdv_tile(const BackwardArgs& a, uint8_t* smem, int64_t bh,
                                                                int kt, const DkdvWave& w) {
    using CF = BCfg<D>;
    using L = DkdvLds<D>;
    constexpr int SD = CF::SD, OD = CF::OD, TB = CF::TB, C = L::C;
    const int qh = w.qh;
    const int n_tiles = a.npt + a.nvt;
    uint8_t* const vl = smem;            // the key tile's V
    uint8_t* const stages = smem + L::VB;  // stage (buffer, quad) at (2 * buffer + quad) * STAGE
    block_barrier();                     // the previous tile's epilogue is done with LDS

    // the query tiles that attend key tile kt: every tile for a prefix key
    // tile; the prefix tiles and then the transposed list for a video one
    int n_iter;
    const int32_t* tl = nullptr;
    if (kt < a.npt) {
        n_iter = n_tiles;
    } else {
        const int64_t* rp = a.rowp + bh * a.nvt + (kt - a.npt);
        const int64_t b0 = min(scalar_load(rp), a.tcap), b1 = min(scalar_load(rp + 1), a.tcap);
        n_iter = a.npt + (int)(b1 - b0);
        tl = a.tlist + b0 - a.npt;
    }
    auto tile_of = [&](int n) -> int {
        if (n < a.npt || kt < a.npt) return n;
        return a.npt + min(max(scalar_load(tl + n), 0), a.nvt - 1);
    };

    // K fragments of key half kh in registers (B operands: key = lane); the
    // key tile's V into LDS (2 KB per wave)
    bf16x8 kreg[SD];
    const int64_t tile_off = (bh * n_tiles + kt) * (int64_t)TB;
    load_n(kreg, (const uint8_t*)a.k_kf + tile_off + w.kh * CF::HALF + w.lane * 16);
    {
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)a.v_kf + tile_off), 0, TB, kBufWord3);
#pragma unroll
        for (int j = 0; j < TB / 1024 / 8; ++j) {
            const int blk = w.wave * (TB / 1024 / 8) + j;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(vl + blk * 1024), 16, blk * 1024 + w.lane * 16,
                                                     0, 0, 0);
        }
    }
    f32x16 dk[OD], dv[OD];
#pragma unroll
    for (int i = 0; i < OD; ++i) dk[i] = dv[i] = f32x16{};

    // Per-lane LDS byte offsets inside a stage.  A row is C * 16 bytes and its
    // chunk position is below that, so row + position = row ^ position.
    // S / dP A operand (32 rows x 16 channels): row rq = 32*qh + swap23(lr),
    // chunk 2*s + hf at position (2*s + hf) ^ rswz(rq):
    //   offset = qa ^ (32 * s),  qa = rq*C*16 ^ ((hf ^ rswz(rq)) * 16)
    // dV^T / dK^T A operand (32 channels x 16 rows), two transposing reads
    // h2 = 0, 1 per fragment (i, c): input lane (G, ta, te) of 16-lane group G
    // addresses row r = r0 + 16*c + 4*h2, r0 = 32*qh + 8*(G/2) + te, chunk
    // 4*i + 2*(G%2) + ta/2, bytes 8*(ta%2).  rswz(r) = rswz(r0) ^ h2, so
    //   offset = tb ^ (64 * i) ^ (16 * h2) + (16*c + 4*h2) * C * 16
    DkdvLane ln;
    {
        const int rq = 32 * qh + swap23(w.lr);
        ln.qa = (rq * C * 16) ^ ((w.hf ^ rswz<D>(rq)) * 16);
        const int G = w.lane >> 4, ta = w.lane & 3, te = (w.lane >> 2) & 3;
        const int r0 = 32 * qh + 8 * (G >> 1) + te;
        ln.tb = (r0 * C * 16) | (((2 * (G & 1) + (ta >> 1)) ^ rswz<D>(r0)) * 16) | ((ta & 1) * 8);
    }

    // step m: quad p computes tile 2m + p from stage (m % 2, p) and loads tile
    // 2m + 2 + p into stage ((m + 1) % 2, p)
    const int n_steps = (n_iter + 1) / 2;
    if (w.quad < n_iter) {
        const QueryTileLoad<D> ld(a, bh, tile_of(w.quad), stages + w.quad * L::STAGE, w);
#pragma unroll
        for (int k = 0; k < L::OPS; ++k) ld.op(k);
    }
    __builtin_amdgcn_s_waitcnt(wait_vm(0));  // K, V and the first tiles
    block_barrier();
    for (int m = 0; m < n_steps; ++m) {
        const int t = 2 * m + w.quad, tn = t + 2;
        const int buf = m & 1;
        if (t < n_iter) {
            dkdv_step<D>(a, stages + (2 * buf + w.quad) * L::STAGE, vl,
                         tn < n_iter ? stages + (2 * (buf ^ 1) + w.quad) * L::STAGE : nullptr, bh,
                         tn < n_iter ? tile_of(tn) : 0, w, ln, kreg, dk, dv);
        }
        // the quad's next tile has landed (this wave's part), then everyone's,
        // and this step's stages are free again
        __builtin_amdgcn_s_waitcnt(wait_vm(0));
        block_barrier();
    }
    float* merge = (float*)stages;
    merge_partials<D>(merge, dk, w, a.scale, a, bh, kt, a.dk);
    merge_partials<D>(merge, dv, w, 1.f, a, bh, kt, a.dv);
}

// Persistent launch of a per-tile body over the BH * (npt + nvt) tiles: block b
// belongs to group b % 8 (the XCD the hardware dispatches it to, so a group
// shares one L2); round r of group g covers tiles [(r*8 + g)*S, (r*8 + g + 1)*S)
// of the (batch, head)-major order, consecutive tiles of one (batch, head).
// The blocks of a group start each round together (bounded wait) and, with
// similar work, walk their ascending lists in near lock-step, so an operand
// tile is fetched into the XCD's L2 once for every block that needs it.  The
// waits only shape the schedule; results do not depend on them.
constexpr int kGroupsB = 8, kMaxGroupSizeB = 64, kMaxSpinB = 2000;

// stats[0] counts the block rounds whose bounded wait gave up before every
// block of the group had arrived, stats[1] the block rounds started.
template <typename Body>
__device__ __attribute__((always_inline)) inline void grouped_rounds(const BackwardArgs& a, int* progress, int* stats,
                                                                     Body body) {
    const int group = blockIdx.x % kGroupsB, slot = blockIdx.x / kGroupsB;
    const int S = gridDim.x / kGroupsB;
    const int n_tiles = a.npt + a.nvt;
    const int64_t n_items = (int64_t)a.BH * n_tiles;
    int* prog = progress + group * kMaxGroupSizeB;
    for (int64_t r = 0;; ++r) {
        const int64_t item = (r * kGroupsB + group) * S + slot;
        if (item >= n_items) break;
        if (threadIdx.x < 64) {
            const int lane = threadIdx.x;
            if (lane == 0) __hip_atomic_store(prog + slot, (int)r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            bool met = false;
            for (int spin = 0; spin < kMaxSpinB; ++spin) {
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
            if (lane == 0) {
                __hip_atomic_fetch_add(stats + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (!met) __hip_atomic_fetch_add(stats, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        body(item / n_tiles, (int)(item % n_tiles));
    }
    // done: never hold the rest of the group back
    if (threadIdx.x == 0) __hip_atomic_store(prog + slot, INT_MAX, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, bool kPad>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dq_kernel(BackwardArgs a,
                                                                                              int* progress) {
    __shared__ __attribute__((aligned(16))) float lds[BCfg<D>::LDS_FLOATS];
    const WaveId w;
    grouped_rounds(a, progress, progress + backward_stats_ints(),
                   [&](int64_t bh, int qt) { dq_tile<D, kPad>(a, lds, bh, qt, w); });
}

template <int D>
__global__ __launch_bounds__(kDkdvThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dkdv_kernel(
    BackwardArgs a, int* progress) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[DkdvLds<D>::BYTES];
    const DkdvWave w;
    grouped_rounds(a, progress, progress + backward_stats_ints() + 2,
                   [&](int64_t bh, int kt) { dkdv_tile<D>(a, smem, bh, kt, w); });
}

__global__ void bwd_clear_progress_kernel(int* progress, int n) {
    for (int i = threadIdx.x; i < n; i += blockDim.x) progress[i] = 0;
}

template <typename K>
hipError_t grouped_grid(K kernel, int threads, int64_t work, int64_t* grid) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0);
    if (e != hipSuccess) return e;
    int64_t g = (int64_t)cus * (per_cu > 0 ? per_cu : 1);
    g = g / kGroupsB * kGroupsB;
    if (g > (int64_t)kGroupsB * kMaxGroupSizeB) g = (int64_t)kGroupsB * kMaxGroupSizeB;
    const int64_t need = (work + kGroupsB - 1) / kGroupsB * kGroupsB;
    if (g > need) g = need;
    if (g < kGroupsB) g = kGroupsB;
    *grid = g;
    return hipSuccess;
}

template <int D, bool kPad>
hipError_t launch_backward_d(const BackwardArgs& a, hipStream_t s) {
    if (a.nvt > 0) {
        const int64_t vt = (int64_t)a.BH * a.nvt;
        const unsigned g = (unsigned)((vt + 255) / 256);
        hipLaunchKernelGGL(bwd_mask_kernel, dim3((unsigned)((int64_t)a.BH * a.mchunks)), dim3(256),
                           (size_t)a.nvt * sizeof(unsigned long long), s, a);
        hipLaunchKernelGGL(bwd_tcount_kernel, dim3(g), dim3(256), 0, s, a);
        hipLaunchKernelGGL(bwd_tscan_kernel, dim3(1), dim3(1024), 0, s, a);
        hipLaunchKernelGGL(bwd_tfill_kernel, dim3((unsigned)((vt * 64 + 255) / 256)), dim3(256), 0, s, a);
    }
    const int64_t tiles = (int64_t)a.BH * (a.npt + a.nvt);
    int64_t gq = 0, gk = 0;
    hipError_t e = grouped_grid(bwd_dq_kernel<D, kPad>, 256, tiles, &gq);
    if (e == hipSuccess) e = grouped_grid(bwd_dkdv_kernel<D>, kDkdvThreads, tiles, &gk);
    if (e != hipSuccess) return e;
    constexpr int NP = kGroupsB * kMaxGroupSizeB;
    static_assert(NP == backward_stats_ints(), "statistics follow the round counters");
    // the first clear takes the statistics too, the second only the counters
    hipLaunchKernelGGL(bwd_clear_progress_kernel, dim3(1), dim3(512), 0, s, a.progress, backward_progress_ints());
    hipLaunchKernelGGL((bwd_dq_kernel<D, kPad>), dim3((unsigned)gq), dim3(256), 0, s, a, a.progress);
    hipLaunchKernelGGL(bwd_clear_progress_kernel, dim3(1), dim3(512), 0, s, a.progress, NP);
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((unsigned)gk), dim3(kDkdvThreads), 0, s, a, a.progress);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, int D, hipStream_t s) {
    if ((int64_t)a.BH * (a.npt + a.nvt) == 0) return hipSuccess;
    if (a.pad.T != 0)
        return D == 128 ? launch_backward_d<128, true>(a, s) : launch_backward_d<64, true>(a, s);
    return D == 128 ? launch_backward_d<128, false>(a, s) : launch_backward_d<64, false>(a, s);
}

}  // namespace bsa
