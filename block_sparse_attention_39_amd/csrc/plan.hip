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
//          Besides the float means it writes each mean as a bf16 hi/lo pair in
//          MFMA operand order, and each mean's norm.
// select : one persistent block of 8 waves per CU; a work item is R query rows
//          of one (batch, head).  The R x nvt scores are computed on bf16 MFMA
//          from the hi/lo pairs (hi*hi + hi*lo + lo*hi, float accumulation)
//          into LDS; no score matrix goes to memory.  Then each wave takes two
//          rows: it brackets the k-th largest float score of both by counts
//          (interpolation steps) and settles every key whose float score lies
//          within the float error bound of the bracket by recomputing its
//          score in double, in the order of the channels, so that the kept set
//          is exactly the top k of the double scores.
#include "bsa_kernels.h"

namespace bsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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
__device__ inline void mean8(float (&m)[8], const double (&acc)[8], double count) {
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = (float)(acc[e] / count);
}

// real tokens of video tile i (64 without padding)
__device__ inline int tile_count(const PadGeo& g, int64_t i) {
    if (g.T == 0) return kTile;
    const int wi = (int)(i % g.Tw), hi = (int)((i / g.Tw) % g.Th), ti = (int)(i / ((int64_t)g.Tw * g.Th));
    return min(g.tt, g.T - ti * g.tt) * min(g.th, g.Hg - hi * g.th) * min(g.tw, g.W - wi * g.tw);
}

template <int D>
__global__ __launch_bounds__(256) void pool_kernel(const uint4* __restrict__ q, const uint4* __restrict__ k,
                                                   PoolOut qo, PoolOut ko, int BH, int n_prefix, int nvt,
                                                   PadGeo pad) {
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
    float m[8];
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
        // every lane holds the sums of its chunk c = lane % C
        mean8(m, acc, count);
        float sq = 0.f;
        if (lane < C) sq = store_pooled8(qo, bh, nvt, D, i, c, m);
#pragma unroll
        for (int o = 1; o < C; o <<= 1) sq += __shfl_xor(sq, o);
        if (lane == 0) qo.norm[t] = sqrtf(sq);
    } else {
        const int grp = lane / LPG, part = lane % LPG;
        const int s = grp >> 1, hf = grp & 1;
        uint4 x[TPL];
#pragma unroll
        for (int u = 0; u < TPL; ++u) {
            const int tok = part * TPL + u;  // 32 kh + m
            const int kh = tok >> 5, mm = tok & 31;
            x[u] = src[(kh * SD + s) * 64 + 32 * hf + mm];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < TPL; ++u) acc8(acc, x[u]);
#pragma unroll
        for (int o = 1; o < LPG; o <<= 1)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o);
        // the LPG lanes of group grp hold the sums of channels 8 * grp .. +7
        mean8(m, acc, count);
        float sq = 0.f;
        if (part == 0) sq = store_pooled8(ko, bh, nvt, D, i, grp, m);
#pragma unroll
        for (int o = LPG; o < 64; o <<= 1) sq += __shfl_xor(sq, o);
        if (lane == 0) ko.norm[t] = sqrtf(sq);
    }
}

// ----------------------------------------------------------------- select --
constexpr int kSelWaves = 8;   // two waves per SIMD: one's latencies hide under the other's work
constexpr int kSelBlocks = 256;  // persistent blocks: one per CU of the MI355X
// per-wave scratch, in 32-bit words: two query rows in double (256 words each
// for D = 128); a lone row's radix counts take the first 256 words, its query
// row the second 256
constexpr int kWaveScratch = 512;
constexpr int kCandidates = 12;  // bracket search stops at this many scores inside the bracket
enum : uint32_t { kTagOut = 0, kTagIn = 1, kTagMember = 2 };

// |float score - double score| <= coef(D) |qbar| |kbar| + tiny: the hi/lo
// split leaves at most 3.1 * 2^-16 |q_d k_d| per product (the dropped lo*lo
// term and the two splits' remainders), and the float accumulation of the
// 3D exact bf16 products (in up to 3D + 2 additions, each allowed a relative
// 2^-23 whatever the MFMA's internal rounding) adds at most
// (3D + 2) 2^-23 (1 + 2^-7)^2 sum_d |q_d k_d|; sum_d |q_d k_d| <= |q| |k|.  The
// factor 2 covers the float norms' own rounding with a wide margin.
template <int D>
__host__ __device__ constexpr float select_coef() {
    return 2.0f * (3.1f / 65536.f + 1.05f * (3 * D + 2) / 8388608.f);
}

__device__ inline float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ inline float wave_min(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fminf(x, __shfl_xor(x, o));
    return x;
}
__device__ inline int wave_sum(int x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}
// Wave-wide max / min through DPP: butterflies inside each quad, mirrors
// inside each row of 16 lanes, then row broadcasts; lane 63 ends with the
// result, which readlane makes uniform.
template <int CTRL, int ROWS>
__device__ inline float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROWS, 0xf, false));
}
__device__ inline float wave_max_dpp(float v) {
    v = fmaxf(v, dpp_f<0xB1, 0xf>(v));   // quad_perm 1,0,3,2
    v = fmaxf(v, dpp_f<0x4E, 0xf>(v));   // quad_perm 2,3,0,1
    v = fmaxf(v, dpp_f<0x141, 0xf>(v));  // row_half_mirror
    v = fmaxf(v, dpp_f<0x140, 0xf>(v));  // row_mirror
    v = fmaxf(v, dpp_f<0x142, 0xa>(v));  // row_bcast15 into rows 1, 3
    v = fmaxf(v, dpp_f<0x143, 0xc>(v));  // row_bcast31 into rows 2, 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
template <int CTRL, int ROWS>
__device__ inline int dpp_i(int v) {  // rows outside ROWS read 0
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xf, false);
}
__device__ inline int wave_sum_dpp(int v) {
    v += dpp_i<0xB1, 0xf>(v);
    v += dpp_i<0x4E, 0xf>(v);
    v += dpp_i<0x141, 0xf>(v);
    v += dpp_i<0x140, 0xf>(v);
    v += dpp_i<0x142, 0xa>(v);
    v += dpp_i<0x143, 0xc>(v);
    return __builtin_amdgcn_readlane(v, 63);
}
__device__ inline float wave_min_dpp(float v) {
    v = fminf(v, dpp_f<0xB1, 0xf>(v));
    v = fminf(v, dpp_f<0x4E, 0xf>(v));
    v = fminf(v, dpp_f<0x141, 0xf>(v));
    v = fminf(v, dpp_f<0x140, 0xf>(v));
    v = fminf(v, dpp_f<0x142, 0xa>(v));
    v = fminf(v, dpp_f<0x143, 0xc>(v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ inline int lanes_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}
__device__ inline int popc(uint64_t m) { return __popcll(m); }

// Order-preserving unsigned image of a double (larger value -> larger key);
// -0 is folded onto +0 so that equal scores give equal keys.
__device__ inline uint64_t order_key64(double x) {
    const uint64_t u = (uint64_t)__double_as_longlong(x + 0.0);
    return (u >> 63) ? ~u : (u | (1ull << 63));
}

// sum_d q[d] k[d] in double, channel by channel in increasing order: every
// product of two floats is exact in double, so this is the plain sequential
// double sum of the exact products.  q: the query row, already widened to
// double in LDS; the key row's loads are all issued before the first product
// (one memory latency per call).
template <int D>
__device__ inline double exact_score(const double* __restrict__ q, const float* __restrict__ k) {
    float4 kv[D / 4];
#pragma unroll
    for (int d = 0; d < D / 4; ++d) kv[d] = ((const float4*)k)[d];
    double s = 0.0;
#pragma unroll
    for (int d = 0; d < D / 4; ++d) {
        s = fma(q[4 * d], (double)kv[d].x, s);
        s = fma(q[4 * d + 1], (double)kv[d].y, s);
        s = fma(q[4 * d + 2], (double)kv[d].z, s);
        s = fma(q[4 * d + 3], (double)kv[d].w, s);
    }
    return s;
}

// A query row widened to double into the wave's scratch (lanes 0 .. D/2-1).
template <int D>
__device__ inline void stage_query(double* dst, const float* __restrict__ q, int lane) {
    if (lane < D / 2) {
        const float2 v = ((const float2*)q)[lane];
        dst[2 * lane] = (double)v.x;
        dst[2 * lane + 1] = (double)v.y;
    }
}

// Threshold digit of a histogram scanned from the top: with lane l holding
// the W counts of digits top - W*l - 0 .. top - W*l - (W-1) in h, the digit
// at which the running count from the top reaches `need`, and the count of
// the digits above it.  Returns false if no lane reaches `need`.
template <int W>
__device__ inline bool top_digit(const int (&h)[W], int top, int need, int lane, int& digit, int& above) {
    int c = 0;
#pragma unroll
    for (int q = 0; q < W; ++q) c += h[q];
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
    }
    const int excl = incl - c;
    const uint64_t cm = __ballot(excl < need && incl >= need);
    if (cm == 0) return false;
    const int cl = __ffsll((long long)cm) - 1;
    int d = 0, run = excl;
    bool found = false;
#pragma unroll
    for (int q = 0; q < W; ++q) {
        if (!found && run + h[q] >= need) {
            d = top - W * lane - q;
            found = true;
        } else if (!found) {
            run += h[q];
        }
    }
    digit = __builtin_amdgcn_readlane(d, cl);
    above = __builtin_amdgcn_readlane(run, cl);
    return true;
}

// The selection of a row by one wave (two rows per wave, side by side), in
// three stages.  The row's n float scores are read from LDS into registers
// (key j = lane + 64 p in x[p]); the LDS row is then reused for the members'
// verdicts and the output.
//  1. classify_pair: a bracket lo <= T <= hi of the k-th largest float score
//     T, from the row's extremes and counts (fewer than k scores above hi, at
//     least k at or above lo), narrowed by interpolation until at most
//     kCandidates scores lie in between.  With e bounding |float score -
//     double score|: a key with float score above hi + 2e has a double score
//     above that of every key whose float score is at most T, and at most
//     k - 1 keys have a float score above T, so it is among the top k; a key
//     below lo - 2e is beaten by the (at least k) keys with float scores >= T,
//     so it is not.  The keys in between are the members.
//  2. resolve: the members are scored again in double (both rows of a wave
//     in one pass when their members fit in 64 lanes) and the best
//     k - (keys above) of them by (-double score, index) complete the set,
//     found by a ballot radix select over the double scores' order keys
//     (best_members); more than 64 members go through an 8-bit radix select
//     through LDS and the workspace.
//  3. output_row: the kept keys written out in ascending order.
template <int P>
struct RowState {
    static constexpr int NW = (P + 31) / 32;
    uint32_t inb[NW], memb[NW];  // this lane's keys above the band / inside it
    int32_t* out;
    int64_t rid;
    float* row;
    int k, nu, nm, need, my_mem, taken;
    bool ok, uniform, done;
};

// The kept count and output of row i; a row keeping none or all of its keys
// is done here (all: written out when `write`).
template <int P>
__device__ inline void row_setup(RowState<P>& st, const SelectArgs& a, float* row, int64_t bh, int i, int lane,
                                 bool write) {
    const int n = a.nvt;
    st.row = row;
    st.rid = bh * n + i;
    if (a.row_ptr) {
        const int64_t b0 = a.row_ptr[st.rid];
        st.k = (int)(a.row_ptr[st.rid + 1] - b0);
        st.out = a.idx + b0;
    } else {
        st.k = a.k_fixed;
        st.out = a.idx + st.rid * a.k_fixed;
    }
    const int k = st.k = min(max(st.k, 0), n);
    st.done = k == 0 || k == n;
    st.nu = st.nm = st.need = st.my_mem = st.taken = 0;
    st.ok = true;
    st.uniform = true;
#pragma unroll
    for (int w = 0; w < RowState<P>::NW; ++w) st.inb[w] = st.memb[w] = 0u;
    if (st.done && k == n && write)  // every key
        for (int j = lane; j < n; j += 64) st.out[j] = j;
}

// Both rows of a wave go through the bracket search together: each counting
// pass counts both rows, so the two chains of wave reductions overlap.  A
// lone row (two = false) runs as row 0 only.
template <int D, int P>
__device__ void classify_pair(RowState<P>& s0, RowState<P>& s1, bool two, const SelectArgs& a, float* row0,
                              float* row1, int64_t bh, int i0, int i1, float kmax, int lane) {
    constexpr int NW = RowState<P>::NW;
    const int n = a.nvt;
    row_setup<P>(s0, a, row0, bh, i0, lane, true);
    row_setup<P>(s1, a, two ? row1 : row0, bh, two ? i1 : i0, lane, two);
    if (!two) s1.done = true;
    if (s0.done && s1.done) return;
    // keys past n (and rows that are done) read as NaN: every ordered
    // comparison below is false for them
    float x0[P], x1[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const bool in = lane + 64 * p < n;
        x0[p] = in && !s0.done ? row0[lane + 64 * p] : __builtin_nanf("");
        x1[p] = in && !s1.done ? row1[lane + 64 * p] : __builtin_nanf("");
    }
    const float qn0 = a.qnorm[s0.rid], qn1 = a.qnorm[s1.rid];
    const float e0 = select_coef<D>() * qn0 * kmax + 0x1p-110f * (1.f + qn0 + kmax);
    const float e1 = select_coef<D>() * qn1 * kmax + 0x1p-110f * (1.f + qn1 + kmax);
    // #{x > t} of both rows: per-lane counters in two chains per row, then
    // one DPP sum per row
    auto count_gt2 = [&](float t0, float t1, int& c0, int& c1) {
        int a0[2] = {0, 0}, a1[2] = {0, 0};
#pragma unroll
        for (int p = 0; p < P; ++p) {
            a0[p & 1] += x0[p] > t0 ? 1 : 0;
            a1[p & 1] += x1[p] > t1 ? 1 : 0;
        }
        c0 = wave_sum_dpp(a0[0] + a0[1]);
        c1 = wave_sum_dpp(a1[0] + a1[1]);
    };
    float mn0 = __builtin_inff(), mx0 = -__builtin_inff(), mn1 = __builtin_inff(), mx1 = -__builtin_inff();
#pragma unroll
    for (int p = 0; p < P; ++p) {
        mn0 = fminf(mn0, x0[p]);
        mx0 = fmaxf(mx0, x0[p]);
        mn1 = fminf(mn1, x1[p]);
        mx1 = fmaxf(mx1, x1[p]);
    }
    mn0 = wave_min_dpp(mn0);
    mx0 = wave_max_dpp(mx0);
    mn1 = wave_min_dpp(mn1);
    mx1 = wave_max_dpp(mx1);
    // the brackets: steps cut them where a straight line through the two
    // counts reaches k (at least a twentieth of the width off either end)
    float lo0 = mn0, hi0 = mx0, lo1 = mn1, hi1 = mx1;
    int gl0, gl1, gh0 = 0, gh1 = 0;
    {
        // #{x >= min} = the row's finite keys
        int a0 = 0, a1 = 0;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            a0 += x0[p] >= mn0 ? 1 : 0;
            a1 += x1[p] >= mn1 ? 1 : 0;
        }
        gl0 = wave_sum_dpp(a0);
        gl1 = wave_sum_dpp(a1);
    }
    const int k0 = s0.k, k1 = s1.k;
    bool act0 = !s0.done && gl0 - gh0 > kCandidates, act1 = !s1.done && gl1 - gh1 > kCandidates;
    for (int it = 0; it < 48 && (act0 || act1); ++it) {
        const float f0 = fminf(fmaxf((float)(k0 - gh0) / (float)(gl0 - gh0), 0.05f), 0.95f);
        const float f1 = fminf(fmaxf((float)(k1 - gh1) / (float)(gl1 - gh1), 0.05f), 0.95f);
        const float mid0 = hi0 - (hi0 - lo0) * f0, mid1 = hi1 - (hi1 - lo1) * f1;
        act0 = act0 && mid0 > lo0 && mid0 < hi0;
        act1 = act1 && mid1 > lo1 && mid1 < hi1;
        int c0, c1;
        count_gt2(mid0, mid1, c0, c1);
        if (act0) {
            if (c0 < k0) {
                hi0 = mid0;
                gh0 = c0;
            } else {
                lo0 = mid0;
                gl0 = c0;  // #{x > mid}: a lower bound of #{x >= lo}, enough to steer
            }
        }
        if (act1) {
            if (c1 < k1) {
                hi1 = mid1;
                gh1 = c1;
            } else {
                lo1 = mid1;
                gl1 = c1;
            }
        }
        act0 = act0 && gl0 - gh0 > kCandidates;
        act1 = act1 && gl1 - gh1 > kCandidates;
    }
    int ch0, ch1;
    count_gt2(hi0, hi1, ch0, ch1);
    s0.ok = gl0 >= k0 && ch0 < k0;
    s1.ok = gl1 >= k1 && ch1 < k1;
    // the band of each row: keys above it in, keys inside it members
    const float hv0 = hi0 + 2.f * e0, lv0 = lo0 - 2.f * e0, hv1 = hi1 + 2.f * e1, lv1 = lo1 - 2.f * e1;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const bool in0 = x0[p] > hv0, m0 = !in0 && x0[p] >= lv0;
        const bool in1 = x1[p] > hv1, m1 = !in1 && x1[p] >= lv1;
        s0.inb[p / 32] |= in0 ? 1u << (p % 32) : 0u;
        s0.memb[p / 32] |= m0 ? 1u << (p % 32) : 0u;
        s1.inb[p / 32] |= in1 ? 1u << (p % 32) : 0u;
        s1.memb[p / 32] |= m1 ? 1u << (p % 32) : 0u;
    }
    int in0 = 0, in1 = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        in0 += __popc(s0.inb[w]);
        s0.my_mem += __popc(s0.memb[w]);
        in1 += __popc(s1.inb[w]);
        s1.my_mem += __popc(s1.memb[w]);
    }
    s0.nu = wave_sum_dpp(in0);
    s0.nm = wave_sum_dpp(s0.my_mem);
    s1.nu = wave_sum_dpp(in1);
    s1.nm = wave_sum_dpp(s1.my_mem);
    s0.need = k0 - s0.nu;
    s1.need = k1 - s1.nu;
    s0.ok = s0.ok && s0.need >= 0 && s0.need <= s0.nm;
    s1.ok = s1.ok && s1.need >= 0 && s1.need <= s1.nm;
    s0.uniform = s0.need == 0 || s0.need == s0.nm;  // members all out or all in
    s1.uniform = s1.need == 0 || s1.need == s1.nm;
    s0.taken = s0.uniform ? s0.need : 0;
    s1.taken = s1.uniform ? s1.need : 0;
}

// List a row's members into ml[base ..] (lane by lane: lane l's run starts
// after the members of the lanes below, a prefix sum from the ballots of the
// count's bits).
template <int P>
__device__ inline void list_members(const RowState<P>& st, int* ml, int base, int lane) {
    int first = base;
#pragma unroll
    for (int b = 0; b < 7; ++b) first += lanes_below(__ballot((st.my_mem >> b) & 1)) << b;
#pragma unroll
    for (int w = 0; w < RowState<P>::NW; ++w) {
        uint32_t bits = st.memb[w];
        while (bits) {
            const int p = 32 * w + __builtin_ctz(bits);
            bits &= bits - 1;
            ml[first++] = lane + 64 * p;
        }
    }
}

// The r0 lanes of mask c0 with the largest keys, equal keys going to the
// lower index j, and likewise r1 of c1 (a second row's lanes), by an MSB-first
// radix select over the 64-bit keys with one ballot per bit: the lanes whose
// bit is set are taken whole while fewer than the remaining count, else the
// search narrows to them.  Equal keys left at the end are chosen the same way
// over the bits of j, zero side first.  Masks and counts stay uniform.
__device__ inline void best_members(uint64_t c0, int r0, uint64_t c1, int r1, uint64_t key, int j, uint64_t& sel0,
                                    uint64_t& sel1) {
    uint64_t t0 = 0, t1 = 0;
    const uint32_t klo = (uint32_t)key, khi = (uint32_t)(key >> 32);
    auto step = [](uint64_t h, uint64_t all, uint64_t& c, int& r, uint64_t& t) {
        const int n = popc(h);
        if (n >= r) {
            c = h;
        } else {
            r -= n;
            t |= h;
            c &= ~all;
        }
    };
    for (int b = 63; b >= 0; --b) {
        if ((r0 <= 0 || popc(c0) == r0) && (r1 <= 0 || popc(c1) == r1)) break;
        const uint64_t ones = __ballot(((b >= 32 ? khi : klo) >> (b & 31)) & 1u);
        step(c0 & ones, ones, c0, r0, t0);
        step(c1 & ones, ones, c1, r1, t1);
    }
    // equal keys: the r lowest j of c (j < 2^14)
    auto ties = [&](uint64_t c, int r) -> uint64_t {
        if (r <= 0) return 0ull;
        if (popc(c) <= r) return c;
        uint64_t chosen = 0;
        for (int b = 13; b >= 0; --b) {
            const uint64_t zero = c & ~__ballot((j >> b) & 1);
            const int nz = popc(zero);
            if (nz >= r) {
                c = zero;
            } else {
                r -= nz;
                chosen |= zero;
                c &= ~zero;
            }
        }
        return chosen | c;
    };
    sel0 = t0 | ties(c0, r0);
    sel1 = t1 | ties(c1, r1);
}

// Members of one row (at most 64) or of two rows (together at most 64) in
// lanes 0 .. nm0 + nm1 - 1: each scored in double, ranked within its row by
// (-double score, index), the verdict written to its row's LDS area.
template <int D, int P>
__device__ void resolve_lanes(RowState<P>& s0, RowState<P>& s1, bool two, const SelectArgs& a, int64_t bh,
                              int lane, double* qd, int* ml) {
    const int n = a.nvt;
    const int nm0 = s0.nm, ntot = nm0 + (two ? s1.nm : 0);
    list_members(s0, ml, 0, lane);
    if (two) list_members(s1, ml, nm0, lane);
    stage_query<D>(qd, a.qbar + s0.rid * D, lane);
    if (two) stage_query<D>(qd + D, a.qbar + s1.rid * D, lane);
    const bool first = lane < nm0;
    const int jm = lane < ntot ? ml[lane] : 0;
    const double s = lane < ntot ? exact_score<D>(first ? qd : qd + D, a.kbar + (bh * n + jm) * D) : 0.0;
    // each row's best need members by (-double score, index), as masks of lanes
    const uint64_t m0 = __ballot(first), m1 = two ? __ballot(lane >= nm0 && lane < ntot) : 0ull;
    uint64_t sel0, sel1;
    best_members(m0, s0.need, m1, two ? s1.need : 0, lane < ntot ? order_key64(s) : 0ull, jm, sel0, sel1);
    const bool sel = ((sel0 | sel1) >> lane) & 1ull;
    if (lane < ntot) ((uint32_t*)(first ? s0.row : s1.row))[jm] = sel ? 1u : 0u;
    s0.taken = popc(sel0);
    if (two) s1.taken = popc(sel1);
}

// Many members: flagged in the LDS row, their double scores as order keys in
// the wave's scratch (indexed by key), then an 8-bit radix select of the
// need-th largest key; equal keys go to the lower index.  (A rare path:
// loops, not unrolled code.)
template <int D, int P>
__device__ void resolve_radix(RowState<P>& st, const SelectArgs& a, int64_t bh, int lane, uint32_t* hw,
                              uint64_t* fb) {
    const int n = a.nvt;
    uint32_t* verdict = (uint32_t*)st.row;
    double* qd = (double*)(hw + 256);
    stage_query<D>(qd, a.qbar + st.rid * D, lane);
    auto mem_p = [&](int p) { return ((st.memb[p / 32] >> (p % 32)) & 1u) != 0u; };
#pragma unroll
    for (int p = 0; p < P; ++p)
        if (lane + 64 * p < n) verdict[lane + 64 * p] = mem_p(p) ? 2u : 0u;
    for (int j = lane; j < n; j += 64)
        if (verdict[j] == 2u)
            __hip_atomic_store(fb + j, order_key64(exact_score<D>(qd, a.kbar + (bh * n + j) * D)), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    __threadfence();
    uint64_t prefix = 0, pmask = 0;
    int rem = st.need;
    bool ok = true;
    for (int shift = 56; ok && shift >= 0; shift -= 8) {
        for (int b = lane; b < 256; b += 64) hw[b] = 0u;
        for (int j = lane; j < n; j += 64)
            if (verdict[j] == 2u) {
                const uint64_t key = __hip_atomic_load(fb + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if ((key & pmask) == prefix) atomicAdd(&hw[(key >> shift) & 255u], 1u);
            }
        int h4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) h4[q] = (int)hw[255 - 4 * lane - q];
        int digit = 0, ab = 0;
        ok = top_digit(h4, 255, rem, lane, digit, ab);
        rem -= ab;
        prefix |= (uint64_t)(uint32_t)digit << shift;
        pmask |= 0xffull << shift;
    }
    int ties = 0;
    st.taken = 0;
    for (int j0 = 0; ok && j0 < n; j0 += 64) {
        const int j = j0 + lane;
        const bool mem = j < n && verdict[j] == 2u;
        const uint64_t key = mem ? __hip_atomic_load(fb + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
        const bool eq = mem && key == prefix;
        const uint64_t em = __ballot(eq);
        const bool sel = mem && (key > prefix || (eq && ties + lanes_below(em) < rem));
        if (mem) verdict[j] = sel ? 1u : 0u;
        ties += popc(em);
        st.taken += popc(__ballot(sel));
    }
    st.ok = st.ok && ok;
}

// Exactly k keys must be kept (always so for finite scores; otherwise, e.g.
// with NaN scores, the first k keys keep the list well formed).  A lane reads
// the verdicts of its own members, then the kept keys are written out in
// ascending order, 64 keys per ballot.
template <int P>
__device__ void output_row(const RowState<P>& st, int n, int lane) {
    constexpr int NW = RowState<P>::NW;
    const bool degenerate = !st.ok || st.nu + st.taken != st.k;
    const uint32_t* verdict = (const uint32_t*)st.row;
    uint32_t selb[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        selb[w] = st.inb[w] | (st.uniform && st.need > 0 ? st.memb[w] : 0u);
        if (!st.uniform) {
            uint32_t bits = st.memb[w];
            while (bits) {
                const int b = __builtin_ctz(bits);
                bits &= bits - 1;
                if (verdict[lane + 64 * (32 * w + b)] != 0u) selb[w] |= 1u << b;
            }
        }
    }
    // each ballot's kept keys take consecutive places: stores straight to the
    // output list, coalesced
    int pos = 0;
#pragma unroll
    for (int p = 0; p < P; ++p) {
        const int j = lane + 64 * p;
        const bool sel = degenerate ? j < st.k : ((selb[p / 32] >> (p % 32)) & 1u) != 0u;
        const uint64_t sm = __ballot(sel);
        if (sel) st.out[pos + lanes_below(sm)] = j;
        pos += popc(sm);
    }
}

// The rows r0 (and r1 when two) of an item, by one wave.
template <int D, int P>
__device__ void select_rows(const SelectArgs& a, float* row0, float* row1, int i0, int i1, bool two, int64_t bh,
                            float kmax, int lane, uint32_t* hw, int* ml, uint64_t* fb) {
    RowState<P> s0, s1;
    classify_pair<D, P>(s0, s1, two, a, row0, row1, bh, i0, i1, kmax, lane);
    const bool act0 = !s0.done && s0.ok && !s0.uniform;
    const bool act1 = two && !s1.done && s1.ok && !s1.uniform;
    double* qd = (double*)hw;
    if (act0 && act1 && s0.nm + s1.nm <= 64) {
        resolve_lanes<D, P>(s0, s1, true, a, bh, lane, qd, ml);
    } else {
        if (act0) {
            if (s0.nm <= 64)
                resolve_lanes<D, P>(s0, s0, false, a, bh, lane, qd, ml);
            else
                resolve_radix<D, P>(s0, a, bh, lane, hw, fb);
        }
        if (act1) {
            if (s1.nm <= 64)
                resolve_lanes<D, P>(s1, s1, false, a, bh, lane, qd, ml);
            else
                resolve_radix<D, P>(s1, a, bh, lane, hw, fb);
        }
    }
    if (!s0.done) output_row<P>(s0, a.nvt, lane);
    if (two && !s1.done) output_row<P>(s1, a.nvt, lane);
}

// Persistent grid of at most kSelBlocks blocks of 8 waves; item = R
// consecutive query rows of one (batch, head).  Phase 1: every wave takes
// every eighth block of 16 keys and computes the 16 x 16 float scores of the rows' 16-row block with
// three v_mfma_f32_16x16x32_bf16 per 32 channels (hi*hi, hi*lo, lo*hi), its
// next key block's operands in flight; the R wanted rows go to LDS.  Phase 2:
// one wave per row (select_row).  R * (NMAX + 4) floats of LDS hold the rows.
template <int D, int R, int NMAX>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void select_kernel(SelectArgs a) {
    constexpr int SD = D / 32;          // 32-channel k-steps
    constexpr int STRIDE = NMAX + 4;    // row stride: the 4 row groups of a store land on distinct banks
    __shared__ __attribute__((aligned(16))) float sc[R * STRIDE];
    __shared__ __attribute__((aligned(16))) uint32_t hist[kSelWaves][kWaveScratch];
    __shared__ int mlist[kSelWaves][64];
    __shared__ float red[kSelWaves];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = a.nvt;
    const int nb = (n + 15) / 16;
    const int per_bh = (n + R - 1) / R;
    const int64_t items = (int64_t)a.BH * per_bh;
    uint64_t* fb = a.scratch + ((int64_t)blockIdx.x * kSelWaves + wave) * n;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int64_t bh = it / per_bh;
        const int i0 = (int)(it % per_bh) * R;
        __syncthreads();  // the previous item's rows and red[] are no longer read
        float km = 0.f;
        for (int j = tid; j < n; j += 64 * kSelWaves) km = fmaxf(km, a.knorm[bh * n + j]);
        km = wave_max_dpp(km);
        if (lane == 0) red[wave] = km;
        {
            const int roff = i0 % 16;
            const uint4* qs = (const uint4*)a.qsplit + (bh * nb + i0 / 16) * SD * 128 + lane;
            const uint4* ks = (const uint4*)a.ksplit + bh * nb * SD * 128 + lane;
            bf16x8 qa[SD][2], ka[SD][2], kb[SD][2];
#pragma unroll
            for (int s2 = 0; s2 < SD; ++s2)
#pragma unroll
                for (int p = 0; p < 2; ++p) qa[s2][p] = __builtin_bit_cast(bf16x8, qs[(2 * s2 + p) * 64]);
            auto load = [&](bf16x8 (&dst)[SD][2], int jb) {
#pragma unroll
                for (int s2 = 0; s2 < SD; ++s2)
#pragma unroll
                    for (int p = 0; p < 2; ++p)
                        dst[s2][p] = __builtin_bit_cast(bf16x8, ks[((int64_t)jb * SD + s2) * 128 + p * 64]);
            };
            auto score = [&](const bf16x8 (&kv)[SD][2], int jb) {
                f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s2 = 0; s2 < SD; ++s2) {
                    c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s2][0], kv[s2][0], c0, 0, 0, 0);
                    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s2][0], kv[s2][1], c1, 0, 0, 0);
                    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s2][1], kv[s2][0], c1, 0, 0, 0);
                }
                const f32x4 c = c0 + c1;
                // lane l holds key 16 jb + l % 16 of rows 4 (l / 16) .. +3
                const int col = 16 * jb + (lane & 15);
                if (col < n) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = 4 * (lane >> 4) + r - roff;
                        if (row >= 0 && row < R) sc[row * STRIDE + col] = c[r];
                    }
                }
            };
            // the next key block's operands are loaded while this one is
            // scored; past the last block the loads repeat it (unconditional
            // loads keep the wait counts exact)
            int jb = wave;
            load(ka, min(jb, nb - 1));
            while (jb < nb) {
                int jn = jb + kSelWaves;
                load(kb, min(jn, nb - 1));
                score(ka, jb);
                jb = jn;
                if (jb >= nb) break;
                jn = jb + kSelWaves;
                load(ka, min(jn, nb - 1));
                score(kb, jb);
                jb = jn;
            }
        }
        __syncthreads();
        float kmax = red[0];
#pragma unroll
        for (int w = 1; w < kSelWaves; ++w) kmax = fmaxf(kmax, red[w]);
        // one wave per row, or per pair of rows (R = 16: rows w and w + 8)
        const int r0 = wave, r1 = wave + kSelWaves;
        if (r0 < R && i0 + r0 < n) {
            const bool two = r1 < R && i0 + r1 < n;
            select_rows<D, NMAX / 64>(a, sc + r0 * STRIDE, sc + (two ? r1 : r0) * STRIDE, i0 + r0, i0 + r1, two, bh,
                                      kmax, lane, hist[wave], mlist[wave], fb);
        }
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

hipError_t launch_pool(const uint16_t* q_tiled, const uint16_t* k_frag, const PoolOut& q, const PoolOut& k, int BH,
                       int n_prefix, int nvt, int D, hipStream_t s, const PadGeo& pad) {
    const int64_t tiles = 2LL * BH * nvt;
    if (tiles == 0) return hipSuccess;
    const dim3 grid((unsigned)((tiles + 3) / 4));
    if (D == 128)
        hipLaunchKernelGGL(pool_kernel<128>, grid, dim3(256), 0, s, (const uint4*)q_tiled, (const uint4*)k_frag, q,
                           k, BH, n_prefix, nvt, pad);
    else
        hipLaunchKernelGGL(pool_kernel<64>, grid, dim3(256), 0, s, (const uint4*)q_tiled, (const uint4*)k_frag, q,
                           k, BH, n_prefix, nvt, pad);
    return hipGetLastError();
}

size_t select_scratch_bytes(int nvt) { return (size_t)kSelBlocks * kSelWaves * (size_t)nvt * sizeof(uint64_t); }

template <int D>
static hipError_t launch_select_d(const SelectArgs& a, hipStream_t s) {
    // rows per item: as many as LDS holds for this many keys
    auto go = [&](auto kern, int R) {
        const int64_t items = (int64_t)a.BH * ((a.nvt + R - 1) / R);
        const unsigned grid = (unsigned)(items < kSelBlocks ? items : kSelBlocks);
        hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * kSelWaves), 0, s, a);
        return hipGetLastError();
    };
    if (a.nvt <= 2176) return go(select_kernel<D, 16, 2176>, 16);
    if (a.nvt <= 4352) return go(select_kernel<D, 8, 4352>, 8);
    return go(select_kernel<D, 4, 8704>, 4);
}

hipError_t launch_select(const SelectArgs& a, int D, hipStream_t s) {
    if ((int64_t)a.BH * a.nvt == 0) return hipSuccess;
    return D == 128 ? launch_select_d<128>(a, s) : launch_select_d<64>(a, s);
}

}  // namespace bsa
