// Internal launchers of libbsa.so (not part of the C ABI).  Each returns the
// HIP error of its launch; all sizes were validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

#include "bsa.h"

namespace bsa {

constexpr int kTile = 64;  // tokens per tile

// A ragged video grid padded up to whole static tiles: the real extents, the
// tile extents and the tile counts per axis.  T == 0: no padding (every tile
// full).  Tile (ti, hi, wi) is video tile (ti*Th + hi)*Tw + wi; its token
// (lt, lh, lw) (raster inside the tile) is real iff ti*tt + lt < T,
// hi*th + lh < Hg and wi*tw + lw < W.  real[c]: bit j set iff token j of a
// tile of boundary class c is real, class bit 2/1/0 meaning the tile is the
// last along t/h/w on an axis cut short (make_pad_geo fills it).
struct PadGeo {
    int T, Hg, W;
    int tt, th, tw;
    int Tt, Th, Tw;
    uint64_t real[8];
};

inline PadGeo make_pad_geo(int T, int Hg, int W, int tt, int th, int tw) {
    PadGeo g{};
    g.T = T, g.Hg = Hg, g.W = W, g.tt = tt, g.th = th, g.tw = tw;
    g.Tt = (T + tt - 1) / tt, g.Th = (Hg + th - 1) / th, g.Tw = (W + tw - 1) / tw;
    for (int c = 0; c < 8; ++c) {
        const int nt = (c & 4) ? T - (g.Tt - 1) * tt : tt;
        const int nh = (c & 2) ? Hg - (g.Th - 1) * th : th;
        const int nw = (c & 1) ? W - (g.Tw - 1) * tw : tw;
        for (int j = 0; j < kTile; ++j) {
            const int lt = j / (th * tw), lh = (j / tw) % th, lw = j % tw;
            if (lt < nt && lh < nh && lw < nw) g.real[c] |= uint64_t(1) << j;
        }
    }
    return g;
}

// Ragged grids in the attention kernels: a tile list staged in LDS carries,
// above the tile number, the boundary class of a video key tile (0: no
// padding slot), and the padding keys of a boundary tile get -inf logits.
constexpr int kTileBits = 0xFFFF;  // tile numbers are below BSA_MAX_TILES <= 2^16

// boundary class of video tile vt, shifted above the tile number
__device__ inline int pad_class(const PadGeo& g, int vt) {
    const int wi = vt % g.Tw, hi = (vt / g.Tw) % g.Th, ti = vt / (g.Tw * g.Th);
    return (((ti + 1) * g.tt > g.T) << 2 | ((hi + 1) * g.th > g.Hg) << 1 | ((wi + 1) * g.tw > g.W)) << 16;
}

// The real keys among one lane's 16 elements of an S^T accumulator of a
// 32-key half kh, given the class's 64-bit mask of real keys: bit r set when
// element r is a real key.  The kfrag token order (swap23) puts key
// 32*kh + 16*c + 8*hf + e at element 8*c + e of lane-half hf.
__device__ inline uint32_t real_key_bits(uint64_t real, int kh, int hf) {
    const uint32_t half = kh ? (uint32_t)(real >> 32) : (uint32_t)real;
    const uint32_t x = half >> (8 * hf);
    return (x & 0xffu) | ((x >> 8) & 0xff00u);
}

// -inf for the elements whose bit is clear: per element a sign-extended bit
// (0 or all ones) selects between the value and -inf bit by bit.
template <class V>
__device__ __attribute__((always_inline)) inline void mask_keys_by_bits(uint32_t bits, V& sv) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)bits, r, 1);
        sv[r] = __uint_as_float((__float_as_uint(sv[r]) & m) | (0xff800000u & ~m));
    }
}

template <class V>
__device__ __attribute__((always_inline)) inline void mask_padding_keys(uint64_t real, int kh, int hf, V& sv) {
    mask_keys_by_bits(real_key_bits(real, kh, hf), sv);
}

// Static tile order: perm[b][p] for all b (the same closed form per batch).
hipError_t launch_perm_static(int B, int T, int Hg, int W, int tt, int th, int tw, int32_t* perm,
                              hipStream_t s);

// Raster [B][n_prefix + n_raster_video][H][D] <-> tiled [B][H][n_prefix + n_video][D]
// through perm (prefix kept in place; perm -1 marks a padding slot: gathered
// as zeros, not scattered).  n_raster_video < 0: the same as n_video.
hipError_t launch_permute_copy(bool to_raster, const uint16_t* src, uint16_t* dst, const int32_t* perm,
                               int B, int H, int D, int n_prefix, int64_t n_video, hipStream_t s,
                               int64_t n_raster_video = -1);

// Raster [B][Ntot][H][D] -> the K-fragment and V-fragment layouts (kfrag, vfrag
// of the C interface): the tiled order with every 64-token tile laid out in
// the operand order of the attention kernel's MFMAs.
hipError_t launch_gather_kf(const uint16_t* src, uint16_t* dst, const int32_t* perm, int B, int H, int D,
                            int n_prefix, int64_t n_video, hipStream_t s, int64_t n_raster_video = -1);
hipError_t launch_gather_vf(const uint16_t* src, uint16_t* dst, const int32_t* perm, int B, int H, int D,
                            int n_prefix, int64_t n_video, hipStream_t s, int64_t n_raster_video = -1);

// Dynamic shapes: per-(b, region, head) partial |delta| sums, then shape choice
// and the permutation.
hipError_t launch_shape_stats(const uint16_t* q_raster, double* partial, int B, int H, int D, int n_prefix,
                              int T, int Hg, int W, hipStream_t s);
hipError_t launch_shape_choose(const double* partial, uint8_t* shape_map, int B, int H, int D, int T, int Hg,
                               int W, float tau, hipStream_t s);
hipError_t launch_perm_dynamic(const uint8_t* shape_map, int32_t* perm, int B, int T, int Hg, int W,
                               hipStream_t s);

// Pooled tile means and what the selection reads of them.  For every video
// tile i of every (batch, head) bh:
//   mean  float [BH][nvt][D]: the mean of the tile's tokens (of its real tokens
//         on a ragged grid), the exact sum rounded once to float;
//   split bf16 [BH][ceil(nvt/16)][D/32][2][64][8]: the same means as a pair of
//         bf16 values (hi = bf16(m), lo = bf16(m - hi)), in the operand order of
//         v_mfma_f32_16x16x32_bf16: in the 1 KB chunk (bh, row block i/16, k-step
//         s, part), lane i%16 + 16*g holds channels 32*s + 8*g .. +7 of row i;
//   norm  float [BH][nvt]: the Euclidean norm of the float mean.
struct PoolOut {
    float* mean;
    uint16_t* split;
    float* norm;
};

__device__ inline uint32_t bf16_rne_bits(float x) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    const bf2 b = __builtin_convertvector((f2){x, x}, bf2);
    return __builtin_bit_cast(uint32_t, b) & 0xffffu;
}

// Store the means of channels 8c .. 8c+7 of video tile i of bh: float, the
// bf16 hi/lo split, and return the sum of their squares (for the norm).
__device__ inline float store_pooled8(const PoolOut& po, int64_t bh, int nvt, int D, int64_t i, int c,
                                      const float (&m)[8]) {
    float4* mp = (float4*)(po.mean + (bh * nvt + i) * D + 8 * c);
    mp[0] = make_float4(m[0], m[1], m[2], m[3]);
    mp[1] = make_float4(m[4], m[5], m[6], m[7]);
    uint32_t hi[4], lo[4];
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const uint32_t h0 = bf16_rne_bits(m[e]), h1 = bf16_rne_bits(m[e + 1]);
        const uint32_t l0 = bf16_rne_bits(m[e] - __uint_as_float(h0 << 16));
        const uint32_t l1 = bf16_rne_bits(m[e + 1] - __uint_as_float(h1 << 16));
        hi[e / 2] = h0 | (h1 << 16);
        lo[e / 2] = l0 | (l1 << 16);
        sq = fmaf(m[e], m[e], sq);
        sq = fmaf(m[e + 1], m[e + 1], sq);
    }
    const int64_t nb = (nvt + 15) / 16, sd = D / 32;
    const int64_t chunk = ((bh * nb + i / 16) * sd + c / 4) * 2 * 64 + (i % 16) + 16 * (c % 4);
    uint4* sp = (uint4*)po.split;
    sp[chunk] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    sp[chunk + 64] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    return sq;
}

// Mean of the tokens of every video tile of Q (tiled) and K (K-fragment
// layout): the exact sum of the tile's real tokens / their number (64 unless
// `pad` marks the tile as a padded boundary tile), into PoolOut q and k.
hipError_t launch_pool(const uint16_t* q_tiled, const uint16_t* k_frag, const PoolOut& q, const PoolOut& k, int BH,
                       int n_prefix, int nvt, int D, hipStream_t s, const PadGeo& pad = PadGeo{});

// Gather with pooling: raster [B][Ntot][H][D] -> tiled (kfrag false) or the
// K-fragment layout (kfrag true) through perm, and the tile means of every
// video tile into `po` (as launch_pool writes them).
hipError_t launch_gather_pool(bool kfrag, const uint16_t* src, uint16_t* dst, const int32_t* perm, int B, int H,
                              int D, int n_prefix, int64_t n_video, const PoolOut& po, hipStream_t s,
                              int64_t n_raster_video = -1);

// The tile means of the video tiles of raster Q alone (no copy), read through
// perm, into `po` exactly as launch_gather_pool writes them.
hipError_t launch_pool_raster(const uint16_t* src, const int32_t* perm, int B, int H, int D, int n_prefix,
                              int64_t n_video, const PoolOut& po, hipStream_t s, int64_t n_raster_video = -1);

// The backward's per-row quantities, taken while dO is gathered: Delta =
// dO . O (O raster), and the forward's lse as lse * log2 e and -lse / scale
// (+inf and -inf on a padding row, whose Delta is 0), all [B*H][Ntot] in the
// tiled row order.
struct DeltaOut {
    const uint16_t* o;
    const float* lse;
    float *delta, *ndelta, *lse2, *nlse;
    float scale;
};
// Raster -> the K-fragment layout and the tiled layout in one read (Q, or dO
// with `dl` set: then also the per-row quantities above).
hipError_t launch_gather_kf_tiled(const uint16_t* src, uint16_t* dst_kf, uint16_t* dst_t, const int32_t* perm, int B,
                                  int H, int D, int n_prefix, int64_t n_video, hipStream_t s, int64_t n_raster_video,
                                  const DeltaOut* dl);
// Raster -> the K-fragment and the V-fragment layouts in one read (K).
hipError_t launch_gather_kf_vf(const uint16_t* src, uint16_t* dst_kf, uint16_t* dst_vf, const int32_t* perm, int B,
                               int H, int D, int n_prefix, int64_t n_video, hipStream_t s, int64_t n_raster_video);

// Tiled [B][H][Ntot][D] -> the K-fragment (kfrag true) or V-fragment layout.
hipError_t launch_tiled_to_frag(bool kfrag, const uint16_t* src, uint16_t* dst, int B, int H, int D, int64_t n_tot,
                                hipStream_t s);

// Selection from the pooled means: per row (bh, i), the k video key tiles j of
// largest s_ij = qbar_i . kbar_j (the sum taken in double), lower j first on
// equal scores, ascending.  Fixed keep (row_ptr null): k_fixed entries per row
// at idx + row * k_fixed; CSR: row r keeps row_ptr[r+1] - row_ptr[r] entries
// written at idx + row_ptr[r].  `scratch`: select_scratch_bytes(nvt) bytes.
struct SelectArgs {
    const float* qbar;
    const float* kbar;
    const uint16_t* qsplit;
    const uint16_t* ksplit;
    const float* qnorm;
    const float* knorm;
    int32_t* idx;
    const int64_t* row_ptr;
    int k_fixed;
    int BH;
    int nvt;
    uint64_t* scratch;
};
size_t select_scratch_bytes(int nvt);
hipError_t launch_select(const SelectArgs& a, int D, hipStream_t s);

// Variable keep: per-head keep counts (kernel argument), per-row counts
// (device, optional), CSR row pointers and the per-row top-k.
struct CsrKeep {
    int32_t k[BSA_MAX_CSR_HEADS];
};
hipError_t launch_csr_rowptr(const CsrKeep& kh, const int32_t* keep_rows, int BH, int H, int nvt, int64_t* row_ptr,
                             hipStream_t s);

// Structured lists: per head a mask kind (BSA_MASK_*), the tile grid and the
// radii; row pointers and the ascending lists of every row.
struct StructRule {
    int32_t kind[BSA_MAX_CSR_HEADS];
    int Tt, Th, Tw, rt, rs;
};
hipError_t launch_structured(const StructRule& sr, int BH, int H, int64_t* row_ptr, int32_t* col, hipStream_t s);

struct ForwardArgs {
    const uint16_t* q;       // tiled [BH][Ntot][D], or raster [B][n_ras][H][D] (raster)
    const uint16_t* k;       // K-fragment layout [BH][Ntot/64][2][D/16][64][8]
    const uint16_t* v;       // V-fragment layout [BH][Ntot/64][2][D/32][2][64][8]
    const int32_t* idx;      // [BH][nvt][keep], or CSR column indices when row_ptr is set
    const int64_t* row_ptr;  // CSR row pointers [BH * nvt + 1], or null (fixed keep)
    int64_t col_entries;     // CSR: entries of idx (list bounds are clamped to it)
    PadGeo pad;              // ragged grid: padding keys of boundary tiles are masked
    uint16_t* o;             // tiled [BH][Ntot][D], or raster [B][n_ras][H][D] (raster)
    float* lse;              // [BH][Ntot] or null
    bool raster;             // Q and O in the raster layout, through perm
    const int32_t* perm;     // raster: tiled video slot -> raster video token [B][nvt*64]
                             // (-1: padding slot)
    int64_t n_ras;           // raster rows per batch element (prefix + real video tokens)
    int H;                   // heads (the raster layout interleaves them)
    int BH;
    int npt;                 // prefix tiles
    int nvt;                 // video tiles
    int keep;                // kept video tiles per video query tile
    float scale_log2;        // scale * log2(e)
};
// progress: forward_workspace_bytes() of device memory for the grouped launch
// of the video query tiles, or null for one block per query tile.
// After the counters: int stats[2] (rounds whose start wait gave up, rounds
// started), cleared with them at the start of every grouped launch.
size_t forward_workspace_bytes();
size_t forward_stats_offset();
hipError_t launch_forward(const ForwardArgs& a, int D, int* progress, hipStream_t s);
// The grouped launch with its counters in a file-scope device array (one per
// GPU, forward_scratch_bytes() long) instead of a workspace: allocates nothing.
size_t forward_scratch_bytes();
hipError_t launch_forward_noalloc(const ForwardArgs& a, int D, hipStream_t s);

struct BackwardArgs {
    // fragment layouts of the tiled tensors (kfrag / vfrag of the C interface)
    const uint16_t *q_kf, *do_kf, *k_kf, *v_kf, *k_vf;
    const uint16_t *q_t, *do_t;  // tiled [BH][Ntot][D]
    const int32_t* idx;        // [BH][nvt][keep], or CSR column indices when row_ptr is set
    const int64_t* row_ptr;    // CSR row pointers [BH * nvt + 1], or null (fixed keep)
    int64_t col_entries;       // CSR: entries of idx (list bounds are clamped to it)
    const int32_t* perm;       // [B][Nvideo], -1 for a padding slot
    float *lse2, *delta;       // [BH][Ntot] scratch: lse * log2 e, dO . O
    float *nlse, *ndelta;      // [BH][Ntot] scratch: -lse / scale, -(dO . O)
    unsigned long long* mask;  // [BH][mchunks][nvt] scratch: bit q of [bh][c][j]: query tile 64c + q kept j
    int32_t* cnt;              // [BH][nvt] scratch: query tiles that kept each key tile
    int64_t* rowp;             // [BH * nvt + 1] scratch: exclusive prefix sums of cnt
    int32_t* tlist;            // [tcap] scratch: the transposed lists, (bh, key tile) order
    int64_t tcap;              // entries of tlist
    uint16_t *dq, *dk, *dv;    // raster [B][Ntot][H][D]
    int* progress;             // backward_progress_ints() ints: grouped-launch round counters,
                               // then 4 statistics (backward_stats_ints())
    int BH, H, npt, nvt, keep, mchunks;
    int64_t npf, n_tot;        // tiled rows per (b, h): prefix + video slots
    int64_t n_ras;             // raster rows per batch element (fewer on a ragged grid)
    PadGeo pad;                // ragged grid (pad.T != 0): perm -1 marks padding slots
    float scale, scale_log2;
};
// the round counters of the grouped gradient launches (8 groups of up to 64
// blocks), then int32 stats[4]: dQ round-start waits that gave up, dQ block
// rounds started, the same two for dK/dV
constexpr int backward_stats_ints() { return 8 * 64; }
constexpr int backward_progress_ints() { return 8 * 64 + 4; }
hipError_t launch_backward(const BackwardArgs& a, int D, hipStream_t s);

}  // namespace bsa
