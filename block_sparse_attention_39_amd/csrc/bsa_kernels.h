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

// -inf for the padding keys among one lane's 16 elements of an S^T
// accumulator of a 32-key half kh, given the class's 64-bit mask of real
// keys.  The kfrag token order (swap23) puts key 32*kh + 16*c + 8*hf + e at
// element 8*c + e of lane-half hf.
template <class V>
__device__ __attribute__((always_inline)) inline void mask_padding_keys(uint64_t real, int kh, int hf, V& sv) {
    const uint32_t half = kh ? (uint32_t)(real >> 32) : (uint32_t)real;
    const uint32_t x = half >> (8 * hf);
    const uint32_t bits = (x & 0xffu) | ((x >> 8) & 0xff00u);  // bit r: element r is a real key
#pragma unroll
    for (int r = 0; r < 16; ++r)
        if (!((bits >> r) & 1u)) sv[r] = -__builtin_inff();
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

// Mean of the 64 tokens of every video tile of Q (tiled) and K (K-fragment
// layout) -> float [BH][nvt][D].
// Tile means: the sum of the tile's real tokens / their number (64 unless
// `pad` marks the tile as a padded boundary tile).
hipError_t launch_pool(const uint16_t* q_tiled, const uint16_t* k_frag, float* qbar, float* kbar, int BH,
                       int n_prefix, int nvt, int D, hipStream_t s, const PadGeo& pad = PadGeo{});

// scores[bh][i][j] = qbar_i . kbar_j (float) for bh in [0, BH).
hipError_t launch_scores(const float* qbar, const float* kbar, float* scores, int BH, int n, int D,
                         hipStream_t s);

// Per row: the k largest scores (lower index first on ties), ascending indices.
hipError_t launch_topk(const float* scores, int32_t* idx, int rows, int n, int k, hipStream_t s);

// Variable keep: per-head keep counts (kernel argument), per-row counts
// (device, optional), CSR row pointers and the per-row top-k.
struct CsrKeep {
    int32_t k[BSA_MAX_CSR_HEADS];
};
hipError_t launch_csr_rowptr(const CsrKeep& kh, const int32_t* keep_rows, int BH, int H, int nvt, int64_t* row_ptr,
                             hipStream_t s);
hipError_t launch_topk_csr(const float* scores, int32_t* col_idx, const int64_t* row_ptr, int64_t row0, int rows,
                           int n, hipStream_t s);

// Structured lists: per head a mask kind (BSA_MASK_*), the tile grid and the
// radii; row pointers and the ascending lists of every row.
struct StructRule {
    int32_t kind[BSA_MAX_CSR_HEADS];
    int Tt, Th, Tw, rt, rs;
};
hipError_t launch_structured(const StructRule& sr, int BH, int H, int64_t* row_ptr, int32_t* col, hipStream_t s);

struct ForwardArgs {
    const uint16_t* q;       // tiled [BH][Ntot][D]
    const uint16_t* k;       // K-fragment layout [BH][Ntot/64][2][D/16][64][8]
    const uint16_t* v;       // V-fragment layout [BH][Ntot/64][2][D/32][2][64][8]
    const int32_t* idx;      // [BH][nvt][keep], or CSR column indices when row_ptr is set
    const int64_t* row_ptr;  // CSR row pointers [BH * nvt + 1], or null (fixed keep)
    int64_t col_entries;     // CSR: entries of idx (list bounds are clamped to it)
    PadGeo pad;              // ragged grid: padding keys of boundary tiles are masked
    uint16_t* o;             // tiled [BH][Ntot][D]
    float* lse;              // [BH][Ntot] or null
    int BH;
    int npt;                 // prefix tiles
    int nvt;                 // video tiles
    int keep;                // kept video tiles per video query tile
    float scale_log2;        // scale * log2(e)
};
// progress: forward_workspace_bytes() of device memory for the grouped launch
// of the video query tiles, or null for one block per query tile.
size_t forward_workspace_bytes();
hipError_t launch_forward(const ForwardArgs& a, int D, int* progress, hipStream_t s);

struct BackwardArgs {
    // fragment layouts of the tiled tensors (kfrag / vfrag of the C interface)
    const uint16_t *q_kf, *do_kf, *k_kf, *v_kf, *k_vf;
    const uint16_t *q_t, *do_t;  // tiled [BH][Ntot][D]
    const uint16_t *o, *dout;  // raster [B][Ntot][H][D]
    const float* lse;          // [BH][Ntot] natural log, tiled order
    const int32_t* idx;        // [BH][nvt][keep], or CSR column indices when row_ptr is set
    const int64_t* row_ptr;    // CSR row pointers [BH * nvt + 1], or null (fixed keep)
    int64_t col_entries;       // CSR: entries of idx (list bounds are clamped to it)
    const int32_t* perm;       // [B][Nvideo], -1 for a padding slot
    float *lse2, *delta;       // [BH][Ntot] scratch: lse * log2 e, dO . O
    float *nlse, *ndelta;      // [BH][Ntot] scratch: -lse / scale, -(dO . O)
    uint32_t* mask;            // [BH][nvt][mwords] scratch
    int32_t* cnt;              // [BH][nvt] scratch: query tiles that kept each key tile
    int64_t* rowp;             // [BH * nvt + 1] scratch: exclusive prefix sums of cnt
    int32_t* tlist;            // [tcap] scratch: the transposed lists, (bh, key tile) order
    int64_t tcap;              // entries of tlist
    uint16_t *dq, *dk, *dv;    // raster [B][Ntot][H][D]
    int* progress;             // backward_progress_ints() ints: grouped-launch round counters
    int BH, H, npt, nvt, keep, mwords;
    int64_t npf, n_tot;        // tiled rows per (b, h): prefix + video slots
    int64_t n_ras;             // raster rows per batch element (fewer on a ragged grid)
    PadGeo pad;                // ragged grid (pad.T != 0): perm -1 marks padding slots
    float scale, scale_log2;
};
constexpr int backward_progress_ints() { return 8 * 64; }
hipError_t launch_backward(const BackwardArgs& a, int D, hipStream_t s);

}  // namespace bsa
