// The C ABI of libbsa.so (declared in include/bsa.h): host-side validation of
// every argument, workspace layout, and the kernel launches in order.
// Validation runs entirely on the host and returns before any HIP call, so a
// rejected call enqueues nothing.
#include "bsa.h"

#include <algorithm>
#include <cmath>
#include <initializer_list>
#include <cstdint>

#include "bsa_kernels.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// n_video: video tokens of the tiled layouts (padding slots included);
// n_ras: video tokens of the raster layouts.  They differ only for a ragged
// grid padded to whole tiles, which `pad` then describes (pad.T == 0 otherwise).
struct Geo {
    int64_t B, H, D, T, Hg, W, npf, n_video, n_ras, n_tot, nvt, npt, BH, k, regions;
    int64_t Tt, Th, Tw;  // static tile grid (tiles per axis)
    bool dynamic;
    bool padded;
    bool empty;
    bsa::PadGeo pad;
};

bool misaligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

// true when the byte ranges [p, p + pb) and [q, q + qb) intersect
bool overlaps(const void* p, size_t pb, const void* q, size_t qb) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return p && q && pb > 0 && qb > 0 && a < b + qb && b < a + pb;
}

// A byte range of a call's argument (null or empty: none).
struct Span {
    const void* p;
    size_t bytes;
};

// True if an output range meets another output or any input range.
bool clash(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
    for (auto o = outs.begin(); o != outs.end(); ++o) {
        for (auto o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlaps(o->p, o->bytes, o2->p, o2->bytes)) return true;
        for (const Span& i : ins)
            if (overlaps(o->p, o->bytes, i.p, i.bytes)) return true;
    }
    return false;
}

bsa_status check_desc(const bsa_desc* d, Geo* g) {
    if (!d) return BSA_ERR_NULL;
    if (d->batch < 0 || d->heads < 0 || d->grid_t < 0 || d->grid_h < 0 || d->grid_w < 0 || d->n_prefix < 0)
        return BSA_ERR_SHAPE;
    if (d->head_dim != 64 && d->head_dim != 128) return BSA_ERR_UNSUPPORTED;
    if (d->n_prefix % bsa::kTile) return BSA_ERR_SHAPE;
    if (!std::isfinite(d->scale) || !(d->scale > 0.f)) return BSA_ERR_ARG;
    g->B = d->batch;
    g->H = d->heads;
    g->D = d->head_dim;
    g->T = d->grid_t;
    g->Hg = d->grid_h;
    g->W = d->grid_w;
    g->npf = d->n_prefix;
    g->n_ras = g->T * g->Hg * g->W;
    g->n_video = g->n_ras;
    g->dynamic = g->padded = false;
    g->pad = bsa::PadGeo{};
    g->Tt = g->Th = g->Tw = 0;
    if (d->tile_mode == BSA_TILE_STATIC || d->tile_mode == BSA_TILE_STATIC_PADDED) {
        if (d->tile_t < 1 || d->tile_h < 1 || d->tile_w < 1) return BSA_ERR_SHAPE;
        if ((int64_t)d->tile_t * d->tile_h * d->tile_w != bsa::kTile) return BSA_ERR_SHAPE;
        g->Tt = (g->T + d->tile_t - 1) / d->tile_t;
        g->Th = (g->Hg + d->tile_h - 1) / d->tile_h;
        g->Tw = (g->W + d->tile_w - 1) / d->tile_w;
        if (d->tile_mode == BSA_TILE_STATIC) {
            if (g->T % d->tile_t || g->Hg % d->tile_h || g->W % d->tile_w) return BSA_ERR_SHAPE;
        } else {
            g->n_video = g->Tt * g->Th * g->Tw * bsa::kTile;
            g->padded = g->n_video != g->n_ras;
            if (g->padded)
                g->pad = bsa::make_pad_geo((int)g->T, (int)g->Hg, (int)g->W, d->tile_t, d->tile_h, d->tile_w);
        }
    } else if (d->tile_mode == BSA_TILE_DYNAMIC) {
        g->dynamic = true;
        if (g->T % 8 || g->Hg % 8 || g->W % 8) return BSA_ERR_SHAPE;
        if (!std::isfinite(d->dyn_tau) || d->dyn_tau < 0.f) return BSA_ERR_ARG;
    } else {
        return BSA_ERR_ARG;
    }
    g->n_tot = g->npf + g->n_video;
    g->nvt = g->n_video / bsa::kTile;
    g->npt = g->npf / bsa::kTile;
    g->BH = g->B * g->H;
    g->regions = (g->T / 8) * (g->Hg / 8) * (g->W / 8);
    g->k = d->keep_tiles;
    if (g->nvt > 0 && (g->k < 1 || g->k > g->nvt)) return BSA_ERR_SHAPE;
    // index arithmetic limits: block counts and per-tensor element counts
    if (g->BH * (g->npt + g->nvt) > INT32_MAX) return BSA_ERR_UNSUPPORTED;
    if (g->n_tot > INT32_MAX / 2) return BSA_ERR_UNSUPPORTED;
    g->empty = (g->BH == 0 || g->n_tot == 0);
    return BSA_OK;
}

struct Layout {
    size_t qbar, kbar, qsplit, ksplit, qnorm, knorm, sel, partial, fwd, total;
};

// Workspace of bsa_plan / bsa_select / bsa_forward / the pooling gathers:
// the float means of Q and K (documented at the front), their bf16 hi/lo
// split in MFMA operand order and their norms, the selection's fallback
// scratch, then the forward's group counters and statistics.  The dynamic
// BUILD's partial sums reuse the front (they are consumed within BUILD).
Layout layout(const Geo& g) {
    Layout L{};
    const size_t pooled = align_up((size_t)g.BH * g.nvt * g.D * sizeof(float));
    const size_t split = align_up((size_t)g.BH * ((g.nvt + 15) / 16) * 16 * g.D * 2 * sizeof(uint16_t));
    const size_t norms = align_up((size_t)g.BH * g.nvt * sizeof(float));
    size_t o = 0;
    L.qbar = o;
    o += pooled;
    L.kbar = o;
    o += pooled;
    L.qsplit = o;
    o += split;
    L.ksplit = o;
    o += split;
    L.qnorm = o;
    o += norms;
    L.knorm = o;
    o += norms;
    L.sel = o;
    o += align_up(g.nvt > 0 ? bsa::select_scratch_bytes((int)g.nvt) : 0);
    const size_t plan_bytes = (g.nvt > 0 && g.BH > 0) ? o : 0;
    const size_t build_bytes = g.dynamic ? align_up((size_t)g.B * g.regions * g.H * 3 * sizeof(double)) : 0;
    L.partial = 0;
    // the forward's block-group progress counters sit after the plan's region,
    // so the pooled means stay readable after a forward call
    L.fwd = align_up(plan_bytes);
    const size_t fwd_end = L.fwd + align_up(bsa::forward_workspace_bytes());
    L.total = fwd_end > build_bytes ? fwd_end : build_bytes;
    return L;
}

struct PoolPair {
    bsa::PoolOut q, k;
};
PoolPair pool_outs(const Layout& L, void* ws) {
    char* w = static_cast<char*>(ws);
    PoolPair p;
    p.q = {reinterpret_cast<float*>(w + L.qbar), reinterpret_cast<uint16_t*>(w + L.qsplit),
           reinterpret_cast<float*>(w + L.qnorm)};
    p.k = {reinterpret_cast<float*>(w + L.kbar), reinterpret_cast<uint16_t*>(w + L.ksplit),
           reinterpret_cast<float*>(w + L.knorm)};
    return p;
}

bsa::SelectArgs select_args(const Geo& g, const Layout& L, void* ws, int32_t* idx, const int64_t* row_ptr) {
    const PoolPair p = pool_outs(L, ws);
    bsa::SelectArgs a{};
    a.qbar = p.q.mean;
    a.kbar = p.k.mean;
    a.qsplit = p.q.split;
    a.ksplit = p.k.split;
    a.qnorm = p.q.norm;
    a.knorm = p.k.norm;
    a.idx = idx;
    a.row_ptr = row_ptr;
    a.k_fixed = (int)g.k;
    a.BH = (int)g.BH;
    a.nvt = (int)g.nvt;
    a.scratch = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + L.sel);
    return a;
}

bsa_status launched(hipError_t e) { return e == hipSuccess ? BSA_OK : BSA_ERR_LAUNCH; }

// Workspace of bsa_backward: five fragment-layout and two tiled copies, then the
// per-row lse (base 2) and Delta and their negated forms, then the transposed
// lists.
struct BwdLayout {
    size_t frag[7], lse2, delta, nlse, ndelta, mask, cnt, rowp, tlist, progress, total;
    int mchunks;
};

// tcap: entries of the transposed lists (B*H*nVT*k for fixed keep, the CSR
// column count for variable lists)
BwdLayout bwd_layout(const Geo& g, int64_t tcap) {
    BwdLayout L{};
    const size_t t = align_up((size_t)g.BH * g.n_tot * g.D * 2);
    size_t o = 0;
    for (int i = 0; i < 7; ++i, o += t) L.frag[i] = o;
    L.lse2 = o;
    o += align_up((size_t)g.BH * g.n_tot * sizeof(float));
    L.delta = o;
    o += align_up((size_t)g.BH * g.n_tot * sizeof(float));
    L.nlse = o;
    o += align_up((size_t)g.BH * g.n_tot * sizeof(float));
    L.ndelta = o;
    o += align_up((size_t)g.BH * g.n_tot * sizeof(float));
    L.mchunks = (int)((g.nvt + 63) / 64);
    L.mask = o;
    o += align_up((size_t)g.BH * L.mchunks * g.nvt * sizeof(uint64_t));
    L.cnt = o;
    o += align_up((size_t)g.BH * g.nvt * sizeof(int32_t));
    L.rowp = o;
    o += align_up((size_t)(g.BH * g.nvt + 1) * sizeof(int64_t));
    L.tlist = o;
    o += align_up((size_t)tcap * sizeof(int32_t));
    L.progress = o;
    o += align_up((size_t)bsa::backward_progress_ints() * sizeof(int));
    L.total = o;
    return L;
}

}  // namespace

extern "C" {

int bsa_version(void) { return BSA_VERSION; }

const char* bsa_status_string(bsa_status s) {
    switch (s) {
        case BSA_OK: return "ok";
        case BSA_ERR_NULL: return "a required pointer is NULL";
        case BSA_ERR_SHAPE: return "inconsistent sizes (grid, tile, prefix or keep_tiles)";
        case BSA_ERR_UNSUPPORTED: return "unsupported size (head_dim must be 64 or 128; too many tiles)";
        case BSA_ERR_ALIGN: return "a tensor pointer is not suitably aligned";
        case BSA_ERR_WORKSPACE: return "workspace missing or too small";
        case BSA_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
        case BSA_ERR_ARG: return "invalid argument (enum value, scale, tau or radius; or an output overlapping an input)";
    }
    return "unknown status";
}

bsa_status bsa_workspace_size(const bsa_desc* desc, size_t* bytes) {
    if (!bytes) return BSA_ERR_NULL;
    Geo g;
    const bsa_status st = check_desc(desc, &g);
    if (st != BSA_OK) return st;
    *bytes = layout(g).total;
    return BSA_OK;
}

bsa_status bsa_permute(const bsa_desc* desc, int op, const void* q_raster, int32_t* perm, uint8_t* shape_map,
                       const void* src, void* dst, void* ws, size_t ws_bytes, void* stream) {
    Geo g;
    bsa_status st = check_desc(desc, &g);
    if (st != BSA_OK) return st;
    if (op < BSA_PERM_BUILD || op > BSA_PERM_POOL) return BSA_ERR_ARG;
    if (g.B == 0 || g.n_tot == 0) return BSA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (op == BSA_PERM_BUILD) {
        if (g.n_ras == 0) return BSA_OK;
        if (!perm) return BSA_ERR_NULL;
        if (misaligned(perm, 4)) return BSA_ERR_ALIGN;
        if (!g.dynamic)
            return launched(bsa::launch_perm_static((int)g.B, (int)g.T, (int)g.Hg, (int)g.W, desc->tile_t,
                                                    desc->tile_h, desc->tile_w, perm, s));
        if (g.H == 0) return BSA_ERR_SHAPE;  // the statistic needs at least one head
        if (!q_raster || !shape_map) return BSA_ERR_NULL;
        if (misaligned(q_raster, 16)) return BSA_ERR_ALIGN;
        const Layout L = layout(g);
        if (!ws || ws_bytes < L.total) return BSA_ERR_WORKSPACE;
        if (misaligned(ws, kAlign)) return BSA_ERR_ALIGN;
        double* partial = reinterpret_cast<double*>(static_cast<char*>(ws) + L.partial);
        hipError_t e = bsa::launch_shape_stats(static_cast<const uint16_t*>(q_raster), partial, (int)g.B, (int)g.H,
                                               (int)g.D, (int)g.npf, (int)g.T, (int)g.Hg, (int)g.W, s);
        if (e == hipSuccess)
            e = bsa::launch_shape_choose(partial, shape_map, (int)g.B, (int)g.H, (int)g.D, (int)g.T, (int)g.Hg,
                                         (int)g.W, desc->dyn_tau, s);
        if (e == hipSuccess) e = bsa::launch_perm_dynamic(shape_map, perm, (int)g.B, (int)g.T, (int)g.Hg, (int)g.W, s);
        return launched(e);
    }
    if (g.H == 0) return BSA_OK;
    const size_t tiled = (size_t)g.BH * g.n_tot * g.D * 2;
    const size_t raster = (size_t)g.B * (g.npf + g.n_ras) * g.H * g.D * 2;
    if (op == BSA_PERM_TILED_TO_KF || op == BSA_PERM_TILED_TO_VF) {
        if (!src || !dst) return BSA_ERR_NULL;
        if (misaligned(src, 16) || misaligned(dst, 16)) return BSA_ERR_ALIGN;
        if (overlaps(src, tiled, dst, tiled)) return BSA_ERR_ARG;
        return launched(bsa::launch_tiled_to_frag(op == BSA_PERM_TILED_TO_KF, static_cast<const uint16_t*>(src),
                                                  static_cast<uint16_t*>(dst), (int)g.B, (int)g.H, (int)g.D,
                                                  g.n_tot, s));
    }
    if (op == BSA_PERM_POOL) {
        if (g.n_video == 0) return BSA_OK;
        if (!src || !perm) return BSA_ERR_NULL;
        if (misaligned(src, 16) || misaligned(perm, 4)) return BSA_ERR_ALIGN;
        if (g.nvt > BSA_MAX_VIDEO_TILES) return BSA_ERR_UNSUPPORTED;
        const Layout L = layout(g);
        if (!ws || ws_bytes < L.total) return BSA_ERR_WORKSPACE;
        if (misaligned(ws, kAlign)) return BSA_ERR_ALIGN;
        return launched(bsa::launch_pool_raster(static_cast<const uint16_t*>(src), perm, (int)g.B, (int)g.H,
                                                (int)g.D, (int)g.npf, g.n_video, pool_outs(L, ws).q, s, g.n_ras));
    }
    if (!src || !dst || (g.n_video > 0 && !perm)) return BSA_ERR_NULL;
    if (misaligned(src, 16) || misaligned(dst, 16) || misaligned(perm, 4)) return BSA_ERR_ALIGN;
    const bool overlap = op == BSA_PERM_SCATTER ? overlaps(src, tiled, dst, raster) : overlaps(src, raster, dst, tiled);
    if (op == BSA_PERM_GATHER_POOL || op == BSA_PERM_GATHER_KF_POOL) {
        if (g.nvt > BSA_MAX_VIDEO_TILES) return BSA_ERR_UNSUPPORTED;
        const Layout L = layout(g);
        if (!ws || ws_bytes < L.total) return BSA_ERR_WORKSPACE;
        if (misaligned(ws, kAlign)) return BSA_ERR_ALIGN;
        if (overlap) return BSA_ERR_ARG;
        const PoolPair p = pool_outs(L, ws);
        const bool kf = op == BSA_PERM_GATHER_KF_POOL;
        return launched(bsa::launch_gather_pool(kf, static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst),
                                                perm, (int)g.B, (int)g.H, (int)g.D, (int)g.npf, g.n_video,
                                                kf ? p.k : p.q, s, g.n_ras));
    }
    if (overlap) return BSA_ERR_ARG;
    if (op == BSA_PERM_GATHER_KF)
        return launched(bsa::launch_gather_kf(static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), perm,
                                              (int)g.B, (int)g.H, (int)g.D, (int)g.npf, g.n_video, s, g.n_ras));
    if (op == BSA_PERM_GATHER_VF)
        return launched(bsa::launch_gather_vf(static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), perm,
                                              (int)g.B, (int)g.H, (int)g.D, (int)g.npf, g.n_video, s, g.n_ras));
    return launched(bsa::launch_permute_copy(op == BSA_PERM_SCATTER, static_cast<const uint16_t*>(src),
                                             static_cast<uint16_t*>(dst), perm, (int)g.B, (int)g.H, (int)g.D,
                                             (int)g.npf, g.n_video, s, g.n_ras));
}

bsa_status bsa_plan(const bsa_desc* desc, const void* q_tiled, const void* k_frag, int32_t* block_idx, void* ws,
                    size_t ws_bytes, void* stream) {
    Geo g;
    bsa_status st = check_desc(desc, &g);
    if (st != BSA_OK) return st;
    if (g.nvt > BSA_MAX_VIDEO_TILES) return BSA_ERR_UNSUPPORTED;
    if (g.empty || g.nvt == 0) return BSA_OK;
    if (!q_tiled || !k_frag || !block_idx) return BSA_ERR_NULL;
    if (misaligned(q_tiled, 16) || misaligned(k_frag, 16) || misaligned(block_idx, 4)) return BSA_ERR_ALIGN;
    const Layout L = layout(g);
    if (!ws || ws_bytes < L.total) return BSA_ERR_WORKSPACE;
    if (misaligned(ws, kAlign)) return BSA_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const PoolPair p = pool_outs(L, ws);
    hipError_t e = bsa::launch_pool(static_cast<const uint16_t*>(q_tiled), static_cast<const uint16_t*>(k_frag),
                                    p.q, p.k, (int)g.BH, (int)g.npf, (int)g.nvt, (int)g.D, s, g.pad);
    if (e == hipSuccess) e = bsa::launch_select(select_args(g, L, ws, block_idx, nullptr), (int)g.D, s);
    return launched(e);
}

bsa_status bsa_select(const bsa_desc* desc, int32_t* block_idx, void* ws, size_t ws_bytes, void* stream) {
    Geo g;
    bsa_status st = check_desc(desc, &g);
    if (st != BSA_OK) return st;
    if (g.nvt > BSA_MAX_VIDEO_TILES) return BSA_ERR_UNSUPPORTED;
    if (g.empty || g.nvt == 0) return BSA_OK;
    if (!block_idx) return BSA_ERR_NULL;
    if (misaligned(block_idx, 4)) return BSA_ERR_ALIGN;
    const Layout L = layout(g);
    if (!ws || ws_bytes < L.total) return BSA_ERR_WORKSPACE;
    if (misaligned(ws, kAlign)) return BSA_ERR_ALIGN;
    return launched(bsa::launch_select(select_args(g, L, ws, block_idx, nullptr), (int)g.D,
                                       static_cast<hipStream_t>(stream)));
}

bsa_status bsa_forward_stats_offset(const bsa_desc* desc, size_t* offset) {
    if (!offset) return BSA_ERR_NULL;
    Geo g;
    const bsa_status st = check_desc(desc, &g);
    if (st != BSA_OK) return st;
    *offset = layout(g).fwd + bsa::forward_stats_offset();
    return BSA_OK;
}

namespace {

// The forward's outputs (O, the lse, the group counters in the workspace)
// must not overlap each other or an input that other blocks still read (the
// last check before a launch): Q and O raster (raster) or tiled, K and V in
// the fragment layouts (the tiled size), the kept lists (fixed keep: idx;
// CSR: row_ptr and col_entries entries of idx), the permutation (raster).
bool forward_io_overlap(const Geo& g, const void* q, const void* k, const void* v, const void* o, bool raster,
                        const float* lse = nullptr, const int32_t* idx = nullptr, const int64_t* row_ptr = nullptr,
                        int64_t col_entries = 0, const int32_t* perm = nullptr, const void* progress = nullptr) {
    const size_t tiled = (size_t)g.BH * g.n_tot * g.D * 2;
    const size_t io = raster ? (size_t)g.B * (g.npf + g.n_ras) * g.H * g.D * 2 : tiled;
    const size_t lse_b = (size_t)g.BH * g.n_tot * sizeof(float);
    const size_t idx_b = (size_t)(row_ptr ? col_entries : g.BH * g.nvt * g.k) * sizeof(int32_t);
    const size_t rp_b = row_ptr ? (size_t)(g.BH * g.nvt + 1) * sizeof(int64_t) : 0;
    const size_t perm_b = raster ? (size_t)g.B * g.n_video * sizeof(int32_t) : 0;
    return clash({{o, io}, {lse, lse_b}, {progress, bsa::forward_workspace_bytes()}},
                 {{q, io}, {k, tiled}, {v, tiled}, {idx, idx_b}, {row_ptr, rp_b}, {perm, perm_b}});
}

// Checks shared by bsa_forward and bsa_forward_noalloc; fills the kernel
// arguments.
bsa_status forward_args(const bsa_desc* desc, const void* q_tiled, const void* k_frag, const void* v_frag,
                        const int32_t* block_idx, void* o_tiled, float* lse, Geo* g, bsa::ForwardArgs* a) {
    bsa_status st = check_desc(desc, g);
    if (st != BSA_OK) return st;
    if (g->npt + g->nvt > BSA_MAX_TILES) return BSA_ERR_UNSUPPORTED;
    if (g->empty) return BSA_OK;
    if (!q_tiled || !k_frag || !v_frag || !o_tiled || (g->nvt > 0 && !block_idx)) return BSA_ERR_NULL;
    if (misaligned(q_tiled, 16) || misaligned(k_frag, 16) || misaligned(v_frag, 16) || misaligned(o_tiled, 16) ||
        misaligned(block_idx, 4) || misaligned(lse, 4))
        return BSA_ERR_ALIGN;
    *a = bsa::ForwardArgs{};
    a->q = static_cast<const uint16_t*>(q_tiled);
    a->k = static_cast<const uint16_t*>(k_frag);
    a->v = static_cast<const uint16_t*>(v_frag);
    a->idx = block_idx;
    a->o = static_cast<uint16_t*>(o_tiled);
    a->lse = lse;
    a->BH = (int)g->BH;
    a->npt = (int)g->npt;
    a->nvt = (int)g->nvt;
    a->keep = (int)g->k;
    a->pad = g->pad;
    a->scale_log2 = desc->scale * 1.4426950408889634f;
    return BSA_OK;
}

}  // namespace

bsa_status bsa_forward(const bsa_desc* desc, const void* q_tiled, const void* k_frag, const void* v_frag,
                       const int32_t* block_idx, void* o_tiled, float* lse, void* ws, size_t ws_bytes,
                       void* stream) {
    Geo g;
    bsa::ForwardArgs a;
    const bsa_status st = forward_args(desc, q_tiled, k_frag, v_frag, block_idx, o_tiled, lse, &g, &a);
    if (st != BSA_OK || g.empty) return st;
    int* progress = nullptr;
    if (ws) {
        const Layout L = layout(g);
        if (ws_bytes < L.total) return BSA_ERR_WORKSPACE;
        if (misaligned(ws, kAlign)) return BSA_ERR_ALIGN;
        progress = reinterpret_cast<int*>(static_cast<char*>(ws) + L.fwd);
    }
    if (forward_io_overlap(g, q_tiled, k_frag, v_frag, o_tiled, false, lse, block_idx, nullptr, 0, nullptr, progress))
        return BSA_ERR_ARG;
    return launched(bsa::launch_forward(a, (int)g.D, progress, static_cast<hipStream_t>(stream)));
}

bsa_status bsa_forward_raster(const bsa_desc* desc, const void* q_raster, const int32_t* perm, const void* k_frag,
                              const void* v_frag, const int32_t* block_idx, void* o_raster, float* lse, void* ws,
                              size_t ws_bytes, void* stream) {
    Geo g;
    bsa::ForwardArgs a;
    const bsa_status st = forward_args(desc, q_raster, k_frag, v_frag, block_idx, o_raster, lse, &g, &a);
    if (st != BSA_OK || g.empty) return st;
    if (g.n_video > 0 && !perm) return BSA_ERR_NULL;
    if (misaligned(perm, 4)) return BSA_ERR_ALIGN;
    // raster rows: prefix + real video tokens, whose raster and slot numbers
    // the kernel keeps in int
    if (g.npf + g.n_ras > INT32_MAX / 2) return BSA_ERR_UNSUPPORTED;
    a.raster = true;
    a.perm = perm;  // read for video slots only
    a.n_ras = g.npf + g.n_ras;
    a.H = (int)g.H;
    int* progress = nullptr;
    if (ws) {
        const Layout L = layout(g);
        if (ws_bytes < L.total) return BSA_ERR_WORKSPACE;
        if (misaligned(ws, kAlign)) return BSA_ERR_ALIGN;
        progress = reinterpret_cast<int*>(static_cast<char*>(ws) + L.fwd);
    }
    if (forward_io_overlap(g, q_raster, k_frag, v_frag, o_raster, true, lse, block_idx, nullptr, 0, perm, progress))
        return BSA_ERR_ARG;
    return launched(bsa::launch_forward(a, (int)g.D, progress, static_cast<hipStream_t>(stream)));
}

bsa_status bsa_forward_noalloc(const bsa_desc* desc, const void* q_tiled, const void* k_frag, const void* v_frag,
                               const int32_t* block_idx, void* o_tiled, float* lse, void* stream) {
    Geo g;
    bsa::ForwardArgs a;
    const bsa_status st = forward_args(desc, q_tiled, k_frag, v_frag, block_idx, o_tiled, lse, &g, &a);
    if (st != BSA_OK || g.empty) return st;
    if (bsa::forward_workspace_bytes() > bsa::forward_scratch_bytes()) return BSA_ERR_UNSUPPORTED;
    if (forward_io_overlap(g, q_tiled, k_frag, v_frag, o_tiled, false, lse, block_idx)) return BSA_ERR_ARG;
    return launched(bsa::launch_forward_noalloc(a, (int)g.D, static_cast<hipStream_t>(stream)));
}

// ---- variable keep (CSR lists) ----------------------------------------------

namespace {

// Per-head keep counts: keep_per_head (host, [H]) or desc->keep_tiles, each
// in 1..nvt; fills kh and the number of list entries B * nvt * sum_h k_h.
bsa_status csr_heads(const Geo& g, const int32_t* keep_per_head, bsa::CsrKeep* kh, int64_t* entries) {
    if (g.H > BSA_MAX_CSR_HEADS) return BSA_ERR_UNSUPPORTED;
    int64_t sum = 0;
    for (int64_t h = 0; h < g.H; ++h) {
        const int64_t k = keep_per_head ? keep_per_head[h] : g.k;
        if (k < 1 || k > g.nvt) return BSA_ERR_SHAPE;
        if (kh) kh->k[h] = (int32_t)k;
        sum += k;
    }
    *entries = g.B * g.nvt * sum;
    return BSA_OK;
}

}  // namespace

bsa_status bsa_csr_entries(const bsa_desc* desc, const int32_t* keep_per_head, int64_t* entries) {
    if (!entries) return BSA_ERR_NULL;
    Geo g;
    bsa_status st = check_desc(desc, &g);
    if (st != BSA_OK) return st;
    if (g.empty || g.nvt == 0) {
        *entries = 0;
        return BSA_OK;
    }
    return csr_heads(g, keep_per_head, nullptr, entries);
}

namespace {

// bsa_plan_csr (pool = true: the tile means from q_tiled and k_frag first) and
// bsa_select_csr (the means already in the workspace).
bsa_status plan_csr_impl(const bsa_desc* desc, const void* q_tiled, const void* k_frag, const int32_t* keep_per_head,
                         const int32_t* keep_rows, int64_t* row_ptr, int32_t* col_idx, int64_t col_entries, void* ws,
                         size_t ws_bytes, void* stream, bool pool) {
    Geo g;
    bsa_status st = check_desc(desc, &g);
    if (st != BSA_OK) return st;
    if (g.nvt > BSA_MAX_VIDEO_TILES) return BSA_ERR_UNSUPPORTED;
    if (g.empty || g.nvt == 0) return BSA_OK;
    bsa::CsrKeep kh{};
    int64_t need = 0;
    st = csr_heads(g, keep_per_head, &kh, &need);
    if (st != BSA_OK) return st;
    if ((pool && (!q_tiled || !k_frag)) || !row_ptr || !col_idx) return BSA_ERR_NULL;
    if (col_entries < need) return BSA_ERR_SHAPE;
    if (misaligned(q_tiled, 16) || misaligned(k_frag, 16) || misaligned(row_ptr, 8) || misaligned(col_idx, 4) ||
        misaligned(keep_rows, 4))
        return BSA_ERR_ALIGN;
    const Layout L = layout(g);
    if (!ws || ws_bytes < L.total) return BSA_ERR_WORKSPACE;
    if (misaligned(ws, kAlign)) return BSA_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const PoolPair p = pool_outs(L, ws);
    hipError_t e = bsa::launch_csr_rowptr(kh, keep_rows, (int)g.BH, (int)g.H, (int)g.nvt, row_ptr, s);
    if (e == hipSuccess && pool)
        e = bsa::launch_pool(static_cast<const uint16_t*>(q_tiled), static_cast<const uint16_t*>(k_frag), p.q, p.k,
                             (int)g.BH, (int)g.npf, (int)g.nvt, (int)g.D, s, g.pad);
    if (e == hipSuccess) e = bsa::launch_select(select_args(g, L, ws, col_idx, row_ptr), (int)g.D, s);
    return launched(e);
}

}  // namespace

bsa_status bsa_plan_csr(const bsa_desc* desc, const void* q_tiled, const void* k_frag, const int32_t* keep_per_head,
                        const int32_t* keep_rows, int64_t* row_ptr, int32_t* col_idx, int64_t col_entries, void* ws,
                        size_t ws_bytes, void* stream) {
    return plan_csr_impl(desc, q_tiled, k_frag, keep_per_head, keep_rows, row_ptr, col_idx, col_entries, ws, ws_bytes,
                         stream, true);
}

bsa_status bsa_select_csr(const bsa_desc* desc, const int32_t* keep_per_head, const int32_t* keep_rows,
                          int64_t* row_ptr, int32_t* col_idx, int64_t col_entries, void* ws, size_t ws_bytes,
                          void* stream) {
    return plan_csr_impl(desc, nullptr, nullptr, keep_per_head, keep_rows, row_ptr, col_idx, col_entries, ws,
                         ws_bytes, stream, false);
}

namespace {

// bsa_forward_csr and bsa_forward_csr_raster: q / o tiled, or raster through
// perm (raster).
bsa_status forward_csr_impl(const bsa_desc* desc, const void* q, const int32_t* perm, const void* k_frag,
                            const void* v_frag, const int64_t* row_ptr, const int32_t* col_idx, int64_t col_entries,
                            void* o, float* lse, void* ws, size_t ws_bytes, void* stream, bool raster) {
    Geo g;
    bsa_status st = check_desc(desc, &g);
    if (st != BSA_OK) return st;
    if (g.npt + g.nvt > BSA_MAX_TILES) return BSA_ERR_UNSUPPORTED;
    if (g.empty) return BSA_OK;
    if (!q || !k_frag || !v_frag || !o || (g.nvt > 0 && (!row_ptr || !col_idx))) return BSA_ERR_NULL;
    if (raster && g.n_video > 0 && !perm) return BSA_ERR_NULL;
    if (g.nvt > 0 && col_entries < 1) return BSA_ERR_SHAPE;
    if (misaligned(q, 16) || misaligned(k_frag, 16) || misaligned(v_frag, 16) || misaligned(o, 16) ||
        misaligned(row_ptr, 8) || misaligned(col_idx, 4) || misaligned(lse, 4) || misaligned(perm, 4))
        return BSA_ERR_ALIGN;
    if (raster && g.npf + g.n_ras > INT32_MAX / 2) return BSA_ERR_UNSUPPORTED;
    int* progress = nullptr;
    if (ws) {
        const Layout L = layout(g);
        if (ws_bytes < L.total) return BSA_ERR_WORKSPACE;
        if (misaligned(ws, kAlign)) return BSA_ERR_ALIGN;
        progress = reinterpret_cast<int*>(static_cast<char*>(ws) + L.fwd);
    }
    if (forward_io_overlap(g, q, k_frag, v_frag, o, raster, lse, g.nvt > 0 ? col_idx : nullptr,
                           g.nvt > 0 ? row_ptr : nullptr, col_entries, raster ? perm : nullptr, progress))
        return BSA_ERR_ARG;
    bsa::ForwardArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k_frag);
    a.v = static_cast<const uint16_t*>(v_frag);
    a.idx = col_idx;
    a.row_ptr = g.nvt > 0 ? row_ptr : nullptr;
    a.col_entries = col_entries;
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse;
    a.BH = (int)g.BH;
    a.npt = (int)g.npt;
    a.nvt = (int)g.nvt;
    a.keep = 1;
    a.pad = g.pad;
    a.scale_log2 = desc->scale * 1.4426950408889634f;
    if (raster) {
        a.raster = true;
        a.perm = perm;
        a.n_ras = g.npf + g.n_ras;
        a.H = (int)g.H;
    }
    return launched(bsa::launch_forward(a, (int)g.D, progress, static_cast<hipStream_t>(stream)));
}

}  // namespace

bsa_status bsa_forward_csr(const bsa_desc* desc, const void* q_tiled, const void* k_frag, const void* v_frag,
                           const int64_t* row_ptr, const int32_t* col_idx, int64_t col_entries, void* o_tiled,
                           float* lse, void* ws, size_t ws_bytes, void* stream) {
    return forward_csr_impl(desc, q_tiled, nullptr, k_frag, v_frag, row_ptr, col_idx, col_entries, o_tiled, lse, ws,
                            ws_bytes, stream, false);
}

bsa_status bsa_forward_csr_raster(const bsa_desc* desc, const void* q_raster, const int32_t* perm,
                                  const void* k_frag, const void* v_frag, const int64_t* row_ptr,
                                  const int32_t* col_idx, int64_t col_entries, void* o_raster, float* lse, void* ws,
                                  size_t ws_bytes, void* stream) {
    return forward_csr_impl(desc, q_raster, perm, k_frag, v_frag, row_ptr, col_idx, col_entries, o_raster, lse, ws,
                            ws_bytes, stream, true);
}

// ---- structured lists (spatial / temporal heads) ------------------------------

namespace {

// sum over x in [0, n) of the size of [x - r, x + r] clipped to [0, n)
int64_t range_sum(int64_t n, int64_t r) {
    int64_t s = 0;
    for (int64_t x = 0; x < n; ++x) s += std::min(x + r, n - 1) - std::max(x - r, (int64_t)0) + 1;
    return s;
}

bsa_status struct_rule(const bsa_desc* desc, const Geo& g, const int32_t* head_mask, int32_t radius_t,
                       int32_t radius_hw, bsa::StructRule* sr, int64_t* entries) {
    if (g.dynamic) return BSA_ERR_UNSUPPORTED;  // the rule needs the regular tile grid
    if (g.H > BSA_MAX_CSR_HEADS) return BSA_ERR_UNSUPPORTED;
    if (!head_mask) return BSA_ERR_NULL;
    if (radius_t < 0 || radius_hw < 0) return BSA_ERR_ARG;
    const int64_t Tt = g.Tt, Th = g.Th, Tw = g.Tw;
    const int64_t spatial = range_sum(Tt, radius_t) * Th * Tw * Th * Tw;
    const int64_t temporal = Tt * Tt * range_sum(Th, radius_hw) * range_sum(Tw, radius_hw);
    int64_t sum = 0;
    for (int64_t h = 0; h < g.H; ++h) {
        if (head_mask[h] != BSA_MASK_SPATIAL && head_mask[h] != BSA_MASK_TEMPORAL) return BSA_ERR_ARG;
        if (sr) sr->kind[h] = head_mask[h];
        sum += head_mask[h] == BSA_MASK_SPATIAL ? spatial : temporal;
    }
    if (sr) {
        sr->Tt = (int)Tt;
        sr->Th = (int)Th;
        sr->Tw = (int)Tw;
        sr->rt = radius_t;
        sr->rs = radius_hw;
    }
    *entries = g.B * sum;
    return BSA_OK;
}

}  // namespace

bsa_status bsa_structured_entries(const bsa_desc* desc, const int32_t* head_mask, int32_t radius_t,
                                  int32_t radius_hw, int64_t* entries) {
    if (!entries) return BSA_ERR_NULL;
    Geo g;
    bsa_status st = check_desc(desc, &g);
    if (st != BSA_OK) return st;
    if (g.empty || g.nvt == 0) {
        *entries = 0;
        return BSA_OK;
    }
    return struct_rule(desc, g, head_mask, radius_t, radius_hw, nullptr, entries);
}

bsa_status bsa_plan_structured(const bsa_desc* desc, const int32_t* head_mask, int32_t radius_t, int32_t radius_hw,
                               int64_t* row_ptr, int32_t* col_idx, int64_t col_entries, void* stream) {
    Geo g;
    bsa_status st = check_desc(desc, &g);
    if (st != BSA_OK) return st;
    if (g.nvt > BSA_MAX_VIDEO_TILES) return BSA_ERR_UNSUPPORTED;
    if (g.empty || g.nvt == 0) return BSA_OK;
    bsa::StructRule sr{};
    int64_t need = 0;
    st = struct_rule(desc, g, head_mask, radius_t, radius_hw, &sr, &need);
    if (st != BSA_OK) return st;
    if (!row_ptr || !col_idx) return BSA_ERR_NULL;
    if (col_entries < need) return BSA_ERR_SHAPE;
    if (misaligned(row_ptr, 8) || misaligned(col_idx, 4)) return BSA_ERR_ALIGN;
    return launched(bsa::launch_structured(sr, (int)g.BH, (int)g.H, row_ptr, col_idx, static_cast<hipStream_t>(stream)));
}

bsa_status bsa_backward_workspace_size(const bsa_desc* desc, size_t* bytes) {
    if (!bytes) return BSA_ERR_NULL;
    Geo g;
    const bsa_status st = check_desc(desc, &g);
    if (st != BSA_OK) return st;
    *bytes = bwd_layout(g, g.BH * g.nvt * g.k).total;
    return BSA_OK;
}

bsa_status bsa_backward_csr_workspace_size(const bsa_desc* desc, int64_t col_entries, size_t* bytes) {
    if (!bytes) return BSA_ERR_NULL;
    Geo g;
    const bsa_status st = check_desc(desc, &g);
    if (st != BSA_OK) return st;
    if (col_entries < 0) return BSA_ERR_SHAPE;
    *bytes = bwd_layout(g, g.nvt > 0 ? col_entries : 0).total;
    return BSA_OK;
}

bsa_status bsa_backward_stats_offset(const bsa_desc* desc, int64_t col_entries, size_t* offset) {
    if (!offset) return BSA_ERR_NULL;
    Geo g;
    const bsa_status st = check_desc(desc, &g);
    if (st != BSA_OK) return st;
    if (col_entries < 0) return BSA_ERR_SHAPE;
    const int64_t tcap = col_entries == 0 ? g.BH * g.nvt * g.k : (g.nvt > 0 ? col_entries : 0);
    *offset = bwd_layout(g, tcap).progress + (size_t)bsa::backward_stats_ints() * sizeof(int);
    return BSA_OK;
}

namespace {

// The backward over fixed-keep lists (row_ptr null) or CSR lists.
bsa_status backward_impl(const bsa_desc* desc, const void* q, const void* k, const void* v, const void* o,
                         const void* d_o, const float* lse, const int32_t* perm, const int32_t* idx,
                         const int64_t* row_ptr, int64_t col_entries, bool csr, void* dq, void* dk, void* dv,
                         void* ws, size_t ws_bytes, void* stream) {
    Geo g;
    bsa_status st = check_desc(desc, &g);
    if (st != BSA_OK) return st;
    if (g.npt + g.nvt > BSA_MAX_TILES || g.nvt > BSA_MAX_VIDEO_TILES) return BSA_ERR_UNSUPPORTED;
    if (g.empty) return BSA_OK;
    if (!q || !k || !v || !o || !d_o || !lse || !dq || !dk || !dv) return BSA_ERR_NULL;
    if (g.nvt > 0 && (!perm || !idx || (csr && !row_ptr))) return BSA_ERR_NULL;
    if (csr && g.nvt > 0 && col_entries < 1) return BSA_ERR_SHAPE;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) || misaligned(d_o, 16) ||
        misaligned(dq, 16) || misaligned(dk, 16) || misaligned(dv, 16) || misaligned(lse, 4) ||
        misaligned(perm, 4) || misaligned(idx, 4) || misaligned(row_ptr, 8))
        return BSA_ERR_ALIGN;
    const int64_t tcap = g.nvt == 0 ? 0 : csr ? col_entries : g.BH * g.nvt * g.k;
    const BwdLayout L = bwd_layout(g, tcap);
    if (!ws || ws_bytes < L.total) return BSA_ERR_WORKSPACE;
    if (misaligned(ws, kAlign)) return BSA_ERR_ALIGN;
    {
        // the gradients (raster, written last) must not overlap each other,
        // an input or the workspace
        const size_t ras = (size_t)g.B * (g.npf + g.n_ras) * g.H * g.D * 2;
        const size_t idx_b = (size_t)(csr ? col_entries : g.BH * g.nvt * g.k) * sizeof(int32_t);
        const size_t rp_b = csr ? (size_t)(g.BH * g.nvt + 1) * sizeof(int64_t) : 0;
        if (clash({{dq, ras}, {dk, ras}, {dv, ras}},
                  {{q, ras}, {k, ras}, {v, ras}, {o, ras}, {d_o, ras}, {lse, (size_t)g.BH * g.n_tot * sizeof(float)},
                   {perm, (size_t)g.B * g.n_video * sizeof(int32_t)}, {idx, g.nvt > 0 ? idx_b : 0},
                   {row_ptr, g.nvt > 0 ? rp_b : 0}, {ws, L.total}}))
            return BSA_ERR_ARG;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* w = static_cast<char*>(ws);
    uint16_t* f[7];
    for (int i = 0; i < 7; ++i) f[i] = reinterpret_cast<uint16_t*>(w + L.frag[i]);
    // f: q_kf, do_kf, k_kf, v_kf (kfrag), k_vf (vfrag), q_t, do_t (tiled).
    // Q, dO and K are read once each for both of their layouts; the dO
    // gather also takes Delta = dO . O and the lse forms per row.
    float* lse2 = reinterpret_cast<float*>(w + L.lse2);
    float* delta = reinterpret_cast<float*>(w + L.delta);
    float* nlse = reinterpret_cast<float*>(w + L.nlse);
    float* ndelta = reinterpret_cast<float*>(w + L.ndelta);
    const bsa::DeltaOut dl{static_cast<const uint16_t*>(o), lse, delta, ndelta, lse2, nlse, desc->scale};
    const int B = (int)g.B, H = (int)g.H, D = (int)g.D, npf = (int)g.npf;
    hipError_t e = bsa::launch_gather_kf_tiled(static_cast<const uint16_t*>(q), f[0], f[5], perm, B, H, D, npf,
                                               g.n_video, s, g.n_ras, nullptr);
    if (e == hipSuccess)
        e = bsa::launch_gather_kf_tiled(static_cast<const uint16_t*>(d_o), f[1], f[6], perm, B, H, D, npf, g.n_video,
                                        s, g.n_ras, &dl);
    if (e == hipSuccess)
        e = bsa::launch_gather_kf_vf(static_cast<const uint16_t*>(k), f[2], f[4], perm, B, H, D, npf, g.n_video, s,
                                     g.n_ras);
    if (e == hipSuccess)
        e = bsa::launch_gather_kf(static_cast<const uint16_t*>(v), f[3], perm, B, H, D, npf, g.n_video, s, g.n_ras);
    if (e != hipSuccess) return launched(e);
    bsa::BackwardArgs a{};
    a.q_kf = f[0];
    a.do_kf = f[1];
    a.k_kf = f[2];
    a.v_kf = f[3];
    a.k_vf = f[4];
    a.q_t = f[5];
    a.do_t = f[6];
    a.idx = idx;
    a.row_ptr = csr && g.nvt > 0 ? row_ptr : nullptr;
    a.col_entries = col_entries;
    a.perm = perm;
    a.lse2 = lse2;
    a.delta = delta;
    a.nlse = nlse;
    a.ndelta = ndelta;
    a.mask = reinterpret_cast<unsigned long long*>(w + L.mask);
    a.cnt = reinterpret_cast<int32_t*>(w + L.cnt);
    a.rowp = reinterpret_cast<int64_t*>(w + L.rowp);
    a.tlist = reinterpret_cast<int32_t*>(w + L.tlist);
    a.tcap = tcap;
    a.progress = reinterpret_cast<int*>(w + L.progress);
    a.dq = static_cast<uint16_t*>(dq);
    a.dk = static_cast<uint16_t*>(dk);
    a.dv = static_cast<uint16_t*>(dv);
    a.BH = (int)g.BH;
    a.H = (int)g.H;
    a.npt = (int)g.npt;
    a.nvt = (int)g.nvt;
    a.keep = (int)g.k;
    a.mchunks = L.mchunks;
    a.npf = g.npf;
    a.n_tot = g.n_tot;
    a.n_ras = g.npf + g.n_ras;
    a.pad = g.pad;
    a.scale = desc->scale;
    a.scale_log2 = desc->scale * 1.4426950408889634f;
    return launched(bsa::launch_backward(a, (int)g.D, s));
}

}  // namespace

bsa_status bsa_backward(const bsa_desc* desc, const void* q, const void* k, const void* v, const void* o,
                        const void* d_o, const float* lse, const int32_t* perm, const int32_t* block_idx, void* dq,
                        void* dk, void* dv, void* ws, size_t ws_bytes, void* stream) {
    return backward_impl(desc, q, k, v, o, d_o, lse, perm, block_idx, nullptr, 0, false, dq, dk, dv, ws, ws_bytes,
                         stream);
}

bsa_status bsa_backward_csr(const bsa_desc* desc, const void* q, const void* k, const void* v, const void* o,
                            const void* d_o, const float* lse, const int32_t* perm, const int64_t* row_ptr,
                            const int32_t* col_idx, int64_t col_entries, void* dq, void* dk, void* dv, void* ws,
                            size_t ws_bytes, void* stream) {
    return backward_impl(desc, q, k, v, o, d_o, lse, perm, col_idx, row_ptr, col_entries, true, dq, dk, dv, ws,
                         ws_bytes, stream);
}

}  // extern "C"
