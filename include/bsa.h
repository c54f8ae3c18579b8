/*
 * bsa.h -- C ABI of libbsa.so: block-sparse self-attention over a video token
 * grid, hand-written HIP for AMD Instinct MI355X (gfx950).
 *
 * The operation (sources by page title and section):
 *   "Prism / Kandinsky 6 speed ablation" (oh-my-gpu.com), section
 *   "같은 계산량 안에서 볼 곳을 고르는 Prism" (Prism picks where to look within the
 *   same compute): tokens of the T x H x W latent grid are grouped into 64-token
 *   tiles (4x4x4 by default, or a per-8x8x8-region shape chosen from how fast
 *   each axis varies); every query tile keeps only its most relevant key tiles,
 *   relevance being judged from the mean of each tile's 64 tokens; sparsity s
 *   keeps (1-s) of the key tiles (s = 0.75 keeps 480 of 1,920).
 *   "Sparse VideoGen TPU 최적화: 비디오 생성 추론 지연을 줄이는 실무 기준"
 *   (aibase.it), section "이론적 sparsity와 물리적 sparsity의 차이": skipped tiles
 *   cost nothing and kept tiles are computed whole, with no per-element mask;
 *   section "실무에서 배울 최적화 기준": tokens are first permuted so that each
 *   tile is contiguous.
 *   "RTX 4090에서 5초 영상 72초: Ref2VA VSA" (pulmap.app), section
 *   "조건 토큰은 왜 다르게 다루나": a conditioning prefix of segment-pure tiles is
 *   attended densely and never pruned; top-k applies to video key tiles only.
 *
 * A call sequence:  bsa_permute(BUILD) -> bsa_permute(GATHER) for Q,
 * bsa_permute(GATHER_KF) for K, bsa_permute(GATHER_VF) for V -> bsa_plan ->
 * bsa_forward -> bsa_permute(SCATTER) for O; for training, bsa_backward with
 * the raster tensors, the forward's lse and dL/dO.  The same result with the
 * tile means taken during the gathers (no second read of Q and K):
 * bsa_permute(GATHER_POOL) for Q and bsa_permute(GATHER_KF_POOL) for K, then
 * bsa_select in place of bsa_plan.  The shortest sequence also skips the
 * tiled copies of Q and O: bsa_permute(POOL) for Q's means,
 * bsa_permute(GATHER_KF_POOL) for K, bsa_permute(GATHER_VF) for V,
 * bsa_select, then bsa_forward_raster, which reads raster Q and writes raster
 * O itself.  A caller holding K and V already in the tiled layout converts
 * them with bsa_permute(TILED_TO_KF / TILED_TO_VF).
 *
 * Layouts (row-major, bf16 = IEEE bfloat16):
 *   raster  bf16 [B][Ntot][H][D]   the dense prefix first (n_prefix tokens, already
 *                                   in 64-token segment-pure tiles), then the video
 *                                   grid in (t, h, w) raster order, t slowest.
 *   tiled   bf16 [B][H][Ntot][D]   prefix unchanged, then the video tokens in tile
 *                                   order: tile 0's 64 tokens, tile 1's, ...; inside
 *                                   a tile, tokens in (t, h, w) raster order.
 *   kfrag   bf16 [B][H][Ntot/64][2][D/16][64][8]  K in the tiled order, each
 *                                   64-token tile in the operand order of the
 *                                   attention kernel's matrix instructions:
 *                                   element [.][t][kh][s][l][e] is channel
 *                                   16*s + 8*(l/32) + e of the tile's token
 *                                   32*kh + swap23(l % 32), where swap23(m)
 *                                   exchanges bits 2 and 3 of m.
 *   vfrag   bf16 [B][H][Ntot/64][2][D/32][2][64][8]  V likewise: element
 *                                   [.][t][kh][i][c][l][e] is channel
 *                                   32*i + (l % 32) of token
 *                                   32*kh + 16*c + 8*(l/32) + e of tile t.
 *                                   (Both are plain permutations of the tiled
 *                                   layout, same size; every 1 KB of them is one
 *                                   wave-wide 16-byte-per-lane load.)
 *   perm    int32 [B][Nvideo]      tiled video slot -> raster video token index
 *                                   (0-based, not counting the prefix).  The
 *                                   kernels clamp a value past the raster's
 *                                   video rows into them (and, without padding,
 *                                   a negative one to 0), so a corrupt perm
 *                                   gives wrong rows but no access outside the
 *                                   tensors.
 *   block_idx int32 [B][H][nVT][k] per video query tile, the k kept video key tiles
 *                                   (video tile numbers 0..nVT-1), ascending.
 * Ntot = n_prefix + Nvideo, Nvideo = grid_t*grid_h*grid_w, nVT = Nvideo/64.
 *
 * Ragged grids (tile_mode BSA_TILE_STATIC_PADDED): the grid need not be a
 * whole number of tiles on any axis.  The tile grid then covers it rounded up
 * (ceil(T/tile_t) x ceil(H/tile_h) x ceil(W/tile_w) tiles); the slots of a
 * boundary tile that fall outside the grid are padding.  The raster layout
 * keeps the real token count (Nraster = grid_t*grid_h*grid_w); every tiled
 * layout (tiled, kfrag, vfrag, perm, block_idx, lse, the pooled means) uses
 * the padded count Nvideo = 64 * tiles, nVT = tiles.  perm holds -1 for a
 * padding slot; gathers write zeros there and the scatter skips it.  A boundary
 * tile's mean is taken over its real tokens only, and its padding keys get
 * zero attention weight; padding query rows of the tiled output are not
 * meaningful and are dropped by the scatter.  No page fixes these rules: they
 * are the plain reading under which a ragged grid computes what the same
 * grid would if its tiles could be cut to size.
 *
 * Ownership and threading: the caller allocates every buffer (device memory),
 * including the workspace.  The library allocates nothing, frees nothing,
 * never synchronises and keeps no state: calls are reentrant.  All work is
 * enqueued on `stream` (a hipStream_t; NULL means the default stream).  Inputs
 * are only read; outputs are entirely overwritten.
 *
 * Errors: every precondition is checked on the host before anything is
 * enqueued; a failed check returns a negative bsa_status and enqueues nothing.
 * A launch failure reported by the HIP runtime returns BSA_ERR_LAUNCH.  Faults
 * inside kernels surface at the caller's next synchronisation.  Nothing throws.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BSA_OK = 0,
    BSA_ERR_NULL = -1,        /* a required pointer is NULL */
    BSA_ERR_SHAPE = -2,       /* sizes inconsistent: grid not divisible, bad prefix, k out of range */
    BSA_ERR_UNSUPPORTED = -3, /* valid but not implemented: head_dim not 64/128, too many tiles */
    BSA_ERR_ALIGN = -4,       /* a tensor pointer is not 16-byte aligned */
    BSA_ERR_WORKSPACE = -5,   /* workspace missing or smaller than bsa_workspace_size() */
    BSA_ERR_LAUNCH = -6,      /* the HIP runtime rejected a kernel launch */
    BSA_ERR_ARG = -7          /* bad enum value, non-finite / non-positive scale, or an
                                 output buffer overlapping an input of the same call */
} bsa_status;

enum { BSA_TILE_STATIC = 0, BSA_TILE_DYNAMIC = 1, BSA_TILE_STATIC_PADDED = 2 };
enum {
    BSA_PERM_BUILD = 0,
    BSA_PERM_GATHER = 1,
    BSA_PERM_SCATTER = 2,
    BSA_PERM_GATHER_KF = 3,
    BSA_PERM_GATHER_VF = 4,
    BSA_PERM_GATHER_POOL = 5,
    BSA_PERM_GATHER_KF_POOL = 6,
    BSA_PERM_TILED_TO_KF = 7,
    BSA_PERM_TILED_TO_VF = 8,
    BSA_PERM_POOL = 9
};

/* Largest number of video tiles per (batch, head) that bsa_plan accepts. */
#define BSA_MAX_VIDEO_TILES 8192
/* Largest number of tiles (prefix + video) per (batch, head) bsa_forward accepts. */
#define BSA_MAX_TILES 16384

typedef struct bsa_desc {
    int32_t batch;      /* B >= 0 (0: every call is a no-op returning BSA_OK)         */
    int32_t heads;      /* H >= 0 (0: no-op)                                           */
    int32_t head_dim;   /* D, 64 or 128                                                */
    int32_t grid_t;     /* video grid T x H x W, each >= 0 (see tile_mode)             */
    int32_t grid_h;
    int32_t grid_w;
    int32_t n_prefix;   /* dense prefix tokens, a multiple of 64, >= 0                 */
    int32_t tile_mode;  /* BSA_TILE_STATIC, BSA_TILE_DYNAMIC or BSA_TILE_STATIC_PADDED */
    int32_t tile_t;     /* static tile extents; product 64; must divide the grid       */
    int32_t tile_h;     /*   (padded mode: any grid; ignored in dynamic mode, where    */
    int32_t tile_w;     /*    the grid must be a multiple of 8 on every axis)          */
    int32_t keep_tiles; /* k: kept video key tiles per video query tile, 1..nVT        */
                        /*   (0 when there is no video)                                */
    float scale;        /* softmax scale applied to q.k, finite and > 0 (1/sqrt(D))    */
    float dyn_tau;      /* dynamic shapes: isotropy margin tau >= 0 (0.10 typical)     */
} bsa_desc;

/*
 * Bytes of device workspace that bsa_plan, bsa_select, bsa_forward and
 * bsa_permute (BUILD in dynamic mode, GATHER_POOL, GATHER_KF_POOL) need for
 * `desc`; one buffer of this size serves all of them on one stream.
 * Host-only; enqueues nothing.  After bsa_plan's work (or the two pooling
 * gathers) has run, the workspace starts with the pooled tile means
 *   float qbar[B][H][nVT][D], then float kbar[B][H][nVT][D]
 * (each the mean of the tile's 64 tokens, or of its real tokens on a ragged
 * grid), each region 256-byte aligned; bsa_forward does not overwrite them.
 * About 4 * B*H*nVT*D floats (the means of Q and K and their bf16 hi/lo
 * pairs) plus 16 KB per video tile of selection scratch: 221 MB for the 720p
 * grid with B = 2, H = 24, D = 128 (nVT = 1,920).
 */
bsa_status bsa_workspace_size(const bsa_desc *desc, size_t *bytes);

/*
 * Token permutation between raster and tiled order ("Sparse VideoGen TPU
 * 최적화", section "실무에서 배울 최적화 기준": the tokens are reordered first so
 * that every tile is contiguous and a kept tile is read whole; "Prism /
 * Kandinsky 6 speed ablation", section "같은 계산량 안에서 볼 곳을 고르는 Prism":
 * the tile's shape may follow how fast each axis of a region varies).
 *  op = BSA_PERM_BUILD: write `perm` [B][Nvideo].  Static mode: the closed-form
 *       tile order (tiles in raster order of the tile grid).  Dynamic mode: read
 *       `q_raster` (bf16 raster, the queries), for every batch element and 8x8x8
 *       region compute the mean |difference| of adjacent tokens along t, h and w
 *       over all heads and channels, choose one of the nine 64-token shapes
 *       (id: 0 4x4x4, 1 2x4x8, 2 2x8x4, 3 8x4x2, 4 4x2x8, 5 4x8x2, 6 8x2x4,
 *       7 2x2x16, 8 16x2x2; extents t x h x w) and write it to `shape_map`
 *       [B][R] (R = regions, raster order), then the permutation: regions in
 *       raster order, 8 tiles per region in raster order inside the region; a
 *       pair of regions sharing a 16-long shape lays its 16 tiles over the two
 *       regions' tile slots.  Uses the workspace; `src`/`dst` unused.
 *  op = BSA_PERM_GATHER: `src` raster -> `dst` tiled (Q, K or V).
 *  op = BSA_PERM_SCATTER: `src` tiled -> `dst` raster (the output).
 *  op = BSA_PERM_GATHER_KF: `src` raster -> `dst` kfrag (K).
 *  op = BSA_PERM_GATHER_VF: `src` raster -> `dst` vfrag (V).
 *  op = BSA_PERM_GATHER_POOL: as GATHER (Q), and the tile means of Q as
 *       bsa_plan computes them, written into the workspace (required) for
 *       bsa_select.
 *  op = BSA_PERM_GATHER_KF_POOL: as GATHER_KF (K), and the tile means of K
 *       into the workspace.
 *  op = BSA_PERM_TILED_TO_KF: `src` tiled -> `dst` kfrag (no perm needed).
 *  op = BSA_PERM_TILED_TO_VF: `src` tiled -> `dst` vfrag.
 *  op = BSA_PERM_POOL: the tile means of Q alone, read from `src` (raster)
 *       through `perm` into the workspace (required), the same values
 *       GATHER_POOL writes, without the tiled copy; `dst` unused.  For
 *       bsa_forward_raster, which reads Q in the raster layout itself.
 * Gather and scatter read `perm` and copy bf16 values exactly; the prefix
 * tokens keep their positions.  Source and destination must not overlap
 * (BSA_ERR_ARG when their byte ranges intersect).
 * The fragment layouts are what bsa_plan and bsa_forward read K and V in:
 * each 1 KB of them is one 16-byte-per-lane load into matrix-instruction
 * operand registers.  A gather writes them straight from the raster layout
 * (as cheap as a tiled gather); TILED_TO_KF / TILED_TO_VF serve callers that
 * already hold tiled tensors, for one more read and write of the tensor.
 */
bsa_status bsa_permute(const bsa_desc *desc, int op, const void *q_raster, int32_t *perm,
                       uint8_t *shape_map, const void *src, void *dst, void *ws,
                       size_t ws_bytes, void *stream);

/*
 * Tile selection ("Prism / Kandinsky 6 speed ablation", section "같은 계산량
 * 안에서 볼 곳을 고르는 Prism": each query tile keeps the key tiles whose
 * 64-token means score highest).  From Q (tiled) and K (kfrag), bf16: the mean
 * of each video tile's 64 tokens (of its real tokens on a ragged grid; summed
 * exactly, divided by the count, rounded once to float), the score
 * s_ij = sum_d qbar_i[d] kbar_j[d] of the float means, and per (b, h, video
 * query tile i) the keep_tiles video key tiles with the largest s_ij, equal
 * scores going to the lower tile number, written ascending to `block_idx`
 * [B][H][nVT][keep_tiles].  The kept set is exactly the top k of the scores
 * summed in double in channel order (candidates near the threshold are
 * re-scored that way), so it does not depend on float rounding.  Prefix
 * tiles are never scored (they are always attended).  Uses the workspace
 * (bsa_workspace_size); no score matrix is written to memory.
 */
bsa_status bsa_plan(const bsa_desc *desc, const void *q_tiled, const void *k_frag,
                    int32_t *block_idx, void *ws, size_t ws_bytes, void *stream);

/*
 * The scoring and top-k of bsa_plan alone, from the tile means that
 * bsa_permute(GATHER_POOL) and bsa_permute(GATHER_KF_POOL) (or an earlier
 * bsa_plan) left in the workspace.  Same output and errors as bsa_plan.
 */
bsa_status bsa_select(const bsa_desc *desc, int32_t *block_idx, void *ws, size_t ws_bytes,
                      void *stream);

/*
 * Attention over the kept tiles ("Sparse VideoGen TPU 최적화", section
 * "이론적 sparsity와 물리적 sparsity의 차이": a skipped tile costs no work and a
 * kept tile is computed whole, unmasked; "RTX 4090에서 5초 영상 72초: Ref2VA
 * VSA", section "조건 토큰은 왜 다르게 다루나": the conditioning prefix is
 * attended densely by every query and attends to everything; "Prism /
 * Kandinsky 6 speed ablation", section "같은 계산량 안에서 볼 곳을 고르는 Prism":
 * the attention itself stays exact over what is kept).  `q_tiled` and `o_tiled` are in the tiled
 * layout, `k_frag` in the kfrag and `v_frag` in the vfrag layout; at most
 * BSA_MAX_TILES tiles per (batch, head).  For each query token of video tile i the
 * keys are the prefix tokens and the tokens of the tiles block_idx[b][h][i][:];
 * prefix query tokens attend to every token.  o = softmax(scale * q K^T) V with
 * bf16 products accumulated in float, a float online softmax, and o rounded to
 * bf16 (`o_tiled`, tiled layout).  `lse` (optional, NULL to skip) receives
 * float [B][H][Ntot]: the natural log of sum_j exp(scale * q.k_j) per query.
 * `block_idx` may be NULL only when there is no video.  The outputs
 * (`o_tiled`, `lse`, and the workspace's group counters) must not overlap
 * each other or an input (`q_tiled`, `k_frag`, `v_frag`, `block_idx`):
 * BSA_ERR_ARG, nothing enqueued.
 * `ws` (optional): a workspace of bsa_workspace_size() bytes, 256-byte aligned.
 * With it, the video query tiles run as a persistent grid whose blocks, per
 * XCD, sweep the key tiles in step so that a key tile is fetched once into the
 * XCD's L2 for all of them; without it (NULL), one block per query tile.  The
 * results are the same either way.  Calls given the same workspace must not
 * run concurrently.
 * The grouped launch relies on two things the hardware does but no API
 * promises: the blocks of one launch are dispatched to the 8 XCDs round-robin
 * (block b to XCD b mod 8), and all of its blocks (one per CU) are resident at
 * once.  The wait at the start of each round is bounded, so results never
 * depend on either; if one fails, rounds start out of step and the run is
 * slower.  The workspace then records, per call, how many rounds' start
 * waits gave up (see bsa_forward_stats_offset).
 */
bsa_status bsa_forward(const bsa_desc *desc, const void *q_tiled, const void *k_frag,
                       const void *v_frag, const int32_t *block_idx, void *o_tiled, float *lse,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * bsa_forward's grouped launch without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The launch's round counters (2 KB)
 * live in a file-scope device array of the library (4 KB, one copy per GPU,
 * held until the process ends) instead of a workspace; this entry point
 * calls no allocator.  Arguments, layouts, results and errors as bsa_forward
 * (every problem size bsa_forward accepts fits the array; BSA_ERR_UNSUPPORTED
 * otherwise).  Every call on a GPU shares that GPU's array, which each call
 * clears on its stream first: calls that overlap on one GPU race.
 */
bsa_status bsa_forward_noalloc(const bsa_desc *desc, const void *q_tiled, const void *k_frag,
                               const void *v_frag, const int32_t *block_idx, void *o_tiled,
                               float *lse, void *stream);

/*
 * bsa_forward with Q read from, and O written to, the raster layout through
 * `perm` (bsa_permute(BUILD)), the token permutation applied inside the
 * kernel ("Sparse VideoGen TPU 최적화", section "실무에서 배울 최적화 기준":
 * the reordering is a cost of its own, to be kept small).  The result equals
 * bsa_permute(GATHER) of Q, bsa_forward, then bsa_permute(SCATTER) of O, bit
 * for bit, without the tiled copies of Q and O: each query tile's 64 token
 * rows are read and its 64 output rows written (256-byte head rows for
 * D = 128) at their raster positions.  Padding slots of a ragged grid read
 * zeros and are not written.  `q_raster` and `o_raster` bf16 [B][Ntot][H][D]
 * (Ntot counting the real tokens), `perm` int32 [B][Nvideo]; `k_frag`,
 * `v_frag`, `block_idx`, `lse` (tiled [B][H][Ntot], padding slots included),
 * `ws` and the errors as bsa_forward.  o_raster, lse and the workspace's
 * counters must not overlap each other, q_raster, perm, k_frag, v_frag or
 * block_idx (BSA_ERR_ARG).
 */
bsa_status bsa_forward_raster(const bsa_desc *desc, const void *q_raster, const int32_t *perm,
                              const void *k_frag, const void *v_frag, const int32_t *block_idx,
                              void *o_raster, float *lse, void *ws, size_t ws_bytes, void *stream);

/*
 * Byte offset, inside the workspace of bsa_workspace_size(desc), of the
 * forward's statistics: int32 stats[2], cleared at the start of every
 * bsa_forward / bsa_forward_csr call given a workspace and, when its work has
 * run, stats[0] = block rounds of the grouped launch (one per video query
 * tile) whose bounded start wait gave up before every block of the group had
 * arrived (0 when the lock step held), stats[1] = block rounds started.
 * Host-only.
 */
bsa_status bsa_forward_stats_offset(const bsa_desc *desc, size_t *offset);

/*
 * Variable keep: per-head and per-row keep counts with the kept lists in CSR
 * form.  The pages keep a fixed share per call ("Prism / Kandinsky 6 speed
 * ablation", section "같은 계산량 안에서 볼 곳을 고르는 Prism": sparsity s keeps
 * (1 - s) of the key tiles); these entry points let that share differ per
 * head or per query tile, with the same selection rule and the same
 * attention kernel.
 *
 *   keep_per_head  host int32 [H], each in 1..nVT; NULL: desc->keep_tiles for
 *                  every head.  At most BSA_MAX_CSR_HEADS heads.
 *   keep_rows      device int32 [B][H][nVT] or NULL: video query tile i of
 *                  (b, h) keeps min(max(keep_rows[b][h][i], 1), keep_per_head[h])
 *                  tiles (keep_per_head[h] when NULL).
 *   row_ptr        device int64 [B*H*nVT + 1]: row r = (b*H + h)*nVT + i holds
 *                  col_idx[row_ptr[r] .. row_ptr[r+1]); row_ptr[0] = 0.
 *   col_idx        device int32, col_entries entries: the kept video tiles of
 *                  each row, ascending.
 *
 * bsa_csr_entries (host only) gives the entries col_idx needs at most:
 * B * nVT * sum_h keep_per_head[h].
 * bsa_plan_csr writes row_ptr and col_idx: the selection of bsa_plan with
 * each row's own count (the largest scores, equal scores to the lower tile
 * number); col_entries below bsa_csr_entries gives BSA_ERR_SHAPE.  Uses the
 * workspace of bsa_workspace_size.
 * bsa_forward_csr is bsa_forward with the lists read from row_ptr/col_idx;
 * each row must hold 1..nVT entries (row bounds are clamped to that and to
 * col_entries, so a corrupt row_ptr cannot address outside col_idx).  Its
 * outputs must not overlap each other or an input, row_ptr and the first
 * col_entries entries of col_idx included (BSA_ERR_ARG).
 */
#define BSA_MAX_CSR_HEADS 256
bsa_status bsa_csr_entries(const bsa_desc *desc, const int32_t *keep_per_head, int64_t *entries);
bsa_status bsa_plan_csr(const bsa_desc *desc, const void *q_tiled, const void *k_frag,
                        const int32_t *keep_per_head, const int32_t *keep_rows, int64_t *row_ptr,
                        int32_t *col_idx, int64_t col_entries, void *ws, size_t ws_bytes, void *stream);
/*
 * The row pointers, scoring and top-k of bsa_plan_csr alone, from the tile
 * means that bsa_permute(POOL or GATHER_POOL) and bsa_permute(GATHER_KF_POOL)
 * (or an earlier plan) left in the workspace: the CSR counterpart of
 * bsa_select.  Same output and errors as bsa_plan_csr.
 */
bsa_status bsa_select_csr(const bsa_desc *desc, const int32_t *keep_per_head, const int32_t *keep_rows,
                          int64_t *row_ptr, int32_t *col_idx, int64_t col_entries, void *ws, size_t ws_bytes,
                          void *stream);
bsa_status bsa_forward_csr(const bsa_desc *desc, const void *q_tiled, const void *k_frag,
                           const void *v_frag, const int64_t *row_ptr, const int32_t *col_idx,
                           int64_t col_entries, void *o_tiled, float *lse, void *ws, size_t ws_bytes,
                           void *stream);
/*
 * bsa_forward_csr with Q read from, and O written to, the raster layout
 * through `perm`, as bsa_forward_raster does for fixed keep: the same result
 * bit for bit as GATHER -> bsa_forward_csr -> SCATTER, without the tiled
 * copies.  Arguments and errors as bsa_forward_csr and bsa_forward_raster.
 */
bsa_status bsa_forward_csr_raster(const bsa_desc *desc, const void *q_raster, const int32_t *perm,
                                  const void *k_frag, const void *v_frag, const int64_t *row_ptr,
                                  const int32_t *col_idx, int64_t col_entries, void *o_raster, float *lse,
                                  void *ws, size_t ws_bytes, void *stream);

/*
 * Structured lists: kept tiles from a fixed spatial or temporal rule per head
 * instead of scores.  "Sparse VideoGen TPU 최적화" (aibase.it), section
 * "Sparse VideoGen의 핵심 아이디어": attention heads are mostly spatial (a
 * query looks at patches of its own or nearby frames) or temporal (it follows
 * its spatial position across frames); section "실무에서 배울 최적화 기준": with
 * tokens permuted into tiles such masks select whole tiles.  Static tile modes
 * only (BSA_ERR_UNSUPPORTED in dynamic mode; a ragged grid uses its rounded-up
 * tile grid).  In the tile grid (Tt x Th x Tw
 * tiles, video tile (t, h, w) numbered (t*Th + h)*Tw + w), video query tile
 * (ti, hi, wi) of a head keeps
 *   BSA_MASK_SPATIAL:  every tile (t, h, w) with |t - ti| <= radius_t;
 *   BSA_MASK_TEMPORAL: every tile (t, h, w) with |h - hi| <= radius_hw and
 *                      |w - wi| <= radius_hw,
 * ascending, written as CSR lists (row_ptr / col_idx as for bsa_plan_csr) for
 * bsa_forward_csr; the prefix stays dense.  head_mask: host int32 [H] of
 * BSA_MASK_* (at most BSA_MAX_CSR_HEADS heads); radii >= 0 (BSA_ERR_ARG
 * otherwise).  bsa_structured_entries (host only) gives the exact entry count;
 * a smaller col_entries gives BSA_ERR_SHAPE.  No workspace.
 */
enum { BSA_MASK_SPATIAL = 0, BSA_MASK_TEMPORAL = 1 };
bsa_status bsa_structured_entries(const bsa_desc *desc, const int32_t *head_mask, int32_t radius_t,
                                  int32_t radius_hw, int64_t *entries);
bsa_status bsa_plan_structured(const bsa_desc *desc, const int32_t *head_mask, int32_t radius_t,
                               int32_t radius_hw, int64_t *row_ptr, int32_t *col_idx,
                               int64_t col_entries, void *stream);

/*
 * Bytes of device workspace that bsa_backward needs for `desc` (about seven
 * times the size of one bf16 [B][H][Ntot][D] tensor: the fragment-layout
 * copies of Q, K, V and dO the gradient kernels stream).  Host-only.
 */
bsa_status bsa_backward_workspace_size(const bsa_desc *desc, size_t *bytes);

/*
 * Gradients of bsa_forward's output.  The pages give no backward; Prism's
 * page ("Prism / Kandinsky 6 speed ablation", section "같은 계산량 안에서 볼 곳을
 * 고르는 Prism") reports that the same block sparsity speeds up training, which
 * needs dQ, dK and dV over the same kept lists.  This is the exact derivative
 * of the function bsa_forward computes: for query q with key set S_q (its
 * kept tiles and the prefix; every token for a prefix query),
 * P_qj = exp(scale q.k_j - lse_q), Delta_q = dO_q . O_q,
 * dS_qj = P_qj (dO_q . v_j - Delta_q):
 *   dQ_q = scale sum_{j in S_q} dS_qj k_j,
 *   dK_j = scale sum_{q: j in S_q} dS_qj q_q,   dV_j = sum_{q: j in S_q} P_qj dO_q.
 * Arguments:
 *   q, k, v, o, d_o  bf16 raster [B][Ntot][H][D]: the forward's inputs, its
 *                    output o and dL/do;
 *   lse              float [B][H][Ntot] from bsa_forward (tiled order);
 *   perm             int32 [B][Nvideo] from bsa_permute(BUILD);
 *   block_idx        int32 [B][H][nVT][k] from bsa_plan (NULL only without video);
 *   dq, dk, dv       bf16 raster [B][Ntot][H][D], overwritten;
 *   ws               bsa_backward_workspace_size() bytes, 256-byte aligned.
 * Products are bf16 MFMAs with float accumulation; P and dS are rounded to
 * bf16 before their products, the gradients to bf16 at the end.  Tensors must
 * be 16-byte aligned (lse, perm, block_idx 4-byte); at most BSA_MAX_TILES
 * tiles and BSA_MAX_VIDEO_TILES video tiles per (batch, head).  Calls given the
 * same workspace must not run concurrently.  dq, dk and dv must not overlap
 * each other, an input or the workspace (BSA_ERR_ARG, nothing enqueued).  On
 * a ragged grid
 * (BSA_TILE_STATIC_PADDED) the gradients are those of the padded forward:
 * padding keys take no weight, padding slots are neither read nor written
 * (perm -1), and the lse is the forward's over the padded tiled order.
 */
bsa_status bsa_backward(const bsa_desc *desc, const void *q, const void *k, const void *v,
                        const void *o, const void *d_o, const float *lse, const int32_t *perm,
                        const int32_t *block_idx, void *dq, void *dk, void *dv, void *ws,
                        size_t ws_bytes, void *stream);

/*
 * The backward over CSR kept lists (bsa_plan_csr / bsa_plan_structured,
 * consumed by bsa_forward_csr): the same gradients as bsa_backward, with
 * video query tile i of (b, h) keeping the video tiles
 * col_idx[row_ptr[r] .. row_ptr[r+1]), r = (b*H + h)*nVT + i, clamped as
 * bsa_forward_csr clamps them.  The transposed lists take col_entries int32
 * of workspace: bsa_backward_csr_workspace_size(desc, col_entries) gives the
 * size.  row_ptr must be non-decreasing from 0 with distinct entries per row
 * (as the planners write it); other lists stay memory-safe but their
 * gradients are unspecified.  Other arguments, layouts and errors as
 * bsa_backward (row_ptr 8-byte aligned; col_entries < 1 with video:
 * BSA_ERR_SHAPE).
 */
bsa_status bsa_backward_csr_workspace_size(const bsa_desc *desc, int64_t col_entries, size_t *bytes);
bsa_status bsa_backward_csr(const bsa_desc *desc, const void *q, const void *k, const void *v,
                            const void *o, const void *d_o, const float *lse, const int32_t *perm,
                            const int64_t *row_ptr, const int32_t *col_idx, int64_t col_entries,
                            void *dq, void *dk, void *dv, void *ws, size_t ws_bytes, void *stream);

/*
 * Byte offset of the gradient launches' statistics inside the backward
 * workspace: int32 stats[4], cleared at the start of every bsa_backward /
 * bsa_backward_csr call and, when its work has run, stats[0] = block rounds
 * of the grouped dQ launch whose bounded start wait gave up before every
 * block of its XCD group arrived, stats[1] = block rounds started (one per
 * query tile), stats[2], stats[3] = the same for the dK/dV launch (one round
 * per key tile).  col_entries = 0: the workspace of bsa_backward_workspace_size;
 * > 0: that of bsa_backward_csr_workspace_size(desc, col_entries).  Like the
 * forward's, the waits only shape the schedule (results never depend on
 * them).  Host-only.
 */
bsa_status bsa_backward_stats_offset(const bsa_desc *desc, int64_t col_entries, size_t *offset);

/* Static text for a status code. */
const char *bsa_status_string(bsa_status status);

/* ABI version of this header (major * 100 + minor). */
int bsa_version(void);

#define BSA_VERSION 1003

#ifdef __cplusplus
}
#endif
#endif /* BSA_H */
