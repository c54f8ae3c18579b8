/*
 * bsa_oracle.c -- slow, plain CPU oracle for block-sparse self-attention on a
 * video token grid.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load this library.  It shares no
 * source, header, table or helper with the GPU library, and the GPU library
 * never calls it.
 *
 * Every step is written out in the order the method takes it, in double
 * precision unless a step fixes another precision.  Sources, by page title and
 * section:
 *
 *  [Prism]  "Prism / Kandinsky 6 speed ablation" (oh-my-gpu.com GPU-hardware blog),
 *           section "같은 계산량 안에서 볼 곳을 고르는 Prism" (Prism picks where to
 *           look within the same compute): tokens are grouped into 64-token blocks;
 *           each query block computes attention only against the key blocks judged
 *           most relevant; sparsity s is the fraction of key blocks skipped (s = 0.75
 *           keeps 480 of 1,920); relevance is judged from the mean of a block's 64
 *           tokens; the default block is 4x4x4 (t,h,w); with dynamic blocks the video
 *           is cut into 8x8x8 token regions and, per region, the axis that varies most
 *           is given the short extent while the block stays at 64 tokens.
 *           Section "토큰 수의 제곱으로 느는 어텐션 비용": the 720p/121-frame grid is
 *           32 x 48 x 80 (t,h,w) tokens including padding.
 *  [SVG]    "Sparse VideoGen TPU 최적화: 비디오 생성 추론 지연을 줄이는 실무 기준"
 *           (aibase.it), section "이론적 sparsity와 물리적 sparsity의 차이": tiles are
 *           full, boundary or empty; empty tiles are skipped entirely.  Section
 *           "실무에서 배울 최적화 기준": tokens are permuted so a pattern's tiles are
 *           contiguous.
 *  [VSA]    "RTX 4090에서 5초 영상 72초: Ref2VA VSA" (pulmap.app), section
 *           "조건 토큰은 왜 다르게 다루나": conditioning tokens sit in segment-pure
 *           tiles, receive fully dense attention and are never pruned; top-k pruning
 *           applies to the video key tiles only.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes): the pooled score is the plain dot product of the two pooled
 * vectors; selection is per (batch, head, query tile); equal scores are ordered
 * by lowest key-tile index; kept lists are emitted in ascending order; prefix
 * queries attend to every key; the dynamic-shape rule is the one in
 * orc_shape_choose below.
 *
 * Layouts (all row-major):
 *   raster  [B][Ntot][H][D]  prefix tokens first, then the video grid in (t,h,w) raster
 *   tiled   [B][H][Ntot][D]  prefix unchanged, then video tokens in tile order
 *   perm    [B][Nvid]        tiled video slot -> raster video token index
 * bf16 values are passed as their uint16 bit patterns.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define TILE 64

/* bf16 bit pattern -> exact double (bf16 is the upper half of an IEEE float). */
static double bf16_to_double(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Tile numbering and the token permutation                                  */
/* ------------------------------------------------------------------------ */

/*
 * Static tiles [Prism, default 4x4x4 block; SVG, token permutation].
 * Tile id = raster position of the tile in the (T/tt, H/th, W/tw) tile grid
 * (t slowest); inside a tile the 64 tokens are in (t,h,w) raster order.
 * perm[p] = raster index of the token stored at tiled slot p.
 * Returns 0, or -1 if the grid is not divisible by the tile.
 */
int orc_perm_static(int T, int Hg, int W, int tt, int th, int tw, int32_t *perm)
{
    if (tt * th * tw != TILE || T % tt || Hg % th || W % tw)
        return -1;
    int64_t p = 0;
    for (int a = 0; a < T / tt; ++a)
        for (int b = 0; b < Hg / th; ++b)
            for (int c = 0; c < W / tw; ++c)
                for (int x = 0; x < tt; ++x)
                    for (int y = 0; y < th; ++y)
                        for (int z = 0; z < tw; ++z) {
                            int t = a * tt + x, h = b * th + y, w = c * tw + z;
                            perm[p++] = (int32_t)(((int64_t)t * Hg + h) * W + w);
                        }
    return 0;
}

/* The nine 64-token shapes (extent along t, h, w).  Ids 0..6 fit an 8x8x8
 * region; 7 and 8 are 16 long and need two regions. */
static const int SHAPES[9][3] = {
    {4, 4, 4}, {2, 4, 8}, {2, 8, 4}, {8, 4, 2}, {4, 2, 8},
    {4, 8, 2}, {8, 2, 4}, {2, 2, 16}, {16, 2, 2},
};

int orc_shape_extent(int id, int axis)
{
    if (id < 0 || id > 8 || axis < 0 || axis > 2)
        return -1;
    return SHAPES[id][axis];
}

/*
 * Per-region variation statistic [Prism, dynamic blocks]: for batch b and
 * 8x8x8 region r, v[a] = mean over every adjacent token pair (x, x+e_a) with
 * both tokens inside the region, over all heads and channels, of
 * |Q[x+e_a] - Q[x]|, for a in (t, h, w).  Accumulated in double.
 * q_raster: [B][n_prefix + T*Hg*W][H][D] bf16.  stats: [B][R][3].
 */
void orc_shape_stats(const uint16_t *q_raster, int B, int n_prefix, int T, int Hg,
                     int W, int H, int D, double *stats)
{
    const int RT = T / 8, RH = Hg / 8, RW = W / 8, R = RT * RH * RW;
    const int64_t Ntot = (int64_t)n_prefix + (int64_t)T * Hg * W;
    const int64_t row = (int64_t)H * D; /* elements per token */
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b)
        for (int r = 0; r < R; ++r) {
            int rt = r / (RH * RW), rh = (r / RW) % RH, rw = r % RW;
            double sum[3] = {0.0, 0.0, 0.0};
            int64_t cnt[3] = {0, 0, 0};
            for (int x = 0; x < 8; ++x)
                for (int y = 0; y < 8; ++y)
                    for (int z = 0; z < 8; ++z) {
                        int t = rt * 8 + x, h = rh * 8 + y, w = rw * 8 + z;
                        int64_t tok = n_prefix + ((int64_t)t * Hg + h) * W + w;
                        const uint16_t *a0 = q_raster + ((int64_t)b * Ntot + tok) * row;
                        for (int ax = 0; ax < 3; ++ax) {
                            int inside = (ax == 0) ? (x + 1 < 8) : (ax == 1) ? (y + 1 < 8) : (z + 1 < 8);
                            if (!inside)
                                continue;
                            int64_t step = (ax == 0) ? (int64_t)Hg * W : (ax == 1) ? W : 1;
                            const uint16_t *a1 = a0 + step * row;
                            for (int64_t e = 0; e < row; ++e)
                                sum[ax] += fabs(bf16_to_double(a1[e]) - bf16_to_double(a0[e]));
                            cnt[ax] += row;
                        }
                    }
            for (int ax = 0; ax < 3; ++ax)
                stats[((int64_t)b * R + r) * 3 + ax] = sum[ax] / (double)cnt[ax];
        }
}

/* |x - y| within rel of the larger magnitude (or both zero). */
static int near_equal(double x, double y, double rel)
{
    double m = fmax(fabs(x), fabs(y));
    return fabs(x - y) <= rel * m;
}

/*
 * Shape choice per region from its statistic (reading of [Prism, dynamic
 * blocks]; the page states the principle, this is the plainest rule that
 * follows it and yields exactly the nine listed shapes):
 *   1. Order the axes by v, largest first; equal values rank t before h before w.
 *      Call them a1, a2, a3.
 *   2. If v[a1] <= (1+tau) v[a3] the region is isotropic: 4x4x4.
 *   3. Otherwise the box: extent 2 on a1, 4 on a2, 8 on a3.
 *   4. If also v[a2] > (1+tau) v[a3] and the calm axis a3 is w (resp. t), the
 *      region asks for the 16-long shape 2x2x16 (resp. 16x2x2).  Regions are
 *      paired along that axis, (0,1), (2,3), ...; a pair takes the long shape
 *      only if both regions ask for the same long shape, otherwise each region
 *      keeps its box.  A region without a partner keeps its box.
 * near[]: 1 when any comparison above is within rel_eps (relative) of flipping;
 * a paired region inherits its partner's flag.
 * shape: [B][R] shape ids; near may be NULL.
 */
void orc_shape_choose(const double *stats, int B, int T, int Hg, int W, double tau,
                      double rel_eps, uint8_t *shape, uint8_t *near)
{
    const int RT = T / 8, RH = Hg / 8, RW = W / 8, R = RT * RH * RW;
    uint8_t *want_long = (uint8_t *)calloc((size_t)B * R, 1); /* 0, 7 or 8 */
    uint8_t *flag = (uint8_t *)calloc((size_t)B * R, 1);
    for (int b = 0; b < B; ++b)
        for (int r = 0; r < R; ++r) {
            const double *v = stats + ((int64_t)b * R + r) * 3;
            int ord[3] = {0, 1, 2};
            /* stable sort by v descending: ties keep t < h < w order */
            for (int i = 0; i < 3; ++i)
                for (int j = 0; j + 1 < 3 - i; ++j)
                    if (v[ord[j + 1]] > v[ord[j]]) {
                        int tmp = ord[j];
                        ord[j] = ord[j + 1];
                        ord[j + 1] = tmp;
                    }
            int a1 = ord[0], a2 = ord[1], a3 = ord[2];
            double lim = (1.0 + tau) * v[a3];
            int f = near_equal(v[0], v[1], rel_eps) || near_equal(v[1], v[2], rel_eps) ||
                    near_equal(v[0], v[2], rel_eps) || near_equal(v[a1], lim, rel_eps);
            int id = 0;
            if (v[a1] > lim) {
                int ext[3];
                ext[a1] = 2;
                ext[a2] = 4;
                ext[a3] = 8;
                for (int s = 1; s <= 6; ++s)
                    if (SHAPES[s][0] == ext[0] && SHAPES[s][1] == ext[1] && SHAPES[s][2] == ext[2])
                        id = s;
                f = f || near_equal(v[a2], lim, rel_eps);
                if (v[a2] > lim) {
                    if (a3 == 2)
                        want_long[(int64_t)b * R + r] = 7;
                    else if (a3 == 0)
                        want_long[(int64_t)b * R + r] = 8;
                }
            }
            shape[(int64_t)b * R + r] = (uint8_t)id;
            flag[(int64_t)b * R + r] = (uint8_t)f;
        }
    /* pairing of 16-long requests */
    for (int b = 0; b < B; ++b)
        for (int r = 0; r < R; ++r) {
            int64_t i = (int64_t)b * R + r;
            int lw = want_long[i];
            if (!lw)
                continue;
            int rt = r / (RH * RW), rh = (r / RW) % RH, rw = r % RW;
            int pos = (lw == 7) ? rw : rt;
            int cnt = (lw == 7) ? RW : RT;
            int partner_pos = (pos % 2 == 0) ? pos + 1 : pos - 1;
            if (partner_pos >= cnt)
                continue;
            int pr = (lw == 7) ? (rt * RH + rh) * RW + partner_pos : (partner_pos * RH + rh) * RW + rw;
            int64_t pi = (int64_t)b * R + pr;
            if (want_long[pi] == lw)
                shape[i] = (uint8_t)lw;
        }
    if (near)
        for (int b = 0; b < B; ++b)
            for (int r = 0; r < R; ++r) {
                int64_t i = (int64_t)b * R + r;
                int f = flag[i];
                int lw = want_long[i];
                if (lw) { /* the pair decision depends on the partner too */
                    int rt = r / (RH * RW), rh = (r / RW) % RH, rw = r % RW;
                    int pos = (lw == 7) ? rw : rt, cnt = (lw == 7) ? RW : RT;
                    int pp = (pos % 2 == 0) ? pos + 1 : pos - 1;
                    if (pp < cnt) {
                        int pr = (lw == 7) ? (rt * RH + rh) * RW + pp : (pp * RH + rh) * RW + rw;
                        f = f || flag[(int64_t)b * R + pr];
                    }
                }
                near[i] = (uint8_t)f;
            }
    free(want_long);
    free(flag);
}

/*
 * Tile numbering with dynamic shapes: regions in (t,h,w) raster order, 8 tile
 * slots per region; inside a region its 8 tiles in raster order of the tile
 * grid, tokens raster inside each tile.  A pair of regions sharing a 16-long
 * shape is cut into 16 tiles, raster over the pair's extent; the first 8 fill
 * the lower region's slots and the last 8 the upper region's slots.
 * Returns 0, or -1 on an invalid shape map.
 */
int orc_perm_dynamic(const uint8_t *shape, int B, int T, int Hg, int W, int32_t *perm)
{
    const int RT = T / 8, RH = Hg / 8, RW = W / 8, R = RT * RH * RW;
    const int64_t Nv = (int64_t)T * Hg * W;
    if (T % 8 || Hg % 8 || W % 8)
        return -1;
    for (int b = 0; b < B; ++b) {
        int32_t *pb = perm + (int64_t)b * Nv;
        for (int r = 0; r < R; ++r) {
            int id = shape[(int64_t)b * R + r];
            if (id > 8)
                return -1;
            int rt = r / (RH * RW), rh = (r / RW) % RH, rw = r % RW;
            int o[3] = {rt * 8, rh * 8, rw * 8}; /* origin of the block of tiles */
            int ext[3] = {8, 8, 8};
            int slot0 = r * 8, skip = 0;
            int upper_slot = -1;
            if (id >= 7) {
                int pos = (id == 7) ? rw : rt;
                int pr;
                if (pos % 2 == 1) { /* upper region of a pair: written by the lower one */
                    pr = (id == 7) ? r - 1 : r - RH * RW;
                    if (shape[(int64_t)b * R + pr] != id)
                        return -1;
                    skip = 1;
                } else {
                    pr = (id == 7) ? r + 1 : r + RH * RW;
                    if ((id == 7 && rw + 1 >= RW) || (id == 8 && rt + 1 >= RT) ||
                        shape[(int64_t)b * R + pr] != id)
                        return -1;
                    upper_slot = pr * 8;
                    if (id == 7)
                        ext[2] = 16;
                    else
                        ext[0] = 16;
                }
            }
            if (skip)
                continue;
            const int *e = SHAPES[id];
            int n = 0; /* tile counter inside this block */
            for (int a = 0; a < ext[0] / e[0]; ++a)
                for (int bb = 0; bb < ext[1] / e[1]; ++bb)
                    for (int c = 0; c < ext[2] / e[2]; ++c, ++n) {
                        int slot = (n < 8) ? slot0 + n : upper_slot + (n - 8);
                        int64_t p = (int64_t)slot * TILE;
                        for (int x = 0; x < e[0]; ++x)
                            for (int y = 0; y < e[1]; ++y)
                                for (int z = 0; z < e[2]; ++z) {
                                    int t = o[0] + a * e[0] + x;
                                    int h = o[1] + bb * e[1] + y;
                                    int w = o[2] + c * e[2] + z;
                                    pb[p++] = (int32_t)(((int64_t)t * Hg + h) * W + w);
                                }
                    }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Gather / scatter [SVG, token permutation]: exact bf16 copies              */
/* ------------------------------------------------------------------------ */

void orc_gather(const uint16_t *src_raster, const int32_t *perm, int B, int n_prefix,
                int64_t Nv, int H, int D, uint16_t *dst_tiled)
{
    const int64_t Ntot = n_prefix + Nv;
#pragma omp parallel for collapse(2)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int64_t p = 0; p < Ntot; ++p) {
                int64_t tok = (p < n_prefix) ? p : n_prefix + perm[(int64_t)b * Nv + (p - n_prefix)];
                const uint16_t *s = src_raster + (((int64_t)b * Ntot + tok) * H + h) * D;
                uint16_t *d = dst_tiled + (((int64_t)b * H + h) * Ntot + p) * D;
                memcpy(d, s, (size_t)D * sizeof(uint16_t));
            }
}

void orc_scatter(const uint16_t *src_tiled, const int32_t *perm, int B, int n_prefix,
                 int64_t Nv, int H, int D, uint16_t *dst_raster)
{
    const int64_t Ntot = n_prefix + Nv;
#pragma omp parallel for collapse(2)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int64_t p = 0; p < Ntot; ++p) {
                int64_t tok = (p < n_prefix) ? p : n_prefix + perm[(int64_t)b * Nv + (p - n_prefix)];
                const uint16_t *s = src_tiled + (((int64_t)b * H + h) * Ntot + p) * D;
                uint16_t *d = dst_raster + (((int64_t)b * Ntot + tok) * H + h) * D;
                memcpy(d, s, (size_t)D * sizeof(uint16_t));
            }
}

/* ------------------------------------------------------------------------ */
/* Pooling [Prism: a block is judged by the mean of its 64 tokens]           */
/* ------------------------------------------------------------------------ */

/*
 * out[b][h][i][d] = (sum of the 64 values of video tile i, channel d) / 64,
 * summed in double and rounded once to float.  Prefix tiles are not pooled:
 * they are never scored [VSA].
 * x_tiled: [B][H][n_prefix + nvt*64][D]; out: [B][H][nvt][D].
 */
void orc_pool(const uint16_t *x_tiled, int B, int H, int n_prefix, int nvt, int D, float *out)
{
    const int64_t Ntot = n_prefix + (int64_t)nvt * TILE;
#pragma omp parallel for collapse(2)
    for (int bh = 0; bh < B * H; ++bh)
        for (int i = 0; i < nvt; ++i)
            for (int d = 0; d < D; ++d) {
                double s = 0.0;
                for (int r = 0; r < TILE; ++r)
                    s += bf16_to_double(x_tiled[((int64_t)bh * Ntot + n_prefix + (int64_t)i * TILE + r) * D + d]);
                out[((int64_t)bh * nvt + i) * D + d] = (float)(s / TILE);
            }
}

/* ------------------------------------------------------------------------ */
/* Score and top-k [Prism: per query block keep the best (1-s) of key blocks] */
/* ------------------------------------------------------------------------ */

typedef struct {
    double s;
    int j;
} scored;

/* order: higher score first; equal scores: lower index first */
static int cmp_scored(const void *a, const void *b)
{
    const scored *x = (const scored *)a, *y = (const scored *)b;
    if (x->s > y->s)
        return -1;
    if (x->s < y->s)
        return 1;
    return (x->j > y->j) - (x->j < y->j);
}

static int cmp_int(const void *a, const void *b)
{
    int x = *(const int *)a, y = *(const int *)b;
    return (x > y) - (x < y);
}

/*
 * For every (b,h) and the query tiles listed in rows[0..nrows) (all tiles if
 * rows is NULL): s_ij = sum_d qp[i][d] * kp[j][d] in double from the float
 * pooled vectors; the kept set is the first k of j ordered by (-s_ij, j),
 * written in ascending j order to idx[b][h][row][0..k).
 * Per row also: s_k (k-th largest), s_k1 ((k+1)-th, or NaN when k == n) and
 * mag = the larger of sum_d |qp_i[d] kp_j[d]| over the k-th and (k+1)-th
 * entries (what bounds the rounding error of a single-precision evaluation of
 * the two scores that decide the boundary).  Any of these may be NULL.
 * qp, kp: [B][H][n][D]; idx: [B][H][nrows][k]; s_k, s_k1, mag: [B][H][nrows].
 */
void orc_topk(const float *qp, const float *kp, int B, int H, int n, int D, int k,
              const int32_t *rows, int nrows, int32_t *idx, double *s_k, double *s_k1,
              double *mag)
{
    if (!rows)
        nrows = n;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int bh = 0; bh < B * H; ++bh)
        for (int rr = 0; rr < nrows; ++rr) {
            int i = rows ? rows[rr] : rr;
            const float *q = qp + ((int64_t)bh * n + i) * D;
            scored *sc = (scored *)malloc(sizeof(scored) * (size_t)n);
            int *keep = (int *)malloc(sizeof(int) * (size_t)k);
            for (int j = 0; j < n; ++j) {
                const float *kk = kp + ((int64_t)bh * n + j) * D;
                double s = 0.0;
                for (int d = 0; d < D; ++d)
                    s += (double)q[d] * (double)kk[d];
                sc[j].s = s;
                sc[j].j = j;
            }
            qsort(sc, (size_t)n, sizeof(scored), cmp_scored);
            double mx = 0.0;
            for (int t = k - 1; t <= k && t < n; ++t) {
                const float *kk = kp + ((int64_t)bh * n + sc[t].j) * D;
                double a = 0.0;
                for (int d = 0; d < D; ++d)
                    a += fabs((double)q[d] * (double)kk[d]);
                if (a > mx)
                    mx = a;
            }
            for (int t = 0; t < k; ++t)
                keep[t] = sc[t].j;
            qsort(keep, (size_t)k, sizeof(int), cmp_int);
            int64_t o = (int64_t)bh * nrows + rr;
            memcpy(idx + o * k, keep, sizeof(int32_t) * (size_t)k);
            if (s_k)
                s_k[o] = sc[k - 1].s;
            if (s_k1)
                s_k1[o] = (k < n) ? sc[k].s : NAN;
            if (mag)
                mag[o] = mx;
            free(sc);
            free(keep);
        }
}

/* ------------------------------------------------------------------------ */
/* Attention over the kept tiles [Prism; SVG: empty tiles skipped, kept tiles */
/* full; VSA: dense prefix]                                                  */
/* ------------------------------------------------------------------------ */

/*
 * Exact softmax attention in double for one (b,h) slice of tiled tensors.
 * Query tile qt (tiled numbering: prefix tiles 0..npt-1, then video tiles):
 *   - a prefix query tile attends to every token;
 *   - video query tile i attends to all prefix tokens and to the tokens of the
 *     kept video tiles idx[i][0..k).
 * For each query token: z_j = scale * (q . k_j); w_j = exp(z_j - max z);
 * o = sum_j w_j v_j / sum_j w_j; lse = max z + log(sum_j w_j).
 * q,k,v: [n_prefix + nvt*64][D] bf16 of one (b,h); idx: [nvt][k] of that (b,h).
 * qtiles[0..nq): tiled query tile numbers; out: [nq][64][D]; lse: [nq][64] (may be NULL).
 */
void orc_attention(const uint16_t *q, const uint16_t *kx, const uint16_t *v, int n_prefix,
                   int nvt, int D, int k, const int32_t *idx, double scale,
                   const int32_t *qtiles, int nq, double *out, double *lse)
{
    const int npt = n_prefix / TILE;
    const int64_t Ntot = n_prefix + (int64_t)nvt * TILE;
#pragma omp parallel for schedule(dynamic)
    for (int a = 0; a < nq; ++a) {
        int qt = qtiles[a];
        /* the key token list */
        int64_t nkeys;
        int64_t *keys;
        if (qt < npt) {
            nkeys = Ntot;
            keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)nkeys);
            for (int64_t j = 0; j < Ntot; ++j)
                keys[j] = j;
        } else {
            int i = qt - npt;
            nkeys = n_prefix + (int64_t)k * TILE;
            keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)nkeys);
            int64_t c = 0;
            for (int64_t j = 0; j < n_prefix; ++j)
                keys[c++] = j;
            for (int t = 0; t < k; ++t) {
                int64_t base = n_prefix + (int64_t)idx[(int64_t)i * k + t] * TILE;
                for (int r = 0; r < TILE; ++r)
                    keys[c++] = base + r;
            }
        }
        double *z = (double *)malloc(sizeof(double) * (size_t)nkeys);
        double *qd = (double *)malloc(sizeof(double) * (size_t)D);
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
        for (int r = 0; r < TILE; ++r) {
            int64_t qi = (int64_t)qt * TILE + r;
            for (int d = 0; d < D; ++d)
                qd[d] = bf16_to_double(q[qi * D + d]);
            double mx = -INFINITY;
            for (int64_t j = 0; j < nkeys; ++j) {
                const uint16_t *kr = kx + keys[j] * D;
                double s = 0.0;
                for (int d = 0; d < D; ++d)
                    s += qd[d] * bf16_to_double(kr[d]);
                z[j] = s * scale;
                if (z[j] > mx)
                    mx = z[j];
            }
            double den = 0.0;
            for (int d = 0; d < D; ++d)
                acc[d] = 0.0;
            for (int64_t j = 0; j < nkeys; ++j) {
                double w = exp(z[j] - mx);
                den += w;
                const uint16_t *vr = v + keys[j] * D;
                for (int d = 0; d < D; ++d)
                    acc[d] += w * bf16_to_double(vr[d]);
            }
            for (int d = 0; d < D; ++d)
                out[((int64_t)a * TILE + r) * D + d] = acc[d] / den;
            if (lse)
                lse[(int64_t)a * TILE + r] = mx + log(den);
        }
        free(z);
        free(qd);
        free(acc);
        free(keys);
    }
}

/*
 * Attention with a kept list of its own length per video query tile (variable
 * keep per head or per query tile, lists in CSR form): as orc_attention, with
 * video query tile i attending to all prefix tokens and to the tokens of the
 * video tiles col[row_ptr[i] .. row_ptr[i+1]).  row_ptr: [nvt + 1] of one
 * (b,h); col: the entries it points into.
 */
void orc_attention_csr(const uint16_t *q, const uint16_t *kx, const uint16_t *v, int n_prefix,
                       int nvt, int D, const int64_t *row_ptr, const int32_t *col, double scale,
                       const int32_t *qtiles, int nq, double *out, double *lse)
{
    const int npt = n_prefix / TILE;
    const int64_t Ntot = n_prefix + (int64_t)nvt * TILE;
#pragma omp parallel for schedule(dynamic)
    for (int a = 0; a < nq; ++a) {
        const int qt = qtiles[a];
        int64_t nkeys, c = 0;
        int64_t *keys;
        if (qt < npt) {
            nkeys = Ntot;
            keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)nkeys);
            for (int64_t j = 0; j < Ntot; ++j)
                keys[c++] = j;
        } else {
            const int i = qt - npt;
            const int64_t b = row_ptr[i], e = row_ptr[i + 1];
            nkeys = n_prefix + (e - b) * TILE;
            keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)(nkeys > 0 ? nkeys : 1));
            for (int64_t j = 0; j < n_prefix; ++j)
                keys[c++] = j;
            for (int64_t t = b; t < e; ++t) {
                const int64_t base = n_prefix + (int64_t)col[t] * TILE;
                for (int r = 0; r < TILE; ++r)
                    keys[c++] = base + r;
            }
        }
        double *z = (double *)malloc(sizeof(double) * (size_t)(nkeys > 0 ? nkeys : 1));
        double *qd = (double *)malloc(sizeof(double) * (size_t)D);
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
        for (int r = 0; r < TILE; ++r) {
            const int64_t qi = (int64_t)qt * TILE + r;
            for (int d = 0; d < D; ++d)
                qd[d] = bf16_to_double(q[qi * D + d]);
            double mx = -INFINITY;
            for (int64_t j = 0; j < nkeys; ++j) {
                const uint16_t *kr = kx + keys[j] * D;
                double s = 0.0;
                for (int d = 0; d < D; ++d)
                    s += qd[d] * bf16_to_double(kr[d]);
                z[j] = s * scale;
                if (z[j] > mx)
                    mx = z[j];
            }
            double den = 0.0;
            for (int d = 0; d < D; ++d)
                acc[d] = 0.0;
            for (int64_t j = 0; j < nkeys; ++j) {
                const double w = exp(z[j] - mx);
                den += w;
                const uint16_t *vr = v + keys[j] * D;
                for (int d = 0; d < D; ++d)
                    acc[d] += w * bf16_to_double(vr[d]);
            }
            for (int d = 0; d < D; ++d)
                out[((int64_t)a * TILE + r) * D + d] = acc[d] / den;
            if (lse)
                lse[(int64_t)a * TILE + r] = mx + log(den);
        }
        free(z);
        free(qd);
        free(acc);
        free(keys);
    }
}

/*
 * Gradients of orc_attention's output with respect to q, k and v (one (b,h)),
 * given dO = dL/dO.  This is the plain derivative of the function orc_attention
 * computes (the pages give no backward; Prism's training speedup, in [Prism]
 * section "같은 계산량 안에서 볼 곳을 고르는 Prism", needs it over the same kept
 * lists).  For query q with key set S_q, z_qj = scale * (q . k_j),
 * P_qj = exp(z_qj - lse_q), O_q = sum_j P_qj v_j:
 *   Delta_q = dO_q . O_q,   dP_qj = dO_q . v_j,   dS_qj = P_qj (dP_qj - Delta_q),
 *   dQ_q = scale * sum_{j in S_q} dS_qj k_j,
 *   dK_j = scale * sum_{q : j in S_q} dS_qj q_q,
 *   dV_j = sum_{q : j in S_q} P_qj dO_q.
 */

/* Key token list of query tile qt (as in orc_attention); returns the count. */
static int64_t key_list(int qt, int n_prefix, int nvt, int k, const int32_t *idx, int64_t *keys)
{
    const int npt = n_prefix / TILE;
    const int64_t Ntot = n_prefix + (int64_t)nvt * TILE;
    int64_t c = 0;
    if (qt < npt) {
        for (int64_t j = 0; j < Ntot; ++j)
            keys[c++] = j;
        return c;
    }
    const int i = qt - npt;
    for (int64_t j = 0; j < n_prefix; ++j)
        keys[c++] = j;
    for (int t = 0; t < k; ++t) {
        const int64_t base = n_prefix + (int64_t)idx[(int64_t)i * k + t] * TILE;
        for (int r = 0; r < TILE; ++r)
            keys[c++] = base + r;
    }
    return c;
}

/* Does query tile qt attend to key tile kt? */
static int attends(int qt, int kt, int npt, int k, const int32_t *idx)
{
    if (qt < npt || kt < npt)
        return 1;
    const int32_t *row = idx + (int64_t)(qt - npt) * k;
    for (int t = 0; t < k; ++t)
        if (row[t] == kt - npt)
            return 1;
    return 0;
}

static double dot_bf16(const uint16_t *a, const uint16_t *b, int D)
{
    double s = 0.0;
    for (int d = 0; d < D; ++d)
        s += bf16_to_double(a[d]) * bf16_to_double(b[d]);
    return s;
}

/*
 * lse_q and Delta_q for every query token of one (b,h): O recomputed as in
 * orc_attention.  lse, delta: [Ntot].
 */
void orc_attention_lse_delta(const uint16_t *q, const uint16_t *kx, const uint16_t *v, const uint16_t *dout,
                             int n_prefix, int nvt, int D, int k, const int32_t *idx, double scale,
                             double *lse, double *delta)
{
    const int npt = n_prefix / TILE;
    const int ntiles = npt + nvt;
    const int64_t Ntot = n_prefix + (int64_t)nvt * TILE;
#pragma omp parallel for schedule(dynamic)
    for (int qt = 0; qt < ntiles; ++qt) {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)Ntot);
        double *z = (double *)malloc(sizeof(double) * (size_t)Ntot);
        double *o = (double *)malloc(sizeof(double) * (size_t)D);
        const int64_t nk = key_list(qt, n_prefix, nvt, k, idx, keys);
        for (int r = 0; r < TILE; ++r) {
            const int64_t qi = (int64_t)qt * TILE + r;
            double mx = -INFINITY;
            for (int64_t j = 0; j < nk; ++j) {
                z[j] = scale * dot_bf16(q + qi * D, kx + keys[j] * D, D);
                if (z[j] > mx)
                    mx = z[j];
            }
            double den = 0.0;
            for (int d = 0; d < D; ++d)
                o[d] = 0.0;
            for (int64_t j = 0; j < nk; ++j) {
                const double w = exp(z[j] - mx);
                den += w;
                for (int d = 0; d < D; ++d)
                    o[d] += w * bf16_to_double(v[keys[j] * D + d]);
            }
            double dl = 0.0;
            for (int d = 0; d < D; ++d)
                dl += bf16_to_double(dout[qi * D + d]) * (o[d] / den);
            lse[qi] = mx + log(den);
            delta[qi] = dl;
        }
        free(keys);
        free(z);
        free(o);
    }
}

/*
 * dQ of the query tiles qtiles[0..nq) (tiled tile numbers), given lse and
 * Delta of every query token.  dq: [nq][64][D].
 */
void orc_attention_backward_dq(const uint16_t *q, const uint16_t *kx, const uint16_t *v, const uint16_t *dout,
                               const double *lse, const double *delta, int n_prefix, int nvt, int D, int k,
                               const int32_t *idx, double scale, const int32_t *qtiles, int nq, double *dq)
{
    const int64_t Ntot = n_prefix + (int64_t)nvt * TILE;
#pragma omp parallel for schedule(dynamic)
    for (int a = 0; a < nq; ++a) {
        const int qt = qtiles[a];
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)Ntot);
        const int64_t nk = key_list(qt, n_prefix, nvt, k, idx, keys);
        for (int r = 0; r < TILE; ++r) {
            const int64_t qi = (int64_t)qt * TILE + r;
            double *g = dq + ((int64_t)a * TILE + r) * D;
            for (int d = 0; d < D; ++d)
                g[d] = 0.0;
            for (int64_t j = 0; j < nk; ++j) {
                const uint16_t *kr = kx + keys[j] * D;
                const double p = exp(scale * dot_bf16(q + qi * D, kr, D) - lse[qi]);
                const double dp = dot_bf16(dout + qi * D, v + keys[j] * D, D);
                const double ds = p * (dp - delta[qi]);
                for (int d = 0; d < D; ++d)
                    g[d] += ds * bf16_to_double(kr[d]);
            }
            for (int d = 0; d < D; ++d)
                g[d] *= scale;
        }
        free(keys);
    }
}

/*
 * dK and dV of the key tiles ktiles[0..nk) (tiled tile numbers), given lse
 * and Delta of every query token: every query of every query tile that
 * attends the key tile contributes.  dk, dv: [nk][64][D].
 */
void orc_attention_backward_dkdv(const uint16_t *q, const uint16_t *kx, const uint16_t *v, const uint16_t *dout,
                                 const double *lse, const double *delta, int n_prefix, int nvt, int D, int k,
                                 const int32_t *idx, double scale, const int32_t *ktiles, int nk, double *dk,
                                 double *dv)
{
    const int npt = n_prefix / TILE;
    const int ntiles = npt + nvt;
#pragma omp parallel for schedule(dynamic)
    for (int a = 0; a < nk; ++a) {
        const int kt = ktiles[a];
        for (int r = 0; r < TILE; ++r) {
            const int64_t kj = (int64_t)kt * TILE + r;
            double *gk = dk + ((int64_t)a * TILE + r) * D;
            double *gv = dv + ((int64_t)a * TILE + r) * D;
            for (int d = 0; d < D; ++d)
                gk[d] = gv[d] = 0.0;
            for (int qt = 0; qt < ntiles; ++qt) {
                if (!attends(qt, kt, npt, k, idx))
                    continue;
                for (int s = 0; s < TILE; ++s) {
                    const int64_t qi = (int64_t)qt * TILE + s;
                    const double p = exp(scale * dot_bf16(q + qi * D, kx + kj * D, D) - lse[qi]);
                    const double dp = dot_bf16(dout + qi * D, v + kj * D, D);
                    const double ds = p * (dp - delta[qi]);
                    for (int d = 0; d < D; ++d) {
                        gk[d] += ds * bf16_to_double(q[qi * D + d]);
                        gv[d] += p * bf16_to_double(dout[qi * D + d]);
                    }
                }
            }
            for (int d = 0; d < D; ++d)
                gk[d] *= scale;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Ragged grids: static tiles over a grid rounded up to whole tiles           */
/* ------------------------------------------------------------------------ */

/*
 * [SVG, section "이론적 sparsity와 물리적 sparsity의 차이"]: against a tile grid
 * a tile is full, partly covered (a boundary tile, which needs an element
 * mask) or empty.  [Prism, section "토큰 수의 제곱으로 느는 어텐션 비용"]: the
 * 32 x 48 x 80 grid of the 720p clip counts padding tokens.  Reading: a grid
 * that is not a whole number of tiles is covered by the tile grid rounded up
 * on every axis; the slots of a boundary tile that fall outside the grid are
 * padding.  Tile order and token order inside a tile are those of
 * orc_perm_static; perm[p] = -1 marks a padding slot.  The padded slot count
 * is ceil(T/tt)*tt * ceil(Hg/th)*th * ceil(W/tw)*tw.
 * Returns 0, or -1 if the tile is not 64 tokens.
 */
int orc_perm_static_padded(int T, int Hg, int W, int tt, int th, int tw, int32_t *perm)
{
    if (tt < 1 || th < 1 || tw < 1 || tt * th * tw != TILE)
        return -1;
    const int Tt = (T + tt - 1) / tt, Th = (Hg + th - 1) / th, Tw = (W + tw - 1) / tw;
    int64_t p = 0;
    for (int a = 0; a < Tt; ++a)
        for (int b = 0; b < Th; ++b)
            for (int c = 0; c < Tw; ++c)
                for (int x = 0; x < tt; ++x)
                    for (int y = 0; y < th; ++y)
                        for (int z = 0; z < tw; ++z) {
                            int t = a * tt + x, h = b * th + y, w = c * tw + z;
                            if (t < T && h < Hg && w < W)
                                perm[p++] = (int32_t)(((int64_t)t * Hg + h) * W + w);
                            else
                                perm[p++] = -1;
                        }
    return 0;
}

/*
 * Gather and scatter over a padded permutation: the raster tensor has
 * n_prefix + Nras tokens, the tiled one n_prefix + Nslots.  A padding slot is
 * gathered as zeros and not scattered.  perm: [B][Nslots].
 */
void orc_gather_padded(const uint16_t *src_raster, const int32_t *perm, int B, int n_prefix, int64_t Nras,
                       int64_t Nslots, int H, int D, uint16_t *dst_tiled)
{
    const int64_t Nr = n_prefix + Nras, Nt = n_prefix + Nslots;
#pragma omp parallel for collapse(2)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int64_t p = 0; p < Nt; ++p) {
                uint16_t *d = dst_tiled + (((int64_t)b * H + h) * Nt + p) * D;
                const int64_t v = (p < n_prefix) ? p : perm[(int64_t)b * Nslots + (p - n_prefix)];
                if (p >= n_prefix && v < 0) {
                    memset(d, 0, (size_t)D * sizeof(uint16_t));
                    continue;
                }
                const int64_t tok = (p < n_prefix) ? p : n_prefix + v;
                memcpy(d, src_raster + (((int64_t)b * Nr + tok) * H + h) * D, (size_t)D * sizeof(uint16_t));
            }
}

void orc_scatter_padded(const uint16_t *src_tiled, const int32_t *perm, int B, int n_prefix, int64_t Nras,
                        int64_t Nslots, int H, int D, uint16_t *dst_raster)
{
    const int64_t Nr = n_prefix + Nras, Nt = n_prefix + Nslots;
#pragma omp parallel for collapse(2)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int64_t p = 0; p < Nt; ++p) {
                const int64_t v = (p < n_prefix) ? p : perm[(int64_t)b * Nslots + (p - n_prefix)];
                if (p >= n_prefix && v < 0)
                    continue;
                const int64_t tok = (p < n_prefix) ? p : n_prefix + v;
                memcpy(dst_raster + (((int64_t)b * Nr + tok) * H + h) * D,
                       src_tiled + (((int64_t)b * H + h) * Nt + p) * D, (size_t)D * sizeof(uint16_t));
            }
}

/*
 * Tile means over a padded permutation [Prism: a block is judged by the mean
 * of its tokens]: the mean of a boundary tile is taken over its real tokens
 * (perm >= 0) only -- the reading under which padding changes no score.
 * Summed in double, divided by the count, rounded once to float.
 * x_tiled: [B][H][n_prefix + nvt*64][D]; perm: [B][nvt*64]; out: [B][H][nvt][D].
 */
void orc_pool_padded(const uint16_t *x_tiled, const int32_t *perm, int B, int H, int n_prefix, int nvt, int D,
                     float *out)
{
    const int64_t Nslots = (int64_t)nvt * TILE, Ntot = n_prefix + Nslots;
#pragma omp parallel for collapse(2)
    for (int bh = 0; bh < B * H; ++bh)
        for (int i = 0; i < nvt; ++i) {
            const int32_t *pt = perm + (int64_t)(bh / H) * Nslots + (int64_t)i * TILE;
            for (int d = 0; d < D; ++d) {
                double s = 0.0;
                int count = 0;
                for (int r = 0; r < TILE; ++r) {
                    if (pt[r] < 0)
                        continue;
                    s += bf16_to_double(x_tiled[((int64_t)bh * Ntot + n_prefix + (int64_t)i * TILE + r) * D + d]);
                    ++count;
                }
                out[((int64_t)bh * nvt + i) * D + d] = (float)(s / count);
            }
        }
}

/*
 * Attention on a ragged grid: as orc_attention_csr, with the keys limited to
 * the real tokens (key_real[j] != 0) -- the element mask of a boundary tile
 * [SVG, section "이론적 sparsity와 물리적 sparsity의 차이"].  Every query row
 * (padding rows included) gets an output; the caller keeps the real ones.
 * key_real: [n_prefix + nvt*64] of one batch element's tiled order.
 */
void orc_attention_padded(const uint16_t *q, const uint16_t *kx, const uint16_t *v, int n_prefix, int nvt, int D,
                          const int64_t *row_ptr, const int32_t *col, const uint8_t *key_real, double scale,
                          const int32_t *qtiles, int nq, double *out, double *lse)
{
    const int npt = n_prefix / TILE;
    const int64_t Ntot = n_prefix + (int64_t)nvt * TILE;
#pragma omp parallel for schedule(dynamic)
    for (int a = 0; a < nq; ++a) {
        const int qt = qtiles[a];
        int64_t c = 0;
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)(Ntot > 0 ? Ntot : 1));
        if (qt < npt) {
            for (int64_t j = 0; j < Ntot; ++j)
                if (key_real[j])
                    keys[c++] = j;
        } else {
            const int i = qt - npt;
            for (int64_t j = 0; j < n_prefix; ++j)
                keys[c++] = j;
            for (int64_t t = row_ptr[i]; t < row_ptr[i + 1]; ++t) {
                const int64_t base = n_prefix + (int64_t)col[t] * TILE;
                for (int r = 0; r < TILE; ++r)
                    if (key_real[base + r])
                        keys[c++] = base + r;
            }
        }
        const int64_t nkeys = c;
        double *z = (double *)malloc(sizeof(double) * (size_t)(nkeys > 0 ? nkeys : 1));
        double *qd = (double *)malloc(sizeof(double) * (size_t)D);
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
        for (int r = 0; r < TILE; ++r) {
            const int64_t qi = (int64_t)qt * TILE + r;
            for (int d = 0; d < D; ++d)
                qd[d] = bf16_to_double(q[qi * D + d]);
            double mx = -INFINITY;
            for (int64_t j = 0; j < nkeys; ++j) {
                const uint16_t *kr = kx + keys[j] * D;
                double s = 0.0;
                for (int d = 0; d < D; ++d)
                    s += qd[d] * bf16_to_double(kr[d]);
                z[j] = s * scale;
                if (z[j] > mx)
                    mx = z[j];
            }
            double den = 0.0;
            for (int d = 0; d < D; ++d)
                acc[d] = 0.0;
            for (int64_t j = 0; j < nkeys; ++j) {
                const double w = exp(z[j] - mx);
                den += w;
                const uint16_t *vr = v + keys[j] * D;
                for (int d = 0; d < D; ++d)
                    acc[d] += w * bf16_to_double(vr[d]);
            }
            for (int d = 0; d < D; ++d)
                out[((int64_t)a * TILE + r) * D + d] = acc[d] / den;
            if (lse)
                lse[(int64_t)a * TILE + r] = mx + log(den);
        }
        free(z);
        free(qd);
        free(acc);
        free(keys);
    }
}

/*
 * Gradients on a ragged grid: the derivative of orc_attention_padded (keys
 * limited to the real tokens, key_real[j] != 0), with the selection fixed.
 * As orc_attention_lse_delta / orc_attention_backward_dq / _dkdv, with:
 *   - every key list filtered to the real keys;
 *   - dK, dV summed over the real queries only (a padding slot is not a token:
 *     it carries no loss), and zero for a padding key row.
 * Padding query rows still get lse and Delta (of their zero query), unused.
 */
static int64_t keep_real(const uint8_t *real, int64_t *keys, int64_t n)
{
    int64_t c = 0;
    for (int64_t j = 0; j < n; ++j)
        if (real[keys[j]])
            keys[c++] = keys[j];
    return c;
}

void orc_attention_lse_delta_padded(const uint16_t *q, const uint16_t *kx, const uint16_t *v,
                                    const uint16_t *dout, int n_prefix, int nvt, int D, int k, const int32_t *idx,
                                    const uint8_t *key_real, double scale, double *lse, double *delta)
{
    const int npt = n_prefix / TILE;
    const int ntiles = npt + nvt;
    const int64_t Ntot = n_prefix + (int64_t)nvt * TILE;
#pragma omp parallel for schedule(dynamic)
    for (int qt = 0; qt < ntiles; ++qt) {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)Ntot);
        double *z = (double *)malloc(sizeof(double) * (size_t)Ntot);
        double *o = (double *)malloc(sizeof(double) * (size_t)D);
        const int64_t nk = keep_real(key_real, keys, key_list(qt, n_prefix, nvt, k, idx, keys));
        for (int r = 0; r < TILE; ++r) {
            const int64_t qi = (int64_t)qt * TILE + r;
            double mx = -INFINITY;
            for (int64_t j = 0; j < nk; ++j) {
                z[j] = scale * dot_bf16(q + qi * D, kx + keys[j] * D, D);
                if (z[j] > mx)
                    mx = z[j];
            }
            double den = 0.0;
            for (int d = 0; d < D; ++d)
                o[d] = 0.0;
            for (int64_t j = 0; j < nk; ++j) {
                const double w = exp(z[j] - mx);
                den += w;
                for (int d = 0; d < D; ++d)
                    o[d] += w * bf16_to_double(v[keys[j] * D + d]);
            }
            double dl = 0.0;
            for (int d = 0; d < D; ++d)
                dl += bf16_to_double(dout[qi * D + d]) * (o[d] / den);
            lse[qi] = mx + log(den);
            delta[qi] = dl;
        }
        free(keys);
        free(z);
        free(o);
    }
}

void orc_attention_backward_dq_padded(const uint16_t *q, const uint16_t *kx, const uint16_t *v,
                                      const uint16_t *dout, const double *lse, const double *delta, int n_prefix,
                                      int nvt, int D, int k, const int32_t *idx, const uint8_t *key_real,
                                      double scale, const int32_t *qtiles, int nq, double *dq)
{
    const int64_t Ntot = n_prefix + (int64_t)nvt * TILE;
#pragma omp parallel for schedule(dynamic)
    for (int a = 0; a < nq; ++a) {
        const int qt = qtiles[a];
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)Ntot);
        const int64_t nk = keep_real(key_real, keys, key_list(qt, n_prefix, nvt, k, idx, keys));
        for (int r = 0; r < TILE; ++r) {
            const int64_t qi = (int64_t)qt * TILE + r;
            double *g = dq + ((int64_t)a * TILE + r) * D;
            for (int d = 0; d < D; ++d)
                g[d] = 0.0;
            for (int64_t j = 0; j < nk; ++j) {
                const uint16_t *kr = kx + keys[j] * D;
                const double p = exp(scale * dot_bf16(q + qi * D, kr, D) - lse[qi]);
                const double dp = dot_bf16(dout + qi * D, v + keys[j] * D, D);
                const double ds = p * (dp - delta[qi]);
                for (int d = 0; d < D; ++d)
                    g[d] += ds * bf16_to_double(kr[d]);
            }
            for (int d = 0; d < D; ++d)
                g[d] *= scale;
        }
        free(keys);
    }
}

void orc_attention_backward_dkdv_padded(const uint16_t *q, const uint16_t *kx, const uint16_t *v,
                                        const uint16_t *dout, const double *lse, const double *delta, int n_prefix,
                                        int nvt, int D, int k, const int32_t *idx, const uint8_t *key_real,
                                        double scale, const int32_t *ktiles, int nk, double *dk, double *dv)
{
    const int npt = n_prefix / TILE;
    const int ntiles = npt + nvt;
#pragma omp parallel for schedule(dynamic)
    for (int a = 0; a < nk; ++a) {
        const int kt = ktiles[a];
        for (int r = 0; r < TILE; ++r) {
            const int64_t kj = (int64_t)kt * TILE + r;
            double *gk = dk + ((int64_t)a * TILE + r) * D;
            double *gv = dv + ((int64_t)a * TILE + r) * D;
            for (int d = 0; d < D; ++d)
                gk[d] = gv[d] = 0.0;
            if (!key_real[kj])
                continue;
            for (int qt = 0; qt < ntiles; ++qt) {
                if (!attends(qt, kt, npt, k, idx))
                    continue;
                for (int s = 0; s < TILE; ++s) {
                    const int64_t qi = (int64_t)qt * TILE + s;
                    if (!key_real[qi]) /* the same mask marks real query rows */
                        continue;
                    const double p = exp(scale * dot_bf16(q + qi * D, kx + kj * D, D) - lse[qi]);
                    const double dp = dot_bf16(dout + qi * D, v + kj * D, D);
                    const double ds = p * (dp - delta[qi]);
                    for (int d = 0; d < D; ++d) {
                        gk[d] += ds * bf16_to_double(q[qi * D + d]);
                        gv[d] += p * bf16_to_double(dout[qi * D + d]);
                    }
                }
            }
            for (int d = 0; d < D; ++d)
                gk[d] *= scale;
        }
    }
}

/*
 * Gradients over CSR kept lists (variable keep per head or per query tile):
 * the derivative of orc_attention_csr with the lists fixed, in the steps of
 * orc_attention_lse_delta / orc_attention_backward_dq / _dkdv, with video
 * query tile i keeping the video tiles col[row_ptr[i] .. row_ptr[i+1]).
 */
static int64_t key_list_csr(int qt, int n_prefix, int nvt, const int64_t *row_ptr, const int32_t *col,
                            int64_t *keys)
{
    const int npt = n_prefix / TILE;
    const int64_t Ntot = n_prefix + (int64_t)nvt * TILE;
    int64_t c = 0;
    if (qt < npt) {
        for (int64_t j = 0; j < Ntot; ++j)
            keys[c++] = j;
        return c;
    }
    const int i = qt - npt;
    for (int64_t j = 0; j < n_prefix; ++j)
        keys[c++] = j;
    for (int64_t t = row_ptr[i]; t < row_ptr[i + 1]; ++t) {
        const int64_t base = n_prefix + (int64_t)col[t] * TILE;
        for (int r = 0; r < TILE; ++r)
            keys[c++] = base + r;
    }
    return c;
}

static int attends_csr(int qt, int kt, int npt, const int64_t *row_ptr, const int32_t *col)
{
    if (qt < npt || kt < npt)
        return 1;
    for (int64_t t = row_ptr[qt - npt]; t < row_ptr[qt - npt + 1]; ++t)
        if (col[t] == kt - npt)
            return 1;
    return 0;
}

void orc_attention_lse_delta_csr(const uint16_t *q, const uint16_t *kx, const uint16_t *v, const uint16_t *dout,
                                 int n_prefix, int nvt, int D, const int64_t *row_ptr, const int32_t *col,
                                 double scale, double *lse, double *delta)
{
    const int npt = n_prefix / TILE;
    const int ntiles = npt + nvt;
    const int64_t Ntot = n_prefix + (int64_t)nvt * TILE;
#pragma omp parallel for schedule(dynamic)
    for (int qt = 0; qt < ntiles; ++qt) {
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)Ntot);
        double *z = (double *)malloc(sizeof(double) * (size_t)Ntot);
        double *o = (double *)malloc(sizeof(double) * (size_t)D);
        const int64_t nk = key_list_csr(qt, n_prefix, nvt, row_ptr, col, keys);
        for (int r = 0; r < TILE; ++r) {
            const int64_t qi = (int64_t)qt * TILE + r;
            double mx = -INFINITY;
            for (int64_t j = 0; j < nk; ++j) {
                z[j] = scale * dot_bf16(q + qi * D, kx + keys[j] * D, D);
                if (z[j] > mx)
                    mx = z[j];
            }
            double den = 0.0;
            for (int d = 0; d < D; ++d)
                o[d] = 0.0;
            for (int64_t j = 0; j < nk; ++j) {
                const double w = exp(z[j] - mx);
                den += w;
                for (int d = 0; d < D; ++d)
                    o[d] += w * bf16_to_double(v[keys[j] * D + d]);
            }
            double dl = 0.0;
            for (int d = 0; d < D; ++d)
                dl += bf16_to_double(dout[qi * D + d]) * (o[d] / den);
            lse[qi] = mx + log(den);
            delta[qi] = dl;
        }
        free(keys);
        free(z);
        free(o);
    }
}

void orc_attention_backward_dq_csr(const uint16_t *q, const uint16_t *kx, const uint16_t *v, const uint16_t *dout,
                                   const double *lse, const double *delta, int n_prefix, int nvt, int D,
                                   const int64_t *row_ptr, const int32_t *col, double scale, const int32_t *qtiles,
                                   int nq, double *dq)
{
    const int64_t Ntot = n_prefix + (int64_t)nvt * TILE;
#pragma omp parallel for schedule(dynamic)
    for (int a = 0; a < nq; ++a) {
        const int qt = qtiles[a];
        int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)Ntot);
        const int64_t nk = key_list_csr(qt, n_prefix, nvt, row_ptr, col, keys);
        for (int r = 0; r < TILE; ++r) {
            const int64_t qi = (int64_t)qt * TILE + r;
            double *g = dq + ((int64_t)a * TILE + r) * D;
            for (int d = 0; d < D; ++d)
                g[d] = 0.0;
            for (int64_t j = 0; j < nk; ++j) {
                const uint16_t *kr = kx + keys[j] * D;
                const double p = exp(scale * dot_bf16(q + qi * D, kr, D) - lse[qi]);
                const double dp = dot_bf16(dout + qi * D, v + keys[j] * D, D);
                const double ds = p * (dp - delta[qi]);
                for (int d = 0; d < D; ++d)
                    g[d] += ds * bf16_to_double(kr[d]);
            }
            for (int d = 0; d < D; ++d)
                g[d] *= scale;
        }
        free(keys);
    }
}

void orc_attention_backward_dkdv_csr(const uint16_t *q, const uint16_t *kx, const uint16_t *v, const uint16_t *dout,
                                     const double *lse, const double *delta, int n_prefix, int nvt, int D,
                                     const int64_t *row_ptr, const int32_t *col, double scale,
                                     const int32_t *ktiles, int nk, double *dk, double *dv)
{
    const int npt = n_prefix / TILE;
    const int ntiles = npt + nvt;
#pragma omp parallel for schedule(dynamic)
    for (int a = 0; a < nk; ++a) {
        const int kt = ktiles[a];
        for (int r = 0; r < TILE; ++r) {
            const int64_t kj = (int64_t)kt * TILE + r;
            double *gk = dk + ((int64_t)a * TILE + r) * D;
            double *gv = dv + ((int64_t)a * TILE + r) * D;
            for (int d = 0; d < D; ++d)
                gk[d] = gv[d] = 0.0;
            for (int qt = 0; qt < ntiles; ++qt) {
                if (!attends_csr(qt, kt, npt, row_ptr, col))
                    continue;
                for (int s = 0; s < TILE; ++s) {
                    const int64_t qi = (int64_t)qt * TILE + s;
                    const double p = exp(scale * dot_bf16(q + qi * D, kx + kj * D, D) - lse[qi]);
                    const double dp = dot_bf16(dout + qi * D, v + kj * D, D);
                    const double ds = p * (dp - delta[qi]);
                    for (int d = 0; d < D; ++d) {
                        gk[d] += ds * bf16_to_double(q[qi * D + d]);
                        gv[d] += p * bf16_to_double(dout[qi * D + d]);
                    }
                }
            }
            for (int d = 0; d < D; ++d)
                gk[d] *= scale;
        }
    }
}
