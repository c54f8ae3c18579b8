// Dynamic tile shapes ("Prism / Kandinsky 6 speed ablation" page, section
// "같은 계산량 안에서 볼 곳을 고르는 Prism"): the video is cut into 8x8x8 token
// regions; in each region the variation of Q along t, h and w is measured and
// the axis that varies most gets the short tile extent, the tile staying at 64
// tokens.  The page gives the principle only; the rule below is the reading
// stated in the design notes (isotropy margin tau, box 2/4/8 by rank, 16-long
// shapes for two varying axes, taken only by a pair of regions that agree).
//
// Three kernels: per-(batch, region, head) sums of |adjacent difference| read
// straight from the raster Q (one HBM pass); a per-batch choice over the
// regions; and the closed-form tile order for the chosen shapes.
#include "bsa_kernels.h"

namespace bsa {
namespace {

// Shape ids: extents (t, h, w).
__constant__ int kShapeExt[9][3] = {{4, 4, 4}, {2, 4, 8}, {2, 8, 4}, {8, 4, 2}, {4, 2, 8},
                                    {4, 8, 2}, {8, 2, 4}, {2, 2, 16}, {16, 2, 2}};

__device__ inline float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ inline float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ inline float absdiff8(const uint4& a, const uint4& b) {
    // sum over the 8 bf16 channels of |a - b|; each difference of two bf16
    // values is formed in float
    float s = 0.f;
    s += fabsf(bf_lo(a.x) - bf_lo(b.x)) + fabsf(bf_hi(a.x) - bf_hi(b.x));
    s += fabsf(bf_lo(a.y) - bf_lo(b.y)) + fabsf(bf_hi(a.y) - bf_hi(b.y));
    s += fabsf(bf_lo(a.z) - bf_lo(b.z)) + fabsf(bf_hi(a.z) - bf_hi(b.z));
    s += fabsf(bf_lo(a.w) - bf_lo(b.w)) + fabsf(bf_hi(a.w) - bf_hi(b.w));
    return s;
}

// One block per (head, region, batch): thread = (16-byte channel chunk c, w).
// w is the fastest thread index so the w-neighbour is one lane up.  The block
// walks the region's 64 (t, h) rows; each thread keeps its previous-t values
// for the 8 h rows in its own LDS slots (no other thread reads them).
__global__ __launch_bounds__(128) void shape_stats_kernel(const uint4* __restrict__ q, double* __restrict__ partial, int H, int C,
                                   int n_prefix, int T, int Hg, int W) {
    const int h = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
    const int RH = Hg / 8, RW = W / 8, R = (T / 8) * RH * RW;
    const int rt = r / (RH * RW), rh = (r / RW) % RH, rw = r % RW;
    const int w = threadIdx.x & 7, c = threadIdx.x >> 3;
    const int64_t n_tot = n_prefix + (int64_t)T * Hg * W;
    double acc_t = 0.0, acc_h = 0.0, acc_w = 0.0;
    __shared__ uint4 prev_t[8][128];  // [h row][thread]
    for (int tt = 0; tt < 8; ++tt) {
        uint4 prev_h = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
            const int64_t tok = n_prefix + ((int64_t)(rt * 8 + tt) * Hg + (rh * 8 + hh)) * W + (rw * 8 + w);
            const uint4 x = q[((b * n_tot + tok) * H + h) * C + c];
            uint4 xn;
            xn.x = __shfl_down(x.x, 1, 8);
            xn.y = __shfl_down(x.y, 1, 8);
            xn.z = __shfl_down(x.z, 1, 8);
            xn.w = __shfl_down(x.w, 1, 8);
            float row_t = 0.f, row_h = 0.f, row_w = 0.f;
            if (w < 7) row_w = absdiff8(xn, x);
            if (hh > 0) row_h = absdiff8(x, prev_h);
            if (tt > 0) row_t = absdiff8(x, prev_t[hh][threadIdx.x]);
            acc_t += row_t;
            acc_h += row_h;
            acc_w += row_w;
            prev_h = x;
            prev_t[hh][threadIdx.x] = x;
        }
    }
    // block reduction in a fixed order
    for (int o = 32; o > 0; o >>= 1) {
        acc_t += __shfl_xor(acc_t, o);
        acc_h += __shfl_xor(acc_h, o);
        acc_w += __shfl_xor(acc_w, o);
    }
    __shared__ double red[2][3];
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[wave][0] = acc_t;
        red[wave][1] = acc_h;
        red[wave][2] = acc_w;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int nw = (blockDim.x + 63) >> 6;
        double* out = partial + (((int64_t)b * R + r) * H + h) * 3;
        for (int a = 0; a < 3; ++a) {
            double s = 0.0;
            for (int i = 0; i < nw; ++i) s += red[i][a];
            out[a] = s;
        }
    }
}

// One block per batch element.  Phase 1: per region the statistic (sum over
// heads in head order, divided by the pair count), the box shape and whether a
// 16-long shape is wanted.  Phase 2: regions are paired along the long axis
// ((0,1), (2,3), ...); a pair takes the long shape only if both ask for it.
__global__ __launch_bounds__(256) void shape_choose_kernel(const double* __restrict__ partial, uint8_t* __restrict__ shape_map, int H,
                                    int D, int T, int Hg, int W, float tau) {
    extern __shared__ uint8_t sm[];  // [R] box id, then [R] long request
    const int b = blockIdx.x;
    const int RT = T / 8, RH = Hg / 8, RW = W / 8, R = RT * RH * RW;
    uint8_t* box = sm;
    uint8_t* want = sm + R;
    const double denom = 448.0 * H * D;  // 7*8*8 adjacent pairs per axis per channel
    const double lim_f = 1.0 + (double)tau;
    for (int r = threadIdx.x; r < R; r += blockDim.x) {
        double v[3] = {0.0, 0.0, 0.0};
        const double* p = partial + ((int64_t)b * R + r) * H * 3;
        for (int h = 0; h < H; ++h)
            for (int a = 0; a < 3; ++a) v[a] += p[h * 3 + a];
        for (int a = 0; a < 3; ++a) v[a] /= denom;
        // axes ranked by v, largest first; equal values keep the order t, h, w
        int o0 = 0, o1 = 1, o2 = 2, tmp;
        if (v[o1] > v[o0]) { tmp = o0; o0 = o1; o1 = tmp; }
        if (v[o2] > v[o1]) {
            tmp = o1; o1 = o2; o2 = tmp;
            if (v[o1] > v[o0]) { tmp = o0; o0 = o1; o1 = tmp; }
        }
        const double lim = lim_f * v[o2];
        uint8_t id = 0, lw = 0;
        if (v[o0] > lim) {
            // extent 2 on the most varying axis, 4 on the next, 8 on the calmest
            const int key = o0 * 3 + o1;  // (a1, a2)
            switch (key) {
                case 0 * 3 + 1: id = 1; break;  // t,h,w -> 2x4x8
                case 0 * 3 + 2: id = 2; break;  // t,w,h -> 2x8x4
                case 2 * 3 + 1: id = 3; break;  // w,h,t -> 8x4x2
                case 1 * 3 + 0: id = 4; break;  // h,t,w -> 4x2x8
                case 2 * 3 + 0: id = 5; break;  // w,t,h -> 4x8x2
                default: id = 6; break;         // h,w,t -> 8x2x4
            }
            if (v[o1] > lim) lw = (o2 == 2) ? 7 : (o2 == 0) ? 8 : 0;
        }
        box[r] = id;
        want[r] = lw;
    }
    __syncthreads();
    for (int r = threadIdx.x; r < R; r += blockDim.x) {
        uint8_t id = box[r];
        const uint8_t lw = want[r];
        if (lw) {
            const int rt = r / (RH * RW), rh = (r / RW) % RH, rw = r % RW;
            const int pos = (lw == 7) ? rw : rt, cnt = (lw == 7) ? RW : RT;
            const int pp = (pos & 1) ? pos - 1 : pos + 1;
            if (pp < cnt) {
                const int pr = (lw == 7) ? (rt * RH + rh) * RW + pp : (pp * RH + rh) * RW + rw;
                if (want[pr] == lw) id = lw;
            }
        }
        shape_map[(int64_t)b * R + r] = id;
    }
}

// Tiled slot -> raster token for the chosen shapes: 8 slots per region in
// region raster order; a region pair sharing a 16-long shape lays out its 16
// tiles (raster over the pair) in the lower region's slots, then the upper's.
__global__ void perm_dynamic_kernel(const uint8_t* __restrict__ shape_map, int32_t* __restrict__ perm, int B,
                                    int T, int Hg, int W) {
    const int64_t n_video = (int64_t)T * Hg * W;
    const int RH = Hg / 8, RW = W / 8, R = (T / 8) * RH * RW;
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < n_video * B;
         g += (int64_t)gridDim.x * blockDim.x) {
        const int b = (int)(g / n_video);
        const int64_t p = g % n_video;
        const int64_t slot = p / kTile;
        const int q = (int)(p % kTile);
        const int r = (int)(slot / 8);
        int local = (int)(slot % 8);
        const int rt = r / (RH * RW), rh = (r / RW) % RH, rw = r % RW;
        const int id = shape_map[(int64_t)b * R + r];
        const int et = kShapeExt[id][0], eh = kShapeExt[id][1], ew = kShapeExt[id][2];
        int ot = rt * 8, oh = rh * 8, ow = rw * 8;
        int xt = 8, xh = 8, xw = 8;  // extent of the block the tiles are cut from
        if (id == 7) {
            xw = 16;
            if (rw & 1) { ow -= 8; local += 8; }
        } else if (id == 8) {
            xt = 16;
            if (rt & 1) { ot -= 8; local += 8; }
        }
        const int nh = xh / eh, nw = xw / ew;
        (void)xt;
        const int a = local / (nh * nw), bb = (local / nw) % nh, cc = local % nw;
        const int x = q / (eh * ew), y = (q / ew) % eh, z = q % ew;
        const int64_t t = ot + a * et + x;
        const int h = oh + bb * eh + y, w = ow + cc * ew + z;
        perm[g] = (int32_t)((t * Hg + h) * W + w);
    }
}

}  // namespace

hipError_t launch_shape_stats(const uint16_t* q_raster, double* partial, int B, int H, int D, int n_prefix, int T,
                              int Hg, int W, hipStream_t s) {
    const int R = (T / 8) * (Hg / 8) * (W / 8);
    if (B == 0 || H == 0 || R == 0) return hipSuccess;
    const int C = D / 8;
    hipLaunchKernelGGL(shape_stats_kernel, dim3(H, R, B), dim3(8 * C), 0, s, (const uint4*)q_raster, partial, H, C,
                       n_prefix, T, Hg, W);
    return hipGetLastError();
}

hipError_t launch_shape_choose(const double* partial, uint8_t* shape_map, int B, int H, int D, int T, int Hg,
                               int W, float tau, hipStream_t s) {
    const int R = (T / 8) * (Hg / 8) * (W / 8);
    if (B == 0 || R == 0) return hipSuccess;
    hipLaunchKernelGGL(shape_choose_kernel, dim3(B), dim3(256), 2 * R, s, partial, shape_map, H, D, T, Hg, W, tau);
    return hipGetLastError();
}

hipError_t launch_perm_dynamic(const uint8_t* shape_map, int32_t* perm, int B, int T, int Hg, int W,
                               hipStream_t s) {
    const int64_t total = (int64_t)T * Hg * W * B;
    if (total == 0) return hipSuccess;
    const int64_t want = (total + 255) / 256;
    hipLaunchKernelGGL(perm_dynamic_kernel, dim3((unsigned)(want < 65536 ? want : 65536)), dim3(256), 0, s,
                       shape_map, perm, B, T, Hg, W);
    return hipGetLastError();
}

}  // namespace bsa
