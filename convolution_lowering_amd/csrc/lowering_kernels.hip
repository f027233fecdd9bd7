// The lowering steps that run before (or after) the main loop:
//   (b) the indirection-buffer builder (The Indirect Convolution Algorithm, abstract),
//   (a) the im2win window reorder ("Im2win: An Efficient Convolution Paradigm on GPU", abstract),
//   the NCHW -> NHWC copy and the OIHW -> OHWI weight regrouping that let
//   NCHW tensors use the channels-last feeds,
//   and the ordered split-K finishing pass.
#include "conv_internal.h"

namespace convlower {

static inline unsigned blocks_for(long long n, int per) { return (unsigned)((n + per - 1) / per); }

// ---------------------------------------------------------------------------
// (b) Indirection buffer: entry [p][t] = offset of input pixel (hi, wi) of
// image 0, channel 0, or -1 where tap t of output pixel p is in the padding.
// One thread per entry; consecutive threads write consecutive entries.
__global__ __launch_bounds__(256) void build_indirection_kernel(int32_t *buf, Geom g, int nhwc) {
    long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)g.P * g.T) return;
    int p = (int)(idx / g.T), t = (int)(idx - (long long)p * g.T);
    int ho = p / g.Wo, wo = p - ho * g.Wo;
    int kh = t / g.KW, kw = t - kh * g.KW;
    int hi = ho * g.s + kh * g.d - g.p;
    int wi = wo * g.s + kw * g.d - g.p;
    int32_t v = -1;
    if (hi >= 0 && hi < g.H && wi >= 0 && wi < g.W) v = nhwc ? (hi * g.W + wi) * g.C : hi * g.W + wi;
    buf[idx] = v;
}

hipError_t launch_build_indirection(int32_t *buf, const Geom &g, bool nhwc, hipStream_t st) {
    long long n = (long long)g.P * g.T;
    hipLaunchKernelGGL(build_indirection_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, st, buf, g,
                       nhwc ? 1 : 0);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// (a) Window reorder: xwin[n][ho][c][kh][ci] = xpad(n, ci, ho*s + kh*d - p, c - p).
//
// NHWC input: every (n, ho, c, kh) destination row of C channels is one
// contiguous source row (or zeros), so the copy runs in 16-byte chunks when C
// allows, each thread one chunk, both sides coalesced.
template <typename S, bool VEC>
__global__ __launch_bounds__(256) void im2win_nhwc_kernel(const S *__restrict__ x, S *__restrict__ xw, Geom g,
                                                          long long units) {
    constexpr int V = VEC ? 16 / (int)sizeof(S) : 1;
    long long u = (long long)blockIdx.x * 256 + threadIdx.x;
    if (u >= units) return;
    const int cvec = g.C / V;  // chunks per channel row (exact when VEC)
    long long row = u / cvec;
    int ci = (int)(u - row * cvec) * V;
    int kh = (int)(row % g.KH);
    long long r2 = row / g.KH;
    int c = (int)(r2 % g.Wwin);
    long long r3 = r2 / g.Wwin;
    int ho = (int)(r3 % g.Ho);
    long long n = r3 / g.Ho;
    int hi = ho * g.s + kh * g.d - g.p, wi = c - g.p;
    bool inside = hi >= 0 && hi < g.H && wi >= 0 && wi < g.W;
    long long src = ((n * g.H + hi) * g.W + wi) * g.C + ci;
    long long dst = row * g.C + ci;
    if constexpr (VEC) {
        uint4 v = inside ? *(const uint4 *)(x + src) : make_uint4(0, 0, 0, 0);
        *(uint4 *)(xw + dst) = v;
    } else {
        xw[dst] = inside ? x[src] : S(0);
    }
}

// NCHW input: the source runs along columns c, the destination along
// channels ci, so each block transposes a 64-channel x 64-column tile of one
// (n, ho, kh) row through LDS: reads coalesced along c, writes along ci.
template <typename S>
__global__ __launch_bounds__(256) void im2win_nchw_kernel(const S *__restrict__ x, S *__restrict__ xw, Geom g) {
    __shared__ S tile[64][65];
    const int tiles_c = (g.Wwin + 63) / 64, tiles_ci = (g.C + 63) / 64;
    long long b = blockIdx.x;
    int tc = (int)(b % tiles_c);
    b /= tiles_c;
    int tci = (int)(b % tiles_ci);
    long long slab = b / tiles_ci;  // (n, ho, kh)
    int kh = (int)(slab % g.KH);
    long long r = slab / g.KH;
    int ho = (int)(r % g.Ho);
    long long n = r / g.Ho;
    int hi = ho * g.s + kh * g.d - g.p;
    bool row_in = hi >= 0 && hi < g.H;
    const int c0 = tc * 64, ci0 = tci * 64;
    const int lx = threadIdx.x & 63, ly = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        int ci = ci0 + ly + 4 * j, c = c0 + lx;
        int wi = c - g.p;
        S v = S(0);
        if (row_in && ci < g.C && c < g.Wwin && wi >= 0 && wi < g.W)
            v = x[((n * g.C + ci) * g.H + hi) * (long long)g.W + wi];
        tile[ly + 4 * j][lx] = v;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        int c = c0 + ly + 4 * j, ci = ci0 + lx;
        if (c < g.Wwin && ci < g.C)
            xw[(((n * g.Ho + ho) * (long long)g.Wwin + c) * g.KH + kh) * g.C + ci] = tile[lx][ly + 4 * j];
    }
}

template <typename S>
static hipError_t im2win_typed(const void *x, void *xw, const Geom &g, bool nhwc, hipStream_t st) {
    if (nhwc) {
        constexpr int V = 16 / (int)sizeof(S);
        bool vec = (g.C % V == 0) && ((uintptr_t)x % 16 == 0) && ((uintptr_t)xw % 16 == 0);
        long long rows = (long long)g.N * g.Ho * g.Wwin * g.KH;
        if (vec) {
            long long units = rows * (g.C / V);
            hipLaunchKernelGGL((im2win_nhwc_kernel<S, true>), dim3(blocks_for(units, 256)), dim3(256), 0, st,
                               (const S *)x, (S *)xw, g, units);
        } else {
            long long units = rows * g.C;
            hipLaunchKernelGGL((im2win_nhwc_kernel<S, false>), dim3(blocks_for(units, 256)), dim3(256), 0, st,
                               (const S *)x, (S *)xw, g, units);
        }
    } else {
        long long blocks = (long long)((g.Wwin + 63) / 64) * ((g.C + 63) / 64) * g.N * g.Ho * g.KH;
        hipLaunchKernelGGL(im2win_nchw_kernel<S>, dim3((unsigned)blocks), dim3(256), 0, st, (const S *)x,
                           (S *)xw, g);
    }
    return hipGetLastError();
}

hipError_t launch_im2win(const void *x, void *xwin, const Geom &g, bool nhwc, bool bf16, hipStream_t st) {
    return bf16 ? im2win_typed<uint16_t>(x, xwin, g, nhwc, st) : im2win_typed<float>(x, xwin, g, nhwc, st);
}

// NCHW -> NHWC copy (each image's [C][H*W] matrix transposed to [H*W][C]).
// A block moves a tile of 64 channels x 64*VEC/... pixels: 16-byte loads run
// along the pixels of one channel, the tile is transposed through LDS, and
// 16-byte stores run along the channels of one pixel.  Used when H*W and C
// are multiples of the 16-byte element count (otherwise the window reorder
// of a 1x1 kernel, which is the same copy element by element, does it).
template <typename S>
__global__ __launch_bounds__(256) void nchw_to_nhwc_kernel(const S *__restrict__ x, S *__restrict__ xc, int C,
                                                           int HW, int tiles_hw) {
    constexpr int V = 16 / (int)sizeof(S);  // elements per 16 bytes
    constexpr int TC = 64;                  // channels per tile
    constexpr int THW = 128;                // pixels per tile
    __shared__ S tile[TC][THW + 2];
    const int tid = threadIdx.x;
    const long long n = blockIdx.y;
    const int c0 = blockIdx.z * TC;
    const int hw0 = blockIdx.x * THW;
    const S *src = x + n * (long long)C * HW;
    S *dst = xc + n * (long long)C * HW;
    // load: chunk q covers pixels hw0 + (q % (THW/V))*V .. +V of channel q / (THW/V)
    constexpr int CPR = THW / V;  // chunks per channel row
    for (int q = tid; q < TC * CPR; q += 256) {
        const int cl = q / CPR, hl = (q % CPR) * V;
        const int c = c0 + cl, hw = hw0 + hl;
        union {
            uint4 v;
            S e[V];
        } u;
        u.v = make_uint4(0, 0, 0, 0);
        if (c < C && hw < HW) u.v = *(const uint4 *)(src + (long long)c * HW + hw);  // HW % V == 0
#pragma unroll
        for (int j = 0; j < V; ++j) tile[cl][hl + j] = u.e[j];
    }
    __syncthreads();
    // store: chunk q covers channels c0 + (q % (TC/V))*V .. +V of pixel q / (TC/V)
    constexpr int CPP = TC / V;  // chunks per pixel
    for (int q = tid; q < THW * CPP; q += 256) {
        const int hl = q / CPP, cl = (q % CPP) * V;
        const int c = c0 + cl, hw = hw0 + hl;
        if (c >= C || hw >= HW) continue;
        union {
            uint4 v;
            S e[V];
        } u;
#pragma unroll
        for (int j = 0; j < V; ++j) u.e[j] = tile[cl + j][hl];
        *(uint4 *)(dst + (long long)hw * C + c) = u.v;  // C % V == 0
    }
}

hipError_t launch_nchw_to_nhwc(const void *x, void *x_cl, const Geom &g, bool bf16, hipStream_t st) {
    const int HW = g.H * g.W, V = bf16 ? 8 : 4;
    const bool aligned = (uintptr_t)x % 16 == 0 && (uintptr_t)x_cl % 16 == 0;
    if (HW % V == 0 && g.C % V == 0 && aligned) {
        const int tiles_hw = (HW + 127) / 128;
        dim3 grid(tiles_hw, g.N, (g.C + 63) / 64);
        if (bf16)
            hipLaunchKernelGGL(nchw_to_nhwc_kernel<uint16_t>, grid, dim3(256), 0, st, (const uint16_t *)x,
                               (uint16_t *)x_cl, g.C, HW, tiles_hw);
        else
            hipLaunchKernelGGL(nchw_to_nhwc_kernel<float>, grid, dim3(256), 0, st, (const float *)x, (float *)x_cl,
                               g.C, HW, tiles_hw);
        return hipGetLastError();
    }
    // The window-ordered tensor of a 1x1 stride-1 unpadded kernel is [N][H][W][1][C].
    Geom one = g;
    one.KH = one.KW = one.s = one.d = 1;
    one.p = 0;
    one.Ho = g.H;
    one.Wo = g.W;
    one.Wwin = g.W;
    one.P = HW;
    one.T = 1;
    return launch_im2win(x, x_cl, one, false, bf16, st);
}

// ---------------------------------------------------------------------------
// OIHW -> OHWI: w_ohwi[co][kh][kw][ci] = w_oihw[co][ci][kh][kw], so that the
// window feed (K order kh, kw, ci) can read NCHW-layout weights in 16-byte
// chunks.  One thread per destination element.
template <typename S>
__global__ __launch_bounds__(256) void pack_ohwi_kernel(const S *__restrict__ w, S *__restrict__ o, Geom g) {
    long long e = (long long)blockIdx.x * 256 + threadIdx.x;
    long long total = (long long)g.Co * g.T * g.C;
    if (e >= total) return;
    int ci = (int)(e % g.C);
    long long r = e / g.C;
    int t = (int)(r % g.T);
    long long co = r / g.T;
    o[e] = w[(co * g.C + ci) * g.T + t];
}

hipError_t launch_pack_weights_ohwi(const void *w, void *o, const Geom &g, bool bf16, hipStream_t st) {
    long long total = (long long)g.Co * g.T * g.C;
    if (bf16)
        hipLaunchKernelGGL(pack_ohwi_kernel<uint16_t>, dim3(blocks_for(total, 256)), dim3(256), 0, st,
                           (const uint16_t *)w, (uint16_t *)o, g);
    else
        hipLaunchKernelGGL(pack_ohwi_kernel<float>, dim3(blocks_for(total, 256)), dim3(256), 0, st,
                           (const float *)w, (float *)o, g);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-K finish: y = round(sum over splits, in split order, + bias).  The
// fixed order keeps the result bit-for-bit repeatable.
__device__ __forceinline__ uint16_t to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <typename S, bool OUT_NCHW>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part, const S *bias,
                                                            S *__restrict__ y, Geom g, int splits) {
    long long e = (long long)blockIdx.x * 256 + threadIdx.x;
    long long total = g.M * g.Co;
    if (e >= total) return;
    long long m = e / g.Co;
    int co = (int)(e - m * g.Co);
    float acc = 0.f;
    for (int z = 0; z < splits; ++z) acc += part[(long long)z * total + e];
    if (bias) {
        if constexpr (sizeof(S) == 2)
            acc += __uint_as_float((uint32_t)((const uint16_t *)bias)[co] << 16);
        else
            acc += ((const float *)bias)[co];
    }
    long long yi = e;
    if constexpr (OUT_NCHW) {
        long long n = m / g.P;
        yi = (n * g.Co + co) * g.P + (m - n * g.P);
    }
    if constexpr (sizeof(S) == 2)
        ((uint16_t *)y)[yi] = to_bf16_rne(acc);
    else
        ((float *)y)[yi] = acc;
}

hipError_t launch_splitk_reduce(const float *part, const void *bias, void *y, const Geom &g, int splits,
                                bool out_nchw, bool bf16, hipStream_t st) {
    long long total = g.M * g.Co;
    dim3 grid(blocks_for(total, 256));
    if (bf16) {
        if (out_nchw)
            hipLaunchKernelGGL((splitk_reduce_kernel<uint16_t, true>), grid, dim3(256), 0, st, part,
                               (const uint16_t *)bias, (uint16_t *)y, g, splits);
        else
            hipLaunchKernelGGL((splitk_reduce_kernel<uint16_t, false>), grid, dim3(256), 0, st, part,
                               (const uint16_t *)bias, (uint16_t *)y, g, splits);
    } else {
        if (out_nchw)
            hipLaunchKernelGGL((splitk_reduce_kernel<float, true>), grid, dim3(256), 0, st, part,
                               (const float *)bias, (float *)y, g, splits);
        else
            hipLaunchKernelGGL((splitk_reduce_kernel<float, false>), grid, dim3(256), 0, st, part,
                               (const float *)bias, (float *)y, g, splits);
    }
    return hipGetLastError();
}

}  // namespace convlower
