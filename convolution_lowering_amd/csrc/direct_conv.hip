// Direct convolution: the seven-loop definition of "Unifying Convolutions and
// GEMM" (section 1) parallelised over outputs, with no lowering and no matrix
// core -- the third point of the comparison in "Im2win: An Efficient
// Convolution Paradigm on GPU" (abstract: im2win against direct convolution
// and the im2col-based PyTorch path).  It is a baseline for the lowered
// paths, not a fast path.
//
// One thread computes CT output channels of one output pixel; a block covers
// 256 consecutive output pixels and one group of CT channels.  The weights a
// block reads are the same for all its threads (uniform addresses), so they
// come through the scalar cache; each input element a thread loads feeds CT
// fused multiply-adds.  fp32 accumulation, the bias added in fp32, one
// rounding at the store, as in the main loops.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "conv_internal.h"

namespace convlower {
namespace {

constexpr int kDirectCT = 8;  // output channels per thread

__device__ __forceinline__ float load_f32(const uint16_t *p, long long i) { return __uint_as_float((uint32_t)p[i] << 16); }
__device__ __forceinline__ float load_f32(const _Float16 *p, long long i) { return (float)p[i]; }
__device__ __forceinline__ float load_f32(const float *p, long long i) { return p[i]; }
__device__ __forceinline__ void store_out(uint16_t *p, long long i, float v) {
    p[i] = __builtin_bit_cast(uint16_t, (__bf16)v);  // round to nearest, ties to even
}
__device__ __forceinline__ void store_out(_Float16 *p, long long i, float v) { p[i] = (_Float16)v; }  // RNE
__device__ __forceinline__ void store_out(float *p, long long i, float v) { p[i] = v; }

template <typename S, bool NHWC>
__global__ __launch_bounds__(256) void direct_conv_kernel(const S *__restrict__ x, const S *__restrict__ w,
                                                          const S *__restrict__ bias, S *__restrict__ y, Geom g) {
    constexpr int CT = kDirectCT;
    const long long m = (long long)blockIdx.x * 256 + threadIdx.x;
    const int co0 = blockIdx.y * CT;
    if (m >= g.M) return;
    const long long n = m / g.P;
    const int p = (int)(m - n * g.P);
    const int ho = p / g.Wo, wo = p - ho * g.Wo;
    float acc[CT];
#pragma unroll
    for (int j = 0; j < CT; ++j) acc[j] = 0.f;
    const int nco = g.Co - co0 < CT ? g.Co - co0 : CT;  // the same for the whole block
    for (int kh = 0; kh < g.KH; ++kh) {
        const int hi = ho * g.s - g.p + kh * g.d;
        if (hi < 0 || hi >= g.H) continue;
        for (int kw = 0; kw < g.KW; ++kw) {
            const int wi = wo * g.s - g.p + kw * g.d;
            if (wi < 0 || wi >= g.W) continue;
            for (int ci = 0; ci < g.C; ++ci) {
                const float xv = NHWC ? load_f32(x, ((n * g.H + hi) * g.W + wi) * g.C + ci)
                                      : load_f32(x, ((n * g.C + ci) * g.H + hi) * (long long)g.W + wi);
#pragma unroll
                for (int j = 0; j < CT; ++j) {
                    if (j < nco) {
                        const long long co = co0 + j;
                        const float wv = NHWC ? load_f32(w, ((co * g.KH + kh) * g.KW + kw) * g.C + ci)
                                              : load_f32(w, ((co * g.C + ci) * g.KH + kh) * (long long)g.KW + kw);
                        acc[j] = fmaf(xv, wv, acc[j]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < CT; ++j) {
        if (j >= nco) break;
        const int co = co0 + j;
        const float v = acc[j] + (bias ? load_f32(bias, co) : 0.f);
        const long long yi = NHWC ? m * g.Co + co : (n * g.Co + co) * g.P + p;
        store_out(y, yi, v);
    }
}

template <typename S>
hipError_t direct_typed(const void *x, const void *w, const void *bias, void *y, const Geom &g, bool nhwc,
                        hipStream_t st) {
    const dim3 grid((unsigned)((g.M + 255) / 256), (unsigned)((g.Co + kDirectCT - 1) / kDirectCT));
    if (nhwc)
        hipLaunchKernelGGL((direct_conv_kernel<S, true>), grid, dim3(256), 0, st, (const S *)x, (const S *)w,
                           (const S *)bias, (S *)y, g);
    else
        hipLaunchKernelGGL((direct_conv_kernel<S, false>), grid, dim3(256), 0, st, (const S *)x, (const S *)w,
                           (const S *)bias, (S *)y, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_direct_conv(const void *x, const void *w, const void *bias, void *y, const Geom &g, bool nhwc,
                              int dtype, hipStream_t st) {
    if (g.Co > 65535LL * kDirectCT) return hipErrorInvalidValue;  // grid.y limit
    if (dtype == 1) return direct_typed<uint16_t>(x, w, bias, y, g, nhwc, st);
    if (dtype == 2) return direct_typed<_Float16>(x, w, bias, y, g, nhwc, st);
    return direct_typed<float>(x, w, bias, y, g, nhwc, st);
}

}  // namespace convlower
