// Implicit-GEMM main loop with the fused bias epilogue (gfx950, MFMA).
//
// Computes Y_col = X_col * W_row^T ("Unifying Convolutions and GEMM",
// section 3) for M = N*Ho*Wo output pixels, Co output channels and depth
// K = C*KH*KW, without building X_col: each K tile of X_col is gathered
// straight into LDS by one of the feeds of conv_internal.h -- through the
// indirection buffer (The Indirect Convolution Algorithm, abstract), out of
// the window-ordered input ("Im2win: An Efficient Convolution Paradigm on
// GPU", abstract), or, for the shapes that already are a GEMM, from the input
// as it lies in memory.
//
// Structure (the techniques the im2win abstract lists -- shared memory,
// tiling, a micro-kernel, double buffering and prefetching -- recast for
// CDNA4):
//   * a 256-thread block owns a BM x BN tile of Y_col; its four 64-wide
//     wavefronts split it 2 x 2;
//   * K advances in tiles of 32; tile k+1 is fetched from memory into
//     registers while the MFMAs consume tile k from LDS, then written to the
//     other half of a double-buffered LDS area (one barrier per tile);
//   * every LDS row holds the 32 K-consecutive values of one output pixel (or
//     one output channel) in 16-byte chunks, padded by one chunk so that the
//     per-lane 16-byte fragment reads of a wavefront do not collide on banks;
//   * the micro-kernel is v_mfma_f32_16x16x32_bf16 (bf16) or
//     v_mfma_f32_16x16x4_f32 (fp32), fp32 accumulators in registers;
//   * the epilogue adds the bias in fp32, rounds once to the output type
//     (round-to-nearest-even for bf16) and stores in the output layout; the
//     MFMA operand order is picked so that each lane's four accumulator rows
//     run along the output's contiguous axis.  With split-K the fp32 partial
//     sums go to the workspace instead and a separate pass finishes them.
#pragma once

#include "conv_internal.h"

namespace convlower {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename S>
struct Elem;
template <>
struct Elem<uint16_t> {  // bf16 stored as raw 16-bit words
    static constexpr int VEC = 8;
};
template <>
struct Elem<float> {
    static constexpr int VEC = 4;
};

__device__ __forceinline__ uint32_t elem_bits(const uint16_t *p, long long i) { return p[i]; }
__device__ __forceinline__ uint32_t elem_bits(const float *p, long long i) {
    return __float_as_uint(p[i]);
}

__device__ __forceinline__ float bits_to_f32(uint16_t, uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float bits_to_f32(float, uint32_t b) { return __uint_as_float(b); }

// fp32 -> bf16, round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ void store_out(uint16_t *y, long long i, float v) { y[i] = f32_to_bf16_rne(v); }
__device__ __forceinline__ void store_out(float *y, long long i, float v) { y[i] = v; }

union Chunk {
    uint4 v;
    uint32_t u[4];
};

template <typename S>
__device__ __forceinline__ void chunk_put(Chunk &c, int j, uint32_t bits) {
    if constexpr (sizeof(S) == 2)
        c.u[j >> 1] |= bits << (16 * (j & 1));
    else
        c.u[j] = bits;
}

// Per-thread, per-chunk description of one A row (one output pixel); fixed
// for the whole K loop.
struct ARow {
    long long base;  // feed-specific element offset of the row's origin
    int p;           // output pixel within its image (for the indirection buffer)
    bool ok;         // row lies inside M
};

template <int FEED>
__device__ __forceinline__ ARow make_arow(const Geom &g, long long m) {
    ARow r;
    r.ok = m < g.M;
    if (!r.ok) m = 0;
    long long n = m / g.P;
    int p = (int)(m - n * g.P);
    r.p = p;
    if constexpr (FEED == FEED_ROWMAJOR) {
        r.base = m * g.K;
    } else if constexpr (FEED == FEED_NCHW_1X1) {
        r.base = n * g.C * (long long)g.P + p;
    } else if constexpr (FEED == FEED_IND_NHWC) {
        r.base = n * (long long)g.H * g.W * g.C;
    } else if constexpr (FEED == FEED_IND_NCHW) {
        r.base = n * (long long)g.C * g.H * g.W;
    } else {  // FEED_WIN
        int ho = p / g.Wo, wo = p - ho * g.Wo;
        r.base = ((n * g.Ho + ho) * (long long)g.Wwin + (long long)wo * g.s) * g.KH * g.C;
    }
    return r;
}

// One element A[m][k] of the virtual X_col (0 in the padding).
template <typename S, int FEED>
__device__ __forceinline__ uint32_t a_elem(const GemmArgs &A, const ARow &r, int k) {
    const S *src = (const S *)A.a_src;
    const Geom &g = A.g;
    if constexpr (FEED == FEED_ROWMAJOR) {
        return elem_bits(src, r.base + k);
    } else if constexpr (FEED == FEED_NCHW_1X1) {
        return elem_bits(src, r.base + (long long)k * g.P);
    } else if constexpr (FEED == FEED_IND_NHWC) {
        int t = k / g.C, ci = k - t * g.C;
        int off = A.ibuf[r.p * g.T + t];
        return off < 0 ? 0u : elem_bits(src, r.base + off + ci);
    } else if constexpr (FEED == FEED_IND_NCHW) {
        int ci = k / g.T, t = k - ci * g.T;
        int off = A.ibuf[r.p * g.T + t];
        return off < 0 ? 0u : elem_bits(src, r.base + (long long)ci * g.H * g.W + off);
    } else {
        int t = k / g.C, ci = k - t * g.C;
        int kh = t / g.KW, kw = t - kh * g.KW;
        return elem_bits(src, r.base + (long long)(kw * g.d * g.KH + kh) * g.C + ci);
    }
}

// 16 contiguous bytes A[m][k0 .. k0+VEC) (only for feeds whose chunks never
// straddle a tap and are 16-byte aligned; the host checks when that holds).
template <typename S, int FEED>
__device__ __forceinline__ uint4 a_vec(const GemmArgs &A, const ARow &r, int k0) {
    const S *src = (const S *)A.a_src;
    const Geom &g = A.g;
    long long addr;
    if constexpr (FEED == FEED_ROWMAJOR) {
        addr = r.base + k0;
    } else if constexpr (FEED == FEED_IND_NHWC) {
        int t = k0 / g.C, ci = k0 - t * g.C;
        int off = A.ibuf[r.p * g.T + t];
        if (off < 0) return make_uint4(0, 0, 0, 0);
        addr = r.base + off + ci;
    } else {  // FEED_WIN
        int t = k0 / g.C, ci = k0 - t * g.C;
        int kh = t / g.KW, kw = t - kh * g.KW;
        addr = r.base + (long long)(kw * g.d * g.KH + kh) * g.C + ci;
    }
    return *(const uint4 *)(src + addr);
}

template <typename S, int FEED, bool AVEC, bool BVEC, bool OUT_NCHW, int BM, int BN>
__global__ __launch_bounds__(256) void igemm_kernel(GemmArgs A) {
    constexpr int VEC = Elem<S>::VEC;
    constexpr int BK = 32;
    constexpr int KCH = BK / VEC;  // 16-byte chunks per LDS row
    constexpr int RS = KCH + 1;    // padded row stride, in chunks
    constexpr int A_CH = BM * KCH, B_CH = BN * KCH;
    constexpr int A_PER = (A_CH + 255) / 256, B_PER = (B_CH + 255) / 256;
    constexpr int WPM = BM / 2, WCN = BN / 2;  // wavefront tile
    constexpr int TP = WPM / 16, TC = WCN / 16;
    static_assert(TP >= 1 && TC >= 1, "tile too small");
    // Element-wise feeds put consecutive lanes on consecutive pixels.
    constexpr bool A_LANES_ON_M = !AVEC;

    __shared__ uint4 sm[2 * (BM + BN) * RS];

    const Geom &g = A.g;
    const int tid = threadIdx.x;
    const long long m0 = (long long)blockIdx.x * BM;
    const int co0 = blockIdx.y * BN;
    const int kbeg = blockIdx.z * A.k_per_split;
    const int kend = min((long long)kbeg + A.k_per_split, g.K);
    const int nk = (kend - kbeg + BK - 1) / BK;

    // Fixed per-thread chunk assignment.
    ARow arow[A_PER];
    int a_lds[A_PER], a_kc[A_PER];
    bool a_act[A_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
        int c = tid + i * 256;
        a_act[i] = c < A_CH;
        int row = A_LANES_ON_M ? c % BM : c / KCH;
        int kc = A_LANES_ON_M ? c / BM : c % KCH;
        if (!a_act[i]) row = 0, kc = 0;
        a_lds[i] = row * RS + kc;
        a_kc[i] = kc * VEC;
        arow[i] = make_arow<FEED>(g, m0 + row);
    }
    const S *bsrc = (const S *)A.b;
    long long b_off[B_PER];
    int b_lds[B_PER], b_kc[B_PER];
    bool b_ok[B_PER];
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
        int c = tid + i * 256;
        int row = c / KCH, kc = c % KCH;
        bool act = c < B_CH;
        if (!act) row = 0, kc = 0;
        int co = co0 + row;
        b_ok[i] = act && co < g.Co;
        b_off[i] = (long long)(b_ok[i] ? co : 0) * g.K;
        b_lds[i] = act ? row * RS + kc : -1;
        b_kc[i] = kc * VEC;
    }

    Chunk ra[A_PER], rb[B_PER];

    auto fetch = [&](int kt0) {
#pragma unroll
        for (int i = 0; i < A_PER; ++i) {
            int k0 = kt0 + a_kc[i];
            ra[i].v = make_uint4(0, 0, 0, 0);
            if (!a_act[i] || !arow[i].ok) continue;
            if constexpr (AVEC) {
                if (k0 < kend) ra[i].v = a_vec<S, FEED>(A, arow[i], k0);
            } else {
#pragma unroll
                for (int j = 0; j < VEC; ++j)
                    if (k0 + j < kend) chunk_put<S>(ra[i], j, a_elem<S, FEED>(A, arow[i], k0 + j));
            }
        }
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            int k0 = kt0 + b_kc[i];
            rb[i].v = make_uint4(0, 0, 0, 0);
            if (!b_ok[i]) continue;
            if constexpr (BVEC) {
                if (k0 < kend) rb[i].v = *(const uint4 *)(bsrc + b_off[i] + k0);
            } else {
#pragma unroll
                for (int j = 0; j < VEC; ++j)
                    if (k0 + j < kend) chunk_put<S>(rb[i], j, elem_bits(bsrc, b_off[i] + k0 + j));
            }
        }
    };
    auto stash = [&](int stage) {
        uint4 *As = sm + stage * (BM + BN) * RS;
        uint4 *Bs = As + BM * RS;
#pragma unroll
        for (int i = 0; i < A_PER; ++i)
            if (a_act[i]) As[a_lds[i]] = ra[i].v;
#pragma unroll
        for (int i = 0; i < B_PER; ++i)
            if (b_lds[i] >= 0) Bs[b_lds[i]] = rb[i].v;
    };

    f32x4_t acc[TP][TC];
#pragma unroll
    for (int ip = 0; ip < TP; ++ip)
#pragma unroll
        for (int ic = 0; ic < TC; ++ic) acc[ip][ic] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int lane = tid & 63, wave = tid >> 6;
    const int wp = wave >> 1, wc = wave & 1;
    const int frow = lane & 15, fchunk = lane >> 4;

    auto compute = [&](int stage) {
        const uint4 *As = sm + stage * (BM + BN) * RS;
        const uint4 *Bs = As + BM * RS;
#pragma unroll
        for (int grp = 0; grp < KCH / 4; ++grp) {
            uint4 af[TP], bf[TC];
#pragma unroll
            for (int ip = 0; ip < TP; ++ip) af[ip] = As[(wp * WPM + ip * 16 + frow) * RS + grp * 4 + fchunk];
#pragma unroll
            for (int ic = 0; ic < TC; ++ic) bf[ic] = Bs[(wc * WCN + ic * 16 + frow) * RS + grp * 4 + fchunk];
#pragma unroll
            for (int ip = 0; ip < TP; ++ip)
#pragma unroll
                for (int ic = 0; ic < TC; ++ic) {
                    if constexpr (sizeof(S) == 2) {
                        bf16x8_t xa = __builtin_bit_cast(bf16x8_t, af[ip]);
                        bf16x8_t xb = __builtin_bit_cast(bf16x8_t, bf[ic]);
                        if constexpr (OUT_NCHW)
                            acc[ip][ic] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, xb, acc[ip][ic], 0, 0, 0);
                        else
                            acc[ip][ic] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, xa, acc[ip][ic], 0, 0, 0);
                    } else {
                        f32x4_t xa = __builtin_bit_cast(f32x4_t, af[ip]);
                        f32x4_t xb = __builtin_bit_cast(f32x4_t, bf[ic]);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            if constexpr (OUT_NCHW)
                                acc[ip][ic] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa[j], xb[j], acc[ip][ic], 0, 0, 0);
                            else
                                acc[ip][ic] = __builtin_amdgcn_mfma_f32_16x16x4f32(xb[j], xa[j], acc[ip][ic], 0, 0, 0);
                        }
                    }
                }
        }
    };

    if (nk > 0) {
        fetch(kbeg);
        stash(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const bool more = kt + 1 < nk;
            if (more) fetch(kbeg + (kt + 1) * BK);
            compute(kt & 1);
            if (more) stash((kt + 1) & 1);
            __syncthreads();
        }
    }

    // Epilogue.  MFMA 16x16 result: lane holds column (lane & 15) and rows
    // 4*(lane >> 4) + v, v = 0..3.
    S *y = (S *)A.y;
    const S *bias = (const S *)A.bias;
#pragma unroll
    for (int ip = 0; ip < TP; ++ip)
#pragma unroll
        for (int ic = 0; ic < TC; ++ic)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                long long m;
                int co;
                if constexpr (OUT_NCHW) {
                    m = m0 + wp * WPM + ip * 16 + 4 * fchunk + v;
                    co = co0 + wc * WCN + ic * 16 + frow;
                } else {
                    m = m0 + wp * WPM + ip * 16 + frow;
                    co = co0 + wc * WCN + ic * 16 + 4 * fchunk + v;
                }
                if (m >= g.M || co >= g.Co) continue;
                float val = acc[ip][ic][v];
                if (A.part) {
                    A.part[((long long)blockIdx.z * g.M + m) * g.Co + co] = val;
                    continue;
                }
                if (bias) val += bits_to_f32(S(), elem_bits(bias, co));
                long long yi;
                if constexpr (OUT_NCHW) {
                    long long n = m / g.P;
                    yi = (n * g.Co + co) * g.P + (m - n * g.P);
                } else {
                    yi = m * g.Co + co;
                }
                store_out(y, yi, val);
            }
}

template <typename S, int FEED, bool AVEC, bool BVEC, bool OUT_NCHW>
static hipError_t launch_tile(const GemmArgs &a, int tile, int splits, hipStream_t st) {
    const Geom &g = a.g;
    auto go = [&](auto kern, int BM, int BN) {
        dim3 grid((unsigned)((g.M + BM - 1) / BM), (unsigned)((g.Co + BN - 1) / BN), (unsigned)splits);
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, a);
        return hipGetLastError();
    };
    switch (tile) {
        case TILE_128x128:
            return go(igemm_kernel<S, FEED, AVEC, BVEC, OUT_NCHW, 128, 128>, 128, 128);
        case TILE_128x64:
            return go(igemm_kernel<S, FEED, AVEC, BVEC, OUT_NCHW, 128, 64>, 128, 64);
        case TILE_32x64:
            return go(igemm_kernel<S, FEED, AVEC, BVEC, OUT_NCHW, 32, 64>, 32, 64);
        default:
            return hipErrorInvalidValue;
    }
}

// All (vector-load, output-layout) variants a feed can need.
template <typename S, int FEED>
hipError_t launch_feed(const GemmArgs &a, bool out_nchw, bool a_vec, bool b_vec, int tile, int splits,
                       hipStream_t st) {
    constexpr bool CAN_AVEC = FEED == FEED_ROWMAJOR || FEED == FEED_IND_NHWC || FEED == FEED_WIN;
    constexpr bool CAN_NCHW = FEED == FEED_NCHW_1X1 || FEED == FEED_IND_NCHW || FEED == FEED_WIN;
    constexpr bool CAN_NHWC = FEED == FEED_ROWMAJOR || FEED == FEED_IND_NHWC || FEED == FEED_WIN;
    if (a_vec && !b_vec) return hipErrorInvalidValue;
    if (out_nchw) {
        if constexpr (CAN_NCHW) {
            if (a_vec) {
                if constexpr (CAN_AVEC) return launch_tile<S, FEED, true, true, true>(a, tile, splits, st);
                return hipErrorInvalidValue;
            }
            if (b_vec) return launch_tile<S, FEED, false, true, true>(a, tile, splits, st);
            return launch_tile<S, FEED, false, false, true>(a, tile, splits, st);
        }
        return hipErrorInvalidValue;
    }
    if constexpr (CAN_NHWC) {
        if (a_vec) {
            if constexpr (CAN_AVEC) return launch_tile<S, FEED, true, true, false>(a, tile, splits, st);
            return hipErrorInvalidValue;
        }
        if (b_vec) return launch_tile<S, FEED, false, true, false>(a, tile, splits, st);
        return launch_tile<S, FEED, false, false, false>(a, tile, splits, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace convlower
