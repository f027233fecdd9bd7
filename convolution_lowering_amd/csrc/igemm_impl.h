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
//     wavefronts split it 2 x 2 and each keeps its (BM/2) x (BN/2) fp32
//     accumulators in registers;
//   * K advances in tiles of BK; the global loads of tile k+2 are issued
//     into registers before the MFMAs consume tile k from LDS, and tile k+1
//     (loaded one iteration earlier) is then written to the other half of a
//     double-buffered LDS area -- one barrier per tile;
//   * every LDS row holds the BK K-consecutive values of one output pixel (or
//     one output channel) as 16-byte chunks whose positions are XOR-swizzled
//     by the row index, so the per-lane 16-byte fragment reads of a
//     wavefront (16 rows, one chunk column) hit distinct banks;
//   * for the indirection feed the block's slice of the buffer (its BM rows
//     times KH*KW taps) is copied to LDS once, so no global load waits on
//     another; the (tap, channel) position of each thread's chunk advances
//     incrementally, without divisions;
//   * the micro-kernel is v_mfma_f32_16x16x32_bf16 (bf16) or
//     v_mfma_f32_16x16x4_f32 (fp32);
//   * the epilogue adds the bias in fp32, rounds once to the output type
//     (round-to-nearest-even for bf16), stages the tile in LDS and writes it
//     with 16-byte stores along the output's contiguous axis.  With split-K
//     the fp32 partial sums go to the workspace instead and a separate pass
//     finishes them;
//   * tile order: see tile_coords.
#pragma once

#include "conv_internal.h"
#include <hip/hip_ext.h>

namespace convlower {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <typename S>
struct Elem;
template <>
struct Elem<uint16_t> {  // bf16 stored as raw 16-bit words
    static constexpr int VEC = 8;
};
template <>
struct Elem<uint8_t> {  // OCP fp8 e4m3 as raw bytes (inputs only; the output is bf16)
    static constexpr int VEC = 16;
};
template <>
struct Elem<_Float16> {  // IEEE half
    static constexpr int VEC = 8;
};
template <>
struct Elem<float> {
    static constexpr int VEC = 4;
};

__device__ __forceinline__ uint32_t elem_bits(const uint16_t *p, long long i) { return p[i]; }
__device__ __forceinline__ uint32_t elem_bits(const _Float16 *p, long long i) {
    return __builtin_bit_cast(uint16_t, p[i]);
}
__device__ __forceinline__ uint32_t elem_bits(const float *p, long long i) {
    return __float_as_uint(p[i]);
}

__device__ __forceinline__ float bits_to_f32(uint16_t, uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float bits_to_f32(_Float16, uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}
__device__ __forceinline__ float bits_to_f32(float, uint32_t b) { return __uint_as_float(b); }

// fp32 -> bf16, round to nearest, ties to even (NaN stays a NaN): gfx950's
// v_cvt_pk_bf16_f32, one instruction for a pair, no branch.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// Two values, a in the low half.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint16_t to_out(uint16_t, float v) { return f32_to_bf16_rne(v); }
// fp32 -> fp16, round to nearest, ties to even (the default rounding mode).
__device__ __forceinline__ _Float16 to_out(_Float16, float v) { return (_Float16)v; }
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_f16x2_rne(float a, float b) {
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
__device__ __forceinline__ float to_out(float, float v) { return v; }

// Buffer loads: an offset past the buffer's size reads as zeros, so padding
// taps and out-of-range rows need neither a branch nor a select, and every
// load is issued unconditionally (keeping the compiler's count of
// outstanding loads exact).  Offsets are in bytes.
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

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

// Per-row description of one A row (one output pixel), fixed for the K loop.
struct ARow {
    long long base;  // feed-specific element offset of the row's origin
    int p;           // output pixel within its image (indirection buffer row)
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
    } else if constexpr (FEED == FEED_IND_NHWC || FEED == FEED_IND_CHUNK) {
        r.base = n * (long long)g.H * g.W * g.C;
    } else if constexpr (FEED == FEED_IND_NCHW) {
        r.base = n * (long long)g.C * g.H * g.W;
    } else {  // FEED_WIN
        int ho = p / g.Wo, wo = p - ho * g.Wo;
        r.base = ((n * g.Ho + ho) * (long long)g.Wwin + (long long)wo * g.s) * g.KH * g.C;
    }
    return r;
}

// One element A[m][k] of the virtual X_col (0 in the padding); the general
// path for feeds and shapes whose rows cannot be read in 16-byte chunks.
template <typename S, int FEED>
__device__ __forceinline__ uint32_t a_elem(const GemmArgs &A, const ARow &r, int k) {
    const S *src = (const S *)A.a_src;
    const Geom &g = A.g;
    if constexpr (FEED == FEED_ROWMAJOR) {
        return elem_bits(src, r.base + k);
    } else if constexpr (FEED == FEED_NCHW_1X1) {
        return elem_bits(src, r.base + (long long)k * g.P);
    } else if constexpr (FEED == FEED_IND_NHWC || FEED == FEED_IND_CHUNK) {
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


// Tile order.  The grid is one-dimensional over the (pixel tile, channel
// tile) pairs; blocks are dealt to the eight XCDs round-robin, so block b
// runs on XCD b % 8 as that XCD's (b / 8)-th block.  When the channel-tile
// count divides 8, each XCD is given one channel tile -- its slice of W_row
// then stays in that XCD's L2 -- and a contiguous share of the pixel tiles
// (the input rows of neighbouring pixel tiles overlap).  Otherwise each XCD
// takes a contiguous run of pairs, channel tiles of one pixel tile adjacent
// (those blocks read the same X_col rows); with a grid that is not a
// multiple of 8, XCD x holds total/8 blocks, one more for the first
// total % 8 XCDs, and its run starts where the previous XCDs' runs end.
__device__ __forceinline__ void tile_coords(int ntile_m, int ntile_n, int &mt, int &nt) {
    const int b = blockIdx.x, total = gridDim.x;
    const int xcd = b & 7, j = b >> 3;
    if ((total & 7) == 0 && (8 % ntile_n) == 0 && (ntile_m % (8 / ntile_n)) == 0) {
        const int groups = 8 / ntile_n;
        nt = xcd % ntile_n;
        mt = (xcd / ntile_n) * (ntile_m / groups) + j;
        return;
    }
    const int q = total >> 3, r = total & 7;
    const int l = xcd * q + min(xcd, r) + j;
    mt = l / ntile_n;
    nt = l - mt * ntile_n;
}

// Tile order with the weight bytes in view: each XCD takes a contiguous
// share of the pixel tiles and, of the channel tiles, the fewest groups
// whose weight slices together still fit kXcdWeightBudget of its L2, so the
// blocks of one pixel tile run on one XCD and read its input rows from that
// XCD's L2 once, not once per XCD.  Group count q (dividing 8 and the
// channel-tile count, 8 / q dividing the pixel-tile count): XCD x serves
// channel tiles (x % q) * ntile_n / q .. +ntile_n / q - 1 for pixel tiles
// (x / q) * ntile_m * q / 8 onwards, channel tile fastest.  With no such q
// this is tile_coords.
constexpr long long kXcdWeightBudget = 5LL << 19;  // 2.5 MiB of a 4 MiB L2
__device__ __forceinline__ void tile_coords_l2(int ntile_m, int ntile_n, long long wbytes_per_ntile, int &mt,
                                               int &nt) {
    const int b = blockIdx.x;
    if ((gridDim.x & 7) == 0) {
        for (int q = 1; q <= 8; q *= 2) {
            if (ntile_n % q != 0 || ntile_m % (8 / q) != 0) continue;
            const int nper = ntile_n / q;
            if ((long long)nper * wbytes_per_ntile > kXcdWeightBudget) continue;
            const int xcd = b & 7, j = b >> 3;
            mt = (xcd / q) * (ntile_m / (8 / q)) + j / nper;
            nt = (xcd % q) * nper + j % nper;
            return;
        }
    }
    tile_coords(ntile_m, ntile_n, mt, nt);
}

constexpr int kThreads = 256;
constexpr int kIbufLdsEntries = 3072;  // LDS slots for the block's indirection-buffer slice

// LDS position (in 16-byte chunks) of chunk c of row `row`, rows of kch chunks.
__device__ __forceinline__ constexpr int lds_slot(int row, int c, int kch) { return row * kch + (c ^ (row & 7)); }

template <typename S, int BM, int BN, int BK>
struct TileCfg {
    static constexpr int VEC = Elem<S>::VEC;
    static constexpr int KCH = BK / VEC;  // 16-byte chunks per LDS row
    static constexpr int RS = KCH;        // row stride, in chunks (chunks XOR-swizzled within a row)
    static constexpr int A_CH = BM * KCH, B_CH = BN * KCH;
    static constexpr int A_PER = A_CH / kThreads, B_PER = B_CH / kThreads;
    static constexpr int STAGE = (BM + BN) * RS;  // uint4 per LDS stage
    static constexpr int WPM = BM / 2, WCN = BN / 2;
    static constexpr int TP = WPM / 16, TC = WCN / 16;
    // epilogue tile in LDS: [BN][BM + EPAD] (NCHW) or [BM][BN + EPAD] (NHWC), in S
    static constexpr int EPAD = 16 / (int)sizeof(S);
    static constexpr int EPI_BYTES = (BM > BN ? BM : BN) * ((BM > BN ? BN : BM) + EPAD) * (int)sizeof(S);
    static constexpr int MAIN_BYTES = 2 * STAGE * 16;
    static constexpr int SMEM_UINT4 = ((MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES) + 15) / 16;
    static_assert(KCH % 8 == 0, "a K tile must be 128 bytes per row (whole MFMA K steps, 8-way swizzle)");
    static_assert(A_CH % kThreads == 0 && B_CH % kThreads == 0, "chunks must divide evenly");
    static_assert(kThreads % KCH == 0, "rows must divide evenly");
    static_assert(TP >= 1 && TC >= 1, "tile too small");
};

template <typename S, int FEED, bool AVEC, bool BVEC, bool OUT_NCHW, int BM, int BN, int BK>
__global__ __launch_bounds__(kThreads) void igemm_kernel(GemmArgs A) {
    using C = TileCfg<S, BM, BN, BK>;
    constexpr int VEC = C::VEC, KCH = C::KCH, RS = C::RS;
    constexpr int A_PER = C::A_PER, B_PER = C::B_PER;
    constexpr int WPM = C::WPM, WCN = C::WCN, TP = C::TP, TC = C::TC;
    constexpr bool IND = FEED == FEED_IND_NHWC || FEED == FEED_IND_NCHW;

    __shared__ uint4 sm[C::SMEM_UINT4];
    __shared__ int ib_lds[IND && AVEC ? kIbufLdsEntries : 1];

    const Geom &g = A.g;
    const int tid = threadIdx.x;

    int mt, nt;
    tile_coords((int)((g.M + BM - 1) / BM), (g.Co + BN - 1) / BN, mt, nt);
    const long long m0 = (long long)mt * BM;
    const int co0 = nt * BN;
    const int kbeg = blockIdx.z * A.k_per_split;
    const int kend = (int)min((long long)kbeg + A.k_per_split, g.K);
    const int nk = (kend - kbeg + BK - 1) / BK;

    // The block's slice of the indirection buffer, rows m0 .. m0+BM-1 (the
    // vector path requires BM * KH*KW <= kIbufLdsEntries; the host checks).
    if constexpr (IND && AVEC) {
        for (int e = tid; e < BM * g.T; e += kThreads) {
            int row = e / g.T, t = e - row * g.T;
            long long m = m0 + row;
            int v = -1;
            if (m < g.M) {
                long long n = m / g.P;
                int p = (int)(m - n * g.P);
                v = A.ibuf[p * g.T + t];
            }
            ib_lds[e] = v;
        }
    }

    // ---- A operand assignment --------------------------------------------
    // Vector feeds: thread owns chunk column kc = tid % KCH of rows
    // tid / KCH + i * (256 / KCH).  Element-wise feeds: lanes run along rows.
    constexpr bool LANES_ON_M = !AVEC;
    ARow arow[A_PER];
    int a_lds[A_PER];
    int a_rowl[A_PER];
    const int a_kc_vec = (tid % KCH) * VEC;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
        int c = tid + i * kThreads;
        int row = LANES_ON_M ? c % BM : c / KCH;
        int kc = LANES_ON_M ? c / BM : c % KCH;
        a_lds[i] = lds_slot(row, kc, KCH);
        a_rowl[i] = row;
        arow[i] = make_arow<FEED>(g, m0 + row);
    }
    int a_kc_el[A_PER];
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
        int c = tid + i * kThreads;
        a_kc_el[i] = (LANES_ON_M ? c / BM : c % KCH) * VEC;
    }

    // (tap, channel) of this thread's vector chunk, advanced per K tile.
    int cur_t = 0, cur_ci = 0, cur_kh = 0, cur_kw = 0;
    if constexpr (AVEC && (FEED == FEED_IND_NHWC || FEED == FEED_WIN)) {
        int k0 = kbeg + a_kc_vec;
        cur_t = k0 / g.C;
        cur_ci = k0 - cur_t * g.C;
        cur_kh = cur_t / g.KW;
        cur_kw = cur_t - cur_kh * g.KW;
    }

    // ---- B operand assignment ----------------------------------------------
    const S *bsrc = (const S *)A.b;
    long long b_off[B_PER];
    int b_lds[B_PER];
    bool b_ok[B_PER];
    const int b_kc = (tid % KCH) * VEC;
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
        int c = tid + i * kThreads;
        int row = c / KCH;
        int co = co0 + row;
        b_ok[i] = co < g.Co;
        b_off[i] = (long long)(b_ok[i] ? co : 0) * g.K;
        b_lds[i] = lds_slot(row, c % KCH, KCH);
    }

    __syncthreads();  // ib_lds ready

    Chunk ra[2][A_PER], rb[2][B_PER];

    // Global -> registers for K tile starting at kt0 (register set `set`).
    // The vector paths use buffer loads, issued unconditionally, so the
    // compiler can count outstanding loads exactly and wait only for the tile
    // it is about to store.
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A.a_src, A.a_bytes);
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(A.b, A.b_bytes);
    auto fetch = [&](int kt0, auto set_c) {
        constexpr int set = decltype(set_c)::value;
        if constexpr (AVEC) {
            const int k0 = kt0 + a_kc_vec;
            const bool kin = k0 < kend;
            long long koff = 0;
            if constexpr (FEED == FEED_ROWMAJOR) koff = k0;
            if constexpr (FEED == FEED_IND_NHWC) koff = cur_ci;
            if constexpr (FEED == FEED_WIN) koff = (long long)(cur_kw * g.d * g.KH + cur_kh) * g.C + cur_ci;
#pragma unroll
            for (int i = 0; i < A_PER; ++i) {
                bool valid = arow[i].ok && kin;
                long long addr = arow[i].base + koff;
                if constexpr (FEED == FEED_IND_NHWC) {
                    int off = ib_lds[a_rowl[i] * g.T + cur_t];
                    valid = valid && off >= 0;
                    addr += off;
                }
                ra[set][i].v = buf_load16(a_rsrc, valid ? (uint32_t)(addr * (long long)sizeof(S)) : kOutOfRange);
            }
            // advance the (tap, channel) position by one K tile
            if constexpr (FEED == FEED_IND_NHWC || FEED == FEED_WIN) {
                cur_ci += BK;
                while (cur_ci >= g.C) {
                    cur_ci -= g.C;
                    ++cur_t;
                    if (++cur_kw == g.KW) {
                        cur_kw = 0;
                        ++cur_kh;
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < A_PER; ++i) {
                ra[set][i].v = make_uint4(0, 0, 0, 0);
                if (!arow[i].ok) continue;
                int k0 = kt0 + a_kc_el[i];
#pragma unroll
                for (int j = 0; j < VEC; ++j)
                    if (k0 + j < kend) chunk_put<S>(ra[set][i], j, a_elem<S, FEED>(A, arow[i], k0 + j));
            }
        }
        const int kb = kt0 + b_kc;
#pragma unroll
        for (int i = 0; i < B_PER; ++i) {
            if constexpr (BVEC) {
                bool valid = b_ok[i] && kb < kend;
                rb[set][i].v = buf_load16(b_rsrc, valid ? (uint32_t)((b_off[i] + kb) * (long long)sizeof(S)) : kOutOfRange);
            } else {
                rb[set][i].v = make_uint4(0, 0, 0, 0);
                if (!b_ok[i]) continue;
#pragma unroll
                for (int j = 0; j < VEC; ++j)
                    if (kb + j < kend) chunk_put<S>(rb[set][i], j, elem_bits(bsrc, b_off[i] + kb + j));
            }
        }
    };
    auto stash = [&](int stage, auto set_c) {
        constexpr int set = decltype(set_c)::value;
        uint4 *As = sm + stage * C::STAGE;
        uint4 *Bs = As + BM * RS;
#pragma unroll
        for (int i = 0; i < A_PER; ++i) As[a_lds[i]] = ra[set][i].v;
#pragma unroll
        for (int i = 0; i < B_PER; ++i) Bs[b_lds[i]] = rb[set][i].v;
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
        const uint4 *As = sm + stage * C::STAGE;
        const uint4 *Bs = As + BM * RS;
#pragma unroll
        for (int grp = 0; grp < KCH / 4; ++grp) {
            uint4 af[TP], bf[TC];
#pragma unroll
            for (int ip = 0; ip < TP; ++ip) af[ip] = As[lds_slot(wp * WPM + ip * 16 + frow, grp * 4 + fchunk, KCH)];
#pragma unroll
            for (int ic = 0; ic < TC; ++ic) bf[ic] = Bs[lds_slot(wc * WCN + ic * 16 + frow, grp * 4 + fchunk, KCH)];
#pragma unroll
            for (int ip = 0; ip < TP; ++ip)
#pragma unroll
                for (int ic = 0; ic < TC; ++ic) {
                    if constexpr (std::is_same<S, _Float16>::value) {
                        f16x8_t xa = __builtin_bit_cast(f16x8_t, af[ip]);
                        f16x8_t xb = __builtin_bit_cast(f16x8_t, bf[ic]);
                        if constexpr (OUT_NCHW)
                            acc[ip][ic] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, xb, acc[ip][ic], 0, 0, 0);
                        else
                            acc[ip][ic] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xb, xa, acc[ip][ic], 0, 0, 0);
                    } else if constexpr (sizeof(S) == 2) {
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

    using Z = std::integral_constant<int, 0>;
    using O = std::integral_constant<int, 1>;
    if (nk > 0) {
        // Fetches and stores run unconditionally (tiles past the end read as
        // zeros and land in a stage nobody reads), so the loads in flight are
        // the same on every path and each wait covers exactly one tile.
        fetch(kbeg, Z{});
        fetch(kbeg + BK, O{});
        stash(0, Z{});
        __syncthreads();
        // Two K tiles per trip so the register sets are named statically.
        for (int kt = 0;; kt += 2) {
            fetch(kbeg + (kt + 2) * BK, Z{});
            compute(0);
            stash(1, O{});
            __syncthreads();
            if (kt + 1 >= nk) break;
            fetch(kbeg + (kt + 3) * BK, O{});
            compute(1);
            stash(0, Z{});
            __syncthreads();
            if (kt + 2 >= nk) break;
        }
    }

    // ---- epilogue ------------------------------------------------------------
    // MFMA 16x16 result: lane holds column (lane & 15), rows 4*(lane >> 4) + v.
    const S *bias = (const S *)A.bias;
    if (A.part) {  // split-K: raw fp32 partials, finished by the reduce pass
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
                    if (m < g.M && co < g.Co) A.part[((long long)blockIdx.z * g.M + m) * g.Co + co] = acc[ip][ic][v];
                }
        return;
    }

    // Stage the rounded tile in LDS, laid out along the output's contiguous
    // axis, then write it out in 16-byte chunks.
    S *E = (S *)sm;
    constexpr int EPAD = C::EPAD;
    constexpr int ER = OUT_NCHW ? BM + EPAD : BN + EPAD;  // elements per LDS row
#pragma unroll
    for (int ic = 0; ic < TC; ++ic) {
#pragma unroll
        for (int ip = 0; ip < TP; ++ip) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                int ml, cl;
                if constexpr (OUT_NCHW) {
                    ml = wp * WPM + ip * 16 + 4 * fchunk + v;
                    cl = wc * WCN + ic * 16 + frow;
                } else {
                    ml = wp * WPM + ip * 16 + frow;
                    cl = wc * WCN + ic * 16 + 4 * fchunk + v;
                }
                float val = acc[ip][ic][v];
                int co = co0 + cl;
                if (bias && co < g.Co) val += bits_to_f32(S(), elem_bits(bias, co));
                if constexpr (OUT_NCHW)
                    E[cl * ER + ml] = to_out(S(), val);
                else
                    E[ml * ER + cl] = to_out(S(), val);
            }
        }
    }
    __syncthreads();

    S *y = (S *)A.y;
    if constexpr (OUT_NCHW) {
        // rows: output channels; columns: BM consecutive pixels
        constexpr int CPR = BM / VEC;  // chunks per row
        for (int c = tid; c < BN * CPR; c += kThreads) {
            int cl = c / CPR, mc = (c - cl * CPR) * VEC;
            int co = co0 + cl;
            if (co >= g.Co) continue;
            long long m = m0 + mc;
            if (m >= g.M) continue;
            long long n = m / g.P;
            long long p = m - n * g.P;
            long long yi = (n * g.Co + co) * g.P + p;
            const S *src = E + cl * ER + mc;
            if (p + VEC <= g.P && m + VEC <= g.M && ((uintptr_t)(y + yi) & 15) == 0) {
                *(uint4 *)(y + yi) = *(const uint4 *)src;
            } else {
                for (int j = 0; j < VEC; ++j) {
                    long long mj = m + j;
                    if (mj >= g.M) break;
                    long long nj = mj / g.P;
                    y[(nj * g.Co + co) * g.P + (mj - nj * g.P)] = src[j];
                }
            }
        }
    } else {
        constexpr int CPR = BN / VEC;
        for (int c = tid; c < BM * CPR; c += kThreads) {
            int ml = c / CPR, cc = (c - ml * CPR) * VEC;
            long long m = m0 + ml;
            int co = co0 + cc;
            if (m >= g.M || co >= g.Co) continue;
            long long yi = m * g.Co + co;
            const S *src = E + ml * ER + cc;
            if (co + VEC <= g.Co && ((uintptr_t)(y + yi) & 15) == 0) {
                *(uint4 *)(y + yi) = *(const uint4 *)src;
            } else {
                for (int j = 0; j < VEC && co + j < g.Co; ++j) y[yi + j] = src[j];
            }
        }
    }
}

}  // namespace convlower

#include "igemm_dma.h"
#include "igemm_dual.h"
#include "igemm_rowwin.h"
#include "igemm_rowwin_pp.h"

namespace convlower {

template <typename S, int FEED, bool AVEC, bool BVEC, bool OUT_NCHW>
static hipError_t launch_tile(const GemmArgs &a, int tile, int splits, hipStream_t st) {
    const Geom &g = a.g;
    auto go = [&](auto kern, int BM, int BN, int threads = kThreads, bool sk = false) {
        dim3 grid((unsigned)(((g.M + BM - 1) / BM) * ((g.Co + BN - 1) / BN)), 1, (unsigned)splits);
        if (sk) grid = dim3((unsigned)kSkBlocks);
        hipEvent_t t0, t1;
        take_main_loop_events(&t0, &t1);
        if (t0 || t1)
            hipExtLaunchKernelGGL(kern, grid, dim3(threads), 0, st, t0, t1, 0, a);
        else
            hipLaunchKernelGGL(kern, grid, dim3(threads), 0, st, a);
        return hipGetLastError();
    };
    constexpr int BKW = sizeof(S) == 2 ? 64 : 32;  // 128-byte LDS rows
    if constexpr (FEED == FEED_ROWWIN) {  // its own loop only, 16-byte rows only
        if constexpr (AVEC) {
            if (tile == TILE_256x128_ROWWIN) return go(igemm_rowwin_kernel<S, OUT_NCHW>, 256, 128, 256);
            if (tile == TILE_256x64_ROWWIN) return go(igemm_rowwin_kernel<S, OUT_NCHW, 64>, 256, 64, 256);
            if constexpr (sizeof(S) > 1)
                if (tile == TILE_512x128_ROWWIN_PP) {
                    if (a.skp) return go(igemm_rowwin_pp_kernel<S, OUT_NCHW, true>, 512, 128, 512, true);
                    return go(igemm_rowwin_pp_kernel<S, OUT_NCHW>, 512, 128, 512);
                }
        }
        return hipErrorInvalidValue;
    } else if constexpr (FEED == FEED_ROWWIN_NCHW) {  // NCHW read in place: 16-bit types, NCHW output
        if constexpr (AVEC && sizeof(S) == 2 && OUT_NCHW) {
            if (tile == TILE_256x128_ROWWIN) return go(igemm_rowwin_kernel<S, OUT_NCHW, 128, true>, 256, 128, 256);
            if (tile == TILE_256x64_ROWWIN) return go(igemm_rowwin_kernel<S, OUT_NCHW, 64, true>, 256, 64, 256);
        }
        return hipErrorInvalidValue;
    } else if constexpr (FEED == FEED_GEMM_NCHW) {  // 1x1 NCHW read in place: 16-bit types, NCHW output
        if constexpr (AVEC && sizeof(S) == 2 && OUT_NCHW) {
            switch (tile) {
                case TILE_256x128_DUAL: return go(igemm_dual_kernel<S, FEED, OUT_NCHW>, 256, 128);
                case TILE_256x128_OCT: return go(igemm_oct_kernel<S, FEED, OUT_NCHW>, 256, 128, 512);
                case TILE_128x64_QUAD: return go(igemm_quad_kernel<S, FEED, OUT_NCHW>, 128, 64);
                case TILE_256x256_OCT: return go(igemm_oct_sq_kernel<S, FEED, OUT_NCHW>, 256, 256, 512);
                default: return hipErrorInvalidValue;
            }
        }
        return hipErrorInvalidValue;
    } else if constexpr (AVEC && (FEED == FEED_IND_CHUNK || FEED == FEED_WIN_CHUNK)) {  // one tap per chunk: the two-wavefront loops only
        switch (tile) {
            case TILE_256x128_DUAL: return go(igemm_dual_kernel<S, FEED, OUT_NCHW>, 256, 128);
            case TILE_256x128_OCT: return go(igemm_oct_kernel<S, FEED, OUT_NCHW>, 256, 128, 512);
            case TILE_128x64_QUAD: return go(igemm_quad_kernel<S, FEED, OUT_NCHW>, 128, 64);
            case TILE_256x256_OCT: return go(igemm_oct_sq_kernel<S, FEED, OUT_NCHW>, 256, 256, 512);
            default: return hipErrorInvalidValue;
        }
    } else if constexpr (AVEC) {  // 16-byte rows: straight-to-LDS pipeline
        switch (tile) {
            case TILE_128x128: return go(igemm_dma_kernel<S, FEED, OUT_NCHW, 128, 128, BKW>, 128, 128);
            case TILE_128x64: return go(igemm_dma_kernel<S, FEED, OUT_NCHW, 128, 64, BKW>, 128, 64);
            case TILE_32x64: return go(igemm_dma_kernel<S, FEED, OUT_NCHW, 32, 64, BKW>, 32, 64);
            case TILE_256x128: return go(igemm_dma_kernel<S, FEED, OUT_NCHW, 256, 128, BKW>, 256, 128);
            case TILE_256x128_DUAL: return go(igemm_dual_kernel<S, FEED, OUT_NCHW>, 256, 128);
            case TILE_256x128_OCT: return go(igemm_oct_kernel<S, FEED, OUT_NCHW>, 256, 128, 512);
            case TILE_128x64_QUAD: return go(igemm_quad_kernel<S, FEED, OUT_NCHW>, 128, 64);
            case TILE_256x256_OCT: return go(igemm_oct_sq_kernel<S, FEED, OUT_NCHW>, 256, 256, 512);
            default: return hipErrorInvalidValue;
        }
    } else {  // element gathers through registers
        switch (tile) {
            case TILE_128x128: return go(igemm_kernel<S, FEED, AVEC, BVEC, OUT_NCHW, 128, 128, BKW>, 128, 128);
            case TILE_128x64: return go(igemm_kernel<S, FEED, AVEC, BVEC, OUT_NCHW, 128, 64, BKW>, 128, 64);
            case TILE_32x64: return go(igemm_kernel<S, FEED, AVEC, BVEC, OUT_NCHW, 32, 64, BKW>, 32, 64);
            default: return hipErrorInvalidValue;
        }
    }
}

// All (vector-load, output-layout) variants a feed can need.
template <typename S, int FEED>
hipError_t launch_feed(const GemmArgs &a, bool out_nchw, bool a_vec, bool b_vec, int tile, int splits,
                       hipStream_t st) {
    constexpr bool CAN_AVEC = FEED == FEED_ROWMAJOR || FEED == FEED_IND_NHWC || FEED == FEED_WIN ||
                              FEED == FEED_IND_CHUNK || FEED == FEED_WIN_CHUNK || FEED == FEED_ROWWIN ||
                              FEED == FEED_ROWWIN_NCHW || FEED == FEED_GEMM_NCHW;
    constexpr bool CAN_NCHW = true;  // every feed can write NCHW output
    constexpr bool CAN_NHWC = FEED == FEED_ROWMAJOR || FEED == FEED_IND_NHWC || FEED == FEED_WIN ||
                              FEED == FEED_IND_CHUNK || FEED == FEED_WIN_CHUNK || FEED == FEED_ROWWIN ||
                              FEED == FEED_ROWWIN_NCHW;
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
