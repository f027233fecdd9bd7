// The lowering steps that run before (or after) the main loop:
//   (b) the indirection-buffer builder (The Indirect Convolution Algorithm, abstract),
//   (a) the im2win window reorder ("Im2win: An Efficient Convolution Paradigm on GPU", abstract),
//   the NCHW -> NHWC copy and the OIHW -> OHWI weight regrouping that let
//   NCHW tensors use the channels-last feeds,
//   and the ordered split-K finishing pass.
#include <type_traits>

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

// X_col, the im2col matrix ("Unifying Convolutions and GEMM", section 2):
// row m = (n, ho, wo), columns (ci, kh, kw) from NCHW input or (kh, kw, ci)
// from NHWC input, zero in the padding.  From NHWC input: one thread per
// 16-byte chunk of a row (VEC consecutive columns), consecutive threads on
// consecutive chunks.  CHUNK_LOAD: the chunk is VEC channels of one tap,
// read as one 16-byte load.
template <typename S, bool CHUNK_LOAD>
__global__ __launch_bounds__(256) void im2col_nhwc_kernel(const S *__restrict__ x, S *__restrict__ xc, Geom g) {
    constexpr int VEC = 16 / (int)sizeof(S);
    const long long cpr = (g.K + VEC - 1) / VEC;  // chunks per row
    const long long q = (long long)blockIdx.x * 256 + threadIdx.x;
    if (q >= g.M * cpr) return;
    const long long m = q / cpr;
    const int k0 = (int)(q - m * cpr) * VEC;
    const long long n = m / g.P;
    const int p = (int)(m - n * g.P);
    const int ho = p / g.Wo, wo = p - ho * g.Wo;
    const int hb = ho * g.s - g.p, wb = wo * g.s - g.p;
    S e[VEC];
    if constexpr (CHUNK_LOAD) {
        const int t = k0 / g.C, ci = k0 - t * g.C;
        const int kh = t / g.KW, kw = t - kh * g.KW;
        const int hi = hb + kh * g.d, wi = wb + kw * g.d;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (hi >= 0 && hi < g.H && wi >= 0 && wi < g.W)
            v = *(const uint4 *)(x + ((n * g.H + hi) * g.W + wi) * g.C + ci);
        __builtin_memcpy(e, &v, 16);
    } else {
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
            const int k = k0 + j;
            S v = S(0);
            if (k < g.K) {
                const int t = k / g.C, ci = k - t * g.C;
                const int kh = t / g.KW, kw = t - kh * g.KW;
                const int hi = hb + kh * g.d, wi = wb + kw * g.d;
                if (hi >= 0 && hi < g.H && wi >= 0 && wi < g.W) v = x[((n * g.H + hi) * g.W + wi) * g.C + ci];
            }
            e[j] = v;
        }
    }
    S *dst = xc + m * g.K + k0;
    if (g.K % VEC == 0) {
        uint4 out;
        __builtin_memcpy(&out, e, 16);
        *(uint4 *)dst = out;
    } else {
#pragma unroll
        for (int j = 0; j < VEC; ++j)
            if (k0 + j < g.K) dst[j] = e[j];
    }
}

// X_col from NCHW input through a 64 x 64 LDS tile (rows m, columns k): the
// gathers walk consecutive output pixels of one column (neighbouring input
// pixels of one channel plane) and the stores leave as whole row pieces.
template <typename S>
__global__ __launch_bounds__(256) void im2col_nchw_tiled_kernel(const S *__restrict__ x, S *__restrict__ xc,
                                                                Geom g) {
    constexpr int TM = 64, TK = 64, VEC = 16 / (int)sizeof(S);
    __shared__ S tile[TM][TK + VEC];
    const int ktiles = (int)((g.K + TK - 1) / TK);
    const long long m0 = (long long)(blockIdx.x / ktiles) * TM;
    const int kt0 = (int)(blockIdx.x % ktiles) * TK;
    const int tid = threadIdx.x;
    const int ml = tid % TM;
    const long long m = m0 + ml;
    const bool mok = m < g.M;
    const long long n = mok ? m / g.P : 0;
    const int p = mok ? (int)(m - n * g.P) : 0;
    const int ho = p / g.Wo, wo = p - ho * g.Wo;
    const int hb = ho * g.s - g.p, wb = wo * g.s - g.p;
    const S *xn = x + n * g.C * (long long)g.H * g.W;
#pragma unroll 4
    for (int i = 0; i < TK / 4; ++i) {  // column kl = tid / 64 + 4 i of the tile
        const int kl = tid / TM + 4 * i;
        const int k = kt0 + kl;
        S v = S(0);
        if (mok && k < g.K) {
            const int ci = k / g.T, t = k - ci * g.T;
            const int kh = t / g.KW, kw = t - kh * g.KW;
            const int hi = hb + kh * g.d, wi = wb + kw * g.d;
            if (hi >= 0 && hi < g.H && wi >= 0 && wi < g.W) v = xn[((long long)ci * g.H + hi) * g.W + wi];
        }
        tile[ml][kl] = v;
    }
    __syncthreads();
    constexpr int CPR = TK / VEC;  // chunks per tile row
    const bool vec_rows = g.K % VEC == 0;
    for (int c = tid; c < TM * CPR; c += 256) {
        const int r = c / CPR, kc = (c - r * CPR) * VEC;
        const long long mr = m0 + r;
        const int k = kt0 + kc;
        if (mr >= g.M || k >= g.K) continue;
        S *dst = xc + mr * g.K + k;
        if (vec_rows) {  // K % VEC == 0: the chunk is whole and aligned
            uint4 out;
            __builtin_memcpy(&out, &tile[r][kc], 16);
            *(uint4 *)dst = out;
        } else {
            for (int j = 0; j < VEC && k + j < g.K; ++j) dst[j] = tile[r][kc + j];
        }
    }
}

template <typename S>
static hipError_t im2col_typed(const void *x, void *xcol, const Geom &g, bool nhwc, hipStream_t st) {
    constexpr int VEC = 16 / (int)sizeof(S);
    const long long chunks = g.M * ((g.K + VEC - 1) / VEC);
    const dim3 grid(blocks_for(chunks, 256));
    const S *xs = (const S *)x;
    S *xd = (S *)xcol;
    if (nhwc && g.C % VEC == 0 && (uintptr_t)x % 16 == 0)
        hipLaunchKernelGGL((im2col_nhwc_kernel<S, true>), grid, dim3(256), 0, st, xs, xd, g);
    else if (nhwc)
        hipLaunchKernelGGL((im2col_nhwc_kernel<S, false>), grid, dim3(256), 0, st, xs, xd, g);
    else
        hipLaunchKernelGGL(im2col_nchw_tiled_kernel<S>, dim3((unsigned)(((g.M + 63) / 64) * ((g.K + 63) / 64))),
                           dim3(256), 0, st, xs, xd, g);
    return hipGetLastError();
}

hipError_t launch_im2col(const void *x, void *xcol, const Geom &g, bool nhwc, bool bf16, hipStream_t st) {
    // 16-byte stores need 16-byte rows on a 16-byte-aligned matrix.
    const int VEC = bf16 ? 8 : 4;
    if (g.K % VEC == 0 && (uintptr_t)xcol % 16 != 0) return hipErrorInvalidValue;
    return bf16 ? im2col_typed<uint16_t>(x, xcol, g, nhwc, st) : im2col_typed<float>(x, xcol, g, nhwc, st);
}

// The window-ordered tensor with the channels of every (column, kernel row)
// cell padded to cp, a multiple of the 16-byte chunk VEC = 16 / sizeof(S):
// Xwin[n][ho][c][kh][cp], zero for channels >= C and in the padding.  One
// thread per 16-byte chunk, chunks in memory order, so the stores are
// contiguous.
template <typename S, bool NHWC_IN>
__global__ __launch_bounds__(256) void im2win_pad_kernel(const S *__restrict__ x, S *__restrict__ xw, Geom g,
                                                         int cp) {
    constexpr int VEC = 16 / (int)sizeof(S);
    const int cpt = cp / VEC;  // chunks per cell
    const long long q = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long chunks = (long long)g.N * g.Ho * g.Wwin * g.KH * cpt;
    if (q >= chunks) return;
    long long r = q / cpt;
    const int ch = (int)(q - r * cpt) * VEC;
    const int kh = (int)(r % g.KH);
    r /= g.KH;
    const int c = (int)(r % g.Wwin);
    r /= g.Wwin;
    const int ho = (int)(r % g.Ho);
    const long long n = r / g.Ho;
    const int hi = ho * g.s + kh * g.d - g.p, wi = c - g.p;
    S e[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) e[j] = S(0);
    if (hi >= 0 && hi < g.H && wi >= 0 && wi < g.W) {
        const long long pix = ((long long)hi * g.W + wi);
#pragma unroll
        for (int j = 0; j < VEC; ++j)
            if (ch + j < g.C)
                e[j] = NHWC_IN ? x[(n * g.H * g.W + pix) * g.C + ch + j]
                               : x[(n * g.C + ch + j) * (long long)g.H * g.W + pix];
    }
    uint4 out;
    __builtin_memcpy(&out, e, 16);
    *(uint4 *)(xw + q * VEC) = out;
}

hipError_t launch_im2win_pad(const void *x, void *xwin, const Geom &g, int cp, bool nhwc, bool bf16,
                             hipStream_t st) {
    const int VEC = bf16 ? 8 : 4;
    if ((uintptr_t)xwin % 16 != 0 || cp % VEC != 0 || cp < g.C) return hipErrorInvalidValue;
    const long long chunks = (long long)g.N * g.Ho * g.Wwin * g.KH * (cp / VEC);
    const dim3 grid(blocks_for(chunks, 256));
    if (bf16) {
        if (nhwc)
            hipLaunchKernelGGL((im2win_pad_kernel<uint16_t, true>), grid, dim3(256), 0, st, (const uint16_t *)x,
                               (uint16_t *)xwin, g, cp);
        else
            hipLaunchKernelGGL((im2win_pad_kernel<uint16_t, false>), grid, dim3(256), 0, st, (const uint16_t *)x,
                               (uint16_t *)xwin, g, cp);
    } else {
        if (nhwc)
            hipLaunchKernelGGL((im2win_pad_kernel<float, true>), grid, dim3(256), 0, st, (const float *)x,
                               (float *)xwin, g, cp);
        else
            hipLaunchKernelGGL((im2win_pad_kernel<float, false>), grid, dim3(256), 0, st, (const float *)x,
                               (float *)xwin, g, cp);
    }
    return hipGetLastError();
}

// NCHW -> channels-last copy of x, transposed through LDS in tiles of 64
// channels x 64 pixels.  Loads run along the pixels of one channel plane in
// LW-byte chunks (the widest that the plane length H*W and the pointer
// alignment allow, so a chunk never leaves its plane); stores run along the
// channels of one pixel in 16-byte chunks.  The copy's pixel rows hold CP >= C
// channels (CP a multiple of the 16-byte element count); channels C..CP-1 are
// written as zeros.
constexpr int kTrC = 64, kTrP = 64;  // tile: channels x pixels

template <typename S, int LW>
__device__ __forceinline__ void transpose_tile(const S *__restrict__ x, S *__restrict__ xc, int C, int CP, int HW,
                                               int n, int c0, int p0, S (*tile)[kTrP + 2]) {
    constexpr int LE = LW / (int)sizeof(S);  // elements per load
    constexpr int CPR = kTrP / LE;           // loads per channel row
    constexpr int NL = kTrC * CPR / 256;     // loads per thread
    static_assert(NL >= 1 && (kTrC * CPR) % 256 == 0, "tile must split evenly");
    typedef typename std::conditional<LW == 16, uint4,
            typename std::conditional<LW == 8, uint2,
            typename std::conditional<LW == 4, uint32_t, S>::type>::type>::type chunk_t;
    const int tid = threadIdx.x;
    const S *src = x + (long long)n * C * HW;
    chunk_t v[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {  // every load first, then the LDS writes
        const int q = tid + 256 * i;
        const int cl = q / CPR, pl = (q % CPR) * LE;
        const int c = c0 + cl, p = p0 + pl;
        v[i] = chunk_t{};
        if (c < C && p < HW) v[i] = *(const chunk_t *)(src + (long long)c * HW + p);
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int q = tid + 256 * i;
        const int cl = q / CPR, pl = (q % CPR) * LE;
        S e[LE];
        __builtin_memcpy(e, &v[i], LW);
#pragma unroll
        for (int j = 0; j < LE; ++j) tile[cl][pl + j] = e[j];
    }
    __syncthreads();
    constexpr int V = 16 / (int)sizeof(S);
    constexpr int CPP = kTrC / V;  // 16-byte chunks per pixel
    S *dst = xc + (long long)n * CP * HW;
#pragma unroll
    for (int i = 0; i < kTrP * CPP / 256; ++i) {
        const int q = tid + 256 * i;
        const int pl = q / CPP, cl = (q % CPP) * V;
        const int c = c0 + cl, p = p0 + pl;
        if (c >= CP || p >= HW) continue;
        S e[V];
#pragma unroll
        for (int j = 0; j < V; ++j) e[j] = tile[cl + j][pl];
        uint4 out;
        __builtin_memcpy(&out, e, 16);
        *(uint4 *)(dst + (long long)p * CP + c) = out;
    }
}

// One launch for the preparation of a call that reads a channels-last copy
// of x: blocks [0, nt) make the copy (transposed from NCHW, or re-strided
// from NHWC, with pixel rows of CP channels), the next nib blocks build the
// indirection buffer over the copy, the rest put the weights in (kh, kw, ci)
// order with CP channels (from OIHW or OHWI; when nw > 0).
struct PrepArgs {
    const void *x;
    void *xc;
    int32_t *ib;
    const void *w;
    void *wo;
    Geom g;                // of the call (C = the input's channel count)
    int cp;                // channels per pixel row of the copy and the weights
    int tiles_p, tiles_c;  // transpose tiles per image along pixels, channels
    int nt, nib;           // blocks of the first two kinds
    long long nw;          // weight elements to write (0: none)
    int w_ohwi;            // weights given as OHWI (else OIHW)
    uint32_t *zero;        // words block 0 sets to zero (nzero of them), or null
    int nzero;
};

template <typename S, int LW, bool NHWC_IN>
__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a) {
    __shared__ S tile[NHWC_IN ? 1 : kTrC][kTrP + 2];
    const Geom &g = a.g;
    const int CP = a.cp;
    int b = blockIdx.x;
    if (b == 0)
        for (int i = threadIdx.x; i < a.nzero; i += 256) a.zero[i] = 0u;
    if (b < a.nt) {
        if constexpr (NHWC_IN) {  // one thread per 16-byte chunk (pixel, channels 8q.. or 4q..) of the copy
            constexpr int V = 16 / (int)sizeof(S);
            const int CQ = CP / V;  // chunks per pixel row of the copy
            const long long e = (long long)b * 256 + threadIdx.x;
            if (e >= (long long)g.N * g.H * g.W * CQ) return;
            const long long pix = e / CQ;
            const int c0 = (int)(e - pix * CQ) * V;
            const S *src = (const S *)a.x + pix * g.C;
            S v[V];
#pragma unroll
            for (int j = 0; j < V; ++j) v[j] = c0 + j < g.C ? src[c0 + j] : S(0);
            uint4 out;
            __builtin_memcpy(&out, v, 16);
            *(uint4 *)((S *)a.xc + pix * CP + c0) = out;
        } else {
            // Blocks go to the eight XCDs in turn (block b to XCD b % 8).  Each
            // XCD takes a contiguous run of the tiles instead, so neighbouring
            // pixel tiles of one channel group run on one XCD, one after the
            // other, and the cache line a tile's rows share with the next
            // tile's (plane rows need not start on a line) is read from HBM
            // once, not by two XCDs.
            const int nt8 = a.nt & ~7;
            if (b < nt8) b = (b & 7) * (nt8 >> 3) + (b >> 3);
            const int pt = b % a.tiles_p;
            b /= a.tiles_p;
            const int ct = b % a.tiles_c, n = b / a.tiles_c;
            transpose_tile<S, LW>((const S *)a.x, (S *)a.xc, g.C, CP, g.H * g.W, n, ct * kTrC, pt * kTrP, tile);
        }
        return;
    }
    b -= a.nt;
    if (b < a.nib) {
        const long long idx = (long long)b * 256 + threadIdx.x;
        if (idx >= (long long)g.P * g.T) return;
        const int p = (int)(idx / g.T), t = (int)(idx - (long long)p * g.T);
        const int ho = p / g.Wo, wo = p - ho * g.Wo;
        const int kh = t / g.KW, kw = t - kh * g.KW;
        const int hi = ho * g.s + kh * g.d - g.p, wi = wo * g.s + kw * g.d - g.p;
        a.ib[idx] = (hi >= 0 && hi < g.H && wi >= 0 && wi < g.W) ? (hi * g.W + wi) * CP : -1;
        return;
    }
    b -= a.nib;
    const long long e = (long long)b * 256 + threadIdx.x;
    if (e >= a.nw) return;
    const int ci = (int)(e % CP);
    const long long r = e / CP;
    const int t = (int)(r % g.T);
    const long long co = r / g.T;
    S v = S(0);
    if (ci < g.C)
        v = a.w_ohwi ? ((const S *)a.w)[(co * g.T + t) * g.C + ci] : ((const S *)a.w)[(co * g.C + ci) * g.T + t];
    ((S *)a.wo)[e] = v;
}

hipError_t launch_prep(const void *x, bool nhwc_in, void *x_cl, int cp, int32_t *ib, const void *w, bool w_ohwi,
                       void *w_out, const Geom &g, int es, hipStream_t st, uint32_t *zero, int nzero) {
    const int ES = es, HW = g.H * g.W;
    const bool bf16 = es == 2;
    PrepArgs a;
    a.x = x;
    a.xc = x_cl;
    a.ib = ib;
    a.w = w;
    a.wo = w_out;
    a.g = g;
    a.cp = cp;
    a.w_ohwi = w_ohwi ? 1 : 0;
    a.tiles_p = (HW + kTrP - 1) / kTrP;
    a.tiles_c = (cp + kTrC - 1) / kTrC;
    if (x_cl)
        a.nt = nhwc_in ? (int)blocks_for((long long)g.N * HW * (cp / (16 / ES)), 256) : g.N * a.tiles_c * a.tiles_p;
    else
        a.nt = 0;
    a.nib = ib ? (int)blocks_for((long long)g.P * g.T, 256) : 0;
    a.nw = w_out ? (long long)g.Co * g.T * cp : 0;
    a.zero = zero;
    a.nzero = zero ? nzero : 0;
    long long blocks = (long long)a.nt + a.nib + blocks_for(a.nw, 256);
    if (blocks == 0 && a.nzero > 0) blocks = 1;
    if (blocks == 0) return hipSuccess;
    // Widest load that keeps every chunk inside its channel plane and aligned.
    int lw = 16;
    while (lw > ES && ((long long)HW * ES % lw != 0 || (uintptr_t)x % lw != 0)) lw >>= 1;
    if (x_cl && ((uintptr_t)x_cl % 16 != 0 || (cp * ES) % 16 != 0)) return hipErrorInvalidValue;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, st, a);
        return hipGetLastError();
    };
    if (es == 1) {
        // 8-bit elements (fp8 inputs): NCHW input read in 4- to 16-byte pieces only.
        if (nhwc_in) return hipErrorInvalidValue;
        switch (lw) {
            case 16: return go(prep_kernel<uint8_t, 16, false>);
            case 8: return go(prep_kernel<uint8_t, 8, false>);
            case 4: return go(prep_kernel<uint8_t, 4, false>);
            default: return hipErrorInvalidValue;
        }
    }
    if (nhwc_in) return bf16 ? go(prep_kernel<uint16_t, 2, true>) : go(prep_kernel<float, 4, true>);
    if (bf16) {
        switch (lw) {
            case 16: return go(prep_kernel<uint16_t, 16, false>);
            case 8: return go(prep_kernel<uint16_t, 8, false>);
            case 4: return go(prep_kernel<uint16_t, 4, false>);
            default: return go(prep_kernel<uint16_t, 2, false>);
        }
    }
    switch (lw) {
        case 16: return go(prep_kernel<float, 16, false>);
        case 8: return go(prep_kernel<float, 8, false>);
        default: return go(prep_kernel<float, 4, false>);
    }
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

// OIHW weights regrouped tap-major for the NCHW window-row loop:
// o[((s*T + t)*Co + co)*bk + c] = w[co][s*bk + c][t] for channel slices s of
// bk channels (the loop's K tiles), so that the B rows one tap of one slice
// needs for consecutive output channels are consecutive.  One thread per
// destination element; sizes are below 2^31 elements.
template <typename S>
__global__ __launch_bounds__(256) void pack_tapmajor_kernel(const S *__restrict__ w, S *__restrict__ o, Geom g,
                                                            int bk) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    const int total = g.Co * g.T * g.C;
    if (e >= total) return;
    const int c = e % bk;
    const int r = e / bk;
    const int co = r % g.Co;
    const int st = r / g.Co;  // s*T + t
    const int t = st % g.T, sl = st / g.T;
    o[e] = w[(co * g.C + sl * bk + c) * g.T + t];
}

hipError_t launch_pack_weights_tapmajor(const void *w, void *o, const Geom &g, int bk, hipStream_t st) {
    const long long total = (long long)g.Co * g.T * g.C;
    hipLaunchKernelGGL(pack_tapmajor_kernel<uint16_t>, dim3(blocks_for(total, 256)), dim3(256), 0, st,
                       (const uint16_t *)w, (uint16_t *)o, g, bk);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split-K finish: y = round(sum over splits, in split order, + bias).  The
// fixed order keeps the result bit-for-bit repeatable.  Rounding to nearest,
// ties to even (gfx950's v_cvt_pk_bf16_f32; the default mode for fp16).
__device__ __forceinline__ float red_load(const uint16_t *p, int i) { return __uint_as_float((uint32_t)p[i] << 16); }
__device__ __forceinline__ float red_load(const _Float16 *p, int i) { return (float)p[i]; }
__device__ __forceinline__ float red_load(const float *p, int i) { return p[i]; }
__device__ __forceinline__ uint16_t red_out(uint16_t, float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ _Float16 red_out(_Float16, float f) { return (_Float16)f; }
__device__ __forceinline__ float red_out(float, float f) { return f; }

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
    if (bias) acc += red_load(bias, co);
    long long yi = e;
    if constexpr (OUT_NCHW) {
        long long n = m / g.P;
        yi = (n * g.Co + co) * g.P + (m - n * g.P);
    }
    y[yi] = red_out(S(), acc);
}

template <typename S>
static void reduce_typed(const float *part, const void *bias, void *y, const Geom &g, int splits, bool out_nchw,
                         dim3 grid, hipStream_t st) {
    if (out_nchw)
        hipLaunchKernelGGL((splitk_reduce_kernel<S, true>), grid, dim3(256), 0, st, part, (const S *)bias, (S *)y, g,
                           splits);
    else
        hipLaunchKernelGGL((splitk_reduce_kernel<S, false>), grid, dim3(256), 0, st, part, (const S *)bias, (S *)y, g,
                           splits);
}

hipError_t launch_splitk_reduce(const float *part, const void *bias, void *y, const Geom &g, int splits,
                                bool out_nchw, int dtype, hipStream_t st) {
    long long total = g.M * g.Co;
    dim3 grid(blocks_for(total, 256));
    if (dtype == 1)
        reduce_typed<uint16_t>(part, bias, y, g, splits, out_nchw, grid, st);
    else if (dtype == 2)
        reduce_typed<_Float16>(part, bias, y, g, splits, out_nchw, grid, st);
    else
        reduce_typed<float>(part, bias, y, g, splits, out_nchw, grid, st);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t *p, int n) {
    const int i = (int)blockIdx.x * 256 + (int)threadIdx.x;
    if (i < n) p[i] = 0u;
}

hipError_t launch_zero_words(uint32_t *p, int n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks_for(n, 256)), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

}  // namespace convlower
