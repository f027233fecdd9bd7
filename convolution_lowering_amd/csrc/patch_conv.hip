// Inputs with at most four channels: the indirect convolution of "The
// Indirect Convolution Algorithm" (abstract), with the input patch of a few
// output rows staged in LDS and each tap's input pixel addressed there on the
// fly, instead of an indirection buffer in memory.
//
// With C_in <= 4, a 16-byte chunk of the lowered row X_col[m] (K order: tap,
// then channel, channels padded to 4) is two whole taps for 16-bit types and
// one for fp32, so each A fragment is one or two aligned LDS reads of a
// staged pixel.  The weights of a block's 64 output channels, zero-padded the
// same way, stay in registers as MFMA B fragments for all of K (at most 16
// K steps).  A block is persistent: it stages the input rows that R output
// rows of one image need (4 channels per pixel, zeros for padding and for
// channels past C_in), multiplies every 32-pixel fragment of those rows
// against its weights, stores the results with the bias added in fp32 and
// one rounding, and moves on to the next group of rows.  No workspace.
#include <type_traits>

#include "igemm_impl.h"

namespace convlower {
namespace {

constexpr int kPatchStageBytes = 24 * 1024;  // LDS of the staged input rows
constexpr int kPatchMaxKSteps = 16;          // K steps of register-resident weights
constexpr int kPatchThreads = 256;

struct PatchArgs {
    const void *x, *w, *bias;
    void *y;
    Geom g;
    int R;              // output rows per unit
    int RIN, WIN;       // staged input rows and columns of a unit
    int hgroups;        // ceil(Ho / R)
    int units;          // N * hgroups
    int ksteps;         // ceil(KH*KW / taps per K step)
    // 16-bit input staged in 16-byte loads of 8 consecutive input columns
    // (W a multiple of 8, x 16-byte aligned, below 2^31 bytes, at most
    // 2 * kPatchThreads such loads of each channel per unit), else one
    // element at a time.
    int vec;
    unsigned x_bytes;   // |x| in bytes when vec (the loads' range check)
};

// Four outputs, rounded once to nearest-even, into LDS at p.
__device__ __forceinline__ void obuf_put4_impl(uint16_t, char *p, float a, float b, float c, float d) {
    *(uint2 *)p = make_uint2(f32x2_to_bf16x2_rne(a, b), f32x2_to_bf16x2_rne(c, d));
}
__device__ __forceinline__ void obuf_put4_impl(_Float16, char *p, float a, float b, float c, float d) {
    *(uint2 *)p = make_uint2(f32x2_to_f16x2_rne(a, b), f32x2_to_f16x2_rne(c, d));
}
__device__ __forceinline__ void obuf_put4_impl(float, char *p, float a, float b, float c, float d) {
    *(float4 *)p = make_float4(a, b, c, d);
}
__device__ __forceinline__ uint16_t raw16(const uint16_t *p, long long i) { return p[i]; }
__device__ __forceinline__ uint16_t raw16(const _Float16 *p, long long i) {
    return __builtin_bit_cast(uint16_t, p[i]);
}

// KS: K steps the kernel holds weights for (3, 4, 8, 13 or 16; the layer's own
// count P.ksteps is at most that).
// Resident blocks per compute unit: three for channels-last output in 16-bit
// types with at most 4 K steps (registers and LDS allow it there, and it
// measured faster: C4a 225 -> 198 us, where NCHW output measured slower),
// else two.  The persistent grid is sized to exactly the resident blocks.
constexpr int patch_blocks_per_cu(int ks, int es, bool nchw) { return (ks <= 4 && es == 2 && !nchw) ? 3 : 2; }

// VS: the input staged in 16-byte loads (PatchArgs::vec; 16-bit types).
template <typename S, bool NCHW, int KS, bool VS = false>
__global__ __launch_bounds__(kPatchThreads, patch_blocks_per_cu(KS, (int)sizeof(S), NCHW)) void patch_conv_kernel(PatchArgs P) {
    static_assert(!VS || sizeof(S) == 2, "16-byte staging for 16-bit types");
    using MF = MfmaShape<S, 32>;
    constexpr int ES = (int)sizeof(S);
    auto obuf_put4 = [](char *p, float a, float b, float c, float d) { obuf_put4_impl(S(), p, a, b, c, d); };
    constexpr int PB = 4 * ES;        // bytes of one staged pixel (4 channels)
    constexpr int TPC = 16 / PB;      // taps per 16-byte chunk: 2 (16-bit) or 1 (fp32)
    constexpr int TPS = 2 * TPC;      // taps per MFMA K step (two chunks: lanes 0-31, 32-63)
    constexpr int NQ = MF::NQ;
    __shared__ uint4 stage[kPatchStageBytes / 16];
    char *const sbytes = (char *)stage;
    // Each wavefront's output tile: rows of the output's contiguous axis
    // (NCHW: 64 channel rows of 32 pixels; NHWC: 32 pixel rows of 64
    // channels), each padded by 16 bytes against bank conflicts.
    constexpr int ORS = (NCHW ? 32 : 64) * ES + 16;  // row stride, bytes
    constexpr int OROWS = NCHW ? 64 : 32;
    __shared__ uint4 obuf[4][(OROWS * ORS) / 16];
    __shared__ float4 bias_s[16];  // the block's 64 channels' bias (0 past C_out or without bias)
    __shared__ uint4 zero16;       // what a tap past the last reads
    const char *const zb = (const char *)&zero16;

    const Geom &g = P.g;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    char *const ob = (char *)obuf[wave];
    const int half = lane >> 5, col = lane & 31;
    const int cob = blockIdx.y * 64;
    const int T = g.KH * g.KW;
    const S *x = (const S *)P.x;
    const S *w = (const S *)P.w;
    S *y = (S *)P.y;

    // ---- weights as B fragments: lane (half, col) of K step ks holds, for
    // output channel cob + 32*ic + col, the channels 0..3 of taps
    // ks*TPS + half*TPC .. +TPC-1 (zero past C_in, past the last tap and past
    // C_out).
    // Weights in LDS, one copy for the block: registers stay free for the
    // next unit's input loads.
    __shared__ uint4 wlds[KS * 2 * 64];
    // Byte offset (within the stage) of each of this lane's taps relative to
    // its output pixel's first tap, 16 bits per tap (the stage is 24 KB),
    // 0xFFFF for a tap past the last.
    uint32_t toff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        toff[ks] = 0;
#pragma unroll
        for (int tt = 0; tt < TPC; ++tt) {
            const int t = ks * TPS + half * TPC + tt;
            const uint32_t o = (ks < P.ksteps && t < T)
                                   ? (uint32_t)(((t / g.KW) * g.d * P.WIN + (t % g.KW) * g.d) * PB)
                                   : 0xFFFFu;
            toff[ks] |= o << (16 * tt);
        }
    }
    // B fragment of K step ks, channel half ic for this lane: the channels
    // 0..3 of taps ks*TPS + half*TPC .. +TPC-1 of output channel
    // cob + 32*ic + col (zero past C_in, past the last tap and past C_out).
    auto wfrag = [&](int ks, int ic) {
        const int co = cob + 32 * ic + col;
        uint32_t wv[4] = {0u, 0u, 0u, 0u};
        if (ks < P.ksteps && co < g.Co) {
#pragma unroll
            for (int tt = 0; tt < TPC; ++tt) {
                const int t = ks * TPS + half * TPC + tt;
                if (t >= T) continue;
                const int kh = t / g.KW, kw = t % g.KW;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (c >= g.C) continue;
                    const long long wi = NCHW ? (((long long)co * g.C + c) * g.KH + kh) * g.KW + kw
                                              : (((long long)co * g.KH + kh) * g.KW + kw) * g.C + c;
                    if constexpr (ES == 2) {
                        const uint32_t v = raw16(w, wi);
                        const int e = tt * 4 + c;  // element of the 8 in the chunk
                        wv[e >> 1] |= v << (16 * (e & 1));
                    } else {
                        wv[c] = __float_as_uint(((const float *)w)[wi]);
                    }
                }
            }
        }
        return make_uint4(wv[0], wv[1], wv[2], wv[3]);
    };
    for (int ks = wave; ks < KS; ks += kPatchThreads / 64)  // published by the unit loop's first barrier
        for (int ic = 0; ic < 2; ++ic) wlds[(ks * 2 + ic) * 64 + lane] = wfrag(ks, ic);

    if (tid == 64) zero16 = make_uint4(0u, 0u, 0u, 0u);  // published by the unit loop's first barrier
    if (tid < 64) {
        const int co = cob + tid;
        ((float *)bias_s)[tid] = (P.bias && co < g.Co) ? bits_to_f32(S(), elem_bits((const S *)P.bias, co)) : 0.f;
    }  // published by the barrier at the top of the unit loop

    const int frags_per_row = (g.Wo + 31) / 32;
    // 16-byte global stores: every piece's address then a multiple of 16.
    const bool vec_store = NCHW ? ((g.Wo * ES) % 16 == 0 && (uintptr_t)y % 16 == 0)
                                : ((g.Co * ES) % 16 == 0 && (uintptr_t)y % 16 == 0);

    // ---- staging: pixel (r, c) of unit u's stage is x[n][hi_base + r][c - p],
    // channels 0..3, zeros outside the image and past C_in.  A thread loads
    // SB pixels (for NCHW input each channel's loads run along a plane row)
    // before it writes any; the first SB pixels of the next unit are loaded
    // while the current one is multiplied.
    constexpr int SB = 12;
    const int npix = P.RIN * P.WIN;
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    // 16-bit types: two channels per register (loaded into its halves);
    // fp32: one per register.
    u16x2 hv[ES == 2 && !VS ? SB : 1][2];
    float v[ES == 2 ? 1 : SB][4];
    auto load_batch = [&](int u, int base) {
        const int n = u / P.hgroups;
        const int hi_base = (u - n * P.hgroups) * P.R * g.s - g.p;
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int idx = base + j * kPatchThreads + tid;
            const int r = idx / P.WIN, c = idx - r * P.WIN;
            const int hi = hi_base + r, wi = c - g.p;
            const bool in = idx < npix && hi >= 0 && hi < g.H && wi >= 0 && wi < g.W;
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
                const long long xi = NCHW ? (((long long)n * g.C + ch) * g.H + hi) * g.W + wi
                                          : (((long long)n * g.H + hi) * g.W + wi) * g.C + ch;
                const bool ld = in && ch < g.C;
                if constexpr (ES == 2)
                    hv[j][ch >> 1][ch & 1] = ld ? raw16(x, xi) : (unsigned short)0;
                else
                    v[j][ch] = ld ? ((const float *)x)[xi] : 0.f;
            }
        }
    };
    auto write_batch = [&](int base) {
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int idx = base + j * kPatchThreads + tid;
            if (idx >= npix) continue;
            if constexpr (ES == 2) {
                *(uint2 *)(sbytes + (size_t)idx * PB) =
                    make_uint2(__builtin_bit_cast(uint32_t, hv[j][0]), __builtin_bit_cast(uint32_t, hv[j][1]));
            } else {
                *(float4 *)(sbytes + (size_t)idx * PB) = make_float4(v[j][0], v[j][1], v[j][2], v[j][3]);
            }
        }
    };

    // ---- 16-bit input in 16-byte loads (P.vec): item i of a unit is input
    // row hi_base + i / NCK, columns 8*(i % NCK) .. +7, all C_in channels: one
    // load per channel plane (NCHW) or C_in loads of the 8 pixels' channel
    // vectors (NHWC).  Every load is issued, with an offset past x where the
    // row is outside the image (the range check returns zeros), so no load
    // waits behind a branch.  A thread takes items tid and tid + 256.  The
    // stage starts zeroed and its padding columns are never written.
    const int NCK = g.W >> 3;  // 8-column chunks of an input row
    const int nitems = P.RIN * NCK;
    uint4 vb[VS ? 2 : 1][4];
    const __amdgpu_buffer_rsrc_t x_rsrc = make_rsrc(P.x, VS ? P.x_bytes : 0u);
    auto vload = [&](int u) {
        if constexpr (!VS) return;
        const int n = u / P.hgroups;
        const int hi_base = (u - n * P.hgroups) * P.R * g.s - g.p;
#pragma unroll
        for (int k = 0; k < (VS ? 2 : 0); ++k) {
            const int i = tid + k * kPatchThreads;
            const int r = i / NCK, q = i - r * NCK;
            const int hi = hi_base + r;
            const bool in = i < nitems && hi >= 0 && hi < g.H;
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
                uint32_t off = kOutOfRange;
                if (in && ch < g.C)
                    off = NCHW ? (uint32_t)((((n * g.C + ch) * g.H + hi) * g.W + 8 * q) * 2)
                               : (uint32_t)((((n * g.H + hi) * g.W + 8 * q) * g.C) * 2 + 16 * ch);
                vb[k][ch] = ch < g.C ? __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(x_rsrc, off, 0, 0))
                                     : make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };
    // Element e (16-bit) of the 16 bytes d.
    auto h16 = [](const uint4 &d, int e) -> uint32_t {
        const uint32_t w = e < 2 ? d.x : e < 4 ? d.y : e < 6 ? d.z : d.w;
        return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
    };
    auto vwrite = [&]() {
        if constexpr (!VS) return;
#pragma unroll
        for (int k = 0; k < (VS ? 2 : 0); ++k) {
            const int i = tid + k * kPatchThreads;
            if (i >= nitems) continue;
            const int r = i / NCK, q = i - r * NCK;
            char *const row = sbytes + (size_t)r * P.WIN * PB;
            // Pixel j (input column 8q + j, stage column 8q + p + j): its
            // channels 0..3 as two words (zeros past C_in).
            auto put = [&](int j, uint32_t lo, uint32_t hi) {
                const int col = 8 * q + g.p + j;
                if (col < P.WIN) *(uint2 *)(row + (size_t)col * PB) = make_uint2(lo, hi);
            };
            if constexpr (NCHW) {
                // channel ch of the 8 pixels is load ch
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    put(j, h16(vb[k][0], j) | (h16(vb[k][1], j) << 16), h16(vb[k][2], j) | (h16(vb[k][3], j) << 16));
            } else if (g.C == 4) {
                // the 8 pixels' channel vectors are the stage pixels as they are
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint4 &v = vb[k][j >> 1];
                    put(j, (j & 1) ? v.z : v.x, (j & 1) ? v.w : v.y);
                }
            } else {
                // pixel j channel ch is element j*C + ch of the 8*C loaded
                auto unpack = [&](auto cc) {
                    constexpr int CC = decltype(cc)::value;
                    auto el = [&](int j, int ch) -> uint32_t {
                        return ch < CC ? h16(vb[k][(j * CC + ch) / 8], (j * CC + ch) % 8) : 0u;
                    };
#pragma unroll
                    for (int j = 0; j < 8; ++j) put(j, el(j, 0) | (el(j, 1) << 16), el(j, 2) | (el(j, 3) << 16));
                };
                if (g.C == 1) unpack(std::integral_constant<int, 1>{});
                else if (g.C == 2) unpack(std::integral_constant<int, 2>{});
                else unpack(std::integral_constant<int, 3>{});
            }
        }
    };

    if constexpr (VS) {
        for (int i = tid; i < kPatchStageBytes / 16; i += kPatchThreads) stage[i] = make_uint4(0u, 0u, 0u, 0u);
        if (blockIdx.x < (unsigned)P.units) vload(blockIdx.x);
    } else if (blockIdx.x < (unsigned)P.units) {
        load_batch(blockIdx.x, 0);
    }
    for (int u = blockIdx.x; u < P.units; u += gridDim.x) {
        const int n = u / P.hgroups;
        const int ho0 = (u - n * P.hgroups) * P.R;
        const int rows = min(P.R, g.Ho - ho0);

        __syncthreads();  // the previous unit's reads of the stage are done (and the stage zeroed)
        if constexpr (VS) {
            vwrite();
            if (u + (int)gridDim.x < P.units) vload(u + gridDim.x);  // lands while this unit is multiplied
        } else {
            write_batch(0);
            for (int base = kPatchThreads * SB; base < npix; base += kPatchThreads * SB) {
                load_batch(u, base);
                write_batch(base);
            }
            if (u + (int)gridDim.x < P.units) load_batch(u + gridDim.x, 0);  // lands while this unit is multiplied
        }
        __syncthreads();

        // ---- 32-pixel fragments of the unit's output rows.  A wavefront
        // multiplies NF fragments together (two for long K loops: the two
        // independent accumulator chains hide each other's LDS latency, and
        // each weight fragment read serves both), then stores them one by one.
        constexpr int NF = KS >= 8 ? 2 : 1;
        const int nfrag = rows * frags_per_row;
        // The epilogue of fragment f: bias in fp32, one rounding; the
        // wavefront's 32 x 64 tile goes through its own LDS buffer so that it
        // leaves in 16-byte pieces along the output's contiguous axis: for
        // NHWC the 32 pixels' 64-channel runs (one contiguous block when
        // C_out is 64), for NCHW 64 channel rows of 32 pixels.
        auto emit = [&](int f, typename MF::acc_t (&acc)[2]) {
            const int r = f / frags_per_row;
            const int wo0 = (f - r * frags_per_row) * 32;
            const int ho = ho0 + r;
            const int npx = min(32, g.Wo - wo0), nco = min(64, g.Co - cob);
#pragma unroll
            for (int ic = 0; ic < 2; ++ic)
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const int i4 = MF::qrow(q, lane);  // first of the lane's 4 consecutive rows
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[ic][4 * q + e];
                    int off;
                    if constexpr (NCHW) {
                        const float bb = ((const float *)bias_s)[32 * ic + col];
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] += bb;
                        off = (32 * ic + col) * ORS + i4 * ES;
                    } else {
                        const float4 bb = bias_s[(32 * ic + i4) / 4];
                        v[0] += bb.x, v[1] += bb.y, v[2] += bb.z, v[3] += bb.w;
                        off = col * ORS + (32 * ic + i4) * ES;
                    }
                    obuf_put4(ob + off, v[0], v[1], v[2], v[3]);
                }
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the tile is in the buffer
            // The fragment's first output: NCHW (n, cob, ho, wo0), whose
            // channel planes are `plane` apart; NHWC (n, ho, wo0, cob).
            const long long plane = (long long)g.Ho * g.Wo;
            S *const yrow = NCHW ? y + ((long long)n * g.Co + cob) * plane + (long long)ho * g.Wo + wo0
                                 : y + (((long long)n * g.Ho + ho) * g.Wo + wo0) * g.Co + cob;
            if constexpr (NCHW) {
                constexpr int CPR = 32 * ES / 16;  // 16-byte pieces per channel row
                constexpr int EPC = 16 / ES;       // elements per piece
                if (vec_store && npx % EPC == 0) {  // wavefront-uniform: whole pieces only
#pragma unroll
                    for (int i = 0; i < CPR; ++i) {
                        const int c = lane + 64 * i;
                        const int cl = c / CPR, p0 = (c % CPR) * EPC;
                        const uint4 d = *(const uint4 *)(ob + cl * ORS + p0 * ES);
                        if (cl < nco && p0 < npx)
                            *(uint4 *)__builtin_assume_aligned(yrow + (long long)cl * plane + p0, 16) = d;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < CPR; ++i) {
                        const int c = lane + 64 * i;
                        const int cl = c / CPR, p0 = (c % CPR) * EPC;
                        if (cl >= nco) continue;
                        const S *src = (const S *)(ob + cl * ORS + p0 * ES);
                        S *dst = yrow + (long long)cl * plane + p0;
                        for (int e = 0; e < EPC; ++e)
                            if (p0 + e < npx) dst[e] = src[e];
                    }
                }
            } else {
                constexpr int CPP = 64 * ES / 16;  // 16-byte pieces per pixel
                constexpr int EPC = 16 / ES;
                if (vec_store && nco % EPC == 0) {  // wavefront-uniform: whole pieces only
#pragma unroll
                    for (int i = 0; i < 32 * CPP / 64; ++i) {
                        const int c = lane + 64 * i;
                        const int px = c / CPP, c0 = (c % CPP) * EPC;
                        const uint4 d = *(const uint4 *)(ob + px * ORS + c0 * ES);
                        if (px < npx && c0 < nco)
                            *(uint4 *)__builtin_assume_aligned(yrow + px * g.Co + c0, 16) = d;
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 32 * CPP / 64; ++i) {
                        const int c = lane + 64 * i;
                        const int px = c / CPP, c0 = (c % CPP) * EPC;
                        if (px >= npx) continue;
                        const S *src = (const S *)(ob + px * ORS + c0 * ES);
                        S *dst = yrow + px * g.Co + c0;
                        for (int e = 0; e < EPC; ++e)
                            if (c0 + e < nco) dst[e] = src[e];
                    }
                }
            }
        };
        for (int f0 = wave * NF; f0 < nfrag; f0 += NF * (kPatchThreads / 64)) {
            int pbase[NF];
#pragma unroll
            for (int j = 0; j < NF; ++j) {
                const int f = min(f0 + j, nfrag - 1);  // past the last fragment: a repeated one, not stored
                const int r = f / frags_per_row;
                const int wo0 = (f - r * frags_per_row) * 32;
                const int wo = min(wo0 + col, g.Wo - 1);  // past the row's end: a repeated pixel, not stored
                pbase[j] = (r * g.s * P.WIN + wo * g.s) * PB;
            }
            typename MF::acc_t acc[NF][2];
#pragma unroll
            for (int j = 0; j < NF; ++j) acc[j][0] = acc[j][1] = typename MF::acc_t{};
            // Every K step up to the capacity KS, with no test against the
            // layer's own count: past it the weights are zeros and every tap
            // reads as zero, so those MFMAs add exact zeros, and the loop
            // stays one straight block for the accumulators.  A tap past the
            // last reads the 16 zero bytes at zb (an address select, not a
            // branch), and each K step's fragments are read from LDS while
            // the previous step's MFMAs run.
            auto frags = [&](int ks, uint4 (&a)[NF], uint4 (&b)[2]) {
                const uint32_t o0 = toff[ks] & 0xFFFFu;
#pragma unroll
                for (int j = 0; j < NF; ++j) {
                    const char *p0 = o0 != 0xFFFFu ? sbytes + pbase[j] + o0 : zb;
                    if constexpr (ES == 2) {
                        const uint32_t o1 = toff[ks] >> 16;
                        const char *p1 = o1 != 0xFFFFu ? sbytes + pbase[j] + o1 : zb;
                        const uint2 lo = *(const uint2 *)p0, hi = *(const uint2 *)p1;
                        a[j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
                    } else {
                        a[j] = *(const uint4 *)p0;
                    }
                }
#pragma unroll
                for (int ic = 0; ic < 2; ++ic) b[ic] = wlds[(ks * 2 + ic) * 64 + lane];
            };
            uint4 fa[2][NF], fb[2][2];
            frags(0, fa[0], fb[0]);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int c = ks & 1;
                if (ks + 1 < KS) frags(ks + 1, fa[c ^ 1], fb[c ^ 1]);
#pragma unroll
                for (int ic = 0; ic < 2; ++ic)
#pragma unroll
                    for (int j = 0; j < NF; ++j) {
                        if constexpr (NCHW)
                            MF::mma(fa[c][j], fb[c][ic], acc[j][ic]);  // rows: pixels, columns: channels
                        else
                            MF::mma(fb[c][ic], fa[c][j], acc[j][ic]);  // rows: channels, columns: pixels
                    }
            }
#pragma unroll
            for (int j = 0; j < NF; ++j)
                if (f0 + j < nfrag) emit(f0 + j, acc[j]);
        }
    }
}

}  // namespace

// Plan for one layer: output rows per unit so that the staged rows fit
// kPatchStageBytes, or false when the layer is outside this kernel.
bool patch_conv_plan(const Geom &g, int dtype, int *R_out) {
    const int ES = dtype == CONV_DTYPE_FP32 ? 4 : 2;
    const int TPS = dtype == CONV_DTYPE_FP32 ? 2 : 4;
    if (g.C > 4) return false;
    if ((g.KH * g.KW + TPS - 1) / TPS > kPatchMaxKSteps) return false;
    const long long WIN = (long long)(g.Wo - 1) * g.s + (long long)(g.KW - 1) * g.d + 1;
    int R = 0;
    for (int r = 1; r <= 8 && r <= g.Ho; ++r) {
        const long long RIN = (long long)(r - 1) * g.s + (long long)(g.KH - 1) * g.d + 1;
        if (RIN * WIN * 4 * ES <= kPatchStageBytes) R = r;
    }
    if (R == 0) return false;
    if (R_out) *R_out = R;
    return true;
}

hipError_t launch_patch_conv(const void *x, const void *w, const void *bias, void *y, const Geom &g, bool nhwc,
                             int dtype, hipStream_t st) {
    int R = 0;
    if (!patch_conv_plan(g, dtype, &R)) return hipErrorInvalidValue;
    PatchArgs P;
    P.x = x; P.w = w; P.bias = bias; P.y = y; P.g = g;
    P.R = R;
    P.RIN = (R - 1) * g.s + (g.KH - 1) * g.d + 1;
    P.WIN = (g.Wo - 1) * g.s + (g.KW - 1) * g.d + 1;
    P.hgroups = (g.Ho + R - 1) / R;
    P.units = g.N * P.hgroups;
    const int TPS = dtype == CONV_DTYPE_FP32 ? 2 : 4;
    P.ksteps = (g.KH * g.KW + TPS - 1) / TPS;
    const long long x_bytes = (long long)g.N * g.C * g.H * g.W * (dtype == CONV_DTYPE_FP32 ? 4 : 2);
    P.vec = dtype != CONV_DTYPE_FP32 && g.W % 8 == 0 && (uintptr_t)x % 16 == 0 && x_bytes < (1LL << 31) - 16 &&
            (long long)P.RIN * (g.W / 8) <= 2LL * kPatchThreads;
    P.x_bytes = P.vec ? (unsigned)x_bytes : 0u;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return hipErrorInvalidValue;
    const int ntn = (g.Co + 63) / 64;
    // The resident blocks of all compute units, spread over the channel tiles.
    const int ks_cap = P.ksteps <= 3 ? 3 : P.ksteps <= 4 ? 4 : P.ksteps <= 8 ? 8 : P.ksteps <= 13 ? 13 : 16;
    const int per_cu = patch_blocks_per_cu(ks_cap, dtype == CONV_DTYPE_FP32 ? 4 : 2, !nhwc);
    const int per_tile = max(1, min(P.units, (per_cu * cus + ntn - 1) / ntn));
    const dim3 grid((unsigned)per_tile, (unsigned)ntn);
    auto launch = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(kPatchThreads), 0, st, P); };
    auto by_ks = [&](auto k3, auto k4, auto k8, auto k13, auto k16) {
        if (P.ksteps <= 3) launch(k3);  // 3x3 kernels in 16-bit types
        else if (P.ksteps <= 4) launch(k4);
        else if (P.ksteps <= 8) launch(k8);
        else if (P.ksteps <= 13) launch(k13);  // 7x7 kernels in 16-bit types
        else launch(k16);
    };
    if (dtype == CONV_DTYPE_FP32) {
        if (nhwc) by_ks(patch_conv_kernel<float, false, 3>, patch_conv_kernel<float, false, 4>, patch_conv_kernel<float, false, 8>, patch_conv_kernel<float, false, 13>, patch_conv_kernel<float, false, 16>);
        else by_ks(patch_conv_kernel<float, true, 3>, patch_conv_kernel<float, true, 4>, patch_conv_kernel<float, true, 8>, patch_conv_kernel<float, true, 13>, patch_conv_kernel<float, true, 16>);
    } else {
        // 16-bit types: the two staging forms, each layout.
        auto by_form = [&](auto s_tag) {
            using T = decltype(s_tag);
            if (P.vec) {
                if (nhwc) by_ks(patch_conv_kernel<T, false, 3, true>, patch_conv_kernel<T, false, 4, true>, patch_conv_kernel<T, false, 8, true>, patch_conv_kernel<T, false, 13, true>, patch_conv_kernel<T, false, 16, true>);
                else by_ks(patch_conv_kernel<T, true, 3, true>, patch_conv_kernel<T, true, 4, true>, patch_conv_kernel<T, true, 8, true>, patch_conv_kernel<T, true, 13, true>, patch_conv_kernel<T, true, 16, true>);
            } else {
                if (nhwc) by_ks(patch_conv_kernel<T, false, 3>, patch_conv_kernel<T, false, 4>, patch_conv_kernel<T, false, 8>, patch_conv_kernel<T, false, 13>, patch_conv_kernel<T, false, 16>);
                else by_ks(patch_conv_kernel<T, true, 3>, patch_conv_kernel<T, true, 4>, patch_conv_kernel<T, true, 8>, patch_conv_kernel<T, true, 13>, patch_conv_kernel<T, true, 16>);
            }
        };
        if (dtype == CONV_DTYPE_FP16) by_form(_Float16());
        else by_form(uint16_t());
    }
    return hipGetLastError();
}

}  // namespace convlower
