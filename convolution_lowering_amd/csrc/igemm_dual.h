// The main loop with two or more wavefronts on every SIMD, so that while one
// waits (at its barrier, for its loads, in its prologue or epilogue) or
// issues its address arithmetic, another keeps the matrix core busy.  Four
// shapes (DualCfg instances below):
//
//   * DualCfg4: two blocks per compute unit, each 256 threads with 80 KB of
//     LDS; K tiles of 64-byte rows (32 bf16 / 16 fp32 values); wavefront
//     tiles 128 x 64; block tile 256 x 128.
//   * DualCfg8: one block of 512 threads per compute unit with 150 KB of
//     LDS; K tiles of 128-byte rows (64 bf16 / 32 fp32 values), so every
//     load moves whole cache lines; wavefront tiles 64 x 64.
//   * QuadCfg: four 256-thread blocks of 128 x 64 per compute unit, for at
//     most 64 output channels.
//   * DualCfg8Sq: one 512-thread block of 256 x 256, wavefront tiles 128 x 64.
//
// Common structure:
//   * v_mfma_f32_32x32x16_bf16 or v_mfma_f32_32x32x2_f32 tiles of Y_col.
//   * Three LDS stages filled by the buffer-load-to-LDS instructions; tile
//     k+3 is issued while tile k is multiplied, so two tiles cover the load
//     latency.
//   * Every K tile lies inside one tap (the host asks C to be a multiple of
//     the K tile), so a tile's loads share one tap and one channel offset --
//     except in the padded-channel feeds, where each 16-byte chunk of a tile
//     is addressed on its own.
//     The tiles are visited tap-fastest: all KH*KW taps of one channel
//     slice, then the next slice.  Consecutive tiles then read the same input
//     rows shifted by one tap, which the L2 still holds; (kh, kw, ci) order
//     would come back to a row only after streaming C / (K tile) tiles of
//     every resident block through the L2.  A and B walk the same order, so
//     the sum is unchanged.
//   * The indirection buffer's slice for the block (BM rows x KH*KW taps)
//     is copied to LDS once, as 16-bit pixel indices (entry / C, 0xFFFF for
//     a padding tap).  The indices a tile's loads need are read one tile
//     ahead.
//   * The bias of the block's BN output channels is staged in LDS.
//
// All LDS-refill and read ordering follows the pipeline of igemm_dma.h: each
// wavefront waits (vmcnt) for its own loads of the tile it is about to read
// and (lgkmcnt) for its own reads of the stage about to be refilled, then
// the block barrier makes both hold for all wavefronts.
#pragma once

#include <type_traits>

namespace convlower {

constexpr int kDualMaxTaps = 12;  // KH*KW taps the LDS slice of the indirection buffer holds
// ... and in the 128-row block of the padded-channel indirection feed (5x5
// kernels over few channels), where the larger slice costs 8 KB of LDS.
constexpr int kQuadChunkMaxTaps = 32;

// Shape of one main-loop variant: block tile BM x BN, KCH 16-byte chunks
// per stage row, NW wavefronts in a WGM x (NW / WGM) grid.
template <typename S, int KCH_, int NW_, int WGM_, int BM_ = 256, int BN_ = 128>
struct DualCfg {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int ES = (int)sizeof(S);
    static constexpr int VEC = 16 / ES;
    static constexpr int KCH = KCH_;                 // 16-byte chunks per stage row
    static constexpr int NW = NW_, NTHR = 64 * NW_;  // wavefronts, threads
    static constexpr int RPI = 64 / KCH;             // stage rows one 64-lane load fills
    static constexpr int RPL = 16 / KCH;             // stage rows per 256-byte LDS line
    static constexpr int BK = KCH * VEC;             // K values per tile
    static constexpr int NSLOT = (BM + BN) * KCH;    // 16-byte slots per stage
    static constexpr int IPW_A = BM * KCH / 64 / NW;  // A loads per wavefront per tile
    static constexpr int IPW_B = BN * KCH / 64 / NW;  // B loads per wavefront per tile
    static constexpr int IPW = IPW_A + IPW_B;
    static constexpr int WGM = WGM_, WGN = NW_ / WGM_;
    static constexpr int WPM = BM / WGM, WCN = BN / WGN;  // wavefront tile
    static constexpr int MT = 32, TP = WPM / MT, TC = WCN / MT;
    static constexpr int NG = KCH / 2;  // MFMA K steps per tile (two chunks per step)
    static constexpr long long STAGE_BYTES = 3LL * NSLOT * 16;  // the three stages, reused by the epilogue

    static_assert(IPW_A * NW * 64 == BM * KCH && IPW_B * NW * 64 == BN * KCH, "loads must split evenly");
    static_assert(TP >= 1 && TC >= 1 && WGM * WGN == NW, "wavefront grid");
};
// 64-byte rows, four wavefronts of 128 x 64, two blocks per compute unit
// (80 KB of LDS each).
template <typename S>
using DualCfg4 = DualCfg<S, 4, 4, 2>;
// 128-byte rows, eight wavefronts of 64 x 64, one block per compute unit
// (150 KB of LDS): whole-cache-line loads, two wavefronts per SIMD.
template <typename S>
using DualCfg8 = DualCfg<S, 8, 8, 4>;
// Block tile 128 x 64 for layers with at most 64 output channels: four
// wavefronts of 32 x 64 stacked along the pixels, four blocks per compute
// unit (40 KB of LDS each).  With few K tiles per block (small C), four
// blocks hide each other's prologues, pipeline fills and epilogues better
// than two blocks of twice the size.
template <typename S>
using QuadCfg = DualCfg<S, 4, 4, 4, 128, 64>;
// Eight wavefronts of 128 x 64 (two per SIMD), one block per compute unit,
// 64-byte rows, block tile 256 x 256 (wavefront grid 2 x 4, 103 KB of LDS):
// it loads 32 bytes per MFMA cycle of the compute unit, against 48 for
// 256 x 128.
template <typename S>
using DualCfg8Sq = DualCfg<S, 4, 8, 2, 256, 256>;

// Stage slot of chunk c of row r (rows of KCH chunks).  A b128 LDS read is
// served 16 lanes per cycle from one 256-byte line of banks; XOR-ing the
// chunk with (r / rows-per-line) mod KCH puts any 16 consecutive rows of one
// chunk column on 16 distinct 16-byte bank groups.
template <int KCH>
__device__ __forceinline__ constexpr int dual_swz(int r) {
    return (r / (16 / KCH)) & (KCH - 1);
}
template <int KCH>
__device__ __forceinline__ constexpr int dual_slot(int r, int c) {
    return r * KCH + (c ^ dual_swz<KCH>(r));
}

// The epilogue shared by the main loops of this file: the block's fp32
// accumulators (wavefront (wp, wc) of the block's WGM x WGN grid) leave as
// split-K partials, or, bias added and rounded once, through the LDS stage
// memory `stg` (C::STAGE_BYTES bytes, free once every wavefront has passed
// the first barrier below) as whole rows of the output.
template <typename S, bool OUT_NCHW, typename C>
__device__ __forceinline__ void dual_store(const GemmArgs &A,
                                           typename MfmaShape<S, 32>::acc_t (&acc)[C::TP][C::TC], uint4 *stg,
                                           const float *bias_s, uint32_t m0, int co0, int wp, int wc, int lane,
                                           int tid) {
    // S is the output type (the input type too, except for 8-bit inputs).
    constexpr int BM = C::BM, BN = C::BN, VEC = 16 / (int)sizeof(S), TP = C::TP, TC = C::TC, WPM = C::WPM,
                  WCN = C::WCN;
    constexpr int NTHR = C::NTHR;
    using MF = MfmaShape<S, 32>;
    constexpr int NQ = MF::NQ;
    const Geom &g = A.g;
    const int frow = lane & 31;
    // ---- epilogue -------------------------------------------------------------
    S *y = (S *)A.y;
    if (A.part) {
        // Split K: this split's fp32 sums go to its slice of the workspace;
        // the reduce pass adds the bias and rounds.
#pragma unroll
        for (int ip = 0; ip < TP; ++ip)
#pragma unroll
            for (int ic = 0; ic < TC; ++ic)
#pragma unroll
                for (int q = 0; q < NQ; ++q)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int pr = wp * WPM + ip * 32, cr = wc * WCN + ic * 32;
                        const int ml = OUT_NCHW ? pr + MF::qrow(q, lane) + v : pr + frow;
                        const int cl = OUT_NCHW ? cr + frow : cr + MF::qrow(q, lane) + v;
                        const long long m = (long long)m0 + ml;
                        const int co = co0 + cl;
                        if (m < g.M && co < g.Co)
                            A.part[((long long)blockIdx.z * g.M + m) * g.Co + co] = acc[ip][ic][4 * q + v];
                    }
        return;
    }
    // The tile goes through LDS (the stage memory, free once every wavefront
    // has passed the barrier below) so that it leaves as whole rows along the
    // output's contiguous axis: [channel][pixel] for NCHW, [pixel][channel]
    // for NHWC, each row padded by 16 bytes to spread the bank groups.  A
    // tile larger than the stage memory (fp32 with 80 KB blocks) goes in two
    // passes over halves of its rows.
    constexpr int ROWS = OUT_NCHW ? BN : BM;  // output runs in the tile
    constexpr int COLS = OUT_NCHW ? BM : BN;  // elements per run
    constexpr int PADE = 16 / (int)sizeof(S);
    constexpr int RSTR = COLS + PADE;  // LDS row stride, elements
    constexpr long long TILE_BYTES = (long long)ROWS * RSTR * (int)sizeof(S);
    constexpr int NPASS = TILE_BYTES <= C::STAGE_BYTES       ? 1
                          : TILE_BYTES <= 2 * C::STAGE_BYTES ? 2
                                                               : 4;
    constexpr int PROWS = ROWS / NPASS;
    constexpr int CPR = COLS / VEC;  // 16-byte chunks per run
    static_assert((long long)PROWS * RSTR * (int)sizeof(S) <= C::STAGE_BYTES, "epilogue tile fits the stages");
    static_assert(NTHR % CPR == 0, "each thread keeps one chunk column");
    S *tile = (S *)stg;

    // This thread's chunk column and, for NCHW, the output pixel it starts
    // at (the same for every run it stores).
    const int cc = tid % CPR;
    int n0 = 0, p0 = 0;
    bool fast = false;  // whole 16-byte chunk inside one image, aligned
    int sub = 1;        // NCHW: widest piece (elements) that never crosses an image
    if constexpr (OUT_NCHW) {
        const uint32_t m = m0 + (uint32_t)(cc * VEC);  // M < 2^31
        n0 = (int)(m / (uint32_t)g.P);
        p0 = (int)(m - (uint32_t)n0 * (uint32_t)g.P);
        if ((uintptr_t)y % 16 == 0) {
            sub = VEC;
            while (g.P % sub != 0) sub >>= 1;
        }
        fast = sub == VEC && (long long)m + VEC <= g.M;
    } else {
        fast = g.Co % VEC == 0 && co0 + cc * VEC + VEC <= g.Co && ((uintptr_t)y % 16) == 0;
    }

#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
        __syncthreads();  // stages (or the previous pass's rows) no longer read
        const int r_lo = pass * PROWS;
        // Accumulators -> LDS, bias added in fp32, rounded once.
#pragma unroll
        for (int ip = 0; ip < TP; ++ip)
#pragma unroll
            for (int ic = 0; ic < TC; ++ic)
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const int pr = wp * WPM + ip * 32, cr = wc * WCN + ic * 32;
                    const float a0 = acc[ip][ic][4 * q], a1 = acc[ip][ic][4 * q + 1];
                    const float a2 = acc[ip][ic][4 * q + 2], a3 = acc[ip][ic][4 * q + 3];
                    if constexpr (OUT_NCHW) {
                        const int row = cr + frow, col = pr + MF::qrow(q, lane);
                        if (row < r_lo || row >= r_lo + PROWS) continue;
                        const float b = bias_s[row];
                        store4(tile + (row - r_lo) * RSTR + col, a0 + b, a1 + b, a2 + b, a3 + b);
                    } else {
                        const int row = pr + frow, col = cr + MF::qrow(q, lane);
                        if (row < r_lo || row >= r_lo + PROWS) continue;
                        store4(tile + (row - r_lo) * RSTR + col, a0 + bias_s[col], a1 + bias_s[col + 1],
                               a2 + bias_s[col + 2], a3 + bias_s[col + 3]);
                    }
                }
        __syncthreads();
        // LDS -> global, one 16-byte chunk per thread per run.  Where every
        // chunk of this thread is whole and aligned (the common case), all of
        // its LDS reads are issued before its stores, so their latencies
        // overlap; otherwise the general loop below.
        constexpr int RSTEP = NTHR / CPR;  // runs per sweep of the block
        constexpr int ITER = PROWS / RSTEP;
        static_assert(PROWS % RSTEP == 0, "runs split evenly over the threads");
        if (fast) {
            uint4 vals[ITER];
#pragma unroll
            for (int i = 0; i < ITER; ++i)
                vals[i] = *(const uint4 *)(tile + (tid / CPR + i * RSTEP) * RSTR + cc * VEC);
#pragma unroll
            for (int i = 0; i < ITER; ++i) {
                const int row = r_lo + tid / CPR + i * RSTEP;
                if constexpr (OUT_NCHW) {
                    const int co = co0 + row;
                    if (co < g.Co) *(uint4 *)(y + ((long long)n0 * g.Co + co) * g.P + p0) = vals[i];
                } else {
                    const long long m = (long long)m0 + row;
                    if (m < g.M) *(uint4 *)(y + m * g.Co + co0 + cc * VEC) = vals[i];
                }
            }
            continue;  // next pass
        }
        for (int r = tid / CPR; r < PROWS; r += NTHR / CPR) {
            const int row = r_lo + r;
            const uint4 val = *(const uint4 *)(tile + r * RSTR + cc * VEC);
            if constexpr (OUT_NCHW) {
                const int co = co0 + row;
                if (co >= g.Co) continue;
                if (fast) {
                    *(uint4 *)(y + ((long long)n0 * g.Co + co) * g.P + p0) = val;
                } else {
                    // Pieces of `sub` elements: P and the chunk start are
                    // multiples of sub, so no piece crosses an image and each
                    // is aligned to its size.
                    S e[VEC];
                    __builtin_memcpy(e, &val, 16);
                    const long long m = (long long)m0 + cc * VEC;
                    auto pieces = [&](auto sub_c) {
                        constexpr int SUB = decltype(sub_c)::value;
                        int n = n0, p = p0;
#pragma unroll
                        for (int v = 0; v < VEC; v += SUB) {
                            S *dst = y + ((long long)n * g.Co + co) * g.P + p;
                            if constexpr (SUB * sizeof(S) == 8) {
                                if (m + v + SUB <= g.M) {
                                    *(uint2 *)dst = make_uint2(*(const uint32_t *)&e[v], *(const uint32_t *)&e[v + SUB / 2]);
                                    goto next;
                                }
                            } else if constexpr (SUB * sizeof(S) == 4) {
                                if (m + v + SUB <= g.M) {
                                    *(uint32_t *)dst = *(const uint32_t *)&e[v];
                                    goto next;
                                }
                            }
#pragma unroll
                            for (int u = 0; u < SUB; ++u)
                                if (m + v + u < g.M) dst[u] = e[v + u];
                        next:
                            p += SUB;
                            if (p == g.P) {
                                p = 0;
                                ++n;
                            }
                        }
                    };
                    if (sub == VEC / 2)
                        pieces(std::integral_constant<int, VEC / 2>{});
                    else if (sub == 2 && VEC >= 4)
                        pieces(std::integral_constant<int, (VEC >= 4 ? 2 : 1)>{});
                    else
                        pieces(std::integral_constant<int, 1>{});
                }
            } else {
                const long long m = (long long)m0 + row;
                if (m >= g.M) continue;
                const int co = co0 + cc * VEC;
                if (fast) {
                    *(uint4 *)(y + m * g.Co + co) = val;
                } else {
                    S e[VEC];
                    __builtin_memcpy(e, &val, 16);
#pragma unroll
                    for (int v = 0; v < VEC; ++v)
                        if (co + v < g.Co) y[m * g.Co + co + v] = e[v];
                }
            }
        }
    }
}

template <typename S, int FEED, bool OUT_NCHW, typename C>
__device__ __forceinline__ void igemm_dual_body(const GemmArgs &A) {
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, VEC = C::VEC, KCH = C::KCH, NSLOT = C::NSLOT;
    constexpr int IPW_A = C::IPW_A, IPW_B = C::IPW_B, IPW = C::IPW;
    constexpr int WPM = C::WPM, WCN = C::WCN, TP = C::TP, TC = C::TC, NG = C::NG;
    constexpr int NW = C::NW, NTHR = C::NTHR, RPI = C::RPI;
    constexpr uint32_t ES = (uint32_t)sizeof(S);
    constexpr bool WCHUNK = FEED == FEED_WIN_CHUNK;
    constexpr bool CHUNK = FEED == FEED_IND_CHUNK || WCHUNK;  // each 16-byte chunk its own (tap, channels)
    constexpr bool IND = FEED == FEED_IND_NHWC || FEED == FEED_IND_CHUNK;
    constexpr bool TAPS = FEED == FEED_IND_NHWC || FEED == FEED_WIN;  // K tiles inside one tap
    // 1x1 NCHW read in place: the A part of a stage is the tile's BK channel
    // rows of BM pixels as they lie in x ([channel][pixel], CPRA chunks of
    // VEC pixels per row, RPIA rows per 64-lane load), chunk columns
    // XOR-ed by 4 * (row mod 4).  Each MFMA A fragment (32 pixels x 16
    // channels) is two transpose reads of 4 channels x 16 pixels per
    // 16-lane group; the XOR puts the 16 chunks a 32-lane half of such a
    // read touches (4 rows x 4 chunks) on 16 distinct bank groups.
    constexpr bool GN = FEED == FEED_GEMM_NCHW;
    static_assert(!GN || sizeof(S) == 2, "the transpose reads move 16-bit elements");
    constexpr int CPRA = GN ? BM / VEC : 1;
    constexpr int RPIA = GN ? 64 / CPRA : 1;
    static_assert(!GN || (CPRA >= 16 && CPRA <= 64 && BK * CPRA == BM * KCH && (NW * RPIA) % 4 == 0),
                  "A rows of whole 64-byte groups; each lane's swizzle the same in all its loads");
    using MF = MfmaShape<S, 32>;
    constexpr int NQ = MF::NQ;

    __shared__ uint4 stg[3][NSLOT];  // the three stages; the epilogue reuses them
    uint4 *const st0 = stg[0], *const st1 = stg[1], *const st2 = stg[2];
    constexpr int MAXT = FEED == FEED_IND_CHUNK && BM == 128 ? kQuadChunkMaxTaps : kDualMaxTaps;
    __shared__ uint16_t ibs[IND ? BM * MAXT : 2];
    static_assert((BM * MAXT) % NTHR == 0, "slice must split evenly");
    __shared__ float bias_s[BN];

    const Geom &g = A.g;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    int mt, nt;
    tile_coords((int)((g.M + BM - 1) / BM), (g.Co + BN - 1) / BN, mt, nt);
    const uint32_t M = (uint32_t)g.M;
    const uint32_t m0 = (uint32_t)mt * BM;
    const int co0 = nt * BN;
    const int kbeg = blockIdx.z * A.k_per_split;
    const int kend = (int)min((long long)kbeg + A.k_per_split, g.K);
    const int nk = (kend - kbeg + BK - 1) / BK;

    // ---- prologue: indirection slice and bias to LDS ------------------------
    // Element e of the slice is tap e % T of tile row e / T, i.e. entry
    // ((m0 + e / T) mod P) * T + e % T = (m0 mod P) * T + e (mod P*T) of the
    // buffer: consecutive threads read consecutive entries.  Rows past M
    // read some valid entry; their loads are out of range anyway.
    if constexpr (IND) {
        const uint32_t PT = (uint32_t)g.P * (uint32_t)g.T;
        constexpr int NJ = BM * MAXT / NTHR;
        const int nent = BM * g.T;
        uint32_t idx = ((m0 % (uint32_t)g.P) * (uint32_t)g.T + (uint32_t)tid) % PT;
        int v[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            v[j] = 0;
            if (j * NTHR < nent) v[j] = A.ibuf[idx];  // (entries past the slice read a valid one)
            idx += NTHR;
            if (idx >= PT) idx -= PT;
            if (idx >= PT) idx %= PT;
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            if (j * NTHR + tid < nent)
                ibs[tid + NTHR * j] =
                    v[j] < 0 ? (uint16_t)0xFFFF : (uint16_t)(((uint32_t)v[j] >> A.c_shift) * A.c_inv);
    }
    if (tid < BN) {
        const int co = co0 + tid;
        float b = 0.f;
        if (A.bias && co < g.Co) b = bits_to_f32(S(), elem_bits((const S *)A.bias, co));
        bias_s[tid] = b;
    }

    // ---- per-lane load geometry ---------------------------------------------
    // Load i of this wavefront covers stage rows (i*NW + wave)*RPI .. +RPI-1
    // (A rows for i < IPW_A, B rows after); lane L fills slot L of it, i.e.
    // row L/KCH, chunk (L%KCH) ^ swz(row).  swz(row) does not depend on i,
    // so each lane always fetches the same chunk column kc.
    const int lrow = lane / KCH;
    const uint32_t kc = (uint32_t)(((lane % KCH) ^ dual_swz<KCH>(wave * RPI + lrow)) * VEC);
    uint32_t rbA[IPW_A], rbB[IPW_B];
    int ib_row[IPW_A];
    if constexpr (GN) {
        // Slot L of A load i: channel row (i*NW + wave)*RPIA + L/CPRA of the
        // tile, chunk column (L % CPRA) ^ swizzle, i.e. pixels m0 + 8*column;
        // rows of pixels past M read zeros.  P is a multiple of VEC, so no
        // chunk crosses an image.
        const int lr = lane / CPRA;
        const int col = (lane % CPRA) ^ (4 * ((wave * RPIA + lr) & 3));
        const uint32_t m = m0 + (uint32_t)(col * VEC);
        const uint32_t n = m / (uint32_t)g.P;
        const uint32_t pix = n * (uint32_t)g.C * (uint32_t)g.P + (m - n * (uint32_t)g.P);
#pragma unroll
        for (int i = 0; i < IPW_A; ++i) {
            const uint32_t k = (uint32_t)((i * NW + wave) * RPIA + lr);
            rbA[i] = m < M ? (pix + k * (uint32_t)g.P) * ES : kOutOfRange;
            ib_row[i] = 0;
        }
    }
#pragma unroll
    for (int i = 0; i < (GN ? 0 : IPW_A); ++i) {
        const int r = (i * NW + wave) * RPI + lrow;
        ib_row[i] = r * g.T;
        const uint32_t m = m0 + (uint32_t)r;
        const bool ok = m < M;
        const uint32_t mm = ok ? m : 0u;
        const uint32_t n = mm / (uint32_t)g.P;
        uint32_t base;
        if constexpr (FEED == FEED_ROWMAJOR) {
            base = mm * (uint32_t)g.K;
        } else if constexpr (IND) {
            base = n * ((uint32_t)g.H * (uint32_t)g.W * (uint32_t)g.C);
        } else {  // the window-ordered feeds
            const uint32_t p = mm - n * (uint32_t)g.P;
            const uint32_t ho = p / (uint32_t)g.Wo, wo = p - ho * (uint32_t)g.Wo;
            base = ((n * (uint32_t)g.Ho + ho) * (uint32_t)g.Wwin + wo * (uint32_t)g.s) * (uint32_t)(g.KH * g.C);
        }
        rbA[i] = ok ? base * ES : kOutOfRange;
    }
#pragma unroll
    for (int j = 0; j < IPW_B; ++j) {
        const int co = co0 + (j * NW + wave) * RPI + lrow;
        rbB[j] = co < g.Co ? (uint32_t)co * (uint32_t)g.K * ES : kOutOfRange;
    }

    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A.a_src, A.a_bytes);
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(A.b, A.b_bytes);
    const uint32_t lds_w = (uint32_t)wave * 1024u;  // this wavefront's first slot group, in bytes

    // Tap and channel offset of the K tiles (tile j of the whole K range is
    // tap j % T of channel slice j / T), advanced one tile at a time: `iss`
    // for the next tile to issue, `pre` for the tile whose pixel indices are
    // read next (one ahead of `iss`).  Past the last tile the channel offset
    // runs beyond C; those tiles load nothing.
    int iss_t = 0, iss_ci = 0, pre_t = 0, pre_ci = 0;
    if constexpr (TAPS) {
        const int j0 = kbeg / BK;
        iss_t = j0 % g.T;
        iss_ci = (j0 / g.T) * BK;
        pre_t = iss_t;
        pre_ci = iss_ci;
    }
    auto advance = [&](int &t, int &ci) {
        if (++t == g.T) {
            t = 0;
            ci += BK;
        }
    };
    // Chunk-granular K (C a multiple of VEC, padded): K chunk q is channels
    // (q mod C/VEC)*VEC .. +VEC-1 of tap q / (C/VEC), so each chunk of a K
    // tile has its own tap.  Tile j holds chunks j*KCH .. j*KCH + KCH-1 and
    // this lane's column is chunk (tile's first chunk) + ccol; `pre_t` counts
    // chunks here.
    const int ccol = (int)(kc / VEC);
    const uint32_t cpt = (uint32_t)g.C / VEC;  // chunks per tap
    if constexpr (CHUNK) pre_t = kbeg / VEC;

    // Pixel indices (entry / C) of this lane's A rows for the tile at `pre`
    // (0xFFFF where the tap is padding or, chunk-granular, past the last) and,
    // chunk-granular, the channel offset `pch` of this lane's chunk.  From the
    // window-ordered tensor: the offset of this lane's chunk within a row,
    // (kw*d*KH + kh)*C + channels, the same for all its rows (~0 past the
    // last tap).
    uint32_t pix[IPW_A];
    uint32_t wtap = 0, pch = 0;
    auto read_pix = [&]() {
        if constexpr (CHUNK) {
            const uint32_t q = (uint32_t)(pre_t + ccol);
            const uint32_t t = q / cpt;
            const uint32_t ch = (q - t * cpt) * VEC;
            const bool in = t < (uint32_t)g.T;
            if constexpr (WCHUNK) {
                const uint32_t kh = t / (uint32_t)g.KW, kw = t - kh * (uint32_t)g.KW;
                wtap = in ? (kw * (uint32_t)(g.d * g.KH) + kh) * (uint32_t)g.C + ch : ~0u;
            } else {
#pragma unroll
                for (int i = 0; i < IPW_A; ++i) pix[i] = in ? (uint32_t)ibs[ib_row[i] + t] : 0xFFFFu;
                pch = ch;
            }
            pre_t += KCH;
        } else if constexpr (IND) {
#pragma unroll
            for (int i = 0; i < IPW_A; ++i) pix[i] = ibs[ib_row[i] + pre_t];
        }
        if constexpr (TAPS) advance(pre_t, pre_ci);
    };

    // Issue the loads of K tile kt (block-relative) into stage st.
    auto issue = [&](int kt, uint4 *st) {
        const bool live = kt < nk;
        const uint32_t k0 = (uint32_t)(kbeg + kt * BK);
        const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)st + lds_w;
        uint32_t voff[IPW];
        uint32_t ua = 0;  // this tile's offset within an A row, less kc
        if constexpr (FEED == FEED_WIN) {
            const int kh = iss_t / g.KW, kw = iss_t - kh * g.KW;
            ua = (uint32_t)((kw * g.d * g.KH + kh) * g.C + iss_ci);
        }
#pragma unroll
        for (int i = 0; i < IPW_A; ++i) {
            uint32_t o;
            bool valid;
            if constexpr (FEED == FEED_ROWMAJOR) {
                o = rbA[i] + (k0 + kc) * ES;
                valid = k0 + kc < (uint32_t)kend;
            } else if constexpr (GN) {  // channels k0 + row of this lane's pixels
                o = rbA[i] + k0 * (uint32_t)g.P * ES;
                valid = k0 < (uint32_t)kend && rbA[i] != kOutOfRange;
            } else if constexpr (WCHUNK) {  // this lane's chunk of the window cell
                o = rbA[i] + wtap * ES;
                valid = live && wtap != ~0u;
            } else if constexpr (CHUNK) {  // this lane's chunk of the pixel's channels
                o = rbA[i] + (pix[i] * (uint32_t)g.C + pch) * ES;
                valid = live && pix[i] != 0xFFFFu;
            } else if constexpr (FEED == FEED_IND_NHWC) {
                o = rbA[i] + (pix[i] * (uint32_t)g.C + (uint32_t)iss_ci + kc) * ES;
                valid = live && pix[i] != 0xFFFFu;
            } else {
                o = rbA[i] + (ua + kc) * ES;
                valid = live;
            }
            voff[i] = valid ? o : kOutOfRange;
        }
#pragma unroll
        for (int j = 0; j < IPW_B; ++j) {
            if constexpr (TAPS) {  // W_row column t*C + ci of the same tile
                const uint32_t o = rbB[j] + ((uint32_t)(iss_t * g.C + iss_ci) + kc) * ES;
                voff[IPW_A + j] = live ? o : kOutOfRange;
            } else {
                const uint32_t o = rbB[j] + (k0 + kc) * ES;
                voff[IPW_A + j] = k0 + kc < (uint32_t)kend ? o : kOutOfRange;
            }
        }
#pragma unroll
        for (int i = 0; i < IPW_A; ++i) lds_dma16(a_rsrc, voff[i], lds0 + (uint32_t)(i * NW * 1024));
#pragma unroll
        for (int j = 0; j < IPW_B; ++j)
            lds_dma16(b_rsrc, voff[IPW_A + j], lds0 + (uint32_t)(BM * KCH * 16 + j * NW * 1024));
        if constexpr (TAPS) advance(iss_t, iss_ci);
    };

    typename MF::acc_t acc[TP][TC];
#pragma unroll
    for (int ip = 0; ip < TP; ++ip)
#pragma unroll
        for (int ic = 0; ic < TC; ++ic) acc[ip][ic] = typename MF::acc_t{};

    const int wp = wave / C::WGN, wc = wave % C::WGN;
    const int frow = lane & 31, fch = lane >> 5;
    // GN: byte offset in the stage of this lane's first transpose read for
    // fragment row block ip.  In 16-lane group G, lane t reads channel row
    // 8*(G/2) + t/4 (+4 for the second read, +16 per MFMA K step), pixels
    // 16*(G%2) + 4*(t%4) .. +3 of the block; it receives the 4 channels of
    // pixel 16*(G%2) + t, so lanes 0-31 get channels 0-7 and lanes 32-63
    // channels 8-15 of pixels lane%32: the MFMA A operand.
    uint32_t aoff[GN ? TP : 1];
    if constexpr (GN) {
        const int G = lane >> 4, t = lane & 15;
        const int kr = 8 * (G >> 1) + (t >> 2);
        const int px = 16 * (G & 1) + 4 * (t & 3);
#pragma unroll
        for (int ip = 0; ip < TP; ++ip) {
            const int p = wp * WPM + ip * 32 + px;
            aoff[ip] = (uint32_t)((kr * CPRA + ((p / VEC) ^ (4 * (t >> 2)))) * 16 + (p % VEC) * 2);
        }
    }
    typedef short v4s_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s_t *lds_v4s_ptr;
    typedef __attribute__((address_space(3))) char *lds_byte_ptr;
    uint4 fa[NG][TP], fb[NG][TC];
    auto lds_read = [&](const uint4 *st, int grp) {
        if constexpr (GN) {
            const lds_byte_ptr sb = (lds_byte_ptr)(lds_ptr_t)st;
#pragma unroll
            for (int ip = 0; ip < TP; ++ip) {
                const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4s_ptr)(sb + aoff[ip] + grp * 16 * CPRA * 16));
                const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4s_ptr)(sb + aoff[ip] + (grp * 16 + 4) * CPRA * 16));
                const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
                fa[grp][ip] = make_uint4(l2.x, l2.y, h2.x, h2.y);
            }
        } else {
#pragma unroll
            for (int ip = 0; ip < TP; ++ip)
                fa[grp][ip] = st[dual_slot<KCH>(wp * WPM + ip * 32 + frow, grp * 2 + fch)];
        }
#pragma unroll
        for (int ic = 0; ic < TC; ++ic)
            fb[grp][ic] = st[BM * KCH + dual_slot<KCH>(wc * WCN + ic * 32 + frow, grp * 2 + fch)];
    };
    auto mfma_group = [&](int grp) {
#pragma unroll
        for (int ip = 0; ip < TP; ++ip)
#pragma unroll
            for (int ic = 0; ic < TC; ++ic) {
                if constexpr (OUT_NCHW)
                    MF::mma(fa[grp][ip], fb[grp][ic], acc[ip][ic]);
                else
                    MF::mma(fb[grp][ic], fa[grp][ip], acc[ip][ic]);
            }
    };
    // Tile kt: its fragments are in registers; st_cur (where it came from)
    // receives tile kt+3 after the barrier, and tile kt+1's fragments are read
    // from st_next, each register group as soon as its MFMAs are issued.
    auto phase = [&](int kt, uint4 *st_cur, const uint4 *st_next) {
        mfma_group(0);
        __builtin_amdgcn_sched_barrier(0);
        CONVLOWER_WAIT_VMCNT_LDS(IPW);
        block_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(kt + 3, st_cur);
        __builtin_amdgcn_sched_barrier(0);
        lds_read(st_next, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int grp = 1; grp < NG; ++grp) {
            mfma_group(grp);
            __builtin_amdgcn_sched_barrier(0);
            lds_read(st_next, grp);
            __builtin_amdgcn_sched_barrier(0);
        }
        read_pix();  // for tile kt+4, issued in the next phase
        __builtin_amdgcn_sched_barrier(0);
    };

    __syncthreads();  // ibs and bias_s written

    if (nk > 0) {
        read_pix();
        issue(0, st0);
        read_pix();
        issue(1, st1);
        read_pix();
        issue(2, st2);
        read_pix();
        CONVLOWER_WAIT_VMCNT(2 * IPW);
        block_barrier();
#pragma unroll
        for (int grp = 0; grp < NG; ++grp) lds_read(st0, grp);
        for (int kt = 0;; kt += 3) {
            phase(kt, st0, st1);
            if (kt + 1 >= nk) break;
            phase(kt + 1, st1, st2);
            if (kt + 2 >= nk) break;
            phase(kt + 2, st2, st0);
            if (kt + 3 >= nk) break;
        }
        CONVLOWER_WAIT_VMCNT(0);  // no load may still write LDS when the block ends
    }

    dual_store<S, OUT_NCHW, C>(A, acc, &stg[0][0], bias_s, m0, co0, wp, wc, lane, tid);
}

template <typename S, int FEED, bool OUT_NCHW>
__global__ __launch_bounds__(256, 2) void igemm_dual_kernel(GemmArgs A) {
    igemm_dual_body<S, FEED, OUT_NCHW, DualCfg4<S>>(A);
}

template <typename S, int FEED, bool OUT_NCHW>
__global__ __launch_bounds__(512, 1) void igemm_oct_kernel(GemmArgs A) {
    igemm_dual_body<S, FEED, OUT_NCHW, DualCfg8<S>>(A);
}

template <typename S, int FEED, bool OUT_NCHW>
__global__ __launch_bounds__(256, 4) void igemm_quad_kernel(GemmArgs A) {
    igemm_dual_body<S, FEED, OUT_NCHW, QuadCfg<S>>(A);
}

template <typename S, int FEED, bool OUT_NCHW>
__global__ __launch_bounds__(512, 1) void igemm_oct_sq_kernel(GemmArgs A) {
    igemm_dual_body<S, FEED, OUT_NCHW, DualCfg8Sq<S>>(A);
}

}  // namespace convlower
