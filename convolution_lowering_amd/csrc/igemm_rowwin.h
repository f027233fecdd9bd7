// The window-ordered layout of "Im2win: An Efficient Convolution Paradigm on
// GPU" (abstract) built in LDS instead of in memory.  For stride 1 and
// dilation 1, the KW taps of one kernel row read the same input row shifted
// by one pixel per tap.  So a K step here is (channel slice, kernel row kh):
// for every output row the block's 256 pixels touch, the LDS stage holds the
// run of input pixels those windows cover on input row ho - pad + kh (its
// Wo-pixel segment plus KW - 1 more), one slice of channels per pixel.  The
// KW taps of the step then read their MFMA fragments from that one run, at
// row offsets 0 .. KW-1.  Each input pixel crosses from L2 into LDS once per
// (slice, kh), not KW times.
//
// Two 256-thread blocks per compute unit (four wavefronts of 128 x 64 each,
// two wavefronts on every SIMD), so one block's barriers and epilogue hide
// behind the other's MFMAs; block tile 256 x 128; channels-last input, OHWI
// weights.  The A runs of a step and the B rows of a tap pipeline
// separately: two A stages (the next step's runs load during a whole step)
// and four B stages (each tap's weights load three taps ahead).  Swizzle and
// epilogue are those of igemm_dual.h.
#pragma once

namespace convlower {

// Stage geometry for KW taps per kernel row.  A tile of 256 consecutive
// output pixels spans at most kRowWinMaxSeg output rows (the host checks
// 255 / Wo + 2 against it); each adds KW - 1 pixels to the stage.
// BN_: output channels per block tile, 128 (four 128 x 64 wavefront tiles,
// 2 x 2) or 64 (four 64 x 64 wavefront tiles stacked along M, for layers with
// at most 64 output channels, which a 128-wide tile would half waste).
template <typename S, int KW_, int BN_ = 128>
struct RowWinCfg {
    static_assert(BN_ == 128 || BN_ == 64, "block tiles 256 x 128 or 256 x 64");
    static constexpr int KW = KW_;
    static constexpr int BM = 256, BN = BN_;
    static constexpr int ES = (int)sizeof(S);
    static constexpr int VEC = 16 / ES;
    static constexpr int KCH = 4;                    // 16-byte chunks per stage row (one channel slice)
    static constexpr int NW = 4, NTHR = 256;
    static constexpr int RPI = 64 / KCH;             // stage rows one 64-lane load fills
    static constexpr int BK = KCH * VEC;             // channels per slice
    static constexpr int ROWS_A = BM + (KW - 1) * kRowWinMaxSeg;  // input-pixel runs of a step
    static constexpr int A_SLOTS = ROWS_A * KCH, B_SLOTS = BN * KCH;
    static constexpr int NA = 2, NB = 4;             // A and B stages
    static constexpr int IPW_A = ROWS_A * KCH / 64 / NW;
    static constexpr int IPW_B = BN * KCH / 64 / NW;
    static constexpr int WGM = BN_ == 128 ? 2 : 4, WGN = BN_ == 128 ? 2 : 1;
    static constexpr int WPM = BM / WGM, WCN = BN / WGN;  // wavefront tile 128 x 64 or 64 x 64
    static constexpr int MT = 32, TP = WPM / MT, TC = WCN / MT;
    static constexpr int NG = KCH / 2;
    static constexpr int LDS_SLOTS = NA * A_SLOTS + NB * B_SLOTS;
    static constexpr long long STAGE_BYTES = 16LL * LDS_SLOTS;  // all stages, reused by the epilogue
    static_assert(IPW_A * NW * 64 == ROWS_A * KCH && IPW_B * NW * 64 == BN * KCH, "loads must split evenly");
    static_assert(2 * (STAGE_BYTES + BN * 4) <= 160 * 1024, "two blocks per compute unit");
};

template <typename S, bool OUT_NCHW, typename C>
__device__ __forceinline__ void igemm_rowwin_body(const GemmArgs &A) {
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, VEC = C::VEC, KCH = C::KCH;
    constexpr int IPW_A = C::IPW_A, IPW_B = C::IPW_B;
    constexpr int WPM = C::WPM, WCN = C::WCN, TP = C::TP, TC = C::TC, NG = C::NG;
    constexpr int NW = C::NW, RPI = C::RPI, KW = C::KW, A_SLOTS = C::A_SLOTS, B_SLOTS = C::B_SLOTS;
    constexpr uint32_t ES = (uint32_t)sizeof(S);
    using MF = MfmaShape<S, 32>;
    static_assert(KW == 3, "the schedule below is written for three taps per kernel row");

    __shared__ uint4 lds[C::LDS_SLOTS];  // A stages, then B stages; the epilogue reuses them
    uint4 *const sa0 = lds, *const sa1 = lds + A_SLOTS;
    uint4 *const sb0 = lds + 2 * A_SLOTS;  // B stage i at sb0 + i * B_SLOTS; tap u uses stage u % 4
    __shared__ float bias_s[BN];

    const Geom &g = A.g;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    int mt, nt;
    tile_coords_l2((int)((g.M + BM - 1) / BM), (g.Co + BN - 1) / BN, (long long)BN * g.K * (long long)sizeof(S), mt, nt);
    const uint32_t M = (uint32_t)g.M;
    const uint32_t m0 = (uint32_t)mt * BM;
    const int co0 = nt * BN;
    const int nk = (g.C / BK) * g.KH;  // K steps: channel slice, then kernel row fastest

    // The bias is read only by the epilogue: its load is issued here and its
    // value goes to LDS after the K loop, so the load's latency passes behind
    // the main loop instead of delaying the block's first loads.
    float bias_r = 0.f;
    if (tid < BN) {
        const int co = co0 + tid;
        if (A.bias && co < g.Co) bias_r = bits_to_f32(S(), elem_bits((const S *)A.bias, co));
    }

    // ---- the block's segments ------------------------------------------------
    // Output row R (of all N*Ho) holds pixels R*Wo .. R*Wo + Wo-1.  The tile's
    // pixels [m0, mend) fall into rows R0, R0+1, ...; segment j is the part
    // in row R0 + j, and its stage rows are its pixels plus KW - 1 more, the
    // segments back to back.  Segment 0 starts at pixel m0; every later one
    // starts at the beginning of its row and, except the last, has Wo pixels,
    // so it takes SW = Wo + KW - 1 stage rows.
    const uint32_t Wo = (uint32_t)g.Wo;
    const uint32_t mend = min(m0 + (uint32_t)BM, M);
    const uint32_t R0 = m0 / Wo;
    const uint32_t SW = Wo + (uint32_t)(KW - 1);
    const uint32_t rows0 = min(mend, (R0 + 1) * Wo) - m0 + (uint32_t)(KW - 1);

    // ---- per-lane load geometry -------------------------------------------------
    // As in igemm_dual.h: load i of this wavefront covers stage rows
    // (i*NW + wave)*RPI .. +RPI-1 and lane L fetches chunk column kc of row
    // L/KCH.  An A row is input pixel (n, ho - pad + kh, wi) of its segment's
    // output row; out-of-image pixels and rows past the last segment load
    // zeros (offsets past the buffer).
    const int lrow = lane / KCH;
    const uint32_t kc = (uint32_t)(((lane % KCH) ^ dual_swz<KCH>(wave * RPI + lrow)) * VEC);
    const int HWC = g.H * g.W * g.C, WC = g.W * g.C;
    int abase[IPW_A], ahi[IPW_A];
    bool aok[IPW_A];
#pragma unroll
    for (int i = 0; i < IPW_A; ++i) {
        const uint32_t r = (uint32_t)((i * NW + wave) * RPI + lrow);
        // Segment j of stage row r and r's place in it (off), in closed form.
        uint32_t j = 0, off = r;
        if (r >= rows0) {
            const uint32_t t = r - rows0;
            j = 1 + t / SW;
            off = t - (j - 1) * SW;
        }
        const uint32_t R = R0 + j;
        const uint32_t first = max(m0, R * Wo);
        // A row past the last segment (or in the unused tail of a partial last
        // segment) loads zeros.
        const bool live = first < mend && off < min(mend, (R + 1) * Wo) - first + (uint32_t)(KW - 1);
        const uint32_t n = R / (uint32_t)g.Ho, ho = R - n * (uint32_t)g.Ho;
        const int wi = (int)(first - R * Wo) + (int)off - g.p;
        const int hi0 = (int)ho - g.p;
        aok[i] = live && wi >= 0 && wi < g.W;
        ahi[i] = hi0;
        abase[i] = live ? (int)n * HWC + hi0 * WC + wi * g.C : 0;  // may be negative while hi0 < 0
    }
    int wbase[IPW_B];
    bool wok[IPW_B];
#pragma unroll
    for (int j = 0; j < IPW_B; ++j) {
        const int co = co0 + (j * NW + wave) * RPI + lrow;
        wok[j] = co < g.Co;
        wbase[j] = co * g.KH * KW * g.C;  // OHWI, tap (0, 0)
    }

    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A.a_src, A.a_bytes);
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(A.b, A.b_bytes);
    const uint32_t lds_w = (uint32_t)wave * 1024u;

    // The A runs of K step kt into stage sa, and the B rows of tap u (step
    // u / KW, kw = u % KW) into stage sb.  Past the end nothing is loaded,
    // but the loads are still issued so the count in flight stays fixed.
    auto issue_a = [&](int kt, uint4 *sa) {
        const bool live = kt < nk;
        const int slice = kt / g.KH, kh = kt - slice * g.KH;
        const int cofs = slice * BK + (int)kc;
        const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)sa + lds_w;
        uint32_t voff[IPW_A];
#pragma unroll
        for (int i = 0; i < IPW_A; ++i) {
            const int hi = ahi[i] + kh;
            const bool valid = live && aok[i] && hi >= 0 && hi < g.H;
            voff[i] = valid ? (uint32_t)(abase[i] + kh * WC + cofs) * ES : kOutOfRange;
        }
#pragma unroll
        for (int i = 0; i < IPW_A; ++i) lds_dma16(a_rsrc, voff[i], lds0 + (uint32_t)(i * NW * 1024));
    };
    auto issue_b = [&](int u, uint4 *sb) {
        const int kt = u / KW, kw = u - kt * KW;
        const bool live = kt < nk;
        const int slice = kt / g.KH, kh = kt - slice * g.KH;
        const int wofs = (kh * KW + kw) * g.C + slice * BK + (int)kc;
        const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)sb + lds_w;
        uint32_t voff[IPW_B];
#pragma unroll
        for (int j = 0; j < IPW_B; ++j) voff[j] = live && wok[j] ? (uint32_t)(wbase[j] + wofs) * ES : kOutOfRange;
#pragma unroll
        for (int j = 0; j < IPW_B; ++j) lds_dma16(b_rsrc, voff[j], lds0 + (uint32_t)(j * NW * 1024));
    };

    typename MF::acc_t acc[TP][TC];
#pragma unroll
    for (int ip = 0; ip < TP; ++ip)
#pragma unroll
        for (int ic = 0; ic < TC; ++ic) acc[ip][ic] = typename MF::acc_t{};

    // Stage row of this lane's fragment rows for tap 0: pixel m0 + p sits at
    // row p + (KW - 1) * (its segment); tap kw reads row + kw.
    const int wp = wave / C::WGN, wc = wave % C::WGN;
    const int frow = lane & 31, fch = lane >> 5;
    int arow[TP];
#pragma unroll
    for (int ip = 0; ip < TP; ++ip) {
        const uint32_t pl = (uint32_t)(wp * WPM + ip * 32 + frow);
        arow[ip] = (int)pl + (KW - 1) * (int)((m0 + pl) / Wo - R0);
    }
    uint4 fa[NG][TP], fb[NG][TC];
    auto lds_read = [&](const uint4 *sa, const uint4 *sb, int kw, int grp) {
#pragma unroll
        for (int ip = 0; ip < TP; ++ip) fa[grp][ip] = sa[dual_slot<KCH>(arow[ip] + kw, grp * 2 + fch)];
#pragma unroll
        for (int ic = 0; ic < TC; ++ic) fb[grp][ic] = sb[dual_slot<KCH>(wc * WCN + ic * 32 + frow, grp * 2 + fch)];
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
    // Tap u = (kt, kw): its fragments are in registers.  After its first MFMA
    // group: wait until tap u+1's weights (and, before the last tap of a
    // step, step kt+1's runs) have landed and this wavefront's LDS reads are
    // done, barrier, refill the B stage tap u used with tap u+4's weights
    // (and, at kw = 0 and before them, the other A stage with step kt+1's
    // runs), then read tap u+1's fragments group by group behind the
    // remaining MFMAs.  Loads complete in issue order, so each wait allows
    // exactly the loads issued after the ones it needs: taps u+2 and u+3's
    // weights, and at kw = 1 also step kt+1's runs, issued between them.
    auto sub = [&](int kt, int kw, uint4 *sa, uint4 *sa_next, uint4 *sb, const uint4 *sb_next) {
        mfma_group(0);
        __builtin_amdgcn_sched_barrier(0);
        if (kw == 1)
            CONVLOWER_WAIT_VMCNT_LDS(IPW_A + 2 * IPW_B);
        else
            CONVLOWER_WAIT_VMCNT_LDS(2 * IPW_B);
        block_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (kw == 0) issue_a(kt + 1, sa_next);
        issue_b(kt * KW + kw + 4, sb);
        __builtin_amdgcn_sched_barrier(0);
        const uint4 *ra = kw + 1 < KW ? sa : sa_next;
        const int rkw = kw + 1 < KW ? kw + 1 : 0;
        lds_read(ra, sb_next, rkw, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int grp = 1; grp < NG; ++grp) {
            mfma_group(grp);
            __builtin_amdgcn_sched_barrier(0);
            lds_read(ra, sb_next, rkw, grp);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // One K step whose first tap uses B stage b0 (taps rotate through four
    // B stages, steps through two A stages).
    auto step = [&](int kt, uint4 *sa, uint4 *sa_next, int b0) {
#pragma unroll
        for (int kw = 0; kw < KW; ++kw)
            sub(kt, kw, sa, sa_next, sb0 + ((b0 + kw) & 3) * B_SLOTS, sb0 + ((b0 + kw + 1) & 3) * B_SLOTS);
    };

    if (nk > 0) {
        issue_a(0, sa0);
#pragma unroll
        for (int u = 0; u < 4; ++u) issue_b(u, sb0 + u * B_SLOTS);
        CONVLOWER_WAIT_VMCNT(3 * IPW_B);  // step 0's runs and tap 0's weights
        block_barrier();
#pragma unroll
        for (int grp = 0; grp < NG; ++grp) lds_read(sa0, sb0, 0, grp);
        // Four steps (twelve taps) bring A and B stages back into phase.
        for (int kt = 0;; kt += 4) {
            step(kt, sa0, sa1, 0);
            if (kt + 1 >= nk) break;
            step(kt + 1, sa1, sa0, 3);
            if (kt + 2 >= nk) break;
            step(kt + 2, sa0, sa1, 2);
            if (kt + 3 >= nk) break;
            step(kt + 3, sa1, sa0, 1);
            if (kt + 4 >= nk) break;
        }
        CONVLOWER_WAIT_VMCNT(0);  // no load may still write LDS when the block ends
    }

    // bias_s is a separate array from the stages; the epilogue's first
    // barrier publishes it.
    if (tid < BN) bias_s[tid] = bias_r;
    dual_store<S, OUT_NCHW, C>(A, acc, lds, bias_s, m0, co0, wp, wc, lane, tid);
}

template <typename S, bool OUT_NCHW, int BN = 128>
__global__ __launch_bounds__(256, 2) void igemm_rowwin_kernel(GemmArgs A) {
    igemm_rowwin_body<S, OUT_NCHW, RowWinCfg<S, 3, BN>>(A);
}

}  // namespace convlower
