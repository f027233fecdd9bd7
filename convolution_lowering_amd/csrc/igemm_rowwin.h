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
// Pipeline, swizzle and epilogue are those of igemm_dual.h; one 512-thread
// block per compute unit (eight wavefronts of 64 x 64 in a 4 x 2 grid, two
// on every SIMD); block tile 256 x 128; channels-last input, OHWI weights.
#pragma once

namespace convlower {

// Stage geometry for KW taps per kernel row.  A tile of 256 consecutive
// output pixels spans at most kRowWinMaxSeg output rows (the host checks
// 255 / Wo + 2 against it); each adds KW - 1 pixels to the stage.
template <typename S, int KW_>
struct RowWinCfg {
    static constexpr int KW = KW_;
    static constexpr int BM = 256, BN = 128;
    static constexpr int ES = (int)sizeof(S);
    static constexpr int VEC = 16 / ES;
    static constexpr int KCH = 4;                    // 16-byte chunks per stage row (one channel slice)
    static constexpr int NW = 8, NTHR = 512;
    static constexpr int RPI = 64 / KCH;             // stage rows one 64-lane load fills
    static constexpr int BK = KCH * VEC;             // channels per slice
    static constexpr int ROWS_A = BM + (KW - 1) * kRowWinMaxSeg;  // input-pixel runs
    static constexpr int ROWS_B = KW * BN;           // the KW taps' weights
    static constexpr int NSLOT = (ROWS_A + ROWS_B) * KCH;
    static constexpr int IPW_A = ROWS_A * KCH / 64 / NW;
    static constexpr int IPW_B = ROWS_B * KCH / 64 / NW;
    static constexpr int IPW = IPW_A + IPW_B;
    static constexpr int WGM = 4, WGN = 2;
    static constexpr int WPM = BM / WGM, WCN = BN / WGN;  // wavefront tile 64 x 64
    static constexpr int MT = 32, TP = WPM / MT, TC = WCN / MT;
    static constexpr int NG = KCH / 2;
    static constexpr long long STAGE_BYTES = 3LL * NSLOT * 16;
    static_assert(IPW_A * NW * 64 == ROWS_A * KCH && IPW_B * NW * 64 == ROWS_B * KCH, "loads must split evenly");
    static_assert(STAGE_BYTES + BN * 4 <= 160 * 1024, "one block per compute unit");
};

template <typename S, bool OUT_NCHW, typename C>
__device__ __forceinline__ void igemm_rowwin_body(const GemmArgs &A) {
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, VEC = C::VEC, KCH = C::KCH, NSLOT = C::NSLOT;
    constexpr int IPW_A = C::IPW_A, IPW_B = C::IPW_B, IPW = C::IPW;
    constexpr int WPM = C::WPM, WCN = C::WCN, TP = C::TP, TC = C::TC, NG = C::NG;
    constexpr int NW = C::NW, RPI = C::RPI, KW = C::KW, ROWS_A = C::ROWS_A;
    constexpr uint32_t ES = (uint32_t)sizeof(S);
    using MF = MfmaShape<S, 32>;

    __shared__ uint4 stg[3][NSLOT];  // the three stages; the epilogue reuses them
    uint4 *const st0 = stg[0], *const st1 = stg[1], *const st2 = stg[2];
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
    const int nk = (g.C / BK) * g.KH;  // K steps: channel slice, then kernel row fastest

    if (tid < BN) {
        const int co = co0 + tid;
        float b = 0.f;
        if (A.bias && co < g.Co) b = bits_to_f32(S(), elem_bits((const S *)A.bias, co));
        bias_s[tid] = b;
    }

    // ---- the block's segments ------------------------------------------------
    // Output row R (of all N*Ho) holds pixels R*Wo .. R*Wo + Wo-1.  The tile's
    // pixels [m0, mend) fall into rows R0, R0+1, ...; segment j is the part
    // in row R0 + j, and its stage rows are its pixels plus KW - 1 more, the
    // segments back to back.
    const uint32_t Wo = (uint32_t)g.Wo;
    const uint32_t mend = min(m0 + (uint32_t)BM, M);
    const uint32_t R0 = m0 / Wo;

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
        uint32_t start = 0, j = 0;
        aok[i] = false;
        abase[i] = 0;
        ahi[i] = 0;
        for (; j < (uint32_t)kRowWinMaxSeg; ++j) {
            const uint32_t R = R0 + j;
            const uint32_t first = max(m0, R * Wo);
            if (first >= mend) break;
            const uint32_t len = min(mend, (R + 1) * Wo) - first;
            const uint32_t rows = len + (uint32_t)(KW - 1);
            if (r < start + rows) {
                const uint32_t n = R / (uint32_t)g.Ho, ho = R - n * (uint32_t)g.Ho;
                const int wi = (int)(first - R * Wo) + (int)(r - start) - g.p;
                const int hi0 = (int)ho - g.p;
                aok[i] = wi >= 0 && wi < g.W;
                ahi[i] = hi0;
                abase[i] = (int)n * HWC + hi0 * WC + wi * g.C;  // may be negative while hi0 < 0
                break;
            }
            start += rows;
        }
    }
    int wbase[IPW_B];
    bool wok[IPW_B];
#pragma unroll
    for (int j = 0; j < IPW_B; ++j) {
        const int rb = (j * NW + wave) * RPI + lrow;  // tap rb / BN, channel co0 + rb % BN
        const int kw = rb / BN, co = co0 + rb % BN;
        wok[j] = co < g.Co;
        wbase[j] = (co * g.KH * KW + kw) * g.C;  // OHWI, kernel row 0
    }

    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A.a_src, A.a_bytes);
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(A.b, A.b_bytes);
    const uint32_t lds_w = (uint32_t)wave * 1024u;

    // Issue the loads of K step kt into stage st (steps past the end load
    // nothing but keep the count of loads in flight the same).
    auto issue = [&](int kt, uint4 *st) {
        const bool live = kt < nk;
        const int slice = kt / g.KH, kh = kt - slice * g.KH;
        const int cofs = slice * BK + (int)kc;
        const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)st + lds_w;
        uint32_t voff[IPW];
#pragma unroll
        for (int i = 0; i < IPW_A; ++i) {
            const int hi = ahi[i] + kh;
            const bool valid = live && aok[i] && hi >= 0 && hi < g.H;
            voff[i] = valid ? (uint32_t)(abase[i] + kh * WC + cofs) * ES : kOutOfRange;
        }
#pragma unroll
        for (int j = 0; j < IPW_B; ++j)
            voff[IPW_A + j] = live && wok[j] ? (uint32_t)(wbase[j] + kh * KW * g.C + cofs) * ES : kOutOfRange;
#pragma unroll
        for (int i = 0; i < IPW_A; ++i) lds_dma16(a_rsrc, voff[i], lds0 + (uint32_t)(i * NW * 1024));
#pragma unroll
        for (int j = 0; j < IPW_B; ++j)
            lds_dma16(b_rsrc, voff[IPW_A + j], lds0 + (uint32_t)(ROWS_A * KCH * 16 + j * NW * 1024));
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
    auto lds_read = [&](const uint4 *st, int kw, int grp) {
#pragma unroll
        for (int ip = 0; ip < TP; ++ip) fa[grp][ip] = st[dual_slot<KCH>(arow[ip] + kw, grp * 2 + fch)];
#pragma unroll
        for (int ic = 0; ic < TC; ++ic)
            fb[grp][ic] = st[ROWS_A * KCH + dual_slot<KCH>(kw * BN + wc * WCN + ic * 32 + frow, grp * 2 + fch)];
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
    // Step kt: the fragments of its tap 0 are in registers.  Taps 0 .. KW-2
    // are multiplied while the next tap's fragments are read from st_cur;
    // then (all reads of st_cur done) the barrier, st_cur receives step
    // kt+3, and the last tap is multiplied while step kt+1's tap-0 fragments
    // are read from st_next.
    auto phase = [&](int kt, uint4 *st_cur, const uint4 *st_next) {
#pragma unroll
        for (int kw = 0; kw + 1 < KW; ++kw) {
#pragma unroll
            for (int grp = 0; grp < NG; ++grp) {
                mfma_group(grp);
                __builtin_amdgcn_sched_barrier(0);
                lds_read(st_cur, kw + 1, grp);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        mfma_group(0);
        __builtin_amdgcn_sched_barrier(0);
        CONVLOWER_WAIT_VMCNT_LDS(IPW);
        block_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(kt + 3, st_cur);
        __builtin_amdgcn_sched_barrier(0);
        lds_read(st_next, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int grp = 1; grp < NG; ++grp) {
            mfma_group(grp);
            __builtin_amdgcn_sched_barrier(0);
            lds_read(st_next, 0, grp);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    __syncthreads();  // bias_s written

    if (nk > 0) {
        issue(0, st0);
        issue(1, st1);
        issue(2, st2);
        CONVLOWER_WAIT_VMCNT(2 * IPW);
        block_barrier();
#pragma unroll
        for (int grp = 0; grp < NG; ++grp) lds_read(st0, 0, grp);
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

template <typename S, bool OUT_NCHW>
__global__ __launch_bounds__(512, 1) void igemm_rowwin_kernel(GemmArgs A) {
    igemm_rowwin_body<S, OUT_NCHW, RowWinCfg<S, 3>>(A);
}

}  // namespace convlower
