// The window-row loop of igemm_rowwin.h (the window-ordered layout of
// "Im2win: An Efficient Convolution Paradigm on GPU", abstract, built in LDS)
// as one 512-thread block per compute unit over a 512 x 128 output tile,
// with its two halves in ping-pong.
//
// Waves 0-3 (half P) own output rows 0-255 of the tile, waves 4-7 (half Q)
// rows 256-511; each half is a 2 x 2 grid of 128 x 64 wavefront tiles.  A
// compute unit places wave w on SIMD w % 4, so every SIMD holds one wave of
// each half.  Each tap u runs as two phases separated by block barriers:
//
//   X(u): P multiplies tap u;  Q issues the loads of tap u+3 and reads its
//         fragments of tap u from LDS.
//   Y(u): Q multiplies tap u;  P issues the loads of tap u+4 and reads its
//         fragments of tap u+1.
//
// A buffer load to LDS waits at issue until the address unit takes it, and
// in-order issue puts that wait in front of everything after it.  Here the
// waits of one half fall in the phase in which the other half keeps the
// SIMD's matrix core busy.  The 128 weight rows of a tap are loaded once for
// 512 output pixels, half the weight bytes per MAC of two 256 x 128 blocks.
//
// Stages: two A stages (the runs of one K step = channel slice x kernel
// row; rows for the 512 pixels' segments plus KW - 1 each) and four B stages
// (one tap's weight rows each).  Each tap's loads are split over all eight
// wavefronts; P issues its share of tap t in Y(t-4), Q in X(t-3), and every
// wavefront waits for its share before the barrier that ends X(t-1), after
// which P reads tap t (in Y(t-1)) and then Q (in X(t)).  A B stage is
// refilled only after Q's reads of the tap it held (X(t)) and P's (Y(t-1));
// an A stage after both halves have read the last tap of its step.
#pragma once

namespace convlower {

template <typename S, int KW_>
struct RowWinPPCfg {
    static constexpr int KW = KW_;
    static constexpr int BM = 512, BN = 128;
    static constexpr int ES = (int)sizeof(S);
    static constexpr int VEC = 16 / ES;
    static constexpr int KCH = 4;         // 16-byte chunks per stage row (one channel slice)
    static constexpr int NW = 8, NTHR = 512;
    static constexpr int RPI = 64 / KCH;  // stage rows one 64-lane load fills
    static constexpr int BK = KCH * VEC;  // channels per slice
    static constexpr int MAXSEG = 2 * kRowWinMaxSeg;  // output rows 512 pixels may span
    static constexpr int ROWS_A = BM + (KW - 1) * MAXSEG;
    static constexpr int A_SLOTS = ROWS_A * KCH, B_SLOTS = BN * KCH;
    static constexpr int NA = 2, NB = 4;
    static constexpr int IPW_A = ROWS_A * KCH / 64 / NW;
    static constexpr int IPW_B = BN * KCH / 64 / NW;
    static constexpr int WGM = 4, WGN = 2;                // wave grid; waves 0-3 are rows 0-255
    static constexpr int WPM = BM / WGM, WCN = BN / WGN;  // wavefront tile 128 x 64
    static constexpr int MT = 32, TP = WPM / MT, TC = WCN / MT;
    static constexpr int NG = KCH / 2;
    static constexpr int LDS_SLOTS = NA * A_SLOTS + NB * B_SLOTS;
    static constexpr long long STAGE_BYTES = 16LL * LDS_SLOTS;  // all stages, reused by the epilogue
    static_assert(IPW_A * NW * 64 == ROWS_A * KCH && IPW_B * NW * 64 == BN * KCH, "loads must split evenly");
    static_assert(STAGE_BYTES + BN * 4 <= 160 * 1024, "one block per compute unit");
    static_assert(WGM * WGN == NW && (NW / 2) % WGN == 0, "each half is whole rows of the wave grid");
};

// Stream-K (SK, a grid of kSkBlocks blocks): the K steps of all tiles, tile
// after tile, are shared out evenly.  Each XCD (blocks b with b % 8 the same;
// blocks go to the XCDs in turn) takes a contiguous run of whole tiles, so
// its blocks share their weights and input rows in its L2, and its 32 blocks
// split the run's steps into 32 near-equal ranges.  A block takes the tiles
// of its range from the last to the first.  Where a range begins or ends
// inside a tile, the tile is split: the block that holds the tile's last
// step finishes it, and only after all its other work; each other block
// writes its fp32 sums to its own slot first thing (a block holds at most
// one such piece) and raises its flag.  A finishing block waits for the
// flags of lower-numbered blocks only, and adds their sums in block order
// (deterministic results).  The partial sums and flags move with device-
// coherent loads and stores, so no cache needs flushing.  The wait is
// bounded (kSkSpinMax polls); blocks start in index order, so it always ends
// long before that (were it ever to run out, the tile is written as NaN).
constexpr int kSkSpinMax = 1 << 16;
constexpr int kCachePolicySc1 = 16;  // buffer-instruction cache policy: coherent across the device

template <typename S, bool OUT_NCHW, typename C, bool SK>
__device__ __forceinline__ void igemm_rowwin_pp_body(const GemmArgs &A) {
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, VEC = C::VEC, KCH = C::KCH;
    constexpr int IPW_A = C::IPW_A, IPW_B = C::IPW_B;
    constexpr int WPM = C::WPM, WCN = C::WCN, TP = C::TP, TC = C::TC, NG = C::NG;
    constexpr int NW = C::NW, RPI = C::RPI, KW = C::KW, A_SLOTS = C::A_SLOTS, B_SLOTS = C::B_SLOTS;
    constexpr uint32_t ES = (uint32_t)sizeof(S);
    using MF = MfmaShape<S, 32>;
    static_assert(KW == 3, "the schedule below is written for three taps per kernel row");

    __shared__ uint4 lds[C::LDS_SLOTS];  // A stages, then B stages; the epilogue reuses them
    uint4 *const sa0 = lds;
    uint4 *const sb0 = lds + C::NA * A_SLOTS;  // tap t in B stage t % 4, step s in A stage s % 2
    __shared__ float bias_s[BN];

    const Geom &g = A.g;
    const int ntm = (int)((g.M + BM - 1) / BM), ntn = (g.Co + BN - 1) / BN;
    const uint32_t M = (uint32_t)g.M;
    const int nk = (g.C / BK) * g.KH;  // K steps: channel slice, then kernel row fastest
    const uint32_t Wo = (uint32_t)g.Wo;
    const uint32_t SW = Wo + (uint32_t)(KW - 1);
    const int HWC = g.H * g.W * g.C, WC = g.W * g.C;

    typename MF::acc_t acc[TP][TC];
    float bias_r = 0.f;

    // K steps [klo, khi) of tile (mt, nt) into acc, which starts at zero.
    // The tile's bias is loaded into bias_r as well: read only by the
    // epilogue, its load's latency passes behind the K loop.  Every per-lane
    // value is derived from `tid` here, so that in the stream-K loop, which
    // passes an opaque copy of it, none is hoisted and held across the loop.
    auto piece = [&](int tid, int mt, int nt, int klo, int khi) {
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const bool half_p = wave < NW / 2;  // wave-uniform
        // Load i of this wavefront covers stage rows (i*NW + wave)*RPI .. +RPI-1;
        // lane L fetches chunk column kc of row L/KCH.
        const int lrow = lane / KCH;
        const uint32_t kc = (uint32_t)(((lane % KCH) ^ dual_swz<KCH>(wave * RPI + lrow)) * VEC);
        const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A.a_src, A.a_bytes);
        const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(A.b, A.b_bytes);
        const uint32_t lds_w = (uint32_t)wave * 1024u;
        const int wp = wave / C::WGN, wc = wave % C::WGN;
        const int frow = lane & 31, fch = lane >> 5;
        const uint32_t m0 = (uint32_t)mt * BM;
        const int co0 = nt * BN;
        bias_r = 0.f;
        if (tid < BN) {
            const int co = co0 + tid;
            if (A.bias && co < g.Co) bias_r = bits_to_f32(S(), elem_bits((const S *)A.bias, co));
        }

        // ---- the tile's segments (as in igemm_rowwin.h) ----------------------
        const uint32_t mend = min(m0 + (uint32_t)BM, M);
        const uint32_t R0 = m0 / Wo;
        const uint32_t rows0 = min(mend, (R0 + 1) * Wo) - m0 + (uint32_t)(KW - 1);

        // ---- per-lane load geometry -------------------------------------------
        int abase[IPW_A], ahi[IPW_A];
        bool aok[IPW_A];
#pragma unroll
        for (int i = 0; i < IPW_A; ++i) {
            const uint32_t r = (uint32_t)((i * NW + wave) * RPI + lrow);
            uint32_t j = 0, off = r;
            if (r >= rows0) {
                const uint32_t t = r - rows0;
                j = 1 + t / SW;
                off = t - (j - 1) * SW;
            }
            const uint32_t R = R0 + j;
            const uint32_t first = max(m0, R * Wo);
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

        // This wavefront's share of the loads of tap t of the piece (K step
        // klo + t / 3): when t opens a K step, that step's A runs (into A
        // stage as), then tap t's B rows (into B stage bs); kw = t % 3,
        // as = (t / 3) % 2 and bs = t % 4, passed as constants of the unrolled
        // loop.  Past the piece's last tap the loads are still issued, as
        // zeros, so every wavefront's count in flight follows the same pattern.
        auto issue_tap = [&](int t, int kw, int as, int bs) {
            const int kt = klo + t / KW;  // kw = t % KW, a constant like as and bs
            const bool live = kt < khi;
            const int slice = kt / g.KH, kh = kt - slice * g.KH;
            if (kw == 0) {
                const int cofs = slice * BK + (int)kc;
                const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)(sa0 + as * A_SLOTS) + lds_w;
                uint32_t voff[IPW_A];
#pragma unroll
                for (int i = 0; i < IPW_A; ++i) {
                    const int hi = ahi[i] + kh;
                    const bool valid = live && aok[i] && hi >= 0 && hi < g.H;
                    voff[i] = valid ? (uint32_t)(abase[i] + kh * WC + cofs) * ES : kOutOfRange;
                }
#pragma unroll
                for (int i = 0; i < IPW_A; ++i) lds_dma16(a_rsrc, voff[i], lds0 + (uint32_t)(i * NW * 1024));
            }
            const int wofs = (kh * KW + kw) * g.C + slice * BK + (int)kc;
            const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)(sb0 + bs * B_SLOTS) + lds_w;
            uint32_t voff[IPW_B];
#pragma unroll
            for (int j = 0; j < IPW_B; ++j) voff[j] = live && wok[j] ? (uint32_t)(wbase[j] + wofs) * ES : kOutOfRange;
#pragma unroll
            for (int j = 0; j < IPW_B; ++j) lds_dma16(b_rsrc, voff[j], lds0 + (uint32_t)(j * NW * 1024));
        };

#pragma unroll
        for (int ip = 0; ip < TP; ++ip)
#pragma unroll
            for (int ic = 0; ic < TC; ++ic) acc[ip][ic] = typename MF::acc_t{};

        // Stage row of this lane's fragment rows for kw = 0: pixel m0 + p sits at
        // row p + (KW - 1) * (its segment); tap kw reads row + kw.
        int arow[TP];
#pragma unroll
        for (int ip = 0; ip < TP; ++ip) {
            const uint32_t pl = (uint32_t)(wp * WPM + ip * 32 + frow);
            arow[ip] = (int)pl + (KW - 1) * (int)((m0 + pl) / Wo - R0);
        }
        uint4 fa[NG][TP], fb[NG][TC];
        // All of a tap's fragments of this wavefront: kernel column kw, A stage
        // as, B stage bs (constants of the unrolled loop).
        auto read_tap = [&](int kw, int as, int bs) {
            const uint4 *sa = sa0 + as * A_SLOTS;
            const uint4 *sb = sb0 + bs * B_SLOTS;
#pragma unroll
            for (int grp = 0; grp < NG; ++grp) {
#pragma unroll
                for (int ip = 0; ip < TP; ++ip) fa[grp][ip] = sa[dual_slot<KCH>(arow[ip] + kw, grp * 2 + fch)];
#pragma unroll
                for (int ic = 0; ic < TC; ++ic) fb[grp][ic] = sb[dual_slot<KCH>(wc * WCN + ic * 32 + frow, grp * 2 + fch)];
            }
        };
        auto mfma_tap = [&]() {
#pragma unroll
            for (int grp = 0; grp < NG; ++grp)
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

        // The loop body, the same for both halves: multiply tap w, barrier, read
        // this wavefront's fragments of tap w+1 and issue its share of tap w+4
        // (the reads first, so the LDS works while the loads wait at issue),
        // barrier.  Half P runs body(w) over X(w) and Y(w); half Q runs it one
        // phase later, over Y(w) and X(w+1).  w = u0 + j with u0 a multiple of 12
        // and j a constant: kw = j % 3, A stage of tap t = (t / 3) % 2, B stage t % 4.
        // Before each barrier a wavefront waits until, after the share it must
        // have landed, only its shares of the next two taps remain in flight --
        // one B load each, plus the A loads of whichever of them opens a K step.
        // That is tap w+1 at the first barrier (ending X(w) for P) and tap w+2
        // at the second (ending X(w+1) for Q); for the other half each wait
        // asks for loads it would wait for one phase later.
        auto body = [&](int w, int j) {
            const int kw = j % 3;
            mfma_tap();
            __builtin_amdgcn_sched_barrier(0);
            if (kw == 2)
                CONVLOWER_WAIT_VMCNT_LDS(2 * IPW_B);
            else
                CONVLOWER_WAIT_VMCNT_LDS(2 * IPW_B + IPW_A);
            block_barrier();
            __builtin_amdgcn_sched_barrier(0);
            read_tap((j + 1) % 3, ((j + 1) / 3) & 1, (j + 1) & 3);
            issue_tap(w + 4, (j + 4) % 3, ((j + 4) / 3) & 1, (j + 4) & 3);
            __builtin_amdgcn_sched_barrier(0);
            if (kw == 1)
                CONVLOWER_WAIT_VMCNT_LDS(2 * IPW_B);
            else
                CONVLOWER_WAIT_VMCNT_LDS(2 * IPW_B + IPW_A);
            block_barrier();
            __builtin_amdgcn_sched_barrier(0);
        };

        const int ntap = (khi - klo) * KW;
        if (ntap > 0) {
            // Taps 0-2 from every wavefront; once tap 0 has landed, P issues tap 3
            // and reads tap 0 (phase Y(-1)); Q does the same in X(0), while P
            // multiplies tap 0 in its first body.  Each wavefront passes 2T + 3
            // barriers in all (T taps).
            issue_tap(0, 0, 0, 0);
            issue_tap(1, 1, 0, 1);
            issue_tap(2, 2, 0, 2);
            CONVLOWER_WAIT_VMCNT(2 * IPW_B);  // after tap 0: taps 1 and 2, one B load each, no A
            block_barrier();
            if (half_p) {
                read_tap(0, 0, 0);
                issue_tap(3, 0, 1, 3);
            }
            CONVLOWER_WAIT_VMCNT_LDS(63);  // LDS reads done (vmcnt unconstrained)
            block_barrier();
            if (!half_p) {
                read_tap(0, 0, 0);
                issue_tap(3, 0, 1, 3);
                CONVLOWER_WAIT_VMCNT_LDS(2 * IPW_B + IPW_A);  // tap 1 landed: taps 2 and 3 remain
                block_barrier();
            }
            // Four K steps (twelve taps) bring the A and B stages back into phase;
            // the loop leaves after any whole step.
            for (int u0 = 0;; u0 += 12) {
                body(u0, 0), body(u0 + 1, 1), body(u0 + 2, 2);
                if (u0 + 3 >= ntap) break;
                body(u0 + 3, 3), body(u0 + 4, 4), body(u0 + 5, 5);
                if (u0 + 6 >= ntap) break;
                body(u0 + 6, 6), body(u0 + 7, 7), body(u0 + 8, 8);
                if (u0 + 9 >= ntap) break;
                body(u0 + 9, 9), body(u0 + 10, 10), body(u0 + 11, 11);
                if (u0 + 12 >= ntap) break;
            }
            if (half_p) block_barrier();  // pairs with Q's last barrier
            CONVLOWER_WAIT_VMCNT(0);      // no load may still write LDS when the piece ends
        }
    };
    // Bias, rounding and the store of tile (mt, nt) from acc.
    auto finish = [&](int tid, int mt, int nt) {
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        if (tid < BN) bias_s[tid] = bias_r;  // the epilogue's first barrier publishes it
        dual_store<S, OUT_NCHW, C>(A, acc, lds, bias_s, (uint32_t)mt * BM, nt * BN, wave / C::WGN, wave % C::WGN,
                                   lane, tid);
    };

    if constexpr (!SK) {
        const int tid = threadIdx.x;
        int mt, nt;
        tile_coords_l2(ntm, ntn, (long long)BN * g.K * (long long)sizeof(S), mt, nt);
        piece(tid, mt, nt, 0, nk);
        finish(tid, mt, nt);
    } else {
        // acc[ip][ic] as NQ 16-byte chunks: chunk c = (ip*TC + ic)*NQ + q of
        // thread tid sits at byte (c*NTHR + tid)*16 of a block's slot.
        constexpr int NQ = (int)(sizeof(typename MF::acc_t) / 16);
        constexpr int NTHR = C::NTHR;
        typedef unsigned int v4u32_t __attribute__((ext_vector_type(4)));
        static_assert((size_t)TP * TC * NQ * NTHR * 16 == kSkSlotBytes, "one slot holds a block's tile");
        // A block's range is shorter than one tile (the host takes this form
        // only then), so it holds at most two pieces: k = 0 is the range's
        // last tile, k = 1 the one before.  Each piece recomputes the block's
        // range from an opaque copy of the block index, so that none of it is
        // held in registers across the K loop.
        struct Range {
            int xcd, jb, nbx, ts, klo, khi, mt, nt;
            long long sx;
            bool live;
        };
        auto range = [&](int k) {
            int bid = (int)blockIdx.x;
            asm volatile("" : "+s"(bid));
            Range r;
            r.xcd = bid & 7, r.jb = bid >> 3, r.nbx = (int)gridDim.x >> 3;
            const int ntiles = ntm * ntn;
            const int t_lo = (int)((long long)ntiles * r.xcd / 8), t_hi = (int)((long long)ntiles * (r.xcd + 1) / 8);
            r.sx = (long long)(t_hi - t_lo) * nk;  // K steps of this XCD's tiles
            const int s0 = (int)(r.sx * r.jb / r.nbx), s1 = (int)(r.sx * (r.jb + 1) / r.nbx);
            const int tl = (s1 - 1) / nk - k;
            r.live = s0 < s1 && tl >= s0 / nk;
            r.ts = tl * nk;
            r.klo = max(s0, r.ts) - r.ts, r.khi = min(s1, r.ts + nk) - r.ts;
            const int t = t_lo + tl;
            r.mt = t / ntn, r.nt = t - r.mt * ntn;
            return r;
        };
        for (int k = 0; k < 2; ++k) {
            {
                const Range r = range(k);
                if (!r.live) return;  // no (more) steps for this block
                if (k > 0) __syncthreads();  // the previous piece's epilogue no longer reads the stages
                int tid = threadIdx.x;
                asm volatile("" : "+v"(tid));  // opaque per piece: nothing derived from it leaves the loop body
                piece(tid, r.mt, r.nt, r.klo, r.khi);
            }
            // The range once more, rather than held across the K loop.
            const Range r = range(k);
            const int xcd = r.xcd, jb = r.jb, ts = r.ts, klo = r.klo, khi = r.khi, mt = r.mt, nt = r.nt;
            auto sbeg = [&](int j) { return (int)(r.sx * j / r.nbx); };
            int tid = threadIdx.x;
            asm volatile("" : "+v"(tid));
            const __amdgpu_buffer_rsrc_t p_rsrc = make_rsrc(A.skp, (uint32_t)(kSkBlocks * kSkSlotBytes));
            if (klo > 0 && khi == nk) {
                // Steps [0, klo) of the tile are held by blocks jf .. jb-1 of
                // this XCD (those with steps at all): wait for their flags,
                // then add their sums in block order.
                int jf = jb;
                while (jf > 0 && sbeg(jf) > ts) --jf;
                __shared__ int sk_late;  // a wait ran out: the tile is written as NaN, not silently wrong
                if (tid == 0) {
                    int late = 0;
                    for (int j = jf; j < jb; ++j) {
                        if (sbeg(j) >= sbeg(j + 1)) continue;
                        const uint32_t *f = &A.skf[xcd + 8 * j];
                        int it = 0;
                        for (; it < kSkSpinMax; ++it) {
                            if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) break;
                            __builtin_amdgcn_s_sleep(8);
                        }
                        if (it == kSkSpinMax) late = 1;
                    }
                    sk_late = late;
                }
                __syncthreads();
                if (sk_late) {
#pragma unroll
                    for (int ip = 0; ip < TP; ++ip)
#pragma unroll
                        for (int ic = 0; ic < TC; ++ic)
#pragma unroll
                            for (int e = 0; e < 4 * NQ; ++e) acc[ip][ic][e] = __builtin_nanf("");
                }
                for (int j = jf; j < jb; ++j) {
                    if (sbeg(j) >= sbeg(j + 1)) continue;
                    const uint32_t base = (uint32_t)(xcd + 8 * j) * (uint32_t)kSkSlotBytes;
                    // Half of the chunks in flight at a time.
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        float4 v[TP / 2][TC][NQ];
#pragma unroll
                        for (int ip = 0; ip < TP / 2; ++ip)
#pragma unroll
                            for (int ic = 0; ic < TC; ++ic)
#pragma unroll
                                for (int q = 0; q < NQ; ++q) {
                                    const int c = ((h * TP / 2 + ip) * TC + ic) * NQ + q;
                                    v[ip][ic][q] = __builtin_bit_cast(
                                        float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    p_rsrc, (int)(base + (uint32_t)(c * NTHR + tid) * 16u), 0,
                                                    kCachePolicySc1));
                                }
#pragma unroll
                        for (int ip = 0; ip < TP / 2; ++ip)
#pragma unroll
                            for (int ic = 0; ic < TC; ++ic)
#pragma unroll
                                for (int q = 0; q < NQ; ++q) {
                                    auto &a = acc[h * TP / 2 + ip][ic];
                                    a[4 * q] += v[ip][ic][q].x;
                                    a[4 * q + 1] += v[ip][ic][q].y;
                                    a[4 * q + 2] += v[ip][ic][q].z;
                                    a[4 * q + 3] += v[ip][ic][q].w;
                                }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
            if (khi < nk) {
                // Not the tile's last step: the sums go to this block's slot.
                const uint32_t base = (uint32_t)blockIdx.x * (uint32_t)kSkSlotBytes;
#pragma unroll
                for (int ip = 0; ip < TP; ++ip)
#pragma unroll
                    for (int ic = 0; ic < TC; ++ic)
#pragma unroll
                        for (int q = 0; q < NQ; ++q) {
                            const int c = (ip * TC + ic) * NQ + q;
                            const float4 v = make_float4(acc[ip][ic][4 * q], acc[ip][ic][4 * q + 1],
                                                         acc[ip][ic][4 * q + 2], acc[ip][ic][4 * q + 3]);
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32_t, v), p_rsrc,
                                                                   (int)(base + (uint32_t)(c * NTHR + tid) * 16u), 0,
                                                                   kCachePolicySc1);
                        }
                CONVLOWER_WAIT_VMCNT(0);  // every wavefront's stores have completed
                __syncthreads();
                if (tid == 0) __hip_atomic_store(&A.skf[blockIdx.x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
                finish(tid, mt, nt);
            }
        }
    }
}

template <typename S, bool OUT_NCHW, bool SK = false>
__global__ __launch_bounds__(512, 1) void igemm_rowwin_pp_kernel(GemmArgs A) {
    igemm_rowwin_pp_body<S, OUT_NCHW, RowWinPPCfg<S, 3>, SK>(A);
}

}  // namespace convlower
