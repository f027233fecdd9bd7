// The main loop for feeds whose X_col rows are read in 16-byte chunks (the
// indirection buffer over channels-last input, the window-ordered tensor, and
// the plain-GEMM shapes): global memory is copied straight into LDS by the
// buffer-load-to-LDS instructions of gfx950, three K tiles in flight.
//
//   * A K tile of the block (BM rows of X_col and BN rows of W_row, BK values
//     each, 128 bytes per row) is one LDS stage.  Each of the four
//     wavefronts issues its share of the stage as 64-lane loads of 16 bytes;
//     lane L of a load lands in LDS slot base + L, so the stage layout is
//     chosen slot by slot: slot s holds chunk (s % 8) ^ (row % 8) of row
//     s / 8.  The XOR keeps a wavefront's 16-lane fragment reads (16 rows,
//     one chunk column) on distinct banks, and because every load covers 8
//     whole rows starting at a multiple of 8, each lane always fetches the
//     same chunk column -- one (tap, channel) position per lane.
//   * Three stages.  During tile k
//     the loads of tile k+3 are issued into the stage tile k came from, so
//     two tiles of MFMA work cover their latency.  Before the barrier in
//     tile k every wavefront waits (vmcnt) for its own loads of tile k+1 and
//     (lgkmcnt) for its own reads of the stage about to be refilled; after
//     it, all of tile k+1 is in LDS and nobody still reads that stage.  Out-of-range rows, padding taps
//     and tiles past the end read as zeros (buffer range check), so every
//     load is issued unconditionally.
//   * Each tile's MFMA steps are split around the barrier, the load issue
//     and the LDS reads of the next tile's fragments (one register slot per
//     MFMA K step), so the matrix pipe keeps running through them.
//   * The epilogue adds the bias in fp32, rounds once, and stores straight
//     from the accumulators: each lane's four accumulator rows run along the
//     output's contiguous axis, so they leave as one 8-byte (bf16) or
//     16-byte (fp32) store.
#pragma once

namespace convlower {

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define CONVLOWER_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt((((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14)))
// ... and also every LDS access of this wavefront complete (lgkmcnt 0).
#define CONVLOWER_WAIT_VMCNT_LDS(n) \
    __builtin_amdgcn_s_waitcnt((((n) & 15) | (7 << 4) | (0 << 8) | (((n) >> 4) << 14)))
// Only every LDS access of this wavefront complete (vmcnt left at its maximum, 63).
#define CONVLOWER_WAIT_LDS() CONVLOWER_WAIT_VMCNT_LDS(63)

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// One 64-lane buffer load of 16 bytes per lane straight into LDS: lane L's
// data lands at LDS byte address lds_base + 16*L (M0 holds lds_base).  Issued
// as inline assembly so that the compiler neither tracks nor waits for these
// loads itself -- its per-object tracking of such loads degrades to "wait for
// everything" where control flow merges, which would drain the pipeline.
// All waits for them are the explicit vmcnt waits in the main loop.  M0 is
// used by nothing else in these kernels (LDS instructions on gfx9 and later
// do not read it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Workgroup barrier that is also a compiler barrier for memory accesses (the
// s_barrier builtin alone does not stop LDS reads from moving across it).
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// MFMA shapes.  For both, an operand fragment is one 16-byte chunk per
// lane: lane L holds row L % MT of the operand's tile and chunk L / MT of
// each MFMA K step (CPG chunks per step); A-side and B-side fragments use the
// same lane-to-K mapping, so each MFMA sums over exactly the K values of its
// step.  The result tile: lane L holds column L % MT and, for q < NQ, the 4
// consecutive rows qrow(q, L) .. +3 in accumulator elements 4q .. 4q+3.
template <typename S, int MT_>
struct MfmaShape;
template <>
struct MfmaShape<uint16_t, 16> {  // v_mfma_f32_16x16x32_bf16
    static constexpr int MT = 16, CPG = 4, NQ = 1, QSTEP = 16;
    typedef f32x4_t acc_t;
    __device__ static __forceinline__ int qrow(int, int lane) { return 4 * (lane >> 4); }
    __device__ static __forceinline__ void mma(const uint4 &a, const uint4 &b, acc_t &c) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
};
template <>
struct MfmaShape<uint16_t, 32> {  // v_mfma_f32_32x32x16_bf16
    static constexpr int MT = 32, CPG = 2, NQ = 4, QSTEP = 8;
    typedef f32x16_t acc_t;
    __device__ static __forceinline__ int qrow(int q, int lane) { return 8 * q + 4 * (lane >> 5); }
    __device__ static __forceinline__ void mma(const uint4 &a, const uint4 &b, acc_t &c) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
};
template <>
struct MfmaShape<_Float16, 16> {  // v_mfma_f32_16x16x32_f16
    static constexpr int MT = 16, CPG = 4, NQ = 1, QSTEP = 16;
    typedef f32x4_t acc_t;
    __device__ static __forceinline__ int qrow(int, int lane) { return 4 * (lane >> 4); }
    __device__ static __forceinline__ void mma(const uint4 &a, const uint4 &b, acc_t &c) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
};
template <>
struct MfmaShape<_Float16, 32> {  // v_mfma_f32_32x32x16_f16
    static constexpr int MT = 32, CPG = 2, NQ = 4, QSTEP = 8;
    typedef f32x16_t acc_t;
    __device__ static __forceinline__ int qrow(int q, int lane) { return 8 * q + 4 * (lane >> 5); }
    __device__ static __forceinline__ void mma(const uint4 &a, const uint4 &b, acc_t &c) {
        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
};
template <>
struct MfmaShape<float, 16> {  // v_mfma_f32_16x16x4_f32, four per 16-byte chunk
    static constexpr int MT = 16, CPG = 4, NQ = 1, QSTEP = 16;
    typedef f32x4_t acc_t;
    __device__ static __forceinline__ int qrow(int, int lane) { return 4 * (lane >> 4); }
    __device__ static __forceinline__ void mma(const uint4 &a, const uint4 &b, acc_t &c) {
        f32x4_t x = __builtin_bit_cast(f32x4_t, a), y = __builtin_bit_cast(f32x4_t, b);
#pragma unroll
        for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(x[j], y[j], c, 0, 0, 0);
    }
};
template <>
struct MfmaShape<float, 32> {  // v_mfma_f32_32x32x2_f32, four per 16-byte chunk
    static constexpr int MT = 32, CPG = 2, NQ = 4, QSTEP = 8;
    typedef f32x16_t acc_t;
    __device__ static __forceinline__ int qrow(int q, int lane) { return 8 * q + 4 * (lane >> 5); }
    __device__ static __forceinline__ void mma(const uint4 &a, const uint4 &b, acc_t &c) {
        f32x4_t x = __builtin_bit_cast(f32x4_t, a), y = __builtin_bit_cast(f32x4_t, b);
#pragma unroll
        for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(x[j], y[j], c, 0, 0, 0);
    }
};

template <>
struct MfmaShape<uint8_t, 32> {  // v_mfma_f32_32x32x16_fp8_fp8 (OCP e4m3 on gfx950), two per 16-byte chunk
    static constexpr int MT = 32, CPG = 2, NQ = 4, QSTEP = 8;
    typedef f32x16_t acc_t;
    __device__ static __forceinline__ int qrow(int q, int lane) { return 8 * q + 4 * (lane >> 5); }
    __device__ static __forceinline__ void mma(const uint4 &a, const uint4 &b, acc_t &c) {
        const long a0 = (long)(((unsigned long)a.y << 32) | a.x), a1 = (long)(((unsigned long)a.w << 32) | a.z);
        const long b0 = (long)(((unsigned long)b.y << 32) | b.x), b1 = (long)(((unsigned long)b.w << 32) | b.z);
        c = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a0, b0, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a1, b1, c, 0, 0, 0);
    }
};

// Four consecutive outputs, rounded once, in one 8-byte (bf16) or 16-byte
// (fp32) store; the address must be aligned to that size.
__device__ __forceinline__ void store4(uint16_t *p, float a, float b, float c, float d) {
    uint2 pk;
    pk.x = f32x2_to_bf16x2_rne(a, b);
    pk.y = f32x2_to_bf16x2_rne(c, d);
    *(uint2 *)p = pk;
}
__device__ __forceinline__ void store4(_Float16 *p, float a, float b, float c, float d) {
    uint2 pk;
    pk.x = f32x2_to_f16x2_rne(a, b);
    pk.y = f32x2_to_f16x2_rne(c, d);
    *(uint2 *)p = pk;
}
__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d) {
    *(float4 *)p = make_float4(a, b, c, d);
}

// The body is a device function so that only the device compilation ever
// instantiates it; the kernel below is a thin entry point.
template <typename S, int FEED, bool OUT_NCHW, int BM, int BN, int BK>
__device__ __forceinline__ void igemm_dma_body(const GemmArgs &A) {
    using C = TileCfg<S, BM, BN, BK>;
    constexpr int VEC = C::VEC, KCH = C::KCH;
    constexpr int WPM = C::WPM, WCN = C::WCN;
    // MFMA shape: 32x32 output tiles wherever the wavefront tile allows (the
    // 32x32 instructions sustain about 2.5x the rate of the 16x16 ones from
    // one wavefront per SIMD), else 16x16.
    using MF = MfmaShape<S, (WPM % 32 == 0 && WCN % 32 == 0) ? 32 : 16>;
    constexpr int MT = MF::MT;
    constexpr int TP = WPM / MT, TC = WCN / MT;
    constexpr int NQ = MF::NQ;  // groups of 4 consecutive accumulator rows per lane
    constexpr int NSLOT = (BM + BN) * KCH;  // 16-byte slots per stage
    constexpr int NINST = NSLOT / 64;       // 64-lane loads per stage
    constexpr int IPW = NINST / 4;          // per wavefront
    constexpr int A_INST = BM * KCH / 64;   // loads that fill the A rows
    constexpr bool IND = FEED == FEED_IND_NHWC;
    static_assert(KCH == 8, "stage rows are 128 bytes");
    static_assert(NINST % 4 == 0 && (BM * KCH) % 64 == 0, "loads must split evenly");
    static_assert(2 * IPW <= 63, "vmcnt budget");

    __shared__ uint4 st0[NSLOT];
    __shared__ uint4 st1[NSLOT];
    __shared__ uint4 st2[NSLOT];
    __shared__ int ib_lds[IND ? kIbufLdsEntries : 1];

    const Geom &g = A.g;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;

    int mt, nt;
    tile_coords((int)((g.M + BM - 1) / BM), (g.Co + BN - 1) / BN, mt, nt);
    const long long m0 = (long long)mt * BM;
    const int co0 = nt * BN;
    const int kbeg = blockIdx.z * A.k_per_split;
    const int kend = (int)min((long long)kbeg + A.k_per_split, g.K);
    const int nk = (kend - kbeg + BK - 1) / BK;

    if constexpr (IND) {
        // Loads are issued unconditionally (rows past M read row M-1 and are
        // then marked as padding) so they all overlap.
        for (int e = tid; e < BM * g.T; e += kThreads) {
            int row = e / g.T, t = e - row * g.T;
            long long m = m0 + row;
            long long mc = m < g.M ? m : g.M - 1;
            long long n = mc / g.P;
            int v = A.ibuf[(int)(mc - n * g.P) * g.T + t];
            ib_lds[e] = m < g.M ? v : -1;
        }
    }

    // This lane's chunk column and the rows its IPW loads cover.  Load q of
    // the stage goes to wavefront q % 4, so every wavefront issues the same
    // mix of A and B loads; load i of this wavefront covers rows
    // (i*4 + wave)*8 .. +7 of the stage, this lane row (i*4 + wave)*8 + lane/8.
    // Rows outside the tensors get an offset at or past 2^31, which stays out
    // of range whatever in-row offset is added.
    const int kc = ((lane & 7) ^ (lane >> 3)) * VEC;
    const int row0 = wave * 8 + (lane >> 3);  // row of load 0; load i adds 32*i
    uint32_t rbase[IPW];  // byte offset of the row's origin (A: feed origin; B: row of W_row)
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int q = i * 4 + wave;
        const int row = row0 + 32 * i;
        if (q < A_INST) {
            ARow r = make_arow<FEED>(g, m0 + row);
            rbase[i] = r.ok ? (uint32_t)(r.base * (long long)sizeof(S)) : kOutOfRange;
        } else {
            const int co = co0 + row - BM;
            rbase[i] = co < g.Co ? (uint32_t)((long long)co * g.K * (long long)sizeof(S)) : kOutOfRange;
        }
    }

    int cur_t = 0, cur_ci = 0, cur_kh = 0, cur_kw = 0;
    if constexpr (FEED == FEED_IND_NHWC || FEED == FEED_WIN) {
        const int k0 = kbeg + kc;
        cur_t = k0 / g.C;
        cur_ci = k0 - cur_t * g.C;
        cur_kh = cur_t / g.KW;
        cur_kw = cur_t - cur_kh * g.KW;
    }

    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A.a_src, A.a_bytes);
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(A.b, A.b_bytes);
    constexpr long long ES = sizeof(S);

    __syncthreads();  // ib_lds ready

    // Issue the loads of the K tile starting at kt0 into stage `st`: all
    // offsets first (one batch of indirection-buffer reads from LDS), then
    // the loads.
    auto issue = [&](int kt0, uint4 *st) {
        const int k0 = kt0 + kc;
        const bool kin = k0 < kend;
        uint32_t aoff = 0;  // byte offset within the row for the A loads
        if constexpr (FEED == FEED_ROWMAJOR) aoff = (uint32_t)k0 * (uint32_t)sizeof(S);
        if constexpr (FEED == FEED_IND_NHWC) aoff = (uint32_t)cur_ci * (uint32_t)sizeof(S);
        if constexpr (FEED == FEED_WIN)
            aoff = (uint32_t)((cur_kw * g.d * g.KH + cur_kh) * g.C + cur_ci) * (uint32_t)sizeof(S);
        const uint32_t boff = (uint32_t)k0 * (uint32_t)sizeof(S);
        int ib[IPW];
        if constexpr (IND) {
#pragma unroll
            for (int i = 0; i < IPW; ++i)
                ib[i] = (i * 4 + wave < A_INST) ? ib_lds[(row0 + 32 * i) * g.T + cur_t] : 0;
        }
        uint32_t voff[IPW];
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int q = i * 4 + wave;
            bool valid = kin;
            uint32_t o;
            if (q < A_INST) {
                o = rbase[i] + aoff;
                if constexpr (IND) {
                    valid = valid && ib[i] >= 0;
                    o += (uint32_t)ib[i] * (uint32_t)sizeof(S);
                }
            } else {
                o = rbase[i] + boff;
            }
            voff[i] = valid ? o : kOutOfRange;
        }
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int q = i * 4 + wave;
            const uint32_t dst = (uint32_t)(uintptr_t)(lds_ptr_t)(st + q * 64);
            if (q < A_INST)
                lds_dma16(a_rsrc, voff[i], dst);
            else
                lds_dma16(b_rsrc, voff[i], dst);
        }
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
    };

    typename MF::acc_t acc[TP][TC];
#pragma unroll
    for (int ip = 0; ip < TP; ++ip)
#pragma unroll
        for (int ic = 0; ic < TC; ++ic) acc[ip][ic] = typename MF::acc_t{};

    const int wp = wave >> 1, wc = wave & 1;
    // Fragment position of this lane: row (lane % MT) of a tile, chunk
    // (lane / MT) of each MFMA K step.  Result position: column (lane % MT),
    // rows MF::qrow(q, lane) + 0..3.
    const int frow = lane % MT, fchunk = lane / MT;

    // Bias values this lane adds in the epilogue, loaded once up front (the
    // output stores could alias the bias pointer, which would otherwise force
    // a reload after every store).  Every load is issued unconditionally
    // (clamped index), then selected.
    const S *bias = (const S *)A.bias;
    constexpr int NB = OUT_NCHW ? 1 : 4 * NQ;
    float bv[TC][NB];
#pragma unroll
    for (int ic = 0; ic < TC; ++ic)
#pragma unroll
        for (int e = 0; e < NB; ++e) {
            const int co = OUT_NCHW ? co0 + wc * WCN + ic * MT + frow
                                    : co0 + wc * WCN + ic * MT + MF::qrow(e >> 2, lane) + (e & 3);
            float val = 0.f;
            if (bias) val = bits_to_f32(S(), elem_bits(bias, co < g.Co ? co : g.Co - 1));
            bv[ic][e] = co < g.Co ? val : 0.f;
        }

    // MFMA fragments, one register slot per MFMA K step of a tile.  A slot
    // is refilled with the next tile's fragments as soon as this tile's MFMAs
    // for that step are issued, so LDS latency hides behind MFMA work.
    constexpr int NG = KCH / MF::CPG;  // MFMA K steps per tile
    uint4 fa[NG][TP], fb[NG][TC];
    auto lds_read = [&](const uint4 *st, int grp) {
        const uint4 *As = st;
        const uint4 *Bs = st + BM * KCH;
#pragma unroll
        for (int ip = 0; ip < TP; ++ip)
            fa[grp][ip] = As[lds_slot(wp * WPM + ip * MT + frow, grp * MF::CPG + fchunk, KCH)];
#pragma unroll
        for (int ic = 0; ic < TC; ++ic)
            fb[grp][ic] = Bs[lds_slot(wc * WCN + ic * MT + frow, grp * MF::CPG + fchunk, KCH)];
    };
    // D[rows][cols] += A-side * B-side; the operand order puts output pixels
    // on the rows for NCHW (each lane's 4 consecutive rows are 4 consecutive
    // pixels of one channel plane) and output channels on the rows for NHWC.
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
    // One K tile kt, whose fragments were read from stage st_cur.  The first
    // MFMA step runs while the wavefront waits for tile kt+1's loads and the
    // barrier; then st_cur (no longer read by anyone) receives tile kt+3 and
    // tile kt+1's fragments are read from st_next, each slot right after
    // its MFMAs for tile kt are issued.
    // sched_barrier(0) pins this order: left to itself the scheduler clusters
    // the MFMAs and sinks every fragment read to the end of the tile, where
    // their latency is exposed at the start of the next one.
    auto phase = [&](int kt, uint4 *st_cur, const uint4 *st_next) {
        mfma_group(0);
        __builtin_amdgcn_sched_barrier(0);
        // Before the barrier: this wavefront's loads of tile kt+1 have landed,
        // and its reads of st_cur have completed (st_cur is refilled right
        // after the barrier; loads of tiles past the end return almost at once).
        CONVLOWER_WAIT_VMCNT_LDS(IPW);
        block_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(kbeg + (kt + 3) * BK, st_cur);
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
    };

    if (nk > 0) {
        issue(kbeg, st0);
        issue(kbeg + BK, st1);
        issue(kbeg + 2 * BK, st2);
        CONVLOWER_WAIT_VMCNT(2 * IPW);
        block_barrier();
#pragma unroll
        for (int grp = 0; grp < NG; ++grp) lds_read(st0, grp);
        // Tiles past the end load as zeros into stages no one reads, so every
        // phase issues the same loads and each wait covers exactly one tile.
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

    // ---- epilogue ------------------------------------------------------------
    S *y = (S *)A.y;
    if constexpr (OUT_NCHW) {
        // Rows are pixels: this lane's rows are m = m0 + wp*WPM + ip*MT +
        // qrow(q) + v, visited in increasing order with a fixed step, so the
        // (image, pixel) position advances incrementally instead of dividing.
        constexpr int STEP = MF::QSTEP;
        int m = (int)(m0 + wp * WPM + MF::qrow(0, lane));
        int n = m / g.P;
        int p = m - n * g.P;
#pragma unroll
        for (int ip = 0; ip < TP; ++ip) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                if (m < g.M) {
#pragma unroll
                    for (int ic = 0; ic < TC; ++ic) {
                        const int co = co0 + wc * WCN + ic * MT + frow;
                        if (co >= g.Co) continue;
                        const float a4[4] = {acc[ip][ic][4 * q], acc[ip][ic][4 * q + 1], acc[ip][ic][4 * q + 2], acc[ip][ic][4 * q + 3]};
                        if (A.part) {
                            for (int v = 0; v < 4 && m + v < g.M; ++v)
                                A.part[((long long)blockIdx.z * g.M + m + v) * g.Co + co] = a4[v];
                            continue;
                        }
                        const float b = bv[ic][0];
                        const long long yi = ((long long)n * g.Co + co) * g.P + p;
                        if (p + 4 <= g.P && m + 4 <= g.M && ((uintptr_t)(y + yi) % (4 * sizeof(S))) == 0) {
                            store4(y + yi, a4[0] + b, a4[1] + b, a4[2] + b, a4[3] + b);
                        } else {
                            int nv = n, pv = p;
                            for (int v = 0; v < 4 && m + v < g.M; ++v) {
                                y[((long long)nv * g.Co + co) * g.P + pv] = to_out(S(), a4[v] + b);
                                if (++pv == g.P) {
                                    pv = 0;
                                    ++nv;
                                }
                            }
                        }
                    }
                }
                m += STEP;
                p += STEP;
                while (p >= g.P) {
                    p -= g.P;
                    ++n;
                }
            }
        }
    } else {
        // Rows are output channels: each lane's 4 consecutive rows are 4
        // consecutive channels of one output pixel.
#pragma unroll
        for (int ip = 0; ip < TP; ++ip) {
            const long long m = m0 + wp * WPM + ip * MT + frow;
            if (m >= g.M) continue;
#pragma unroll
            for (int ic = 0; ic < TC; ++ic) {
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const int co = co0 + wc * WCN + ic * MT + MF::qrow(q, lane);
                    if (co >= g.Co) continue;
                    const float a4[4] = {acc[ip][ic][4 * q], acc[ip][ic][4 * q + 1], acc[ip][ic][4 * q + 2], acc[ip][ic][4 * q + 3]};
                    if (A.part) {
                        for (int v = 0; v < 4 && co + v < g.Co; ++v)
                            A.part[((long long)blockIdx.z * g.M + m) * g.Co + co + v] = a4[v];
                        continue;
                    }
                    const float *b = &bv[ic][4 * q];
                    const long long yi = m * g.Co + co;
                    if (co + 4 <= g.Co && ((uintptr_t)(y + yi) % (4 * sizeof(S))) == 0) {
                        store4(y + yi, a4[0] + b[0], a4[1] + b[1], a4[2] + b[2], a4[3] + b[3]);
                    } else {
                        for (int v = 0; v < 4 && co + v < g.Co; ++v) y[yi + v] = to_out(S(), a4[v] + b[v]);
                    }
                }
            }
        }
    }
}

template <typename S, int FEED, bool OUT_NCHW, int BM, int BN, int BK>
__global__ __launch_bounds__(kThreads) void igemm_dma_kernel(GemmArgs A) {
    igemm_dma_body<S, FEED, OUT_NCHW, BM, BN, BK>(A);
}

}  // namespace convlower
