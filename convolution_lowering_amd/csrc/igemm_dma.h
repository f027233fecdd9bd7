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
//   * Three stages, each its own LDS object: the loads for tile k+2 are
//     issued right after the barrier that opens tile k, so two tiles of
//     MFMA work cover their latency.  Before that barrier every wavefront
//     waits (vmcnt) for its own loads of tile k; after it, all of tile k is
//     in LDS.  Out-of-range rows, padding taps and tiles past the end read
//     as zeros (buffer range check), so every load is issued unconditionally.
//   * The epilogue adds the bias in fp32, rounds once, and stores straight
//     from the accumulators: each lane's four accumulator rows run along the
//     output's contiguous axis, so they leave as one 8-byte (bf16) or
//     16-byte (fp32) store.
#pragma once

namespace convlower {

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define CONVLOWER_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt((((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14)))

typedef __attribute__((address_space(3))) void *lds_ptr_t;

template <typename S, int FEED, bool OUT_NCHW, int BM, int BN, int BK>
__global__ __launch_bounds__(kThreads) void igemm_dma_kernel(GemmArgs A) {
    using C = TileCfg<S, BM, BN, BK>;
    constexpr int VEC = C::VEC, KCH = C::KCH;
    constexpr int WPM = C::WPM, WCN = C::WCN, TP = C::TP, TC = C::TC;
    constexpr int NSLOT = (BM + BN) * KCH;  // 16-byte slots per stage
    constexpr int NINST = NSLOT / 64;       // 64-lane loads per stage
    constexpr int IPW = NINST / 4;          // per wavefront
    constexpr int A_INST = BM * KCH / 64;   // loads that fill the A rows
    constexpr bool IND = FEED == FEED_IND_NHWC;
    static_assert(KCH == 8, "stage rows are 128 bytes");
    static_assert(NINST % 4 == 0 && (BM * KCH) % 64 == 0, "loads must split evenly");
    static_assert(IPW <= 15, "vmcnt budget");

    __shared__ uint4 st0[NSLOT];
    __shared__ uint4 st1[NSLOT];
    __shared__ uint4 st2[NSLOT];
    __shared__ int ib_lds[IND ? kIbufLdsEntries : 1];

    const Geom &g = A.g;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;

    int bx = blockIdx.x;
    const int nbx = gridDim.x;
    if ((nbx & 7) == 0) bx = (bx & 7) * (nbx >> 3) + (bx >> 3);
    const long long m0 = (long long)bx * BM;
    const int co0 = blockIdx.y * BN;
    const int kbeg = blockIdx.z * A.k_per_split;
    const int kend = (int)min((long long)kbeg + A.k_per_split, g.K);
    const int nk = (kend - kbeg + BK - 1) / BK;

    if constexpr (IND) {
        for (int e = tid; e < BM * g.T; e += kThreads) {
            int row = e / g.T, t = e - row * g.T;
            long long m = m0 + row;
            int v = -1;
            if (m < g.M) {
                long long n = m / g.P;
                v = A.ibuf[(int)(m - n * g.P) * g.T + t];
            }
            ib_lds[e] = v;
        }
    }

    // This lane's chunk column and the rows its IPW loads cover.
    const int kc = ((lane & 7) ^ (lane >> 3)) * VEC;
    long long rbase[IPW];  // A: feed origin of the row; B: row offset in W_row
    int rrow[IPW];         // A: row within the block's A tile
    bool rok[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int q = wave * IPW + i;
        const int row = q * 8 + (lane >> 3);
        if (q < A_INST) {
            ARow r = make_arow<FEED>(g, m0 + row);
            rbase[i] = r.base;
            rok[i] = r.ok;
            rrow[i] = row;
        } else {
            const int co = co0 + row - BM;
            rok[i] = co < g.Co;
            rbase[i] = (long long)(rok[i] ? co : 0) * g.K;
            rrow[i] = 0;
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

    // Issue the loads of the K tile starting at kt0 into stage `st`.
    auto issue = [&](int kt0, uint4 *st) {
        const int k0 = kt0 + kc;
        const bool kin = k0 < kend;
        long long koff = 0;
        if constexpr (FEED == FEED_ROWMAJOR) koff = k0;
        if constexpr (FEED == FEED_IND_NHWC) koff = cur_ci;
        if constexpr (FEED == FEED_WIN) koff = (long long)(cur_kw * g.d * g.KH + cur_kh) * g.C + cur_ci;
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int q = wave * IPW + i;
            lds_ptr_t dst = (lds_ptr_t)(st + q * 64);
            if (q < A_INST) {
                bool valid = rok[i] && kin;
                long long addr = rbase[i] + koff;
                if constexpr (IND) {
                    int off = ib_lds[rrow[i] * g.T + cur_t];
                    valid = valid && off >= 0;
                    addr += off;
                }
                uint32_t voff = valid ? (uint32_t)(addr * ES) : kOutOfRange;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, dst, 16, voff, 0, 0, 0);
            } else {
                bool valid = rok[i] && kin;
                uint32_t voff = valid ? (uint32_t)((rbase[i] + k0) * ES) : kOutOfRange;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, dst, 16, voff, 0, 0, 0);
            }
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

    f32x4_t acc[TP][TC];
#pragma unroll
    for (int ip = 0; ip < TP; ++ip)
#pragma unroll
        for (int ic = 0; ic < TC; ++ic) acc[ip][ic] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int wp = wave >> 1, wc = wave & 1;
    const int frow = lane & 15, fchunk = lane >> 4;

    auto compute = [&](const uint4 *st) {
        const uint4 *As = st;
        const uint4 *Bs = st + BM * KCH;
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
        issue(kbeg, st0);
        issue(kbeg + BK, st1);
        for (int kt = 0;; kt += 3) {
            CONVLOWER_WAIT_VMCNT(IPW);  // this wavefront's loads of tile kt are in LDS
            __builtin_amdgcn_s_barrier();
            issue(kbeg + (kt + 2) * BK, st2);
            compute(st0);
            if (kt + 1 >= nk) break;
            CONVLOWER_WAIT_VMCNT(IPW);
            __builtin_amdgcn_s_barrier();
            issue(kbeg + (kt + 3) * BK, st0);
            compute(st1);
            if (kt + 2 >= nk) break;
            CONVLOWER_WAIT_VMCNT(IPW);
            __builtin_amdgcn_s_barrier();
            issue(kbeg + (kt + 4) * BK, st1);
            compute(st2);
            if (kt + 3 >= nk) break;
        }
        CONVLOWER_WAIT_VMCNT(0);  // no load may still write LDS when the block ends
    }

    // ---- epilogue: lane holds column (lane & 15), rows 4*(lane >> 4) + v ----
    const S *bias = (const S *)A.bias;
    S *y = (S *)A.y;
#pragma unroll
    for (int ip = 0; ip < TP; ++ip) {
#pragma unroll
        for (int ic = 0; ic < TC; ++ic) {
            if constexpr (OUT_NCHW) {
                const long long m = m0 + wp * WPM + ip * 16 + 4 * fchunk;  // 4 consecutive pixels
                const int co = co0 + wc * WCN + ic * 16 + frow;
                if (m >= g.M || co >= g.Co) continue;
                if (A.part) {
                    for (int v = 0; v < 4 && m + v < g.M; ++v)
                        A.part[((long long)blockIdx.z * g.M + m + v) * g.Co + co] = acc[ip][ic][v];
                    continue;
                }
                const float b = bias ? bits_to_f32(S(), elem_bits(bias, co)) : 0.f;
                const long long n = m / g.P;
                const long long p = m - n * g.P;
                const long long yi = (n * g.Co + co) * g.P + p;
                if (p + 4 <= g.P && m + 4 <= g.M && ((uintptr_t)(y + yi) % (4 * sizeof(S))) == 0) {
                    if constexpr (sizeof(S) == 2) {
                        uint2 pk;
                        pk.x = (uint32_t)f32_to_bf16_rne(acc[ip][ic][0] + b) |
                               ((uint32_t)f32_to_bf16_rne(acc[ip][ic][1] + b) << 16);
                        pk.y = (uint32_t)f32_to_bf16_rne(acc[ip][ic][2] + b) |
                               ((uint32_t)f32_to_bf16_rne(acc[ip][ic][3] + b) << 16);
                        *(uint2 *)(y + yi) = pk;
                    } else {
                        *(float4 *)(y + yi) = make_float4(acc[ip][ic][0] + b, acc[ip][ic][1] + b,
                                                          acc[ip][ic][2] + b, acc[ip][ic][3] + b);
                    }
                } else {
                    for (int v = 0; v < 4; ++v) {
                        const long long mv = m + v;
                        if (mv >= g.M) break;
                        const long long nv = mv / g.P;
                        y[(nv * g.Co + co) * g.P + (mv - nv * g.P)] = to_out(S(), acc[ip][ic][v] + b);
                    }
                }
            } else {
                const long long m = m0 + wp * WPM + ip * 16 + frow;
                const int co = co0 + wc * WCN + ic * 16 + 4 * fchunk;  // 4 consecutive channels
                if (m >= g.M || co >= g.Co) continue;
                if (A.part) {
                    for (int v = 0; v < 4 && co + v < g.Co; ++v)
                        A.part[((long long)blockIdx.z * g.M + m) * g.Co + co + v] = acc[ip][ic][v];
                    continue;
                }
                float b[4];
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    b[v] = (bias && co + v < g.Co) ? bits_to_f32(S(), elem_bits(bias, co + v)) : 0.f;
                const long long yi = m * g.Co + co;
                if (co + 4 <= g.Co && ((uintptr_t)(y + yi) % (4 * sizeof(S))) == 0) {
                    if constexpr (sizeof(S) == 2) {
                        uint2 pk;
                        pk.x = (uint32_t)f32_to_bf16_rne(acc[ip][ic][0] + b[0]) |
                               ((uint32_t)f32_to_bf16_rne(acc[ip][ic][1] + b[1]) << 16);
                        pk.y = (uint32_t)f32_to_bf16_rne(acc[ip][ic][2] + b[2]) |
                               ((uint32_t)f32_to_bf16_rne(acc[ip][ic][3] + b[3]) << 16);
                        *(uint2 *)(y + yi) = pk;
                    } else {
                        *(float4 *)(y + yi) = make_float4(acc[ip][ic][0] + b[0], acc[ip][ic][1] + b[1],
                                                          acc[ip][ic][2] + b[2], acc[ip][ic][3] + b[3]);
                    }
                } else {
                    for (int v = 0; v < 4 && co + v < g.Co; ++v) y[yi + v] = to_out(S(), acc[ip][ic][v] + b[v]);
                }
            }
        }
    }
}

}  // namespace convlower
