// A plain implicit-GEMM main loop whose techniques can be switched off one
// at a time, for the ablation that "Im2win: An Efficient Convolution
// Paradigm on GPU" (abstract) reports for its own kernel: shared memory,
// tiling, the micro-kernel, double buffering and prefetching.
//
// The feed is the indirection buffer over channels-last input (The Indirect
// Convolution Algorithm, abstract): K tiles of 32 channels of one tap, so K
// runs (kh, kw, ci) as the OHWI weights do.  A block of four wavefronts owns
// a 128 x 128 tile of Y_col (wavefront tiles 64 x 64), or, for the tiling
// switch, one wavefront owns a 64 x 64 tile alone.  All variants share the
// loads (16 bytes per lane, through buffer descriptors whose range check
// turns padding taps and rows past M into zeros) and one epilogue (bias in
// fp32, one rounding, an element store per output), so they differ only in
// the technique switched:
//   * USE_LDS   the tile is staged in LDS (16-byte chunks XOR-swizzled by
//               row) and each wavefront reads its fragments there; without
//               it every wavefront loads its own fragments from global
//               memory, two tiles' worth in registers;
//   * STAGES    two LDS stages (one barrier per tile: tile k+1 is written
//               into the stage tile k-1 used) or one (a barrier before the
//               write, as every wavefront must be done reading);
//   * PREFETCH  tile k+1's global loads issued before tile k's MFMAs (their
//               latency hidden behind them) or after;
//   * MICRO     v_mfma_f32_32x32x16 (2 x 2 tiles per wavefront), 16x16x32
//               (4 x 4 tiles), or a VALU micro-kernel: each lane an 8 x 8
//               block of outputs by fp32 FMAs from LDS.
#pragma once

namespace convlower {

enum AblMicro : int { ABL_MFMA32 = 0, ABL_MFMA16 = 1, ABL_VALU = 2 };

template <typename S, bool OUT_NCHW, bool USE_LDS, int STAGES, bool PREFETCH, int MICRO, int BT>
__device__ __forceinline__ void igemm_ablate_body(const GemmArgs &A) {
    static_assert(sizeof(S) == 2, "16-bit element types");
    static_assert(BT == 128 || BT == 64, "block tiles 128 x 128 or 64 x 64");
    static_assert(USE_LDS || MICRO == ABL_MFMA32, "the no-LDS variant uses the 32x32 MFMA micro-kernel");
    constexpr int NT = BT == 128 ? 256 : 64;  // threads
    constexpr int KCH = 4;                     // 16-byte chunks per row: 32 channels
    constexpr int BK = 32;
    constexpr int CPT = BT * KCH / NT;         // chunks per thread per operand
    constexpr int ROWS = 2 * BT;               // A rows, then B rows, per stage
    __shared__ uint4 st[USE_LDS ? STAGES : 1][USE_LDS ? ROWS * KCH : 1];

    const Geom &g = A.g;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = BT == 128 ? wave >> 1 : 0, wn = BT == 128 ? wave & 1 : 0;  // wavefront tile (64 x 64)
    int mt, nt;
    tile_coords((int)((g.M + BT - 1) / BT), (g.Co + BT - 1) / BT, mt, nt);
    const long long m0 = (long long)mt * BT;
    const int co0 = nt * BT;
    const int NS = g.C / BK, T = g.T;
    const int nk = NS * T;  // K tiles, (tap, slice) with the slice fastest
    const int HWC = g.H * g.W * g.C;
    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A.a_src, A.a_bytes);
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(A.b, A.b_bytes);

    // Byte offset of chunk ch of row `row` (A: pixel m0 + row; B: output
    // channel co0 + row) in K tile kt; kOutOfRange where it reads zeros.
    auto a_off = [&](int row, int ch, int kt) -> uint32_t {
        const long long m = m0 + row;
        if (m >= g.M) return kOutOfRange;
        const int t = kt / NS, s = kt - t * NS;
        const int n = (int)(m / g.P), p = (int)(m - (long long)n * g.P);
        const int off = A.ibuf[p * T + t];
        if (off < 0) return kOutOfRange;
        return (uint32_t)(n * HWC + off + s * BK + ch * 8) * 2u;
    };
    auto b_off = [&](int row, int ch, int kt) -> uint32_t {
        const int co = co0 + row;
        if (co >= g.Co) return kOutOfRange;
        const int t = kt / NS, s = kt - t * NS;
        return (uint32_t)((co * T + t) * g.C + s * BK + ch * 8) * 2u;
    };

    // Accumulators: MFMA32 2 x 2 tiles of f32x16; MFMA16 4 x 4 of f32x4;
    // VALU an 8 x 8 block of floats.
    using MF32 = MfmaShape<S, 32>;
    using MF16 = MfmaShape<S, 16>;
    typename MF32::acc_t acc32[2][2];
    typename MF16::acc_t acc16[4][4];
    float accv[MICRO == ABL_VALU ? 8 : 1][MICRO == ABL_VALU ? 8 : 1];
    if constexpr (MICRO == ABL_MFMA32) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc32[i][j] = typename MF32::acc_t{};
    } else if constexpr (MICRO == ABL_MFMA16) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc16[i][j] = typename MF16::acc_t{};
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) accv[i][j] = 0.f;
    }

    if constexpr (USE_LDS) {
        uint4 ra[CPT], rb[CPT];
        auto load = [&](int kt) {
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                const int id = tid + NT * j, row = id >> 2, ch = id & 3;
                ra[j] = buf_load16(a_rsrc, a_off(row, ch, kt));
                rb[j] = buf_load16(b_rsrc, b_off(row, ch, kt));
            }
        };
        auto store = [&](int stage) {
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                const int id = tid + NT * j, row = id >> 2, ch = id & 3;
                st[stage][dual_slot<KCH>(row, ch)] = ra[j];
                st[stage][dual_slot<KCH>(BT + row, ch)] = rb[j];
            }
        };
        auto compute = [&](int stage) {
            const uint4 *s = st[stage];
            const int arow = wm * 64, brow = BT + wn * 64;
            if constexpr (MICRO == ABL_MFMA32) {
#pragma unroll
                for (int grp = 0; grp < 2; ++grp) {
                    uint4 fa[2], fb[2];
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        fa[i] = s[dual_slot<KCH>(arow + i * 32 + (lane & 31), grp * 2 + (lane >> 5))];
                        fb[i] = s[dual_slot<KCH>(brow + i * 32 + (lane & 31), grp * 2 + (lane >> 5))];
                    }
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j) MF32::mma(fa[i], fb[j], acc32[i][j]);
                }
            } else if constexpr (MICRO == ABL_MFMA16) {
                uint4 fa[4], fb[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    fa[i] = s[dual_slot<KCH>(arow + i * 16 + (lane & 15), lane >> 4)];
                    fb[i] = s[dual_slot<KCH>(brow + i * 16 + (lane & 15), lane >> 4)];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) MF16::mma(fa[i], fb[j], acc16[i][j]);
            } else {
                const int r0 = arow + 8 * (lane >> 3), c0 = brow + 8 * (lane & 7);
#pragma unroll
                for (int ch = 0; ch < KCH; ++ch) {
                    float av[8][8], bv[8][8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const uint4 a = s[dual_slot<KCH>(r0 + i, ch)], b = s[dual_slot<KCH>(c0 + i, ch)];
                        const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            av[i][2 * k] = bits_to_f32(S(), aw[k] & 0xFFFFu);
                            av[i][2 * k + 1] = bits_to_f32(S(), aw[k] >> 16);
                            bv[i][2 * k] = bits_to_f32(S(), bw[k] & 0xFFFFu);
                            bv[i][2 * k + 1] = bits_to_f32(S(), bw[k] >> 16);
                        }
                    }
#pragma unroll
                    for (int k = 0; k < 8; ++k)
#pragma unroll
                        for (int i = 0; i < 8; ++i)
#pragma unroll
                            for (int j = 0; j < 8; ++j) accv[i][j] = __builtin_fmaf(av[i][k], bv[j][k], accv[i][j]);
                }
            }
        };

        if (nk > 0) {
            load(0);
            store(0);
            __syncthreads();
            for (int kt = 0; kt < nk; ++kt) {
                const int cur = STAGES == 2 ? (kt & 1) : 0;
                const bool more = kt + 1 < nk;
                if (PREFETCH && more) load(kt + 1);
                compute(cur);
                if (!PREFETCH && more) load(kt + 1);
                if (more) {
                    if (STAGES == 1) __syncthreads();  // every wavefront done reading the one stage
                    store(STAGES == 2 ? cur ^ 1 : 0);
                    __syncthreads();
                }
            }
        }
    } else {
        // No LDS: each lane loads the fragments it feeds to the MFMAs, for
        // tile k+1 while tile k is multiplied.
        uint4 fa[2][2][2], fb[2][2][2];  // [buffer][group][tile]
        auto load = [&](int kt, int buf) {
#pragma unroll
            for (int grp = 0; grp < 2; ++grp)
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int ch = grp * 2 + (lane >> 5);
                    fa[buf][grp][i] = buf_load16(a_rsrc, a_off(wm * 64 + i * 32 + (lane & 31), ch, kt));
                    fb[buf][grp][i] = buf_load16(b_rsrc, b_off(wn * 64 + i * 32 + (lane & 31), ch, kt));
                }
        };
        auto compute = [&](int buf) {
#pragma unroll
            for (int grp = 0; grp < 2; ++grp)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) MF32::mma(fa[buf][grp][i], fb[buf][grp][j], acc32[i][j]);
        };
        if (nk > 0) {
            load(0, 0);
            for (int kt = 0; kt < nk; kt += 2) {
                if (kt + 1 < nk) load(kt + 1, 1);
                compute(0);
                if (kt + 1 >= nk) break;
                if (kt + 2 < nk) load(kt + 2, 0);
                compute(1);
            }
        }
    }

    // Epilogue: the bias in fp32, one rounding, one store per output.
    S *y = (S *)A.y;
    auto put = [&](int row, int col, float v) {
        const long long m = m0 + row;
        const int co = co0 + col;
        if (m >= g.M || co >= g.Co) return;
        if (A.bias) v += bits_to_f32(S(), elem_bits((const S *)A.bias, co));
        long long yi = m * g.Co + co;
        if constexpr (OUT_NCHW) {
            const long long n = m / g.P;
            yi = (n * g.Co + co) * g.P + (m - n * g.P);
        }
        y[yi] = to_out(S(), v);
    };
    if constexpr (MICRO == ABL_MFMA32) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        put(wm * 64 + i * 32 + MF32::qrow(q, lane) + v, wn * 64 + j * 32 + (lane & 31),
                            acc32[i][j][4 * q + v]);
    } else if constexpr (MICRO == ABL_MFMA16) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    put(wm * 64 + i * 16 + MF16::qrow(0, lane) + v, wn * 64 + j * 16 + (lane & 15), acc16[i][j][v]);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                put(wm * 64 + 8 * (lane >> 3) + i, wn * 64 + 8 * (lane & 7) + j, accv[i][j]);
    }
}

template <typename S, bool OUT_NCHW, bool USE_LDS, int STAGES, bool PREFETCH, int MICRO, int BT>
__global__ __launch_bounds__(BT == 128 ? 256 : 64) void igemm_ablate_kernel(GemmArgs A) {
    igemm_ablate_body<S, OUT_NCHW, USE_LDS, STAGES, PREFETCH, MICRO, BT>(A);
}

}  // namespace convlower
