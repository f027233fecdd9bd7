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
//
// NCHW input is read where it lies (16-bit types).  There a pixel's channels
// are a plane apart, so 16-byte loads carry 8 consecutive pixels of one
// channel.  Each step's runs are loaded straight into a raw LDS buffer as
// such chunks, for every channel of the slice: the chunks of a run are
// aligned to multiples of 8 input columns and cover the run's in-image
// columns only.  Once the step's raw chunks have landed (and the previous
// step's stage is no longer read), the block copies them into the stage:
// LDS transpose reads (four channels x sixteen pixels per 16 lanes, each
// lane then holding four channels of one pixel) and 8-byte writes to the
// pixel's stage row.  The stage then has the same layout as for NHWC input,
// and the taps read it the same way.  Stage rows of padding columns are
// zeroed once, and no copy writes them.  One stage and one raw buffer take
// the LDS of the two NHWC stages; the copy costs one more barrier per step.
#pragma once

#include <type_traits>

namespace convlower {

// Stage geometry for KW taps per kernel row.  A tile of 256 consecutive
// output pixels spans at most kRowWinMaxSeg output rows (the host checks
// 255 / Wo + 2 against it); each adds KW - 1 pixels to the stage.
// BN_: output channels per block tile, 128 (four 128 x 64 wavefront tiles,
// 2 x 2) or 64 (four 64 x 64 wavefront tiles stacked along M, for layers with
// at most 64 output channels, which a 128-wide tile would half waste).
template <typename S, int KW_, int BN_ = 128, bool IN_NCHW_ = false>
struct RowWinCfg {
    static_assert(BN_ == 128 || BN_ == 64, "block tiles 256 x 128 or 256 x 64");
    static_assert(!IN_NCHW_ || sizeof(S) == 2, "NCHW input is read in place for 16-bit types");
    static constexpr bool IN_NCHW = IN_NCHW_;
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
    static constexpr int NA = IN_NCHW ? 1 : 2, NB = 4;  // A and B stages
    static constexpr int IPW_A = ROWS_A * KCH / 64 / NW;
    // NCHW input: raw chunk positions (8 input columns of all BK channels of
    // the slice each) one step may stage, the raw-chunk loads per wavefront,
    // and the copy's units per wavefront (sixteen columns x four channels per
    // 16 lanes).
    static constexpr int RAW_CH = 40;
    static constexpr int RAW_SLOTS = IN_NCHW ? RAW_CH * BK : 0;
    static constexpr int IPW_RAW = RAW_CH * BK / 64 / NW;
    static constexpr int UPW = RAW_CH / 2 * (BK / 4) / (4 * NW);
    static constexpr int IPW_B = BN * KCH / 64 / NW;
    static constexpr int WGM = BN_ == 128 ? 2 : 4, WGN = BN_ == 128 ? 2 : 1;
    static constexpr int WPM = BM / WGM, WCN = BN / WGN;  // wavefront tile 128 x 64 or 64 x 64
    static constexpr int MT = 32, TP = WPM / MT, TC = WCN / MT;
    static constexpr int NG = KCH / 2;
    static constexpr int LDS_SLOTS = NA * A_SLOTS + RAW_SLOTS + NB * B_SLOTS;
    static constexpr long long STAGE_BYTES = 16LL * LDS_SLOTS;  // all stages, reused by the epilogue
    static_assert(IPW_A * NW * 64 == ROWS_A * KCH && IPW_B * NW * 64 == BN * KCH, "loads must split evenly");
    static_assert(!IN_NCHW || (IPW_RAW * NW * 64 == RAW_CH * BK && UPW * 4 * NW == RAW_CH / 2 * (BK / 4)),
                  "raw loads and copy units must split evenly");
    static_assert(!IN_NCHW || A_SLOTS * 16 + RAW_SLOTS * 16 <= 65536, "stage and raw buffer within 16-bit offsets");
    static_assert(2 * (STAGE_BYTES + BN * 4 + (IN_NCHW ? UPW / 2 * NTHR * 4 : 0)) <= 160 * 1024,
                  "two blocks per compute unit");
};

template <typename S, bool OUT_NCHW, typename C>
__device__ __forceinline__ void igemm_rowwin_body(const GemmArgs &A) {
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, VEC = C::VEC, KCH = C::KCH;
    constexpr int IPW_A = C::IPW_A, IPW_B = C::IPW_B;
    constexpr int WPM = C::WPM, WCN = C::WCN, TP = C::TP, TC = C::TC, NG = C::NG;
    constexpr int NW = C::NW, RPI = C::RPI, KW = C::KW, A_SLOTS = C::A_SLOTS, B_SLOTS = C::B_SLOTS;
    constexpr bool NCHW_IN = C::IN_NCHW;
    constexpr int IPW_RAW = C::IPW_RAW, UPW = C::UPW;
    constexpr int IPW_AL = NCHW_IN ? IPW_RAW : IPW_A;  // A-side loads per wavefront per step
    constexpr uint32_t ES = (uint32_t)sizeof(S);
    using MF = MfmaShape<S, 32>;
    // Output (and bias) type: the input type, except bf16 for fp8 inputs.
    using O = typename std::conditional<sizeof(S) == 1, uint16_t, S>::type;
    static_assert(KW == 3, "the schedule below is written for three taps per kernel row");

    // A stages (NHWC: two; NCHW: one, then the raw buffer), then B stages;
    // the epilogue reuses all of them.
    __shared__ uint4 lds[C::LDS_SLOTS];
    uint4 *const sa0 = lds, *const sa1 = NCHW_IN ? lds : lds + A_SLOTS;
    uint4 *const raw = lds + A_SLOTS;                  // NCHW: raw chunks, slot (chunk, channel)
    uint4 *const sb0 = lds + C::NA * A_SLOTS + C::RAW_SLOTS;  // B stage i at sb0 + i * B_SLOTS; tap u uses stage u % 4
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
        if (A.bias && co < g.Co) bias_r = bits_to_f32(O(), elem_bits((const O *)A.bias, co));
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
    int abase[IPW_AL], ahi[IPW_AL];
    bool aok[IPW_AL];
    // NCHW copy units: this lane's raw byte offset for unit 0 (unit i reads
    // 2048*i bytes further on), and in LDS the stage byte offsets of its
    // units 2k and 2k+1 in the halves of word cw_lds[k][tid] (0xFFFF: no
    // write), read back once per step rather than held in registers.
    uint32_t craw = 0;
    __shared__ uint32_t cw_lds[NCHW_IN ? UPW / 2 : 1][NCHW_IN ? C::NTHR : 1];
    if constexpr (!NCHW_IN) {
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
    } else {
        // Segment j has S_j stage rows from row0_j on, for input columns
        // wi0_j .. wi0_j + S_j - 1; its in-image columns are covered by nch_j
        // raw chunks from column 8*cA_j on, at raw positions rc_j onwards.
        // Segment 0 and the last one may be partial; the ones between are
        // whole output rows and alike.
        const int p = g.p, W = g.W;
        const uint32_t nseg = (mend - 1) / Wo - R0 + 1;
        const int len0 = (int)(min(mend, (R0 + 1) * Wo) - m0);
        const int wi00 = (int)(m0 - R0 * Wo) - p;
        const int lenl = (int)(mend - max(m0, (R0 + nseg - 1) * Wo));
        auto span = [&](int wi0, int S_, int &cA) {
            const int vlo = max(wi0, 0), vhi = min(wi0 + S_, W);
            cA = vlo >> 3;
            return vhi > vlo ? ((vhi - 1) >> 3) - cA + 1 : 0;
        };
        int cA0, cAf, cAl;
        const int n0 = span(wi00, len0 + KW - 1, cA0);
        const int nf = max(span(-p, (int)SW, cAf), 1);
        const int nl = span(-p, lenl + KW - 1, cAl);
        const int total = nseg > 1 ? n0 + (int)(nseg - 2) * nf + nl : n0;
        // Segment of raw position rc (< total): index, first raw position, cA.
        auto seg_of = [&](int rc, int &j, int &rcj, int &cA) {
            if (rc < n0) {
                j = 0; rcj = 0; cA = cA0;
                return;
            }
            const int t = (rc - n0) / nf;
            if (1 + t >= (int)nseg - 1) {
                j = (int)nseg - 1; rcj = n0 + (int)(nseg - 2) * nf; cA = cAl;
            } else {
                j = 1 + t; rcj = n0 + t * nf; cA = cAf;
            }
        };
        const int HW = g.H * W;
        // Raw loads: load d = i*NW + wave of the block fills raw positions
        // 8*(d / 4) .. +7 of channels 8*(d % 4) .. +7; lane L takes channel
        // c = 8*(d % 4) + L/8 and position 8*(d / 4) + ((L % 8) ^ swz(c)),
        // so each 8 lanes read 8 consecutive chunks (128 bytes) of one
        // channel's row.  swz(c) = 2*((c/2) % 4) keeps the transpose reads
        // of the copy free of bank conflicts (see raw_slot below).
#pragma unroll
        for (int i = 0; i < IPW_RAW; ++i) {
            const int d = i * NW + wave, c = (d & 3) * 8 + (lane >> 3);
            const int rc = (d >> 2) * 8 + ((lane & 7) ^ (2 * ((c >> 1) & 3)));
            int j, rcj, cA;
            seg_of(rc, j, rcj, cA);
            const uint32_t R = R0 + (uint32_t)j;
            const uint32_t n = R / (uint32_t)g.Ho, ho = R - n * (uint32_t)g.Ho;
            const int hi0 = (int)ho - p;
            const bool live = rc < total;
            aok[i] = live;
            ahi[i] = hi0;
            abase[i] = live ? (((int)n * g.C + c) * g.H + hi0) * W + 8 * (cA + rc - rcj) : 0;  // may be negative while hi0 < 0
        }
        // Copy units: unit u = (i*NW + wave)*4 + lane/16 moves pixel block
        // pb = u / 8 (raw positions 2pb, 2pb+1) of channels 4q .. 4q+3,
        // q = u % 8.  Lane t of the 16 reads channel 4q + t/4, columns
        // 4*(t%4) .. +3 of the block, and after the transpose holds the four
        // channels of the block's column t, which go to that column's stage
        // row (none when it lies outside the segment's run or the image).
        // Raw position rc of channel c is slot ((rc/8)*4 + c/8)*64 + (c%8)*8
        // + ((rc%8) ^ swz(c)).  Unit i + 1 is unit i two pixel blocks (four
        // raw positions) on (NW*4 = 16 units): an odd unit's slot is the
        // even one's with bit 2 flipped -- bit 6 of the byte offset, which
        // the raw buffer's base (a multiple of 4096) leaves alone -- and every
        // second unit moves on by one block of 8 positions (4096 bytes).
        static_assert(NW * 4 == 16 && BK == 32, "one pixel-block pair per unit step, four channel octets");
        static_assert(A_SLOTS * 16 % 4096 == 0, "raw buffer base");
        {
            const int u = wave * 4 + (lane >> 4), pb = u >> 3, q = u & 7, t = lane & 15;
            const int rc0 = 2 * pb + ((t & 3) >> 1), c = q * 4 + (t >> 2);  // rc0 < 4
            const int lo = rc0 ^ (2 * ((c >> 1) & 3));
            const int slot = (c >> 3) * 64 + (c & 7) * 8 + lo;
            craw = (uint32_t)(slot * 16 + (t & 1) * 8) + (uint32_t)(A_SLOTS * 16);
        }
#pragma unroll
        for (int i = 0; i < UPW; ++i) {
            const int u = (i * NW + wave) * 4 + (lane >> 4), pb = u >> 3, q = u & 7, t = lane & 15;
            const int rc = 2 * pb + (t >> 3);
            int j, rcj, cA;
            seg_of(rc, j, rcj, cA);
            const int wi = 8 * (cA + rc - rcj) + (t & 7);
            const int wi0 = j == 0 ? wi00 : -p;
            const int Sj = j == 0 ? len0 + KW - 1 : (j == (int)nseg - 1 ? lenl + KW - 1 : (int)SW);
            const int row0 = j == 0 ? 0 : (int)rows0 + (j - 1) * (int)SW;
            const bool ok = rc < total && wi < W && wi >= wi0 && wi < wi0 + Sj;
            const uint32_t wb = ok ? (uint32_t)(dual_slot<KCH>(row0 + wi - wi0, q >> 1) * 16 + (q & 1) * 8) : 0xFFFFu;
            if (i % 2 == 0)
                cw_lds[i / 2][tid] = wb;
            else
                cw_lds[i / 2][tid] |= wb << 16;
        }
        // Stage rows of padding columns (wi < 0 or >= W inside a segment's
        // run) hold zeros for the whole K loop: no copy writes them.
        for (int r = tid; r < C::ROWS_A; r += C::NTHR) {
            int j = 0, e = r;
            if (r >= (int)rows0) {
                j = 1 + (r - (int)rows0) / (int)SW;
                e = r - (int)rows0 - (j - 1) * (int)SW;
            }
            if (j >= (int)nseg) continue;
            const int wi0 = j == 0 ? wi00 : -p;
            const int Sj = j == 0 ? len0 + KW - 1 : (j == (int)nseg - 1 ? lenl + KW - 1 : (int)SW);
            const int wi = wi0 + e;
            if (e < Sj && (wi < 0 || wi >= W)) {
#pragma unroll
                for (int c = 0; c < KCH; ++c) sa0[r * KCH + c] = make_uint4(0, 0, 0, 0);
            }
        }
    }
    // Weights: OHWI for NHWC input; for NCHW input regrouped tap-major,
    // [slice][kh][kw][co][BK channels], so that one tap's B rows of the block
    // are one contiguous run.
    int wbase[IPW_B];
    bool wok[IPW_B];
#pragma unroll
    for (int j = 0; j < IPW_B; ++j) {
        const int co = co0 + (j * NW + wave) * RPI + lrow;
        wok[j] = co < g.Co;
        // tap (0, 0) of slice 0 (NCHW input: with this lane's chunk column)
        wbase[j] = NCHW_IN ? co * BK + (int)kc : co * g.KH * KW * g.C;
    }

    const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(A.a_src, A.a_bytes);
    const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(A.b, A.b_bytes);
    const uint32_t lds_w = (uint32_t)wave * 1024u;

    // The A runs of K step kt into stage sa (NCHW: the raw chunks into the
    // raw buffer), and the B rows of tap u (step u / KW, kw = u % KW) into
    // stage sb.  Past the end nothing is loaded, but the loads are still
    // issued so the count in flight stays fixed.
    auto issue_a = [&](int kt, uint4 *sa) {
        const bool live = kt < nk;
        const int slice = kt / g.KH, kh = kt - slice * g.KH;
        const int cofs = NCHW_IN ? slice * BK * g.H * g.W + kh * g.W : kh * WC + slice * BK + (int)kc;
        const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)(NCHW_IN ? raw : sa) + lds_w;
        uint32_t voff[IPW_AL];
#pragma unroll
        for (int i = 0; i < IPW_AL; ++i) {
            const int hi = ahi[i] + kh;
            const bool valid = live && aok[i] && hi >= 0 && hi < g.H;
            voff[i] = valid ? (uint32_t)(abase[i] + cofs) * ES : kOutOfRange;
        }
#pragma unroll
        for (int i = 0; i < IPW_AL; ++i) lds_dma16(a_rsrc, voff[i], lds0 + (uint32_t)(i * NW * 1024));
    };
    auto issue_b = [&](int u, uint4 *sb) {
        const int kt = u / KW, kw = u - kt * KW;
        const bool live = kt < nk;
        const int slice = kt / g.KH, kh = kt - slice * g.KH;
        const int wofs = NCHW_IN ? __builtin_amdgcn_readfirstlane(((slice * g.KH + kh) * KW + kw) * g.Co * BK)
                                 : (kh * KW + kw) * g.C + slice * BK + (int)kc;
        const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)sb + lds_w;
        uint32_t voff[IPW_B];
#pragma unroll
        for (int j = 0; j < IPW_B; ++j) voff[j] = live && wok[j] ? (uint32_t)(wbase[j] + wofs) * ES : kOutOfRange;
#pragma unroll
        for (int j = 0; j < IPW_B; ++j) lds_dma16(b_rsrc, voff[j], lds0 + (uint32_t)(j * NW * 1024));
    };
    // NCHW: the raw chunks of the next step into the stage (see the top of
    // this file), in two halves of UPW / 2 units: transpose reads, then the
    // writes.
    typedef short v4s_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s_t *lds_v4s_ptr;
    typedef __attribute__((address_space(3))) char *lds_byte_ptr;
    constexpr int UH = NCHW_IN ? UPW / 2 : 1;
    v4s_t cbuf[UH];
    uint32_t cwr[NCHW_IN ? UPW / 2 : 1];
    auto copy_offsets = [&]() {
        if constexpr (NCHW_IN) {
#pragma unroll
            for (int k = 0; k < UPW / 2; ++k) cwr[k] = cw_lds[k][tid];
        }
    };
    auto copy_read = [&](int half) {
        if constexpr (NCHW_IN) {
            const lds_byte_ptr base0 = (lds_byte_ptr)(lds_ptr_t)lds + craw;
            const lds_byte_ptr base1 = (lds_byte_ptr)(lds_ptr_t)lds + (craw ^ 64u);
#pragma unroll
            for (int j = 0; j < UH; ++j) {
                const int i = half * UH + j;
                cbuf[j] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_v4s_ptr)((i & 1 ? base1 : base0) + (i >> 1) * 4096));
            }
        }
    };
    auto copy_write = [&](int half) {
        if constexpr (NCHW_IN) {
            const lds_byte_ptr base = (lds_byte_ptr)(lds_ptr_t)lds;
#pragma unroll
            for (int j = 0; j < UH; ++j) {
                const int i = half * UH + j;
                const uint32_t wb = (i % 2 == 0 ? cwr[i / 2] : cwr[i / 2] >> 16) & 0xFFFFu;
                if (wb != 0xFFFFu) *(lds_v4s_ptr)(base + wb) = cbuf[j];
            }
        }
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
    auto mfma_group = [&](int grp, int ip0 = 0, int ip1 = C::TP) {
#pragma unroll
        for (int ip = ip0; ip < ip1; ++ip)
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
    // NCHW input, last tap of a step: after the barrier the step's stage is
    // no longer read and step kt+1's raw chunks are in LDS, so the copy into
    // the stage runs behind half of the remaining MFMAs, a second barrier
    // publishes it, and tap u+1's first fragments are read from the new stage
    // behind the other half.
    auto sub = [&](int kt, int kw, uint4 *sa, uint4 *sa_next, uint4 *sb, const uint4 *sb_next) {
        mfma_group(0);
        __builtin_amdgcn_sched_barrier(0);
        if (kw == 1)
            CONVLOWER_WAIT_VMCNT_LDS(IPW_AL + 2 * IPW_B);
        else
            CONVLOWER_WAIT_VMCNT_LDS(2 * IPW_B);
        block_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (kw == 0) issue_a(kt + 1, sa_next);
        issue_b(kt * KW + kw + 4, sb);
        __builtin_amdgcn_sched_barrier(0);
        if (NCHW_IN && kw + 1 == KW) {
            static_assert(NG == 2, "two MFMA groups per tap");
            copy_offsets();
            copy_read(0);
            __builtin_amdgcn_sched_barrier(0);
            mfma_group(1, 0, TP / 2);
            __builtin_amdgcn_sched_barrier(0);
            copy_write(0);
            copy_read(1);
            copy_write(1);
            __builtin_amdgcn_sched_barrier(0);
            CONVLOWER_WAIT_LDS();  // this wavefront's stage writes are done
            block_barrier();
            __builtin_amdgcn_sched_barrier(0);
            lds_read(sa_next, sb_next, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            mfma_group(1, TP / 2, TP);
            __builtin_amdgcn_sched_barrier(0);
            lds_read(sa_next, sb_next, 0, 1);
            __builtin_amdgcn_sched_barrier(0);
            return;
        }
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
        if constexpr (NCHW_IN) {
            // Step 0's raw chunks into the stage (padding rows were zeroed
            // above; the barrier's wait covers those writes too).
            CONVLOWER_WAIT_VMCNT_LDS(3 * IPW_B);
            block_barrier();
            copy_offsets();
            copy_read(0);
            copy_write(0);
            copy_read(1);
            copy_write(1);
            CONVLOWER_WAIT_VMCNT_LDS(3 * IPW_B);
        }
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
    dual_store<O, OUT_NCHW, C>(A, acc, lds, bias_s, m0, co0, wp, wc, lane, tid);
}

template <typename S, bool OUT_NCHW, int BN = 128, bool IN_NCHW = false>
__global__ __launch_bounds__(256, 2) void igemm_rowwin_kernel(GemmArgs A) {
    igemm_rowwin_body<S, OUT_NCHW, RowWinCfg<S, 3, BN, IN_NCHW>>(A);
}

}  // namespace convlower
