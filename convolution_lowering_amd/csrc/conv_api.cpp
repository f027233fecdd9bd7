// The C ABI of include/convlower.h: argument checks, the lowering plan
// (feed, tile, split-K, workspace layout) and the launch sequence.
//
// Every decision here is a fixed function of the call's sizes (and of the
// calling thread's main-loop override, when one is set for ablation), so the
// workspace query and the launch agree.
#include <string.h>

#include <algorithm>
#include <climits>
#include <atomic>
#include <mutex>
#include <numeric>

#include "conv_internal.h"

namespace convlower {
namespace {

constexpr long long kLimit = (1LL << 31) - 1;  // element counts the kernels index with 32-bit parts
constexpr long long kBufMax = (1LL << 31) - 64;  // bytes the vector paths address with 32-bit buffer offsets
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool dtype_ok(conv_dtype_t d) {
    return d == CONV_DTYPE_FP32 || d == CONV_DTYPE_BF16 || d == CONV_DTYPE_FP16 || d == CONV_DTYPE_FP8_E4M3;
}
// Bytes of one element of x (and w); y and bias are bf16 for fp8 inputs.
size_t dtype_bytes(conv_dtype_t d) { return d == CONV_DTYPE_FP32 ? 4 : d == CONV_DTYPE_FP8_E4M3 ? 1 : 2; }

// Main-loop variant forced on this thread's plans (CONV_MAIN_LOOP_AUTO: none).
thread_local int t_forced_main_loop = CONV_MAIN_LOOP_AUTO;

// Main loops whose indirection slice in LDS holds up to 12 taps at any
// tile height (the others hold 3072 entries).
bool wide_slice(int tile) {
    return tile == TILE_256x128_DUAL || tile == TILE_256x128_OCT || tile == TILE_128x64_QUAD ||
           tile == TILE_256x256_OCT;
}

int tile_rows(int tile) {
    return tile == TILE_32x64                                                                     ? 32
           : tile == TILE_128x64_QUAD                                                          ? 128
           : (tile == TILE_256x128 || wide_slice(tile))                                        ? 256
                                                                                               : 128;
}

struct Plan {
    Geom g;
    bool e16, nhwc;  // 16-bit elements (bf16 or fp16); channels-last tensors
    int dtype;       // conv_dtype_t
    int feed;
    bool out_nchw;
    int tile, splits, kps;
    bool need_ibuf, need_win, need_wpack;
    bool need_col;  // X_col materialised (the im2col baseline)
    bool direct;    // the direct-convolution baseline: no lowering, no main loop
    bool patch;     // C_in <= 4: input patches staged in LDS (patch_conv.hip), no workspace
    bool need_xcl;  // channels-last copy of an NCHW input
    int chunk_n;    // images per main-loop pass (< N: the batch goes through the copy in parts)
    int cp;         // channels per pixel row of the channels-last copy (> C: zero-padded)
    Geom gm;        // geometry the main loop sees (C = cp, K = T*cp)
    bool rows16;  // the feed can read X_col rows in 16-byte chunks (by shape)
    bool force_element;  // main loop forced to the element-gather loop
    int ablate;          // a CONV_MAIN_LOOP_ABL_ variant forced (0: none)
    bool sk;             // the ping-pong loop in its stream-K form (partial tiles and flags in the workspace)
    size_t off_ibuf, off_win, off_xcl, off_wpack, off_col, off_part, off_sk, total;
    size_t esize;
};

// Window placements along one axis (0: none fits); may exceed int for
// extreme padding, which the callers refuse.
long long out_extent(int in, int k, int s, int p, int d) {
    long long span = (long long)in + 2LL * p - (long long)d * (k - 1) - 1;
    if (span < 0) return 0;
    return span / s + 1;
}

conv_status_t make_geom(int N, int C, int H, int W, int Co, int KH, int KW, int s, int p, int d, Geom *g) {
    if (N <= 0 || C <= 0 || H <= 0 || W <= 0 || Co <= 0 || KH <= 0 || KW <= 0 || s <= 0 || d <= 0 || p < 0)
        return CONV_ERR_INVALID_ARG;
    const long long Hl = out_extent(H, KH, s, p, d), Wl = out_extent(W, KW, s, p, d);
    if (Hl <= 0 || Wl <= 0) return CONV_ERR_INVALID_ARG;
    // Extents, per-image and per-window counts kept as int: valid requests
    // beyond that are not served.
    if (Hl > INT_MAX || Wl > INT_MAX) return CONV_ERR_UNSUPPORTED;
    const int Ho = (int)Hl, Wo = (int)Wl;
    const long long P = (long long)Ho * Wo, T = (long long)KH * KW;
    const long long Wwin = (long long)(Wo - 1) * s + (long long)(KW - 1) * d + 1;
    if (P > INT_MAX || T > INT_MAX || Wwin > INT_MAX) return CONV_ERR_UNSUPPORTED;
    g->N = N; g->C = C; g->H = H; g->W = W; g->Co = Co; g->KH = KH; g->KW = KW;
    g->s = s; g->p = p; g->d = d; g->Ho = Ho; g->Wo = Wo;
    g->P = (int)P;
    g->T = (int)T;
    g->Wwin = (int)Wwin;
    g->M = (long long)N * Ho * Wo;
    g->K = (long long)C * KH * KW;
    return CONV_OK;
}

// Raw chunks (8 in-image input columns of one channel, starting at a
// multiple of 8 columns) the NCHW window-row loop stages per channel for one
// 256-pixel tile, the most over the layer's tiles.  The count depends only on
// where a tile starts within its output row -- which repeats every
// Wo / gcd(256, Wo) tiles -- and, for the last tile, on where M cuts it.
int rowwin_nchw_chunks(const Geom &g) {
    const long long Wo = g.Wo, M = g.M;
    auto tile_chunks = [&](long long m0) {
        const long long mend = std::min(m0 + 256, M);
        int total = 0;
        for (long long R = m0 / Wo; R * Wo < mend; ++R) {
            const long long first = std::max(m0, R * Wo), last = std::min(mend, (R + 1) * Wo);
            const int wi0 = (int)(first - R * Wo) - g.p;
            const int vlo = std::max(wi0, 0), vhi = std::min(wi0 + (int)(last - first) + g.KW - 1, g.W);
            if (vhi > vlo) total += (vhi - 1) / 8 - vlo / 8 + 1;
        }
        return total;
    };
    const long long ntiles = (M + 255) / 256, period = Wo / std::gcd(256LL, Wo);
    int worst = tile_chunks((ntiles - 1) * 256);
    for (long long t = 0; t < std::min(period, ntiles); ++t) worst = std::max(worst, tile_chunks(t * 256));
    return worst;
}

// Element counts of every tensor must stay inside 32-bit signed range (the
// kernels form 64-bit addresses but index within one image in 32 bits).
bool sizes_supported(const Geom &g) {
    long long Hp = (long long)g.H, Wp = (long long)g.W;
    long long x = (long long)g.N * g.C * Hp * Wp;
    long long y = g.M * g.Co;
    long long w = g.K * g.Co;
    long long win = (long long)g.N * g.Ho * g.Wwin * g.KH * g.C;
    long long ibuf = (long long)g.P * g.T;
    return (long long)g.Ho * g.Wo <= kLimit && g.K <= kLimit && g.M <= kLimit && x <= kLimit && y <= kLimit &&
           w <= kLimit && win <= kLimit && ibuf <= kLimit;
}

conv_status_t make_plan(int N, int C, int H, int W, int Co, int KH, int KW, int s, int p, int d,
                        conv_layout_t layout, conv_dtype_t dtype, conv_algo_t algo, Plan *pl,
                        bool allow_pad = true) {
    if (layout != CONV_LAYOUT_NCHW && layout != CONV_LAYOUT_NHWC) return CONV_ERR_INVALID_ARG;
    if (!dtype_ok(dtype)) return CONV_ERR_INVALID_ARG;
    if (algo < CONV_ALGO_AUTO || algo > CONV_ALGO_PATCH) return CONV_ERR_INVALID_ARG;
    memset(pl, 0, sizeof(*pl));
    conv_status_t st = make_geom(N, C, H, W, Co, KH, KW, s, p, d, &pl->g);
    if (st != CONV_OK) return st;
    pl->chunk_n = N;
    pl->cp = C;
    const Geom &g = pl->g;
    if (!sizes_supported(g)) return CONV_ERR_UNSUPPORTED;
    pl->e16 = dtype == CONV_DTYPE_BF16 || dtype == CONV_DTYPE_FP16;
    pl->dtype = dtype;
    pl->nhwc = layout == CONV_LAYOUT_NHWC;
    pl->esize = dtype_bytes(dtype);
    if (dtype == CONV_DTYPE_FP8_E4M3) {
        // fp8 e4m3 inputs through the window-row loop (K tiles of 64
        // channels).  Channels-last tensors are read as they lie (no
        // workspace); NCHW input is first copied channels-last (|x| bytes,
        // H*W a multiple of 4 so the copy reads whole 4-byte pieces) and its
        // OIHW weights regrouped to (kh, kw, ci) (|w| bytes), as the 16-bit
        // NCHW layers too wide for the in-place read are.
        if (algo != CONV_ALGO_AUTO && algo != CONV_ALGO_IM2WIN_LDS) return CONV_ERR_UNSUPPORTED;
        if (t_forced_main_loop != CONV_MAIN_LOOP_AUTO) return CONV_ERR_UNSUPPORTED;
        const bool ok = g.s == 1 && g.d == 1 && g.KW == 3 && g.C % 64 == 0 && 255 / g.Wo + 2 <= kRowWinMaxSeg &&
                        (long long)g.N * g.C * g.H * g.W <= kBufMax && g.K * g.Co <= kBufMax &&
                        (pl->nhwc || (g.H * g.W) % 4 == 0);
        if (!ok) return CONV_ERR_UNSUPPORTED;
        pl->feed = FEED_ROWWIN;
        pl->gm = g;
        pl->out_nchw = !pl->nhwc;
        pl->tile = g.Co <= 64 ? TILE_256x64_ROWWIN : TILE_256x128_ROWWIN;
        pl->splits = 1;
        pl->kps = (int)((g.K + 127) / 128 * 128);
        pl->total = 0;
        if (!pl->nhwc) {
            pl->need_xcl = pl->need_wpack = true;
            pl->off_xcl = 0;
            pl->off_wpack = align_up((size_t)g.N * g.C * g.H * g.W);
            pl->total = align_up(pl->off_wpack + (size_t)g.Co * g.K);
        }
        return CONV_OK;
    }

    // A 1x1 stride-1 unpadded convolution is a GEMM call (The Indirect
    // Convolution Algorithm, abstract); a kernel that covers the whole
    // unpadded input is a dense layer ("Unifying Convolutions and GEMM",
    // section 4).  Both are fed from the input as it lies in memory.
    const bool whole = KH == H && KW == W && p == 0;
    const bool one = KH == 1 && KW == 1 && s == 1 && p == 0;
    // Channels that are not a whole number of 16-byte chunks: padding each
    // pixel (or window cell) to the next chunk lets the main loop address
    // every chunk of a K tile on its own, whatever tap it falls in.  The
    // indirection buffer then has to fit the main loop's LDS slice (at most
    // 12 taps); larger kernels read a window tensor padded the same way.
    const int VEC = pl->e16 ? 8 : 4;
    const int cpad = (g.C + VEC - 1) / VEC * VEC;
    const bool pad_c = allow_pad && g.C % VEC != 0;
    const long long im2col_bytes = g.M * g.K * (long long)pl->esize;
    const long long pad_w_bytes = (long long)g.Co * g.T * cpad * pl->esize;
    // Up to 12 taps every two-wavefront loop holds the block's slice of the
    // buffer in LDS; up to 32 only the 128 x 64 block (at most 64 output
    // channels, more than 64 output pixels, the library's own loop choice).
    const bool chunk_taps = g.T <= 12 || (g.T <= 32 && g.Co <= 64 && g.M > 64 &&
                                          t_forced_main_loop == CONV_MAIN_LOOP_AUTO);
    const bool chunk_ind = pad_c && chunk_taps && (long long)g.H * g.W <= 65535 &&
                           (long long)g.N * g.H * g.W * cpad * pl->esize + pad_w_bytes + (long long)g.P * g.T * 4 +
                                   1024 <
                               im2col_bytes;
    const long long win_pad = (long long)g.N * g.Ho * g.Wwin * g.KH * cpad;  // elements
    const bool chunk_win =
        pad_c && win_pad <= kLimit && win_pad * (long long)pl->esize + pad_w_bytes + 512 < im2col_bytes;
    // Window rows in LDS (igemm_rowwin.h): stride 1, dilation 1, three taps
    // per kernel row, channel slices of whole K tiles, a 256-pixel tile
    // spanning at most kRowWinMaxSeg output rows, 32-bit byte offsets.
    const bool rowwin_ok = g.s == 1 && g.d == 1 && g.KW == 3 && g.C % (pl->e16 ? 32 : 16) == 0 &&
                           255 / g.Wo + 2 <= kRowWinMaxSeg &&
                           (long long)g.N * g.C * g.H * g.W * (long long)pl->esize <= kBufMax &&
                           g.K * g.Co * (long long)pl->esize <= kBufMax;
    // NCHW input read where it lies by the window-row loop (16-bit types):
    // every tile's raw chunks must fit the loop's LDS buffer, and an even W
    // keeps each chunk of a run on 4-byte boundaries of x, so the loads'
    // per-dword range check never drops an in-image element at the end of x.
    // The in-place loop transposes each block's input rows in LDS, once for
    // every 128-channel output tile; the channels-last copy moves x once.
    // Up to 256 output channels the copy costs more (measured on the 3x3
    // layers 64->128@56, 64->64@56, 64->128@112, 128->256@56: 4-12% faster
    // whole calls in place); at 512 it costs less (256->512@28, 512->512@14:
    // 3-5% slower in place), so wider layers keep the copy.
    const bool rowwin_inplace = rowwin_ok && !pl->nhwc && pl->e16 && g.W % 2 == 0 && g.Co <= 256 &&
                                rowwin_nchw_chunks(g) <= kRowWinRawChunks;
    // AUTO takes the window rows in LDS where they apply and the grid gives
    // every CU a block without splitting K (tiles 256 x 64 up to 64 output
    // channels, 256 x 128 above).
    const int rowwin_bn = g.Co <= 64 ? 64 : 128;
    const bool rowwin_auto = rowwin_ok && t_forced_main_loop == CONV_MAIN_LOOP_AUTO &&
                             ((g.M + 255) / 256) * ((g.Co + rowwin_bn - 1) / rowwin_bn) >= 256;
    // A 1x1 NCHW input read where it lies (16-bit types): K tiles of whole
    // channel rows (C a multiple of 32), 16-byte pixel chunks that never
    // cross an image (P a multiple of 8), 32-bit offsets, and the library's
    // own choice of main loop.
    const bool gemm_nchw = one && !pl->nhwc && pl->e16 && g.C % 32 == 0 && g.P % 8 == 0 && g.M > 64 &&
                           (long long)g.N * g.C * g.H * g.W * (long long)pl->esize <= kBufMax &&
                           g.K * g.Co * (long long)pl->esize <= kBufMax &&
                           t_forced_main_loop == CONV_MAIN_LOOP_AUTO;
    const bool patch_ok = patch_conv_plan(g, pl->dtype, nullptr);
    // The ablation loops run on the indirection feed only.
    const bool ablate = t_forced_main_loop >= CONV_MAIN_LOOP_ABL_FULL;
    if (ablate && algo == CONV_ALGO_AUTO) algo = CONV_ALGO_INDIRECT;
    if (algo == CONV_ALGO_AUTO)
        algo = (whole || one) ? CONV_ALGO_GEMM
               : patch_ok                  ? CONV_ALGO_PATCH
               : (!chunk_ind && chunk_win) ? CONV_ALGO_IM2WIN
               : rowwin_auto             ? CONV_ALGO_IM2WIN_LDS
                                         : CONV_ALGO_INDIRECT;
    switch (algo) {
        case CONV_ALGO_GEMM:
            if (whole) {
                pl->feed = FEED_ROWMAJOR;  // Ho = Wo = 1: both layouts store y as [N][Co]
            } else if (one && pl->nhwc) {
                pl->feed = FEED_ROWMAJOR;
            } else if (gemm_nchw) {
                // x[n] is the GEMM's A operand transposed ([C][pixels]), the
                // weights [Co][C] are W_row as they lie: no workspace.
                pl->feed = FEED_GEMM_NCHW;
            } else if (one && g.C % (pl->e16 ? 8 : 4) == 0 && g.N >= 2) {
                // NCHW 1x1: half the batch at a time is copied channels-last
                // and multiplied as a plain GEMM (the copy of all of x would
                // be as large as X_col itself).
                pl->feed = FEED_ROWMAJOR;
                pl->need_xcl = true;
                pl->chunk_n = (g.N + 1) / 2;
            } else if (one) {
                pl->feed = FEED_NCHW_1X1;
            } else {
                return CONV_ERR_UNSUPPORTED;
            }
            break;
        case CONV_ALGO_INDIRECT:
            // The indirection buffer addresses each input pixel's row of C
            // channels.  An NCHW input whose rows can be read in 16-byte
            // chunks is first copied channels-last (|x| bytes of workspace);
            // otherwise the buffer addresses channel 0 of the pixel and the
            // main loop steps through the channel planes element by element.
            // Channels not a whole number of 16-byte chunks (and at most 12
            // taps): the copy (from either layout) pads every pixel to whole
            // chunks, each addressed on its own by the main loop.
            pl->need_ibuf = true;
            if (chunk_ind) {
                pl->feed = FEED_IND_CHUNK;
                pl->cp = cpad;
                pl->need_xcl = true;
                pl->need_wpack = true;
            } else if (pl->nhwc) {
                pl->feed = FEED_IND_NHWC;
            } else if (g.C % (pl->e16 ? 8 : 4) == 0 && 256LL * g.T <= 3072 &&
                       (long long)g.T * g.Ho * g.Wo >= 2LL * g.H * g.W) {  // copy well below im2col
                pl->feed = FEED_IND_NHWC;
                pl->need_xcl = true;
                pl->need_wpack = g.T > 1;  // OIHW regrouped to (kh, kw, ci) order
            } else {
                pl->feed = FEED_IND_NCHW;
            }
            break;
        case CONV_ALGO_IM2WIN:
            pl->need_win = true;
            if (chunk_win) {  // cells padded to whole chunks, weights to (kh, kw, cp)
                pl->feed = FEED_WIN_CHUNK;
                pl->cp = cpad;
                pl->need_wpack = true;
            } else {
                pl->feed = FEED_WIN;
                pl->need_wpack = !pl->nhwc && g.T > 1;  // OIHW regrouped to (kh, kw, ci) order
            }
            break;
        case CONV_ALGO_IM2WIN_LDS:
            if (!rowwin_ok || t_forced_main_loop != CONV_MAIN_LOOP_AUTO) return CONV_ERR_UNSUPPORTED;
            pl->feed = FEED_ROWWIN;
            if (pl->nhwc) {
                // Reserved for the element-gather fallback on misaligned
                // pointers; not built otherwise.
                pl->need_ibuf = true;
            } else if (rowwin_inplace) {
                // NCHW read where it lies: the weights regrouped tap-major
                // ([slice][kh][kw][co][32 channels]), and an indirection
                // buffer reserved for the element-gather fallback on a
                // misaligned x.
                pl->feed = FEED_ROWWIN_NCHW;
                pl->need_wpack = true;
                pl->need_ibuf = true;
            } else {  // NCHW: the channels-last copy and OHWI weights
                pl->need_xcl = true;
                pl->need_wpack = true;
            }
            break;
        case CONV_ALGO_PATCH:
            if (!patch_ok) return CONV_ERR_UNSUPPORTED;
            pl->patch = true;
            pl->gm = g;
            pl->out_nchw = !pl->nhwc;
            pl->splits = 1;
            pl->total = 0;
            return CONV_OK;
        case CONV_ALGO_DIRECT:
            pl->direct = true;
            pl->gm = g;
            pl->out_nchw = !pl->nhwc;
            pl->splits = 1;
            pl->total = 0;
            return CONV_OK;
        case CONV_ALGO_IM2COL:
            // X_col in the workspace, multiplied as a plain row-major matrix.
            // Its columns follow the weights' own order: (ci, kh, kw) for
            // OIHW, (kh, kw, ci) for OHWI.
            if (g.M * g.K > kLimit) return CONV_ERR_UNSUPPORTED;
            pl->feed = FEED_ROWMAJOR;
            pl->need_col = true;
            break;
        default:
            return CONV_ERR_INVALID_ARG;
    }
    pl->gm = g;
    pl->gm.C = pl->cp;
    pl->gm.K = (long long)pl->cp * g.T;
    pl->out_nchw = !pl->nhwc && !(pl->feed == FEED_ROWMAJOR && whole);
    // GEMM rows of one main-loop pass.
    const long long Mt = (long long)pl->chunk_n * g.P;

    // Tile shape and split-K.  The 256x128 tile (wavefront tiles of 128x64,
    // a quarter less LDS and L2 traffic per MFMA) needs the 16-byte-row feeds.
    bool rows16;
    switch (pl->feed) {
        case FEED_ROWMAJOR: rows16 = g.K % VEC == 0; break;
        case FEED_IND_NHWC: rows16 = g.C % VEC == 0 && 256LL * g.T <= 3072; break;
        case FEED_IND_CHUNK: rows16 = true; break;
        case FEED_WIN: rows16 = g.C % VEC == 0; break;
        case FEED_WIN_CHUNK: rows16 = true; break;
        case FEED_GEMM_NCHW: rows16 = true; break;
        default: rows16 = false;
    }
    pl->rows16 = rows16;
    // The main loops with two wavefronts per SIMD: K tiles that stay inside
    // one tap (C a multiple of the tile: 128-byte rows for the 512-thread
    // loop, 64-byte rows for the two-blocks-per-CU loop), and an indirection
    // slice of at most 12 taps whose entries divided by C fit 16 bits.
    const int BK8 = pl->e16 ? 64 : 32, BK4 = pl->e16 ? 32 : 16;
    bool dual = rows16, oct = rows16;
    switch (pl->feed) {
        case FEED_ROWMAJOR: break;
        case FEED_WIN:
            dual = dual && g.C % BK4 == 0;
            oct = oct && g.C % BK8 == 0;
            break;
        case FEED_IND_NHWC: {
            const bool slice = g.T <= 12 && (long long)g.H * g.W <= 65535;
            dual = dual && slice && g.C % BK4 == 0;
            oct = oct && slice && g.C % BK8 == 0;
            break;
        }
        case FEED_IND_CHUNK: break;  // slice checked when the feed was chosen
        case FEED_WIN_CHUNK: break;
        case FEED_GEMM_NCHW:  // C a multiple of 32 (checked when the feed was chosen): dual always holds
            oct = oct && g.C % BK8 == 0;
            break;
        default: dual = oct = false;
    }
    const long long tiles256 = ((Mt + 255) / 256) * ((g.Co + 127) / 128);
    int BM, BN;
    if (Mt <= 64) {
        pl->tile = TILE_32x64; BM = 32; BN = 64;
    } else if (g.Co <= 64 && dual) {
        pl->tile = TILE_128x64_QUAD; BM = 128; BN = 64;
    } else if (dual && g.Co >= 256 && pl->gm.K >= 512 && ((Mt + 255) / 256) * ((g.Co + 255) / 256) > 256) {
        // Deep layers with many output channels and more 256 x 256 tiles
        // than CUs: the larger block tile loads a third fewer bytes per MFMA.
        pl->tile = TILE_256x256_OCT; BM = 256; BN = 256;
    } else if (g.Co <= 64) {
        pl->tile = TILE_128x64; BM = 128; BN = 64;
    } else if (oct && tiles256 <= 256) {
        // No more tiles than CUs: one 512-thread block per CU (two wavefronts
        // on every SIMD from one block, whole-cache-line loads).
        pl->tile = TILE_256x128_OCT; BM = 256; BN = 128;
    } else if (dual) {
        // Two blocks per CU: their prologues and epilogues overlap each
        // other's main loops, in one round or many.
        pl->tile = TILE_256x128_DUAL; BM = 256; BN = 128;
    } else if (oct) {
        pl->tile = TILE_256x128_OCT; BM = 256; BN = 128;
    } else if (rows16 && Mt >= 65536) {
        pl->tile = TILE_256x128; BM = 256; BN = 128;
    } else {
        pl->tile = TILE_128x128; BM = 128; BN = 128;
    }
    if (pl->feed == FEED_ROWWIN || pl->feed == FEED_ROWWIN_NCHW) {
        // The ping-pong form (one 512 x 128 block per CU) where all its tiles
        // fit one round on the 256 CUs and the K loop has at least 72 taps
        // (channel slices x KH x KW): its faster taps then outweigh its
        // larger per-tile prologue and epilogue.  Over several rounds, two
        // 256 x 128 blocks per CU leave a shorter last round.  (NCHW input
        // read in place has the two-block forms only.)
        const long long taps = pl->gm.K / (pl->e16 ? 32 : 16);
        if (g.Co <= 64) {
            pl->tile = TILE_256x64_ROWWIN; BM = 256; BN = 64;
        } else if (pl->feed == FEED_ROWWIN && ((Mt + 511) / 512) * ((g.Co + 127) / 128) <= 256 && taps >= 72) {
            pl->tile = TILE_512x128_ROWWIN_PP; BM = 512; BN = 128;
        } else {
            pl->tile = TILE_256x128_ROWWIN; BM = 256; BN = 128;
        }
    }
    // A forced variant (ablation) replaces the choice above when the feed
    // and shape allow it.
    const bool chunk_feed = pl->feed == FEED_IND_CHUNK || pl->feed == FEED_WIN_CHUNK;
    switch (t_forced_main_loop) {
        case CONV_MAIN_LOOP_AUTO: break;
        case CONV_MAIN_LOOP_ELEMENT_128x128:
            pl->tile = TILE_128x128; BM = 128; BN = 128;
            pl->force_element = true;
            break;
        case CONV_MAIN_LOOP_DMA_128x128:
            if (!rows16 || chunk_feed) return CONV_ERR_UNSUPPORTED;
            pl->tile = TILE_128x128; BM = 128; BN = 128;
            break;
        case CONV_MAIN_LOOP_DMA_256x128:
            if (!rows16 || chunk_feed) return CONV_ERR_UNSUPPORTED;
            pl->tile = TILE_256x128; BM = 256; BN = 128;
            break;
        case CONV_MAIN_LOOP_DUAL_256x128:
            if (!dual) return CONV_ERR_UNSUPPORTED;
            pl->tile = TILE_256x128_DUAL; BM = 256; BN = 128;
            break;
        case CONV_MAIN_LOOP_OCT_256x128:
            if (!oct) return CONV_ERR_UNSUPPORTED;
            pl->tile = TILE_256x128_OCT; BM = 256; BN = 128;
            break;
        case CONV_MAIN_LOOP_OCT_256x256:
            if (!dual) return CONV_ERR_UNSUPPORTED;
            pl->tile = TILE_256x256_OCT; BM = 256; BN = 256;
            break;
        case CONV_MAIN_LOOP_QUAD_128x64:
            if (!dual) return CONV_ERR_UNSUPPORTED;
            pl->tile = TILE_128x64_QUAD; BM = 128; BN = 64;
            break;
        case CONV_MAIN_LOOP_ABL_FULL:
        case CONV_MAIN_LOOP_ABL_NO_LDS:
        case CONV_MAIN_LOOP_ABL_ONE_STAGE:
        case CONV_MAIN_LOOP_ABL_NO_PREFETCH:
        case CONV_MAIN_LOOP_ABL_MFMA16:
        case CONV_MAIN_LOOP_ABL_VALU:
        case CONV_MAIN_LOOP_ABL_TILE64:
            if (!pl->e16 || pl->feed != FEED_IND_NHWC || pl->gm.C % 32 != 0) return CONV_ERR_UNSUPPORTED;
            pl->ablate = t_forced_main_loop;
            pl->tile = TILE_128x128;  // bookkeeping only: the ablation loop has its own tiles
            BM = BN = t_forced_main_loop == CONV_MAIN_LOOP_ABL_TILE64 ? 64 : 128;
            break;
        default:
            return CONV_ERR_INVALID_ARG;
    }
    // Workspace regions other than the split-K partials.
    size_t lowered = 0;
    if (pl->need_ibuf) lowered = align_up(lowered + (size_t)g.P * g.T * sizeof(int32_t));
    if (pl->need_win) lowered = align_up(lowered + (size_t)g.N * g.Ho * g.Wwin * g.KH * pl->cp * pl->esize);
    if (pl->need_xcl) lowered = align_up(lowered + (size_t)pl->chunk_n * pl->cp * g.H * g.W * pl->esize);
    if (pl->need_wpack) lowered = align_up(lowered + (size_t)g.Co * pl->gm.K * pl->esize);
    if (pl->need_col) lowered = align_up(lowered + (size_t)g.M * g.K * pl->esize);

    const int BK = pl->e16 ? 64 : 32;  // the main loop's K tile (128-byte LDS rows)
    long long blocks = ((Mt + BM - 1) / BM) * ((g.Co + BN - 1) / BN);
    long long ktiles = (pl->gm.K + BK - 1) / BK;
    int splits = 1;
    // Split K only where too few tiles leave most CUs idle: the two-wavefront
    // loops keep a CU busy with a single block, and the partials cost a pass
    // over M x Co fp32 values per split.
    const bool two_wave = wide_slice(pl->tile) || pl->tile == TILE_256x128_ROWWIN || pl->tile == TILE_512x128_ROWWIN_PP ||
                          pl->tile == TILE_256x64_ROWWIN;
    if (pl->feed != FEED_ROWWIN && pl->feed != FEED_ROWWIN_NCHW && !pl->ablate && blocks < (two_wave ? 64 : 256) &&
        ktiles >= 16) {
        // Enough splits to give every compute unit work, each split at least
        // 4 K tiles, and the whole workspace (partials included) kept below
        // the im2col footprint.
        long long want = (512 + blocks - 1) / blocks;
        long long by_depth = ktiles / 4;
        long long per_split = (long long)align_up((size_t)(Mt * g.Co * 4LL));
        // (The im2col baseline holds X_col itself; its partials get another
        // im2col footprint, so it splits where the lowered paths do.)
        long long room = pl->need_col ? im2col_bytes : im2col_bytes - (long long)lowered - 1;
        long long by_space = room > 0 ? room / per_split : 0;
        long long sp = want;
        if (sp > by_depth) sp = by_depth;
        if (sp > by_space) sp = by_space;
        if (sp > 1) splits = (int)sp;
    }
    long long kps = (pl->gm.K + splits - 1) / splits;
    kps = (kps + BK - 1) / BK * BK;
    splits = (int)((pl->gm.K + kps - 1) / kps);
    pl->splits = splits;
    pl->kps = (int)kps;

    size_t off = 0;
    if (pl->need_ibuf) {
        pl->off_ibuf = off;
        off = align_up(off + (size_t)g.P * g.T * sizeof(int32_t));
    }
    if (pl->need_win) {
        pl->off_win = off;
        off = align_up(off + (size_t)g.N * g.Ho * g.Wwin * g.KH * pl->cp * pl->esize);
    }
    if (pl->need_xcl) {
        pl->off_xcl = off;
        off = align_up(off + (size_t)pl->chunk_n * pl->cp * g.H * g.W * pl->esize);
    }
    if (pl->need_wpack) {
        pl->off_wpack = off;
        off = align_up(off + (size_t)g.Co * pl->gm.K * pl->esize);
    }
    if (pl->need_col) {
        pl->off_col = off;
        off = align_up(off + (size_t)g.M * g.K * pl->esize);
    }
    if (splits > 1) {
        pl->off_part = off;
        off = align_up(off + (size_t)splits * Mt * g.Co * sizeof(float));
    }
    // The ping-pong loop runs one 512 x 128 tile per CU.  With well under one
    // tile per CU, its stream-K form shares all tiles' K steps among
    // kSkBlocks blocks instead, at the cost of one fp32 partial tile per
    // block written and read back, kept below the im2col footprint.  Measured
    // on 3x3 512->512 @14 (channels-last): fp32 with 196 tiles 1116 -> 929-950
    // us; bf16 with 100 tiles 110 -> 91 us, 147 tiles 125 -> 116 us, but 196
    // tiles unchanged (the chip is then near what this loop reaches in bf16
    // with fewer CUs busy), so 16-bit types take it up to 3/4 of a tile per CU.
    const long long sk_bytes = (long long)kSkBlocks * (long long)kSkSlotBytes + 4LL * kSkBlocks;
    const bool sk_few = pl->e16 ? blocks * 4 <= kSkBlocks * 3 : blocks * 8 <= kSkBlocks * 7;
    if (pl->tile == TILE_512x128_ROWWIN_PP && sk_few && (long long)off + sk_bytes < im2col_bytes) {
        pl->sk = true;
        pl->off_sk = off;
        off = align_up(off + (size_t)sk_bytes);
    }
    pl->total = off;
    return CONV_OK;
}

}  // namespace
}  // namespace convlower

namespace convlower {
namespace {
thread_local hipEvent_t t_time_start = nullptr, t_time_stop = nullptr;
}  // namespace

void take_main_loop_events(hipEvent_t *start, hipEvent_t *stop) {
    *start = t_time_start;
    *stop = t_time_stop;
    t_time_start = t_time_stop = nullptr;
}
}  // namespace convlower

using namespace convlower;

extern "C" {

const char *conv_status_string(conv_status_t s) {
    switch (s) {
        case CONV_OK: return "CONV_OK";
        case CONV_ERR_INVALID_ARG: return "CONV_ERR_INVALID_ARG";
        case CONV_ERR_UNSUPPORTED: return "CONV_ERR_UNSUPPORTED";
        case CONV_ERR_WORKSPACE: return "CONV_ERR_WORKSPACE";
        case CONV_ERR_HIP: return "CONV_ERR_HIP";
        default: return "CONV_ERR_UNKNOWN";
    }
}

conv_status_t conv2d_output_size(int H, int W, int KH, int KW, int stride, int pad, int dilation, int *ho_out,
                                 int *wo_out) {
    if (H <= 0 || W <= 0 || KH <= 0 || KW <= 0 || stride <= 0 || dilation <= 0 || pad < 0)
        return CONV_ERR_INVALID_ARG;
    const long long Ho = out_extent(H, KH, stride, pad, dilation), Wo = out_extent(W, KW, stride, pad, dilation);
    if (Ho <= 0 || Wo <= 0) return CONV_ERR_INVALID_ARG;
    if (Ho > INT_MAX || Wo > INT_MAX) return CONV_ERR_UNSUPPORTED;
    if (ho_out) *ho_out = (int)Ho;
    if (wo_out) *wo_out = (int)Wo;
    return CONV_OK;
}

conv_status_t conv2d_fwd_workspace_size(int N, int C_in, int H, int W, int C_out, int KH, int KW, int stride,
                                        int pad, int dilation, conv_layout_t layout, conv_dtype_t dtype,
                                        conv_algo_t algo, size_t *bytes_out) {
    if (!bytes_out) return CONV_ERR_INVALID_ARG;
    Plan pl;
    conv_status_t st = make_plan(N, C_in, H, W, C_out, KH, KW, stride, pad, dilation, layout, dtype, algo, &pl);
    if (st != CONV_OK) return st;
    *bytes_out = pl.total;
    return CONV_OK;
}

conv_status_t conv2d_im2col_bytes(int N, int C_in, int H, int W, int KH, int KW, int stride, int pad,
                                  int dilation, conv_dtype_t dtype, size_t *bytes_out) {
    if (!bytes_out) return CONV_ERR_INVALID_ARG;
    if (!dtype_ok(dtype)) return CONV_ERR_INVALID_ARG;
    Geom g;
    conv_status_t st = make_geom(N, C_in, H, W, 1, KH, KW, stride, pad, dilation, &g);
    if (st != CONV_OK) return st;
    *bytes_out = (size_t)g.M * (size_t)g.K * dtype_bytes(dtype);
    return CONV_OK;
}

}  // extern "C"

namespace {

// The launch sequence of one call.  `prebuilt` (may be null) is an
// indirection buffer the caller built before; then step (b) is skipped.
// Steps the plan does not ask for (need_*) are not run.
// The main loop (and the split-K finish) for one pass: a.g is the pass's
// geometry, a.a_src / a.b / a.y its operands.
conv_status_t launch_main(const Plan &pl, GemmArgs &a, hipStream_t s) {
    const Geom &g = a.g;
    const int VEC = pl.e16 ? 8 : 4;
    auto al16 = [](const void *ptr) { return (uintptr_t)ptr % 16 == 0; };
    bool a_vec;
    switch (pl.feed) {
        case FEED_ROWMAJOR: a_vec = g.K % VEC == 0 && al16(a.a_src); break;
        case FEED_IND_NHWC:  // the vector path keeps the block's BM x KH*KW buffer slice in LDS
            a_vec = pl.rows16 && al16(a.a_src) && (wide_slice(pl.tile) || (long long)tile_rows(pl.tile) * g.T <= 3072);
            break;
        case FEED_WIN: a_vec = g.C % VEC == 0 && al16(a.a_src); break;
        case FEED_IND_CHUNK:
        case FEED_WIN_CHUNK: a_vec = al16(a.a_src) && wide_slice(pl.tile); break;
        case FEED_ROWWIN:
        case FEED_ROWWIN_NCHW:
        case FEED_GEMM_NCHW: a_vec = al16(a.a_src); break;
        default: a_vec = false;
    }
    if (pl.force_element) a_vec = false;
    // A split plan needs its partial-sum region: without it every K slice
    // would write its own partial sum (plus bias) straight into y.
    if (pl.splits > 1 && a.part == nullptr) return CONV_ERR_INVALID_ARG;
    if (pl.ablate) {
        // The ablation loop loads x and w in 16-byte pieces.
        if (!al16(a.a_src) || !al16(a.b)) return CONV_ERR_UNSUPPORTED;
        a.a_bytes = (uint32_t)((long long)g.N * g.C * g.H * g.W * (long long)pl.esize);
        a.b_bytes = (uint32_t)((long long)g.Co * g.K * (long long)pl.esize);
        return launch_ablate(a, pl.ablate, pl.out_nchw, pl.dtype, s) == hipSuccess ? CONV_OK : CONV_ERR_HIP;
    }
    bool b_vec = g.K % VEC == 0 && al16(a.b);
    // The vector paths address A and B with 32-bit buffer offsets.
    // The extent of what the A feed reads: the window tensor for im2win
    // (built here or handed in), else the input or its channels-last copy.
    const bool win = pl.feed == FEED_WIN || pl.feed == FEED_WIN_CHUNK;
    long long a_bytes = (long long)pl.esize * (win                         ? (long long)g.N * g.Ho * g.Wwin * g.KH * g.C
                                               : pl.feed == FEED_ROWMAJOR ? g.M * g.K
                                                                          : (long long)g.N * g.C * g.H * g.W);
    long long b_bytes = (long long)pl.esize * g.Co * g.K;
    if (a_bytes > kBufMax) a_vec = false;
    if (b_bytes > kBufMax) a_vec = b_vec = false;
    a.a_bytes = (uint32_t)(a_bytes > kBufMax ? kBufMax : a_bytes);
    a.b_bytes = (uint32_t)(b_bytes > kBufMax ? kBufMax : b_bytes);
    if (a_vec && !b_vec) a_vec = false;

    // Misaligned pointers fall back to the element-gather loop, which has no
    // 256x128 variant; the split count (and so the workspace) is unchanged.
    // (The in-place 1x1 NCHW feed falls back to its element-gather twin,
    // which needs no workspace either.)
    const int feed = pl.feed == FEED_GEMM_NCHW && !a_vec ? (int)FEED_NCHW_1X1 : pl.feed;
    int tile = pl.tile;
    if (!a_vec && (tile == TILE_256x128 || wide_slice(tile)))
        tile = tile == TILE_128x64_QUAD ? TILE_128x64 : TILE_128x128;
    {
        uint32_t c = (uint32_t)g.C, sh = 0;
        while (!(c & 1u)) {
            c >>= 1;
            ++sh;
        }
        uint32_t inv = c;  // Newton's iteration for the inverse of an odd number modulo 2^32
        for (int i = 0; i < 5; ++i) inv *= 2u - c * inv;
        a.c_shift = sh;
        a.c_inv = inv;
    }
    hipError_t e = pl.dtype == CONV_DTYPE_FP8_E4M3 ? launch_igemm_fp8(a, feed, pl.out_nchw, a_vec, b_vec, tile, pl.splits, s)
                   : pl.dtype == CONV_DTYPE_FP16 ? launch_igemm_f16(a, feed, pl.out_nchw, a_vec, b_vec, tile, pl.splits, s)
                   : pl.e16 ? launch_igemm_bf16(a, feed, pl.out_nchw, a_vec, b_vec, tile, pl.splits, s)
                            : launch_igemm_f32(a, feed, pl.out_nchw, a_vec, b_vec, tile, pl.splits, s);
    if (e != hipSuccess) return CONV_ERR_HIP;
    if (pl.splits > 1) {
        if (launch_splitk_reduce(a.part, a.bias, a.y, g, pl.splits, pl.out_nchw, pl.dtype, s) != hipSuccess)
            return CONV_ERR_HIP;
    }
    return CONV_OK;
}


conv_status_t run(const Plan &pl, const void *x, const void *w, const void *bias, void *y, const int32_t *prebuilt,
                  conv_stream_t stream, void *workspace, size_t workspace_bytes) {
    if (!x || !w || !y) return CONV_ERR_INVALID_ARG;
    const size_t es = pl.esize;
    const size_t eo = pl.dtype == CONV_DTYPE_FP8_E4M3 ? 2 : es;  // y and bias elements
    if ((uintptr_t)x % es || (uintptr_t)w % es || (uintptr_t)y % eo || (bias && (uintptr_t)bias % eo))
        return CONV_ERR_INVALID_ARG;
    if (pl.dtype == CONV_DTYPE_FP8_E4M3 && ((uintptr_t)x % 16 || (uintptr_t)w % 16)) return CONV_ERR_UNSUPPORTED;
    if (pl.total > 0 && (!workspace || workspace_bytes < pl.total)) return CONV_ERR_WORKSPACE;
    if (pl.total > 0 && (uintptr_t)workspace % 16) return CONV_ERR_INVALID_ARG;

    hipStream_t s = (hipStream_t)stream;
    const Geom &g = pl.g;
    char *ws = (char *)workspace;
    if (pl.direct)
        return launch_direct_conv(x, w, bias, y, g, pl.nhwc, pl.dtype, s) == hipSuccess ? CONV_OK : CONV_ERR_HIP;
    if (pl.patch)
        return launch_patch_conv(x, w, bias, y, g, pl.nhwc, pl.dtype, s) == hipSuccess ? CONV_OK : CONV_ERR_HIP;

    GemmArgs a;
    memset(&a, 0, sizeof(a));
    if (pl.chunk_n < g.N) {
        // NCHW 1x1 in parts: each part of the batch is copied channels-last
        // into the same workspace region, then multiplied as a plain GEMM
        // whose NCHW output lands in that part's slice of y.  A split plan
        // reuses one partial-sum region for every part (the parts run one
        // after another on the stream, each finished by its own reduce).
        void *xc = ws + pl.off_xcl;
        float *part = pl.splits > 1 ? (float *)(ws + pl.off_part) : nullptr;
        for (int n0 = 0; n0 < g.N; n0 += pl.chunk_n) {
            Geom gc = g;
            gc.N = g.N - n0 < pl.chunk_n ? g.N - n0 : pl.chunk_n;
            gc.M = (long long)gc.N * g.P;
            const char *xs = (const char *)x + (size_t)n0 * g.C * g.H * g.W * es;
            if (launch_prep(xs, false, xc, g.C, nullptr, nullptr, false, nullptr, gc, (int)pl.esize, s) != hipSuccess)
                return CONV_ERR_HIP;
            a.g = gc;
            a.bias = bias;
            a.y = (char *)y + (size_t)n0 * g.Co * g.P * es;
            a.k_per_split = pl.kps;
            a.b = w;
            a.a_src = xc;
            a.part = part;
            conv_status_t st = launch_main(pl, a, s);
            if (st != CONV_OK) return st;
        }
        return CONV_OK;
    }
    a.g = pl.gm;
    a.bias = bias;
    a.y = y;
    a.k_per_split = pl.kps;
    a.b = w;
    a.a_src = x;

    if (pl.feed == FEED_ROWWIN && pl.nhwc && ((uintptr_t)x % 16 || (uintptr_t)w % 16)) {
        // Operands the window-row loop cannot read in 16-byte chunks: the
        // element-gather loop through the indirection buffer reserved in
        // the workspace instead.
        Plan fb = pl;
        fb.feed = FEED_IND_NHWC;
        fb.tile = TILE_128x128;
        fb.sk = false;
        return run(fb, x, w, bias, y, prebuilt, stream, workspace, workspace_bytes);
    }
    if (pl.feed == FEED_ROWWIN_NCHW && (uintptr_t)x % 16) {
        // An x the window-row loop cannot load in 16-byte chunks: the
        // element-gather loop through the indirection buffer reserved in the
        // workspace, with the weights as they lie (K in (ci, kh, kw) order).
        Plan fb = pl;
        fb.feed = FEED_IND_NCHW;
        fb.tile = TILE_128x128;
        fb.need_wpack = false;
        fb.sk = false;
        return run(fb, x, w, bias, y, prebuilt, stream, workspace, workspace_bytes);
    }
    // Offsets of the indirection buffer follow the layout the main loop reads.
    const bool ib_rows = pl.feed == FEED_IND_NHWC;
    int32_t *ib_build = nullptr;  // buffer still to build
    if (prebuilt) {
        a.ibuf = prebuilt;
    } else if (pl.need_ibuf && pl.feed != FEED_ROWWIN && pl.feed != FEED_ROWWIN_NCHW) {
        ib_build = (int32_t *)(ws + pl.off_ibuf);
        a.ibuf = ib_build;
    }
    void *wp = pl.need_wpack ? (void *)(ws + pl.off_wpack) : nullptr;
    bool wp_done = false;
    // Stream-K: partial tiles, then the flags, which start each call at zero.
    uint32_t *skf = nullptr;
    if (pl.sk) {
        a.skp = (float *)(ws + pl.off_sk);
        skf = (uint32_t *)(ws + pl.off_sk + (size_t)kSkBlocks * kSkSlotBytes);
        a.skf = skf;
    }
    if (pl.need_xcl) {
        // One launch: the channels-last copy of x (rows of cp channels), the
        // indirection buffer over it and the weights in (kh, kw, ci) order
        // (and the stream-K flags cleared).
        void *xc = ws + pl.off_xcl;
        if (launch_prep(x, pl.nhwc, xc, pl.cp, ib_build, w, pl.nhwc, wp, g, (int)pl.esize, s, skf,
                        skf ? kSkBlocks : 0) != hipSuccess)
            return CONV_ERR_HIP;
        skf = nullptr;
        a.a_src = xc;
        ib_build = nullptr;
        wp_done = true;
    }
    if (ib_build && launch_build_indirection(ib_build, g, ib_rows, s) != hipSuccess) return CONV_ERR_HIP;
    if (skf && launch_zero_words(skf, kSkBlocks, s) != hipSuccess) return CONV_ERR_HIP;
    if (pl.need_col) {
        void *xcol = ws + pl.off_col;
        if (launch_im2col(x, xcol, g, pl.nhwc, pl.e16, s) != hipSuccess) return CONV_ERR_HIP;
        a.a_src = xcol;
    }
    if (pl.need_win) {
        void *xw = ws + pl.off_win;
        if (pl.feed == FEED_WIN_CHUNK) {
            if (launch_im2win_pad(x, xw, g, pl.cp, pl.nhwc, pl.e16, s) != hipSuccess) return CONV_ERR_HIP;
            // Weights zero-padded to (kh, kw, cp) order from either layout.
            if (launch_prep(nullptr, pl.nhwc, nullptr, pl.cp, nullptr, w, pl.nhwc, wp, g, (int)pl.esize, s) != hipSuccess)
                return CONV_ERR_HIP;
            wp_done = true;
        } else if (launch_im2win(x, xw, g, pl.nhwc, pl.e16, s) != hipSuccess) {
            return CONV_ERR_HIP;
        }
        a.a_src = xw;
    }
    if (wp) {
        if (pl.feed == FEED_ROWWIN_NCHW) {
            if (launch_pack_weights_tapmajor(w, wp, g, 32, s) != hipSuccess) return CONV_ERR_HIP;
        } else if (!wp_done && launch_pack_weights_ohwi(w, wp, g, pl.e16, s) != hipSuccess) {
            return CONV_ERR_HIP;
        }
        a.b = wp;
    }
    if (pl.splits > 1) a.part = (float *)(ws + pl.off_part);

    return launch_main(pl, a, s);
}

// ---- scratch memory of the no-allocation entry point ------------------------
// One array per GPU, in the library's own device memory, that
// conv2d_fwd_noalloc uses as its workspace.  In host code `scratch` names a
// host-side stand-in, not the device array: its device address is looked up
// once per device (hipGetSymbolAddress, with that device current) and only
// that address is ever passed to a kernel.
constexpr size_t kScratchBytes = (size_t)CONV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on device `dev` (nullptr on a HIP error).
void *scratch_on(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p) return p;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void *addr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !addr) return nullptr;
    g_scratch_ptr[dev].store(addr, std::memory_order_release);
    return addr;
}

}  // namespace

extern "C" {

conv_status_t conv2d_fwd_noalloc(const void *x, const void *w, const void *bias, void *y, int N, int C_in, int H,
                                 int W, int C_out, int KH, int KW, int stride, int pad, int dilation,
                                 conv_layout_t layout, conv_dtype_t dtype, conv_stream_t stream, conv_algo_t algo) {
    Plan pl;
    conv_status_t st = make_plan(N, C_in, H, W, C_out, KH, KW, stride, pad, dilation, layout, dtype, algo, &pl);
    if (st != CONV_OK) return st;
    if (pl.total > kScratchBytes && pl.sk) {  // the stream-K regions are the last: without them it may fit
        pl.sk = false;
        pl.total = pl.off_sk;
    }
    if (pl.total > kScratchBytes) return CONV_ERR_WORKSPACE;
    void *ws = nullptr;
    if (pl.total > 0) {
        // The device the work runs on: the stream's, or the current one for
        // the default stream.
        int dev = -1;
        const hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
        if (e != hipSuccess) return CONV_ERR_HIP;
        ws = scratch_on(dev);
        if (!ws) return CONV_ERR_HIP;
    }
    return run(pl, x, w, bias, y, nullptr, stream, ws, ws ? kScratchBytes : 0);
}

conv_status_t conv2d_fwd(const void *x, const void *w, const void *bias, void *y, int N, int C_in, int H, int W,
                         int C_out, int KH, int KW, int stride, int pad, int dilation, conv_layout_t layout,
                         conv_dtype_t dtype, conv_stream_t stream, void *workspace, size_t workspace_bytes,
                         conv_algo_t algo) {
    Plan pl;
    conv_status_t st = make_plan(N, C_in, H, W, C_out, KH, KW, stride, pad, dilation, layout, dtype, algo, &pl);
    if (st != CONV_OK) return st;
    return run(pl, x, w, bias, y, nullptr, stream, workspace, workspace_bytes);
}

conv_status_t conv2d_main_loop(const void *lowered, const int32_t *indirection, const void *w_ohwi, const void *bias,
                               void *y, int N, int C_in, int H, int W, int C_out, int KH, int KW, int stride, int pad,
                               int dilation, conv_algo_t algo, conv_layout_t out_layout, conv_dtype_t dtype,
                               conv_stream_t stream, void *workspace, size_t workspace_bytes) {
    if (algo != CONV_ALGO_INDIRECT && algo != CONV_ALGO_IM2WIN && algo != CONV_ALGO_IM2COL)
        return CONV_ERR_INVALID_ARG;
    if (out_layout != CONV_LAYOUT_NCHW && out_layout != CONV_LAYOUT_NHWC) return CONV_ERR_INVALID_ARG;
    // The lowered operands are channels-last, so plan as for an NHWC call.
    Plan pl;
    conv_status_t st =
        make_plan(N, C_in, H, W, C_out, KH, KW, stride, pad, dilation, CONV_LAYOUT_NHWC, dtype, algo, &pl, false);
    if (st != CONV_OK) return st;
    if (algo == CONV_ALGO_INDIRECT && (!indirection || (uintptr_t)indirection % 4)) return CONV_ERR_INVALID_ARG;
    pl.out_nchw = out_layout == CONV_LAYOUT_NCHW;
    pl.need_ibuf = pl.need_win = pl.need_xcl = pl.need_wpack = pl.need_col = false;
    // Only the split-K partials live in the workspace here; with less room
    // than they need the main loop runs unsplit.
    pl.off_part = 0;
    pl.total = pl.splits > 1 ? align_up((size_t)pl.splits * pl.g.M * pl.g.Co * sizeof(float)) : 0;
    if (pl.total > 0 && (!workspace || workspace_bytes < pl.total)) {
        const int BK = pl.e16 ? 64 : 32;
        pl.splits = 1;
        pl.kps = (int)((pl.gm.K + BK - 1) / BK * BK);
        pl.total = 0;
    }
    return run(pl, lowered, w_ohwi, bias, y, indirection, stream, workspace, workspace_bytes);
}

conv_status_t conv2d_force_main_loop(conv_main_loop_t variant) {
    if (variant < CONV_MAIN_LOOP_AUTO || variant > CONV_MAIN_LOOP_ABL_TILE64) return CONV_ERR_INVALID_ARG;
    t_forced_main_loop = variant;
    return CONV_OK;
}

conv_status_t conv2d_time_next_main_loop(void *start_event, void *stop_event) {
    t_time_start = (hipEvent_t)start_event;
    t_time_stop = (hipEvent_t)stop_event;
    return CONV_OK;
}

conv_status_t conv2d_build_indirection(int32_t *buf, int C_in, int H, int W, int KH, int KW, int stride, int pad,
                                       int dilation, conv_layout_t layout, conv_stream_t stream) {
    if (layout != CONV_LAYOUT_NCHW && layout != CONV_LAYOUT_NHWC) return CONV_ERR_INVALID_ARG;
    Geom g;
    conv_status_t st = make_geom(1, C_in, H, W, 1, KH, KW, stride, pad, dilation, &g);
    if (st != CONV_OK) return st;
    if (!buf || (uintptr_t)buf % 4) return CONV_ERR_INVALID_ARG;
    if (!sizes_supported(g)) return CONV_ERR_UNSUPPORTED;
    if (launch_build_indirection(buf, g, layout == CONV_LAYOUT_NHWC, (hipStream_t)stream) != hipSuccess)
        return CONV_ERR_HIP;
    return CONV_OK;
}

conv_status_t conv2d_im2win_transform(const void *x, void *xwin, int N, int C_in, int H, int W, int KH, int KW,
                                      int stride, int pad, int dilation, conv_layout_t layout, conv_dtype_t dtype,
                                      conv_stream_t stream) {
    if (layout != CONV_LAYOUT_NCHW && layout != CONV_LAYOUT_NHWC) return CONV_ERR_INVALID_ARG;
    if (!dtype_ok(dtype)) return CONV_ERR_INVALID_ARG;
    if (dtype == CONV_DTYPE_FP8_E4M3) return CONV_ERR_UNSUPPORTED;  // 16- and 32-bit elements only
    Geom g;
    conv_status_t st = make_geom(N, C_in, H, W, 1, KH, KW, stride, pad, dilation, &g);
    if (st != CONV_OK) return st;
    size_t es = dtype_bytes(dtype);
    if (!x || !xwin || (uintptr_t)x % es || (uintptr_t)xwin % es) return CONV_ERR_INVALID_ARG;
    if (!sizes_supported(g)) return CONV_ERR_UNSUPPORTED;
    if (launch_im2win(x, xwin, g, layout == CONV_LAYOUT_NHWC, es == 2, (hipStream_t)stream) !=
        hipSuccess)
        return CONV_ERR_HIP;
    return CONV_OK;
}

conv_status_t conv2d_im2col_transform(const void *x, void *xcol, int N, int C_in, int H, int W, int KH, int KW,
                                      int stride, int pad, int dilation, conv_layout_t layout, conv_dtype_t dtype,
                                      conv_stream_t stream) {
    if (layout != CONV_LAYOUT_NCHW && layout != CONV_LAYOUT_NHWC) return CONV_ERR_INVALID_ARG;
    if (!dtype_ok(dtype)) return CONV_ERR_INVALID_ARG;
    if (dtype == CONV_DTYPE_FP8_E4M3) return CONV_ERR_UNSUPPORTED;  // 16- and 32-bit elements only
    Geom g;
    conv_status_t st = make_geom(N, C_in, H, W, 1, KH, KW, stride, pad, dilation, &g);
    if (st != CONV_OK) return st;
    size_t es = dtype_bytes(dtype);
    if (!x || !xcol || (uintptr_t)x % es || (uintptr_t)xcol % es) return CONV_ERR_INVALID_ARG;
    if (!sizes_supported(g) || g.M * g.K > kLimit) return CONV_ERR_UNSUPPORTED;
    if (launch_im2col(x, xcol, g, layout == CONV_LAYOUT_NHWC, es == 2, (hipStream_t)stream) !=
        hipSuccess)
        return CONV_ERR_HIP;
    return CONV_OK;
}

}  // extern "C"
