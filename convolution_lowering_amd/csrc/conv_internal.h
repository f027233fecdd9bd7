// Internal declarations shared by the host planner and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "convlower.h"

namespace convlower {

// How the main loop reads row m, column k of the virtual X_col operand.
// K is enumerated in the order given beside each feed; the weight operand
// B[co][k] is read in the same order.
enum Feed : int {
    FEED_ROWMAJOR = 0,  // A = the input itself as an [M][K] matrix (1x1 NHWC, whole-input kernel); K natural
    FEED_NCHW_1X1 = 1,  // A[m][ci] = x[n][ci][pixel] (1x1 stride-1 NCHW); K = ci
    FEED_IND_NHWC = 2,  // through the indirection buffer, channels-last input; K = (kh, kw, ci)
    FEED_IND_NCHW = 3,  // through the indirection buffer, NCHW input; K = (ci, kh, kw)
    FEED_WIN = 4,       // out of the window-ordered tensor (either input layout); K = (kh, kw, ci)
    // C not a multiple of the 16-byte chunk: channels zero-padded to the next
    // multiple (C = that in the main loop's geometry) and every chunk of a K
    // tile addressed on its own, tap q / (C/VEC); K = (kh, kw, ci)
    FEED_IND_CHUNK = 5,  // indirection buffer over the padded channels-last copy
    FEED_WIN_CHUNK = 6,  // window-ordered tensor with padded cells
    FEED_ROWWIN = 7,     // channels-last input, each block's window rows staged in LDS (stride 1, dilation 1,
                         // KW = 3); K = (ci slice, kh, kw)
    FEED_ROWWIN_NCHW = 8,  // the same window rows, read from NCHW input where it lies (16-bit types); K as
                           // FEED_ROWWIN, weights in (kh, kw, ci) order
    FEED_GEMM_NCHW = 9,  // 1x1 stride-1 NCHW input read where it lies (16-bit types): each K tile's channel
                         // rows of BM pixels staged in LDS as they lie, MFMA fragments formed by transpose
                         // reads; K = ci, weights [Co][C] as they lie
};
constexpr int kNumFeeds = 10;
// Raw chunks (8 input columns each) one 256-pixel tile of the NCHW window-row
// loop stages per channel, at most.
constexpr int kRowWinRawChunks = 40;
// Output rows a 256-pixel tile of the LDS window-row loop may span.
constexpr int kRowWinMaxSeg = 32;

struct Geom {
    int N, C, H, W, Co, KH, KW, s, p, d;
    int Ho, Wo, P, T, Wwin;  // P = Ho*Wo output pixels per image, T = KH*KW taps
    long long M, K;          // GEMM rows (N*P) and depth (C*T)
};

struct GemmArgs {
    const void *a_src;    // x, or the window-ordered tensor for FEED_WIN
    const int32_t *ibuf;  // indirection buffer for FEED_IND_*
    const void *b;        // weights as [Co][K] in the feed's K order
    const void *bias;     // nullable
    void *y;              // output (final layout)
    float *part;          // split-K partial sums [splits][M][Co], or nullptr
    Geom g;
    int k_per_split;      // multiple of the K tile; == K rounded up when not split
    uint32_t a_bytes;     // size of a_src in bytes (< 2^31 on the vector paths)
    uint32_t b_bytes;     // size of b in bytes (< 2^31 on the vector paths)
    uint32_t c_shift;     // C = c_odd << c_shift; c_inv * c_odd == 1 (mod 2^32): exact
    uint32_t c_inv;       // division of a channels-last indirection entry by C
    // Stream-K form of the ping-pong window-row loop (null: one block per
    // tile): the K steps of all tiles shared evenly by kSkBlocks blocks.  A
    // tile split between blocks is finished by the block that holds its last
    // K step, which adds the fp32 partial tiles of the others (one slot of
    // kSkSlotBytes per block in skp, and a ready flag per block in skf,
    // zero when the launch starts).
    float *skp;
    uint32_t *skf;
};
// Stream-K grid: 32 blocks on each of MI355X's 8 XCDs (one per compute unit),
// and the bytes of one block's partial tile (512 x 128 fp32 sums).
constexpr int kSkBlocks = 256;
constexpr size_t kSkSlotBytes = 512 * 128 * sizeof(float);

// Tile shapes of the main loop (block = 256 threads = 4 wavefronts, 2x2).
// TILE_256x128_DUAL and TILE_256x128_OCT are the 256 x 128 main loops with
// two wavefronts per SIMD (two 256-thread blocks per compute unit with 64-byte
// K tiles, or one 512-thread block with 128-byte K tiles; TILE_128x64_QUAD is
// the four-blocks-per-CU loop for at most 64 output channels; the 256x256 OCT
// tile is a 512-thread block of eight 128 x 64 wavefront tiles),
// for 16-byte-row feeds whose K tiles stay inside one tap.
enum Tile : int {
    TILE_128x128 = 0,
    TILE_128x64 = 1,
    TILE_32x64 = 2,
    TILE_256x128 = 3,
    TILE_256x128_DUAL = 4,
    TILE_256x128_OCT = 5,
    TILE_128x64_QUAD = 6,
    TILE_256x256_OCT = 7,
    TILE_256x128_ROWWIN = 8,     // the LDS window-row loop of igemm_rowwin.h (FEED_ROWWIN[_NCHW] only)
    TILE_512x128_ROWWIN_PP = 9,  // its one-block-per-CU ping-pong form, igemm_rowwin_pp.h (FEED_ROWWIN only)
    TILE_256x64_ROWWIN = 10,     // its 256 x 64 form for at most 64 output channels (FEED_ROWWIN[_NCHW] only)
    TILE_COUNT = 11
};

hipError_t launch_igemm_bf16(const GemmArgs &a, int feed, bool out_nchw, bool a_vec, bool b_vec,
                             int tile, int splits, hipStream_t st);
hipError_t launch_igemm_f32(const GemmArgs &a, int feed, bool out_nchw, bool a_vec, bool b_vec,
                            int tile, int splits, hipStream_t st);
hipError_t launch_igemm_f16(const GemmArgs &a, int feed, bool out_nchw, bool a_vec, bool b_vec,
                            int tile, int splits, hipStream_t st);
// fp8 e4m3 inputs, bf16 bias and output; FEED_ROWWIN only.
hipError_t launch_igemm_fp8(const GemmArgs &a, int feed, bool out_nchw, bool a_vec, bool b_vec,
                            int tile, int splits, hipStream_t st);
// dtype: 0 fp32, 1 bf16, 2 fp16 (the conv_dtype_t values).
hipError_t launch_splitk_reduce(const float *part, const void *bias, void *y, const Geom &g,
                                int splits, bool out_nchw, int dtype, hipStream_t st);
hipError_t launch_build_indirection(int32_t *buf, const Geom &g, bool nhwc, hipStream_t st);
hipError_t launch_im2win(const void *x, void *xwin, const Geom &g, bool nhwc, bool bf16,
                         hipStream_t st);
// Direct convolution (no lowering, no matrix core): y from x, w and bias in
// `nhwc` or NCHW layout.
hipError_t launch_direct_conv(const void *x, const void *w, const void *bias, void *y, const Geom &g, bool nhwc,
                              int dtype, hipStream_t st);

// Inputs with at most four channels, input patches staged in LDS
// (patch_conv.hip): whether a layer fits (and its output rows per unit), and
// the launch.  Both layouts; x, w and y in `nhwc` or NCHW layout.
bool patch_conv_plan(const Geom &g, int dtype, int *R_out);
hipError_t launch_patch_conv(const void *x, const void *w, const void *bias, void *y, const Geom &g, bool nhwc,
                             int dtype, hipStream_t st);

// X_col, rows (n, ho, wo), columns (ci, kh, kw) for NCHW input, (kh, kw, ci)
// for NHWC input.
hipError_t launch_im2col(const void *x, void *xcol, const Geom &g, bool nhwc, bool bf16, hipStream_t st);

// The ablation main loop (igemm_ablate.h): `variant` a CONV_MAIN_LOOP_ABL_
// value, 16-bit dtype, channels-last input through the NHWC indirection buffer.
hipError_t launch_ablate(const GemmArgs &a, int variant, bool out_nchw, int dtype, hipStream_t st);

// Events the next main-loop launch of this host thread stamps (null: none);
// reading them clears the request.
void take_main_loop_events(hipEvent_t *start, hipEvent_t *stop);

// The window-ordered tensor with each cell's channels zero-padded to cp (a
// multiple of the 16-byte chunk, >= C).
hipError_t launch_im2win_pad(const void *x, void *xwin, const Geom &g, int cp, bool nhwc, bool bf16,
                             hipStream_t st);
// One launch: the channels-last copy of x with cp channels per pixel row
// (from NCHW or NHWC input; null x_cl: none), plus (when given) the
// indirection buffer over that copy and the weights in (kh, kw, ci) order
// with cp channels (from OIHW or OHWI).  Channels past C are zeros.
// `zero` (when given): nzero 32-bit words set to zero by the same launch.
hipError_t launch_prep(const void *x, bool nhwc_in, void *x_cl, int cp, int32_t *ib, const void *w, bool w_ohwi,
                       void *w_out, const Geom &g, int es, hipStream_t st, uint32_t *zero = nullptr,
                       int nzero = 0);
// n 32-bit words set to zero (a kernel, not a memset: safe in captured graphs).
hipError_t launch_zero_words(uint32_t *p, int n, hipStream_t st);
// 16-bit OIHW weights regrouped tap-major, [C/bk][KH][KW][Co][bk], for the NCHW
// window-row loop (C a multiple of bk).
hipError_t launch_pack_weights_tapmajor(const void *w, void *o, const Geom &g, int bk, hipStream_t st);
hipError_t launch_pack_weights_ohwi(const void *w_oihw, void *w_ohwi, const Geom &g, bool bf16,
                                    hipStream_t st);

}  // namespace convlower
