/*
 * convlower -- forward pass of a batched 2-D convolution on MI355X (gfx950),
 * lowered onto a dense MFMA contraction without materialising im2col.
 *
 * What is computed (cross-correlation, zero padding, one stride / pad /
 * dilation for both spatial axes):
 *
 *   y[n,co,ho,wo] = bias[co] + sum_{ci<C_in, kh<KH, kw<KW}
 *                     x[n, ci, ho*stride + kh*dilation - pad, wo*stride + kw*dilation - pad] * w[co,ci,kh,kw]
 *
 * with x taken as zero outside the image.  This is the seven-loop definition
 * of "Unifying Convolutions and GEMM" (section 1) with the padding and bias of
 * its section 5 and the dilation named by The Indirect Convolution Algorithm
 * (abstract).  Output extents: Ho = (H + 2*pad - dilation*(KH-1) - 1)/stride + 1,
 * likewise Wo (section 5 of the same page gives the dilation-1 form).
 *
 * The contraction is  Y_col = X_col * W_row^T  ("Unifying Convolutions and
 * GEMM", section 3) with M = N*Ho*Wo rows, C_out columns and K = C_in*KH*KW,
 * but X_col is never built: the MFMA main loop gathers its rows either
 * through an indirection buffer (The Indirect Convolution Algorithm,
 * abstract) or out of a window-ordered copy of the input ("Im2win: An
 * Efficient Convolution Paradigm on GPU", abstract).  1x1 stride-1 unpadded
 * layers, and layers whose kernel covers the whole unpadded input, are
 * already plain matrix products and are fed directly.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout (one value for x, w and y together; every tensor dense, contiguous):
 *   CONV_LAYOUT_NCHW: x[N][C_in][H][W], w[C_out][C_in][KH][KW], y[N][C_out][Ho][Wo]
 *   CONV_LAYOUT_NHWC: x[N][H][W][C_in], w[C_out][KH][KW][C_in], y[N][Ho][Wo][C_out]
 * Dtype (one value for x, w, bias and y): fp32, or bf16 stored as raw 16-bit
 *   words.  Products are accumulated in fp32; the bias is added in fp32; bf16
 *   results are rounded once, to nearest-even, at the store.
 * Pointers are device pointers (HIP), except where stated.  The caller owns
 *   every buffer; the library allocates nothing, never synchronises the
 *   device, and enqueues all work on `stream` (NULL = the default stream).
 *   Buffers must not overlap.  Pointers need only the alignment of their
 *   element type.
 * State kept between calls: only (1) the calling host thread's main-loop
 *   override (conv2d_force_main_loop, until it is reset to AUTO) and its
 *   pending request for timing stamps (conv2d_time_next_main_loop, consumed
 *   by the next main-loop launch), both thread-local and set by nothing else;
 *   and (2) the scratch array of conv2d_fwd_noalloc, one per GPU, and its
 *   looked-up device address.  Every other call's result depends on its
 *   arguments alone.
 * Errors are returned as conv_status_t; no call launches anything when it
 *   returns an error detected on the host.
 */
#ifndef CONVLOWER_H
#define CONVLOWER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same underlying type as hipStream_t. */
struct ihipStream_t;
typedef struct ihipStream_t *conv_stream_t;

typedef enum { CONV_LAYOUT_NCHW = 0, CONV_LAYOUT_NHWC = 1 } conv_layout_t;
/* Element type of x, w, bias and y (all the same); the sums are fp32 in
 * every case, rounded once to the element type at the store.
 * CONV_DTYPE_FP8_E4M3 is the exception: x and w hold OCP fp8 e4m3 bytes
 * (1 sign, 4 exponent, 3 mantissa bits, bias 7, no infinities), bias and y
 * are bf16, and y is rounded once to bf16.  It is served by the window-row
 * loop (CONV_ALGO_IM2WIN_LDS, which AUTO means here) for 3x3-wide stride-1
 * layers with C_in a multiple of 64 and x and w 16-byte aligned:
 * channels-last tensors as they lie (no workspace), NCHW tensors with H*W a
 * multiple of 4 through a channels-last copy of x and the weights regrouped
 * (kh, kw, ci) in the workspace (|x| + |w| bytes); any other fp8 request
 * returns CONV_ERR_UNSUPPORTED. */
typedef enum { CONV_DTYPE_FP32 = 0, CONV_DTYPE_BF16 = 1, CONV_DTYPE_FP16 = 2, CONV_DTYPE_FP8_E4M3 = 3 } conv_dtype_t;

/* Which lowering feeds the contraction.
 *   AUTO      1x1 stride-1 unpadded, or kernel == whole unpadded input: the
 *             plain-GEMM feed; channels not a whole number of 16-byte chunks
 *             with more than 12 taps: IM2WIN (cells padded to whole chunks)
 *             when that tensor is smaller than im2col (PATCH first where
 *             C_in <= 4 and it applies); shapes IM2WIN_LDS
 *             serves with at least 256 of its tiles (256 x 64 up to 64
 *             output channels, else 256 x 128): IM2WIN_LDS; otherwise
 *             INDIRECT.
 *   INDIRECT  indirection buffer of per-(output pixel, tap) input offsets.
 *   IM2WIN    window-ordered copy of the input in the workspace (each
 *             (column, kernel row) cell padded to one 16-byte chunk when
 *             that is smaller than im2col and C is below a chunk).
 *   GEMM      the input read as the GEMM operand as it lies in memory; only
 *             valid for the two plain-GEMM shapes named under AUTO (The
 *             Indirect Convolution Algorithm, abstract: a 1x1 convolution is
 *             a GEMM call; "Unifying Convolutions and GEMM", section 4: a
 *             whole-input kernel is a dense layer).  1x1 NCHW in a 16-bit
 *             type with C_in a multiple of 32, H*W a multiple of 8 and more
 *             than 64 output pixels: x[n] ([C_in][H*W]) is the operand
 *             transposed and is read where it lies, MFMA fragments formed by
 *             LDS transpose reads; no workspace beyond split-K partials (x
 *             or w not 16-byte aligned: the element-gather loop, same
 *             workspace).  Other 1x1 NCHW input with N >= 2 and C_in a
 *             multiple of 8 (16-bit) or 4 (fp32): half the batch at a time
 *             copied channels-last (workspace |x|/2); else the
 *             element-gather loop.
 *   IM2COL    the baseline the lowering avoids: X_col materialised in the
 *             workspace ("Unifying Convolutions and GEMM", section 2; the
 *             workspace is then the whole im2col footprint), then the same
 *             MFMA main loop multiplies it as a row-major matrix (section 3).
 *             Never chosen by AUTO.
 *   DIRECT    the other baseline: the seven-loop definition ("Unifying
 *             Convolutions and GEMM", section 1) run directly on the vector
 *             ALUs, one thread per output pixel and 8 output channels, fp32
 *             accumulation; no lowering, no workspace, no matrix core
 *             ("Im2win: An Efficient Convolution Paradigm on GPU", abstract,
 *             compares against such a kernel).  Never chosen by AUTO.
 *   IM2WIN_LDS  the window-ordered layout built in LDS, never in memory:
 *             each block stages, per channel slice and kernel row, the runs
 *             of input pixels its output rows' windows cover, and the KW taps
 *             of that kernel row read their MFMA operands from the one run.
 *             A grid of at most 256 tiles of 512 x 128 over a K loop of at
 *             least 72 taps runs as one block per compute unit whose two
 *             halves alternate between multiplying and loading; other
 *             shapes as two 256 x 128 blocks per unit.
 *             Stride 1, dilation 1, KW = 3, C_in a multiple of 32 (16-bit
 *             types) or 16 (fp32), an output at least 9 pixels wide (a
 *             256-pixel tile then spans at most 32 output rows), x and w
 *             below 2^31 bytes only, else CONV_ERR_UNSUPPORTED.  NCHW input
 *             of a 16-bit type with an even W and at most 256 output
 *             channels is read where it lies when each 256-pixel tile's
 *             input runs fit the loop's LDS buffer (at most 40 runs of 8
 *             in-image columns per channel; true for outputs at least 14
 *             wide): its workspace is the weights regrouped tap-major plus a
 *             spare indirection buffer, used only when x is not 16-byte
 *             aligned (then the element-gather loop runs).  Other NCHW
 *             input: the channels-last copy of x and OHWI weights.  NHWC: a spare
 *             indirection buffer, used only when x or w is not 16-byte
 *             aligned (then the call runs the element-gather loop).  Deep
 *             channels-last layers with fewer 512 x 128 output tiles than
 *             compute units (3/4 of them for 16-bit types, 7/8 for fp32)
 *             share the tiles' K steps among 256 blocks; their workspace adds
 *             256 fp32 partial tiles of 512 x 128 and 256 flags (64 MB + 1
 *             KB), where the total stays below the im2col footprint.
 *   PATCH     inputs with at most 4 channels: the indirect convolution with
 *             the input rows of a few output rows staged in LDS (channels
 *             padded to 4) and each tap's pixel addressed there, so that a
 *             16-byte MFMA operand chunk is two taps (16-bit types) or one
 *             (fp32); the weights of 64 output channels stay in registers.
 *             C_in <= 4, KH*KW <= 64 (16-bit) or 32 (fp32), and the staged
 *             rows of one output row within 24 KB, else
 *             CONV_ERR_UNSUPPORTED.  No workspace.  */
typedef enum {
    CONV_ALGO_AUTO = 0,
    CONV_ALGO_INDIRECT = 1,
    CONV_ALGO_IM2WIN = 2,
    CONV_ALGO_GEMM = 3,
    CONV_ALGO_IM2COL = 4,
    CONV_ALGO_DIRECT = 5,
    CONV_ALGO_IM2WIN_LDS = 6,
    CONV_ALGO_PATCH = 7
} conv_algo_t;

typedef enum {
    CONV_OK = 0,
    CONV_ERR_INVALID_ARG = 1, /* bad size, enum, NULL pointer, or no output placement fits */
    CONV_ERR_UNSUPPORTED = 2, /* valid request this library does not implement (e.g. GEMM on a windowed layer, sizes past 2^31 elements) */
    CONV_ERR_WORKSPACE = 3,   /* workspace_bytes below the size the query returns, or NULL workspace when it is not 0 */
    CONV_ERR_HIP = 4          /* a HIP launch reported an error */
} conv_status_t;

/* Human-readable name of a status code (static storage). */
const char *conv_status_string(conv_status_t status);

/* Output extents for the geometry (host only, no HIP call).  Returns
 * CONV_ERR_INVALID_ARG if a size is not positive, pad < 0, or no window
 * placement fits; CONV_ERR_UNSUPPORTED if an extent exceeds INT_MAX.
 * Formula: "Unifying Convolutions and GEMM", section 5, with the dilation
 * term.  ho_out / wo_out may be NULL. */
conv_status_t conv2d_output_size(int H, int W, int KH, int KW, int stride, int pad, int dilation,
                                 int *ho_out, int *wo_out);

/* Workspace bytes conv2d_fwd needs for this call (host only; no HIP call, so
 * it works without a GPU).  The figure covers the lowering structure of the
 * chosen algorithm (indirection buffer, or window-ordered input plus, for
 * NCHW, the weights regrouped channel-innermost), the channels-last copy of
 * an NCHW input where the path reads one (for a 1x1 layer, of half the
 * batch at a time), fp32 split-K partials on skinny layers, and the fp32
 * partial tiles of the window-row loop's stream-K form.  It is 0 for
 * the plain-GEMM feed on NHWC input, and below the im2col footprint
 * N*Ho*Wo*C_in*KH*KW elements for every algorithm except CONV_ALGO_IM2COL,
 * whose workspace is that footprint (plus, on skinny layers, split-K
 * partials of at most as much again).  *bytes_out receives the size; errors
 * as for conv2d_fwd's host checks. */
conv_status_t conv2d_fwd_workspace_size(int N, int C_in, int H, int W, int C_out, int KH, int KW,
                                        int stride, int pad, int dilation,
                                        conv_layout_t layout, conv_dtype_t dtype, conv_algo_t algo,
                                        size_t *bytes_out);

/* Bytes of the im2col matrix X_col the pages' GEMM route would build:
 * N*Ho*Wo * C_in*KH*KW elements ("Unifying Convolutions and GEMM", section 2). */
conv_status_t conv2d_im2col_bytes(int N, int C_in, int H, int W, int KH, int KW,
                                  int stride, int pad, int dilation, conv_dtype_t dtype,
                                  size_t *bytes_out);

/* The forward convolution.
 *   x, w, y    device tensors in `layout` (see above); y is fully overwritten.
 *   bias       device vector of C_out values, or NULL for none.
 *   workspace  device scratch of at least the queried size (NULL allowed when
 *              that size is 0); contents undefined afterwards.
 * Work is enqueued on `stream`; the call returns without waiting. */
conv_status_t conv2d_fwd(const void *x, const void *w, const void *bias, void *y,
                         int N, int C_in, int H, int W, int C_out, int KH, int KW,
                         int stride, int pad, int dilation,
                         conv_layout_t layout, conv_dtype_t dtype, conv_stream_t stream,
                         void *workspace, size_t workspace_bytes, conv_algo_t algo);

/* conv2d_fwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace is a scratch array of
 * CONV_NOALLOC_SCRATCH_BYTES bytes that the library holds in each GPU's
 * memory from the first call on that GPU until the process ends; the call
 * itself allocates nothing (no hipMalloc, hipFree or allocating library
 * routine).  The first call on a device looks up that device's array
 * (hipGetSymbolAddress); later calls do not.
 *   Arguments, layouts, ownership and errors as for conv2d_fwd (the caller
 *   still passes x, w, bias and y).  A call whose conv2d_fwd_workspace_size
 *   exceeds CONV_NOALLOC_SCRATCH_BYTES runs without the stream-K form where
 *   that brings it within the array, else returns CONV_ERR_WORKSPACE before
 *   any launch.  The work runs on the device of `stream` (the current device
 *   for NULL).
 *   Every call on one GPU shares that GPU's array, which keeps the last
 *   call's contents; nothing in it has to start at zero.  Calls that overlap
 *   on one GPU (on different streams, or from different host threads without
 *   ordering) race on the array and give undefined results: order them. */
#define CONV_NOALLOC_SCRATCH_BYTES (128u << 20)
conv_status_t conv2d_fwd_noalloc(const void *x, const void *w, const void *bias, void *y,
                                 int N, int C_in, int H, int W, int C_out, int KH, int KW,
                                 int stride, int pad, int dilation,
                                 conv_layout_t layout, conv_dtype_t dtype, conv_stream_t stream,
                                 conv_algo_t algo);

/* Steps (c) and (d) alone -- the MFMA main loop and its fused epilogue -- on
 * operands that are already lowered, for callers that keep the lowering
 * between calls (the indirection buffer depends only on the geometry, the
 * regrouped weights only on w):
 *   lowered      CONV_ALGO_INDIRECT: the input channels-last, [N][H][W][C_in];
 *                CONV_ALGO_IM2COL: X_col as conv2d_im2col_transform writes
 *                it for CONV_LAYOUT_NHWC;
 *                CONV_ALGO_IM2WIN: the window-ordered tensor that
 *                conv2d_im2win_transform writes.
 *   indirection  CONV_ALGO_INDIRECT: a buffer from conv2d_build_indirection
 *                for the same geometry with CONV_LAYOUT_NHWC; ignored (may
 *                be NULL) for CONV_ALGO_IM2WIN and CONV_ALGO_IM2COL.
 *   w_ohwi       weights as [C_out][KH][KW][C_in].
 *   out_layout   layout of y: [N][C_out][Ho][Wo] (NCHW) or [N][Ho][Wo][C_out].
 *   workspace    split-K partials only: conv2d_fwd_workspace_size(...,
 *                CONV_LAYOUT_NHWC, dtype, algo) bytes always suffice; with
 *                less (or NULL) the main loop runs without split-K.
 * Other arguments and errors as for conv2d_fwd; any algo other than INDIRECT,
 * IM2WIN or IM2COL is CONV_ERR_INVALID_ARG. */
conv_status_t conv2d_main_loop(const void *lowered, const int32_t *indirection, const void *w_ohwi,
                               const void *bias, void *y,
                               int N, int C_in, int H, int W, int C_out, int KH, int KW,
                               int stride, int pad, int dilation, conv_algo_t algo,
                               conv_layout_t out_layout, conv_dtype_t dtype, conv_stream_t stream,
                               void *workspace, size_t workspace_bytes);

/* Step (b) on its own: build the indirection buffer of The Indirect
 * Convolution Algorithm (abstract) into `buf` (device, int32, Ho*Wo*KH*KW
 * entries).  Entry [p][t] for output pixel p = ho*Wo + wo and tap
 * t = kh*KW + kw is the element offset, within one image, of the first
 * channel of input pixel (hi, wi) = (ho*stride + kh*dilation - pad,
 * wo*stride + kw*dilation - pad): hi*W + wi for NCHW, (hi*W + wi)*C_in for
 * NHWC; it is -1 where the tap falls in the zero padding.  The buffer does
 * not depend on the batch index. */
conv_status_t conv2d_build_indirection(int32_t *buf, int C_in, int H, int W, int KH, int KW,
                                       int stride, int pad, int dilation, conv_layout_t layout,
                                       conv_stream_t stream);

/* Step (a) on its own: write the window-ordered tensor of "Im2win: An
 * Efficient Convolution Paradigm on GPU" (abstract), under the reading taken
 * here, into `xwin` (device, dtype elements):
 *   xwin[n][ho][c][kh][ci] = xpad(n, ci, ho*stride + kh*dilation - pad, c - pad)
 * for c < Wwin = (Wo-1)*stride + (KW-1)*dilation + 1.  For every output row
 * it holds the KH input rows that row's windows touch, interleaved column by
 * column with channels innermost, so the window of output pixel (ho, wo) is
 * one contiguous run of KW*KH*C_in values when dilation is 1.  `x` is in
 * `layout`; the result is the same for both layouts. */
conv_status_t conv2d_im2win_transform(const void *x, void *xwin, int N, int C_in, int H, int W,
                                      int KH, int KW, int stride, int pad, int dilation,
                                      conv_layout_t layout, conv_dtype_t dtype, conv_stream_t stream);

/* The im2col matrix X_col ("Unifying Convolutions and GEMM", section 2):
 * row m = (n, ho, wo) of N*Ho*Wo, each row the C_in*KH*KW values of that
 * output pixel's window, zero where the window overlaps the padding.  The
 * columns run (ci, kh, kw) for CONV_LAYOUT_NCHW -- the order of OIHW
 * weights -- and (kh, kw, ci) for CONV_LAYOUT_NHWC, the order of OHWI
 * weights, so either layout's weights are W_row as they lie.  `xcol` holds
 * conv2d_im2col_bytes bytes, is fully overwritten, and is the caller's.
 * Errors as for conv2d_im2win_transform. */
conv_status_t conv2d_im2col_transform(const void *x, void *xcol, int N, int C_in, int H, int W,
                                      int KH, int KW, int stride, int pad, int dilation,
                                      conv_layout_t layout, conv_dtype_t dtype, conv_stream_t stream);

/* Main-loop variants, for ablation ("Im2win: An Efficient Convolution
 * Paradigm on GPU", abstract, ablates its kernel's techniques the same way).
 * Each computes the same convolution; only the summation order of the K
 * sum may differ.
 *   AUTO            the library's own choice (the default).
 *   ELEMENT_128x128 element gathers through registers into LDS: no 16-byte
 *                   vector loads, no load-to-LDS DMA.
 *   DMA_128x128     16-byte loads straight to LDS, one wavefront per SIMD,
 *                   128 x 128 block tile, wavefront tiles 64 x 64.
 *   DMA_256x128     the same with a 256 x 128 block tile (wavefronts 128 x 64).
 *   DUAL_256x128    two 256-thread blocks per CU, two wavefronts per SIMD,
 *                   wavefront tiles 128 x 64, 64-byte K rows.
 *   OCT_256x128     one 512-thread block per CU, two wavefronts per SIMD,
 *                   wavefront tiles 64 x 64, 128-byte K rows.
 *   OCT_256x256     one 512-thread block per CU, 256 x 256 block tile.
 *   QUAD_128x64     four 256-thread blocks per CU, 128 x 64 block tile.
 * The ABL_ variants are one plain implicit-GEMM main loop (indirection
 * buffer over channels-last input, K tiles of 32 channels of one tap,
 * 16-bit types, C_in a multiple of 32; AUTO then means INDIRECT) with the
 * techniques the Im2win abstract ablates switched off one at a time; they
 * share loads and epilogue, and never split K:
 *   ABL_FULL        LDS staging, two LDS stages, prefetch (tile k+1's global
 *                   loads before tile k's MFMAs), v_mfma 32x32x16, 128 x 128
 *                   block tile of four 64 x 64 wavefront tiles;
 *   ABL_NO_LDS      no LDS: each wavefront loads its own fragments;
 *   ABL_ONE_STAGE   one LDS stage (no double buffer);
 *   ABL_NO_PREFETCH tile k+1's loads issued after tile k's MFMAs;
 *   ABL_MFMA16      micro-kernel v_mfma 16x16x32;
 *   ABL_VALU        micro-kernel on the vector ALUs (fp32 FMA, 8 x 8 outputs
 *                   per lane);
 *   ABL_TILE64      64 x 64 block tile, one wavefront per block.  */
typedef enum {
    CONV_MAIN_LOOP_AUTO = 0,
    CONV_MAIN_LOOP_ELEMENT_128x128 = 1,
    CONV_MAIN_LOOP_DMA_128x128 = 2,
    CONV_MAIN_LOOP_DMA_256x128 = 3,
    CONV_MAIN_LOOP_DUAL_256x128 = 4,
    CONV_MAIN_LOOP_OCT_256x128 = 5,
    CONV_MAIN_LOOP_OCT_256x256 = 6,
    CONV_MAIN_LOOP_QUAD_128x64 = 7,
    CONV_MAIN_LOOP_ABL_FULL = 8,
    CONV_MAIN_LOOP_ABL_NO_LDS = 9,
    CONV_MAIN_LOOP_ABL_ONE_STAGE = 10,
    CONV_MAIN_LOOP_ABL_NO_PREFETCH = 11,
    CONV_MAIN_LOOP_ABL_MFMA16 = 12,
    CONV_MAIN_LOOP_ABL_VALU = 13,
    CONV_MAIN_LOOP_ABL_TILE64 = 14
} conv_main_loop_t;

/* Force the main-loop variant of every plan the calling host thread makes
 * from now on (workspace queries, conv2d_fwd, conv2d_main_loop), for
 * ablation and benchmarking; CONV_MAIN_LOOP_AUTO restores the library's
 * choice.  A call whose feed or shape the forced variant cannot serve (the
 * two-wavefront loops need K tiles inside one tap; the DMA loops need
 * 16-byte rows; the ABL_ loops the conditions above, and 16-byte aligned x
 * and w) returns CONV_ERR_UNSUPPORTED before any launch.  Query the
 * workspace under the same setting as the call.  Returns
 * CONV_ERR_INVALID_ARG for an unknown variant, else CONV_OK. */
conv_status_t conv2d_force_main_loop(conv_main_loop_t variant);

/* Instrumentation for measuring the main loop on its own.  The next
 * implicit-GEMM main-loop kernel (step c with its fused epilogue d, as
 * launched by conv2d_fwd or conv2d_main_loop) that the calling host thread
 * launches stamps `start_event` when it begins executing and `stop_event`
 * when it ends, through hipExtLaunchKernel; hipEventElapsedTime on the pair
 * is then that kernel's own duration, without the dispatch gaps an event
 * recorded before and after the call would include.  Both are hipEvent_t
 * handles the caller created (either may be NULL; both NULL cancels a
 * pending request).  The request covers one launch: a split-K finish or a
 * second part of the batch is not included.  Returns CONV_OK. */
conv_status_t conv2d_time_next_main_loop(void *start_event, void *stop_event);

#ifdef __cplusplus
}
#endif

#endif /* CONVLOWER_H */
