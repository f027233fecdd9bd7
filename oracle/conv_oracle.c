/*
 * Oracle for the batched 2-D convolution forward pass -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The product path (the HIP library) never calls it,
 * and it shares no code, header or table with that path.
 *
 * What it computes is the plain definition, written as the seven nested loops
 * of "Unifying Convolutions and GEMM" (projectaiml.com, section 1, "The 7-Loop
 * Fallacy"), extended with the three terms the rest of the pages use:
 *   - zero padding `pad` on every side (same page, section 5: F.unfold with
 *     `padding`, and the output-size formula there),
 *   - dilation `dil` between kernel taps (The Indirect Convolution Algorithm,
 *     abstract: dilation is among the convolution parameters its method
 *     supports, beside kernel size, padding and stride),
 *   - an optional per-output-channel bias (section 5: the bias vector is
 *     added to every output pixel of its channel by broadcasting).
 * It is a cross-correlation (no kernel flip), exactly as the loop indexes
 * X[.., ho*stride+kh, ..] * W[.., kh, ..].
 *
 *   y[n,co,ho,wo] = bias[co] + sum_{ci,kh,kw} xpad(n, ci, ho*s+kh*d-p, wo*s+kw*d-p) * w[co,ci,kh,kw]
 *
 * All arithmetic is fp64 on the exact input values.  Beside y it returns the
 * error normaliser  D = sum |xpad|*|w| + |bias|  over the same terms, so a
 * caller can form |y_gpu - y| / D.
 *
 * Layout 0 (NCHW): x[N][C][H][W], w[Co][C][KH][KW], y[N][Co][Ho][Wo].
 * Layout 1 (NHWC): x[N][H][W][C], w[Co][KH][KW][C], y[N][Ho][Wo][Co].
 * The layout only changes where an element lives, never the arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Output extent along one axis: the number of window placements that fit,
 * (in + 2p - d*(k-1) - 1) / s + 1 (section 5 of the blog gives the d = 1 case).
 * Returns 0 when not even one placement fits. */
int oracle_out_size(int in, int k, int s, int p, int d)
{
    long span = (long)in + 2L * p - (long)d * (k - 1) - 1;
    if (span < 0) return 0;
    return (int)(span / s) + 1;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static inline size_t x_index(int layout, int n, int ci, int h, int w, int C, int H, int W)
{
    if (layout == 0) return (((size_t)n * C + ci) * H + h) * W + w;
    return (((size_t)n * H + h) * W + w) * C + ci;
}

static inline size_t w_index(int layout, int co, int ci, int kh, int kw, int C, int KH, int KW)
{
    if (layout == 0) return (((size_t)co * C + ci) * KH + kh) * KW + kw;
    return (((size_t)co * KH + kh) * KW + kw) * C + ci;
}

static inline size_t y_index(int layout, int n, int co, int ho, int wo, int Co, int Ho, int Wo)
{
    if (layout == 0) return (((size_t)n * Co + co) * Ho + ho) * Wo + wo;
    return (((size_t)n * Ho + ho) * Wo + wo) * Co + co;
}

/* One output element: the inner three loops (ci, kh, kw) of the 7-loop. */
static void one_output(const double *x, const double *w, const double *b,
                       int n, int co, int ho, int wo,
                       int C, int H, int W, int KH, int KW, int s, int p, int d, int layout,
                       double *y_out, double *d_out)
{
    double acc = 0.0, den = 0.0;
    for (int ci = 0; ci < C; ++ci)
        for (int kh = 0; kh < KH; ++kh)
            for (int kw = 0; kw < KW; ++kw) {
                int hi = ho * s + kh * d - p;
                int wi = wo * s + kw * d - p;
                if (hi < 0 || hi >= H || wi < 0 || wi >= W) continue; /* zero padding */
                double xv = x[x_index(layout, n, ci, hi, wi, C, H, W)];
                double wv = w[w_index(layout, co, ci, kh, kw, C, KH, KW)];
                acc += xv * wv;
                den += fabs(xv) * fabs(wv);
            }
    if (b) {
        acc += b[co];
        den += fabs(b[co]);
    }
    *y_out = acc;
    if (d_out) *d_out = den;
}

/* The whole output tensor.  `b` and `dnorm` may be NULL.
 * Returns 0, or -1 if the geometry admits no output. */
int oracle_conv2d_f64(const double *x, const double *w, const double *b,
                      double *y, double *dnorm,
                      int N, int C, int H, int W, int Co, int KH, int KW,
                      int s, int p, int d, int layout)
{
    int Ho = oracle_out_size(H, KH, s, p, d);
    int Wo = oracle_out_size(W, KW, s, p, d);
    if (Ho <= 0 || Wo <= 0) return -1;
    long total = (long)N * Co;
#pragma omp parallel for schedule(dynamic, 1)
    for (long nc = 0; nc < total; ++nc) {
        int n = (int)(nc / Co), co = (int)(nc % Co);
        for (int ho = 0; ho < Ho; ++ho)
            for (int wo = 0; wo < Wo; ++wo) {
                size_t yi = y_index(layout, n, co, ho, wo, Co, Ho, Wo);
                one_output(x, w, b, n, co, ho, wo, C, H, W, KH, KW, s, p, d, layout,
                           &y[yi], dnorm ? &dnorm[yi] : NULL);
            }
    }
    return 0;
}

/* Selected outputs only: pts holds npts quadruples (n, co, ho, wo) in logical
 * coordinates; y[i] and dnorm[i] receive output i.  Used to check full-size
 * tensors where the whole 7-loop would take too long. */
int oracle_conv2d_points_f64(const double *x, const double *w, const double *b,
                             const int32_t *pts, long npts, double *y, double *dnorm,
                             int N, int C, int H, int W, int Co, int KH, int KW,
                             int s, int p, int d, int layout)
{
    int Ho = oracle_out_size(H, KH, s, p, d);
    int Wo = oracle_out_size(W, KW, s, p, d);
    if (Ho <= 0 || Wo <= 0) return -1;
    for (long i = 0; i < npts; ++i) {
        const int32_t *q = pts + 4 * i;
        if (q[0] < 0 || q[0] >= N || q[1] < 0 || q[1] >= Co || q[2] < 0 || q[2] >= Ho ||
            q[3] < 0 || q[3] >= Wo)
            return -2;
    }
#pragma omp parallel for schedule(static)
    for (long i = 0; i < npts; ++i) {
        const int32_t *q = pts + 4 * i;
        one_output(x, w, b, q[0], q[1], q[2], q[3], C, H, W, KH, KW, s, p, d, layout,
                   &y[i], dnorm ? &dnorm[i] : NULL);
    }
    return 0;
}
