/* Runs the oracle (linked in from oracle/conv_oracle.c) on one case read from
 * a binary file, for the sanitizer build of the test suite:
 *   oracle_driver IN OUT
 * IN:  11 int32 (N C H W Co KH KW s p d layout), a flag int32 (1 = with
 *      bias), then x, w and (if flagged) bias as float64 in that layout.
 * OUT: y, then D, as float64; and the oracle's points routine on every
 *      output, which must agree with the full one.  Exit status: 0 on
 *      success, 2 on a malformed file, 3 when the two routines disagree. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_out_size(int in, int k, int s, int p, int d);
int oracle_conv2d_f64(const double *x, const double *w, const double *b, double *y, double *dnorm, int N, int C,
                      int H, int W, int Co, int KH, int KW, int s, int p, int d, int layout);
int oracle_conv2d_points_f64(const double *x, const double *w, const double *b, const int32_t *pts, long npts,
                             double *y, double *dnorm, int N, int C, int H, int W, int Co, int KH, int KW, int s,
                             int p, int d, int layout);

static double *read_f64(FILE *f, size_t n)
{
    double *a = malloc(n * sizeof(double));
    if (!a || fread(a, sizeof(double), n, f) != n) exit(2);
    return a;
}

int main(int argc, char **argv)
{
    if (argc != 3) return 2;
    FILE *f = fopen(argv[1], "rb");
    if (!f) return 2;
    int32_t hdr[12];
    if (fread(hdr, sizeof(int32_t), 12, f) != 12) return 2;
    int N = hdr[0], C = hdr[1], H = hdr[2], W = hdr[3], Co = hdr[4], KH = hdr[5], KW = hdr[6];
    int s = hdr[7], p = hdr[8], d = hdr[9], layout = hdr[10], has_b = hdr[11];
    double *x = read_f64(f, (size_t)N * C * H * W);
    double *w = read_f64(f, (size_t)Co * C * KH * KW);
    double *b = has_b ? read_f64(f, (size_t)Co) : NULL;
    fclose(f);
    int Ho = oracle_out_size(H, KH, s, p, d), Wo = oracle_out_size(W, KW, s, p, d);
    if (Ho <= 0 || Wo <= 0) return 2;
    size_t ny = (size_t)N * Co * Ho * Wo;
    double *y = malloc(ny * sizeof(double)), *dn = malloc(ny * sizeof(double));
    if (oracle_conv2d_f64(x, w, b, y, dn, N, C, H, W, Co, KH, KW, s, p, d, layout) != 0) return 2;
    /* every output through the points routine, logical (n, co, ho, wo) order */
    int32_t *pts = malloc(ny * 4 * sizeof(int32_t));
    double *yp = malloc(ny * sizeof(double)), *dp = malloc(ny * sizeof(double));
    size_t i = 0;
    for (int n = 0; n < N; ++n)
        for (int co = 0; co < Co; ++co)
            for (int ho = 0; ho < Ho; ++ho)
                for (int wo = 0; wo < Wo; ++wo, ++i) {
                    pts[4 * i] = n; pts[4 * i + 1] = co; pts[4 * i + 2] = ho; pts[4 * i + 3] = wo;
                }
    if (oracle_conv2d_points_f64(x, w, b, pts, (long)ny, yp, dp, N, C, H, W, Co, KH, KW, s, p, d, layout) != 0)
        return 2;
    i = 0;
    for (int n = 0; n < N; ++n)
        for (int co = 0; co < Co; ++co)
            for (int ho = 0; ho < Ho; ++ho)
                for (int wo = 0; wo < Wo; ++wo, ++i) {
                    size_t j = layout == 0 ? (((size_t)n * Co + co) * Ho + ho) * Wo + wo
                                           : (((size_t)n * Ho + ho) * Wo + wo) * Co + co;
                    if (memcmp(&yp[i], &y[j], sizeof(double)) || memcmp(&dp[i], &dn[j], sizeof(double))) return 3;
                }
    FILE *o = fopen(argv[2], "wb");
    if (!o || fwrite(y, sizeof(double), ny, o) != ny || fwrite(dn, sizeof(double), ny, o) != ny) return 2;
    fclose(o);
    free(x); free(w); free(b); free(y); free(dn); free(pts); free(yp); free(dp);
    return 0;
}
