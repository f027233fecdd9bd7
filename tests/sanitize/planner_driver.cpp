// Runs the library's host-side planning through its public C ABI, for the
// sanitizer build of the test suite.  Reads one query per line from stdin:
//   N C H W Co KH KW stride pad dilation layout dtype algo main_loop
// and prints, per query, the status and byte count of
// conv2d_fwd_workspace_size, the status of conv2d_fwd with a NULL input
// (rejected before any launch), and conv2d_output_size / conv2d_im2col_bytes.
// Nothing here launches a kernel or touches a device.
#include <cstdio>

#include "convlower.h"

int main() {
    int v[14];
    while (std::scanf("%d %d %d %d %d %d %d %d %d %d %d %d %d %d", &v[0], &v[1], &v[2], &v[3], &v[4], &v[5], &v[6],
                      &v[7], &v[8], &v[9], &v[10], &v[11], &v[12], &v[13]) == 14) {
        const int N = v[0], C = v[1], H = v[2], W = v[3], Co = v[4], KH = v[5], KW = v[6], s = v[7], p = v[8],
                  d = v[9];
        const conv_layout_t layout = (conv_layout_t)v[10];
        const conv_dtype_t dtype = (conv_dtype_t)v[11];
        const conv_algo_t algo = (conv_algo_t)v[12];
        const conv_status_t fst = conv2d_force_main_loop((conv_main_loop_t)v[13]);
        size_t ws = 0;
        const conv_status_t st = conv2d_fwd_workspace_size(N, C, H, W, Co, KH, KW, s, p, d, layout, dtype, algo, &ws);
        const conv_status_t fw = conv2d_fwd(nullptr, nullptr, nullptr, nullptr, N, C, H, W, Co, KH, KW, s, p, d,
                                            layout, dtype, nullptr, nullptr, 0, algo);
        int ho = -1, wo = -1;
        const conv_status_t os = conv2d_output_size(H, W, KH, KW, s, p, d, &ho, &wo);
        size_t ib = 0;
        const conv_status_t is = conv2d_im2col_bytes(N, C, H, W, KH, KW, s, p, d, dtype, &ib);
        conv2d_force_main_loop(CONV_MAIN_LOOP_AUTO);
        std::printf("%d %d %zu %d %d %d %d %d %zu %s\n", (int)fst, (int)st, ws, (int)fw, (int)os, ho, wo, (int)is, ib,
                    conv_status_string(st) ? "s" : "-");
    }
    return 0;
}
