// Runtime selection among the main-loop instantiations of igemm_inst.hip.
#include "conv_internal.h"

namespace convlower {

template <typename S, int FEED>
hipError_t launch_feed(const GemmArgs &a, bool out_nchw, bool a_vec, bool b_vec, int tile, int splits,
                       hipStream_t st);

template <typename S>
static hipError_t dispatch(const GemmArgs &a, int feed, bool out_nchw, bool a_vec, bool b_vec, int tile,
                           int splits, hipStream_t st) {
    switch (feed) {
        case FEED_ROWMAJOR: return launch_feed<S, FEED_ROWMAJOR>(a, out_nchw, a_vec, b_vec, tile, splits, st);
        case FEED_NCHW_1X1: return launch_feed<S, FEED_NCHW_1X1>(a, out_nchw, a_vec, b_vec, tile, splits, st);
        case FEED_IND_NHWC: return launch_feed<S, FEED_IND_NHWC>(a, out_nchw, a_vec, b_vec, tile, splits, st);
        case FEED_IND_NCHW: return launch_feed<S, FEED_IND_NCHW>(a, out_nchw, a_vec, b_vec, tile, splits, st);
        case FEED_WIN: return launch_feed<S, FEED_WIN>(a, out_nchw, a_vec, b_vec, tile, splits, st);
        case FEED_IND_CHUNK: return launch_feed<S, FEED_IND_CHUNK>(a, out_nchw, a_vec, b_vec, tile, splits, st);
        case FEED_WIN_CHUNK: return launch_feed<S, FEED_WIN_CHUNK>(a, out_nchw, a_vec, b_vec, tile, splits, st);
        case FEED_ROWWIN: return launch_feed<S, FEED_ROWWIN>(a, out_nchw, a_vec, b_vec, tile, splits, st);
        case FEED_ROWWIN_NCHW: return launch_feed<S, FEED_ROWWIN_NCHW>(a, out_nchw, a_vec, b_vec, tile, splits, st);
        case FEED_GEMM_NCHW: return launch_feed<S, FEED_GEMM_NCHW>(a, out_nchw, a_vec, b_vec, tile, splits, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_igemm_bf16(const GemmArgs &a, int feed, bool out_nchw, bool a_vec, bool b_vec, int tile,
                             int splits, hipStream_t st) {
    return dispatch<uint16_t>(a, feed, out_nchw, a_vec, b_vec, tile, splits, st);
}

hipError_t launch_igemm_f32(const GemmArgs &a, int feed, bool out_nchw, bool a_vec, bool b_vec, int tile,
                            int splits, hipStream_t st) {
    return dispatch<float>(a, feed, out_nchw, a_vec, b_vec, tile, splits, st);
}

// fp8 e4m3 inputs (bf16 output): the window-row feed only.
hipError_t launch_igemm_fp8(const GemmArgs &a, int feed, bool out_nchw, bool a_vec, bool b_vec, int tile,
                            int splits, hipStream_t st) {
    if (feed != FEED_ROWWIN) return hipErrorInvalidValue;
    return launch_feed<uint8_t, FEED_ROWWIN>(a, out_nchw, a_vec, b_vec, tile, splits, st);
}

hipError_t launch_igemm_f16(const GemmArgs &a, int feed, bool out_nchw, bool a_vec, bool b_vec, int tile,
                            int splits, hipStream_t st) {
    return dispatch<_Float16>(a, feed, out_nchw, a_vec, b_vec, tile, splits, st);
}

}  // namespace convlower
