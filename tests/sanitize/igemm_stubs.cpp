// Stand-ins for the kernel launchers, for the sanitizer build of the host
// planner: that build compiles the planner (conv_api.cpp) and the stem
// kernel's planner (patch_conv.hip) only, and the planning checks never
// launch a kernel.  Each reports an error if it were ever called.
#include "conv_internal.h"

namespace convlower {
namespace {
hipError_t never() { return hipErrorInvalidValue; }
}  // namespace
hipError_t launch_igemm_bf16(const GemmArgs &, int, bool, bool, bool, int, int, hipStream_t) { return never(); }
hipError_t launch_igemm_f32(const GemmArgs &, int, bool, bool, bool, int, int, hipStream_t) { return never(); }
hipError_t launch_igemm_f16(const GemmArgs &, int, bool, bool, bool, int, int, hipStream_t) { return never(); }
hipError_t launch_igemm_fp8(const GemmArgs &, int, bool, bool, bool, int, int, hipStream_t) { return never(); }
hipError_t launch_splitk_reduce(const float *, const void *, void *, const Geom &, int, bool, int, hipStream_t) {
    return never();
}
hipError_t launch_build_indirection(int32_t *, const Geom &, bool, hipStream_t) { return never(); }
hipError_t launch_im2win(const void *, void *, const Geom &, bool, bool, hipStream_t) { return never(); }
hipError_t launch_direct_conv(const void *, const void *, const void *, void *, const Geom &, bool, int,
                              hipStream_t) {
    return never();
}
hipError_t launch_im2col(const void *, void *, const Geom &, bool, bool, hipStream_t) { return never(); }
hipError_t launch_ablate(const GemmArgs &, int, bool, int, hipStream_t) { return never(); }
hipError_t launch_im2win_pad(const void *, void *, const Geom &, int, bool, bool, hipStream_t) { return never(); }
hipError_t launch_prep(const void *, bool, void *, int, int32_t *, const void *, bool, void *, const Geom &, int,
                       hipStream_t, uint32_t *, int) {
    return never();
}
hipError_t launch_zero_words(uint32_t *, int, hipStream_t) { return never(); }
hipError_t launch_pack_weights_tapmajor(const void *, void *, const Geom &, int, hipStream_t) { return never(); }
hipError_t launch_pack_weights_ohwi(const void *, void *, const Geom &, bool, hipStream_t) { return never(); }
}  // namespace convlower
