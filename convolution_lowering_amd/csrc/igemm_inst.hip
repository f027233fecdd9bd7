// One (dtype, feed) slice of the main-loop instantiations.  The build
// compiles this file once per pair, with IGEMM_DTYPE (0 fp32, 1 bf16,
// 2 fp16) and IGEMM_FEED set, so the many template variants build in
// parallel.
#include "igemm_impl.h"

#ifndef IGEMM_FEED
#error "IGEMM_FEED must be defined"
#endif

namespace convlower {
#if IGEMM_DTYPE == 1
using SliceT = uint16_t;  // bf16 as raw 16-bit words
#elif IGEMM_DTYPE == 2
using SliceT = _Float16;
#elif IGEMM_DTYPE == 3
using SliceT = uint8_t;  // fp8 e4m3 as raw bytes (the window-row feed only)
#else
using SliceT = float;
#endif
template hipError_t launch_feed<SliceT, IGEMM_FEED>(const GemmArgs &, bool, bool, bool, int, int,
                                                     hipStream_t);
}  // namespace convlower
