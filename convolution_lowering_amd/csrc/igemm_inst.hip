// One (dtype, feed) slice of the main-loop instantiations.  The build
// compiles this file once per pair, with IGEMM_BF16 and IGEMM_FEED set, so
// the many template variants build in parallel.
#include "igemm_impl.h"

#ifndef IGEMM_FEED
#error "IGEMM_FEED must be defined"
#endif

namespace convlower {
#if IGEMM_BF16
using SliceT = uint16_t;
#else
using SliceT = float;
#endif
template hipError_t launch_feed<SliceT, IGEMM_FEED>(const GemmArgs &, bool, bool, bool, int, int,
                                                     hipStream_t);
}  // namespace convlower
