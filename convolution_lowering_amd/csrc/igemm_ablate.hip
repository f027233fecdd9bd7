// Launches of the ablation main loop (igemm_ablate.h), one instantiation per
// forced variant, 16-bit element types, either output layout.
#include "igemm_impl.h"
#include "igemm_ablate.h"

namespace convlower {

template <typename S, bool OUT_NCHW>
static hipError_t launch_ablate_t(const GemmArgs &a, int variant, hipStream_t st) {
    const Geom &g = a.g;
    auto go = [&](auto kern, int bt) {
        dim3 grid((unsigned)(((g.M + bt - 1) / bt) * ((g.Co + bt - 1) / bt)));
        hipEvent_t t0, t1;
        take_main_loop_events(&t0, &t1);
        if (t0 || t1)
            hipExtLaunchKernelGGL(kern, grid, dim3(bt == 128 ? 256 : 64), 0, st, t0, t1, 0, a);
        else
            hipLaunchKernelGGL(kern, grid, dim3(bt == 128 ? 256 : 64), 0, st, a);
        return hipGetLastError();
    };
    switch (variant) {
        case CONV_MAIN_LOOP_ABL_FULL:
            return go(igemm_ablate_kernel<S, OUT_NCHW, true, 2, true, ABL_MFMA32, 128>, 128);
        case CONV_MAIN_LOOP_ABL_NO_LDS:
            return go(igemm_ablate_kernel<S, OUT_NCHW, false, 2, true, ABL_MFMA32, 128>, 128);
        case CONV_MAIN_LOOP_ABL_ONE_STAGE:
            return go(igemm_ablate_kernel<S, OUT_NCHW, true, 1, true, ABL_MFMA32, 128>, 128);
        case CONV_MAIN_LOOP_ABL_NO_PREFETCH:
            return go(igemm_ablate_kernel<S, OUT_NCHW, true, 2, false, ABL_MFMA32, 128>, 128);
        case CONV_MAIN_LOOP_ABL_MFMA16:
            return go(igemm_ablate_kernel<S, OUT_NCHW, true, 2, true, ABL_MFMA16, 128>, 128);
        case CONV_MAIN_LOOP_ABL_VALU:
            return go(igemm_ablate_kernel<S, OUT_NCHW, true, 2, true, ABL_VALU, 128>, 128);
        case CONV_MAIN_LOOP_ABL_TILE64:
            return go(igemm_ablate_kernel<S, OUT_NCHW, true, 2, true, ABL_MFMA32, 64>, 64);
        default:
            return hipErrorInvalidValue;
    }
}

hipError_t launch_ablate(const GemmArgs &a, int variant, bool out_nchw, int dtype, hipStream_t st) {
    if (dtype == CONV_DTYPE_BF16)
        return out_nchw ? launch_ablate_t<uint16_t, true>(a, variant, st) : launch_ablate_t<uint16_t, false>(a, variant, st);
    if (dtype == CONV_DTYPE_FP16)
        return out_nchw ? launch_ablate_t<_Float16, true>(a, variant, st) : launch_ablate_t<_Float16, false>(a, variant, st);
    return hipErrorInvalidValue;
}

}  // namespace convlower
