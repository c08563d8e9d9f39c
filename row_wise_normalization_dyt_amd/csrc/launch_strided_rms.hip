// RMSNorm launchers for strided operands (the general kernels' layout 1): forward, backward
// stage 1 and the residency query of strided RMSNorm plans.
#include "rwn_general.hpp"

namespace rwn {

hipError_t launch_rms_fwd_strided(const Plan& p, int xdt, int pdt, int variant, const void* x, const void* w,
                                  float eps, void* y, float* rstd, hipStream_t s) {
    return general_rms_fwd<true>(p, xdt, pdt, variant, x, w, eps, y, rstd, s);
}

hipError_t launch_rms_bwd_strided(const Plan& p, int xdt, int pdt, int variant, const void* x, const void* dy,
                                  const float* rstd, const void* w, float eps, void* dx, float* ws, hipStream_t s) {
    return general_rms_bwd<true>(p, xdt, pdt, variant, x, dy, rstd, w, eps, dx, ws, s);
}

int resident_wgs_rms_strided(bool backward, const Plan& p, int xdt, int pdt) {
    return backward ? general_resident_wgs<true, LAYER_RMS, true>(p, xdt, pdt)
                    : general_resident_wgs<true, LAYER_RMS, false>(p, xdt, pdt);
}

}  // namespace rwn
