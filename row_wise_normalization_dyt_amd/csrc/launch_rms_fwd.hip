// RMSNorm forward launcher for dense operands (general or split-row kernels), and the residency
// query of RMSNorm plans.
#include "rwn_general.hpp"

namespace rwn {

hipError_t launch_rms_fwd(const Plan& p, int xdt, int pdt, int variant, const void* x, const void* w,
                          float eps, void* y, float* rstd, hipStream_t s) {
    if (p.split) return launch_rms_fwd_split(p, xdt, pdt, variant, x, w, eps, y, rstd, s);
    if (p.layout) return launch_rms_fwd_strided(p, xdt, pdt, variant, x, w, eps, y, rstd, s);
    return general_rms_fwd<false>(p, xdt, pdt, variant, x, w, eps, y, rstd, s);
}

int resident_wgs_rms(bool backward, const Plan& p, int xdt, int pdt) {
    if (p.split) return resident_wgs_split(LAYER_RMS, backward, p, xdt, pdt);
    if (p.layout) return resident_wgs_rms_strided(backward, p, xdt, pdt);
    if (backward) return resident_wgs_rms_bwd(p, xdt, pdt);
    return general_resident_wgs<false, LAYER_RMS, false>(p, xdt, pdt);
}

}  // namespace rwn
