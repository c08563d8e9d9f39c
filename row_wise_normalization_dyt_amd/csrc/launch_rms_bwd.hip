// RMSNorm backward stage-1 launcher for dense operands (general or split-row kernels).
#include "rwn_general.hpp"

namespace rwn {

hipError_t launch_rms_bwd(const Plan& p, int xdt, int pdt, int variant, const void* x, const void* dy,
                          const float* rstd, const void* w, float eps, void* dx, float* ws,
                          hipStream_t s) {
    if (p.split) return launch_rms_bwd_split(p, xdt, pdt, variant, x, dy, rstd, w, eps, dx, ws, s);
    if (p.layout) return launch_rms_bwd_strided(p, xdt, pdt, variant, x, dy, rstd, w, eps, dx, ws, s);
    return general_rms_bwd<false>(p, xdt, pdt, variant, x, dy, rstd, w, eps, dx, ws, s);
}

int resident_wgs_rms_bwd(const Plan& p, int xdt, int pdt) {
    return general_resident_wgs<false, LAYER_RMS, true>(p, xdt, pdt);
}

}  // namespace rwn
