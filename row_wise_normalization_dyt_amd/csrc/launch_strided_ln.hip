// LayerNorm launchers for strided operands (the general kernels' layout 1): forward, backward
// stage 1 and the residency query of strided LayerNorm plans.
#include "rwn_general.hpp"

namespace rwn {

hipError_t launch_ln_fwd_strided(const Plan& p, int xdt, int pdt, const void* x, const void* gamma,
                                 const void* beta, float eps, void* y, float* mean, float* rstd, hipStream_t s) {
    return general_ln_fwd<true>(p, xdt, pdt, x, gamma, beta, eps, y, mean, rstd, s);
}

hipError_t launch_ln_bwd_strided(const Plan& p, int xdt, int pdt, const void* x, const void* dy,
                                 const float* mean, const float* rstd, const void* gamma, float eps,
                                 void* dx, float* ws, int grads, hipStream_t s) {
    return general_ln_bwd<true>(p, xdt, pdt, x, dy, mean, rstd, gamma, eps, dx, ws, grads, s);
}

int resident_wgs_ln_strided(bool backward, const Plan& p, int xdt, int pdt) {
    return backward ? general_resident_wgs<true, LAYER_LN, true>(p, xdt, pdt)
                    : general_resident_wgs<true, LAYER_LN, false>(p, xdt, pdt);
}

}  // namespace rwn
