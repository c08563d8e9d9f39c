// DyT launchers for strided operands (the general kernels' layout 1): forward, backward
// stage 1 and the residency query of strided DyT plans.
#include "rwn_general.hpp"

namespace rwn {

hipError_t launch_dyt_fwd_strided(const Plan& p, int xdt, int pdt, const void* x, const void* alpha,
                                  const void* gamma, const void* beta, void* y, hipStream_t s) {
    return general_dyt_fwd<true>(p, xdt, pdt, x, alpha, gamma, beta, y, s);
}

hipError_t launch_dyt_bwd_strided(const Plan& p, int xdt, int pdt, const void* x, const void* dy,
                                  const void* alpha, const void* gamma, void* dx, float* ws, hipStream_t s) {
    return general_dyt_bwd<true>(p, xdt, pdt, x, dy, alpha, gamma, dx, ws, s);
}

int resident_wgs_dyt_strided(bool backward, const Plan& p, int xdt, int pdt) {
    return backward ? general_resident_wgs<true, LAYER_DYT, true>(p, xdt, pdt)
                    : general_resident_wgs<true, LAYER_DYT, false>(p, xdt, pdt);
}

}  // namespace rwn
