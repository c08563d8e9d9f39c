// LayerNorm forward launcher for dense operands (general, flat or split-row kernels), and the
// residency query of LayerNorm plans.
#include "rwn_general.hpp"

namespace rwn {

hipError_t launch_ln_fwd(const Plan& p, int xdt, int pdt, const void* x, const void* gamma,
                         const void* beta, float eps, void* y, float* mean, float* rstd,
                         hipStream_t s) {
    if (p.split) return launch_ln_fwd_split(p, xdt, pdt, x, gamma, beta, eps, y, mean, rstd, s);
    if (p.flat) return launch_ln_fwd_flat(p, xdt, pdt, x, gamma, beta, eps, y, mean, rstd, s);
    if (p.layout) return launch_ln_fwd_strided(p, xdt, pdt, x, gamma, beta, eps, y, mean, rstd, s);
    return general_ln_fwd<false>(p, xdt, pdt, x, gamma, beta, eps, y, mean, rstd, s);
}

int resident_wgs_ln(bool backward, const Plan& p, int xdt, int pdt) {
    if (p.split) return resident_wgs_split(LAYER_LN, backward, p, xdt, pdt);
    if (p.flat) return resident_wgs_ln_flat(backward, p, xdt, pdt);
    if (p.layout) return resident_wgs_ln_strided(backward, p, xdt, pdt);
    if (backward) return resident_wgs_ln_bwd(p, xdt, pdt);
    return general_resident_wgs<false, LAYER_LN, false>(p, xdt, pdt);
}

}  // namespace rwn
