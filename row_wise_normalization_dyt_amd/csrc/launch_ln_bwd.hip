// LayerNorm backward stage-1 launcher for dense operands (general kernels for every requested
// gradient set, or the flat / split-row ones).
#include "rwn_general.hpp"

namespace rwn {

hipError_t launch_ln_bwd(const Plan& p, int xdt, int pdt, const void* x, const void* dy,
                         const float* mean, const float* rstd, const void* gamma, float eps,
                         void* dx, float* ws, int grads, hipStream_t s) {
    if (p.split) return launch_ln_bwd_split(p, xdt, pdt, x, dy, mean, rstd, gamma, eps, dx, ws, grads, s);
    if (p.flat) return launch_ln_bwd_flat(p, xdt, pdt, x, dy, mean, rstd, gamma, eps, dx, ws, grads, s);
    if (p.layout) return launch_ln_bwd_strided(p, xdt, pdt, x, dy, mean, rstd, gamma, eps, dx, ws, grads, s);
    return general_ln_bwd<false>(p, xdt, pdt, x, dy, mean, rstd, gamma, eps, dx, ws, grads, s);
}

int resident_wgs_ln_bwd(const Plan& p, int xdt, int pdt) {
    return general_resident_wgs<false, LAYER_LN, true>(p, xdt, pdt);
}

}  // namespace rwn
