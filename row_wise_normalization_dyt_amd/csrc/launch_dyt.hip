// DyT launchers for dense operands: forward and backward stage 1 (general kernels, or the
// split-row or 12-byte ones), and the residency query of DyT plans.
#include "rwn_general.hpp"

namespace rwn {

hipError_t launch_dyt_fwd(const Plan& p, int xdt, int pdt, const void* x, const void* alpha,
                          const void* gamma, const void* beta, void* y, hipStream_t s) {
    if (p.split) return launch_dyt_fwd_split(p, xdt, pdt, x, alpha, gamma, beta, y, s);
    if (p.flat) return launch_dyt_fwd_flat(p, xdt, pdt, x, alpha, gamma, beta, y, s);
    if (p.layout) return launch_dyt_fwd_strided(p, xdt, pdt, x, alpha, gamma, beta, y, s);
    return general_dyt_fwd<false>(p, xdt, pdt, x, alpha, gamma, beta, y, s);
}

hipError_t launch_dyt_bwd(const Plan& p, int xdt, int pdt, const void* x, const void* dy,
                          const void* alpha, const void* gamma, void* dx, float* ws,
                          hipStream_t s) {
    if (p.split) return launch_dyt_bwd_split(p, xdt, pdt, x, dy, alpha, gamma, dx, ws, s);
    if (p.flat) return launch_dyt_bwd_flat(p, xdt, pdt, x, dy, alpha, gamma, dx, ws, s);
    if (p.layout) return launch_dyt_bwd_strided(p, xdt, pdt, x, dy, alpha, gamma, dx, ws, s);
    return general_dyt_bwd<false>(p, xdt, pdt, x, dy, alpha, gamma, dx, ws, s);
}

int resident_wgs_dyt(bool backward, const Plan& p, int xdt, int pdt) {
    if (p.split) return resident_wgs_split(LAYER_DYT, backward, p, xdt, pdt);
    if (p.flat) return resident_wgs_dyt_flat(backward, p, xdt, pdt);
    if (p.layout) return resident_wgs_dyt_strided(backward, p, xdt, pdt);
    return backward ? general_resident_wgs<false, LAYER_DYT, true>(p, xdt, pdt)
                    : general_resident_wgs<false, LAYER_DYT, false>(p, xdt, pdt);
}

}  // namespace rwn
