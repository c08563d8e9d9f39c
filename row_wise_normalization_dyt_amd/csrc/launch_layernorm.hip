// LayerNorm launchers: forward and backward stage 1 for every (dtype pair, mode, CPT, RT, prefetch,
// requested parameter gradients).
#include "rwn_kernels.hpp"
#include "rwn_launch.hpp"

namespace rwn {

hipError_t launch_ln_fwd(const Plan& p, int xdt, int pdt, const void* x, const void* gamma,
                         const void* beta, float eps, void* y, float* mean, float* rstd,
                         hipStream_t s) {
    const Geom g = make_geom(p);
    if (p.split) return launch_ln_fwd_split(p, xdt, pdt, x, gamma, beta, eps, y, mean, rstd, s);
    if (p.flat) return launch_ln_fwd_flat(p, xdt, pdt, x, gamma, beta, eps, y, mean, rstd, s);
    return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
        using T = typename decltype(tt)::type;
        using PT = typename decltype(pt)::type;
        return dispatch_shape<T>(p, [&](auto mode, auto cpt, auto rt, auto pf, auto lay) {
            constexpr int kMax = MaxBlock<T, decltype(rt)::value, decltype(cpt)::value>::value;
            if (p.block > kMax || p.block < 1) return hipErrorInvalidConfiguration;
            return launch(ln_fwd_kernel<T, PT, decltype(mode)::value, decltype(cpt)::value,
                                              decltype(rt)::value, decltype(pf)::value, decltype(lay)::value>,
                               dim3((unsigned)p.grid), dim3(p.block), 0, s, (const T*)x,
                               (const PT*)gamma, (const PT*)beta, eps, (T*)y, mean, rstd, g);
        });
    });
}

hipError_t launch_ln_bwd(const Plan& p, int xdt, int pdt, const void* x, const void* dy,
                         const float* mean, const float* rstd, const void* gamma, float eps,
                         void* dx, float* ws, int grads, hipStream_t s) {
    const Geom g = make_geom(p);
    if (p.split) return launch_ln_bwd_split(p, xdt, pdt, x, dy, mean, rstd, gamma, eps, dx, ws, grads, s);
    if (p.flat) return launch_ln_bwd_flat(p, xdt, pdt, x, dy, mean, rstd, gamma, eps, dx, ws, grads, s);
    return dispatch_ln_grads(ws, grads, [&](auto pg) {
        return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
            using T = typename decltype(tt)::type;
            using PT = typename decltype(pt)::type;
            return dispatch_shape<T>(p, [&](auto mode, auto cpt, auto rt, auto pf, auto lay) {
                constexpr int kMax = MaxBlock<T, decltype(rt)::value, decltype(cpt)::value>::value;
                if (p.block > kMax || p.block < 1) return hipErrorInvalidConfiguration;
                return launch(ln_bwd_kernel<T, PT, decltype(mode)::value, decltype(cpt)::value,
                                            decltype(rt)::value, decltype(pf)::value, decltype(pg)::value, decltype(lay)::value>,
                              dim3((unsigned)p.grid), dim3(p.block), p.lds_bytes, s, (const T*)x,
                              (const T*)dy, mean, rstd, (const PT*)gamma, eps, (T*)dx, ws, g);
            });
        });
    });
}

int resident_wgs_ln(bool backward, const Plan& p, int xdt, int pdt) {
    int n = 0;
    if (p.split) return resident_wgs_split(LAYER_LN, backward, p, xdt, pdt);
    if (p.flat) return resident_wgs_ln_flat(backward, p, xdt, pdt);
    (void)dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
        using T = typename decltype(tt)::type;
        using PT = typename decltype(pt)::type;
        return dispatch_shape<T>(p, [&](auto mode, auto cpt, auto rt, auto pf, auto lay) {
            {
                constexpr int M_ = decltype(mode)::value, C_ = decltype(cpt)::value;
                constexpr int R_ = decltype(rt)::value, P_ = decltype(pf)::value, L_ = decltype(lay)::value;
                const void* k = backward ? (const void*)ln_bwd_kernel<T, PT, M_, C_, R_, P_, 3, L_>
                                         : (const void*)ln_fwd_kernel<T, PT, M_, C_, R_, P_, L_>;
                n = kernel_occupancy(k, p.block, backward ? p.lds_bytes : 0);
                return hipSuccess;
            }
        });
    });
    return n;
}

}  // namespace rwn
