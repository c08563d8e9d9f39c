// DyT launchers: forward and backward stage 1 for every (dtype pair, mode, RT, prefetch).  DyT plans
// always take one chunk per thread (wide rows are cut into column blocks instead), so the
// CPT > 1 shapes are not instantiated.
#include "rwn_kernels.hpp"
#include "rwn_launch.hpp"

namespace rwn {

hipError_t launch_dyt_fwd(const Plan& p, int xdt, int pdt, const void* x, const void* alpha,
                          const void* gamma, const void* beta, void* y, hipStream_t s) {
    if (p.split) return launch_dyt_fwd_split(p, xdt, pdt, x, alpha, gamma, beta, y, s);
    const Geom g = make_geom(p);
    return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
        using T = typename decltype(tt)::type;
        using PT = typename decltype(pt)::type;
        return dispatch_shape<T>(p, [&](auto mode, auto cpt, auto rt, auto pf, auto lay) {
            constexpr int kMax = MaxBlock<T, decltype(rt)::value, decltype(cpt)::value>::value;
            if constexpr (decltype(cpt)::value > 1) return hipErrorInvalidValue;
            else if (p.block > kMax || p.block < 1) return hipErrorInvalidConfiguration;
            else return launch(dyt_fwd_kernel<T, PT, decltype(mode)::value, decltype(cpt)::value,
                                               decltype(rt)::value, decltype(pf)::value, decltype(lay)::value>,
                               dim3((unsigned)p.grid), dim3(p.block), 0, s, (const T*)x,
                               (const PT*)alpha, (const PT*)gamma, (const PT*)beta, (T*)y, g);
        });
    });
}

hipError_t launch_dyt_bwd(const Plan& p, int xdt, int pdt, const void* x, const void* dy,
                          const void* alpha, const void* gamma, void* dx, float* ws,
                          hipStream_t s) {
    if (p.split) return launch_dyt_bwd_split(p, xdt, pdt, x, dy, alpha, gamma, dx, ws, s);
    const Geom g = make_geom(p);
    return dispatch_pg(ws, [&](auto pg) {
        return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
            using T = typename decltype(tt)::type;
            using PT = typename decltype(pt)::type;
            return dispatch_shape<T>(p, [&](auto mode, auto cpt, auto rt, auto pf, auto lay) {
                constexpr int kMax = MaxBlock<T, decltype(rt)::value, decltype(cpt)::value>::value;
                if constexpr (decltype(cpt)::value > 1) return hipErrorInvalidValue;
                else if (p.block > kMax || p.block < 1) return hipErrorInvalidConfiguration;
                else return launch(dyt_bwd_kernel<T, PT, decltype(mode)::value, decltype(cpt)::value,
                                                  decltype(rt)::value, decltype(pf)::value, decltype(pg)::value, decltype(lay)::value>,
                                   dim3((unsigned)p.grid), dim3(p.block), p.lds_bytes, s, (const T*)x,
                                   (const T*)dy, (const PT*)alpha, (const PT*)gamma, (T*)dx, ws, g);
            });
        });
    });
}

int resident_wgs_dyt(bool backward, const Plan& p, int xdt, int pdt) {
    if (p.split) return resident_wgs_split(LAYER_DYT, backward, p, xdt, pdt);
    int n = 0;
    (void)dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
        using T = typename decltype(tt)::type;
        using PT = typename decltype(pt)::type;
        return dispatch_shape<T>(p, [&](auto mode, auto cpt, auto rt, auto pf, auto lay) {
            if constexpr (decltype(cpt)::value > 1) return hipErrorInvalidValue;
            else {
                constexpr int M_ = decltype(mode)::value, C_ = decltype(cpt)::value;
                constexpr int R_ = decltype(rt)::value, P_ = decltype(pf)::value, L_ = decltype(lay)::value;
                const void* k = backward ? (const void*)dyt_bwd_kernel<T, PT, M_, C_, R_, P_, 1, L_>
                                         : (const void*)dyt_fwd_kernel<T, PT, M_, C_, R_, P_, L_>;
                n = kernel_occupancy(k, p.block, backward ? p.lds_bytes : 0);
                return hipSuccess;
            }
        });
    });
    return n;
}

}  // namespace rwn
