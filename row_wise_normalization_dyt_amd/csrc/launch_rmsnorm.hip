// RMSNorm launchers: forward and backward stage 1 for every (dtype pair, mode, CPT, RT, prefetch,
// form).
#include "rwn_kernels.hpp"
#include "rwn_launch.hpp"

namespace rwn {

// The form as a template value: 0 for the Llama form, 1 for both float32 forms (the
// (1 + weight) one adds g.w_offset = 1 to the weight).
template <typename F>
hipError_t dispatch_variant(int variant, Geom& g, F&& f) {
    g.w_offset = variant == RMS_ONE_PLUS_WEIGHT ? 1.0f : 0.0f;
    if (variant == RMS_CAST_THEN_WEIGHT) return f(IC<0>{});
    if (variant == RMS_WEIGHT_THEN_CAST || variant == RMS_ONE_PLUS_WEIGHT) return f(IC<1>{});
    return hipErrorInvalidValue;
}

hipError_t launch_rms_fwd(const Plan& p, int xdt, int pdt, int variant, const void* x, const void* w,
                          float eps, void* y, float* rstd, hipStream_t s) {
    if (p.split) return launch_rms_fwd_split(p, xdt, pdt, variant, x, w, eps, y, rstd, s);
    Geom g = make_geom(p);
    return dispatch_variant(variant, g, [&](auto var) {
        return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
            using T = typename decltype(tt)::type;
            using PT = typename decltype(pt)::type;
            return dispatch_shape<T>(p, [&](auto mode, auto cpt, auto rt, auto pf, auto lay) {
                constexpr int kMax = MaxBlock<T, decltype(rt)::value, decltype(cpt)::value>::value;
                if (p.block > kMax || p.block < 1) return hipErrorInvalidConfiguration;
                return launch(rms_fwd_kernel<T, PT, decltype(mode)::value, decltype(cpt)::value,
                                             decltype(rt)::value, decltype(pf)::value, decltype(var)::value, decltype(lay)::value>,
                              dim3((unsigned)p.grid), dim3(p.block), 0, s, (const T*)x,
                              (const PT*)w, eps, (T*)y, rstd, g);
            });
        });
    });
}

hipError_t launch_rms_bwd(const Plan& p, int xdt, int pdt, int variant, const void* x, const void* dy,
                          const float* rstd, const void* w, float eps, void* dx, float* ws,
                          hipStream_t s) {
    if (p.split) return launch_rms_bwd_split(p, xdt, pdt, variant, x, dy, rstd, w, eps, dx, ws, s);
    Geom g = make_geom(p);
    return dispatch_variant(variant, g, [&](auto var) {
        return dispatch_pg(ws, [&](auto pg) {
            return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
                using T = typename decltype(tt)::type;
                using PT = typename decltype(pt)::type;
                return dispatch_shape<T>(p, [&](auto mode, auto cpt, auto rt, auto pf, auto lay) {
                    constexpr int kMax = MaxBlock<T, decltype(rt)::value, decltype(cpt)::value>::value;
                    if (p.block > kMax || p.block < 1) return hipErrorInvalidConfiguration;
                    return launch(rms_bwd_kernel<T, PT, decltype(mode)::value, decltype(cpt)::value,
                                                 decltype(rt)::value, decltype(pf)::value, decltype(var)::value,
                                                 decltype(pg)::value, decltype(lay)::value>,
                                  dim3((unsigned)p.grid), dim3(p.block), p.lds_bytes, s, (const T*)x,
                                  (const T*)dy, rstd, (const PT*)w, eps, (T*)dx, ws, g);
                });
            });
        });
    });
}

int resident_wgs_rms(bool backward, const Plan& p, int xdt, int pdt) {
    if (p.split) return resident_wgs_split(LAYER_RMS, backward, p, xdt, pdt);
    int n = 0;
    (void)dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
        using T = typename decltype(tt)::type;
        using PT = typename decltype(pt)::type;
        return dispatch_shape<T>(p, [&](auto mode, auto cpt, auto rt, auto pf, auto lay) {
            {
                constexpr int M_ = decltype(mode)::value, C_ = decltype(cpt)::value;
                constexpr int R_ = decltype(rt)::value, P_ = decltype(pf)::value, L_ = decltype(lay)::value;
                // The Llama form decides the plan; the float32 forms use the same shapes.
                const void* k = backward ? (const void*)rms_bwd_kernel<T, PT, M_, C_, R_, P_, 0, 1, L_>
                                         : (const void*)rms_fwd_kernel<T, PT, M_, C_, R_, P_, 0, L_>;
                n = kernel_occupancy(k, p.block, backward ? p.lds_bytes : 0);
                return hipSuccess;
            }
        });
    });
    return n;
}

}  // namespace rwn
