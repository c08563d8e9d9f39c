// Launchers of the split-row kernels (rwn_split.hpp): plans with p.split set, every dtype pair,
// 1, 2 or 4 whole chunks per lane, plain or pipelined tile loop, with and without
// parameter-gradient partials.
#include "rwn_launch.hpp"
#include "rwn_split.hpp"

namespace rwn {

// Calls f(IC<CPT>, IC<PF>) for the plan's chunks per lane and pipelining.
template <typename F>
static hipError_t dispatch_split_cpt(const Plan& p, F&& f) {
    if (p.block < 1 || p.block > kSplitBlock) return hipErrorInvalidConfiguration;
    auto by_pf = [&](auto cpt) { return p.pf ? f(cpt, IC<1>{}) : f(cpt, IC<0>{}); };
    switch (p.cpt) {
    case 1: return by_pf(IC<1>{});
    case 2: return by_pf(IC<2>{});
    case 4: return by_pf(IC<4>{});
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dyt_fwd_split(const Plan& p, int xdt, int pdt, const void* x, const void* alpha,
                                const void* gamma, const void* beta, void* y, hipStream_t s) {
    const Geom g = make_geom(p);
    return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
        using T = typename decltype(tt)::type;
        using PT = typename decltype(pt)::type;
        return dispatch_split_cpt(p, [&](auto cpt, auto pf) {
            return launch(dyt_fwd_split_kernel<T, PT, decltype(cpt)::value, decltype(pf)::value>, dim3((unsigned)p.grid), dim3(p.block), 0,
                          s, (const T*)x, (const PT*)alpha, (const PT*)gamma, (const PT*)beta, (T*)y, g);
        });
    });
}

hipError_t launch_dyt_bwd_split(const Plan& p, int xdt, int pdt, const void* x, const void* dy,
                                const void* alpha, const void* gamma, void* dx, float* ws, hipStream_t s) {
    const Geom g = make_geom(p);
    return dispatch_pg(ws, [&](auto pg) {
        return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
            using T = typename decltype(tt)::type;
            using PT = typename decltype(pt)::type;
            return dispatch_split_cpt(p, [&](auto cpt, auto pf) {
                return launch(dyt_bwd_split_kernel<T, PT, decltype(cpt)::value, decltype(pf)::value, decltype(pg)::value>,
                              dim3((unsigned)p.grid), dim3(p.block), p.lds_bytes, s, (const T*)x, (const T*)dy,
                              (const PT*)alpha, (const PT*)gamma, (T*)dx, ws, g);
            });
        });
    });
}

hipError_t launch_ln_fwd_split(const Plan& p, int xdt, int pdt, const void* x, const void* gamma,
                               const void* beta, float eps, void* y, float* mean, float* rstd, hipStream_t s) {
    const Geom g = make_geom(p);
    return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
        using T = typename decltype(tt)::type;
        using PT = typename decltype(pt)::type;
        return dispatch_split_cpt(p, [&](auto cpt, auto pf) {
            return launch(ln_fwd_split_kernel<T, PT, decltype(cpt)::value, decltype(pf)::value>, dim3((unsigned)p.grid), dim3(p.block), 0,
                          s, (const T*)x, (const PT*)gamma, (const PT*)beta, eps, (T*)y, mean, rstd, g);
        });
    });
}

hipError_t launch_ln_bwd_split(const Plan& p, int xdt, int pdt, const void* x, const void* dy,
                               const float* mean, const float* rstd, const void* gamma, float eps,
                               void* dx, float* ws, int grads, hipStream_t s) {
    const Geom g = make_geom(p);
    return dispatch_ln_grads(ws, grads, [&](auto pg) {
        return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
            using T = typename decltype(tt)::type;
            using PT = typename decltype(pt)::type;
            return dispatch_split_cpt(p, [&](auto cpt, auto pf) {
                return launch(ln_bwd_split_kernel<T, PT, decltype(cpt)::value, decltype(pf)::value, decltype(pg)::value>,
                              dim3((unsigned)p.grid), dim3(p.block), p.lds_bytes, s, (const T*)x, (const T*)dy,
                              mean, rstd, (const PT*)gamma, eps, (T*)dx, ws, g);
            });
        });
    });
}

hipError_t launch_rms_fwd_split(const Plan& p, int xdt, int pdt, int variant, const void* x, const void* w,
                                float eps, void* y, float* rstd, hipStream_t s) {
    Geom g = make_geom(p);
    return dispatch_variant(variant, g, [&](auto var) {
        return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
            using T = typename decltype(tt)::type;
            using PT = typename decltype(pt)::type;
            return dispatch_split_cpt(p, [&](auto cpt, auto pf) {
                return launch(rms_fwd_split_kernel<T, PT, decltype(cpt)::value, decltype(pf)::value, decltype(var)::value>,
                              dim3((unsigned)p.grid), dim3(p.block), 0, s, (const T*)x, (const PT*)w, eps, (T*)y,
                              rstd, g);
            });
        });
    });
}

hipError_t launch_rms_bwd_split(const Plan& p, int xdt, int pdt, int variant, const void* x, const void* dy,
                                const float* rstd, const void* w, float eps, void* dx, float* ws, hipStream_t s) {
    Geom g = make_geom(p);
    return dispatch_variant(variant, g, [&](auto var) {
        return dispatch_pg(ws, [&](auto pg) {
            return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
                using T = typename decltype(tt)::type;
                using PT = typename decltype(pt)::type;
                return dispatch_split_cpt(p, [&](auto cpt, auto pf) {
                    return launch(rms_bwd_split_kernel<T, PT, decltype(cpt)::value, decltype(pf)::value,
                                                       decltype(var)::value, decltype(pg)::value>,
                                  dim3((unsigned)p.grid), dim3(p.block), p.lds_bytes, s, (const T*)x, (const T*)dy,
                                  rstd, (const PT*)w, eps, (T*)dx, ws, g);
                });
            });
        });
    });
}

int resident_wgs_split(int layer, bool backward, const Plan& p, int xdt, int pdt) {
    int n = 0;
    (void)dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
        using T = typename decltype(tt)::type;
        using PT = typename decltype(pt)::type;
        return dispatch_split_cpt(p, [&](auto cpt, auto pf) {
            constexpr int C = decltype(cpt)::value, F = decltype(pf)::value;
            const void* k;
            if (layer == LAYER_DYT)
                k = backward ? (const void*)dyt_bwd_split_kernel<T, PT, C, F, 1> : (const void*)dyt_fwd_split_kernel<T, PT, C, F>;
            else if (layer == LAYER_LN)
                k = backward ? (const void*)ln_bwd_split_kernel<T, PT, C, F, 3> : (const void*)ln_fwd_split_kernel<T, PT, C, F>;
            else
                k = backward ? (const void*)rms_bwd_split_kernel<T, PT, C, F, 0, 1>
                             : (const void*)rms_fwd_split_kernel<T, PT, C, F, 0>;
            n = kernel_occupancy(k, p.block, backward ? p.lds_bytes : 0);
            return hipSuccess;
        });
    });
    return n;
}

}  // namespace rwn
