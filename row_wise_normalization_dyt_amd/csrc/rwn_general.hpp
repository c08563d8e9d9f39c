// Launch bodies of the general row kernels (rwn_kernels.hpp), as templates on the operand layout:
// S = false instantiates the dense [M, N] kernels, S = true the strided ones (layout 1).  The
// dense launchers (launch_dyt.hip, launch_ln_*.hip, launch_rms_*.hip) and the strided ones
// (launch_strided_*.hip) each instantiate one side, so the two sets compile in separate units.
#pragma once

#include "rwn_kernels.hpp"
#include "rwn_launch.hpp"

namespace rwn {

// DyT plans always take one chunk per thread (wide rows are cut into column blocks instead), so
// the CPT > 1 shapes are not instantiated.
template <bool S>
hipError_t general_dyt_fwd(const Plan& p, int xdt, int pdt, const void* x, const void* alpha,
                           const void* gamma, const void* beta, void* y, hipStream_t s) {
    const Geom g = make_geom(p);
    return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
        using T = typename decltype(tt)::type;
        using PT = typename decltype(pt)::type;
        return dispatch_shape<T, S>(p, [&](auto mode, auto cpt, auto rt, auto pf, auto lay) {
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

template <bool S>
hipError_t general_dyt_bwd(const Plan& p, int xdt, int pdt, const void* x, const void* dy,
                           const void* alpha, const void* gamma, void* dx, float* ws, hipStream_t s) {
    const Geom g = make_geom(p);
    return dispatch_pg(ws, [&](auto pg) {
        return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
            using T = typename decltype(tt)::type;
            using PT = typename decltype(pt)::type;
            return dispatch_shape<T, S>(p, [&](auto mode, auto cpt, auto rt, auto pf, auto lay) {
                constexpr int kMax = MaxBlock<T, decltype(rt)::value, decltype(cpt)::value>::value;
                if constexpr (decltype(cpt)::value > 1) return hipErrorInvalidValue;
                else if (p.block > kMax || p.block < 1) return hipErrorInvalidConfiguration;
                else return launch(dyt_bwd_kernel<T, PT, decltype(mode)::value, decltype(cpt)::value,
                                                  decltype(rt)::value, decltype(pf)::value, decltype(pg)::value,
                                                  decltype(lay)::value>,
                                   dim3((unsigned)p.grid), dim3(p.block), p.lds_bytes, s, (const T*)x,
                                   (const T*)dy, (const PT*)alpha, (const PT*)gamma, (T*)dx, ws, g);
            });
        });
    });
}

template <bool S>
hipError_t general_ln_fwd(const Plan& p, int xdt, int pdt, const void* x, const void* gamma, const void* beta,
                          float eps, void* y, float* mean, float* rstd, hipStream_t s) {
    const Geom g = make_geom(p);
    return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
        using T = typename decltype(tt)::type;
        using PT = typename decltype(pt)::type;
        return dispatch_shape<T, S>(p, [&](auto mode, auto cpt, auto rt, auto pf, auto lay) {
            constexpr int kMax = MaxBlock<T, decltype(rt)::value, decltype(cpt)::value>::value;
            if (p.block > kMax || p.block < 1) return hipErrorInvalidConfiguration;
            return launch(ln_fwd_kernel<T, PT, decltype(mode)::value, decltype(cpt)::value, decltype(rt)::value,
                                        decltype(pf)::value, decltype(lay)::value>,
                          dim3((unsigned)p.grid), dim3(p.block), 0, s, (const T*)x, (const PT*)gamma,
                          (const PT*)beta, eps, (T*)y, mean, rstd, g);
        });
    });
}

// Strided plans take the LayerNorm backward with both gradients or none: a single requested
// gradient runs the both-gradient kernel, whose extra partial columns stage 2 does not read.
template <bool S>
hipError_t general_ln_bwd(const Plan& p, int xdt, int pdt, const void* x, const void* dy, const float* mean,
                          const float* rstd, const void* gamma, float eps, void* dx, float* ws, int grads,
                          hipStream_t s) {
    const Geom g = make_geom(p);
    return dispatch_ln_grads(ws, S ? (grads ? 3 : 0) : grads, [&](auto pg) {
        constexpr int PG = decltype(pg)::value;
        if constexpr (S && (PG == 1 || PG == 2)) {
            return hipErrorInvalidValue;   // not reached: strided masks are 0 or 3
        } else {
            return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
                using T = typename decltype(tt)::type;
                using PT = typename decltype(pt)::type;
                return dispatch_shape<T, S>(p, [&](auto mode, auto cpt, auto rt, auto pf, auto lay) {
                    constexpr int kMax = MaxBlock<T, decltype(rt)::value, decltype(cpt)::value>::value;
                    if (p.block > kMax || p.block < 1) return hipErrorInvalidConfiguration;
                    return launch(ln_bwd_kernel<T, PT, decltype(mode)::value, decltype(cpt)::value,
                                                decltype(rt)::value, decltype(pf)::value, PG, decltype(lay)::value>,
                                  dim3((unsigned)p.grid), dim3(p.block), p.lds_bytes, s, (const T*)x,
                                  (const T*)dy, mean, rstd, (const PT*)gamma, eps, (T*)dx, ws, g);
                });
            });
        }
    });
}

template <bool S>
hipError_t general_rms_fwd(const Plan& p, int xdt, int pdt, int variant, const void* x, const void* w,
                           float eps, void* y, float* rstd, hipStream_t s) {
    Geom g = make_geom(p);
    return dispatch_variant(variant, g, [&](auto var) {
        return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
            using T = typename decltype(tt)::type;
            using PT = typename decltype(pt)::type;
            return dispatch_shape<T, S>(p, [&](auto mode, auto cpt, auto rt, auto pf, auto lay) {
                constexpr int kMax = MaxBlock<T, decltype(rt)::value, decltype(cpt)::value>::value;
                if (p.block > kMax || p.block < 1) return hipErrorInvalidConfiguration;
                return launch(rms_fwd_kernel<T, PT, decltype(mode)::value, decltype(cpt)::value, decltype(rt)::value,
                                             decltype(pf)::value, decltype(var)::value, decltype(lay)::value>,
                              dim3((unsigned)p.grid), dim3(p.block), 0, s, (const T*)x, (const PT*)w, eps, (T*)y,
                              rstd, g);
            });
        });
    });
}

template <bool S>
hipError_t general_rms_bwd(const Plan& p, int xdt, int pdt, int variant, const void* x, const void* dy,
                           const float* rstd, const void* w, float eps, void* dx, float* ws, hipStream_t s) {
    Geom g = make_geom(p);
    return dispatch_variant(variant, g, [&](auto var) {
        return dispatch_pg(ws, [&](auto pg) {
            return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
                using T = typename decltype(tt)::type;
                using PT = typename decltype(pt)::type;
                return dispatch_shape<T, S>(p, [&](auto mode, auto cpt, auto rt, auto pf, auto lay) {
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

// Workgroups per CU of the general kernel a plan runs: forward, or the backward with every
// parameter gradient (for RMSNorm, the Llama form; the float32 forms use the same shapes).
template <bool S, int LAYER, bool BWD>
int general_resident_wgs(const Plan& p, int xdt, int pdt) {
    int n = 0;
    (void)dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
        using T = typename decltype(tt)::type;
        using PT = typename decltype(pt)::type;
        return dispatch_shape<T, S>(p, [&](auto mode, auto cpt, auto rt, auto pf, auto lay) {
            constexpr int M_ = decltype(mode)::value, C_ = decltype(cpt)::value;
            constexpr int R_ = decltype(rt)::value, P_ = decltype(pf)::value, L_ = decltype(lay)::value;
            const void* k = nullptr;
            if constexpr (LAYER == LAYER_DYT) {
                if constexpr (C_ == 1)
                    k = BWD ? (const void*)dyt_bwd_kernel<T, PT, M_, C_, R_, P_, 1, L_>
                            : (const void*)dyt_fwd_kernel<T, PT, M_, C_, R_, P_, L_>;
            } else if constexpr (LAYER == LAYER_LN) {
                if constexpr (BWD) k = (const void*)ln_bwd_kernel<T, PT, M_, C_, R_, P_, 3, L_>;
                else k = (const void*)ln_fwd_kernel<T, PT, M_, C_, R_, P_, L_>;
            } else {
                if constexpr (BWD) k = (const void*)rms_bwd_kernel<T, PT, M_, C_, R_, P_, 0, 1, L_>;
                else k = (const void*)rms_fwd_kernel<T, PT, M_, C_, R_, P_, 0, L_>;
            }
            if (!k) return hipErrorInvalidValue;
            n = kernel_occupancy(k, p.block, BWD ? p.lds_bytes : 0);
            return hipSuccess;
        });
    });
    return n;
}

}  // namespace rwn
