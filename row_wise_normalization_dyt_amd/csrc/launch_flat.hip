// Launchers of the flat LayerNorm kernels (narrow rows; p.flat 1: 16-byte chunks on aligned rows,
// 2: 12-byte chunks): every dtype pair, group size 1..64 lanes, with and without
// parameter-gradient partials and given statistics; and of the 12-byte DyT kernels.
#include "rwn_kernels.hpp"
#include "rwn_launch.hpp"

namespace rwn {

// Calls f(IC<TPR>) for the plan's lanes per row (a power of two up to 64).
template <typename F>
static hipError_t dispatch_tpr(const Plan& p, F&& f) {
    switch (p.tpr) {
    case 1: return f(IC<1>{});
    case 2: return f(IC<2>{});
    case 4: return f(IC<4>{});
    case 8: return f(IC<8>{});
    case 16: return f(IC<16>{});
    case 32: return f(IC<32>{});
    case 64: return f(IC<64>{});
    default: return hipErrorInvalidValue;
    }
}

// The 12-byte forward's steps per tile: two, or one for single-lane rows (a wave's tile of 64
// rows already fills its lanes' statistics store).
template <int TPR>
constexpr int flat12_rt() { return TPR == 1 ? 1 : 2; }

hipError_t launch_ln_fwd_flat(const Plan& p, int xdt, int pdt, const void* x, const void* gamma,
                              const void* beta, float eps, void* y, float* mean, float* rstd,
                              hipStream_t s) {
    if (p.block > 256 || p.block < 1) return hipErrorInvalidConfiguration;
    const Geom g = make_geom(p);
    return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
        using T = typename decltype(tt)::type;
        using PT = typename decltype(pt)::type;
        return dispatch_tpr(p, [&](auto tpr) {
            constexpr int R = decltype(tpr)::value;
            if (p.flat == 2) {
                if (p.rt != flat12_rt<R>() || p.block % 64) return hipErrorInvalidValue;
                return launch(ln_fwd_flat12_kernel<T, PT, R, flat12_rt<R>()>, dim3((unsigned)p.grid),
                              dim3(p.block), 0, s, (const T*)x, (const PT*)gamma, (const PT*)beta, eps,
                              (T*)y, mean, rstd, g);
            }
            return launch(ln_fwd_flat_kernel<T, PT, R>, dim3((unsigned)p.grid),
                          dim3(p.block), 0, s, (const T*)x, (const PT*)gamma, (const PT*)beta, eps,
                          (T*)y, mean, rstd, g);
        });
    });
}

hipError_t launch_ln_bwd_flat(const Plan& p, int xdt, int pdt, const void* x, const void* dy,
                              const float* mean, const float* rstd, const void* gamma, float eps,
                              void* dx, float* ws, int grads, hipStream_t s) {
    if (p.block > 256 || p.block < 1) return hipErrorInvalidConfiguration;
    const Geom g = make_geom(p);
    const bool st = mean != nullptr && rstd != nullptr;
    return dispatch_ln_grads(ws, grads, [&](auto pg) {
        return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
            using T = typename decltype(tt)::type;
            using PT = typename decltype(pt)::type;
            return dispatch_tpr(p, [&](auto tpr) {
                constexpr int R = decltype(tpr)::value, G = decltype(pg)::value;
                if (p.flat == 2) {
                    if (p.rt != 1 || p.block % 64) return hipErrorInvalidValue;
                    auto k = st ? ln_bwd_flat12_kernel<T, PT, R, G, 1> : ln_bwd_flat12_kernel<T, PT, R, G, 0>;
                    return launch(k, dim3((unsigned)p.grid), dim3(p.block), p.lds_bytes, s, (const T*)x,
                                  (const T*)dy, mean, rstd, (const PT*)gamma, eps, (T*)dx, ws, g);
                }
                auto k = st ? ln_bwd_flat_kernel<T, PT, R, G, 1> : ln_bwd_flat_kernel<T, PT, R, G, 0>;
                return launch(k, dim3((unsigned)p.grid), dim3(p.block), p.lds_bytes, s, (const T*)x,
                              (const T*)dy, mean, rstd, (const PT*)gamma, eps, (T*)dx, ws, g);
            });
        });
    });
}

int resident_wgs_ln_flat(bool backward, const Plan& p, int xdt, int pdt) {
    int n = 0;
    (void)dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
        using T = typename decltype(tt)::type;
        using PT = typename decltype(pt)::type;
        return dispatch_tpr(p, [&](auto tpr) {
            constexpr int R = decltype(tpr)::value;
            const void* k;
            if (p.flat == 2)
                k = backward ? (const void*)ln_bwd_flat12_kernel<T, PT, R, 3, 1>
                             : (const void*)ln_fwd_flat12_kernel<T, PT, R, flat12_rt<R>()>;
            else
                k = backward ? (const void*)ln_bwd_flat_kernel<T, PT, R, 3, 1>
                             : (const void*)ln_fwd_flat_kernel<T, PT, R>;
            n = kernel_occupancy(k, p.block, backward ? p.lds_bytes : 0);
            return hipSuccess;
        });
    });
    return n;
}

// DyT in 12-byte chunks (p.flat == 2 only).
hipError_t launch_dyt_fwd_flat(const Plan& p, int xdt, int pdt, const void* x, const void* alpha,
                               const void* gamma, const void* beta, void* y, hipStream_t s) {
    if (p.flat != 2 || p.block > 256 || p.block < 1 || p.block % 64) return hipErrorInvalidConfiguration;
    const Geom g = make_geom(p);
    return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
        using T = typename decltype(tt)::type;
        using PT = typename decltype(pt)::type;
        return dispatch_tpr(p, [&](auto tpr) {
            constexpr int R = decltype(tpr)::value;
            if (p.rt != flat12_rt<R>()) return hipErrorInvalidValue;
            return launch(dyt_fwd_flat12_kernel<T, PT, R, flat12_rt<R>()>, dim3((unsigned)p.grid),
                          dim3(p.block), 0, s, (const T*)x, (const PT*)alpha, (const PT*)gamma,
                          (const PT*)beta, (T*)y, g);
        });
    });
}

hipError_t launch_dyt_bwd_flat(const Plan& p, int xdt, int pdt, const void* x, const void* dy,
                               const void* alpha, const void* gamma, void* dx, float* ws, hipStream_t s) {
    if (p.flat != 2 || p.block > 256 || p.block < 1 || p.block % 64) return hipErrorInvalidConfiguration;
    if (p.rt != 1) return hipErrorInvalidValue;
    const Geom g = make_geom(p);
    return dispatch_pg(ws, [&](auto pg) {
        return dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
            using T = typename decltype(tt)::type;
            using PT = typename decltype(pt)::type;
            return dispatch_tpr(p, [&](auto tpr) {
                constexpr int R = decltype(tpr)::value, G = decltype(pg)::value;
                return launch(dyt_bwd_flat12_kernel<T, PT, R, G>, dim3((unsigned)p.grid), dim3(p.block),
                              p.lds_bytes, s, (const T*)x, (const T*)dy, (const PT*)alpha, (const PT*)gamma,
                              (T*)dx, ws, g);
            });
        });
    });
}

int resident_wgs_dyt_flat(bool backward, const Plan& p, int xdt, int pdt) {
    int n = 0;
    (void)dispatch_dtypes(xdt, pdt, [&](auto tt, auto pt) {
        using T = typename decltype(tt)::type;
        using PT = typename decltype(pt)::type;
        return dispatch_tpr(p, [&](auto tpr) {
            constexpr int R = decltype(tpr)::value;
            const void* k = backward ? (const void*)dyt_bwd_flat12_kernel<T, PT, R, 1>
                                     : (const void*)dyt_fwd_flat12_kernel<T, PT, R, flat12_rt<R>()>;
            n = kernel_occupancy(k, p.block, backward ? p.lds_bytes : 0);
            return hipSuccess;
        });
    });
    return n;
}

}  // namespace rwn
