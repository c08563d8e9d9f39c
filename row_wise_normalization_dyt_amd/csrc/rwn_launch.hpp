// Host-side launch plan and kernel dispatch (shared by the launcher and API translation units).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rwn_device.hpp"

namespace rwn {

enum Layer { LAYER_DYT = 0, LAYER_LN = 1, LAYER_RMS = 2 };
enum DType { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2 };
// RMSNorm forms: the Llama form rounds the normalized value to x's dtype before the weight
// multiply; the two others multiply in float32 and round once, by weight or by (1 + weight).
enum RmsVariant { RMS_CAST_THEN_WEIGHT = 0, RMS_WEIGHT_THEN_CAST = 1, RMS_ONE_PLUS_WEIGHT = 2 };

// Supported (x dtype, parameter dtype) pairs: float32 x takes float32 parameters; a 16-bit x
// takes float32 parameters or parameters of its own dtype.
constexpr bool dtype_pair_ok(int xdt, int pdt) {
    return (xdt == DT_F32 && pdt == DT_F32) || (xdt == DT_BF16 && (pdt == DT_F32 || pdt == DT_BF16)) ||
           (xdt == DT_F16 && (pdt == DT_F32 || pdt == DT_F16));
}

// Widest row a plan covers: 16 waves x 64 lanes x 2 chunks (bf16) or x 4 chunks (f32).
constexpr int64_t kMaxN = 16384;

struct Plan {
    int mode = MODE_ALIGNED;  // Mode
    int cpt = 1;              // 16-byte chunks per thread per row
    int rt = 1;               // rows per thread per tile
    int tpr = 1;              // threads per row
    int rpp = 1;              // row slots per workgroup
    int block = 64;           // workgroup size
    int64_t ntiles = 0;       // row tiles of rpp * rt rows
    int64_t grid = 0;         // workgroups (= partial rows of a backward)
    int64_t kt = 1;           // blocked assignment: consecutive tiles per workgroup
    int strided = 0;          // 1: grid-stride over tiles (grid * rpp a multiple of V)
    int ncb = 1;              // DyT column blocks per row (grid a multiple of ncb)
    int xcd_remap = 0;        // renumber workgroups XCD-contiguously (needs grid % 8 == 0)
    int flat = 0;             // LayerNorm narrow rows through the flat kernels: 1 with 16-byte
                              // chunks (aligned rows), 2 with 12-byte chunks (12 * 2^k-byte rows)
    int split = 0;            // wide unaligned rows through the split-row kernels (rwn_split.hpp)
    int pf = 0;               // software-pipelined tile loop: 0 off, 1 one tile ahead (cpt * rt <= 2),
                              // 2 two tiles ahead (cpt * rt == 1, vector modes)
    int base_shift = 0;       // SHIFTED: base misalignment in elements
    int64_t ws_rs = 0;        // backward partials: element (p, c) at ws[p * ws_rs + c * ws_cs]
    int64_t ws_cs = 0;
    size_t lds_bytes = 0;     // dynamic LDS of the backward stage 1
    int64_t M = 0, N = 0;
    int layout = 0;           // row operands: 0 dense [M, N]; 1 strided, every row 16-byte chunks
                              // at one shift; 2 strided, element by element (SCALAR)
    int64_t ps0 = 1, ps1 = 1; // parameter vectors' element strides
    RowMap rm{};              // strided row map (layouts 1 and 2), filled in by the caller

    int64_t partial_rows() const { return grid / ncb; }
};

// Plan for one call.  misalign_bytes: address of the [M, N] operands modulo 16 (a multiple of
// the element size).  layout: 0 for dense [M, N] operands; 1 for strided operands whose rows
// all start misalign_bytes past a 16-byte boundary; 2 for strided operands of any alignment
// (SCALAR).  Strided plans run the general kernels with one row per thread.  cus: compute
// units of the device.  pdt: the parameter dtype, or -1 when
// the plan must hold for every parameter dtype of x's dtype (the workspace query).  occupancy:
// ask the runtime how many workgroups of the chosen kernel fit on a CU (needs a current device;
// false plans from launch bounds alone).  Returns false if N is too wide.
bool make_plan(int layer, bool backward, int64_t M, int64_t N, int xdt, int pdt, int misalign_bytes,
               int cus, bool occupancy, Plan* out, int layout = 0);

// Workgroups of the plan's kernel that fit on one CU at once (registers, LDS, wave slots), from
// the runtime; 0 if unknown.  One function per layer, defined beside that layer's launchers.
int resident_wgs_dyt(bool backward, const Plan& p, int xdt, int pdt);
int resident_wgs_ln(bool backward, const Plan& p, int xdt, int pdt);
int resident_wgs_rms(bool backward, const Plan& p, int xdt, int pdt);
int resident_wgs_ln_bwd(const Plan& p, int xdt, int pdt);
int resident_wgs_rms_bwd(const Plan& p, int xdt, int pdt);
// Strided plans (layouts 1 and 2), launched from launch_strided_*.hip.
int resident_wgs_dyt_strided(bool backward, const Plan& p, int xdt, int pdt);
int resident_wgs_ln_strided(bool backward, const Plan& p, int xdt, int pdt);
int resident_wgs_rms_strided(bool backward, const Plan& p, int xdt, int pdt);

// hipOccupancyMaxActiveBlocksPerMultiprocessor for one kernel, cached (0 on failure).
int kernel_occupancy(const void* kernel, int block, size_t dyn_lds);

// Partial-row columns of a backward: 2N + ncb (DyT: dgamma | dbeta | one dalpha column per
// column block), 2N (LayerNorm), N (RMSNorm).
inline int64_t partial_cols(int layer, int64_t N, int ncb = 1) {
    return layer == LAYER_DYT ? 2 * N + ncb : layer == LAYER_LN ? 2 * N : N;
}

inline Geom make_geom(const Plan& p) {
    Geom g;
    g.M = p.M;
    g.N = p.N;
    g.ntiles = p.ntiles;
    g.kt = p.kt;
    g.ws_rs = p.ws_rs;
    g.ws_cs = p.ws_cs;
    g.strided = p.strided;
    g.ncb = p.ncb;
    g.xcd_remap = p.xcd_remap;
    g.tpr = p.tpr;
    g.rpp = p.rpp;
    g.base_shift = p.base_shift;
    g.inv_n = 1.0f / (float)p.N;
    g.w_offset = 0.0f;
    g.pitch = p.layout ? 0 : p.N;
    g.ps0 = p.ps0;
    g.ps1 = p.ps1;
    g.rm = p.rm;
    return g;
}

template <typename T> struct TypeTag { using type = T; };

// Backward stage 1 with (PG = 1) or without (PG = 0) parameter-gradient partials: a NULL
// workspace means no parameter gradient is wanted.
template <typename F>
hipError_t dispatch_pg(const float* ws, F&& f) {
    return ws ? f(IC<1>{}) : f(IC<0>{});
}

// LayerNorm's gradient selection as a template value: bit 0 dgamma, bit 1 dbeta (no workspace:
// dx only, whatever the mask says).
template <typename F>
hipError_t dispatch_ln_grads(const float* ws, int grads, F&& f) {
    if (!ws) return f(IC<0>{});
    switch (grads & 3) {
    case 1: return f(IC<1>{});
    case 2: return f(IC<2>{});
    case 3: return f(IC<3>{});
    default: return f(IC<0>{});
    }
}

// The form as a template value: 0 for the Llama form, 1 for both float32 forms (the
// (1 + weight) one adds g.w_offset = 1 to the weight).
template <typename F>
hipError_t dispatch_variant(int variant, Geom& g, F&& f) {
    g.w_offset = variant == RMS_ONE_PLUS_WEIGHT ? 1.0f : 0.0f;
    if (variant == RMS_CAST_THEN_WEIGHT) return f(IC<0>{});
    if (variant == RMS_WEIGHT_THEN_CAST || variant == RMS_ONE_PLUS_WEIGHT) return f(IC<1>{});
    return hipErrorInvalidValue;
}

// Calls f(TypeTag<T>, TypeTag<PT>) for the supported dtype pairs.
template <typename F>
hipError_t dispatch_dtypes(int xdt, int pdt, F&& f) {
    if (xdt == DT_F32 && pdt == DT_F32) return f(TypeTag<float>{}, TypeTag<float>{});
    if (xdt == DT_BF16 && pdt == DT_F32) return f(TypeTag<bf16_t>{}, TypeTag<float>{});
    if (xdt == DT_BF16 && pdt == DT_BF16) return f(TypeTag<bf16_t>{}, TypeTag<bf16_t>{});
    if (xdt == DT_F16 && pdt == DT_F32) return f(TypeTag<f16_t>{}, TypeTag<float>{});
    if (xdt == DT_F16 && pdt == DT_F16) return f(TypeTag<f16_t>{}, TypeTag<f16_t>{});
    return hipErrorInvalidValue;
}

// The pipelined tile loop (PF = 1) exists for shapes with at most two chunks per thread per
// tensor.
template <typename F>
hipError_t dispatch_pf(const Plan& p, F&& f) {
    return p.pf ? f(IC<1>{}) : f(IC<0>{});
}

// One chunk, one row per thread: the two-tile-deep pipeline (PF = 2) exists as well.
template <typename F>
hipError_t dispatch_pf2(const Plan& p, F&& f) {
    return p.pf == 2 ? f(IC<2>{}) : p.pf ? f(IC<1>{}) : f(IC<0>{});
}

// Calls f(IC<MODE>, IC<CPT>, IC<RT>, IC<PF>, IC<LAY>) for the instantiated shapes of one side:
// S = false the dense plans (LAY 0), S = true the strided ones (LAY 1: layouts 1 and 2, one row
// per thread).  A plan of the other side returns hipErrorInvalidValue.
template <typename T, bool S, typename F>
hipError_t dispatch_shape(const Plan& p, F&& f) {
    if ((p.pf && p.cpt * p.rt > 2) || (p.pf == 2 && (p.cpt * p.rt != 1 || p.mode == MODE_SCALAR)))
        return hipErrorInvalidValue;
    if ((p.layout != 0) != S) return hipErrorInvalidValue;
    if constexpr (S) {
        if (p.rt != 1) return hipErrorInvalidValue;
        const IC<1> strided;
        auto by_cpt = [&](auto mode) {
            if (p.cpt == 1) {
                if constexpr (decltype(mode)::value == MODE_SCALAR)
                    return dispatch_pf(p, [&](auto pf) { return f(mode, IC<1>{}, IC<1>{}, pf, strided); });
                else
                    return dispatch_pf2(p, [&](auto pf) { return f(mode, IC<1>{}, IC<1>{}, pf, strided); });
            }
            if (p.cpt == 2) return dispatch_pf(p, [&](auto pf) { return f(mode, IC<2>{}, IC<1>{}, pf, strided); });
            if (p.cpt == 4) return f(mode, IC<4>{}, IC<1>{}, IC<0>{}, strided);
            return hipErrorInvalidValue;
        };
        if (p.mode == MODE_ALIGNED) return by_cpt(IC<MODE_ALIGNED>{});
        if (p.mode == MODE_SHIFTED) return by_cpt(IC<MODE_SHIFTED>{});
        return by_cpt(IC<MODE_SCALAR>{});
    } else {
        const IC<0> dense;
        if (p.mode == MODE_ALIGNED) {
            if (p.rt == 4 && p.cpt == 1) return f(IC<MODE_ALIGNED>{}, IC<1>{}, IC<4>{}, IC<0>{}, dense);
            if (p.rt == 2 && p.cpt == 1)
                return dispatch_pf(p, [&](auto pf) { return f(IC<MODE_ALIGNED>{}, IC<1>{}, IC<2>{}, pf, dense); });
            if (p.rt == 1) {
                if (p.cpt == 1)
                    return dispatch_pf2(p, [&](auto pf) { return f(IC<MODE_ALIGNED>{}, IC<1>{}, IC<1>{}, pf, dense); });
                if (p.cpt == 2)
                    return dispatch_pf(p, [&](auto pf) { return f(IC<MODE_ALIGNED>{}, IC<2>{}, IC<1>{}, pf, dense); });
                if (p.cpt == 4) return f(IC<MODE_ALIGNED>{}, IC<4>{}, IC<1>{}, IC<0>{}, dense);
            }
        } else if (p.mode == MODE_SHIFTED && p.rt == 1) {
            if (p.cpt == 1)
                return dispatch_pf2(p, [&](auto pf) { return f(IC<MODE_SHIFTED>{}, IC<1>{}, IC<1>{}, pf, dense); });
            if (p.cpt == 2)
                return dispatch_pf(p, [&](auto pf) { return f(IC<MODE_SHIFTED>{}, IC<2>{}, IC<1>{}, pf, dense); });
            if (p.cpt == 4) return f(IC<MODE_SHIFTED>{}, IC<4>{}, IC<1>{}, IC<0>{}, dense);
        } else if (p.mode == MODE_SCALAR && p.rt == 1) {
            if (p.cpt == 1)
                return dispatch_pf(p, [&](auto pf) { return f(IC<MODE_SCALAR>{}, IC<1>{}, IC<1>{}, pf, dense); });
            if (p.cpt == 2)
                return dispatch_pf(p, [&](auto pf) { return f(IC<MODE_SCALAR>{}, IC<2>{}, IC<1>{}, pf, dense); });
            if (p.cpt == 4) return f(IC<MODE_SCALAR>{}, IC<4>{}, IC<1>{}, IC<0>{}, dense);
        }
        return hipErrorInvalidValue;
    }
}

// Largest workgroup each kernel shape is compiled for (its amdgpu_flat_work_group_size):
// narrow plans (RT > 1) 256 threads; one chunk per thread, and bfloat16 with four, 512;
// otherwise 1024.  The planner keeps to it and every launcher checks it.
constexpr int max_block(int rt, int cpt, int esz) {
    return rt > 1 ? 256 : (cpt == 1 || (cpt == 4 && esz == 2)) ? 512 : 1024;
}

// Trace events of the next launch on this thread (set by the API while tracing).  When set,
// the kernel goes out through hipExtLaunchKernelGGL, which records the start and stop
// timestamps inside the dispatch packet itself instead of as separate queue packets.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& launch_events();

template <typename K, typename... Args>
hipError_t launch(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, Args... args) {
    const LaunchEvents ev = launch_events();
    if (ev.start)
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, ev.start, ev.stop, 0u, args...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
    return hipGetLastError();
}

// ---------------------------------------------------------------- launchers (one per kernel)
hipError_t launch_dyt_fwd(const Plan& p, int xdt, int pdt, const void* x, const void* alpha,
                          const void* gamma, const void* beta, void* y, hipStream_t s);
hipError_t launch_dyt_bwd(const Plan& p, int xdt, int pdt, const void* x, const void* dy,
                          const void* alpha, const void* gamma, void* dx, float* ws,
                          hipStream_t s);
hipError_t launch_ln_fwd(const Plan& p, int xdt, int pdt, const void* x, const void* gamma,
                         const void* beta, float eps, void* y, float* mean, float* rstd,
                         hipStream_t s);
hipError_t launch_ln_bwd(const Plan& p, int xdt, int pdt, const void* x, const void* dy,
                         const float* mean, const float* rstd, const void* gamma, float eps,
                         void* dx, float* ws, int grads, hipStream_t s);
// The flat LayerNorm kernels of narrow aligned rows (plans with p.flat set).
hipError_t launch_ln_fwd_flat(const Plan& p, int xdt, int pdt, const void* x, const void* gamma,
                              const void* beta, float eps, void* y, float* mean, float* rstd,
                              hipStream_t s);
hipError_t launch_ln_bwd_flat(const Plan& p, int xdt, int pdt, const void* x, const void* dy,
                              const float* mean, const float* rstd, const void* gamma, float eps,
                              void* dx, float* ws, int grads, hipStream_t s);
int resident_wgs_ln_flat(bool backward, const Plan& p, int xdt, int pdt);
hipError_t launch_dyt_fwd_flat(const Plan& p, int xdt, int pdt, const void* x, const void* alpha,
                               const void* gamma, const void* beta, void* y, hipStream_t s);
hipError_t launch_dyt_bwd_flat(const Plan& p, int xdt, int pdt, const void* x, const void* dy,
                               const void* alpha, const void* gamma, void* dx, float* ws, hipStream_t s);
int resident_wgs_dyt_flat(bool backward, const Plan& p, int xdt, int pdt);

hipError_t launch_rms_fwd(const Plan& p, int xdt, int pdt, int variant, const void* x, const void* w,
                          float eps, void* y, float* rstd, hipStream_t s);
hipError_t launch_rms_bwd(const Plan& p, int xdt, int pdt, int variant, const void* x, const void* dy,
                          const float* rstd, const void* w, float eps, void* dx, float* ws,
                          hipStream_t s);
// Stage 2: P partial rows of ng columns (element (p, c) at ws[p * rs + c * cs]) ->
// out0 [N], out1 [N], out2 [1] in param dtype pdt.
// The split-row kernels (plans with p.split set): wide rows not aligned to 16-byte chunks.
hipError_t launch_dyt_fwd_split(const Plan& p, int xdt, int pdt, const void* x, const void* alpha,
                                const void* gamma, const void* beta, void* y, hipStream_t s);
hipError_t launch_dyt_bwd_split(const Plan& p, int xdt, int pdt, const void* x, const void* dy,
                                const void* alpha, const void* gamma, void* dx, float* ws, hipStream_t s);
hipError_t launch_ln_fwd_split(const Plan& p, int xdt, int pdt, const void* x, const void* gamma,
                               const void* beta, float eps, void* y, float* mean, float* rstd, hipStream_t s);
hipError_t launch_ln_bwd_split(const Plan& p, int xdt, int pdt, const void* x, const void* dy,
                               const float* mean, const float* rstd, const void* gamma, float eps,
                               void* dx, float* ws, int grads, hipStream_t s);
hipError_t launch_rms_fwd_split(const Plan& p, int xdt, int pdt, int variant, const void* x, const void* w,
                                float eps, void* y, float* rstd, hipStream_t s);
hipError_t launch_rms_bwd_split(const Plan& p, int xdt, int pdt, int variant, const void* x, const void* dy,
                                const float* rstd, const void* w, float eps, void* dx, float* ws, hipStream_t s);
int resident_wgs_split(int layer, bool backward, const Plan& p, int xdt, int pdt);
hipError_t launch_dyt_fwd_strided(const Plan& p, int xdt, int pdt, const void* x, const void* alpha,
                                  const void* gamma, const void* beta, void* y, hipStream_t s);
hipError_t launch_dyt_bwd_strided(const Plan& p, int xdt, int pdt, const void* x, const void* dy,
                                  const void* alpha, const void* gamma, void* dx, float* ws, hipStream_t s);
hipError_t launch_ln_fwd_strided(const Plan& p, int xdt, int pdt, const void* x, const void* gamma,
                                 const void* beta, float eps, void* y, float* mean, float* rstd, hipStream_t s);
hipError_t launch_ln_bwd_strided(const Plan& p, int xdt, int pdt, const void* x, const void* dy,
                                 const float* mean, const float* rstd, const void* gamma, float eps,
                                 void* dx, float* ws, int grads, hipStream_t s);
hipError_t launch_rms_fwd_strided(const Plan& p, int xdt, int pdt, int variant, const void* x, const void* w,
                                  float eps, void* y, float* rstd, hipStream_t s);
hipError_t launch_rms_bwd_strided(const Plan& p, int xdt, int pdt, int variant, const void* x, const void* dy,
                                  const float* rstd, const void* w, float eps, void* dx, float* ws, hipStream_t s);

// Stage 2: sums the P partial rows of columns [c_lo, c_hi) (column c at ws + c * cs, partial
// row p at + p * rs) into out0 (columns [0, N)), out1 ([N, 2N)) and out2 (column 2N, which also
// takes the columns after it).  Only the requested gradients' columns are read.
hipError_t launch_colreduce(int pdt, const float* ws, int64_t P, int64_t ng, int64_t rs, int64_t cs,
                            int64_t N, int64_t c_lo, int64_t c_hi, void* out0, void* out1, void* out2,
                            hipStream_t s);
hipError_t launch_stream_probe(const void* a, const void* b, void* out, size_t bytes, int unroll,
                               int nontemporal, int wg_per_cu, int cus, hipStream_t s);

}  // namespace rwn
