// C ABI of librwnorm: argument validation, launch planning and kernel-duration tracing.
// Declarations and the contract of each entry point are in include/rwnorm.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/rwnorm.h"
#include "rwn_launch.hpp"

#define RWN_API extern "C" __attribute__((visibility("default")))

using namespace rwn;

namespace {

thread_local char g_err[512] = "";

rwn_status ok() {
    g_err[0] = '\0';
    return RWN_OK;
}

rwn_status fail(rwn_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

rwn_status hip_fail(hipError_t e, const char* what) {
    return fail(RWN_ERR_LAUNCH, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

// Compute units of the current device, cached per device.
rwn_status device_cus(int* cus) {
    static std::atomic<int> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev >= 0 && dev < 64) {
        int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) {
            *cus = v;
            return RWN_OK;
        }
    }
    int v = 0;
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(MultiprocessorCount)");
    if (v <= 0) return fail(RWN_ERR_LAUNCH, "device reports %d compute units", v);
    if (dev >= 0 && dev < 64) cache[dev].store(v, std::memory_order_relaxed);
    *cus = v;
    return RWN_OK;
}

rwn_status check_shape_dtypes(const char* fn, int64_t M, int64_t N, rwn_dtype xdt, rwn_dtype pdt) {
    if (M < 0) return fail(RWN_ERR_INVALID_ARG, "%s: M must be >= 0 (got %lld)", fn, (long long)M);
    if (N < 1) return fail(RWN_ERR_INVALID_ARG, "%s: N must be >= 1 (got %lld)", fn, (long long)N);
    if ((int)xdt != RWN_F32 && (int)xdt != RWN_BF16 && (int)xdt != RWN_F16)
        return fail(RWN_ERR_INVALID_ARG, "%s: unknown x dtype code %d", fn, (int)xdt);
    if ((int)pdt != RWN_F32 && (int)pdt != RWN_BF16 && (int)pdt != RWN_F16)
        return fail(RWN_ERR_INVALID_ARG, "%s: unknown parameter dtype code %d", fn, (int)pdt);
    if (!dtype_pair_ok((int)xdt, (int)pdt)) {
        static const char* names[3] = {"float32", "bfloat16", "float16"};
        return fail(RWN_ERR_UNSUPPORTED, "%s: %s x with %s parameters is not supported", fn,
                    names[(int)xdt], names[(int)pdt]);
    }
    if (N > kMaxN)
        return fail(RWN_ERR_UNSUPPORTED, "%s: N = %lld is wider than the supported %lld", fn,
                    (long long)N, (long long)kMaxN);
    if (M > 0 && N > INT64_MAX / M)
        return fail(RWN_ERR_INVALID_ARG, "%s: M * N overflows", fn);
    return RWN_OK;
}

rwn_status check_eps(const char* fn, float eps) {
    if (!(eps >= 0.0f) || isinf(eps))
        return fail(RWN_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
    return RWN_OK;
}

// The [M, N] operands must be element aligned and share their address modulo 16.
rwn_status check_operands(const char* fn, rwn_dtype xdt, const void* const* ptrs,
                          const char* const* names, int n, int* misalign) {
    const uintptr_t esz = xdt == RWN_F32 ? 4 : 2;
    int m = -1;
    for (int i = 0; i < n; ++i) {
        if (!ptrs[i]) return fail(RWN_ERR_INVALID_ARG, "%s: %s is NULL", fn, names[i]);
        const uintptr_t a = (uintptr_t)ptrs[i];
        if (a % esz) return fail(RWN_ERR_INVALID_ARG, "%s: %s is not aligned to its element size", fn, names[i]);
        const int mm = (int)(a % 16);
        if (m < 0) m = mm;
        else if (mm != m)
            return fail(RWN_ERR_UNSUPPORTED,
                        "%s: %s does not share the address modulo 16 of %s (%d vs %d); pass freshly "
                        "allocated or equally offset buffers", fn, names[i], names[0], mm, m);
    }
    *misalign = m < 0 ? 0 : m;
    return RWN_OK;
}

// --------------------------------------------------------------------------- tracing

struct TraceEntry {
    int tag;
    hipEvent_t a, b;
};

struct Trace {
    bool on = false;
    int cap = 0;
    int used = 0;
    std::vector<TraceEntry> ev;
};

thread_local Trace g_trace;

template <typename F>
hipError_t traced(int tag, hipStream_t s, F&& launch) {
    Trace& t = g_trace;
    if (!t.on || t.used >= t.cap) return launch();
    TraceEntry& e = t.ev[t.used];
    // The launch records its own start/stop timestamps (see rwn::launch).
    (void)s;
    launch_events() = LaunchEvents{e.a, e.b};
    hipError_t r = launch();
    launch_events() = LaunchEvents{};
    if (r != hipSuccess) return r;
    e.tag = tag;
    ++t.used;
    return hipSuccess;
}

// Row operands of a *_strided call, validated by strided_rows(): the plan's layout (0 when the
// operands are dense after all), the rows' common misalignment and the row map.
struct Strided {
    int layout = 0;
    int misalign = 0;
    int64_t ps0 = 1, ps1 = 1;
    RowMap rm{};
};

rwn_status plan_for(const char* fn, int layer, bool bwd, int64_t M, int64_t N, rwn_dtype xdt,
                    rwn_dtype pdt, int misalign, Plan* p, const Strided* sr = nullptr) {
    int cus = 0;
    rwn_status st = device_cus(&cus);
    if (st != RWN_OK) return st;
    const int layout = sr ? sr->layout : 0;
    if (sr) misalign = sr->misalign;
    // The backward's grid is also its workspace's row count: it is planned for every parameter
    // dtype at once, exactly as the workspace query plans it.
    if (!make_plan(layer, bwd, M, N, (int)xdt, bwd ? -1 : (int)pdt, misalign, cus, true, p, layout)) {
        if (layout == 2)
            return fail(RWN_ERR_UNSUPPORTED,
                        "%s: N = %lld is too wide for strided rows that do not all start at one "
                        "16-byte offset with strides a multiple of %d elements (element-wise rows "
                        "take at most %d elements)", fn, (long long)N, xdt == RWN_F32 ? 4 : 8,
                        xdt == RWN_F32 ? 4096 : 2048);
        return fail(RWN_ERR_UNSUPPORTED,
                    "%s: N = %lld with operands %d bytes past a 16-byte boundary needs more than "
                    "1024 threads per row; use 16-byte-aligned operands and N a multiple of %d",
                    fn, (long long)N, misalign, xdt == RWN_F32 ? 4 : 8);
    }
    if (sr) {
        p->rm = sr->rm;
        p->ps0 = sr->ps0;
        p->ps1 = sr->ps1;
    }
    return RWN_OK;
}

// One strided row operand of a call: base, the caller's nlead strides, the row-map slot it takes
// (OP_X, OP_DY, OP_OUT) and whether the call writes it.
struct StridedOperand {
    const void* p;
    const int64_t* strides;
    const char* name;
    int slot;
    bool out;
};

// Largest byte span of a strided operand: one buffer descriptor covers it, with offsets below
// the out-of-range marker.
constexpr int64_t kMaxSpanBytes = kMaxRecords - 16;

// Validates the leading sizes, the operands' strides and the parameter strides of a *_strided
// call, and chooses the plan layout: 0 when every operand is in fact a dense [M, N] matrix at
// one address modulo 16 and the parameters are contiguous (the dense kernels then run); 1 when
// every row of every operand starts at one offset modulo 16 bytes (strides multiples of the
// 16-byte chunk, bases at one address modulo 16); 2 otherwise (rows element by element).
rwn_status strided_rows(const char* fn, int nlead, const int64_t* lead, int64_t N, rwn_dtype xdt,
                        rwn_dtype pdt, const StridedOperand* ops, int nops, int64_t ps0, int64_t ps1,
                        int64_t* M_out, Strided* sr) {
    if (nlead < 1 || nlead > 3) return fail(RWN_ERR_INVALID_ARG, "%s: nlead must be 1, 2 or 3 (got %d)", fn, nlead);
    if (!lead) return fail(RWN_ERR_INVALID_ARG, "%s: lead is NULL", fn);
    int64_t sz[3] = {1, 1, 1};
    int64_t M = 1;
    for (int i = 0; i < nlead; ++i) {
        if (lead[i] < 0) return fail(RWN_ERR_INVALID_ARG, "%s: lead[%d] = %lld is negative", fn, i, (long long)lead[i]);
        sz[3 - nlead + i] = lead[i];
    }
    for (int d = 0; d < 3; ++d) {
        if (sz[d] == 0) M = 0;
        else if (M > 0 && sz[d] > (int64_t)INT32_MAX / M) M = -1;
        else if (M > 0) M *= sz[d];
    }
    if (M < 0) return fail(RWN_ERR_UNSUPPORTED, "%s: more than 2^31 - 1 strided rows", fn);
    rwn_status st = check_shape_dtypes(fn, M, N, xdt, pdt);
    if (st != RWN_OK) return st;
    if (ps0 < 0 || ps1 < 0) return fail(RWN_ERR_INVALID_ARG, "%s: parameter strides must be >= 0", fn);
    const int64_t esz = xdt == RWN_F32 ? 4 : 2, V = 16 / esz;
    bool uniform = true, dense = N == 1 || (ps0 == 1 && ps1 == 1);
    int mis = -1;
    *sr = Strided{};
    for (int k = 0; k < nops; ++k) {
        const StridedOperand& o = ops[k];
        if (!o.strides) return fail(RWN_ERR_INVALID_ARG, "%s: %s strides are NULL", fn, o.name);
        int64_t str[3] = {0, 0, 0};
        for (int i = 0; i < nlead; ++i) {
            if (o.strides[i] < 0)
                return fail(RWN_ERR_INVALID_ARG, "%s: %s stride %d is negative", fn, o.name, i);
            str[3 - nlead + i] = o.strides[i];
        }
        if (M == 0) continue;   // nothing is read or written
        if (!o.p) return fail(RWN_ERR_INVALID_ARG, "%s: %s is NULL", fn, o.name);
        const uintptr_t a = (uintptr_t)o.p;
        if (a % (uintptr_t)esz) return fail(RWN_ERR_INVALID_ARG, "%s: %s is not aligned to its element size", fn, o.name);
        // Offset of the last row's first element; stays far below 2^63 while within the span cap.
        int64_t last = 0;
        for (int d = 0; d < 3; ++d) {
            if (sz[d] < 2) continue;
            if (str[d] > (kMaxSpanBytes / esz) / (sz[d] - 1)) { last = -1; break; }
            last += (sz[d] - 1) * str[d];
            if (last > kMaxSpanBytes / esz) { last = -1; break; }
        }
        const int64_t span = last < 0 ? -1 : (last + N) * esz;
        if (span < 0 || span > kMaxSpanBytes)
            return fail(RWN_ERR_UNSUPPORTED, "%s: %s spans more than %lld bytes; pass a contiguous copy", fn, o.name,
                        (long long)kMaxSpanBytes);
        if (o.out) {
            // Rows that never share an element: with the dimensions in increasing stride order,
            // each stride at least spans everything inside it.
            int order[3] = {0, 1, 2};
            for (int i = 0; i < 3; ++i)
                for (int j = i + 1; j < 3; ++j)
                    if (str[order[j]] < str[order[i]]) std::swap(order[i], order[j]);
            int64_t extent = N;
            for (int i = 0; i < 3; ++i) {
                const int d = order[i];
                if (sz[d] < 2) continue;
                if (str[d] < extent) return fail(RWN_ERR_INVALID_ARG, "%s: rows of %s overlap", fn, o.name);
                extent += (sz[d] - 1) * str[d];
            }
        }
        const int m = (int)(a % 16);
        if (mis < 0) mis = m;
        else if (m != mis) uniform = dense = false;
        int64_t expect = N;
        for (int d = 2; d >= 0; --d) {
            if (sz[d] > 1) {
                if (str[d] % V) uniform = false;
                if (str[d] != expect) dense = false;
            }
            expect *= sz[d];
        }
        for (int d = 0; d < 3; ++d) sr->rm.st[o.slot][d] = str[d];
        sr->rm.span[o.slot] = span;
    }
    *M_out = M;
    if (M == 0) return RWN_OK;
    sr->layout = dense ? 0 : uniform ? 1 : 2;
    sr->misalign = sr->layout == 2 ? 0 : mis;
    sr->ps0 = ps0;
    sr->ps1 = ps1;
    sr->rm.d1 = make_divisor((uint32_t)sz[1]);
    sr->rm.d2 = make_divisor((uint32_t)sz[2]);
    return RWN_OK;
}

rwn_status workspace_size(int layer, int64_t M, int64_t N, rwn_dtype xdt, size_t* bytes) {
    const char* fn = layer == LAYER_DYT ? "dyt_bwd_workspace_size"
                     : layer == LAYER_LN ? "layernorm_bwd_workspace_size"
                                         : "rmsnorm_bwd_workspace_size";
    if (!bytes) return fail(RWN_ERR_INVALID_ARG, "%s: bytes is NULL", fn);
    rwn_status st = check_shape_dtypes(fn, M, N, xdt, RWN_F32);
    if (st != RWN_OK) return st;
    if (M == 0) {
        *bytes = 0;
        return ok();
    }
    // The plan depends on the operands' address modulo 16; size for the largest.
    const int esz = xdt == RWN_F32 ? 4 : 2;
    size_t most = 0;
    int cus = 0;
    if ((st = device_cus(&cus)) != RWN_OK) return st;
    // Dense and strided operands (layouts 0, 1 and 2) alike.
    for (int layout = 0; layout < 3; ++layout) {
        for (int mis = 0; mis < 16; mis += esz) {
            if (layout == 2 && mis) break;
            Plan p;
            // a shape with no plan is rejected by the backward itself
            if (!make_plan(layer, true, M, N, (int)xdt, -1, mis, cus, true, &p, layout)) continue;
            const size_t need = (size_t)p.partial_rows() * (size_t)partial_cols(layer, N, p.ncb) * sizeof(float);
            if (need > most) most = need;
        }
    }
    *bytes = most;
    return ok();
}

rwn_status check_workspace(const char* fn, const Plan& p, int layer, const void* ws, size_t ws_bytes) {
    const size_t need = (size_t)p.partial_rows() * (size_t)partial_cols(layer, p.N, p.ncb) * sizeof(float);
    if (need == 0) return RWN_OK;
    if (!ws) return fail(RWN_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", fn, need);
    if (ws_bytes < need)
        return fail(RWN_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", fn, ws_bytes, need);
    if ((uintptr_t)ws % 4) return fail(RWN_ERR_INVALID_ARG, "%s: workspace is not 4-byte aligned", fn);
    return RWN_OK;
}

// Stage 2 (also the whole backward when M == 0: P = 0 partial rows give zeros).  Reads only
// the columns from the first requested output's to the last's.
rwn_status finish_bwd(const char* fn, int pdt, const float* ws, int64_t P, int64_t ng, int64_t rs,
                      int64_t cs, int64_t N, void* out0, void* out1, void* out2, hipStream_t s) {
    if (!out0 && !out1 && !out2) return ok();
    const int64_t c_lo = out0 ? 0 : out1 ? N : 2 * N;
    const int64_t c_hi = out2 ? ng : out1 ? 2 * N : N;
    hipError_t e = traced(RWN_K_COLREDUCE, s, [&] {
        return launch_colreduce(pdt, ws, P, ng, rs, cs, N, c_lo, c_hi, out0, out1, out2, s);
    });
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

}  // namespace

// ====================================================================================== DyT

namespace {

rwn_status dyt_fwd_impl(const char* fn, int64_t M, int64_t N, const void* x, rwn_dtype x_dtype,
                        const void* alpha, const void* gamma, const void* beta, rwn_dtype param_dtype,
                        void* y, void* stream, const Strided* sr) {
    rwn_status st = check_shape_dtypes(fn, M, N, x_dtype, param_dtype);
    if (st != RWN_OK) return st;
    if (!alpha || !gamma || !beta) return fail(RWN_ERR_INVALID_ARG, "%s: alpha, gamma and beta are required", fn);
    if (M == 0) return ok();
    const void* ops[2] = {x, y};
    const char* names[2] = {"x", "y"};
    int mis = 0;
    if (!sr && (st = check_operands(fn, x_dtype, ops, names, 2, &mis)) != RWN_OK) return st;
    Plan p;
    if ((st = plan_for(fn, LAYER_DYT, false, M, N, x_dtype, param_dtype, mis, &p, sr)) != RWN_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = traced(RWN_K_DYT_FWD, s, [&] {
        return launch_dyt_fwd(p, x_dtype, param_dtype, x, alpha, gamma, beta, y, s);
    });
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

rwn_status dyt_bwd_impl(const char* fn, int64_t M, int64_t N, const void* x, const void* dy,
                        rwn_dtype x_dtype, const void* alpha, const void* gamma, rwn_dtype param_dtype,
                        void* dx, void* dalpha, void* dgamma, void* dbeta, void* workspace,
                        size_t workspace_bytes, void* stream, const Strided* sr) {
    rwn_status st = check_shape_dtypes(fn, M, N, x_dtype, param_dtype);
    if (st != RWN_OK) return st;
    if (!alpha || !gamma) return fail(RWN_ERR_INVALID_ARG, "%s: alpha and gamma are required", fn);
    hipStream_t s = (hipStream_t)stream;
    const int64_t ng = partial_cols(LAYER_DYT, N);
    if (M == 0) return finish_bwd(fn, param_dtype, nullptr, 0, ng, ng, 1, N, dgamma, dbeta, dalpha, s);
    const void* ops[3] = {x, dy, dx};
    const char* names[3] = {"x", "dy", "dx"};
    int mis = 0;
    if (!sr && (st = check_operands(fn, x_dtype, ops, names, 3, &mis)) != RWN_OK) return st;
    Plan p;
    if ((st = plan_for(fn, LAYER_DYT, true, M, N, x_dtype, param_dtype, mis, &p, sr)) != RWN_OK) return st;
    // No parameter gradient wanted: dx only, no workspace, no stage 2.
    const bool grads = dgamma || dbeta || dalpha;
    if (grads && (st = check_workspace(fn, p, LAYER_DYT, workspace, workspace_bytes)) != RWN_OK) return st;
    float* ws = grads ? (float*)workspace : nullptr;
    hipError_t e = traced(RWN_K_DYT_BWD, s, [&] {
        return launch_dyt_bwd(p, x_dtype, param_dtype, x, dy, alpha, gamma, dx, ws, s);
    });
    if (e != hipSuccess) return hip_fail(e, fn);
    return finish_bwd(fn, param_dtype, ws, p.partial_rows(), partial_cols(LAYER_DYT, N, p.ncb), p.ws_rs,
                      p.ws_cs, N, dgamma, dbeta, dalpha, s);
}

}  // namespace

RWN_API rwn_status dyt_fwd(int64_t M, int64_t N, const void* x, rwn_dtype x_dtype,
                           const void* alpha, const void* gamma, const void* beta,
                           rwn_dtype param_dtype, void* y, void* stream) {
    return dyt_fwd_impl("dyt_fwd", M, N, x, x_dtype, alpha, gamma, beta, param_dtype, y, stream, nullptr);
}

RWN_API rwn_status dyt_bwd(int64_t M, int64_t N, const void* x, const void* dy, rwn_dtype x_dtype,
                           const void* alpha, const void* gamma, rwn_dtype param_dtype, void* dx,
                           void* dalpha, void* dgamma, void* dbeta, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return dyt_bwd_impl("dyt_bwd", M, N, x, dy, x_dtype, alpha, gamma, param_dtype, dx, dalpha, dgamma, dbeta,
                        workspace, workspace_bytes, stream, nullptr);
}

RWN_API rwn_status dyt_bwd_workspace_size(int64_t M, int64_t N, rwn_dtype x_dtype, size_t* bytes) {
    return workspace_size(LAYER_DYT, M, N, x_dtype, bytes);
}

// ================================================================================ LayerNorm

namespace {

rwn_status ln_fwd_impl(const char* fn, int64_t M, int64_t N, const void* x, rwn_dtype x_dtype,
                       const void* gamma, const void* beta, rwn_dtype param_dtype, float eps, void* y,
                       float* mean, float* rstd, void* stream, const Strided* sr) {
    rwn_status st = check_shape_dtypes(fn, M, N, x_dtype, param_dtype);
    if (st != RWN_OK) return st;
    if ((st = check_eps(fn, eps)) != RWN_OK) return st;
    if (M == 0) return ok();
    const void* ops[2] = {x, y};
    const char* names[2] = {"x", "y"};
    int mis = 0;
    if (!sr && (st = check_operands(fn, x_dtype, ops, names, 2, &mis)) != RWN_OK) return st;
    if (((uintptr_t)mean % 4) || ((uintptr_t)rstd % 4))
        return fail(RWN_ERR_INVALID_ARG, "%s: mean/rstd must be float aligned", fn);
    Plan p;
    if ((st = plan_for(fn, LAYER_LN, false, M, N, x_dtype, param_dtype, mis, &p, sr)) != RWN_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = traced(RWN_K_LN_FWD, s, [&] {
        return launch_ln_fwd(p, x_dtype, param_dtype, x, gamma, beta, eps, y, mean, rstd, s);
    });
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

}  // namespace

RWN_API rwn_status layernorm_fwd(int64_t M, int64_t N, const void* x, rwn_dtype x_dtype,
                                 const void* gamma, const void* beta, rwn_dtype param_dtype,
                                 float eps, void* y, float* mean, float* rstd, void* stream) {
    return ln_fwd_impl("layernorm_fwd", M, N, x, x_dtype, gamma, beta, param_dtype, eps, y, mean, rstd, stream,
                       nullptr);
}

namespace {

// Static scratch of layernorm_bwd_noalloc: the partial rows live in this array instead of a
// caller workspace.  Each device that runs the library holds its own copy until the process
// ends; every call on a device shares it.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of this device's copy of `scratch`, looked up once per device (with that
// device current) and kept.  The array's name is a host-side stand-in in host code: only this
// address may be handed to kernels.
rwn_status scratch_address(const char* fn, float** out) {
    static std::mutex mu;
    static void* addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(RWN_ERR_UNSUPPORTED, "%s: device ordinal %d above 63", fn, dev);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(RWN_ERR_LAUNCH, "%s: hipGetSymbolAddress returned NULL", fn);
        addr[dev] = p;
    }
    *out = (float*)addr[dev];
    return RWN_OK;
}

// layernorm_bwd with the partial rows in the caller's workspace, or (static_scratch) in this
// device's copy of `scratch`.
rwn_status ln_bwd_impl(const char* fn, int64_t M, int64_t N, const void* x, const void* dy,
                       rwn_dtype x_dtype, const float* mean, const float* rstd, const void* gamma,
                       rwn_dtype param_dtype, float eps, void* dx, void* dgamma, void* dbeta,
                       void* workspace, size_t workspace_bytes, bool static_scratch, void* stream,
                       const Strided* sr = nullptr) {
    rwn_status st = check_shape_dtypes(fn, M, N, x_dtype, param_dtype);
    if (st != RWN_OK) return st;
    if ((st = check_eps(fn, eps)) != RWN_OK) return st;
    if ((mean == nullptr) != (rstd == nullptr))
        return fail(RWN_ERR_INVALID_ARG, "%s: pass both mean and rstd, or neither", fn);
    hipStream_t s = (hipStream_t)stream;
    const int64_t ng = partial_cols(LAYER_LN, N);
    if (M == 0) return finish_bwd(fn, param_dtype, nullptr, 0, ng, ng, 1, N, dgamma, dbeta, nullptr, s);
    const void* ops[3] = {x, dy, dx};
    const char* names[3] = {"x", "dy", "dx"};
    int mis = 0;
    if (!sr && (st = check_operands(fn, x_dtype, ops, names, 3, &mis)) != RWN_OK) return st;
    Plan p;
    if ((st = plan_for(fn, LAYER_LN, true, M, N, x_dtype, param_dtype, mis, &p, sr)) != RWN_OK) return st;
    // No parameter gradient wanted: dx only, no workspace, no stage 2.  Otherwise stage 1 writes
    // the partial columns of the requested gradients only.
    const bool grads = dgamma || dbeta;
    const int mask = (dgamma ? 1 : 0) | (dbeta ? 2 : 0);
    float* ws = nullptr;
    if (grads && static_scratch) {
        const size_t need = (size_t)p.partial_rows() * (size_t)ng * sizeof(float);
        if (need > kScratchBytes)
            return fail(RWN_ERR_UNSUPPORTED,
                        "%s: [%lld, %lld] needs %zu bytes of partial rows, more than the %zu-byte static "
                        "scratch; call layernorm_bwd with a workspace instead",
                        fn, (long long)M, (long long)N, need, kScratchBytes);
        if ((st = scratch_address(fn, &ws)) != RWN_OK) return st;
    } else if (grads) {
        if ((st = check_workspace(fn, p, LAYER_LN, workspace, workspace_bytes)) != RWN_OK) return st;
        ws = (float*)workspace;
    }
    hipError_t e = traced(RWN_K_LN_BWD, s, [&] {
        return launch_ln_bwd(p, x_dtype, param_dtype, x, dy, mean, rstd, gamma, eps, dx, ws, mask, s);
    });
    if (e != hipSuccess) return hip_fail(e, fn);
    return finish_bwd(fn, param_dtype, ws, p.partial_rows(), ng, p.ws_rs, p.ws_cs, N, dgamma, dbeta, nullptr, s);
}

}  // namespace

RWN_API rwn_status layernorm_bwd(int64_t M, int64_t N, const void* x, const void* dy,
                                 rwn_dtype x_dtype, const float* mean, const float* rstd,
                                 const void* gamma, rwn_dtype param_dtype, float eps, void* dx,
                                 void* dgamma, void* dbeta, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    return ln_bwd_impl("layernorm_bwd", M, N, x, dy, x_dtype, mean, rstd, gamma, param_dtype, eps, dx,
                       dgamma, dbeta, workspace, workspace_bytes, false, stream);
}

RWN_API rwn_status layernorm_bwd_noalloc(int64_t M, int64_t N, const void* x, const void* dy,
                                         rwn_dtype x_dtype, const float* mean, const float* rstd,
                                         const void* gamma, rwn_dtype param_dtype, float eps,
                                         void* dx, void* dgamma, void* dbeta, void* stream) {
    return ln_bwd_impl("layernorm_bwd_noalloc", M, N, x, dy, x_dtype, mean, rstd, gamma, param_dtype,
                       eps, dx, dgamma, dbeta, nullptr, 0, true, stream);
}

RWN_API rwn_status layernorm_bwd_workspace_size(int64_t M, int64_t N, rwn_dtype x_dtype, size_t* bytes) {
    return workspace_size(LAYER_LN, M, N, x_dtype, bytes);
}

// ================================================================================== RMSNorm

namespace {

rwn_status check_variant(const char* fn, int variant) {
    if (variant != RWN_RMS_CAST_THEN_WEIGHT && variant != RWN_RMS_WEIGHT_THEN_CAST &&
        variant != RWN_RMS_ONE_PLUS_WEIGHT)
        return fail(RWN_ERR_INVALID_ARG, "%s: unknown RMSNorm form %d", fn, variant);
    return RWN_OK;
}

rwn_status rms_fwd_impl(const char* fn, int64_t M, int64_t N, const void* x, rwn_dtype x_dtype,
                        const void* weight, rwn_dtype weight_dtype, float eps, int variant, void* y,
                        float* rstd, void* stream, const Strided* sr = nullptr) {
    rwn_status st = check_shape_dtypes(fn, M, N, x_dtype, weight_dtype);
    if (st != RWN_OK) return st;
    if ((st = check_variant(fn, variant)) != RWN_OK) return st;
    if ((st = check_eps(fn, eps)) != RWN_OK) return st;
    if (!weight) return fail(RWN_ERR_INVALID_ARG, "%s: weight is required", fn);
    if (M == 0) return ok();
    const void* ops[2] = {x, y};
    const char* names[2] = {"x", "y"};
    int mis = 0;
    if (!sr && (st = check_operands(fn, x_dtype, ops, names, 2, &mis)) != RWN_OK) return st;
    if ((uintptr_t)rstd % 4) return fail(RWN_ERR_INVALID_ARG, "%s: rstd must be float aligned", fn);
    Plan p;
    if ((st = plan_for(fn, LAYER_RMS, false, M, N, x_dtype, weight_dtype, mis, &p, sr)) != RWN_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = traced(RWN_K_RMS_FWD, s, [&] {
        return launch_rms_fwd(p, x_dtype, weight_dtype, variant, x, weight, eps, y, rstd, s);
    });
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

rwn_status rms_bwd_impl(const char* fn, int64_t M, int64_t N, const void* x, const void* dy,
                        rwn_dtype x_dtype, const float* rstd, const void* weight,
                        rwn_dtype weight_dtype, float eps, int variant, void* dx, void* dweight,
                        void* workspace, size_t workspace_bytes, void* stream, const Strided* sr = nullptr) {
    rwn_status st = check_shape_dtypes(fn, M, N, x_dtype, weight_dtype);
    if (st != RWN_OK) return st;
    if ((st = check_variant(fn, variant)) != RWN_OK) return st;
    if ((st = check_eps(fn, eps)) != RWN_OK) return st;
    if (!weight) return fail(RWN_ERR_INVALID_ARG, "%s: weight is required", fn);
    hipStream_t s = (hipStream_t)stream;
    const int64_t ng = partial_cols(LAYER_RMS, N);
    if (M == 0) return finish_bwd(fn, weight_dtype, nullptr, 0, ng, ng, 1, N, dweight, nullptr, nullptr, s);
    const void* ops[3] = {x, dy, dx};
    const char* names[3] = {"x", "dy", "dx"};
    int mis = 0;
    if (!sr && (st = check_operands(fn, x_dtype, ops, names, 3, &mis)) != RWN_OK) return st;
    Plan p;
    if ((st = plan_for(fn, LAYER_RMS, true, M, N, x_dtype, weight_dtype, mis, &p, sr)) != RWN_OK) return st;
    // No parameter gradient wanted: dx only, no workspace, no stage 2.
    const bool grads = dweight;
    if (grads && (st = check_workspace(fn, p, LAYER_RMS, workspace, workspace_bytes)) != RWN_OK) return st;
    float* ws = grads ? (float*)workspace : nullptr;
    hipError_t e = traced(RWN_K_RMS_BWD, s, [&] {
        return launch_rms_bwd(p, x_dtype, weight_dtype, variant, x, dy, rstd, weight, eps, dx, ws, s);
    });
    if (e != hipSuccess) return hip_fail(e, fn);
    return finish_bwd(fn, weight_dtype, ws, p.partial_rows(), ng, p.ws_rs, p.ws_cs, N, dweight, nullptr, nullptr, s);
}

}  // namespace

RWN_API rwn_status rmsnorm_fwd(int64_t M, int64_t N, const void* x, rwn_dtype x_dtype,
                               const void* weight, rwn_dtype weight_dtype, float eps, void* y,
                               float* rstd, void* stream) {
    return rms_fwd_impl("rmsnorm_fwd", M, N, x, x_dtype, weight, weight_dtype, eps,
                        RWN_RMS_CAST_THEN_WEIGHT, y, rstd, stream);
}

RWN_API rwn_status rmsnorm_bwd(int64_t M, int64_t N, const void* x, const void* dy,
                               rwn_dtype x_dtype, const float* rstd, const void* weight,
                               rwn_dtype weight_dtype, float eps, void* dx, void* dweight,
                               void* workspace, size_t workspace_bytes, void* stream) {
    return rms_bwd_impl("rmsnorm_bwd", M, N, x, dy, x_dtype, rstd, weight, weight_dtype, eps,
                        RWN_RMS_CAST_THEN_WEIGHT, dx, dweight, workspace, workspace_bytes, stream);
}

RWN_API rwn_status rmsnorm_fwd_form(int64_t M, int64_t N, const void* x, rwn_dtype x_dtype,
                                    const void* weight, rwn_dtype weight_dtype, float eps,
                                    rwn_rms_form form, void* y, float* rstd, void* stream) {
    return rms_fwd_impl("rmsnorm_fwd_form", M, N, x, x_dtype, weight, weight_dtype, eps, (int)form,
                        y, rstd, stream);
}

RWN_API rwn_status rmsnorm_bwd_form(int64_t M, int64_t N, const void* x, const void* dy,
                                    rwn_dtype x_dtype, const float* rstd, const void* weight,
                                    rwn_dtype weight_dtype, float eps, rwn_rms_form form, void* dx,
                                    void* dweight, void* workspace, size_t workspace_bytes,
                                    void* stream) {
    return rms_bwd_impl("rmsnorm_bwd_form", M, N, x, dy, x_dtype, rstd, weight, weight_dtype, eps,
                        (int)form, dx, dweight, workspace, workspace_bytes, stream);
}

RWN_API rwn_status rmsnorm_bwd_workspace_size(int64_t M, int64_t N, rwn_dtype x_dtype, size_t* bytes) {
    return workspace_size(LAYER_RMS, M, N, x_dtype, bytes);
}

// ======================================================================= strided operands

RWN_API rwn_status dyt_fwd_strided(int nlead, const int64_t* lead, int64_t N, const void* x,
                                   const int64_t* x_strides, rwn_dtype x_dtype, const void* alpha,
                                   const void* gamma, int64_t gamma_stride, const void* beta,
                                   int64_t beta_stride, rwn_dtype param_dtype, void* y,
                                   const int64_t* y_strides, void* stream) {
    const char* fn = "dyt_fwd_strided";
    const StridedOperand ops[2] = {{x, x_strides, "x", OP_X, false}, {y, y_strides, "y", OP_OUT, true}};
    int64_t M = 0;
    Strided sr;
    rwn_status st = strided_rows(fn, nlead, lead, N, x_dtype, param_dtype, ops, 2, gamma_stride, beta_stride, &M, &sr);
    if (st != RWN_OK) return st;
    return dyt_fwd_impl(fn, M, N, x, x_dtype, alpha, gamma, beta, param_dtype, y, stream, &sr);
}

RWN_API rwn_status dyt_bwd_strided(int nlead, const int64_t* lead, int64_t N, const void* x,
                                   const int64_t* x_strides, const void* dy, const int64_t* dy_strides,
                                   rwn_dtype x_dtype, const void* alpha, const void* gamma,
                                   int64_t gamma_stride, rwn_dtype param_dtype, void* dx,
                                   const int64_t* dx_strides, void* dalpha, void* dgamma, void* dbeta,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "dyt_bwd_strided";
    const StridedOperand ops[3] = {{x, x_strides, "x", OP_X, false}, {dy, dy_strides, "dy", OP_DY, false},
                                   {dx, dx_strides, "dx", OP_OUT, true}};
    int64_t M = 0;
    Strided sr;
    rwn_status st = strided_rows(fn, nlead, lead, N, x_dtype, param_dtype, ops, 3, gamma_stride, 1, &M, &sr);
    if (st != RWN_OK) return st;
    return dyt_bwd_impl(fn, M, N, x, dy, x_dtype, alpha, gamma, param_dtype, dx, dalpha, dgamma, dbeta, workspace,
                        workspace_bytes, stream, &sr);
}

RWN_API rwn_status layernorm_fwd_strided(int nlead, const int64_t* lead, int64_t N, const void* x,
                                         const int64_t* x_strides, rwn_dtype x_dtype, const void* gamma,
                                         int64_t gamma_stride, const void* beta, int64_t beta_stride,
                                         rwn_dtype param_dtype, float eps, void* y, const int64_t* y_strides,
                                         float* mean, float* rstd, void* stream) {
    const char* fn = "layernorm_fwd_strided";
    const StridedOperand ops[2] = {{x, x_strides, "x", OP_X, false}, {y, y_strides, "y", OP_OUT, true}};
    int64_t M = 0;
    Strided sr;
    rwn_status st = strided_rows(fn, nlead, lead, N, x_dtype, param_dtype, ops, 2, gamma_stride, beta_stride, &M, &sr);
    if (st != RWN_OK) return st;
    return ln_fwd_impl(fn, M, N, x, x_dtype, gamma, beta, param_dtype, eps, y, mean, rstd, stream, &sr);
}

RWN_API rwn_status layernorm_bwd_strided(int nlead, const int64_t* lead, int64_t N, const void* x,
                                         const int64_t* x_strides, const void* dy, const int64_t* dy_strides,
                                         rwn_dtype x_dtype, const float* mean, const float* rstd,
                                         const void* gamma, int64_t gamma_stride, rwn_dtype param_dtype,
                                         float eps, void* dx, const int64_t* dx_strides, void* dgamma,
                                         void* dbeta, void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "layernorm_bwd_strided";
    const StridedOperand ops[3] = {{x, x_strides, "x", OP_X, false}, {dy, dy_strides, "dy", OP_DY, false},
                                   {dx, dx_strides, "dx", OP_OUT, true}};
    int64_t M = 0;
    Strided sr;
    rwn_status st = strided_rows(fn, nlead, lead, N, x_dtype, param_dtype, ops, 3, gamma_stride, 1, &M, &sr);
    if (st != RWN_OK) return st;
    return ln_bwd_impl(fn, M, N, x, dy, x_dtype, mean, rstd, gamma, param_dtype, eps, dx, dgamma, dbeta, workspace,
                       workspace_bytes, false, stream, &sr);
}

RWN_API rwn_status rmsnorm_fwd_strided(int nlead, const int64_t* lead, int64_t N, const void* x,
                                       const int64_t* x_strides, rwn_dtype x_dtype, const void* weight,
                                       int64_t weight_stride, rwn_dtype weight_dtype, float eps,
                                       rwn_rms_form form, void* y, const int64_t* y_strides, float* rstd,
                                       void* stream) {
    const char* fn = "rmsnorm_fwd_strided";
    const StridedOperand ops[2] = {{x, x_strides, "x", OP_X, false}, {y, y_strides, "y", OP_OUT, true}};
    int64_t M = 0;
    Strided sr;
    rwn_status st = strided_rows(fn, nlead, lead, N, x_dtype, weight_dtype, ops, 2, weight_stride, 1, &M, &sr);
    if (st != RWN_OK) return st;
    return rms_fwd_impl(fn, M, N, x, x_dtype, weight, weight_dtype, eps, (int)form, y, rstd, stream, &sr);
}

RWN_API rwn_status rmsnorm_bwd_strided(int nlead, const int64_t* lead, int64_t N, const void* x,
                                       const int64_t* x_strides, const void* dy, const int64_t* dy_strides,
                                       rwn_dtype x_dtype, const float* rstd, const void* weight,
                                       int64_t weight_stride, rwn_dtype weight_dtype, float eps,
                                       rwn_rms_form form, void* dx, const int64_t* dx_strides, void* dweight,
                                       void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "rmsnorm_bwd_strided";
    const StridedOperand ops[3] = {{x, x_strides, "x", OP_X, false}, {dy, dy_strides, "dy", OP_DY, false},
                                   {dx, dx_strides, "dx", OP_OUT, true}};
    int64_t M = 0;
    Strided sr;
    rwn_status st = strided_rows(fn, nlead, lead, N, x_dtype, weight_dtype, ops, 3, weight_stride, 1, &M, &sr);
    if (st != RWN_OK) return st;
    return rms_bwd_impl(fn, M, N, x, dy, x_dtype, rstd, weight, weight_dtype, eps, (int)form, dx, dweight, workspace,
                        workspace_bytes, stream, &sr);
}

// ================================================================================== support

RWN_API const char* rwn_last_error(void) { return g_err; }

RWN_API const char* rwn_version(void) { return "rwnorm 0.1.0 (gfx950)"; }

RWN_API rwn_status rwn_trace_begin(int capacity) {
    Trace& t = g_trace;
    if (capacity < 1 || capacity > (1 << 20))
        return fail(RWN_ERR_INVALID_ARG, "rwn_trace_begin: capacity must be in [1, 2^20]");
    if (t.on) return fail(RWN_ERR_INVALID_ARG, "rwn_trace_begin: a trace is already running");
    t.ev.assign((size_t)capacity, TraceEntry{0, nullptr, nullptr});
    for (int i = 0; i < capacity; ++i) {
        hipError_t e = hipEventCreate(&t.ev[i].a);
        if (e == hipSuccess) e = hipEventCreate(&t.ev[i].b);
        if (e != hipSuccess) {
            for (int j = 0; j <= i; ++j) {
                if (t.ev[j].a) (void)hipEventDestroy(t.ev[j].a);
                if (t.ev[j].b) (void)hipEventDestroy(t.ev[j].b);
            }
            t.ev.clear();
            return hip_fail(e, "rwn_trace_begin: hipEventCreate");
        }
    }
    t.cap = capacity;
    t.used = 0;
    t.on = true;
    return ok();
}

RWN_API int rwn_trace_end(float* ms, int* tags, int capacity) {
    Trace& t = g_trace;
    if (!t.on) {
        fail(RWN_ERR_INVALID_ARG, "rwn_trace_end: no trace is running");
        return -1;
    }
    int n = 0;
    int rc = 0;
    for (int i = 0; i < t.used; ++i) {
        if (n >= capacity) break;
        hipError_t e = hipEventSynchronize(t.ev[i].b);
        float v = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&v, t.ev[i].a, t.ev[i].b);
        if (e != hipSuccess) {
            hip_fail(e, "rwn_trace_end");
            rc = -1;
            break;
        }
        if (ms) ms[n] = v;
        if (tags) tags[n] = t.ev[i].tag;
        ++n;
    }
    for (auto& e : t.ev) {
        (void)hipEventDestroy(e.a);
        (void)hipEventDestroy(e.b);
    }
    t.ev.clear();
    t.on = false;
    t.cap = t.used = 0;
    if (rc < 0) return -1;
    ok();
    return n;
}

RWN_API rwn_status rwn_stream_probe(const void* src, const void* src2, void* dst, size_t bytes, int unroll,
                                    int nontemporal, int wg_per_cu, void* stream) {
    const char* fn = "rwn_stream_probe";
    if (!src || !dst) return fail(RWN_ERR_INVALID_ARG, "%s: NULL buffer", fn);
    if (((uintptr_t)src | (uintptr_t)src2 | (uintptr_t)dst | bytes) % 16)
        return fail(RWN_ERR_INVALID_ARG, "%s: buffers and size must be 16-byte multiples", fn);
    if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8)
        return fail(RWN_ERR_INVALID_ARG, "%s: unroll must be 1, 2, 4 or 8", fn);
    if (wg_per_cu < 1 || wg_per_cu > 32) return fail(RWN_ERR_INVALID_ARG, "%s: wg_per_cu must be in [1, 32]", fn);
    if (bytes == 0) return ok();
    int cus = 0;
    rwn_status st = device_cus(&cus);
    if (st != RWN_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = traced(RWN_K_COPY, s, [&] {
        return launch_stream_probe(src, src2, dst, bytes, unroll, nontemporal != 0, wg_per_cu, cus, s);
    });
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

RWN_API rwn_status rwn_plan(int layer, int backward, int64_t M, int64_t N, rwn_dtype x_dtype,
                            int param_dtype, int misalign_bytes, int cus, int layout, int64_t* out) {
    const char* fn = "rwn_plan";
    if (!out) return fail(RWN_ERR_INVALID_ARG, "%s: out is NULL", fn);
    if (layer < 0 || layer > 2) return fail(RWN_ERR_INVALID_ARG, "%s: layer must be 0, 1 or 2", fn);
    rwn_status st = check_shape_dtypes(fn, M, N, x_dtype, RWN_F32);
    if (st != RWN_OK) return st;
    const int esz = x_dtype == RWN_F32 ? 4 : 2;
    if (misalign_bytes < 0 || misalign_bytes >= 16 || misalign_bytes % esz)
        return fail(RWN_ERR_INVALID_ARG, "%s: misalign_bytes must be a multiple of the element size below 16", fn);
    if (cus < 0) return fail(RWN_ERR_INVALID_ARG, "%s: cus must be >= 0", fn);
    if (layout < 0 || layout > 2) return fail(RWN_ERR_INVALID_ARG, "%s: layout must be 0, 1 or 2", fn);
    if (layout == 2 && misalign_bytes)
        return fail(RWN_ERR_INVALID_ARG, "%s: layout 2 takes misalign_bytes = 0", fn);
    if (param_dtype != -1 && param_dtype != RWN_F32 && param_dtype != RWN_BF16 && param_dtype != RWN_F16)
        return fail(RWN_ERR_INVALID_ARG, "%s: param_dtype must be -1, RWN_F32, RWN_BF16 or RWN_F16", fn);
    if (param_dtype != -1 && !dtype_pair_ok((int)x_dtype, param_dtype))
        return fail(RWN_ERR_UNSUPPORTED, "%s: x dtype %d with parameter dtype %d is not supported", fn,
                    (int)x_dtype, param_dtype);
    const bool device = cus == 0;
    if (device && (st = device_cus(&cus)) != RWN_OK) return st;
    Plan p;
    // As the entry points plan: a backward for every parameter dtype at once.
    const int pd = backward ? -1 : param_dtype;
    if (!make_plan(layer, backward != 0, M, N, (int)x_dtype, pd, misalign_bytes, cus, device, &p, layout))
        return fail(RWN_ERR_UNSUPPORTED, "%s: no launch plan for N = %lld", fn, (long long)N);
    out[0] = p.mode; out[1] = p.cpt; out[2] = p.rt; out[3] = p.tpr; out[4] = p.rpp;
    out[5] = p.block; out[6] = p.grid; out[7] = p.ntiles;
    out[8] = p.flat == 2 ? 12 / esz : p.mode == MODE_SCALAR ? 1 : 16 / esz;
    out[9] = p.strided ? 0 : p.kt;
    out[10] = p.strided;
    out[11] = p.ncb;
    out[12] = p.xcd_remap;
    out[13] = p.pf;
    out[14] = p.flat;
    out[15] = p.split;
    return ok();
}
