/*
 * rwnorm.h -- C ABI of librwnorm: forward and backward of three row-wise per-channel
 * normalization layers over a row-major [M, N] activation matrix on an AMD Instinct MI355X
 * (gfx950), with hand-written HIP kernels.
 *
 * Layers (each entry point cites the passage that defines it):
 *   DyT        y = gamma * tanh(alpha * x) + beta, scalar alpha
 *              (Liger-Kernel PR #1617 "fix(dyt): use a 1D grid and tile small-width rows", Summary)
 *   LayerNorm  y = (x - mean) * rstd * gamma + beta, biased variance, eps inside the square root
 *              (intel/torch-xpu-ops PR #1880 "Layernorm bwd OPT", description; torch.nn.LayerNorm)
 *   RMSNorm    y = weight * (x.float() * rsqrt(mean(x.float()^2) + eps)).to(x.dtype)
 *              (DeepSpeed PR #8645 / #8664, Summary and Semantics)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout     x, dy, y, dx are row-major contiguous [M, N] (row pitch N elements).  Any
 *            element-aligned address is accepted, but x, dy, y and dx of one call must share
 *            the same address modulo 16 bytes (fresh allocations always do).  Parameters are
 *            contiguous [N] vectors; alpha is a one-element device buffer; statistics are
 *            float32 [M].  The *_strided entry points take strided rows and parameters.
 * Dtypes     x, dy, y, dx use x_dtype.  The parameters (alpha, gamma, beta, weight) and their
 *            gradients use param_dtype.  Supported pairs (x_dtype, param_dtype): (F32, F32),
 *            (BF16, F32), (BF16, BF16), (F16, F32), (F16, F16).  Arithmetic is float32;
 *            outputs are rounded once (round to nearest even; float16 overflows to +-inf) to
 *            their dtype, except for the RMSNorm rounding points.
 * Ownership  Every pointer is device memory owned by the caller.  The library never allocates,
 *            frees or synchronizes on these calls; work is enqueued on `stream` (a hipStream_t,
 *            NULL = the default stream) and the call returns after launch.
 * Errors     Invalid arguments are reported before anything is launched or written, with a
 *            message available from rwn_last_error() (thread-local).  No C++ exception crosses
 *            this boundary.
 * Empty M    M == 0 is valid: a forward writes nothing; a backward writes zeros to every
 *            requested parameter gradient (the sum over no rows).
 * Backward   Parameter gradients are column sums over all M rows, computed by a two-stage,
 *            atomic-free reduction: per-workgroup float32 partial rows in the caller's workspace,
 *            then a fixed-order float64 pass over them.  Results are bitwise reproducible run
 *            to run for the same inputs, device and library build.  A NULL gradient pointer
 *            skips writing that gradient; when every gradient pointer of a call is NULL the
 *            backward computes dx only (no column partials, no second pass) and the workspace
 *            may be NULL.
 * Gradients  First-order only; eps is a constant.
 * Width      1 <= N <= 16384.  A row is cut into 16-byte chunks (4 float32 / 8 bfloat16 or
 *            float16 elements) spread over at most 1024 threads.  A wide row that is not a whole
 *            number of aligned chunks (N not a multiple of the chunk, or operands not 16-byte
 *            aligned) is cut into its aligned chunks plus up to 2 * chunk - 2 single head and
 *            tail elements; float32 LayerNorm/RMSNorm rows of that kind wider than 8192 instead
 *            straddle one more chunk, so those calls take N <= 16381 and otherwise return
 *            RWN_ERR_UNSUPPORTED.  DyT splits wide rows into column blocks and takes every N up
 *            to 16384.  LayerNorm rows of 12 * 2^k bytes (float32 N = 3, 6, ..., 192; 16-bit
 *            N = 6, 12, ..., 384) on 4-byte aligned operands move in 12-byte chunks instead, and
 *            so do such DyT rows in the backward (and in the forward where they are not whole
 *            16-byte chunks).
 */
#ifndef RWNORM_H
#define RWNORM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { RWN_F32 = 0, RWN_BF16 = 1, RWN_F16 = 2 } rwn_dtype;

typedef enum {
    RWN_OK = 0,
    RWN_ERR_INVALID_ARG = 1,  /* negative M, N < 1, NULL required pointer, bad eps, bad dtype code */
    RWN_ERR_UNSUPPORTED = 2,  /* valid but unsupported: dtype pair, mismatched 16-byte alignment */
    RWN_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than the *_workspace_size query */
    RWN_ERR_LAUNCH = 4,       /* a HIP launch or device query failed (message names the HIP error) */
} rwn_status;

/* ---------------------------------------------------------------------------------- DyT */

/* Forward (Liger-Kernel PR #1617, Summary): y_ij = gamma_j * tanh(alpha * x_ij) + beta_j.
 * alpha: device [1]; gamma, beta: device [N]; y: device [M, N] in x_dtype.  With alpha = +inf
 * an element x = 0 gives tanh(inf * 0) = NaN, as in exact arithmetic. */
rwn_status dyt_fwd(int64_t M, int64_t N, const void* x, rwn_dtype x_dtype, const void* alpha,
                   const void* gamma, const void* beta, rwn_dtype param_dtype, void* y,
                   void* stream);

/* Backward (same passage): with t = tanh(alpha x), s = sech^2(alpha x):
 *   dx = dy * gamma * alpha * s, where alpha * s is taken as 0 when s == 0 (so alpha = +inf
 *        gives dx = 0 instead of inf * 0),
 *   dgamma_j = sum_i dy*t,  dbeta_j = sum_i dy,  dalpha = sum_ij dy*gamma*x*s.
 * Rows beyond M inside a tile are masked after the arithmetic, so they cannot inject NaN.
 * dx: [M, N] x_dtype.  dalpha [1], dgamma [N], dbeta [N] in param_dtype (each may be NULL).
 * workspace: device buffer of at least dyt_bwd_workspace_size() bytes, any content. */
rwn_status dyt_bwd(int64_t M, int64_t N, const void* x, const void* dy, rwn_dtype x_dtype,
                   const void* alpha, const void* gamma, rwn_dtype param_dtype, void* dx,
                   void* dalpha, void* dgamma, void* dbeta, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Workspace bytes dyt_bwd needs for (M, N, x_dtype) on the current HIP device. */
rwn_status dyt_bwd_workspace_size(int64_t M, int64_t N, rwn_dtype x_dtype, size_t* bytes);

/* ---------------------------------------------------------------------------- LayerNorm */

/* Forward (intel/torch-xpu-ops PR #1880, description; torch.nn.LayerNorm semantics):
 *   mean = sum_j x / N,  var = sum_j (x - mean)^2 / N,  rstd = 1 / sqrt(var + eps),
 *   y = (x - mean) * rstd * gamma + beta.
 * eps: finite, >= 0, used as the float32 value given.  mean, rstd: device float32 [M], each
 * may be NULL (not written). */
rwn_status layernorm_fwd(int64_t M, int64_t N, const void* x, rwn_dtype x_dtype,
                         const void* gamma, const void* beta, rwn_dtype param_dtype, float eps,
                         void* y, float* mean, float* rstd, void* stream);

/* Backward (same passage: the dgamma/dbeta column reduction that dominates when M >> N).
 * With xhat = (x - mean) * rstd, g = dy * gamma, c1 = mean_j g, c2 = mean_j g * xhat:
 *   dx = rstd * (g - c1 - xhat * c2),  dgamma_j = sum_i dy * xhat,  dbeta_j = sum_i dy.
 * mean/rstd: the forward's statistics; pass both NULL to recompute them from x with eps.
 * dgamma, dbeta: [N] param_dtype, each may be NULL. */
rwn_status layernorm_bwd(int64_t M, int64_t N, const void* x, const void* dy, rwn_dtype x_dtype,
                         const float* mean, const float* rstd, const void* gamma,
                         rwn_dtype param_dtype, float eps, void* dx, void* dgamma, void* dbeta,
                         void* workspace, size_t workspace_bytes, void* stream);

rwn_status layernorm_bwd_workspace_size(int64_t M, int64_t N, rwn_dtype x_dtype, size_t* bytes);

/* layernorm_bwd without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving or training loops, harnesses that forbid
 * hipMalloc).  The partial rows go to a static device array of 32 MiB that the library holds on
 * each device it runs on until the process ends; nothing is allocated or freed by the call.
 * Arguments, results and errors are layernorm_bwd's, and so are the kernels: results are bitwise
 * those of layernorm_bwd with a workspace.  A shape whose partial rows need more than 32 MiB
 * (layernorm_bwd_workspace_size reports the need) returns RWN_ERR_UNSUPPORTED before anything
 * is launched.  Every call on a device shares that device's array, and nothing in it needs to
 * start at zero (each call writes every partial it reads), but calls that overlap in time on
 * one device -- concurrent streams, or host threads -- race on it: serialize them. */
rwn_status layernorm_bwd_noalloc(int64_t M, int64_t N, const void* x, const void* dy,
                                 rwn_dtype x_dtype, const float* mean, const float* rstd,
                                 const void* gamma, rwn_dtype param_dtype, float eps, void* dx,
                                 void* dgamma, void* dbeta, void* stream);

/* ------------------------------------------------------------------------------ RMSNorm */

/* Forward (DeepSpeed PR #8645, Summary and Semantics): float32 statistics
 *   rstd = 1 / sqrt(sum_j x^2 / N + eps),  n = round_x_dtype(x * rstd),
 *   y = round_x_dtype(float32(weight * n)).
 * y keeps x_dtype also for a float32 weight.  rstd: device float32 [M] or NULL. */
rwn_status rmsnorm_fwd(int64_t M, int64_t N, const void* x, rwn_dtype x_dtype, const void* weight,
                       rwn_dtype weight_dtype, float eps, void* y, float* rstd, void* stream);

/* Backward (same passage): g = round_x_dtype(float32(dy * weight)), h = x * rstd (unrounded),
 *   c = mean_j g * h,  dx = rstd * (g - h * c),
 *   dweight_j = sum_i round_weight_dtype(float32(dy * n)), n = round_x_dtype(h).
 * rstd: the forward's statistic, or NULL to recompute it from x with eps.  dweight may be
 * NULL. */
rwn_status rmsnorm_bwd(int64_t M, int64_t N, const void* x, const void* dy, rwn_dtype x_dtype,
                       const float* rstd, const void* weight, rwn_dtype weight_dtype, float eps,
                       void* dx, void* dweight, void* workspace, size_t workspace_bytes,
                       void* stream);

rwn_status rmsnorm_bwd_workspace_size(int64_t M, int64_t N, rwn_dtype x_dtype, size_t* bytes);

/* RMSNorm forms.  The same passage (DeepSpeed PR #8645, "Which modules are replaced" and "Not
 * covered") names two forms besides the Llama one whose math differs only in where the weight
 * meets the rounding: classes that multiply by the weight before the cast to x's dtype, and
 * the Gemma family's (1 + weight).  Both multiply in float32 and round once:
 *   RWN_RMS_CAST_THEN_WEIGHT  y = weight * (x * rstd).to(x.dtype)        (rmsnorm_fwd above)
 *   RWN_RMS_WEIGHT_THEN_CAST  y = (weight * (x * rstd)).to(x.dtype)
 *   RWN_RMS_ONE_PLUS_WEIGHT   y = ((1 + weight) * (x * rstd)).to(x.dtype), 1 + weight in float32
 * Backward of the two float32 forms, with s = weight or (1 + weight) and h = x * rstd:
 *   g = dy * s (float32, not rounded), c = mean_j g * h, dx = rstd * (g - h * c),
 *   dweight_j = sum_i dy * h in float32, rounded once to the weight's dtype. */
typedef enum {
    RWN_RMS_CAST_THEN_WEIGHT = 0,
    RWN_RMS_WEIGHT_THEN_CAST = 1,
    RWN_RMS_ONE_PLUS_WEIGHT = 2
} rwn_rms_form;

/* rmsnorm_fwd / rmsnorm_bwd for any form; the other arguments and rules are theirs.  An unknown
 * form returns RWN_ERR_INVALID_ARG. */
rwn_status rmsnorm_fwd_form(int64_t M, int64_t N, const void* x, rwn_dtype x_dtype,
                            const void* weight, rwn_dtype weight_dtype, float eps, rwn_rms_form form,
                            void* y, float* rstd, void* stream);
rwn_status rmsnorm_bwd_form(int64_t M, int64_t N, const void* x, const void* dy, rwn_dtype x_dtype,
                            const float* rstd, const void* weight, rwn_dtype weight_dtype, float eps,
                            rwn_rms_form form, void* dx, void* dweight, void* workspace,
                            size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------- strided operands */

/* The six entry points above with strided row operands and parameter vectors, so that views
 * (a slice of a wider matrix, a head-major [B, S, H, D] tensor whose rows are D-wide, a
 * gradient in another layout than x) run without copies.  The DeepSpeed RMSNorm pages
 * (PR #8645, "Where the kernels run" and "Correctness evidence"; PR #8664, Tests) test
 * head-major non-contiguous inputs, transposed incoming gradients and non-contiguous weights.
 *
 * Rows     The M rows are the index space of nlead (1..3) leading dimensions of sizes
 *          lead[0..nlead-1] (host array; M = their product, at most 2^31 - 1), the last one
 *          fastest.  Each row operand has its own host array of nlead element strides:
 *          row (i_0, ..., i_{nlead-1}) starts at sum_k i_k * strides[k] elements past the
 *          operand's base, and its N elements are contiguous.  Statistics (mean, rstd) are
 *          contiguous float32 [M] in that row order.  Strides must be >= 0; an output (y, dx)
 *          whose rows would share an element returns RWN_ERR_INVALID_ARG; an operand spanning
 *          more than 2^31 - 32 bytes returns RWN_ERR_UNSUPPORTED.
 * Params   gamma_stride / beta_stride / weight_stride: element strides (>= 0) of the parameter
 *          vectors.  alpha is one element.  Parameter gradients are written contiguous.
 * Kernels  Operands that are dense [M, N] after all, at one address modulo 16, with contiguous
 *          parameters, take exactly the dense entry points' path.  Otherwise, when every row of
 *          every operand starts at one offset modulo 16 bytes (bases at one address modulo 16,
 *          strides multiples of 16 bytes), rows move in 16-byte chunks as in the dense path
 *          (LayerNorm / RMSNorm rows not a whole number of aligned chunks take N <= 16384 - V + 1,
 *          V the elements of a chunk); else element by element, which takes N <= 2048 (16-bit)
 *          or 4096 (float32) for LayerNorm / RMSNorm and any N for DyT.  Either way results follow the same
 *          arithmetic as the dense entry points; the backward's workspace is sized by the
 *          *_bwd_workspace_size queries, which cover strided plans.
 * All other arguments, rules and errors are those of the dense entry point of the same name. */
rwn_status dyt_fwd_strided(int nlead, const int64_t* lead, int64_t N, const void* x,
                           const int64_t* x_strides, rwn_dtype x_dtype, const void* alpha,
                           const void* gamma, int64_t gamma_stride, const void* beta,
                           int64_t beta_stride, rwn_dtype param_dtype, void* y,
                           const int64_t* y_strides, void* stream);
rwn_status dyt_bwd_strided(int nlead, const int64_t* lead, int64_t N, const void* x,
                           const int64_t* x_strides, const void* dy, const int64_t* dy_strides,
                           rwn_dtype x_dtype, const void* alpha, const void* gamma,
                           int64_t gamma_stride, rwn_dtype param_dtype, void* dx,
                           const int64_t* dx_strides, void* dalpha, void* dgamma, void* dbeta,
                           void* workspace, size_t workspace_bytes, void* stream);
rwn_status layernorm_fwd_strided(int nlead, const int64_t* lead, int64_t N, const void* x,
                                 const int64_t* x_strides, rwn_dtype x_dtype, const void* gamma,
                                 int64_t gamma_stride, const void* beta, int64_t beta_stride,
                                 rwn_dtype param_dtype, float eps, void* y, const int64_t* y_strides,
                                 float* mean, float* rstd, void* stream);
rwn_status layernorm_bwd_strided(int nlead, const int64_t* lead, int64_t N, const void* x,
                                 const int64_t* x_strides, const void* dy, const int64_t* dy_strides,
                                 rwn_dtype x_dtype, const float* mean, const float* rstd,
                                 const void* gamma, int64_t gamma_stride, rwn_dtype param_dtype,
                                 float eps, void* dx, const int64_t* dx_strides, void* dgamma,
                                 void* dbeta, void* workspace, size_t workspace_bytes, void* stream);
rwn_status rmsnorm_fwd_strided(int nlead, const int64_t* lead, int64_t N, const void* x,
                               const int64_t* x_strides, rwn_dtype x_dtype, const void* weight,
                               int64_t weight_stride, rwn_dtype weight_dtype, float eps,
                               rwn_rms_form form, void* y, const int64_t* y_strides, float* rstd,
                               void* stream);
rwn_status rmsnorm_bwd_strided(int nlead, const int64_t* lead, int64_t N, const void* x,
                               const int64_t* x_strides, const void* dy, const int64_t* dy_strides,
                               rwn_dtype x_dtype, const float* rstd, const void* weight,
                               int64_t weight_stride, rwn_dtype weight_dtype, float eps,
                               rwn_rms_form form, void* dx, const int64_t* dx_strides,
                               void* dweight, void* workspace, size_t workspace_bytes,
                               void* stream);

/* ------------------------------------------------------------------------------ support */

/* Message of the last failed call on this thread ("" after a successful call). */
const char* rwn_last_error(void);

/* Library version string. */
const char* rwn_version(void);

/* Kernel-duration trace, a measurement aid.  After rwn_trace_begin(capacity) every kernel the
 * entry points launch on this thread is bracketed by a pair of HIP events on its stream (up
 * to `capacity` kernels; the library creates the events here).  rwn_trace_end() waits for
 * the recorded events, writes up to `capacity` durations in milliseconds and kernel tags
 * (see rwn_kernel_tag), releases the events and returns the number of entries, or -1 on a HIP
 * error.  Tracing is off until rwn_trace_begin is called. */
typedef enum {
    RWN_K_DYT_FWD = 1, RWN_K_DYT_BWD = 2, RWN_K_LN_FWD = 3, RWN_K_LN_BWD = 4,
    RWN_K_RMS_FWD = 5, RWN_K_RMS_BWD = 6, RWN_K_COLREDUCE = 7, RWN_K_COPY = 8
} rwn_kernel_tag;
rwn_status rwn_trace_begin(int capacity);
int rwn_trace_end(float* ms, int* tags, int capacity);

/* Streaming probe, a measurement aid: dst = src (src2 NULL) or dst = src XOR src2 over `bytes`
 * (all buffers 16-byte aligned, bytes a multiple of 16), enqueued on `stream`.  A persistent
 * grid of wg_per_cu (1..32) 256-thread workgroups per CU; every lane keeps `unroll` (1, 2, 4 or 8)
 * 16-byte loads per input in flight before it stores; nontemporal != 0 puts the streaming hint
 * on every access.  It bounds the rate of a kernel that reads one or two tensors of that size
 * and writes one. */
rwn_status rwn_stream_probe(const void* src, const void* src2, void* dst, size_t bytes, int unroll,
                            int nontemporal, int wg_per_cu, void* stream);

/* Launch plan the library chooses for an entry point (introspection for tests and tuning).
 * layer: 0 = DyT, 1 = LayerNorm, 2 = RMSNorm; backward: 0/1.  Writes 16 integers to out:
 * {mode (0 aligned vectors, 1 shifted vectors, 2 scalar), chunks per thread, rows per thread,
 *  threads per row, row slots per workgroup, workgroup size, workgroups, row tiles,
 *  elements per chunk, row tiles per workgroup (0 when strided), strided (1: workgroup w
 *  visits tiles w, w + workgroups / column blocks, ...), column blocks per row, XCD remap
 *  (1: workgroup numbers renumbered so consecutive ones share an XCD), prefetch (1: the next
 *  tile's loads are issued before the current tile is processed), flat (1: narrow aligned
 *  LayerNorm rows through plain loads on clamped row indices instead of per-tile buffer
 *  descriptors; 2: the same for LayerNorm and DyT rows of 12 * 2^k bytes, 2^k <= 64, on 4-byte
 *  aligned operands, in 12-byte chunks, so elements per chunk is 12 / element size), split (1: a wide row not aligned to 16-byte chunks is cut into whole aligned
 *  chunks plus scalar head and tail elements)}.  param_dtype: the parameter
 * dtype of a forward (-1: any; a backward is always planned for every parameter dtype, as its
 * workspace is).  misalign_bytes is the common address of x/y/dy/dx modulo 16.  cus: 0 plans
 * for the current device exactly as the entry points do (its CU count, and the workgroups of
 * the chosen kernel that fit on one CU at once); any other value plans for that many CUs from
 * launch bounds alone, without touching a device.  layout: 0 for dense operands, 1 for strided
 * operands whose rows all start misalign_bytes past a 16-byte boundary, 2 for strided operands
 * of mixed alignment (the *_strided entry points choose it). */
rwn_status rwn_plan(int layer, int backward, int64_t M, int64_t N, rwn_dtype x_dtype,
                    int param_dtype, int misalign_bytes, int cus, int layout, int64_t* out);

#ifdef __cplusplus
}
#endif

#endif /* RWNORM_H */
