/*
 * oracle.c -- plain, slow, fp64 CPU reference for three row-wise normalization layers over a
 * row-major [M, N] matrix: DyT, LayerNorm and Llama-style RMSNorm, forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this library.  It shares no code with the GPU library: it has its own element
 * loads, its own bfloat16 rounding and its own loops.
 *
 * What it computes is the plain definition of each layer, written out in fp64:
 *   - every input element is converted exactly to double;
 *   - all arithmetic and every sum is done in double, with libm tanh/cosh/sqrt;
 *   - rounding to a storage dtype happens only at the rounding points the method names
 *     (RMSNorm, see below); the final cast of each output to its dtype is NOT applied:
 *     outputs are returned as the exact double value before that cast, together with a
 *     per-element "scale" (the sum of the magnitudes of the terms that form the element),
 *     which the tests use to bound the fp32 rounding error of the GPU path.
 *
 * Sources (cited by page title and section):
 *   [DyT]  Liger-Kernel PR #1617 "fix(dyt): use a 1D grid and tile small-width rows", Summary:
 *          names tanh, alpha, dalpha/dbeta/dgamma, the tanh(inf*0) NaN of padded rows, and the
 *          rule that parameter gradients take their parameters' dtypes while y keeps x.dtype.
 *          The layer is y = gamma * tanh(alpha * x) + beta with a scalar alpha.
 *   [LN]   intel/torch-xpu-ops PR #1880 "Layernorm bwd OPT", description: ATen layer-norm
 *          backward whose gamma/beta gradients are column sums over M rows.  Read as
 *          torch.nn.LayerNorm: biased variance, eps inside the square root, affine gamma, beta.
 *   [RMS]  DeepSpeed PR #8645 (embedded in PR #8664), sections "Summary" and "Semantics": the
 *          Llama expression weight * (x.float() * rsqrt(mean(x.float()**2) + eps)).to(x.dtype).
 *          Read here as: statistics in float32; the normalized row is stored in x's dtype before
 *          the weight touches it; in the backward the upstream gradient times the weight is
 *          stored in x's dtype before it is used, and each weight-gradient term (upstream
 *          gradient times normalized value) is stored in the weight gradient's dtype before the
 *          float32 column sum.
 *   [W1]   DeepSpeed PR #8664, commit messages and "Numerics": at width one the pre-gamma input
 *          derivative of RMSNorm is eps / (x^2 + eps)^(3/2).
 *
 * Dtype codes: 0 = float32, 1 = bfloat16 (stored as its 16 high bits of a float32),
 * 2 = float64 (no rounding at all; used by the finite-difference and library pins),
 * 3 = float16 (IEEE 754 binary16: 1 sign, 5 exponent, 10 fraction bits).  The float16 pair
 * follows the same reading as bfloat16 (the pages test bfloat16 and float16 alike): float32
 * arithmetic, float16 storage and rounding points.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORA_F32 = 0, ORA_BF16 = 1, ORA_F64 = 2, ORA_F16 = 3 };

/* Rows per block for column sums: each block sums its rows in row order, blocks are then
 * added in block order, so results do not depend on the OpenMP thread count. */
#define ORA_ROW_BLOCK 1024

/* ---------------------------------------------------------------- element access / rounding */

/* Exact value of a binary16 bit pattern: a zero exponent field holds subnormals f * 2^-24,
 * the all-ones field infinities and NaNs, the rest (1024 + f) * 2^(e - 25). */
static double f16_value(uint16_t h) {
    const int e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)f, -24);
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(1024 + f), e - 25);
    return (h & 0x8000) ? -v : v;
}

static double load_elem(const void* p, int dt, int64_t i) {
    if (dt == ORA_F64) return ((const double*)p)[i];
    if (dt == ORA_F32) return (double)((const float*)p)[i];
    if (dt == ORA_F16) return f16_value(((const uint16_t*)p)[i]);
    uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bfloat16 value, ties to even.  bfloat16 has float32's
 * exponent range and 8 significant bits; below 2^-126 its spacing is fixed at 2^-133
 * (subnormals).  Values at or beyond the overflow threshold become +-inf; NaN stays NaN. */
double oracle_round_bf16(double v) {
    if (!isfinite(v) || v == 0.0) return v;
    int e;
    frexp(v, &e);                 /* |v| in [2^(e-1), 2^e) */
    int q = e - 8;                /* spacing of 8-significant-bit numbers in that binade */
    if (q < -133) q = -133;
    double r = ldexp(nearbyint(ldexp(v, -q)), q);   /* nearbyint: ties to even (default mode) */
    const double bf16_max = ldexp(255.0, 120);      /* (2 - 2^-7) * 2^127 */
    if (fabs(r) > bf16_max) r = copysign(INFINITY, v);
    return r;
}

double oracle_round_f32(double v) { return (double)(float)v; }

/* Round a double to the nearest float16 value, ties to even.  float16 has 11 significant bits
 * and normal exponents down to -14, below which its spacing is fixed at 2^-24 (subnormals).
 * The largest finite value is 65504; anything that rounds beyond it becomes +-inf. */
double oracle_round_f16(double v) {
    if (!isfinite(v) || v == 0.0) return v;
    int e;
    frexp(v, &e);                 /* |v| in [2^(e-1), 2^e) */
    int q = e - 11;               /* spacing of 11-significant-bit numbers in that binade */
    if (q < -24) q = -24;
    double r = ldexp(nearbyint(ldexp(v, -q)), q);   /* nearbyint: ties to even (default mode) */
    if (fabs(r) > 65504.0) r = copysign(INFINITY, v);
    return r;
}

static double round_to(int dt, double v) {
    if (dt == ORA_F64) return v;
    if (dt == ORA_F16) return oracle_round_f16(v);
    return dt == ORA_F32 ? oracle_round_f32(v) : oracle_round_bf16(v);
}

/* Eager arithmetic on float32/bfloat16 tensors happens in float32; on float64 tensors in
 * float64.  round_arith(dt, v) rounds a product to the arithmetic dtype of storage dt. */
static double round_arith(int dt, double v) { return dt == ORA_F64 ? v : oracle_round_f32(v); }

/* Column sums of a per-element term over all M rows, in fixed row blocks.
 * term(ctx, i, out_row) writes the ncols terms of row i; the results go to sum[ncols]
 * and the sum of magnitudes to abs_sum[ncols] (either may be NULL). */
typedef void (*row_terms_fn)(const void* ctx, int64_t i, double* terms);

static int column_sums(const void* ctx, row_terms_fn term, int64_t M, int64_t ncols,
                       double* sum, double* abs_sum) {
    int64_t nblk = (M + ORA_ROW_BLOCK - 1) / ORA_ROW_BLOCK;
    double* part = (double*)calloc((size_t)(nblk > 0 ? nblk : 1) * (size_t)ncols * 2, sizeof(double));
    if (!part) return -1;
    int failed = 0;
#pragma omp parallel
    {
        double* terms = (double*)malloc((size_t)ncols * sizeof(double));
        if (!terms) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t b = 0; b < nblk; ++b) {
            if (!terms) continue;
            double* ps = part + (size_t)b * (size_t)ncols * 2;
            double* pa = ps + ncols;
            int64_t i1 = (b + 1) * ORA_ROW_BLOCK < M ? (b + 1) * ORA_ROW_BLOCK : M;
            for (int64_t i = b * ORA_ROW_BLOCK; i < i1; ++i) {
                term(ctx, i, terms);
                for (int64_t c = 0; c < ncols; ++c) {
                    ps[c] += terms[c];
                    pa[c] += fabs(terms[c]);
                }
            }
        }
        free(terms);
    }
    if (failed) { free(part); return -1; }
    for (int64_t c = 0; c < ncols; ++c) {
        double s = 0.0, a = 0.0;
        for (int64_t b = 0; b < nblk; ++b) {
            s += part[(size_t)b * (size_t)ncols * 2 + c];
            a += part[(size_t)b * (size_t)ncols * 2 + ncols + c];
        }
        if (sum) sum[c] = s;
        if (abs_sum) abs_sum[c] = a;
    }
    free(part);
    return 0;
}

/* ---------------------------------------------------------------------------------- DyT */

/* [DyT] Summary.  y_ij = gamma_j * tanh(alpha * x_ij) + beta_j.
 * y_scale_ij = |gamma_j * tanh(alpha x_ij)| + |beta_j|.  With alpha = +inf, tanh(+-inf) = +-1;
 * x_ij = 0 then gives tanh(inf * 0) = NaN, as the page says. */
int oracle_dyt_fwd(int64_t M, int64_t N, const void* x, int xdt, double alpha,
                   const void* gamma, const void* beta, int pdt, double* y, double* y_scale) {
    if (M < 0 || N < 1) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double g = load_elem(gamma, pdt, j), b = load_elem(beta, pdt, j);
            double t = tanh(alpha * load_elem(x, xdt, i * N + j));
            if (y) y[i * N + j] = g * t + b;
            if (y_scale) y_scale[i * N + j] = fabs(g * t) + fabs(b);
        }
    }
    return 0;
}

/* d tanh(z)/dz = sech^2(z) = 1 / cosh(z)^2 (cosh(+-inf) = inf gives exactly 0). */
static double sech2(double z) {
    double c = cosh(z);
    return 1.0 / (c * c);
}

/* alpha * sech^2(alpha x).  For alpha = +inf and x != 0 the product is inf * 0; its limit
 * as alpha grows is 0, which is what is returned (a no-op for every finite alpha, where
 * finite * 0 = 0 already). */
static double alpha_sech2(double alpha, double xv) {
    double s = sech2(alpha * xv);
    return s == 0.0 ? 0.0 : alpha * s;
}

typedef struct {
    int64_t N;
    const void *x, *dy, *gamma;
    int xdt, pdt;
    double alpha;
} dyt_ctx;

/* Column terms of row i: [dy*t (N) | dy (N) | dy*gamma*x*sech^2 summed over the row (1) |
 * the magnitudes of those dalpha terms summed over the row (1)].  dalpha is one sum over all
 * M * N products, so its magnitude sum adds |term| over every (i, j), not |row sum| per row. */
static void dyt_bwd_terms(const void* vctx, int64_t i, double* terms) {
    const dyt_ctx* c = (const dyt_ctx*)vctx;
    double da = 0.0, daa = 0.0;
    for (int64_t j = 0; j < c->N; ++j) {
        double xv = load_elem(c->x, c->xdt, i * c->N + j);
        double g = load_elem(c->dy, c->xdt, i * c->N + j);
        double z = c->alpha * xv;
        terms[j] = g * tanh(z);
        terms[c->N + j] = g;
        double s = sech2(z);
        double t = g * load_elem(c->gamma, c->pdt, j) * xv * s;
        da += t;
        daa += fabs(t);
    }
    terms[2 * c->N] = da;
    terms[2 * c->N + 1] = daa;
}

/* [DyT] Summary.  With t = tanh(alpha x) and s = sech^2(alpha x):
 *   dx_ij    = dy_ij * gamma_j * alpha * s_ij         (dx_scale = |dx|: a pure product)
 *   dgamma_j = sum_i dy_ij * t_ij
 *   dbeta_j  = sum_i dy_ij
 *   dalpha   = sum_ij dy_ij * gamma_j * x_ij * s_ij
 * *_scale = sums of the magnitudes of the same terms.  dx, dx_scale and any gradient
 * pointer may be NULL (not computed). */
int oracle_dyt_bwd(int64_t M, int64_t N, const void* x, const void* dy, int xdt, double alpha,
                   const void* gamma, int pdt, double* dx, double* dx_scale,
                   double* dgamma, double* dbeta, double* dalpha,
                   double* dgamma_scale, double* dbeta_scale, double* dalpha_scale) {
    if (M < 0 || N < 1) return -1;
    if (dx || dx_scale) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < M; ++i) {
            for (int64_t j = 0; j < N; ++j) {
                double v = load_elem(dy, xdt, i * N + j) * load_elem(gamma, pdt, j) *
                           alpha_sech2(alpha, load_elem(x, xdt, i * N + j));
                if (dx) dx[i * N + j] = v;
                if (dx_scale) dx_scale[i * N + j] = fabs(v);
            }
        }
    }
    if (dgamma || dbeta || dalpha || dgamma_scale || dbeta_scale || dalpha_scale) {
        dyt_ctx c = {N, x, dy, gamma, xdt, pdt, alpha};
        int64_t nc = 2 * N + 2;
        double* s = (double*)malloc((size_t)nc * sizeof(double));
        double* a = (double*)malloc((size_t)nc * sizeof(double));
        if (!s || !a || column_sums(&c, dyt_bwd_terms, M, nc, s, a) != 0) {
            free(s); free(a);
            return -2;
        }
        for (int64_t j = 0; j < N; ++j) {
            if (dgamma) dgamma[j] = s[j];
            if (dbeta) dbeta[j] = s[N + j];
            if (dgamma_scale) dgamma_scale[j] = a[j];
            if (dbeta_scale) dbeta_scale[j] = a[N + j];
        }
        if (dalpha) *dalpha = s[2 * N];
        if (dalpha_scale) *dalpha_scale = s[2 * N + 1];
        free(s); free(a);
    }
    return 0;
}

/* ---------------------------------------------------------------------------- LayerNorm */

/* Row statistics: mu = mean(x), var = mean((x - mu)^2) (biased), rstd = 1/sqrt(var + eps). */
static void ln_row_stats(const void* x, int xdt, int64_t i, int64_t N, double eps,
                         double* mu_out, double* rstd_out) {
    double s = 0.0;
    for (int64_t j = 0; j < N; ++j) s += load_elem(x, xdt, i * N + j);
    double mu = s / (double)N;
    double v = 0.0;
    for (int64_t j = 0; j < N; ++j) {
        double d = load_elem(x, xdt, i * N + j) - mu;
        v += d * d;
    }
    v /= (double)N;
    *mu_out = mu;
    *rstd_out = 1.0 / sqrt(v + eps);
}

/* Mean of |x| over row i: the magnitude sum of the terms of mu. */
static double row_abs_mean(const void* x, int xdt, int64_t i, int64_t N) {
    double s = 0.0;
    for (int64_t j = 0; j < N; ++j) s += fabs(load_elem(x, xdt, i * N + j));
    return s / (double)N;
}

/* [LN] (torch.nn.LayerNorm reading).  xhat = (x - mu) * rstd; y = xhat * gamma + beta.
 * y_scale sums the magnitudes of every term of y expanded through mu = sum_j x_j / N:
 * rstd * |gamma| * (|x| + sum_j |x_j| / N) + |beta|.  mean/rstd (may be NULL) receive mu and
 * rstd; mean_scale the magnitude sum of mu (sum_j |x_j| / N); rstd_scale bounds rstd's error
 * through that of var + eps: with V = sum_j (|x_j| + sum_k |x_k| / N)^2 / N, the magnitude sum
 * of the biased variance expanded through mu, rstd_scale = rstd * (V + eps) / (var + eps), twice
 * the first-order propagation (d rstd / rstd = -d(var + eps) / (2 (var + eps))).  Both may be
 * NULL. */
int oracle_layernorm_fwd(int64_t M, int64_t N, const void* x, int xdt, const void* gamma,
                         const void* beta, int pdt, double eps, double* y, double* y_scale,
                         double* mean, double* rstd, double* mean_scale, double* rstd_scale) {
    if (M < 0 || N < 1) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double mu, r;
        ln_row_stats(x, xdt, i, N, eps, &mu, &r);
        if (mean) mean[i] = mu;
        if (rstd) rstd[i] = r;
        const double am = row_abs_mean(x, xdt, i, N);
        if (mean_scale) mean_scale[i] = am;
        if (rstd_scale) {
            double vs = 0.0;
            for (int64_t j = 0; j < N; ++j) {
                double m = fabs(load_elem(x, xdt, i * N + j)) + am;
                vs += m * m;
            }
            vs /= (double)N;
            rstd_scale[i] = r * (vs + eps) * (r * r);   /* r^2 = 1 / (var + eps) */
        }
        for (int64_t j = 0; j < N; ++j) {
            double xv = load_elem(x, xdt, i * N + j);
            double xh = (xv - mu) * r;
            double g = load_elem(gamma, pdt, j), b = load_elem(beta, pdt, j);
            if (y) y[i * N + j] = xh * g + b;
            if (y_scale) y_scale[i * N + j] = r * fabs(g) * (fabs(xv) + am) + fabs(b);
        }
    }
    return 0;
}

typedef struct {
    int64_t N;
    const void *x, *dy;
    int xdt;
    double eps;
} ln_ctx;

/* Column terms of row i: [dy * xhat (N) | dy (N) | |dy| * m (N)], where
 * m = rstd * (|x| + mean_j |x_j|) is the magnitude of xhat's own terms (x and the mean). */
static void ln_bwd_terms(const void* vctx, int64_t i, double* terms) {
    const ln_ctx* c = (const ln_ctx*)vctx;
    double mu, r;
    ln_row_stats(c->x, c->xdt, i, c->N, c->eps, &mu, &r);
    const double am = row_abs_mean(c->x, c->xdt, i, c->N);
    for (int64_t j = 0; j < c->N; ++j) {
        double g = load_elem(c->dy, c->xdt, i * c->N + j);
        double xv = load_elem(c->x, c->xdt, i * c->N + j);
        terms[j] = g * (xv - mu) * r;
        terms[c->N + j] = g;
        terms[2 * c->N + j] = fabs(g) * r * (fabs(xv) + am);
    }
}

/* [LN] backward, statistics recomputed from x in double (the GPU's saved stats are not read).
 * With g = dy * gamma, c1 = mean_j(g), c2 = mean_j(g * xhat):
 *   dx       = rstd * (g - c1 - xhat * c2)
 *   dgamma_j = sum_i dy_ij * xhat_ij,  dbeta_j = sum_i dy_ij  (+ magnitude sums; dgamma's
 *   expands xhat into its terms like dx_scale: sum_i |dy_ij| * m_ij, m as below).
 * dx_scale sums the magnitudes of every term of dx expanded through the row means:
 * with m = rstd * (|x| + mean_j |x_j|) (the magnitude of xhat's terms),
 * rstd * (|g| + mean_j |g_j| + m * mean_j |g_j| m_j). */
int oracle_layernorm_bwd(int64_t M, int64_t N, const void* x, const void* dy, int xdt,
                         const void* gamma, int pdt, double eps, double* dx, double* dx_scale,
                         double* dgamma, double* dbeta, double* dgamma_scale, double* dbeta_scale) {
    if (M < 0 || N < 1) return -1;
    if (dx || dx_scale) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < M; ++i) {
            double mu, r;
            ln_row_stats(x, xdt, i, N, eps, &mu, &r);
            const double am = row_abs_mean(x, xdt, i, N);
            double c1 = 0.0, c2 = 0.0, a1 = 0.0, a2 = 0.0;
            for (int64_t j = 0; j < N; ++j) {
                double xv = load_elem(x, xdt, i * N + j);
                double g = load_elem(dy, xdt, i * N + j) * load_elem(gamma, pdt, j);
                double xh = (xv - mu) * r;
                c1 += g;
                c2 += g * xh;
                a1 += fabs(g);
                a2 += fabs(g) * r * (fabs(xv) + am);
            }
            c1 /= (double)N;
            c2 /= (double)N;
            a1 /= (double)N;
            a2 /= (double)N;
            for (int64_t j = 0; j < N; ++j) {
                double xv = load_elem(x, xdt, i * N + j);
                double g = load_elem(dy, xdt, i * N + j) * load_elem(gamma, pdt, j);
                double xh = (xv - mu) * r;
                if (dx) dx[i * N + j] = r * (g - c1 - xh * c2);
                if (dx_scale) dx_scale[i * N + j] = r * (fabs(g) + a1 + r * (fabs(xv) + am) * a2);
            }
        }
    }
    if (dgamma || dbeta || dgamma_scale || dbeta_scale) {
        ln_ctx c = {N, x, dy, xdt, eps};
        double* s = (double*)malloc((size_t)(3 * N) * sizeof(double));
        double* a = (double*)malloc((size_t)(3 * N) * sizeof(double));
        if (!s || !a || column_sums(&c, ln_bwd_terms, M, 3 * N, s, a) != 0) {
            free(s); free(a);
            return -2;
        }
        for (int64_t j = 0; j < N; ++j) {
            if (dgamma) dgamma[j] = s[j];
            if (dbeta) dbeta[j] = s[N + j];
            if (dgamma_scale) dgamma_scale[j] = a[2 * N + j];
            if (dbeta_scale) dbeta_scale[j] = a[N + j];
        }
        free(s); free(a);
    }
    return 0;
}

/* ------------------------------------------------------------------------------ RMSNorm */

/* rstd = 1 / sqrt(mean_j(x^2) + eps). */
static double rms_row_rstd(const void* x, int xdt, int64_t i, int64_t N, double eps) {
    double s = 0.0;
    for (int64_t j = 0; j < N; ++j) {
        double v = load_elem(x, xdt, i * N + j);
        s += v * v;
    }
    return 1.0 / sqrt(s / (double)N + eps);
}

/* The neighbour a float32 computation could also have rounded h to: when h lies within a
 * relative 2^-18 of the midpoint between two values of the input dtype, a float32 h (which
 * carries a few float32 roundings) can land on either side.  Returns the other neighbour, or
 * n itself when h is not that close to a midpoint. */
static double rounding_alternative(double h, double n, int dt) {
    if ((dt != ORA_BF16 && dt != ORA_F16) || !isfinite(h) || h == n) return n;
    double tol = ldexp(fabs(h), -18);
    double other = round_to(dt, 2.0 * h - n);   /* the neighbour on the other side of h */
    if (other == n) return n;
    double mid = 0.5 * (n + other);
    return fabs(h - mid) <= tol ? other : n;
}

/* [RMS] Summary / Semantics.  r = rstd; h = x * r (unrounded); n = round_xdt(h);
 * y = round_arith(w * n): eager forms the product in float32 (exact for bf16 * bf16).  The
 * final cast of y to x's dtype is left to the caller's tolerance.  y_scale = |y|.  y_alt
 * uses the other rounding of h (see rounding_alternative) and equals y where there is none.
 * rstd may be NULL. */
int oracle_rmsnorm_fwd(int64_t M, int64_t N, const void* x, int xdt, const void* w, int wdt,
                       double eps, double* y, double* y_scale, double* y_alt, double* rstd) {
    if (M < 0 || N < 1) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double r = rms_row_rstd(x, xdt, i, N, eps);
        if (rstd) rstd[i] = r;
        for (int64_t j = 0; j < N; ++j) {
            double h = load_elem(x, xdt, i * N + j) * r;
            double n = round_to(xdt, h);
            double wj = load_elem(w, wdt, j);
            double v = round_arith(xdt, wj * n);
            if (y) y[i * N + j] = v;
            if (y_scale) y_scale[i * N + j] = fabs(v);
            if (y_alt) y_alt[i * N + j] = round_arith(xdt, wj * rounding_alternative(h, n, xdt));
        }
    }
    return 0;
}

typedef struct {
    int64_t N;
    const void *x, *dy;
    int xdt, wdt;
    double eps;
} rms_ctx;

/* Column terms of row i: round_wdt(round_arith(dy * n)) with n = round_xdt(x * rstd).  The
 * weight gradient is formed in the weight's dtype, so a bfloat16 weight rounds each product
 * to bfloat16 before the column sum ([RMS] Semantics); a float32 weight keeps the float32
 * product (exact for bf16 * bf16).  Columns [N, 2N) receive |term(n_alt) - term(n)|, where
 * n_alt is the other rounding of h that a float32 computation may also reach (see
 * rounding_alternative): the slack the column sum may legitimately carry. */
static void rms_bwd_terms(const void* vctx, int64_t i, double* terms) {
    const rms_ctx* c = (const rms_ctx*)vctx;
    double r = rms_row_rstd(c->x, c->xdt, i, c->N, c->eps);
    for (int64_t j = 0; j < c->N; ++j) {
        double h = load_elem(c->x, c->xdt, i * c->N + j) * r;
        double n = round_to(c->xdt, h);
        double g = load_elem(c->dy, c->xdt, i * c->N + j);
        double t = round_to(c->wdt, round_arith(c->xdt, g * n));
        double ta = round_to(c->wdt, round_arith(c->xdt, g * rounding_alternative(h, n, c->xdt)));
        terms[j] = t;
        terms[c->N + j] = fabs(ta - t);
    }
}

/* [RMS] Semantics.  g = round_xdt(round_arith(dy * w)) (the float32 product, rounded to the
 * input dtype as autograd rounds the gradient of the normalized value); h = x * r (unrounded);
 * c = mean_j(g * h); dx = r * (g - h * c); dx_scale = r * (|g| + |h| * mean_j |g_j h_j|), the
 * magnitudes of every term of dx expanded through c.
 * dw_j = sum_i round_wdt(dy_ij * n_ij) (+ magnitude sum; dw_slack_j = sum_i of the change of
 * the term under the other admissible rounding of n, may be NULL). */
int oracle_rmsnorm_bwd(int64_t M, int64_t N, const void* x, const void* dy, int xdt,
                       const void* w, int wdt, double eps, double* dx, double* dx_scale,
                       double* dw, double* dw_scale, double* dw_slack) {
    if (M < 0 || N < 1) return -1;
    if (dx || dx_scale) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < M; ++i) {
            double r = rms_row_rstd(x, xdt, i, N, eps);
            double c = 0.0, a = 0.0;
            for (int64_t j = 0; j < N; ++j) {
                double g = round_to(xdt, round_arith(xdt, load_elem(dy, xdt, i * N + j) * load_elem(w, wdt, j)));
                c += g * load_elem(x, xdt, i * N + j) * r;
                a += fabs(g * load_elem(x, xdt, i * N + j) * r);
            }
            c /= (double)N;
            a /= (double)N;
            for (int64_t j = 0; j < N; ++j) {
                double g = round_to(xdt, round_arith(xdt, load_elem(dy, xdt, i * N + j) * load_elem(w, wdt, j)));
                double h = load_elem(x, xdt, i * N + j) * r;
                if (dx) dx[i * N + j] = r * (g - h * c);
                if (dx_scale) dx_scale[i * N + j] = r * (fabs(g) + fabs(h) * a);
            }
        }
    }
    if (dw || dw_scale || dw_slack) {
        rms_ctx c = {N, x, dy, xdt, wdt, eps};
        double* s = (double*)malloc((size_t)(2 * N) * sizeof(double));
        double* a = (double*)malloc((size_t)(2 * N) * sizeof(double));
        if (!s || !a || column_sums(&c, rms_bwd_terms, M, 2 * N, s, a) != 0) {
            free(s); free(a);
            return -2;
        }
        for (int64_t j = 0; j < N; ++j) {
            if (dw) dw[j] = s[j];
            if (dw_scale) dw_scale[j] = a[j];
            if (dw_slack) dw_slack[j] = s[N + j];
        }
        free(s); free(a);
    }
    return 0;
}

/* The two float32 forms of the same passage ([RMS] "Which modules are replaced" and "Not
 * covered"): classes that multiply by the weight before the cast, and the (1 + weight) family.
 * Both scale the unrounded normalized value h = x * r in float32 and round once:
 * y = s_j * h with s_j = w_j (form 1) or s_j = round_arith(1 + w_j) (form 2; eager adds 1 to
 * the float32 weight).  The final cast is left to the caller's tolerance; y_scale = |y|; there
 * is no alternative rounding (y_alt = y).  Form 0 is the Llama form above. */
static double rms_form_scale(int form, int xdt, double wj) {
    return form == 2 ? round_arith(xdt, 1.0 + wj) : wj;
}

int oracle_rmsnorm_fwd_form(int64_t M, int64_t N, const void* x, int xdt, const void* w, int wdt,
                            double eps, int form, double* y, double* y_scale, double* y_alt,
                            double* rstd) {
    if (form == 0) return oracle_rmsnorm_fwd(M, N, x, xdt, w, wdt, eps, y, y_scale, y_alt, rstd);
    if ((form != 1 && form != 2) || M < 0 || N < 1) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double r = rms_row_rstd(x, xdt, i, N, eps);
        if (rstd) rstd[i] = r;
        for (int64_t j = 0; j < N; ++j) {
            double v = rms_form_scale(form, xdt, load_elem(w, wdt, j)) * (load_elem(x, xdt, i * N + j) * r);
            if (y) y[i * N + j] = v;
            if (y_scale) y_scale[i * N + j] = fabs(v);
            if (y_alt) y_alt[i * N + j] = v;
        }
    }
    return 0;
}

/* Column terms of row i for the float32 forms: dy * h (unrounded; the weight gradient of a
 * float32 product is summed in float32 and rounded once), and no slack. */
static void rms_form_bwd_terms(const void* vctx, int64_t i, double* terms) {
    const rms_ctx* c = (const rms_ctx*)vctx;
    double r = rms_row_rstd(c->x, c->xdt, i, c->N, c->eps);
    for (int64_t j = 0; j < c->N; ++j) {
        terms[j] = load_elem(c->dy, c->xdt, i * c->N + j) * (load_elem(c->x, c->xdt, i * c->N + j) * r);
        terms[c->N + j] = 0.0;
    }
}

/* Backward of the float32 forms: g = dy * s_j (no rounding: the product stays in float32);
 * h = x * r; c = mean_j(g * h); dx = r * (g - h * c), dx_scale as in the Llama form;
 * dw_j = sum_i dy_ij * h_ij (+ magnitude sum; dw_slack = 0). */
int oracle_rmsnorm_bwd_form(int64_t M, int64_t N, const void* x, const void* dy, int xdt,
                            const void* w, int wdt, double eps, int form, double* dx,
                            double* dx_scale, double* dw, double* dw_scale, double* dw_slack) {
    if (form == 0)
        return oracle_rmsnorm_bwd(M, N, x, dy, xdt, w, wdt, eps, dx, dx_scale, dw, dw_scale, dw_slack);
    if ((form != 1 && form != 2) || M < 0 || N < 1) return -1;
    if (dx || dx_scale) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < M; ++i) {
            double r = rms_row_rstd(x, xdt, i, N, eps);
            double c = 0.0, a = 0.0;
            for (int64_t j = 0; j < N; ++j) {
                double g = load_elem(dy, xdt, i * N + j) * rms_form_scale(form, xdt, load_elem(w, wdt, j));
                double h = load_elem(x, xdt, i * N + j) * r;
                c += g * h;
                a += fabs(g * h);
            }
            c /= (double)N;
            a /= (double)N;
            for (int64_t j = 0; j < N; ++j) {
                double g = load_elem(dy, xdt, i * N + j) * rms_form_scale(form, xdt, load_elem(w, wdt, j));
                double h = load_elem(x, xdt, i * N + j) * r;
                if (dx) dx[i * N + j] = r * (g - h * c);
                if (dx_scale) dx_scale[i * N + j] = r * (fabs(g) + fabs(h) * a);
            }
        }
    }
    if (dw || dw_scale || dw_slack) {
        rms_ctx c = {N, x, dy, xdt, wdt, eps};
        double* s = (double*)malloc((size_t)(2 * N) * sizeof(double));
        double* a = (double*)malloc((size_t)(2 * N) * sizeof(double));
        if (!s || !a || column_sums(&c, rms_form_bwd_terms, M, 2 * N, s, a) != 0) {
            free(s); free(a);
            return -2;
        }
        for (int64_t j = 0; j < N; ++j) {
            if (dw) dw[j] = s[j];
            if (dw_scale) dw_scale[j] = a[j];
            if (dw_slack) dw_slack[j] = 0.0;
        }
        free(s); free(a);
    }
    return 0;
}

/* Exported for the pins: round an array of doubles to bfloat16 / float32 values. */
void oracle_round_array(const double* in, double* out, int64_t n, int dt) {
    for (int64_t k = 0; k < n; ++k) out[k] = round_to(dt, in[k]);
}

/* The values the oracle reads from n stored elements of dtype dt. */
void oracle_load_array(const void* p, int dt, int64_t n, double* out) {
    for (int64_t k = 0; k < n; ++k) out[k] = load_elem(p, dt, k);
}
