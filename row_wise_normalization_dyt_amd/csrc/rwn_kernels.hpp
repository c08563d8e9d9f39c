// Row kernels for DyT, LayerNorm and RMSNorm, forward and backward stage 1, plus the
// stage-2 column reduction (gfx950, wave64).
//
// Every row kernel runs a persistent 1D grid: workgroup w visits row tiles w, w + grid, ...
// (a tile is rpp * RT rows), so M is bounded only by 64-bit indexing, and the number of
// workgroups -- which is also the number of partial rows of the backward -- is chosen by the
// host from the device's CU count.  Each thread reads its x (and dy) chunks of a row once
// into registers, reduces across the row's threads (DPP inside a wave, LDS across waves),
// and writes y or dx from the same registers.
//
// Backward stage 1 accumulates the parameter-gradient terms of its columns in float32
// registers over every row the thread visits, then writes one partial row per workgroup to
// the workspace [grid, ng] (ng = 2N+1 DyT: dgamma | dbeta | dalpha; 2N LayerNorm:
// dgamma | dbeta; N RMSNorm: dweight).  Row slots of a workgroup are combined by a fixed tree
// through LDS.  Stage 2 sums the partial rows per column in a fixed order in float64.  No
// atomics anywhere: the reduction order depends only on the launch plan.
#pragma once

#include "rwn_device.hpp"

namespace rwn {

constexpr int kMaxBlock = 64 * kMaxWaves;
// Largest workgroup a plan gives each kernel shape (the planner keeps to it): narrow plans
// (RT > 1) run 256 threads; one chunk per thread, and bf16 with four, at most 8 waves per row
// (a 256-register budget); otherwise up to 16 waves (128 registers).
template <typename T, int RT, int CPT> struct MaxBlock {
    static constexpr int value = RT > 1 ? 256 : (CPT == 1 || (CPT == 4 && sizeof(T) == 2)) ? 512 : kMaxBlock;
};
static_assert(MaxBlock<bf16_t, 1, 4>::value == 512 && MaxBlock<float, 1, 4>::value == 1024 &&
                  MaxBlock<float, 4, 1>::value == 256 && MaxBlock<bf16_t, 1, 2>::value == 1024,
              "kernel launch bounds must match the planner's max_block()");
constexpr int kRedFloats = 2 * kMaxWaves * 8;   // row_sum buffers: 2 halves x waves x K <= 8

// Per-thread setup common to all row kernels: slot/lane, the workgroup's tile range and the
// thread's column map.
template <typename T, int MODE, int CPT, int RT>
struct RowCtx {
    int slot, lane;
    int cblk;           // column block of this workgroup
    int64_t wg;         // workgroup index among those sharing cblk (= its partial row)
    int64_t rows_per_tile;
    int64_t t_begin, t_end, t_step;
    ColMap<T, MODE, CPT> cm;

    __device__ __forceinline__ RowCtx(const Geom& g) {
        // Workgroups are whole waves: with rows of tpr lanes packed without wave alignment,
        // the threads past rpp * tpr form a slot of their own that owns no row (every load
        // reads zeros, nothing is stored), and take part only in the workgroup's reductions.
        slot = threadIdx.x / g.tpr;
        lane = threadIdx.x - slot * g.tpr;
        // Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2).  The
        // remap gives consecutive logical numbers -- and so neighbouring rows, whose shared
        // cache lines both write -- to workgroups on the same XCD.
        int64_t b = blockIdx.x;
        if (g.xcd_remap) b = (b % 8) * (gridDim.x / 8) + b / 8;
        cblk = (int)(b % g.ncb);
        wg = b / g.ncb;
        rows_per_tile = (int64_t)g.rpp * RT;
        if (g.strided) {
            t_begin = wg;
            t_end = g.ntiles;
            t_step = gridDim.x / g.ncb;
        } else {
            t_begin = wg * g.kt;
            t_end = t_begin + g.kt < g.ntiles ? t_begin + g.kt : g.ntiles;
            t_step = 1;
        }
        int s = 0;
        if (MODE == MODE_SHIFTED) {
            // Every row this thread visits differs from the first by a multiple of V (the
            // launcher makes rpp, or the tile stride times rpp, a multiple of V), so the first
            // row fixes the shift.
            const int64_t r0 = t_begin * rows_per_tile + slot;
            s = (int)(((int64_t)g.base_shift + r0 * g.pitch) % ColMap<T, MODE, CPT>::V);
        }
        cm.init(lane, g.tpr, g.N, s, cblk * g.tpr * CPT);
    }
    __device__ __forceinline__ int64_t row(int64_t tile, int u, const Geom& g) const {
        return tile * rows_per_tile + (int64_t)u * g.rpp + slot;
    }
    // Rows of `tile` for this thread; a row is live when the tile is one of this workgroup's
    // and the row exists.
    __device__ __forceinline__ void tile_rows(int64_t tile, const Geom& g, int64_t (&r)[RT],
                                              bool (&ok)[RT]) const {
#pragma unroll
        for (int u = 0; u < RT; ++u) {
            r[u] = row(tile, u, g);
            ok[u] = tile < t_end && r[u] < g.M && slot < g.rpp;
        }
    }
};

// Software pipelining of the tile loop (kernel parameter PF, chosen by the planner).  With
// PF = 1 the loads of the next tile are issued before the current tile is reduced, computed
// and stored, so every wave keeps two tiles of loads in flight and the store of one tile
// overlaps the load of the next; the registers holding a tile's inputs are doubled.  Only
// shapes with at most two 16-byte chunks per thread per tensor have that form.  PF = 2 runs
// two tiles ahead (three buffers), for one chunk per thread.

// Runs body(in) for every tile of the workgroup in order; fetch(tile, in) issues the tile's
// loads (a tile past the workgroup's range loads nothing).  The pipelined form alternates two
// buffers instead of copying the next tile into the current one: a register copy would have
// to wait for the loads it copies and so end the overlap.
template <int PF, typename In, typename Ctx, typename Fetch, typename Body>
__device__ __forceinline__ void tile_loop(const Ctx& c, Fetch&& fetch, Body&& body) {
    if constexpr (PF == 2) {
        // two tiles ahead: three buffers in rotation
        In a, b, d;
        fetch(c.t_begin, a);
        fetch(c.t_begin + c.t_step, b);
        for (int64_t tile = c.t_begin; tile < c.t_end; tile += 3 * c.t_step) {
            fetch(tile + 2 * c.t_step, d);
            body(a);
            if (tile + c.t_step >= c.t_end) break;
            fetch(tile + 3 * c.t_step, a);
            body(b);
            if (tile + 2 * c.t_step >= c.t_end) break;
            fetch(tile + 4 * c.t_step, b);
            body(d);
        }
    } else if constexpr (PF == 1) {
        In a, b;
        fetch(c.t_begin, a);
        for (int64_t tile = c.t_begin; tile < c.t_end; tile += 2 * c.t_step) {
            fetch(tile + c.t_step, b);
            body(a);
            if (tile + c.t_step >= c.t_end) break;
            fetch(tile + 2 * c.t_step, a);
            body(b);
        }
    } else {
        for (int64_t tile = c.t_begin; tile < c.t_end; tile += c.t_step) {
            In cur;
            fetch(tile, cur);
            body(cur);
        }
    }
}

// Load a per-column parameter (or `dflt` for every column when p is NULL).
template <typename T, typename PT, int MODE, int CPT>
__device__ __forceinline__ void load_param_or(const PT* __restrict__ p, float dflt, int64_t N, int64_t ps,
                                              const ColMap<T, MODE, CPT>& cm, float* o) {
    constexpr int E = CPT * ColMap<T, MODE, CPT>::V;
    if (p) {
        load_param<T, PT, MODE, CPT>(p, N, ps, cm, o);
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = dflt;
    }
}

// Write one gradient's partial row: out[col * cs] = sum over the row slots of acc (a fixed
// order that depends only on the plan).
// `part` is LDS of max(E * blockDim.x, N) floats (only used when rpp > 1).
template <typename T, int MODE, int CPT>
__device__ __forceinline__ void write_partial(float* __restrict__ out, int64_t cs, const float* acc,
                                              const ColMap<T, MODE, CPT>& cm, int slot, int lane,
                                              const Geom& g, float* part) {
    constexpr int V = ColMap<T, MODE, CPT>::V;
    constexpr int E = CPT * V;
    if (g.rpp == 1) {
        if (slot != 0) return;   // the idle slot of a packed workgroup
#pragma unroll
        for (int k = 0; k < CPT; ++k)
#pragma unroll
            for (int v = 0; v < V; ++v)
                if (cm.valid(k, v, g.N)) out[(int64_t)(cm.col0[k] + v) * cs] = acc[k * V + v];
        return;
    }
    const int nb = blockDim.x;
    if (MODE == MODE_SHIFTED) {
        // Slots hold different column maps: each slot writes its sums into a column-indexed
        // LDS row of its own (within a slot every column of [0, N) has exactly one owner), then
        // each column adds the slots' rows in slot order.  `part` holds rpp * N floats here.
        // (Only single-column-block plans have SHIFTED slots, so a row is all of [0, N).)
        __syncthreads();   // previous users of `part` are done
        if (slot < g.rpp) {
            float* mine = part + (int64_t)slot * g.N;
#pragma unroll
            for (int k = 0; k < CPT; ++k)
#pragma unroll
                for (int v = 0; v < V; ++v)
                    if (cm.valid(k, v, g.N)) mine[cm.col0[k] + v] = acc[k * V + v];
        }
        __syncthreads();
        for (int64_t j = threadIdx.x; j < g.N; j += nb) {
            float sum = part[j];
            for (int sl = 1; sl < g.rpp; ++sl) sum += part[(int64_t)sl * g.N + j];
            out[j * cs] = sum;
        }
        return;
    }
    if (g.tpr < 64) {
        // Narrow rows: the 64 / tpr slots of a wave share one column map.  An xor butterfly over
        // lane offsets tpr, 2 tpr, ..., 32 leaves every lane with the wave's sum for its columns
        // (both partners of each step add the same two values, so they hold identical bits);
        // then one LDS round adds the waves' sums in wave order.
        const int nw = (nb + 63) >> 6;
        const int wl = nb < 64 ? nb : 64;
        float v[E];
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = acc[e];
        for (int off = g.tpr; off < wl; off <<= 1) {
#pragma unroll
            for (int e = 0; e < E; ++e) v[e] += __shfl_xor(v[e], off, 64);
        }
        const int wave = threadIdx.x >> 6;
        __syncthreads();   // previous users of `part` are done
        if ((threadIdx.x & 63) < g.tpr) {
#pragma unroll
            for (int e = 0; e < E; ++e) part[(wave * g.tpr + lane) * E + e] = v[e];
        }
        __syncthreads();
        if (threadIdx.x < g.tpr) {
#pragma unroll
            for (int k = 0; k < CPT; ++k)
#pragma unroll
                for (int vv = 0; vv < V; ++vv) {
                    const int e = k * V + vv;
                    float sum = part[lane * E + e];
                    for (int w = 1; w < nw; ++w) sum += part[(w * g.tpr + lane) * E + e];
                    if (cm.valid(k, vv, g.N)) out[(int64_t)(cm.col0[k] + vv) * cs] = sum;
                }
        }
        return;
    }
    // Wide rows: slots are whole waves with one column map; a fixed binary tree over the slots,
    // every thread taking part (slot s adds slot s + st for st = P/2, P/4, ..., 1, P the power of
    // two >= rpp).
    __syncthreads();   // previous users of `part` are done
#pragma unroll
    for (int e = 0; e < E; ++e) part[e * nb + threadIdx.x] = acc[e];
    int st = 1;
    while (st < g.rpp) st <<= 1;
    for (st >>= 1; st >= 1; st >>= 1) {
        __syncthreads();
        if (slot < st && slot + st < g.rpp) {
#pragma unroll
            for (int e = 0; e < E; ++e) part[e * nb + threadIdx.x] += part[e * nb + threadIdx.x + st * g.tpr];
        }
    }
    __syncthreads();
    if (slot == 0) {
#pragma unroll
        for (int k = 0; k < CPT; ++k)
#pragma unroll
            for (int v = 0; v < V; ++v)
                if (cm.valid(k, v, g.N)) out[(int64_t)(cm.col0[k] + v) * cs] = part[(k * V + v) * nb + lane];
    }
}

// ================================================================================== DyT

template <typename T, typename PT, int MODE, int CPT, int RT, int PF, int LAY>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, MaxBlock<T, RT, CPT>::value)))
dyt_fwd_kernel(const T* __restrict__ x, const PT* __restrict__ alpha_p,
               const PT* __restrict__ gamma, const PT* __restrict__ beta, T* __restrict__ y,
               Geom g) {
    constexpr int V = Elems<T, MODE>::value;
    constexpr int E = CPT * V;
    RowCtx<T, MODE, CPT, RT> c(g);
    float ga[E], be[E];
    load_param<T, PT, MODE, CPT>(gamma, g.N, g.ps0, c.cm, ga);
    load_param<T, PT, MODE, CPT>(beta, g.N, g.ps1, c.cm, be);
    const float alpha = to_f32(alpha_p[0]);
    struct In {
        RowRegs<T, MODE, CPT> xr[RT];
        int64_t row[RT];
        int64_t row0;
        bool ok[RT];
    };
    auto fetch = [&](int64_t tile, In& in) {
        c.tile_rows(tile, g, in.row, in.ok);
        const int64_t row0 = tile * c.rows_per_tile;
        in.row0 = row0;
        const TileSrc sx = tile_src<T, MODE, LAY>(x, row0, g, OP_X, tile < c.t_end);
#pragma unroll
        for (int u = 0; u < RT; ++u) load_row<T, MODE, CPT>(sx, row_base<LAY>(g, OP_X, in.row[u]), c.cm, in.ok[u], in.xr[u]);
    };
    auto body = [&](const In& in) {
#pragma unroll
        for (int u = 0; u < RT; ++u) {
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                float o[V];
#pragma unroll
                for (int v = 0; v < V; ++v)
                    o[v] = __builtin_fmaf(ga[k * V + v], tanh_only(alpha * in.xr[u].get(k, v)), be[k * V + v]);
                store_chunk<T, MODE, CPT>(y, row_base<LAY>(g, OP_OUT, in.row[u]), g.N, c.cm, k, o, in.ok[u]);
            }
        }
    };
    tile_loop<PF, In>(c, fetch, body);
}

// PG 0: no parameter gradient is wanted; the kernel computes dx only (no column partials,
// nothing written to the workspace, which may be NULL).
template <typename T, typename PT, int MODE, int CPT, int RT, int PF, int PG, int LAY>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, MaxBlock<T, RT, CPT>::value)))
dyt_bwd_kernel(const T* __restrict__ x, const T* __restrict__ dy, const PT* __restrict__ alpha_p,
               const PT* __restrict__ gamma, T* __restrict__ dx, float* __restrict__ ws,
               Geom g) {
    constexpr int V = Elems<T, MODE>::value;
    constexpr int E = CPT * V;
    extern __shared__ float part[];
    __shared__ float red[kRedFloats];
    RowCtx<T, MODE, CPT, RT> c(g);
    float ga[E];
    load_param<T, PT, MODE, CPT>(gamma, g.N, g.ps0, c.cm, ga);
    const float alpha = to_f32(alpha_p[0]);
    float acc_g[E], acc_b[E], acc_a = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc_g[e] = acc_b[e] = 0.f;

    struct In {
        RowRegs<T, MODE, CPT> xr[RT], gr[RT];
        int64_t row[RT];
        int64_t row0;
        bool ok[RT];
    };
    auto fetch = [&](int64_t tile, In& in) {
        c.tile_rows(tile, g, in.row, in.ok);
        const int64_t row0 = tile * c.rows_per_tile;
        in.row0 = row0;
        const bool live = tile < c.t_end;
        const TileSrc sx = tile_src<T, MODE, LAY>(x, row0, g, OP_X, live);
        const TileSrc sg = tile_src<T, MODE, LAY>(dy, row0, g, OP_DY, live);
#pragma unroll
        for (int u = 0; u < RT; ++u) {
            load_row<T, MODE, CPT>(sx, row_base<LAY>(g, OP_X, in.row[u]), c.cm, in.ok[u], in.xr[u]);
            load_row<T, MODE, CPT>(sg, row_base<LAY>(g, OP_DY, in.row[u]), c.cm, in.ok[u], in.gr[u]);
        }
    };
    // With a finite alpha nothing a padded element computes can be NaN: its x, dy and gamma
    // read as 0, so z = 0, tanh = 0, sech^2 = 1 and every term it adds is exactly 0.  That case
    // needs no masks.  With alpha = +-inf a padded x = 0 gives z = inf * 0 = NaN, so those terms
    // are dropped after the arithmetic, and alpha * sech^2 is taken as 0 where sech^2 is 0.
    const bool finite_alpha = __builtin_isfinite(alpha);
    constexpr bool BUF = kBufferStores<MODE, CPT, true>;
    auto body = [&](const In& in) {
        const TileSrc dst = tile_src<T, MODE, LAY>(dx, in.row0, g, OP_OUT, true);
        auto rows = [&](auto finite) {
#pragma unroll
            for (int u = 0; u < RT; ++u) {
#pragma unroll
                for (int k = 0; k < CPT; ++k) {
                    float o[V];
#pragma unroll
                    for (int v = 0; v < V; ++v) {
                        const int e = k * V + v;
                        const float xv = in.xr[u].get(k, v), gv = in.gr[u].get(k, v);
                        const TanhSech2 ts = tanh_sech2(alpha * xv);
                        const float d = gv * ga[e];
                        if constexpr (decltype(finite)::value) {
                            const float ds = d * ts.s;   // dy * gamma * sech^2
                            if constexpr (PG) {
                                acc_g[e] = __builtin_fmaf(gv, ts.t, acc_g[e]);
                                acc_b[e] += gv;
                                acc_a = __builtin_fmaf(xv, ds, acc_a);
                            }
                            o[v] = alpha * ds;
                        } else {
                            const float as = ts.s == 0.f ? 0.f : alpha * ts.s;
                            if constexpr (PG) {
                                const bool live = in.ok[u] && c.cm.valid(k, v, g.N);
                                acc_g[e] += live ? gv * ts.t : 0.f;
                                acc_b[e] += live ? gv : 0.f;
                                acc_a += live ? d * xv * ts.s : 0.f;
                            }
                            o[v] = d * as;
                        }
                    }
                    put_chunk<T, MODE, CPT, BUF>(dx, dst, row_base<LAY>(g, OP_OUT, in.row[u]), g.N, c.cm, k, o, in.ok[u]);
                }
            }
        };
        if (finite_alpha) rows(IC<1>{});
        else rows(IC<0>{});
    };
    tile_loop<PF, In>(c, fetch, body);
    // Partial row c.wg; this workgroup's column block of dgamma | dbeta, and its own dalpha
    // column 2N + cblk (stage 2 adds the ncb dalpha columns together).
    if constexpr (PG) {
        float* out = ws + c.wg * g.ws_rs;
        write_partial<T, MODE, CPT>(out, g.ws_cs, acc_g, c.cm, c.slot, c.lane, g, part);
        write_partial<T, MODE, CPT>(out + g.N * g.ws_cs, g.ws_cs, acc_b, c.cm, c.slot, c.lane, g, part);
        const float da = block_sum(acc_a, red);
        if (threadIdx.x == 0) out[(2 * g.N + c.cblk) * g.ws_cs] = da;
    }
}

// ============================================================================ LayerNorm

// mean and rstd of RT rows (two passes over the registers: sum, then sum of squared
// deviations).
template <typename T, int MODE, int CPT, int RT>
__device__ __forceinline__ void ln_stats(const RowRegs<T, MODE, CPT> (&xr)[RT],
                                         const ColMap<T, MODE, CPT>& cm, const Geom& g, float eps,
                                         float* red, int& parity, float (&mu)[RT], float (&rs)[RT]) {
    constexpr int V = Elems<T, MODE>::value;
    float s[RT];
#pragma unroll
    for (int u = 0; u < RT; ++u) {
        float a = 0.f;
#pragma unroll
        for (int k = 0; k < CPT; ++k)
#pragma unroll
            for (int v = 0; v < V; ++v) a += xr[u].get(k, v);
        s[u] = a;
    }
    row_sum<RT>(s, g.tpr, red, parity);
#pragma unroll
    for (int u = 0; u < RT; ++u) mu[u] = s[u] * g.inv_n;
#pragma unroll
    for (int u = 0; u < RT; ++u) {
        float a = 0.f;
#pragma unroll
        for (int k = 0; k < CPT; ++k)
#pragma unroll
            for (int v = 0; v < V; ++v) {
                if constexpr (MODE == MODE_SHIFTED) {
                    // d masked to exactly 0 for elements outside the row
                    const float d = __builtin_bit_cast(
                        float, __builtin_bit_cast(uint32_t, xr[u].get(k, v) - mu[u]) & cm.row_mask(k, v));
                    a = __builtin_fmaf(d, d, a);
                } else {
                    const float d = xr[u].get(k, v) - mu[u];
                    a += cm.valid(k, v, g.N) ? d * d : 0.f;
                }
            }
        s[u] = a;
    }
    row_sum<RT>(s, g.tpr, red, parity);
#pragma unroll
    for (int u = 0; u < RT; ++u) rs[u] = __builtin_amdgcn_rsqf(s[u] * g.inv_n + eps);
}

template <typename T, typename PT, int MODE, int CPT, int RT, int PF, int LAY>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, MaxBlock<T, RT, CPT>::value)))
ln_fwd_kernel(const T* __restrict__ x, const PT* __restrict__ gamma, const PT* __restrict__ beta,
              float eps, T* __restrict__ y, float* __restrict__ mean_out,
              float* __restrict__ rstd_out, Geom g) {
    constexpr int V = Elems<T, MODE>::value;
    constexpr int E = CPT * V;
    __shared__ float red[kRedFloats];
    int parity = 0;
    RowCtx<T, MODE, CPT, RT> c(g);
    float ga[E], be[E];
    load_param_or<T, PT, MODE, CPT>(gamma, 1.f, g.N, g.ps0, c.cm, ga);
    load_param_or<T, PT, MODE, CPT>(beta, 0.f, g.N, g.ps1, c.cm, be);
    struct In {
        RowRegs<T, MODE, CPT> xr[RT];
        int64_t row[RT];
        int64_t row0;
        bool ok[RT];
    };
    auto fetch = [&](int64_t tile, In& in) {
        c.tile_rows(tile, g, in.row, in.ok);
        const int64_t row0 = tile * c.rows_per_tile;
        in.row0 = row0;
        const TileSrc sx = tile_src<T, MODE, LAY>(x, row0, g, OP_X, tile < c.t_end);
#pragma unroll
        for (int u = 0; u < RT; ++u) load_row<T, MODE, CPT>(sx, row_base<LAY>(g, OP_X, in.row[u]), c.cm, in.ok[u], in.xr[u]);
    };
    auto body = [&](const In& in) {
        float mu[RT], rs[RT];
        ln_stats<T, MODE, CPT, RT>(in.xr, c.cm, g, eps, red, parity, mu, rs);
#pragma unroll
        for (int u = 0; u < RT; ++u) {
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                float o[V];
#pragma unroll
                for (int v = 0; v < V; ++v)
                    o[v] = __builtin_fmaf((in.xr[u].get(k, v) - mu[u]) * rs[u], ga[k * V + v], be[k * V + v]);
                store_chunk<T, MODE, CPT>(y, row_base<LAY>(g, OP_OUT, in.row[u]), g.N, c.cm, k, o, in.ok[u]);
            }
            if (in.ok[u] && c.lane == 0) {
                if (mean_out) mean_out[in.row[u]] = mu[u];
                if (rstd_out) rstd_out[in.row[u]] = rs[u];
            }
        }
    };
    tile_loop<PF, In>(c, fetch, body);
}

// PG: which parameter-gradient partials are accumulated and written (bit 0: dgamma, bit 1:
// dbeta; 0: dx only, the workspace may be NULL).
template <typename T, typename PT, int MODE, int CPT, int RT, int PF, int PG, int LAY>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, MaxBlock<T, RT, CPT>::value)))
ln_bwd_kernel(const T* __restrict__ x, const T* __restrict__ dy, const float* __restrict__ mean_in,
              const float* __restrict__ rstd_in, const PT* __restrict__ gamma, float eps,
              T* __restrict__ dx, float* __restrict__ ws, Geom g) {
    constexpr int V = Elems<T, MODE>::value;
    constexpr int E = CPT * V;
    extern __shared__ float part[];
    __shared__ float red[kRedFloats];
    int parity = 0;
    RowCtx<T, MODE, CPT, RT> c(g);
    float ga[E];
    load_param_or<T, PT, MODE, CPT>(gamma, 1.f, g.N, g.ps0, c.cm, ga);
    const bool have_stats = mean_in != nullptr && rstd_in != nullptr;
    float acc_g[E], acc_b[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc_g[e] = acc_b[e] = 0.f;

    struct In {
        RowRegs<T, MODE, CPT> xr[RT], gr[RT];
        int64_t row[RT];
        int64_t row0;
        bool ok[RT];
        float mu[RT], rs[RT];
    };
    auto fetch = [&](int64_t tile, In& in) {
        c.tile_rows(tile, g, in.row, in.ok);
        const int64_t row0 = tile * c.rows_per_tile;
        in.row0 = row0;
        const bool live = tile < c.t_end;
        const TileSrc sx = tile_src<T, MODE, LAY>(x, row0, g, OP_X, live);
        const TileSrc sg = tile_src<T, MODE, LAY>(dy, row0, g, OP_DY, live);
        const Rsrc sm = stats_src(mean_in, row0, g.M, live && have_stats);
        const Rsrc sr = stats_src(rstd_in, row0, g.M, live && have_stats);
#pragma unroll
        for (int u = 0; u < RT; ++u) {
            load_row<T, MODE, CPT>(sx, row_base<LAY>(g, OP_X, in.row[u]), c.cm, in.ok[u], in.xr[u]);
            load_row<T, MODE, CPT>(sg, row_base<LAY>(g, OP_DY, in.row[u]), c.cm, in.ok[u], in.gr[u]);
            in.mu[u] = load_stat(sm, in.row[u], row0, in.ok[u]);
            in.rs[u] = load_stat(sr, in.row[u], row0, in.ok[u]);
        }
    };
    auto body = [&](const In& in) {
        const auto& xr = in.xr;
        const auto& gr = in.gr;
        const auto& ok = in.ok;
        const auto& row = in.row;
        constexpr bool BUF = kBufferStores<MODE, CPT, true>;
        const TileSrc dst = tile_src<T, MODE, LAY>(dx, in.row0, g, OP_OUT, true);
        float mu[RT], rs[RT];
#pragma unroll
        for (int u = 0; u < RT; ++u) {
            mu[u] = in.mu[u];
            rs[u] = in.rs[u];
        }
        if (!have_stats) ln_stats<T, MODE, CPT, RT>(xr, c.cm, g, eps, red, parity, mu, rs);
        // Padded elements read x = dy = gamma = 0, so every term below is 0 for them as long as
        // x_hat is finite: a padded row's statistics are zeroed (recomputed ones could be
        // infinite with eps = 0).  No per-element masks are needed.
#pragma unroll
        for (int u = 0; u < RT; ++u) {
            mu[u] = ok[u] ? mu[u] : 0.f;
            rs[u] = ok[u] ? rs[u] : 0.f;
        }
        float s[2 * RT];
#pragma unroll
        for (int u = 0; u < RT; ++u) {
            float a = 0.f, b = 0.f;
#pragma unroll
            for (int k = 0; k < CPT; ++k)
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    const float xh = (xr[u].get(k, v) - mu[u]) * rs[u];
                    const float gg = gr[u].get(k, v) * ga[k * V + v];
                    a += gg;
                    b = __builtin_fmaf(gg, xh, b);
                }
            s[2 * u] = a;
            s[2 * u + 1] = b;
        }
        row_sum<2 * RT>(s, g.tpr, red, parity);
#pragma unroll
        for (int u = 0; u < RT; ++u) {
            const float c1 = s[2 * u] * g.inv_n, c2 = s[2 * u + 1] * g.inv_n;
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                float o[V];
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    const int e = k * V + v;
                    const float gv = gr[u].get(k, v);
                    const float xh = (xr[u].get(k, v) - mu[u]) * rs[u];
                    if constexpr (PG & 1) acc_g[e] = __builtin_fmaf(gv, xh, acc_g[e]);
                    if constexpr (PG & 2) acc_b[e] += gv;
                    o[v] = rs[u] * (gv * ga[e] - c1 - xh * c2);
                }
                put_chunk<T, MODE, CPT, BUF>(dx, dst, row_base<LAY>(g, OP_OUT, row[u]), g.N, c.cm, k, o, ok[u]);
            }
        }
    };
    tile_loop<PF, In>(c, fetch, body);
    float* out = ws + c.wg * g.ws_rs;
    if constexpr (PG & 1) write_partial<T, MODE, CPT>(out, g.ws_cs, acc_g, c.cm, c.slot, c.lane, g, part);
    if constexpr (PG & 2)
        write_partial<T, MODE, CPT>(out + g.N * g.ws_cs, g.ws_cs, acc_b, c.cm, c.slot, c.lane, g, part);
}

// ------------------------------------------------------------ LayerNorm, flat narrow rows
// Narrow aligned rows (TPR <= 64 lanes per row, one 16-byte chunk per lane, one row per thread
// per tile, no pipelining) through plain global loads and stores instead of per-tile buffer
// descriptors.  A padded row loads the tensor's last row (a clamped index, always in bounds)
// and a lane past the row's chunks loads the row's first chunk; both are zeroed after the
// load, so every term they feed is 0, as with the descriptors' zero reads.  The group size and
// whether the forward's statistics are given are template values, so a tile is one straight
// line: its loads (x, dy and both statistics) issue together, and the row sums are fixed DPP
// sequences.  The arithmetic, its order, the partial rows and their combine are those of the
// general kernels, except that the backward combines its two partial rows at once.  (LayerNorm
// 401408 x 24 float32, measured: backward stage 1 23.7 -> 22.0 us, dx only 21.4 -> 20.2 us,
// forward 16.4 -> 16.1 us.)
template <typename T>
__device__ __forceinline__ void load_flat(const T* __restrict__ p, int64_t off, bool keep,
                                          RowRegs<T, MODE_ALIGNED, 1>& r) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + off));
#pragma unroll
    for (int w = 0; w < 4; ++w) r.w[0][w] = keep ? v[w] : 0u;
}

// Per-thread setup of the flat kernels, kept short: every workgroup runs it before its first
// load.  The group size is a constant, there is one column block, the tiles keep the hardware's
// workgroup numbering (narrow rows stream faster with it), and the parameters are loaded
// branch-free.
template <typename T, typename PT, int TPR>
struct FlatCtx {
    static constexpr int V = Elems<T, MODE_ALIGNED>::value;
    int slot, lane;
    bool lane_in;        // this lane holds a chunk of its row
    int64_t col;         // column of the chunk (0 for lanes past the row)
    int64_t rows_per_tile, t_begin, t_end, t_step, wg;
    ColMap<T, MODE_ALIGNED, 1> cm;
    __device__ __forceinline__ FlatCtx(const Geom& g) {
        slot = threadIdx.x / TPR;
        lane = threadIdx.x % TPR;
        wg = blockIdx.x;
        rows_per_tile = g.rpp;
        if (g.strided) {
            t_begin = wg;
            t_end = g.ntiles;
            t_step = gridDim.x;
        } else {
            t_begin = wg * g.kt;
            t_end = t_begin + g.kt < g.ntiles ? t_begin + g.kt : g.ntiles;
            t_step = 1;
        }
        cm.init(lane, TPR, g.N, 0, 0);
        lane_in = cm.any[0];
        col = lane_in ? cm.col0[0] : 0;
    }
    // V parameters of this lane's columns (`dflt` for a NULL vector), 0 past the row.
    __device__ __forceinline__ void param(const PT* __restrict__ p, float dflt, float* o) const {
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const float val = p ? to_f32(p[col + v]) : dflt;
            o[v] = lane_in ? val : 0.f;
        }
    }
};

// The requested LayerNorm partial rows of a flat workgroup (PG bit 0: dgamma at out_g, bit 1:
// dbeta at out_b, column stride cs) in one combine: the gradients' butterflies interleave and
// share one LDS round, so the workgroup's tail pays the latency once.  The order is
// write_partial's for narrow rows: an xor butterfly over the wave's row slots, then the waves'
// sums in wave order.
// V: elements per lane (a 16-byte chunk's unless given).
template <typename T, int TPR, int PG, int V = Elems<T, MODE_ALIGNED>::value>
__device__ __forceinline__ void write_partial_pair(float* __restrict__ out_g, float* __restrict__ out_b,
                                                   int64_t cs, const float* acc_g, const float* acc_b,
                                                   int lane, bool lane_in, int64_t col, float* part) {
    constexpr int NGR = ((PG & 1) ? 1 : 0) + ((PG & 2) ? 1 : 0);
    constexpr int E = NGR * V;
    const int nb = blockDim.x;
    float v[E];
#pragma unroll
    for (int e = 0; e < V; ++e) {
        if constexpr (PG & 1) v[e] = acc_g[e];
        if constexpr (PG & 2) v[(PG & 1 ? V : 0) + e] = acc_b[e];
    }
    if constexpr (TPR < 64) {
        const int wl = nb < 64 ? nb : 64;
        for (int off = TPR; off < wl; off <<= 1) {
#pragma unroll
            for (int e = 0; e < E; ++e) v[e] += __shfl_xor(v[e], off, 64);
        }
    }
    const int nw = (nb + 63) >> 6;
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) < TPR) {
#pragma unroll
        for (int e = 0; e < E; ++e) part[(wave * TPR + lane) * E + e] = v[e];
    }
    __syncthreads();
    if (threadIdx.x < TPR && lane_in) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float sum = part[lane * E + e];
            for (int w = 1; w < nw; ++w) sum += part[(w * TPR + lane) * E + e];
            const bool to_g = (PG & 1) && e < V;
            if (to_g) out_g[(col + e) * cs] = sum;
            else out_b[(col + e - ((PG & 1) ? V : 0)) * cs] = sum;
        }
    }
}

// Mean and rstd of one row from its lanes' chunks (lanes past the row hold zeros).
template <typename T, int TPR>
__device__ __forceinline__ void ln_stats_flat(const RowRegs<T, MODE_ALIGNED, 1>& xr, bool lane_in,
                                              const Geom& g, float eps, float& mu, float& rs) {
    constexpr int V = Elems<T, MODE_ALIGNED>::value;
    float a = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) a += xr.get(0, v);
    mu = group_sum(a, TPR) * g.inv_n;
    a = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const float d = xr.get(0, v) - mu;
        a += lane_in ? d * d : 0.f;
    }
    rs = __builtin_amdgcn_rsqf(group_sum(a, TPR) * g.inv_n + eps);
}

template <typename T, typename PT, int TPR>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, 256)))
ln_fwd_flat_kernel(const T* __restrict__ x, const PT* __restrict__ gamma, const PT* __restrict__ beta,
                   float eps, T* __restrict__ y, float* __restrict__ mean_out,
                   float* __restrict__ rstd_out, Geom g) {
    constexpr int V = Elems<T, MODE_ALIGNED>::value;
    const FlatCtx<T, PT, TPR> c(g);
    float ga[V], be[V];
    c.param(gamma, 1.f, ga);
    c.param(beta, 0.f, be);
    const bool lane_in = c.lane_in;
    const int64_t col = c.col;
    for (int64_t tile = c.t_begin; tile < c.t_end; tile += c.t_step) {
        const int64_t row = tile * c.rows_per_tile + c.slot;
        const bool ok = row < g.M;
        RowRegs<T, MODE_ALIGNED, 1> xr;
        load_flat<T>(x, (ok ? row : g.M - 1) * g.N + col, lane_in, xr);
        float mu, rs;
        ln_stats_flat<T, TPR>(xr, lane_in, g, eps, mu, rs);
        float o[V];
#pragma unroll
        for (int v = 0; v < V; ++v) o[v] = __builtin_fmaf((xr.get(0, v) - mu) * rs, ga[v], be[v]);
        if (ok && lane_in)
            __builtin_nontemporal_store(pack_chunk<T>(o), reinterpret_cast<u32x4*>(y + row * g.N + col));
        if (ok && c.lane == 0) {
            if (mean_out) mean_out[row] = mu;
            if (rstd_out) rstd_out[row] = rs;
        }
    }
}

// ST: the forward's statistics are given (1) or recomputed from x (0).
template <typename T, typename PT, int TPR, int PG, int ST>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, 256)))
ln_bwd_flat_kernel(const T* __restrict__ x, const T* __restrict__ dy, const float* __restrict__ mean_in,
                   const float* __restrict__ rstd_in, const PT* __restrict__ gamma, float eps,
                   T* __restrict__ dx, float* __restrict__ ws, Geom g) {
    constexpr int V = Elems<T, MODE_ALIGNED>::value;
    extern __shared__ float part[];
    const FlatCtx<T, PT, TPR> c(g);
    float ga[V];
    c.param(gamma, 1.f, ga);
    const bool lane_in = c.lane_in;
    const int64_t col = c.col;
    float acc_g[V], acc_b[V];
#pragma unroll
    for (int v = 0; v < V; ++v) acc_g[v] = acc_b[v] = 0.f;
    for (int64_t tile = c.t_begin; tile < c.t_end; tile += c.t_step) {
        const int64_t row = tile * c.rows_per_tile + c.slot;
        const bool ok = row < g.M;
        const int64_t lr = ok ? row : g.M - 1;
        RowRegs<T, MODE_ALIGNED, 1> xr, gr;
        load_flat<T>(x, lr * g.N + col, lane_in && ok, xr);
        load_flat<T>(dy, lr * g.N + col, lane_in && ok, gr);
        float mu, rs;
        if constexpr (ST) {
            mu = mean_in[lr];
            rs = rstd_in[lr];
        } else {
            ln_stats_flat<T, TPR>(xr, lane_in, g, eps, mu, rs);
        }
        mu = ok ? mu : 0.f;
        rs = ok ? rs : 0.f;
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const float xh = (xr.get(0, v) - mu) * rs;
            const float gg = gr.get(0, v) * ga[v];
            a += gg;
            b = __builtin_fmaf(gg, xh, b);
        }
        const float c1 = group_sum(a, TPR) * g.inv_n, c2 = group_sum(b, TPR) * g.inv_n;
        float o[V];
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const float gv = gr.get(0, v);
            const float xh = (xr.get(0, v) - mu) * rs;
            if constexpr (PG & 1) acc_g[v] = __builtin_fmaf(gv, xh, acc_g[v]);
            if constexpr (PG & 2) acc_b[v] += gv;
            o[v] = rs * (gv * ga[v] - c1 - xh * c2);
        }
        if (ok && lane_in)
            __builtin_nontemporal_store(pack_chunk<T>(o), reinterpret_cast<u32x4*>(dx + row * g.N + col));
    }
    if constexpr (PG != 0) {
        float* out = ws + c.wg * g.ws_rs;
        write_partial_pair<T, TPR, PG>(out, out + g.N * g.ws_cs, g.ws_cs, acc_g, acc_b, c.lane, c.lane_in,
                                       c.col, part);
    }
}

// ------------------------------------------- flat LayerNorm kernels with 12-byte lane chunks
// Rows of 12 * TPR bytes (TPR a power of two up to 64: float32 N = 3 * TPR, 16-bit N = 6 * TPR),
// such as the [*, 24] float32 rows of the pages' LayerNorm shape.  In 16-byte chunks such a row
// takes 3 * TPR / 4 lanes of a TPR-lane group, a quarter of the lanes idle; in 12-byte chunks
// (three 32-bit words, loaded and stored whole) every lane of the group holds data, so a wave's
// access is one contiguous run of 12 * 64 bytes with every lane live.  Three-word accesses need
// only 4-byte alignment.  The arithmetic and its order are the 16-byte flat kernels', with
// 12 / sizeof(T) elements per lane instead of 16 / sizeof(T).
typedef uint32_t u32x3 __attribute__((ext_vector_type(3), aligned(4)));

template <typename T>
struct Words12 {
    static constexpr int V = 12 / (int)sizeof(T);
    uint32_t w[3];
    __device__ __forceinline__ float get(int v) const {
        if constexpr (sizeof(T) == 4) {
            return __builtin_bit_cast(float, w[v]);
        } else {
            const uint32_t u = w[v >> 1];
            if constexpr (std::is_same<T, bf16_t>::value)
                return __builtin_bit_cast(float, (v & 1) ? (u & 0xFFFF0000u) : (u << 16));
            else
                return half_bits_to_f32<T>((v & 1) ? (u >> 16) : u);
        }
    }
    // The 12 bytes at p (4-byte aligned); zeros where `keep` is false.
    __device__ __forceinline__ void load(const T* __restrict__ p, bool keep) {
        const u32x3 v = __builtin_nontemporal_load(reinterpret_cast<const u32x3*>(p));
#pragma unroll
        for (int i = 0; i < 3; ++i) w[i] = keep ? v[i] : 0u;
    }
};

// V float32 values rounded to T, stored as the 12 bytes at p.
template <typename T>
__device__ __forceinline__ void store12(T* __restrict__ p, const float* o) {
    u32x3 v;
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int i = 0; i < 3; ++i) v[i] = __builtin_bit_cast(uint32_t, o[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const T lo = from_f32<T>(o[2 * i]), hi = from_f32<T>(o[2 * i + 1]);
            v[i] = (uint32_t)__builtin_bit_cast(unsigned short, lo) |
                   ((uint32_t)__builtin_bit_cast(unsigned short, hi) << 16);
        }
    }
    __builtin_nontemporal_store(v, reinterpret_cast<u32x3*>(p));
}

// Forward.  A wave takes RT * (64 / TPR) consecutive rows per tile (RT steps of 64 / TPR rows,
// every step's loads issued first), then writes the tile's means and rstds with one store each
// from its first RT * 64 / TPR lanes: the statistics leave as whole runs rather than one 4-byte
// store per row group (LayerNorm 401408 x 24 float32 in 12-byte chunks, measured in a probe:
// 15.7 us with per-row-group statistics stores, 15.3-15.4 us with the wave tiles' coalesced
// ones).  A workgroup's tile is its waves' tiles, in wave order.
template <typename T, typename PT, int TPR, int RT>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, 256)))
ln_fwd_flat12_kernel(const T* __restrict__ x, const PT* __restrict__ gamma, const PT* __restrict__ beta,
                     float eps, T* __restrict__ y, float* __restrict__ mean_out,
                     float* __restrict__ rstd_out, Geom g) {
    constexpr int V = Words12<T>::V;
    constexpr int R = 64 / TPR;      // rows per wave and step
    static_assert(RT * R <= 64, "a wave's tile statistics fit its lanes");
    const int wl = threadIdx.x & 63, grp = wl / TPR, lane = wl % TPR;
    const int wave = threadIdx.x >> 6;
    const int64_t col = (int64_t)lane * V;
    float ga[V], be[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        ga[v] = gamma ? to_f32(gamma[col + v]) : 1.f;
        be[v] = beta ? to_f32(beta[col + v]) : 0.f;
    }
    // Lane wl keeps the statistics of its wave tile's row wl: step wl / R, row group wl % R.
    const int src = (wl % R) * TPR * 4;   // ds_bpermute byte address of a lane of that group
    const int keep_step = wl / R;
    const int64_t rows_per_tile = g.rpp * RT;
    for (int64_t tile = blockIdx.x; tile < g.ntiles; tile += gridDim.x) {
        const int64_t base = tile * rows_per_tile + (int64_t)wave * (RT * R);
        Words12<T> xr[RT];
#pragma unroll
        for (int j = 0; j < RT; ++j) {
            const int64_t row = base + j * R + grp;
            xr[j].load(x + (row < g.M ? row : g.M - 1) * g.N + col, true);
        }
        // Every step's outputs are formed before the first store: a store issued between two
        // steps would hold the next step's wait for its loads until the store, too, completed
        // (one counter covers both).
        float mk = 0.f, rk = 0.f;
        float o[RT][V];
#pragma unroll
        for (int j = 0; j < RT; ++j) {
            float a = 0.f;
#pragma unroll
            for (int v = 0; v < V; ++v) a += xr[j].get(v);
            const float mu = group_sum(a, TPR) * g.inv_n;
            a = 0.f;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const float d = xr[j].get(v) - mu;
                a += d * d;
            }
            const float rs = __builtin_amdgcn_rsqf(group_sum(a, TPR) * g.inv_n + eps);
#pragma unroll
            for (int v = 0; v < V; ++v) o[j][v] = __builtin_fmaf((xr[j].get(v) - mu) * rs, ga[v], be[v]);
            const float m = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, mu)));
            const float r = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, rs)));
            if (keep_step == j) {
                mk = m;
                rk = r;
            }
        }
#pragma unroll
        for (int j = 0; j < RT; ++j) {
            const int64_t row = base + j * R + grp;
            if (row < g.M) store12<T>(y + row * g.N + col, o[j]);
        }
        const int64_t srow = base + wl;
        if (wl < RT * R && srow < g.M) {
            if (mean_out) mean_out[srow] = mk;
            if (rstd_out) rstd_out[srow] = rk;
        }
    }
}

// Backward stage 1 (ST: statistics given or recomputed), one row per lane group and step; the
// partial rows as in the 16-byte flat backward.
template <typename T, typename PT, int TPR, int PG, int ST>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, 256)))
ln_bwd_flat12_kernel(const T* __restrict__ x, const T* __restrict__ dy, const float* __restrict__ mean_in,
                     const float* __restrict__ rstd_in, const PT* __restrict__ gamma, float eps,
                     T* __restrict__ dx, float* __restrict__ ws, Geom g) {
    constexpr int V = Words12<T>::V;
    constexpr int R = 64 / TPR;
    extern __shared__ float part[];
    const int wl = threadIdx.x & 63, grp = wl / TPR, lane = wl % TPR;
    const int wave = threadIdx.x >> 6;
    const int64_t col = (int64_t)lane * V;
    float ga[V];
#pragma unroll
    for (int v = 0; v < V; ++v) ga[v] = gamma ? to_f32(gamma[col + v]) : 1.f;
    float acc_g[V], acc_b[V];
#pragma unroll
    for (int v = 0; v < V; ++v) acc_g[v] = acc_b[v] = 0.f;
    for (int64_t tile = blockIdx.x; tile < g.ntiles; tile += gridDim.x) {
        const int64_t row = tile * g.rpp + (int64_t)wave * R + grp;
        const bool ok = row < g.M;
        const int64_t lr = ok ? row : g.M - 1;
        Words12<T> xr, gr;
        xr.load(x + lr * g.N + col, ok);
        gr.load(dy + lr * g.N + col, ok);
        float mu, rs;
        if constexpr (ST) {
            mu = mean_in[lr];
            rs = rstd_in[lr];
        } else {
            float a = 0.f;
#pragma unroll
            for (int v = 0; v < V; ++v) a += xr.get(v);
            mu = group_sum(a, TPR) * g.inv_n;
            a = 0.f;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const float d = xr.get(v) - mu;
                a += d * d;
            }
            rs = __builtin_amdgcn_rsqf(group_sum(a, TPR) * g.inv_n + eps);
        }
        mu = ok ? mu : 0.f;
        rs = ok ? rs : 0.f;
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const float xh = (xr.get(v) - mu) * rs;
            const float gg = gr.get(v) * ga[v];
            a += gg;
            b = __builtin_fmaf(gg, xh, b);
        }
        const float c1 = group_sum(a, TPR) * g.inv_n, c2 = group_sum(b, TPR) * g.inv_n;
        float o[V];
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const float gv = gr.get(v);
            const float xh = (xr.get(v) - mu) * rs;
            if constexpr (PG & 1) acc_g[v] = __builtin_fmaf(gv, xh, acc_g[v]);
            if constexpr (PG & 2) acc_b[v] += gv;
            o[v] = rs * (gv * ga[v] - c1 - xh * c2);
        }
        if (ok) store12<T>(dx + row * g.N + col, o);
    }
    if constexpr (PG != 0) {
        float* out = ws + blockIdx.x * g.ws_rs;
        write_partial_pair<T, TPR, PG, V>(out, out + g.N * g.ws_cs, g.ws_cs, acc_g, acc_b, lane, true, col, part);
    }
}

// DyT in 12-byte lane chunks (rows of 12 * 2^k bytes: float32 N = 3 * 2^k, 16-bit N = 6 * 2^k),
// the row and tile layout of the 12-byte LayerNorm kernels above.  The per-element arithmetic is
// the general DyT kernels' (tanh_only, tanh_sech2, the same sums in the same order per lane).
template <typename T, typename PT, int TPR, int RT>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, 256)))
dyt_fwd_flat12_kernel(const T* __restrict__ x, const PT* __restrict__ alpha_p, const PT* __restrict__ gamma,
                      const PT* __restrict__ beta, T* __restrict__ y, Geom g) {
    constexpr int V = Words12<T>::V;
    constexpr int R = 64 / TPR;      // rows per wave and step
    const int wl = threadIdx.x & 63, grp = wl / TPR, lane = wl % TPR;
    const int wave = threadIdx.x >> 6;
    const int64_t col = (int64_t)lane * V;
    float ga[V], be[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        ga[v] = to_f32(gamma[col + v]);
        be[v] = to_f32(beta[col + v]);
    }
    const float alpha = to_f32(alpha_p[0]);
    const int64_t rows_per_tile = g.rpp * RT;
    for (int64_t tile = blockIdx.x; tile < g.ntiles; tile += gridDim.x) {
        const int64_t base = tile * rows_per_tile + (int64_t)wave * (RT * R);
        Words12<T> xr[RT];
#pragma unroll
        for (int j = 0; j < RT; ++j) {
            const int64_t row = base + j * R + grp;
            xr[j].load(x + (row < g.M ? row : g.M - 1) * g.N + col, true);
        }
        // every step's outputs before the first store (see ln_fwd_flat12_kernel)
        float o[RT][V];
#pragma unroll
        for (int j = 0; j < RT; ++j)
#pragma unroll
            for (int v = 0; v < V; ++v) o[j][v] = __builtin_fmaf(ga[v], tanh_only(alpha * xr[j].get(v)), be[v]);
#pragma unroll
        for (int j = 0; j < RT; ++j) {
            const int64_t row = base + j * R + grp;
            if (row < g.M) store12<T>(y + row * g.N + col, o[j]);
        }
    }
}

// Backward stage 1 (PG 0: dx only), one row per lane group and step.  Partial row blockIdx.x:
// dgamma | dbeta through the LDS combine of the 12-byte LayerNorm backward, dalpha (column 2N)
// as the workgroup's sum.  With a finite alpha a row past M (x = dy = 0) adds exactly 0; with
// alpha = +-inf its terms are dropped after the arithmetic, as in the general kernels.
template <typename T, typename PT, int TPR, int PG>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, 256)))
dyt_bwd_flat12_kernel(const T* __restrict__ x, const T* __restrict__ dy, const PT* __restrict__ alpha_p,
                      const PT* __restrict__ gamma, T* __restrict__ dx, float* __restrict__ ws, Geom g) {
    constexpr int V = Words12<T>::V;
    constexpr int R = 64 / TPR;
    extern __shared__ float part[];
    __shared__ float red[kRedFloats];
    const int wl = threadIdx.x & 63, grp = wl / TPR, lane = wl % TPR;
    const int wave = threadIdx.x >> 6;
    const int64_t col = (int64_t)lane * V;
    float ga[V];
#pragma unroll
    for (int v = 0; v < V; ++v) ga[v] = to_f32(gamma[col + v]);
    const float alpha = to_f32(alpha_p[0]);
    const bool finite_alpha = __builtin_isfinite(alpha);
    float acc_g[V], acc_b[V], acc_a = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) acc_g[v] = acc_b[v] = 0.f;
    for (int64_t tile = blockIdx.x; tile < g.ntiles; tile += gridDim.x) {
        const int64_t row = tile * g.rpp + (int64_t)wave * R + grp;
        const bool ok = row < g.M;
        const int64_t lr = ok ? row : g.M - 1;
        Words12<T> xr, gr;
        xr.load(x + lr * g.N + col, ok);
        gr.load(dy + lr * g.N + col, ok);
        float o[V];
        if (finite_alpha) {
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const float xv = xr.get(v), gv = gr.get(v);
                const TanhSech2 ts = tanh_sech2(alpha * xv);
                const float ds = gv * ga[v] * ts.s;   // dy * gamma * sech^2
                if constexpr (PG) {
                    acc_g[v] = __builtin_fmaf(gv, ts.t, acc_g[v]);
                    acc_b[v] += gv;
                    acc_a = __builtin_fmaf(xv, ds, acc_a);
                }
                o[v] = alpha * ds;
            }
        } else {
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const float xv = xr.get(v), gv = gr.get(v);
                const TanhSech2 ts = tanh_sech2(alpha * xv);
                const float d = gv * ga[v];
                const float as = ts.s == 0.f ? 0.f : alpha * ts.s;
                if constexpr (PG) {
                    acc_g[v] += ok ? gv * ts.t : 0.f;
                    acc_b[v] += ok ? gv : 0.f;
                    acc_a += ok ? d * xv * ts.s : 0.f;
                }
                o[v] = d * as;
            }
        }
        if (ok) store12<T>(dx + row * g.N + col, o);
    }
    if constexpr (PG != 0) {
        float* out = ws + blockIdx.x * g.ws_rs;
        write_partial_pair<T, TPR, 3, V>(out, out + g.N * g.ws_cs, g.ws_cs, acc_g, acc_b, lane, true, col, part);
        const float da = block_sum(acc_a, red);
        if (threadIdx.x == 0) out[2 * g.N * g.ws_cs] = da;
    }
}

// ============================================================================== RMSNorm

template <typename T, int MODE, int CPT, int RT>
__device__ __forceinline__ void rms_stats(const RowRegs<T, MODE, CPT> (&xr)[RT], const Geom& g,
                                          float eps, float* red, int& parity, float (&rs)[RT]) {
    constexpr int V = Elems<T, MODE>::value;
    float s[RT];
#pragma unroll
    for (int u = 0; u < RT; ++u) {
        float a = 0.f;
#pragma unroll
        for (int k = 0; k < CPT; ++k)
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const float xv = xr[u].get(k, v);
                a = __builtin_fmaf(xv, xv, a);
            }
        s[u] = a;
    }
    row_sum<RT>(s, g.tpr, red, parity);
#pragma unroll
    for (int u = 0; u < RT; ++u) rs[u] = __builtin_amdgcn_rsqf(s[u] * g.inv_n + eps);
}

// VAR 0: the Llama form (normalized value rounded to x's dtype, then the weight multiply);
// VAR 1: weight (plus g.w_offset) times the float32 normalized value, rounded once.
template <typename T, typename PT, int MODE, int CPT, int RT, int PF, int VAR, int LAY>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, MaxBlock<T, RT, CPT>::value)))
rms_fwd_kernel(const T* __restrict__ x, const PT* __restrict__ weight, float eps,
               T* __restrict__ y, float* __restrict__ rstd_out, Geom g) {
    constexpr int V = Elems<T, MODE>::value;
    constexpr int E = CPT * V;
    __shared__ float red[kRedFloats];
    int parity = 0;
    RowCtx<T, MODE, CPT, RT> c(g);
    float w[E];
    load_param<T, PT, MODE, CPT>(weight, g.N, g.ps0, c.cm, w);
    if constexpr (VAR != 0) {
#pragma unroll
        for (int e = 0; e < E; ++e) w[e] += g.w_offset;   // (1 + weight) in float32
    }
    struct In {
        RowRegs<T, MODE, CPT> xr[RT];
        int64_t row[RT];
        int64_t row0;
        bool ok[RT];
    };
    auto fetch = [&](int64_t tile, In& in) {
        c.tile_rows(tile, g, in.row, in.ok);
        const int64_t row0 = tile * c.rows_per_tile;
        in.row0 = row0;
        const TileSrc sx = tile_src<T, MODE, LAY>(x, row0, g, OP_X, tile < c.t_end);
#pragma unroll
        for (int u = 0; u < RT; ++u) load_row<T, MODE, CPT>(sx, row_base<LAY>(g, OP_X, in.row[u]), c.cm, in.ok[u], in.xr[u]);
    };
    auto body = [&](const In& in) {
        const auto& xr = in.xr;
        const auto& ok = in.ok;
        const auto& row = in.row;
        float rs[RT];
        rms_stats<T, MODE, CPT, RT>(xr, g, eps, red, parity, rs);
#pragma unroll
        for (int u = 0; u < RT; ++u) {
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                float o[V];
                // VAR 0: one rounding of the normalized value to x's dtype, then the weight
                // multiply in float32.  VAR 1: the float32 product of the weight and the
                // unrounded normalized value.  The store rounds the product to x's dtype.
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    const float h = xr[u].get(k, v) * rs[u];
                    o[v] = w[k * V + v] * (VAR == 0 ? round_through<T>(h) : h);
                }
                store_chunk<T, MODE, CPT>(y, row_base<LAY>(g, OP_OUT, row[u]), g.N, c.cm, k, o, ok[u]);
            }
            if (ok[u] && c.lane == 0 && rstd_out) rstd_out[row[u]] = rs[u];
        }
    };
    tile_loop<PF, In>(c, fetch, body);
}

// Resident waves per SIMD the RMSNorm backward is compiled for: the SHIFTED one-chunk shape
// (N = 1025 bf16) fits five when it keeps to 96 VGPRs (one more register costs a wave:
// 87.8 vs 90.8 us); other shapes are left to the compiler.
template <int MODE, int CPT> struct RmsBwdWaves {
    static constexpr int value = (MODE == MODE_SHIFTED && CPT == 1) ? 5 : 1;
};

template <typename T, typename PT, int MODE, int CPT, int RT, int PF, int VAR, int PG, int LAY>
__global__ void __attribute__((amdgpu_flat_work_group_size(1, MaxBlock<T, RT, CPT>::value),
                               amdgpu_waves_per_eu(RmsBwdWaves<MODE, CPT>::value)))
rms_bwd_kernel(const T* __restrict__ x, const T* __restrict__ dy, const float* __restrict__ rstd_in,
               const PT* __restrict__ weight, float eps, T* __restrict__ dx,
               float* __restrict__ ws, Geom g) {
    constexpr int V = Elems<T, MODE>::value;
    constexpr int E = CPT * V;
    extern __shared__ float part[];
    __shared__ float red[kRedFloats];
    int parity = 0;
    RowCtx<T, MODE, CPT, RT> c(g);
    float w[E];
    load_param<T, PT, MODE, CPT>(weight, g.N, g.ps0, c.cm, w);
    if constexpr (VAR != 0) {
#pragma unroll
        for (int e = 0; e < E; ++e) w[e] += g.w_offset;   // (1 + weight) in float32
    }
    float acc_w[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc_w[e] = 0.f;

    struct In {
        RowRegs<T, MODE, CPT> xr[RT], gr[RT];
        int64_t row[RT];
        int64_t row0;
        bool ok[RT];
        float rs[RT];
    };
    auto fetch = [&](int64_t tile, In& in) {
        c.tile_rows(tile, g, in.row, in.ok);
        const int64_t row0 = tile * c.rows_per_tile;
        in.row0 = row0;
        const bool live = tile < c.t_end;
        const TileSrc sx = tile_src<T, MODE, LAY>(x, row0, g, OP_X, live);
        const TileSrc sg = tile_src<T, MODE, LAY>(dy, row0, g, OP_DY, live);
        const Rsrc sr = stats_src(rstd_in, row0, g.M, live);
#pragma unroll
        for (int u = 0; u < RT; ++u) {
            load_row<T, MODE, CPT>(sx, row_base<LAY>(g, OP_X, in.row[u]), c.cm, in.ok[u], in.xr[u]);
            load_row<T, MODE, CPT>(sg, row_base<LAY>(g, OP_DY, in.row[u]), c.cm, in.ok[u], in.gr[u]);
            in.rs[u] = load_stat(sr, in.row[u], row0, in.ok[u]);
        }
    };
    auto body = [&](const In& in) {
        const auto& xr = in.xr;
        const auto& gr = in.gr;
        const auto& ok = in.ok;
        const auto& row = in.row;
        constexpr bool BUF = kBufferStores<MODE, CPT, true>;
        const TileSrc dst = tile_src<T, MODE, LAY>(dx, in.row0, g, OP_OUT, true);
        float rs[RT];
#pragma unroll
        for (int u = 0; u < RT; ++u) rs[u] = in.rs[u];
        if (!rstd_in) rms_stats<T, MODE, CPT, RT>(xr, g, eps, red, parity, rs);
        // Padded elements read x = dy = 0, so their terms are 0 as long as x * rstd is finite:
        // a padded row's rstd is zeroed (a recomputed one is infinite with eps = 0).
#pragma unroll
        for (int u = 0; u < RT; ++u) rs[u] = ok[u] ? rs[u] : 0.f;
        float s[RT];
#pragma unroll
        for (int u = 0; u < RT; ++u) {
            float a = 0.f;
#pragma unroll
            for (int k = 0; k < CPT; ++k)
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    // grad of the normalized value: the float32 product, rounded to x's dtype
                    // in the Llama form (where the normalized value itself was rounded).
                    const float p = gr[u].get(k, v) * w[k * V + v];
                    const float gg = VAR == 0 ? round_through<T>(p) : p;
                    a = __builtin_fmaf(gg, xr[u].get(k, v) * rs[u], a);
                }
            s[u] = a;
        }
        row_sum<RT>(s, g.tpr, red, parity);
#pragma unroll
        for (int u = 0; u < RT; ++u) {
            const float cc = s[u] * g.inv_n;
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                float o[V];
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    const int e = k * V + v;
                    const float gv = gr[u].get(k, v);
                    const float h = xr[u].get(k, v) * rs[u];
                    const float gg = VAR == 0 ? round_through<T>(gv * w[e]) : gv * w[e];
                    // weight-gradient term.  Llama form: dy * n, n = h rounded to x's dtype, the
                    // product rounded to the weight's dtype before the sum.  Float32 forms:
                    // dy * h, summed in float32 and rounded once at the end.
                    if constexpr (PG) {
                        const float term = VAR == 0 ? round_through<PT>(gv * round_through<T>(h)) : gv * h;
                        acc_w[e] += term;
                    }
                    o[v] = rs[u] * (gg - h * cc);
                }
                put_chunk<T, MODE, CPT, BUF>(dx, dst, row_base<LAY>(g, OP_OUT, row[u]), g.N, c.cm, k, o, ok[u]);
            }
        }
    };
    tile_loop<PF, In>(c, fetch, body);
    if constexpr (PG) {
        float* out = ws + c.wg * g.ws_rs;
        write_partial<T, MODE, CPT>(out, g.ws_cs, acc_w, c.cm, c.slot, c.lane, g, part);
    }
}

// ============================================================================ stage 2

// Stage 2.  Partial row p, column c is ws[p * rs + c * cs].  Output columns: [0, N) -> out0,
// [N, 2N) -> out1, 2N -> out2[0] (NULL outputs are skipped); only columns [c_lo, c_hi) are
// read.  A workgroup covers cb columns with L = blockDim.x / cb lanes each; lane l adds partial rows l, l + L, ... in order in
// float64, then the L lane sums are added as a fixed tree.  Threads are laid out along the
// contiguous dimension of ws (columns when cs == 1, partial rows otherwise) so loads coalesce.
template <typename PT>
__global__ void __launch_bounds__(512)
colreduce_kernel(const float* __restrict__ ws, int64_t P, int64_t ng, int64_t rs, int64_t cs,
                 int64_t N, int64_t c_lo, int64_t c_hi, int cb, PT* __restrict__ out0,
                 PT* __restrict__ out1, PT* __restrict__ out2) {
    // Columns [2N, ng) are the dalpha partial columns of the column blocks: the lanes of column
    // 2N add all of them (column by column, in order); the others stay idle.
    __shared__ double red[512];
    const int L = blockDim.x / cb;
    const bool col_fast = cs == 1;
    const int cl = col_fast ? (int)(threadIdx.x % cb) : (int)(threadIdx.x / L);
    const int gl = col_fast ? (int)(threadIdx.x / cb) : (int)(threadIdx.x % L);
    const int64_t col = c_lo + (int64_t)blockIdx.x * cb + cl;
    const bool live = col < c_hi && col < ng && col <= 2 * N;
    double acc = 0.0;
    const int64_t c_end = col == 2 * N ? ng : col + 1;
    if (live) {
        for (int64_t cc = col; cc < c_end; ++cc) {
            const float* base = ws + cc * cs;
            int64_t p = gl;
            for (; p + 3 * L < P; p += 4 * L) {
                const float a0 = base[p * rs], a1 = base[(p + L) * rs];
                const float a2 = base[(p + 2 * L) * rs], a3 = base[(p + 3 * L) * rs];
                acc += a0; acc += a1; acc += a2; acc += a3;
            }
            for (; p < P; p += L) acc += base[p * rs];
        }
    }
    red[gl * cb + cl] = acc;
    __syncthreads();
    for (int st = L / 2; st > 0; st >>= 1) {
        if (gl < st) red[gl * cb + cl] += red[(gl + st) * cb + cl];
        __syncthreads();
    }
    if (gl == 0 && live) {
        const PT v = from_f32<PT>((float)red[cl]);
        if (col < N) {
            if (out0) out0[col] = v;
        } else if (col < 2 * N) {
            if (out1) out1[col - N] = v;
        } else {
            if (out2) out2[0] = v;
        }
    }
}

// Stage 2 for column-major partials (rs == 1: column c is ws[c * cs .. c * cs + P)), the
// layout of short rows.  One workgroup per output column from c_lo on: thread t adds partial rows t,
// t + blockDim, ... in order in float64 (all of its loads issued up front), the wave sums
// are formed by a fixed xor butterfly, and thread 0 adds the wave sums in wave order.  The
// dalpha output (column 2N) adds its ncb partial columns [2N, ng) one after another.
template <typename PT>
__global__ void __launch_bounds__(256)
colreduce_cm_kernel(const float* __restrict__ ws, int64_t P, int64_t ng, int64_t cs, int64_t N,
                    int64_t c_lo, PT* __restrict__ out0, PT* __restrict__ out1, PT* __restrict__ out2) {
    __shared__ double wsum[4];
    const int64_t col = c_lo + blockIdx.x;
    const int64_t c_end = col == 2 * N ? ng : col + 1;
    double acc = 0.0;
    for (int64_t cc = col; cc < c_end; ++cc) {
        const float* base = ws + cc * cs;
        int64_t p = threadIdx.x;
        for (; p + 3 * 256 < P; p += 4 * 256) {
            const float a0 = base[p], a1 = base[p + 256], a2 = base[p + 512], a3 = base[p + 768];
            acc += a0; acc += a1; acc += a2; acc += a3;
        }
        for (; p < P; p += 256) acc += base[p];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double s = wsum[0];
        for (int w = 1; w < (int)(blockDim.x >> 6); ++w) s += wsum[w];
        const PT v = from_f32<PT>((float)s);
        if (col < N) {
            if (out0) out0[col] = v;
        } else if (col < 2 * N) {
            if (out1) out1[col - N] = v;
        } else {
            if (out2) out2[0] = v;
        }
    }
}

}  // namespace rwn
