// Split-row kernels: DyT, LayerNorm and RMSNorm forward and backward stage 1 over wide rows
// whose start is not 16-byte aligned, or whose width is not a multiple of a 16-byte chunk.
//
// Each row is cut into
//   head  h = (V - s) mod V elements, up to the first 16-byte boundary inside the row (s: the
//         row start's offset past a 16-byte boundary, in elements),
//   main  nm = floor((N - h) / V) whole 16-byte chunks, aligned,
//   tail  the N - h - nm V elements left over.
// Head and tail (at most 2V - 2 elements together) are scalar slots of the row's first lanes.  A
// row slot of tpr = 64 W lanes (W waves) holds CPT main chunks per lane, chunk c = lane + k tpr,
// and at most one scalar element per lane, so every vector access is a whole aligned chunk of
// the row itself: no chunk is shared with a neighbouring row, nothing is masked inside a chunk,
// and stores are whole 16-byte stores or single elements.  A workgroup holds rpp slots; tile t
// is rows [t rpp, (t + 1) rpp), and workgroup w visits tiles w, w + G, ... with G a multiple of 8,
// so every row a slot visits starts at the same offset s and the slot's column map is fixed for
// the whole kernel (which is what keeps parameters and column partials in registers).
//
// Loads are plain nontemporal global loads; an unused chunk or scalar slot (or a row past M)
// loads an aligned chunk known to lie inside the tensor and is zeroed after the load, so no load
// sits behind a branch.  PF = 1 issues the next tile's loads before the current tile is reduced,
// computed and stored (tile_loop).  The arithmetic is the general kernels'; only the row is cut
// differently.
#pragma once

#include "rwn_kernels.hpp"

namespace rwn {

constexpr int kSplitBlock = 512;
constexpr int kSplitRed = 2 * kMaxWaves * 2;   // row_sum buffers for up to two values per row

// Per-thread column map of a split row slot (fixed for every row the slot visits).
template <typename T, int CPT>
struct SplitCtx {
    static constexpr int V = ChunkOf<T>::value;
    int slot, lane;
    int64_t t_begin, t_end, t_step;   // this workgroup's tiles: t_begin, t_begin + t_step, ... < t_end
    int64_t wg;                // its partial row (backward)
    int h, nm, nrem;           // head elements, main chunks, head + tail elements
    int col[CPT];              // column of element 0 of main chunk k
    bool ok[CPT];              // chunk k exists
    int scol;                  // column of the scalar element
    bool sok;                  // this lane holds one
    int64_t safe;              // an aligned chunk inside the tensor (target of unused loads)

    __device__ __forceinline__ SplitCtx(const Geom& g) {
        slot = threadIdx.x / g.tpr;
        lane = threadIdx.x - slot * g.tpr;
        int64_t b = blockIdx.x;
        if (g.xcd_remap) b = (b % 8) * (gridDim.x / 8) + b / 8;
        wg = b;
        t_begin = b;
        t_end = g.ntiles;
        t_step = gridDim.x;
        const int64_t r0 = t_begin * g.rpp + slot;
        const int s = (int)(((int64_t)g.base_shift + r0 * g.N) % V);
        h = (V - s) % V;
        nm = (int)((g.N - h) / V);
        nrem = (int)(g.N - (int64_t)nm * V);   // head + tail
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            const int c = lane + k * g.tpr;
            ok[k] = c < nm;
            col[k] = h + c * V;
        }
        sok = lane < nrem;
        scol = lane < h ? lane : lane + nm * V;   // tail element lane - h sits at h + nm V + (lane - h)
        safe = (V - g.base_shift) % V;
    }
    __device__ __forceinline__ int64_t row(int64_t tile, const Geom& g) const { return tile * g.rpp + slot; }
};

// One row slice of a split slot: CPT whole chunks and one scalar element (raw storage bits).
template <typename T, int CPT>
struct SplitRow {
    u32x4 c[CPT];
    uint32_t s;

    __device__ __forceinline__ float get(int k, int v) const {
        if constexpr (sizeof(T) == 4) {
            // The word is copied out of the vector first: __builtin_bit_cast applied directly to
            // a vector element reads element 0 whatever the index (seen with this compiler).
            const uint32_t u = c[k][v];
            return __builtin_bit_cast(float, u);
        } else {
            const uint32_t u = c[k][v >> 1];
            if constexpr (std::is_same<T, bf16_t>::value)
                return __builtin_bit_cast(float, (v & 1) ? (u & 0xFFFF0000u) : (u << 16));
            else
                return half_bits_to_f32<T>((v & 1) ? (u >> 16) : u);
        }
    }
    __device__ __forceinline__ float gets() const {
        if constexpr (sizeof(T) == 4) return __builtin_bit_cast(float, s);
        else return half_bits_to_f32<T>(s);
    }
};

template <typename T, int CPT>
__device__ __forceinline__ void split_load(const T* __restrict__ p, int64_t e0, const SplitCtx<T, CPT>& m,
                                           bool rv, SplitRow<T, CPT>& r) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const bool in = rv && m.ok[k];
        const int64_t e = in ? e0 + m.col[k] : m.safe;
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + e));
#pragma unroll
        for (int w = 0; w < 4; ++w) r.c[k][w] = in ? v[w] : 0u;
    }
    const bool ins = rv && m.sok;
    const int64_t es = ins ? e0 + m.scol : m.safe;
    uint32_t bits;
    if constexpr (sizeof(T) == 4) bits = __builtin_bit_cast(uint32_t, p[es]);
    else bits = (uint32_t)__builtin_bit_cast(unsigned short, p[es]);
    r.s = ins ? bits : 0u;
}

// Discard target of the chunk stores with SINK set: 16 bytes per wave of 64 workgroup numbers.
// Nothing reads it; concurrent kernels may write it at will.
static __device__ __align__(256) u32x4 split_sink[64 * (kSplitBlock / 64)];

// Store of main chunk k.  Without SINK a lane whose chunk does not exist (or whose row is past
// M) skips the store behind a branch; with SINK it stores to split_sink instead, so the store
// is issued on every path.  The compiler can then count the memory operations in flight exactly
// (a store that may or may not have been issued makes it wait for all of them) and schedule the
// arithmetic around the stores.  Measured per kernel, SINK is set where it was faster: DyT
// backwards of two chunks per lane (65536 x N bf16 stage 1: N = 1025 92.7 -> 84.6 us, 4096
// 323.0 -> 292.5) and pipelined LayerNorm backwards of two chunks per lane (N = 2048 135.6 ->
// 130.8); one-chunk LayerNorm / RMSNorm backwards ran far slower with it (N = 1025: 73.8 -> 108.4
// and 70.8 -> 95.1) and forwards no faster.
template <typename T, int CPT, bool SINK = false>
__device__ __forceinline__ void split_store_chunk(T* __restrict__ p, int64_t e0, const SplitCtx<T, CPT>& m, int k,
                                                  const float* o, bool rv) {
    if constexpr (SINK) {
        u32x4* dst = (rv && m.ok[k]) ? reinterpret_cast<u32x4*>(p + e0 + m.col[k])
                                     : split_sink + ((blockIdx.x & 63) * (kSplitBlock / 64) + (threadIdx.x >> 6));
        __builtin_nontemporal_store(pack_chunk<T>(o), dst);
    } else {
        if (rv && m.ok[k]) __builtin_nontemporal_store(pack_chunk<T>(o), reinterpret_cast<u32x4*>(p + e0 + m.col[k]));
    }
}

template <typename T, int CPT>
__device__ __forceinline__ void split_store_scalar(T* __restrict__ p, int64_t e0, const SplitCtx<T, CPT>& m,
                                                   float o, bool rv) {
    if (rv && m.sok) p[e0 + m.scol] = from_f32<T>(o);
}

// Parameters of this lane's columns (dflt for a NULL vector, 0 for unused slots).
template <typename T, typename PT, int CPT>
__device__ __forceinline__ void split_param(const PT* __restrict__ p, float dflt, const SplitCtx<T, CPT>& m,
                                            float* o, float& os) {
    constexpr int V = SplitCtx<T, CPT>::V;
#pragma unroll
    for (int k = 0; k < CPT; ++k)
#pragma unroll
        for (int v = 0; v < V; ++v) o[k * V + v] = m.ok[k] ? (p ? to_f32(p[m.col[k] + v]) : dflt) : 0.f;
    os = m.sok ? (p ? to_f32(p[m.scol]) : dflt) : 0.f;
}

// Writes NG gradients' partial row (gradient n, column j at out[(n N + j) cs]).  With one slot per
// workgroup the slot's lanes write their own columns; otherwise the slots' values are added into
// a column-indexed LDS row `part` (NG * N floats) one slot at a time, in slot order, and the
// workgroup writes it out.
template <typename T, int CPT, int NG>
__device__ __forceinline__ void split_write_partials(float* __restrict__ out, int64_t cs,
                                                     const float (&acc)[NG][CPT * ChunkOf<T>::value],
                                                     const float (&accs)[NG], const SplitCtx<T, CPT>& m,
                                                     const Geom& g, float* part) {
    constexpr int V = SplitCtx<T, CPT>::V;
    if (g.rpp == 1) {
#pragma unroll
        for (int n = 0; n < NG; ++n) {
            float* o = out + (int64_t)n * g.N * cs;
#pragma unroll
            for (int k = 0; k < CPT; ++k)
                if (m.ok[k]) {
#pragma unroll
                    for (int v = 0; v < V; ++v) o[(int64_t)(m.col[k] + v) * cs] = acc[n][k * V + v];
                }
            if (m.sok) o[(int64_t)m.scol * cs] = accs[n];
        }
        return;
    }
    const int nb = blockDim.x;
    const int64_t ncol = (int64_t)NG * g.N;
    __syncthreads();
    for (int64_t j = threadIdx.x; j < ncol; j += nb) part[j] = 0.f;
    for (int sl = 0; sl < g.rpp; ++sl) {
        __syncthreads();
        if (m.slot == sl) {
#pragma unroll
            for (int n = 0; n < NG; ++n) {
                float* pp = part + (int64_t)n * g.N;
#pragma unroll
                for (int k = 0; k < CPT; ++k)
                    if (m.ok[k]) {
#pragma unroll
                        for (int v = 0; v < V; ++v) pp[m.col[k] + v] += acc[n][k * V + v];
                    }
                if (m.sok) pp[m.scol] += accs[n];
            }
        }
    }
    __syncthreads();
    for (int64_t j = threadIdx.x; j < ncol; j += nb) out[j * cs] = part[j];
}

// ================================================================================== DyT

// Row of the tile for this slot, whether it exists (and the tile is one of this workgroup's),
// and its first element.
struct SplitRowPos {
    int64_t row, e0;
    bool rv;
};

template <typename T, int CPT>
__device__ __forceinline__ SplitRowPos split_pos(const SplitCtx<T, CPT>& c, int64_t tile, const Geom& g) {
    SplitRowPos r;
    r.row = c.row(tile, g);
    r.rv = tile < c.t_end && r.row < g.M;
    r.e0 = r.row * g.N;
    return r;
}

template <typename T, typename PT, int CPT, int PF>
__global__ void __launch_bounds__(kSplitBlock)
dyt_fwd_split_kernel(const T* __restrict__ x, const PT* __restrict__ alpha_p, const PT* __restrict__ gamma,
                     const PT* __restrict__ beta, T* __restrict__ y, Geom g) {
    constexpr int V = ChunkOf<T>::value;
    constexpr int E = CPT * V;
    const SplitCtx<T, CPT> c(g);
    float ga[E], be[E], gs, bs;
    split_param<T, PT, CPT>(gamma, 0.f, c, ga, gs);
    split_param<T, PT, CPT>(beta, 0.f, c, be, bs);
    const float alpha = to_f32(alpha_p[0]);
    struct In {
        SplitRow<T, CPT> xr;
        SplitRowPos at;
    };
    auto fetch = [&](int64_t tile, In& in) {
        in.at = split_pos(c, tile, g);
        split_load<T, CPT>(x, in.at.e0, c, in.at.rv, in.xr);
    };
    auto body = [&](const In& in) {
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            float o[V];
#pragma unroll
            for (int v = 0; v < V; ++v) o[v] = __builtin_fmaf(ga[k * V + v], tanh_only(alpha * in.xr.get(k, v)), be[k * V + v]);
            split_store_chunk<T, CPT>(y, in.at.e0, c, k, o, in.at.rv);
        }
        split_store_scalar<T, CPT>(y, in.at.e0, c, __builtin_fmaf(gs, tanh_only(alpha * in.xr.gets()), bs), in.at.rv);
    };
    tile_loop<PF, In>(c, fetch, body);
}

template <typename T, typename PT, int CPT, int PF, int PG>
__global__ void __launch_bounds__(kSplitBlock)
dyt_bwd_split_kernel(const T* __restrict__ x, const T* __restrict__ dy, const PT* __restrict__ alpha_p,
                     const PT* __restrict__ gamma, T* __restrict__ dx, float* __restrict__ ws, Geom g) {
    constexpr int V = ChunkOf<T>::value;
    constexpr int E = CPT * V;
    extern __shared__ float part[];
    __shared__ float red[kSplitRed];
    const SplitCtx<T, CPT> c(g);
    float ga[E], gs;
    split_param<T, PT, CPT>(gamma, 0.f, c, ga, gs);
    const float alpha = to_f32(alpha_p[0]);
    float acc[2][E], accs[2] = {0.f, 0.f}, acc_a = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[0][e] = acc[1][e] = 0.f;
    // With a finite alpha an unused slot (x = dy = gamma = 0) adds exactly 0 to every sum; with
    // alpha = +-inf its z = inf * 0 is NaN, so those terms are dropped after the arithmetic and
    // alpha * sech^2 is taken as 0 where sech^2 is 0.
    const bool finite_alpha = __builtin_isfinite(alpha);
    // one element: returns dx and adds the element's gradient terms (FIN: alpha is finite)
    auto elem = [&](auto fin, float xv, float gv, float gam, bool live, float& ag, float& ab) {
        const TanhSech2 ts = tanh_sech2(alpha * xv);
        const float d = gv * gam;
        if constexpr (decltype(fin)::value) {
            const float ds = d * ts.s;   // dy * gamma * sech^2
            if constexpr (PG) {
                ag = __builtin_fmaf(gv, ts.t, ag);
                ab += gv;
                acc_a = __builtin_fmaf(xv, ds, acc_a);
            }
            return alpha * ds;
        } else {
            const float as = ts.s == 0.f ? 0.f : alpha * ts.s;
            if constexpr (PG) {
                ag += live ? gv * ts.t : 0.f;
                ab += live ? gv : 0.f;
                acc_a += live ? d * xv * ts.s : 0.f;
            }
            return d * as;
        }
    };
    struct In {
        SplitRow<T, CPT> xr, gr;
        SplitRowPos at;
    };
    auto fetch = [&](int64_t tile, In& in) {
        in.at = split_pos(c, tile, g);
        split_load<T, CPT>(x, in.at.e0, c, in.at.rv, in.xr);
        split_load<T, CPT>(dy, in.at.e0, c, in.at.rv, in.gr);
    };
    auto body = [&](const In& in) {
        const bool rv = in.at.rv;
        auto rows = [&](auto fin) {
#pragma unroll
            for (int k = 0; k < CPT; ++k) {
                float o[V];
                const bool live = rv && c.ok[k];
#pragma unroll
                for (int v = 0; v < V; ++v)
                    o[v] = elem(fin, in.xr.get(k, v), in.gr.get(k, v), ga[k * V + v], live, acc[0][k * V + v],
                                acc[1][k * V + v]);
                split_store_chunk<T, CPT, CPT == 2>(dx, in.at.e0, c, k, o, rv);
            }
            const float os = elem(fin, in.xr.gets(), in.gr.gets(), gs, rv && c.sok, accs[0], accs[1]);
            split_store_scalar<T, CPT>(dx, in.at.e0, c, os, rv);
        };
        if (finite_alpha) rows(IC<1>{});
        else rows(IC<0>{});
    };
    tile_loop<PF, In>(c, fetch, body);
    if constexpr (PG) {
        float* out = ws + c.wg * g.ws_rs;
        split_write_partials<T, CPT, 2>(out, g.ws_cs, acc, accs, c, g, part);
        const float da = block_sum(acc_a, red);
        if (threadIdx.x == 0) out[2 * g.N * g.ws_cs] = da;
    }
}

// ============================================================================ LayerNorm

// mean and rstd of one row (two passes over the registers; unused slots hold x = 0 and are
// left out of the squared deviations).
template <typename T, int CPT>
__device__ __forceinline__ void split_ln_stats(const SplitRow<T, CPT>& xr, const SplitCtx<T, CPT>& c, const Geom& g,
                                               float eps, float* red, int& parity, float& mu, float& rs) {
    constexpr int V = SplitCtx<T, CPT>::V;
    float s[1];
    float a = xr.gets();
#pragma unroll
    for (int k = 0; k < CPT; ++k)
#pragma unroll
        for (int v = 0; v < V; ++v) a += xr.get(k, v);
    s[0] = a;
    row_sum<1>(s, g.tpr, red, parity);
    mu = s[0] * g.inv_n;
    const float ds = xr.gets() - mu;
    a = c.sok ? ds * ds : 0.f;
#pragma unroll
    for (int k = 0; k < CPT; ++k)
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const float d = xr.get(k, v) - mu;
            a += c.ok[k] ? d * d : 0.f;
        }
    s[0] = a;
    row_sum<1>(s, g.tpr, red, parity);
    rs = __builtin_amdgcn_rsqf(s[0] * g.inv_n + eps);
}

template <typename T, typename PT, int CPT, int PF>
__global__ void __launch_bounds__(kSplitBlock)
ln_fwd_split_kernel(const T* __restrict__ x, const PT* __restrict__ gamma, const PT* __restrict__ beta, float eps,
                    T* __restrict__ y, float* __restrict__ mean_out, float* __restrict__ rstd_out, Geom g) {
    constexpr int V = ChunkOf<T>::value;
    constexpr int E = CPT * V;
    __shared__ float red[kSplitRed];
    int parity = 0;
    const SplitCtx<T, CPT> c(g);
    float ga[E], be[E], gs, bs;
    split_param<T, PT, CPT>(gamma, 1.f, c, ga, gs);
    split_param<T, PT, CPT>(beta, 0.f, c, be, bs);
    struct In {
        SplitRow<T, CPT> xr;
        SplitRowPos at;
    };
    auto fetch = [&](int64_t tile, In& in) {
        in.at = split_pos(c, tile, g);
        split_load<T, CPT>(x, in.at.e0, c, in.at.rv, in.xr);
    };
    auto body = [&](const In& in) {
        float mu, rs;
        split_ln_stats<T, CPT>(in.xr, c, g, eps, red, parity, mu, rs);
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            float o[V];
#pragma unroll
            for (int v = 0; v < V; ++v)
                o[v] = __builtin_fmaf((in.xr.get(k, v) - mu) * rs, ga[k * V + v], be[k * V + v]);
            split_store_chunk<T, CPT>(y, in.at.e0, c, k, o, in.at.rv);
        }
        split_store_scalar<T, CPT>(y, in.at.e0, c, __builtin_fmaf((in.xr.gets() - mu) * rs, gs, bs), in.at.rv);
        if (in.at.rv && c.lane == 0) {
            if (mean_out) mean_out[in.at.row] = mu;
            if (rstd_out) rstd_out[in.at.row] = rs;
        }
    };
    tile_loop<PF, In>(c, fetch, body);
}

template <typename T, typename PT, int CPT, int PF, int PG>
__global__ void __launch_bounds__(kSplitBlock)
ln_bwd_split_kernel(const T* __restrict__ x, const T* __restrict__ dy, const float* __restrict__ mean_in,
                    const float* __restrict__ rstd_in, const PT* __restrict__ gamma, float eps,
                    T* __restrict__ dx, float* __restrict__ ws, Geom g) {
    constexpr int V = ChunkOf<T>::value;
    constexpr int E = CPT * V;
    extern __shared__ float part[];
    __shared__ float red[kSplitRed];
    int parity = 0;
    const SplitCtx<T, CPT> c(g);
    float ga[E], gs;
    split_param<T, PT, CPT>(gamma, 1.f, c, ga, gs);
    const bool have_stats = mean_in != nullptr && rstd_in != nullptr;
    // PG bit 0: dgamma partials (acc[0]), bit 1: dbeta partials (acc[IB])
    constexpr int NGR = (PG & 1) + ((PG >> 1) & 1) > 0 ? (PG & 1) + ((PG >> 1) & 1) : 1;
    constexpr int IB = (PG & 1) ? 1 : 0;
    float acc[NGR][E], accs[NGR];
#pragma unroll
    for (int n = 0; n < NGR; ++n) {
        accs[n] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[n][e] = 0.f;
    }
    struct In {
        SplitRow<T, CPT> xr, gr;
        SplitRowPos at;
        float mu, rs;
    };
    auto fetch = [&](int64_t tile, In& in) {
        in.at = split_pos(c, tile, g);
        split_load<T, CPT>(x, in.at.e0, c, in.at.rv, in.xr);
        split_load<T, CPT>(dy, in.at.e0, c, in.at.rv, in.gr);
        const int64_t sr = in.at.rv ? in.at.row : 0;
        in.mu = have_stats ? mean_in[sr] : 0.f;
        in.rs = have_stats ? rstd_in[sr] : 0.f;
    };
    auto body = [&](const In& in) {
        const bool rv = in.at.rv;
        float mu = in.mu, rs = in.rs;
        if (!have_stats) split_ln_stats<T, CPT>(in.xr, c, g, eps, red, parity, mu, rs);
        // A row past M adds nothing: its dy is 0 and its statistics are zeroed (recomputed ones
        // are infinite with eps = 0).  Unused slots have dy = gamma = 0, so every term is 0.
        mu = rv ? mu : 0.f;
        rs = rv ? rs : 0.f;
        float s[2];
        {
            const float xh = (in.xr.gets() - mu) * rs;
            const float gg = in.gr.gets() * gs;
            float a = gg, b = gg * xh;
#pragma unroll
            for (int k = 0; k < CPT; ++k)
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    const float xh2 = (in.xr.get(k, v) - mu) * rs;
                    const float gg2 = in.gr.get(k, v) * ga[k * V + v];
                    a += gg2;
                    b = __builtin_fmaf(gg2, xh2, b);
                }
            s[0] = a;
            s[1] = b;
        }
        row_sum<2>(s, g.tpr, red, parity);
        const float c1 = s[0] * g.inv_n, c2 = s[1] * g.inv_n;
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            float o[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int e = k * V + v;
                const float gv = in.gr.get(k, v);
                const float xh = (in.xr.get(k, v) - mu) * rs;
                if constexpr (PG & 1) acc[0][e] = __builtin_fmaf(gv, xh, acc[0][e]);
                if constexpr (PG & 2) acc[IB][e] += gv;
                o[v] = rs * (gv * ga[e] - c1 - xh * c2);
            }
            split_store_chunk<T, CPT, CPT == 2 && PF == 1>(dx, in.at.e0, c, k, o, rv);
        }
        {
            const float gv = in.gr.gets();
            const float xh = (in.xr.gets() - mu) * rs;
            if constexpr (PG & 1) accs[0] = __builtin_fmaf(gv, xh, accs[0]);
            if constexpr (PG & 2) accs[IB] += gv;
            split_store_scalar<T, CPT>(dx, in.at.e0, c, rs * (gv * gs - c1 - xh * c2), rv);
        }
    };
    tile_loop<PF, In>(c, fetch, body);
    // the requested gradients are adjacent in [dgamma | dbeta]: dbeta alone starts at column N
    if constexpr (PG != 0)
        split_write_partials<T, CPT, NGR>(ws + c.wg * g.ws_rs + (PG == 2 ? g.N * g.ws_cs : 0), g.ws_cs, acc, accs,
                                          c, g, part);
}

// ============================================================================== RMSNorm

template <typename T, int CPT>
__device__ __forceinline__ float split_rms_rstd(const SplitRow<T, CPT>& xr, const Geom& g, float eps, float* red,
                                                int& parity) {
    constexpr int V = SplitCtx<T, CPT>::V;
    const float xs = xr.gets();
    float a = xs * xs;
#pragma unroll
    for (int k = 0; k < CPT; ++k)
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const float xv = xr.get(k, v);
            a = __builtin_fmaf(xv, xv, a);
        }
    float s[1] = {a};
    row_sum<1>(s, g.tpr, red, parity);
    return __builtin_amdgcn_rsqf(s[0] * g.inv_n + eps);
}

// VAR 0: the Llama form; VAR 1: weight (plus g.w_offset) times the float32 normalized value.
template <typename T, typename PT, int CPT, int PF, int VAR>
__global__ void __launch_bounds__(kSplitBlock)
rms_fwd_split_kernel(const T* __restrict__ x, const PT* __restrict__ weight, float eps, T* __restrict__ y,
                     float* __restrict__ rstd_out, Geom g) {
    constexpr int V = ChunkOf<T>::value;
    constexpr int E = CPT * V;
    __shared__ float red[kSplitRed];
    int parity = 0;
    const SplitCtx<T, CPT> c(g);
    float w[E], ws_;
    split_param<T, PT, CPT>(weight, 0.f, c, w, ws_);
    if constexpr (VAR != 0) {
#pragma unroll
        for (int e = 0; e < E; ++e) w[e] += g.w_offset;
        ws_ += g.w_offset;
    }
    auto out = [&](float xv, float rs, float wv) {
        const float h = xv * rs;
        return wv * (VAR == 0 ? round_through<T>(h) : h);
    };
    struct In {
        SplitRow<T, CPT> xr;
        SplitRowPos at;
    };
    auto fetch = [&](int64_t tile, In& in) {
        in.at = split_pos(c, tile, g);
        split_load<T, CPT>(x, in.at.e0, c, in.at.rv, in.xr);
    };
    auto body = [&](const In& in) {
        const float rs = split_rms_rstd<T, CPT>(in.xr, g, eps, red, parity);
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            float o[V];
#pragma unroll
            for (int v = 0; v < V; ++v) o[v] = out(in.xr.get(k, v), rs, w[k * V + v]);
            split_store_chunk<T, CPT>(y, in.at.e0, c, k, o, in.at.rv);
        }
        split_store_scalar<T, CPT>(y, in.at.e0, c, out(in.xr.gets(), rs, ws_), in.at.rv);
        if (in.at.rv && c.lane == 0 && rstd_out) rstd_out[in.at.row] = rs;
    };
    tile_loop<PF, In>(c, fetch, body);
}

template <typename T, typename PT, int CPT, int PF, int VAR, int PG>
__global__ void __launch_bounds__(kSplitBlock)
rms_bwd_split_kernel(const T* __restrict__ x, const T* __restrict__ dy, const float* __restrict__ rstd_in,
                     const PT* __restrict__ weight, float eps, T* __restrict__ dx, float* __restrict__ ws, Geom g) {
    constexpr int V = ChunkOf<T>::value;
    constexpr int E = CPT * V;
    extern __shared__ float part[];
    __shared__ float red[kSplitRed];
    int parity = 0;
    const SplitCtx<T, CPT> c(g);
    float w[E], wsc;
    split_param<T, PT, CPT>(weight, 0.f, c, w, wsc);
    if constexpr (VAR != 0) {
#pragma unroll
        for (int e = 0; e < E; ++e) w[e] += g.w_offset;
        wsc += g.w_offset;
    }
    float acc[1][E], accs[1] = {0.f};
#pragma unroll
    for (int e = 0; e < E; ++e) acc[0][e] = 0.f;
    // grad of the normalized value: the float32 product, rounded to x's dtype in the Llama form
    auto grad_n = [&](float gv, float wv) {
        const float p = gv * wv;
        return VAR == 0 ? round_through<T>(p) : p;
    };
    // weight-gradient term: Llama form dy * n (n = h rounded to x's dtype), the product rounded to
    // the weight's dtype; float32 forms dy * h
    auto term = [&](float gv, float h) {
        return VAR == 0 ? round_through<PT>(gv * round_through<T>(h)) : gv * h;
    };
    struct In {
        SplitRow<T, CPT> xr, gr;
        SplitRowPos at;
        float rs;
    };
    auto fetch = [&](int64_t tile, In& in) {
        in.at = split_pos(c, tile, g);
        split_load<T, CPT>(x, in.at.e0, c, in.at.rv, in.xr);
        split_load<T, CPT>(dy, in.at.e0, c, in.at.rv, in.gr);
        in.rs = rstd_in ? rstd_in[in.at.rv ? in.at.row : 0] : 0.f;
    };
    auto body = [&](const In& in) {
        const bool rv = in.at.rv;
        float rs = rstd_in ? in.rs : split_rms_rstd<T, CPT>(in.xr, g, eps, red, parity);
        rs = rv ? rs : 0.f;   // a row past M adds nothing (a recomputed rstd is infinite with eps = 0)
        float s[1];
        {
            float a = grad_n(in.gr.gets(), wsc) * (in.xr.gets() * rs);
#pragma unroll
            for (int k = 0; k < CPT; ++k)
#pragma unroll
                for (int v = 0; v < V; ++v)
                    a = __builtin_fmaf(grad_n(in.gr.get(k, v), w[k * V + v]), in.xr.get(k, v) * rs, a);
            s[0] = a;
        }
        row_sum<1>(s, g.tpr, red, parity);
        const float cc = s[0] * g.inv_n;
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            float o[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int e = k * V + v;
                const float gv = in.gr.get(k, v);
                const float h = in.xr.get(k, v) * rs;
                if constexpr (PG) acc[0][e] += term(gv, h);
                o[v] = rs * (grad_n(gv, w[e]) - h * cc);
            }
            split_store_chunk<T, CPT>(dx, in.at.e0, c, k, o, rv);
        }
        {
            const float gv = in.gr.gets();
            const float h = in.xr.gets() * rs;
            if constexpr (PG) accs[0] += term(gv, h);
            split_store_scalar<T, CPT>(dx, in.at.e0, c, rs * (grad_n(gv, wsc) - h * cc), rv);
        }
    };
    tile_loop<PF, In>(c, fetch, body);
    if constexpr (PG) split_write_partials<T, CPT, 1>(ws + c.wg * g.ws_rs, g.ws_cs, acc, accs, c, g, part);
}

}  // namespace rwn
