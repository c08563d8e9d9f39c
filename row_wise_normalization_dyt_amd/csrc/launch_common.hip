// Launch planning, the stage-2 column reduction and the copy probe.
#include <stdlib.h>

#include "rwn_kernels.hpp"
#include "rwn_launch.hpp"

namespace rwn {

static int64_t next_pow2(int64_t v) {
    int64_t p = 1;
    while (p < v) p <<= 1;
    return p;
}

// Tuning override, read once: RWN_WG_PER_CU=<k> sets the workgroups per CU of the row kernels.
// Changing it changes the reduction order (and so the low bits of parameter gradients).
static int env_wg_per_cu() {
    static int v = [] {
        const char* s = getenv("RWN_WG_PER_CU");
        int k = s ? atoi(s) : 0;
        return (k >= 1 && k <= 32) ? k : 0;
    }();
    return v;
}

bool make_plan(int layer, bool backward, int64_t M, int64_t N, int xdt, int misalign_bytes,
               int cus, Plan* out) {
    (void)layer;
    Plan p;
    p.M = M;
    p.N = N;
    const int esz = xdt == DT_F32 ? 4 : 2;
    const int V = 16 / esz;
    const int b = misalign_bytes / esz;
    int64_t chunks;
    if (N % V == 0 && b == 0) {
        p.mode = MODE_ALIGNED;
        chunks = N / V;
    } else {
        // A row that starts V-1 elements past a 16-byte boundary spans this many chunks.
        const int64_t cs = (N + V - 1 + V - 1) / V;
        if (cs > 64) {
            p.mode = MODE_SHIFTED;
            p.base_shift = b;
            chunks = cs;
        } else {
            p.mode = MODE_SCALAR;
            chunks = N;
        }
    }
    const int v_elems = p.mode == MODE_SCALAR ? 1 : V;
    if (chunks <= 64) {
        // Narrow rows: a power-of-two group of lanes per row, several rows per wave.
        p.tpr = (int)next_pow2(chunks);
        p.cpt = 1;
    } else {
        // Wide rows: W waves per row, CPT chunks per lane; least idle lanes, then CPT = 2.
        const int cpt_max = (xdt == DT_F32 || p.mode == MODE_SCALAR) ? 4 : 2;
        int best_cpt = 0, best_w = 0;
        int64_t best_waste = -1;
        const int order[3] = {2, 4, 1};
        for (int oi = 0; oi < 3; ++oi) {
            const int cpt = order[oi];
            if (cpt > cpt_max) continue;
            const int64_t w = (chunks + 64 * cpt - 1) / (64 * cpt);
            if (w > 16) continue;
            const int64_t waste = w * 64 * cpt - chunks;
            if (best_waste < 0 || waste < best_waste) {
                best_waste = waste;
                best_cpt = cpt;
                best_w = (int)w;
            }
        }
        if (best_cpt == 0) return false;
        p.cpt = best_cpt;
        p.tpr = 64 * best_w;
    }
    p.rt = (p.mode == MODE_ALIGNED && p.cpt == 1 && p.tpr <= 64) ? 4 : 1;
    // SHIFTED rows each have their own shift, so a workgroup holds a single row slot.
    p.rpp = (p.mode == MODE_SHIFTED || p.tpr >= 256) ? 1 : 256 / p.tpr;
    p.block = p.tpr * p.rpp;
    const int64_t rows_per_tile = (int64_t)p.rpp * p.rt;
    p.ntiles = (M + rows_per_tile - 1) / rows_per_tile;
    int wg_per_cu = env_wg_per_cu();
    if (wg_per_cu == 0) wg_per_cu = (int)(1024 / p.block) > 1 ? (int)(1024 / p.block) : 1;
    if (wg_per_cu > 16) wg_per_cu = 16;
    int64_t grid = (int64_t)cus * wg_per_cu;
    if (grid >= p.ntiles) {
        grid = p.ntiles;              // one tile per workgroup
    } else {
        grid -= grid % 8;             // SHIFTED: grid * rpp must be a multiple of V (<= 8)
        if (grid < 8) grid = 8;
    }
    p.grid = grid;
    p.lds_bytes = (backward && p.rpp > 1) ? (size_t)p.cpt * v_elems * p.block * sizeof(float) : 0;
    *out = p;
    return true;
}

hipError_t launch_colreduce(int pdt, const float* ws, int64_t P, int64_t ng, int64_t N,
                            void* out0, void* out1, void* out2, hipStream_t s) {
    const int block = 512;
    const int cb = ng <= 64 ? 8 : (ng <= 1024 ? 16 : 64);
    const unsigned grid = (unsigned)((ng + cb - 1) / cb);
    if (pdt == DT_F32) {
        hipLaunchKernelGGL(colreduce_kernel<float>, dim3(grid), dim3(block), 0, s, ws, P, ng, N, cb,
                           (float*)out0, (float*)out1, (float*)out2);
    } else {
        hipLaunchKernelGGL(colreduce_kernel<bf16_t>, dim3(grid), dim3(block), 0, s, ws, P, ng, N, cb,
                           (bf16_t*)out0, (bf16_t*)out1, (bf16_t*)out2);
    }
    return hipGetLastError();
}

// Bandwidth probe: 16-byte vector copy, grid-stride.
__global__ void __launch_bounds__(256)
copy_probe_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst, int64_t n16) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
         i += (int64_t)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

hipError_t launch_copy_probe(const void* src, void* dst, size_t bytes, hipStream_t s) {
    const int64_t n16 = (int64_t)(bytes / 16);
    int64_t grid = (n16 + 255) / 256;
    if (grid > 65536) grid = 65536;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(copy_probe_kernel, dim3((unsigned)grid), dim3(256), 0, s, (const f32x4*)src,
                       (f32x4*)dst, n16);
    return hipGetLastError();
}

}  // namespace rwn
