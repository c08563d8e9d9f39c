// Launch planning, the stage-2 column reduction and the copy probe.
#include <stdlib.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "rwn_kernels.hpp"
#include "rwn_launch.hpp"
#include "rwn_split.hpp"

namespace rwn {

LaunchEvents& launch_events() {
    static thread_local LaunchEvents ev;
    return ev;
}

static int64_t next_pow2(int64_t v) {
    int64_t p = 1;
    while (p < v) p <<= 1;
    return p;
}

// Tuning overrides, read once (each changes the launch plan, and with it the reduction order
// and so the low bits of parameter gradients):
//   RWN_FWD_RT, RWN_BWD_RT  rows per thread of narrow aligned plans (1, 2 or 4; default: 2
//                           for DyT and 16-bit RMSNorm, 1 otherwise)
//   RWN_WG_PER_CU           workgroups per CU of persistent grids (default: chosen per shape)
//   RWN_MIN_WAVES           minimum resident waves per CU the grid must provide (16; 8 for
//                           backwards of 5-7-wave rows on the general kernels, and of 2-4- and
//                           9-15-wave rows when rows are few per CU)
//   RWN_WIDE_BLOCK          workgroup size for wide rows (64..1024)
//   RWN_BLOCKED_K           > 0: backward workgroups take this many consecutive tiles instead
//                           of striding (fwd stays strided)
//   RWN_XCD_REMAP           0: keep hardware workgroup numbering, 1: XCD-contiguous numbering
//                           (default: XCD-contiguous for rows of a wave or more only)
//   RWN_WIDE_CPT            1, 2 or 4: chunks per thread of wide LayerNorm / RMSNorm rows
//   RWN_PACKED_ROWS         0: SHIFTED DyT rows take whole waves (default 1: packed rows)
//   RWN_NARROW_SHIFTED      0: narrow rows not aligned to 16-byte chunks move one element per
//                           lane (SCALAR) instead of 16-byte chunks (default 1)
//   RWN_DYT_FLAT12          0: DyT rows of 12 * 2^k bytes take the general kernels instead of
//                           the 12-byte ones (default 1)
//   RWN_PREFETCH            0 / 1 / 2: force the plain / one-ahead / two-ahead tile loop where
//                           they exist (and with it the general LayerNorm kernels)
//   RWN_FLAT                0: narrow aligned LayerNorm rows take the general kernels (default 1:
//                           the flat kernels)
//   RWN_SPLIT               0: wide rows take the general kernels only (default 1: the split-row
//                           kernels for unaligned wide rows and the aligned ones they measured
//                           faster on; 2: for every wide row)
//   RWN_SPLIT_CPT           1, 2 or 4: chunks per lane of split-row plans
//   RWN_SPLIT_PF            0 / 1: split-row tile loop plain / one tile ahead
static int env_int(const char* name, int lo, int hi, int dflt) {
    const char* s = getenv(name);
    if (!s) return dflt;
    int k = atoi(s);
    return (k >= lo && k <= hi) ? k : dflt;
}

int kernel_occupancy(const void* kernel, int block, size_t dyn_lds) {
    // Keyed by device as well: the answer is the current device's (devices of one process may
    // differ in registers, LDS or wave slots).
    struct Key {
        const void* k;
        int dev;
        int block;
        size_t lds;
        int n;
    };
    static std::mutex mu;
    static std::vector<Key> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    std::lock_guard<std::mutex> lock(mu);
    for (const Key& e : cache)
        if (e.k == kernel && e.dev == dev && e.block == block && e.lds == dyn_lds) return e.n;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, block, dyn_lds) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    cache.push_back(Key{kernel, dev, block, dyn_lds, n});
    return n;
}

static int resident_wgs(int layer, bool backward, const Plan& p, int xdt, int pdt);

// Persistent grid-stride with c workgroups per CU, all resident at once (occ: workgroups of the
// kernel that fit on a CU, 0 if unknown).  c spans [16, 28] resident waves per CU (fewer waves
// leave HBM latency exposed; more add nothing).  Within that range the c whose tile count per
// workgroup is most even wins: the kernel lasts as long as its busiest workgroup, so ntiles / gt
// against ceil(ntiles / gt) is the fraction of the machine kept busy to the end.  Each extra
// workgroup per CU must buy 2% of balance (measured: narrow LayerNorm backwards at 28 waves per
// CU run 20% slower than at 20).  With ncb column blocks the grid is ncb workgroups per tile
// stride.  The tile stride is a multiple of 8, so rows it separates start at the same offset
// modulo 16 bytes.
static void persistent_grid(Plan& p, int cus, int64_t occ, int wg_per_cu, int min_waves) {
    const int64_t waves_per_wg = (p.block + 63) / 64;
    int64_t c_max = std::max<int64_t>(1, 32 / waves_per_wg);   // 32 waves per CU at most
    if (occ > 0) c_max = std::min(c_max, occ);
    const int64_t c_lo = std::min(c_max, std::max<int64_t>(1, (min_waves + waves_per_wg - 1) / waves_per_wg));
    const int64_t c_hi = std::max<int64_t>(c_lo, std::min<int64_t>(c_max, 28 / waves_per_wg));
    int64_t gt = 0;
    double best = -1.0;
    for (int64_t cc = c_lo; cc <= c_hi; ++cc) {
        if (wg_per_cu > 0 && cc != wg_per_cu) continue;
        int64_t cand = (int64_t)cus * cc / p.ncb;
        cand -= cand % 8;                  // SHIFTED: the tile stride * rpp must be a multiple of V
        if (cand < 8) cand = 8;
        if (cand >= p.ntiles) { gt = p.ntiles; break; }   // one tile per workgroup
        const double per = (double)p.ntiles / (double)cand;
        const double eff = per / std::ceil(per) - 0.02 * (double)(cc - c_lo);
        if (eff > best + 1e-9) { best = eff; gt = cand; }
    }
    if (gt == 0) {   // forced c out of range: nearest in-range candidate
        gt = (int64_t)cus * (wg_per_cu > 0 ? std::min<int64_t>(wg_per_cu, c_max) : c_lo) / p.ncb;
        gt -= gt % 8;
        if (gt < 8) gt = 8;
        if (gt > p.ntiles) gt = p.ntiles;
    }
    p.grid = gt * p.ncb;
}

// Backward partials: column-major when rows are short (stage 2 then reads each column
// contiguously), row-major when wide (stage 1 then writes each row contiguously).
static void partial_layout(int layer, Plan& p) {
    const int64_t ng = partial_cols(layer, p.N, p.ncb);
    if (ng <= 1024) {
        p.ws_rs = 1;
        p.ws_cs = p.partial_rows();
    } else {
        p.ws_rs = ng;
        p.ws_cs = 1;
    }
}

// Split-row plan (rwn_split.hpp) for a wide row: W <= max_w waves per row
// slot and CPT whole chunks per lane covering the row's aligned middle, head and tail elements as
// scalar slots.  Slots fill
// 512-thread workgroups; a backward combines its
// slots' partials in LDS (NG gradients x N floats) when that fits in 48 KB, else takes one slot
// per workgroup.  Returns false where no shape fits (float32 rows wider than 8192), leaving the
// general kernels' shifted mode.
static bool plan_split(int layer, bool backward, int64_t M, int64_t N, int xdt, int pdt, int b, int cus,
                       bool occupancy, int wg_per_cu, int min_waves, bool auto_waves, int xcd_remap, int max_w,
                       Plan* pp) {
    static const int split_cpt = env_int("RWN_SPLIT_CPT", 1, 4, 0);
    static const int split_pf = env_int("RWN_SPLIT_PF", 0, 1, -1);
    Plan& p = *pp;
    const int esz = xdt == DT_F32 ? 4 : 2;
    const int V = 16 / esz;
    const int64_t nm = N / V;   // most whole chunks a row can hold (a row starting aligned)
    // Chunks per lane, in order of preference; the fewest lane slots win and ties go to the
    // earlier entry.  Measured at 65536 x N (forward / backward traced us):
    //   - LayerNorm and RMSNorm backwards run fastest with one chunk per lane: bf16 N = 2049
    //     142.4 / 132.2 against 178.2 / 151.2 with two, N = 4097 286.2 / 275.5 against 356.9 /
    //     302.6; float32 N = 1025 131.6 / 133.7 against 148.8 / 146.3 with two, N = 2049 267.8 /
    //     265.1 against 299.1 / 293.0 (aligned N = 1024 no slower).
    //   - Their forwards run fastest with two (bf16 N = 2049 LayerNorm 105.5 against 118.9 with
    //     one, RMSNorm N = 2048 85.8 against 101.1; float32 N = 1025 LayerNorm 98.0 against 112.7),
    //     except 16-bit RMSNorm rows off the 16-byte grid that two chunks fit in one wave: N = 1025
    //     54.3 against 52.8 with one chunk on two waves (float16 54.1 against 52.3); aligned N = 1024
    //     measured 47.0 against 50.0, so it keeps two.
    //   - DyT runs fastest with 16 elements per lane (bf16 N = 2049 backward 178.5 against 183.4
    //     with one chunk; float32 N = 1025 forward 108.5 / backward 158.0 with four chunks against
    //     113.5 / 174.4 with two).
    // 32 elements per lane (4 bfloat16 chunks) only for LayerNorm / RMSNorm rows too wide for 8
    // waves otherwise: DyT's backward would spill there.
    int cands[3];
    if (layer == LAYER_DYT) {
        if (V == 8) { cands[0] = 2; cands[1] = 1; cands[2] = 4; }
        else { cands[0] = 4; cands[1] = 2; cands[2] = 1; }
    } else if (backward || (layer == LAYER_RMS && V == 8 && nm <= 128 && (N % V != 0 || b != 0))) {
        cands[0] = 1; cands[1] = 2; cands[2] = 4;
    } else if (V == 8) {
        cands[0] = 2; cands[1] = 1; cands[2] = 4;
    } else {
        cands[0] = 2; cands[1] = 4; cands[2] = 1;
    }
    const bool wide_ok = layer != LAYER_DYT && max_w >= 8;   // rows no other plan takes
    int bw = 0, bc = 0;
    int64_t best_slots = -1;
    for (int ci = 0; ci < 3; ++ci) {
        const int c = cands[ci];
        const bool wide = c * V > 16;
        if (wide && !wide_ok) continue;
        if (split_cpt > 0 && c != split_cpt) continue;
        const int64_t w = (nm + 64 * c - 1) / (64 * c);
        if (w > max_w) continue;
        const int64_t slots = 64 * w * c;
        if (wide && bw) continue;   // only when nothing narrower fits
        if (best_slots < 0 || slots < best_slots) {
            best_slots = slots;
            bw = (int)w;
            bc = c;
        }
    }
    if (bw == 0) return false;
    p.mode = MODE_SHIFTED;
    p.split = 1;
    p.base_shift = b;
    p.cpt = bc;
    p.rt = 1;
    p.tpr = 64 * bw;
    p.rpp = std::max(1, kSplitBlock / p.tpr);
    p.ncb = 1;
    // Pipelined (one tile ahead) where it measured faster, at 65536 x N (us per launch, plain ->
    // pipelined): 16-bit LayerNorm forwards of two or more waves per row (bf16 N = 2048 102.6 ->
    // 89.1, 2049 105.3 -> 96.5, 4096 201.8 -> 182.4, 4097 206.0 -> 187.7) and 16-bit LayerNorm
    // backwards of two chunks per lane (N = 2048 156.6 -> 134.4).  Elsewhere it measured slower
    // or no faster: RMSNorm forwards (bf16 N = 4096 172.3 -> 181.5, 4097 191.9 -> 199.3),
    // LayerNorm backwards of one chunk per lane (bf16 N = 2049 140.8 -> 166.5, 4097 285.6 ->
    // 290.6), DyT (bf16 N = 2048 backward 166.2 -> 187.0, 4096 342.9 -> 367.3), float32 LayerNorm
    // (N = 1024 forward 85.2 -> 86.5).  Four chunks per lane stay plain:
    // a second tile in flight would double their 32 elements of registers.
    const bool pf_ln = layer == LAYER_LN && V == 8 && p.cpt == 2 && (backward || p.tpr >= 128);
    p.pf = split_pf >= 0 ? split_pf : (pf_ln ? 1 : 0);
    p.flat = 0;
    const int ngrad = layer == LAYER_RMS ? 1 : 2;
    if (backward && p.rpp > 1 && (int64_t)ngrad * N * 4 > 48 * 1024) p.rpp = 1;
    p.block = p.tpr * p.rpp;
    p.lds_bytes = (backward && p.rpp > 1) ? (size_t)ngrad * N * sizeof(float) : 0;
    p.ntiles = (M + p.rpp - 1) / p.rpp;
    int64_t occ = 0;
    if (occupancy) {
        const int pdts[3] = {DT_F32, DT_BF16, DT_F16};
        for (int i = 0; i < 3; ++i) {
            if (pdt >= 0 && pdts[i] != pdt) continue;
            if (!dtype_pair_ok(xdt, pdts[i])) continue;
            const int n = resident_wgs(layer, backward, p, xdt, pdts[i]);
            if (n > 0) occ = occ == 0 ? n : std::min<int64_t>(occ, n);
        }
    }
    p.strided = 1;
    p.kt = 0;
    // Workgroups of five to seven waves with two or more chunks per lane (3-wave row slots two
    // to a workgroup, 5-7-wave slots alone) take two per CU rather than the 18-21 waves that 16
    // rounds up to: bf16 44739 x 3000 forwards (256 MiB tensors) LayerNorm 122.3 -> 102.4 us,
    // RMSNorm 108.2 -> 92.3, DyT 122.4 -> 117.0; 65536 x 2600 LayerNorm 161.2 -> 136.0.  With
    // one chunk per lane that leaves too few bytes in flight (RMSNorm 65536 x 2300, 5-wave
    // slots: forward 111.2 -> 173.1 us); such LayerNorm backwards take at least 12 waves
    // instead (two or three workgroups per CU: bf16 65536 x 1500 161.2 -> 119.2 us, 65536 x 2300
    // 237.7 -> 183.9), while RMSNorm's ran slower that way (65536 x 1500 106.5 -> 115.4) and
    // DyT's unchanged; forwards keep 16.
    const int wpw = (p.block + 63) / 64;
    int mw = min_waves;
    if (auto_waves && wpw >= 5 && wpw <= 7) mw = p.cpt >= 2 ? 8 : (backward && layer == LAYER_LN) ? 12 : min_waves;
    persistent_grid(p, cus, occ, wg_per_cu, mw);
    const bool remap = xcd_remap >= 0 ? xcd_remap == 1 : true;
    p.xcd_remap = (remap && p.grid % 8 == 0) ? 1 : 0;
    if (backward) partial_layout(layer, p);
    return true;
}

static int resident_wgs(int layer, bool backward, const Plan& p, int xdt, int pdt);

// Flat LayerNorm plan with 12-byte lane chunks (rwn_kernels.hpp) for rows of 12 * 2^k bytes,
// 2^k <= 64 lanes, on 4-byte aligned operands.  Such rows in 16-byte chunks leave a quarter of
// their lanes idle, or are not whole chunks at all.  Measured on one MI355X against the 16-byte
// flat kernels (traced us, forward / backward stage 1): LayerNorm 401408 x 24 float32 16.4 / 22.1
// -> 15.3 / 21.9; 262144 x 48 float32 21.1 / 27.6 -> 19.0 / 27.2; 65536 x 384 bf16 23.4 / 35.1 ->
// 21.8 / 35.3.  Four waves per workgroup (fewer for small M); tiles are the waves' row groups
// (the forward's two steps of them), dealt round-robin over a persistent grid.
static bool plan_flat12(int layer, bool backward, int64_t M, int64_t N, int xdt, int pdt, int cus, bool occupancy,
                        int wg_per_cu, int min_waves, Plan* pp) {
    const int esz = xdt == DT_F32 ? 4 : 2;
    if ((N * esz) % 12) return false;
    const int64_t lanes = N * esz / 12;
    if (lanes > 64 || (lanes & (lanes - 1))) return false;
    Plan& p = *pp;
    p.mode = MODE_ALIGNED;
    p.flat = 2;
    p.split = 0;
    p.cpt = 1;
    p.tpr = (int)lanes;
    p.rt = backward || lanes == 1 ? 1 : 2;
    p.ncb = 1;
    p.pf = 0;
    p.kt = 0;
    const int64_t rows_per_wave = (64 / p.tpr) * p.rt;
    const int64_t waves = std::min<int64_t>(4, (M + rows_per_wave - 1) / rows_per_wave);
    p.block = (int)(64 * std::max<int64_t>(1, waves));
    p.rpp = p.block / p.tpr;
    p.ntiles = (M + (int64_t)p.rpp * p.rt - 1) / ((int64_t)p.rpp * p.rt);
    p.lds_bytes = backward ? (size_t)2 * (12 / esz) * p.block * sizeof(float) : 0;
    int64_t occ = 0;
    if (occupancy) {
        const int pdts[3] = {DT_F32, DT_BF16, DT_F16};
        for (int i = 0; i < 3; ++i) {
            if (pdt >= 0 && pdts[i] != pdt) continue;
            if (!dtype_pair_ok(xdt, pdts[i])) continue;
            const int n = resident_wgs(layer, backward, p, xdt, pdts[i]);
            if (n > 0) occ = occ == 0 ? n : std::min<int64_t>(occ, n);
        }
    }
    p.strided = 1;
    persistent_grid(p, cus, occ, wg_per_cu, min_waves);
    p.xcd_remap = 0;   // narrow rows stream faster in the hardware's workgroup order
    if (backward) partial_layout(layer, p);
    return true;
}

static int resident_wgs(int layer, bool backward, const Plan& p, int xdt, int pdt) {
    if (layer == LAYER_DYT) return resident_wgs_dyt(backward, p, xdt, pdt);
    if (layer == LAYER_LN) return resident_wgs_ln(backward, p, xdt, pdt);
    return resident_wgs_rms(backward, p, xdt, pdt);
}

bool make_plan(int layer, bool backward, int64_t M, int64_t N, int xdt, int pdt, int misalign_bytes,
               int cus, bool occupancy, Plan* out, int layout) {
    static const int fwd_rt = env_int("RWN_FWD_RT", 1, 4, 0);
    static const int bwd_rt = env_int("RWN_BWD_RT", 1, 4, 0);
    static const int wg_per_cu = env_int("RWN_WG_PER_CU", 1, 32, 0);
    static const int min_waves = env_int("RWN_MIN_WAVES", 1, 32, 16);
    static const bool min_waves_set = getenv("RWN_MIN_WAVES") != nullptr;
    static const int wide_block = env_int("RWN_WIDE_BLOCK", 64, 1024, 512);
    static const int blocked_k = env_int("RWN_BLOCKED_K", 1, 1 << 20, 0);
    static const int xcd_remap = env_int("RWN_XCD_REMAP", 0, 1, -1);
    static const int prefetch = env_int("RWN_PREFETCH", 0, 2, -1);
    static const int wide_cpt = env_int("RWN_WIDE_CPT", 1, 4, 0);
    static const int packed_rows = env_int("RWN_PACKED_ROWS", 0, 1, 1);
    static const int flat_rows = env_int("RWN_FLAT", 0, 1, 1);
    static const int split_rows = env_int("RWN_SPLIT", 0, 2, 1);
    static const int flat12_rows = env_int("RWN_FLAT12", 0, 1, 1);
    static const int narrow_shifted = env_int("RWN_NARROW_SHIFTED", 0, 1, 1);
    static const int dyt_flat12 = env_int("RWN_DYT_FLAT12", 0, 1, 1);
    Plan p;
    p.M = M;
    p.N = N;
    p.layout = layout;
    const int esz = xdt == DT_F32 ? 4 : 2;
    const int V = 16 / esz;
    const int b = misalign_bytes / esz;
    int64_t chunks;
    if (layout == 2) {
        p.mode = MODE_SCALAR;
        chunks = N;
    } else if (N % V == 0 && b == 0) {
        p.mode = MODE_ALIGNED;
        chunks = N / V;
    } else {
        // A row that starts V-1 elements past a 16-byte boundary spans this many chunks.
        // Narrow rows take the same 16-byte chunks (a power-of-two group of lanes per row, several
        // rows per workgroup, each row slot with the shift of its rows; strided rows all share the
        // base's) rather than one element per lane: at 64 MiB tensors, bf16 N = 100 ran at 20-22%
        // of 8 TB/s per step in SCALAR mode for all three layers.
        const int64_t cs = (N + V - 1 + V - 1) / V;
        if (cs > 64 || (narrow_shifted && layout <= 1)) {
            p.mode = MODE_SHIFTED;
            p.base_shift = b;
            chunks = cs;
        } else {
            p.mode = MODE_SCALAR;
            chunks = N;
        }
    }
    // DyT takes the 12-byte kernels for backwards, and for forwards of rows that are not whole
    // 16-byte chunks: elsewhere the general forward (two rows per thread, one tile ahead)
    // measured faster.  64 MiB tensors, traced us, general -> 12-byte: bf16 backwards N = 24
    // 45.7 -> 40.8, 96 45.8 -> 41.4, 192 51.6 -> 42.6, 384 52.0 -> 47.4; float32 N = 12 37.6 ->
    // 34.2; bf16 N = 12 (24-byte rows) forward 76.0 -> 32.0, backward 96.7 -> 40.9; forwards of
    // whole chunks 25.0 -> 29.7 (float32 N = 12), 29.4 -> 32.0 (bf16 N = 24).
    const bool dyt12 = layer == LAYER_DYT && dyt_flat12 && (backward || (N * esz) % 16 != 0 || misalign_bytes % 16);
    if (flat_rows && flat12_rows && (layer == LAYER_LN || dyt12) && layout == 0 &&
        prefetch < 0 && blocked_k == 0 && misalign_bytes % 4 == 0 &&
        plan_flat12(layer, backward, M, N, xdt, pdt, cus, occupancy, wg_per_cu, min_waves, &p)) {
        *out = p;
        return true;
    }
    // Split-row kernels: every wide row not aligned to 16-byte chunks, and aligned wide rows of at
    // most max_w waves per row slot.  Measured against the general kernels (65536 x N bf16, forward
    // / backward us): N = 1024 LayerNorm 58.1 / 88.5 -> 48.6 / 86.4, RMSNorm 50.7 / 78.5 -> 46.6 /
    // 73.8, DyT 60.8 / 82.9 -> 50.1 / 81.6; N = 4096 forwards 182.2 -> 174.4 (LayerNorm), 206.5 ->
    // 191.1 (DyT), DyT backward 315.2 -> 306.8; 16384 x 2048 RMSNorm 27.2 / 45.8 -> 25.4 / 44.6.
    // LayerNorm / RMSNorm backwards of four or more waves per row ran slower split (65536 x 4096:
    // 288.2 -> 332.0, 271.5 -> 284.3 us), and forwards of eight no faster (N = 8192).
    // RMSNorm backwards of 4-wave rows split as well when the rows are few per CU (at most 64):
    // 8192 x 4096 bf16 stage 1 43.2 -> 41.1 us, while at 65536 x 4096 the split form measured
    // 268.2 -> 273.0 us.  16-bit LayerNorm rows of 512 chunks or more split up to 8 waves when
    // they are few per CU (64 MiB tensors, forward / backward stage 1 us): bf16 4096 x 8192 38.6
    // / 65.1 -> 27.1 / 45.0, 6553 x 5120 41.5 / 57.9 -> 34.2 / 45.9, 8192 x 4096 backward 54.8 ->
    // 47.1; 12000 x 8192 step 54.7 -> 67.3% of 8 TB/s.  Narrower few rows measured slower split
    // (bf16 11184 x 3000 backward 52.5 -> 67.1), and float32 rows no faster (3276 x 5120 step
    // 46.1 -> 44.8%).  RMSNorm and DyT do the same from 1024 chunks (bf16 N = 8192, step %:
    // RMSNorm 4096 rows 48.8 -> 54.5, 12000 rows 64.2 -> 66.5; DyT 45.2 -> 48.7, 56.9 -> 62.8;
    // at N = 3000 and 5120 they measured slower split).  Rows of 2048 chunks keep the general
    // kernels (bf16 8000 x 16384 step %: RMSNorm 66.7 -> 62.2, LayerNorm 57.0 -> 54.7 split).
    const bool few_rows = M <= (int64_t)64 * cus;
    int split_max_w = 0;
    if (p.mode == MODE_SHIFTED && chunks > 64) split_max_w = 8;
    else if (p.mode == MODE_ALIGNED && chunks > 64)
        split_max_w = split_rows == 2 || (esz == 2 && few_rows && chunks >= (layer == LAYER_LN ? 512 : 1024) &&
                                          chunks <= 1024)
                          ? 8
                          : (!backward || layer == LAYER_DYT || (layer == LAYER_RMS && few_rows)) ? 4 : 2;
    if (split_max_w && split_rows && prefetch < 0 && layout == 0 &&
        plan_split(layer, backward, M, N, xdt, pdt, b, cus, occupancy, wg_per_cu, min_waves, !min_waves_set, xcd_remap,
                   split_max_w, &p)) {
        *out = p;
        return true;
    }
    const int v_elems = p.mode == MODE_SCALAR ? 1 : V;
    bool packed = false;   // DyT SHIFTED rows packed into workgroups without wave alignment
    if (layer == LAYER_DYT && chunks > 64 && p.mode == MODE_SHIFTED && chunks <= 512 &&
        packed_rows) {
        // DyT has no row reduction, so a row's lanes need not fill whole waves: a SHIFTED row
        // takes exactly `chunks` lanes, and as many rows as fit share a workgroup of <= 512
        // threads (N = 1025 bf16: 3 rows of 129 lanes, 387 of 448 lanes busy, against 129 of
        // 192 with three whole waves per row; forward 85.8 -> 76.9 us).  The backward packs its
        // rows too, without pipelining (the pipelined form's registers leave too few waves
        // resident for such workgroups): backward 120.8 -> 103.2 us, stage 2 7.7 -> 4.0 us (a
        // third as many partial rows).
        p.tpr = (int)chunks;
        p.cpt = 1;
        packed = true;
    } else if (layer == LAYER_DYT && chunks > 64 && (p.mode != MODE_SCALAR || layout == 2)) {
        // DyT has no row reduction: wide rows are cut into ncb column blocks of W <= 8 waves,
        // one chunk per lane (its per-element state is the largest of the three layers); so are
        // strided rows of any alignment, one element per lane.
        // Fewest idle lanes, ties to the widest block.
        int64_t best = -1;
        for (int w = 8; w >= 1; --w) {
            const int64_t ncb = (chunks + 64 * w - 1) / (64 * w);
            const int64_t waste = ncb * 64 * w - chunks;
            if (best < 0 || waste < best) {
                best = waste;
                p.tpr = 64 * w;
                p.ncb = (int)ncb;
            }
        }
        p.cpt = 1;
    } else if (chunks <= 64) {
        // Narrow rows: a power-of-two group of lanes per row, several rows per wave.
        p.tpr = (int)next_pow2(chunks);
        p.cpt = 1;
    } else {
        // Wide rows: W waves per row, CPT chunks per lane.  Fewest idle lanes; ties go to
        // CPT = 1, then 4, for DyT (no row reduction, and its per-element state is the largest,
        // so it wants the larger register budget of <= 8-wave rows) and to CPT = 2 otherwise
        // (fewer waves to combine per row).  Wave limits follow the kernels' launch bounds.
        int best_cpt = 0, best_w = 0;
        int64_t best_waste = -1;
        const int order_dyt[3] = {1, 4, 2}, order_norm[3] = {2, 4, 1}, order_few_waves[3] = {4, 2, 1};
        const int* order = layer == LAYER_DYT ? order_dyt : order_norm;
        // SHIFTED RMSNorm forwards run fastest with the fewest waves per row, and so do SHIFTED
        // LayerNorm forwards whose row fits one wave (measured at N = 1025 bf16: one wave with
        // four chunks per lane against three waves with one, RMSNorm 62 vs 72 us, LayerNorm 80.6
        // vs 91.1 us), idle lanes notwithstanding: no cross-wave combine, so no barrier between
        // a row's loads and its stores.
        const bool few_waves = !backward && p.mode == MODE_SHIFTED &&
                               (layer == LAYER_RMS || (layer == LAYER_LN && chunks <= 4 * 64));
        if (few_waves) order = order_few_waves;
        for (int oi = 0; oi < 3; ++oi) {
            const int cpt = order[oi];
            if (wide_cpt > 0 && cpt != wide_cpt) continue;
            const int wmax = (cpt == 1 || (cpt == 4 && esz == 2)) ? 8 : 16;
            const int64_t w = (chunks + 64 * cpt - 1) / (64 * cpt);
            if (w > wmax) continue;
            const int64_t waste = w * 64 * cpt - chunks;
            if (few_waves) {   // first shape that fits
                best_cpt = cpt;
                best_w = (int)w;
                break;
            }
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
    const bool narrow_aligned = p.mode == MODE_ALIGNED && p.cpt == 1 && p.tpr <= 64;
    // Narrow DyT rows run fastest with two rows per thread (one tile ahead in forwards and in
    // backwards of up to 16 lanes per row, no pipelining above: see the pipelining rule below).
    // So do narrow 16-bit RMSNorm rows, not pipelined (traced fwd / bwd us, one -> two rows per
    // thread): 1048576 x 32 bf16 26.5 / 42.2 -> 25.8 / 37.9, x 64 50.4 / 75.0 -> 47.4 / 70.7,
    // x 128 100.2 / 145.3 -> 93.8 / 140.0, f16 x 128 97.6 / 147.1 -> 94.0 / 140.9, 524288 x 256
    // bf16 99.0 / 146.5 -> 94.7 / 141.1.  fp32 RMSNorm keeps one (1048576 x 128 backward 275.6 ->
    // 295.2), and so do narrow LayerNorm rows, which take the flat kernels (two rows per thread
    // on the general kernels: 1048576 x 128 bf16 forward 97.5 -> 103.0, N = 24 fp32 4.6% slower).
    const int rt_auto = (layer == LAYER_DYT || (layer == LAYER_RMS && esz == 2)) ? 2 : 1;
    p.rt = narrow_aligned ? (backward ? (bwd_rt > 0 ? bwd_rt : rt_auto) : (fwd_rt > 0 ? fwd_rt : rt_auto)) : 1;
    if (p.rt == 3) p.rt = 2;
    if (layout) p.rt = 1;

    // Row slots: narrow rows fill 256-thread workgroups; wide rows use wide_block threads.
    // SHIFTED slots each carry their own shift, so a strided SHIFTED workgroup of wide rows has
    // one slot.  Narrow SHIFTED rows and packed DyT rows have several: their slots keep their
    // shifts because the tile stride (grid * rpp rows, the grid a multiple of 8) is a multiple
    // of V.
    // A blocked SHIFTED workgroup walks consecutive tiles, so its slots must be V rows apart
    // (rpp = V) for each slot to keep one shift; where V slots do not fit in a workgroup the
    // backward stays strided.
    bool blocked = backward && blocked_k > 0 && p.ncb == 1 && layout == 0;
    if (p.mode == MODE_SHIFTED && p.tpr <= 64) {
        // narrow rows: 256 threads, or V slots where that is more (whole waves, and slots V apart
        // for a blocked backward)
        p.rpp = std::max(256 / p.tpr, V);
    } else if (p.mode == MODE_SHIFTED) {
        if (blocked && (int64_t)p.tpr * V <= max_block(p.rt, p.cpt, esz)) {
            p.rpp = V;
        } else {
            p.rpp = packed ? std::max(1, max_block(p.rt, p.cpt, esz) / p.tpr) : 1;
            blocked = false;
        }
    } else {
        const int target = p.tpr <= 64 ? 256 : wide_block;
        p.rpp = p.tpr >= target ? 1 : target / p.tpr;
    }
    if (p.ncb > 1 && p.mode == MODE_SHIFTED) p.rpp = 1;
    // Pipelined tile loop (measured): it pays in forwards with one chunk per thread (except
    // the SHIFTED LayerNorm / RMSNorm ones) and in 16-wave rows, and in SHIFTED backwards;
    // elsewhere the doubled input registers cost more than the overlap gains.  Shapes with
    // more than two chunks per thread have no pipelined form.
    // Narrow DyT rows (the most arithmetic per byte) take two rows per thread, one tile ahead
    // (below); with one row per thread (RWN_FWD_RT / RWN_BWD_RT = 1) they run two tiles ahead in
    // the backward always, in the forward from 16 lanes per row up.
    if (p.cpt * p.rt <= 2) {
        const bool one = p.cpt * p.rt == 1;
        const bool narrow_dyt = layer == LAYER_DYT && one && p.mode == MODE_ALIGNED && p.tpr <= 64;
        // Narrow DyT with two rows per thread (1048573 x N bf16, traced us against one row per
        // thread, one or two tiles ahead): forwards one tile ahead, N = 32 28.0 -> 25.8, 128
        // 102.8 -> 99.5, 256 208.8 -> 196.3 (fp32 N = 256: 104.0 -> 93.7); backwards one tile
        // ahead up to 16 lanes per row, N = 32 41.4 -> 40.4, 128 154.8 -> 145.3 (fp32 N = 64: 38.5
        // -> 36.8), and not pipelined from 32 lanes (fp32 N = 256 one tile ahead 132.5 -> 141.1).
        const bool narrow_dyt2 = layer == LAYER_DYT && p.cpt == 1 && p.rt == 2 && p.mode == MODE_ALIGNED &&
                                 p.tpr <= 64;
        // Narrow SHIFTED rows (measured at 64 MiB bf16 tensors, traced us): LayerNorm / RMSNorm
        // forwards run one tile ahead (N = 100: 48.5 -> 46.0, 43.8 -> 41.6; N = 500: 39.4 -> 37.5,
        // 33.9 -> 32.6; float32 LayerNorm N = 250: 103.6 -> 98.3), and DyT backwards do not
        // (N = 500: 52.2 -> 47.7, N = 100: 56.7 -> 55.4).
        const bool narrow_shift = p.mode == MODE_SHIFTED && p.tpr <= 64;
        if (prefetch >= 0) p.pf = (prefetch == 2 && !(one && p.mode != MODE_SCALAR)) ? 1 : prefetch;
        else if (narrow_dyt2) p.pf = (!backward || p.tpr <= 16) ? 1 : 0;
        else if (narrow_dyt && (backward || p.tpr >= 16)) p.pf = 2;
        else if (!backward)
            p.pf = ((one && (layer == LAYER_DYT || p.mode != MODE_SHIFTED || narrow_shift)) || p.tpr >= 1024) ? 1 : 0;
        else if (layer == LAYER_RMS && p.mode == MODE_ALIGNED && p.tpr >= 128 &&
                 (p.tpr >= 1024 || M <= (int64_t)32 * cus * std::max(1, wide_block / p.tpr)))
            // Aligned RMSNorm backwards of two or more waves per row, pipelined (measured): 16-wave
            // rows (65536 x 16384 bf16, 1211 -> 1119 us) and shapes with at most ~32 row tiles per
            // CU (16384 x 2048 and 8192 x 4096 bf16, 3-6% faster); with more tiles per CU, as at
            // 65536 x 4096..8192, it measured 3-7% slower.
            p.pf = 1;
        else p.pf = (p.mode == MODE_SHIFTED && one && !packed && !(layer == LAYER_DYT && narrow_shift)) ? 1 : 0;
    }
    // Narrow aligned LayerNorm rows, one chunk and one row per thread, take the flat kernels
    // (plain loads on clamped row indices, no per-tile descriptors), which run fastest without
    // pipelining.
    if (flat_rows && prefetch < 0 && layout == 0 && layer == LAYER_LN && p.mode == MODE_ALIGNED && p.cpt == 1 &&
        p.rt == 1 && p.tpr <= 64 && p.ncb == 1) {
        p.flat = 1;
        p.pf = 0;
    }
    // Keep to the kernel shape's launch bound (tpr itself always fits: see the wave limits).
    const int maxb = max_block(p.rt, p.cpt, esz);
    if (p.tpr * p.rpp > maxb) p.rpp = maxb / p.tpr > 0 ? maxb / p.tpr : 1;
    if (p.mode == MODE_SHIFTED && blocked && p.rpp % V) {
        p.rpp = 1;
        blocked = false;
    }
    p.block = p.tpr * p.rpp;
    if (packed) p.block = (p.block + 63) / 64 * 64;   // whole waves (see RowCtx)
    if (p.block > maxb) return false;
    const int64_t rows_per_tile = (int64_t)p.rpp * p.rt;
    p.ntiles = (M + rows_per_tile - 1) / rows_per_tile;
    if (backward && (p.rpp > 1 || p.flat)) {   // LDS for combining the row slots' partials
        int64_t e = (int64_t)p.cpt * v_elems * p.block;
        if (p.mode == MODE_SHIFTED && (int64_t)p.rpp * N > e) e = (int64_t)p.rpp * N;   // a row per slot
        if (p.flat) e *= 2;   // the flat backward combines dgamma and dbeta together
        p.lds_bytes = (size_t)e * sizeof(float);
    }
    // Workgroups of this kernel that fit on a CU at once: every workgroup of a persistent grid
    // must be resident, or the ones that are not start only when others finish.  With pdt = -1
    // the plan holds for every parameter dtype (the most restrictive kernel decides).
    int64_t occ = 0;
    if (occupancy) {
        const int pdts[3] = {DT_F32, DT_BF16, DT_F16};
        for (int i = 0; i < 3; ++i) {
            if (pdt >= 0 && pdts[i] != pdt) continue;
            if (!dtype_pair_ok(xdt, pdts[i])) continue;
            const int n = resident_wgs(layer, backward, p, xdt, pdts[i]);
            if (n > 0) occ = occ == 0 ? n : std::min<int64_t>(occ, n);
        }
    }

    if (blocked) {
        p.kt = blocked_k;
        p.grid = (p.ntiles + p.kt - 1) / p.kt;
    } else {
        p.strided = 1;
        // Backwards of wide rows on the general kernels take half the resident waves with rows of
        // five to seven waves, and with rows of two to four or nine to fifteen when rows are few
        // per CU: with 16 per CU the grid leaves each workgroup a handful of rows and a whole
        // partial row to write for them (and stage 2 to read), and 5-7-wave workgroups run 18-21
        // waves per CU.  (float32 3276 x 5120, 10-wave rows, backward stage 1 + stage 2 us:
        // LayerNorm 59.1 -> 48.7, RMSNorm 45.8 -> 39.8, DyT 45.3 -> 42.1.)  Measured (backward stage 1 + stage 2, us, 16 -> 8
        // waves): 64 MiB tensors, LayerNorm bf16 6553 x 5120 95.0 -> 66.6, float32 5592 x 3000
        // 63.3 -> 46.3, RMSNorm bf16 6553 x 5120 60.9 -> 49.0, DyT bf16 6553 x 5120 67.5 -> 53.0;
        // 256 MiB tensors, LayerNorm bf16 26214 x 5120 235.1 -> 176.3, RMSNorm 210.2 -> 161.3,
        // DyT 198.3 -> 168.7, LayerNorm float32 65536 x 3000 557.1 -> 467.6.  4-wave backwards
        // with many rows per CU run slower with it (LayerNorm bf16 65536 x 4096 289.7 -> 341.4),
        // forwards were mostly slower, and 8-wave backwards mixed (float32 LayerNorm 4096 x 4096
        // 45.8 -> 54.5).
        const int rw = p.tpr / 64;   // waves per row
        const bool fewer = rw >= 5 && rw <= 7 ? true : few_rows && ((rw >= 2 && rw <= 4) || (rw >= 9 && rw <= 15));
        // LayerNorm / RMSNorm forwards of 5-wave rows likewise (bf16 N = 5120: LayerNorm 26214
        // rows 122.2 -> 117.8 us, RMSNorm 100.0 -> 98.1, 6553 rows 32.7 -> 30.3; DyT's ran slower).
        const bool fewer_fwd = !backward && layer != LAYER_DYT && rw == 5;
        const int mw = ((backward && fewer) || fewer_fwd) && !min_waves_set ? 8 : min_waves;
        persistent_grid(p, cus, occ, wg_per_cu, mw);
        p.kt = 0;
        // XCD-contiguous numbering pays where a row spans a wave or more (LayerNorm / RMSNorm
        // 65536 x 4096..8192 bf16: 4-6% faster): neighbouring rows share cache lines at their
        // ends, and both writers then sit behind one L2.  Narrow rows come in whole tiles that
        // share no lines, and there the hardware's round-robin numbering streams faster
        // (LayerNorm 401408 x 24 fp32 step 46.0 -> 44.1 us, DyT 1048573 x 128 bf16 forward
        // 122 -> 103 us).
        const bool remap = xcd_remap >= 0 ? xcd_remap == 1 : p.tpr >= 64;
        p.xcd_remap = (remap && p.grid % 8 == 0) ? 1 : 0;
    }
    if (backward) partial_layout(layer, p);
    *out = p;
    return true;
}

hipError_t launch_colreduce(int pdt, const float* ws, int64_t P, int64_t ng, int64_t rs, int64_t cs,
                            int64_t N, int64_t c_lo, int64_t c_hi, void* out0, void* out1, void* out2,
                            hipStream_t s) {
    if (c_hi > 2 * N + 1) c_hi = 2 * N + 1;   // column 2N's workgroup adds the columns after it
    if (c_lo < 0 || c_lo >= c_hi) return hipSuccess;
    if (rs == 1) {
        // Column-major partials: one workgroup per output column.
        const unsigned grid = (unsigned)(c_hi - c_lo);
        if (pdt == DT_F32)
            return launch(colreduce_cm_kernel<float>, dim3(grid), dim3(256), 0, s, ws, P, ng, cs, N, c_lo,
                          (float*)out0, (float*)out1, (float*)out2);
        if (pdt == DT_F16)
            return launch(colreduce_cm_kernel<f16_t>, dim3(grid), dim3(256), 0, s, ws, P, ng, cs, N, c_lo,
                          (f16_t*)out0, (f16_t*)out1, (f16_t*)out2);
        return launch(colreduce_cm_kernel<bf16_t>, dim3(grid), dim3(256), 0, s, ws, P, ng, cs, N, c_lo,
                      (bf16_t*)out0, (bf16_t*)out1, (bf16_t*)out2);
    }
    const int block = 512;
    // Lanes per column: enough that each lane adds ~8 partial rows (column-major partials) or
    // ~16 (row-major, where lanes of one column are not contiguous).
    const int64_t per = cs == 1 ? 16 : 8;
    int64_t L = next_pow2((P + per - 1) / per);
    const int64_t lmax = cs == 1 ? 64 : 512;
    if (L < 8) L = 8;
    if (L > lmax) L = lmax;
    const int cb = (int)(block / L);
    const unsigned grid = (unsigned)((c_hi - c_lo + cb - 1) / cb);
    if (pdt == DT_F32) {
        return launch(colreduce_kernel<float>, dim3(grid), dim3(block), 0, s, ws, P, ng, rs, cs, N, c_lo, c_hi,
                      cb, (float*)out0, (float*)out1, (float*)out2);
    } else if (pdt == DT_F16) {
        return launch(colreduce_kernel<f16_t>, dim3(grid), dim3(block), 0, s, ws, P, ng, rs, cs, N, c_lo, c_hi,
                      cb, (f16_t*)out0, (f16_t*)out1, (f16_t*)out2);
    } else {
        return launch(colreduce_kernel<bf16_t>, dim3(grid), dim3(block), 0, s, ws, P, ng, rs, cs, N, c_lo, c_hi,
                      cb, (bf16_t*)out0, (bf16_t*)out1, (bf16_t*)out2);
    }
}

// Streaming probe (a measurement aid): out = a (one input) or out = a ^ b (two inputs) over n16
// 16-byte chunks.  A persistent grid of wg_per_cu workgroups per CU; each lane keeps U 16-byte
// loads per input in flight (chunks i, i + S, ..., i + (U - 1) S, S the grid's thread count)
// before it stores, optionally with the nontemporal hint on every access.  It bounds what a
// kernel that reads one or two tensors and writes one can stream at a given size.
template <int U, bool TWO, bool NT>
__global__ void __launch_bounds__(256)
stream_probe_kernel(const u32x4* __restrict__ a, const u32x4* __restrict__ b, u32x4* __restrict__ o,
                    int64_t n16) {
    const int64_t S = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    auto ld = [](const u32x4* p) { return NT ? __builtin_nontemporal_load(p) : *p; };
    for (; i + (U - 1) * S < n16; i += U * S) {
        u32x4 v[U], w[U];
#pragma unroll
        for (int j = 0; j < U; ++j) v[j] = ld(a + i + j * S);
        if constexpr (TWO) {
#pragma unroll
            for (int j = 0; j < U; ++j) w[j] = ld(b + i + j * S);
#pragma unroll
            for (int j = 0; j < U; ++j) v[j] ^= w[j];
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
            if constexpr (NT) __builtin_nontemporal_store(v[j], o + i + j * S);
            else o[i + j * S] = v[j];
        }
    }
    for (; i < n16; i += S) {
        u32x4 v = ld(a + i);
        if constexpr (TWO) v ^= ld(b + i);
        if constexpr (NT) __builtin_nontemporal_store(v, o + i);
        else o[i] = v;
    }
}

hipError_t launch_stream_probe(const void* a, const void* b, void* out, size_t bytes, int unroll,
                               int nontemporal, int wg_per_cu, int cus, hipStream_t s) {
    const int64_t n16 = (int64_t)(bytes / 16);
    int64_t grid = (int64_t)cus * wg_per_cu;
    const int64_t need = (n16 + 255) / 256;
    if (grid > need) grid = need;
    if (grid < 1) grid = 1;
    const dim3 g((unsigned)grid), blk(256);
    const u32x4 *pa = (const u32x4*)a, *pb = (const u32x4*)b;
    u32x4* po = (u32x4*)out;
    auto go = [&](auto u, auto two, auto nt) {
        return launch(stream_probe_kernel<decltype(u)::value, decltype(two)::value != 0, decltype(nt)::value != 0>, g,
                      blk, 0, s, pa, pb, po, n16);
    };
    auto by_nt = [&](auto u, auto two) { return nontemporal ? go(u, two, IC<1>{}) : go(u, two, IC<0>{}); };
    auto by_two = [&](auto u) { return b ? by_nt(u, IC<1>{}) : by_nt(u, IC<0>{}); };
    switch (unroll) {
    case 1: return by_two(IC<1>{});
    case 2: return by_two(IC<2>{});
    case 4: return by_two(IC<4>{});
    case 8: return by_two(IC<8>{});
    default: return hipErrorInvalidValue;
    }
}

}  // namespace rwn
