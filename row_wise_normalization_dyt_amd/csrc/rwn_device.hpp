// Device-side building blocks shared by the DyT, LayerNorm and RMSNorm kernels (gfx950).
//
// Thread -> data map used by every row kernel
// -------------------------------------------
// A workgroup of `block` threads holds `rpp` row slots of `tpr` threads each (block = rpp*tpr).
// The thread with local id t owns slot t / tpr and lane t % tpr.  A row is cut into 16-byte
// chunks (V elements: 4 float32 or 8 bfloat16); lane l owns chunks l, l + tpr, ...,
// l + (CPT-1)*tpr of every row it visits, so consecutive lanes touch consecutive 16-byte
// chunks (coalesced) and a thread's columns never change while it walks rows.  That is what
// lets the backward keep its parameter-gradient partials in registers.
//
// Three modes handle every N and base address:
//   ALIGNED  N % V == 0 and 16-byte-aligned rows: chunk c covers columns [cV, cV+V).
//   SHIFTED  any N: row r starts s = (b + rN) mod V elements past a 16-byte boundary; chunk c
//            covers columns [cV - s, cV - s + V).  The launcher makes every thread visit rows
//            that share one s (grid * rpp divisible by V), so the column map is still fixed.
//            Chunks cut by the row ends are loaded/stored element by element.
//   SCALAR   V = 1 (strided rows of mixed alignment).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace rwn {

template <int V> using IC = std::integral_constant<int, V>;

typedef __bf16 bf16_t;
typedef _Float16 f16_t;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

enum Mode { MODE_ALIGNED = 0, MODE_SHIFTED = 1, MODE_SCALAR = 2 };

template <typename T> struct ChunkOf;
template <> struct ChunkOf<float> { static constexpr int value = 4; };
template <> struct ChunkOf<bf16_t> { static constexpr int value = 8; };
template <> struct ChunkOf<f16_t> { static constexpr int value = 8; };

template <typename T, int MODE>
struct Elems { static constexpr int value = (MODE == MODE_SCALAR) ? 1 : ChunkOf<T>::value; };

// Strided row operands (layout 1 kernels).  The M rows are the index space of up to three
// leading dimensions of sizes (s0, d1, d2), the last fastest: row r is (i0, i1, i2) with
// i2 = r mod d2, i1 = (r div d2) mod d1, i0 = r div (d2 d1); operand k's row starts st[k][0] i0 +
// st[k][1] i1 + st[k][2] i2 elements past its base, and its N elements are contiguous.  The
// divisions are multiplications by precomputed reciprocals (exact for r < 2^31: see
// make_divisor), since rows are mapped once per tile.
enum RowOperand { OP_X = 0, OP_DY = 1, OP_OUT = 2 };

struct Divisor {
    uint64_t m;   // ceil(2^sh / d)
    int sh;       // 31 + ceil(log2 d)
    uint32_t d;
};

// floor(n / d) for n < 2^31: with 2^l >= d and m = ceil(2^(31+l) / d) = (2^(31+l) + e) / d,
// 0 <= e < d, n m / 2^(31+l) = n / d + n e / (d 2^(31+l)), and the second term is below 1/d
// because n e < 2^31 2^l; floor(n / d) + frac <= floor(n / d) + (d - 1) / d, so the sum stays
// below the next integer.  m <= 2^32, so n m < 2^63.
__host__ __device__ inline Divisor make_divisor(uint32_t d) {
    int l = 0;
    while (l < 31 && (uint64_t(1) << l) < d) ++l;
    Divisor v;
    v.d = d;
    v.sh = 31 + l;
    v.m = ((uint64_t(1) << v.sh) + d - 1) / d;
    return v;
}
__host__ __device__ inline uint32_t div_by(uint32_t n, const Divisor& v) {
    return (uint32_t)(((uint64_t)n * v.m) >> v.sh);
}

struct RowMap {
    Divisor d1, d2;
    int64_t st[3][3];    // [operand][leading dimension] element strides
    int64_t span[3];     // bytes from an operand's base to the end of its last row
};

// Launch geometry shared by all row kernels (values computed by the host planner).
struct Geom {
    int64_t M, N;
    int64_t ntiles;   // number of row tiles; a tile is rpp * RT rows
    int64_t kt;       // blocked assignment: tiles per workgroup
    int64_t ws_rs;    // backward workspace: element (partial row p, column c) is at
    int64_t ws_cs;    //   ws[p * ws_rs + c * ws_cs]
    int tpr;          // threads per row
    int rpp;          // row slots per workgroup
    int base_shift;   // SHIFTED: misalignment of the [M, N] base address, in elements
    int strided;      // 1: workgroup w visits tiles w, w + grid, ...; 0: tiles [w*kt, (w+1)*kt)
    int ncb;          // column blocks per row (DyT only; 1 otherwise): workgroup w keeps
                      // column block w % ncb and strides over tiles by grid / ncb
    int xcd_remap;    // 1: renumber workgroups so consecutive numbers share an XCD (grid % 8 == 0)
    float inv_n;      // 1 / N
    float w_offset;   // RMSNorm: added to the weight in float32 (1 for the (1 + weight) form)
    int64_t pitch;    // SHIFTED: elements between consecutive rows' starts, for their shifts (N;
                      // 0 for strided operands, whose rows all share the base's shift)
    int64_t ps0, ps1; // element strides of the first and second parameter vectors
    RowMap rm;        // strided operands (layout 1 kernels)
};

// Element offset of row `row` in operand `op`: row * N for dense [M, N] operands (LAY 0), the
// row map's for strided ones (LAY 1).
template <int LAY>
__device__ __forceinline__ int64_t row_base(const Geom& g, int op, int64_t row) {
    if constexpr (LAY == 0) {
        return row * g.N;
    } else {
        const uint32_t r = (uint32_t)row;
        const uint32_t q = div_by(r, g.rm.d2);
        const uint32_t i2 = r - q * g.rm.d2.d;
        const uint32_t i0 = div_by(q, g.rm.d1);
        const uint32_t i1 = q - i0 * g.rm.d1.d;
        return (int64_t)i0 * g.rm.st[op][0] + (int64_t)i1 * g.rm.st[op][1] + (int64_t)i2 * g.rm.st[op][2];
    }
}

// ------------------------------------------------------------------------- conversions

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return (float)v; }
__device__ __forceinline__ float to_f32(f16_t v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// gfx950 lowers this to v_cvt_pk_bf16_f32: round to nearest even, NaN preserved.
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return (bf16_t)v; }
// v_cvt_f16_f32 under the default mode: round to nearest even, overflow to +-inf.
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float v) { return (f16_t)v; }

// float32 value of the 16-bit storage element held in the low half of `bits`.
template <typename T> __device__ __forceinline__ float half_bits_to_f32(uint32_t bits) {
    if constexpr (std::is_same<T, bf16_t>::value)
        return __builtin_bit_cast(float, bits << 16);
    else
        return (float)__builtin_bit_cast(f16_t, (unsigned short)bits);
}

// The float32 value of v after a round trip through storage dtype T.  For float16 the float32
// value is materialized first: otherwise the compiler may fuse the product that feeds it and
// the conversion into one mixed-precision FMA (v_fma_mixlo_f16) that rounds once, straight to
// float16, where a rounding point asks for the float32 product rounded to float16.
template <typename T> __device__ __forceinline__ float round_through(float v) {
    if constexpr (std::is_same<T, f16_t>::value) asm volatile("" : "+v"(v));
    return to_f32(from_f32<T>(v));
}

// Per-thread column map: which columns each of the CPT chunks covers (fixed for all rows the
// thread visits) and whether the chunk is whole inside the row.
template <typename T, int MODE, int CPT>
struct ColMap {
    static constexpr int V = Elems<T, MODE>::value;
    int col0[CPT];      // column of element 0 of chunk k (may be negative in SHIFTED mode)
    bool full[CPT];     // all V columns inside [0, N)
    bool any[CPT];      // at least one column inside [0, N)
    int shift;          // SHIFTED: s of this thread's rows
    // SHIFTED only (fixed per thread, so computed once): the bits of each 32-bit word of chunk
    // k that hold elements inside the row.  Kept as vector registers, they turn the masks of the
    // row loop into one AND per loaded word, and an element's own mask is derived from them
    // where needed (row_mask, in_row) with shifts instead of per-element compares.
    uint32_t keep[CPT][4];

    __device__ __forceinline__ void init(int lane, int tpr, int64_t N, int s, int chunk_base = 0) {
        shift = s;
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            int c = chunk_base + lane + k * tpr;
            int j0 = c * V - (MODE == MODE_SHIFTED ? s : 0);
            col0[k] = j0;
            full[k] = (j0 >= 0) && ((int64_t)j0 + V <= N);
            any[k] = ((int64_t)j0 + V > 0) && ((int64_t)j0 < N);
            if constexpr (MODE == MODE_SHIFTED) {
#pragma unroll
                for (int w = 0; w < 4; ++w) keep[k][w] = 0u;
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    const bool in = j0 + v >= 0 && (int64_t)(j0 + v) < N;
                    if (in) {
                        if constexpr (sizeof(T) == 4) keep[k][v] = 0xFFFFFFFFu;
                        else keep[k][v >> 1] |= (v & 1) ? 0xFFFF0000u : 0x0000FFFFu;
                    }
                }
            }
        }
    }
    // SHIFTED: all ones for element v of chunk k inside the row, zero outside.
    __device__ __forceinline__ uint32_t row_mask(int k, int v) const {
        if constexpr (sizeof(T) == 4) return keep[k][v];
        else return (uint32_t)((int32_t)((v & 1) ? keep[k][v >> 1] : keep[k][v >> 1] << 16) >> 31);
    }
    __device__ __forceinline__ bool in_row(int k, int v) const { return row_mask(k, v) != 0u; }
    __device__ __forceinline__ bool valid(int k, int v, int64_t N) const {
        if (MODE == MODE_SHIFTED) {
            int j = col0[k] + v;
            return j >= 0 && (int64_t)j < N;
        }
        return any[k];
    }
};

// The raw 16-byte chunks of one row slice, kept packed in registers (a bfloat16 pair per
// 32-bit word) and converted to float32 on use.  SCALAR mode keeps one element per word.
template <typename T, int MODE, int CPT>
struct RowRegs {
    static constexpr int V = Elems<T, MODE>::value;
    static constexpr int W = (MODE == MODE_SCALAR) ? 1 : 4;   // 32-bit words per chunk
    uint32_t w[CPT][W];

    __device__ __forceinline__ float get(int k, int v) const {
        if constexpr (sizeof(T) == 4) {
            return __builtin_bit_cast(float, w[k][MODE == MODE_SCALAR ? 0 : v]);
        } else {
            if (MODE == MODE_SCALAR) return half_bits_to_f32<T>(w[k][0]);
            const uint32_t u = w[k][v >> 1];
            if constexpr (std::is_same<T, bf16_t>::value)
                return __builtin_bit_cast(float, (v & 1) ? (u & 0xFFFF0000u) : (u << 16));
            else
                return half_bits_to_f32<T>((v & 1) ? (u >> 16) : u);
        }
    }
};

// ------------------------------------------------------------------ buffer loads
// Row loads go through buffer descriptors rather than flat pointers.  A buffer load whose
// offset lies past the descriptor's record count returns zeros without touching memory, so a
// padded row or column needs no branch around its load: its offset is simply pushed out of
// range.  Branch-free loads are what let the compiler keep the next tile's loads in flight
// while the current one is used (a load under a branch forces a full wait after it).
//
// One descriptor covers one row tile of one tensor: its base is the tile's first element
// (SHIFTED: the 16-byte block holding it), its record count the bytes from there to the
// tensor's end (rounded up to 16: the aligned block that holds the last element), capped at
// just below the out-of-range marker (2 GiB; a dense tile spans at most 16 rows of 16384
// float32, far less).
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr uint32_t kOutOfRange = 0x80000000u;   // above every record count
constexpr int64_t kMaxRecords = int64_t(kOutOfRange) - 16;
constexpr int kBufferFormat = 0x00020000;       // descriptor word 3: 32-bit data format
constexpr int kNontemporal = 2;                 // cache policy: streaming (nt)

// The descriptor's inputs are wave-uniform by construction (they depend only on the tile);
// reading them through readfirstlane states that to the compiler, which otherwise may not
// prove it and would wrap every load in a loop over the distinct descriptors of the wave.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// A buffer offset chosen per lane (in range or kOutOfRange), made opaque so the compiler emits
// it as a select instead of splitting the access into a branch per case.
__device__ __forceinline__ uint32_t lane_offset(bool in, uint32_t off) {
    uint32_t o = in ? off : kOutOfRange;
    asm volatile("" : "+v"(o));
    return o;
}

__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
    bytes = bytes < 0 ? 0 : bytes > kMaxRecords ? kMaxRecords : bytes;
    const uint64_t b = uniform_u64(reinterpret_cast<uint64_t>(base));
    const int n = (int)__builtin_amdgcn_readfirstlane((uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(b), (short)0, n, kBufferFormat);
}

// Source of one tensor's row tile; e0 is the element index (relative to the tensor) at the
// descriptor's base.  `live` false makes every load of the tile read zeros.
struct TileSrc {
    Rsrc rsrc;
    int64_t e0;
};

// Dense operands (LAY 0) get one descriptor per row tile.  Strided operands (LAY 1) get one
// over the operand's whole span (at most kMaxRecords bytes, which the host checks): their rows
// need not lie in order, and every row shares the base's shift.
template <typename T, int MODE, int LAY = 0>
__device__ __forceinline__ TileSrc tile_src(const T* __restrict__ p, int64_t row0, const Geom& g, int op,
                                            bool live) {
    constexpr int V = Elems<T, MODE>::value;
    int64_t e0, bytes;
    if constexpr (LAY == 0) {
        e0 = row0 * g.N;
        if (MODE == MODE_SHIFTED) e0 -= (e0 + g.base_shift) % V;
        bytes = (g.M * g.N - e0) * (int64_t)sizeof(T);
    } else {
        e0 = MODE == MODE_SHIFTED ? -(int64_t)g.base_shift : 0;
        bytes = g.rm.span[op] - e0 * (int64_t)sizeof(T);
    }
    bytes = (bytes + 15) & ~int64_t(15);
    TileSrc t;
    t.rsrc = make_rsrc(reinterpret_cast<const char*>(p) + e0 * (int64_t)sizeof(T), live ? bytes : 0);
    t.e0 = e0;
    return t;
}

// One float32 per row (LayerNorm / RMSNorm statistics) of the tile starting at row0.
__device__ __forceinline__ Rsrc stats_src(const float* p, int64_t row0, int64_t M, bool live) {
    return p ? make_rsrc(p + row0, live ? (M - row0) * 4 : 0) : make_rsrc(nullptr, 0);
}

__device__ __forceinline__ float load_stat(Rsrc r, int64_t row, int64_t row0, bool ok) {
    const uint32_t off = lane_offset(ok, (uint32_t)((row - row0) * 4));
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

// Load the CPT chunks of the row starting at element rb (row_base) from the tile source; columns
// outside the row read as 0, and `rowvalid` false reads zeros.  Every chunk is one 16-byte load (SCALAR: one
// element).  A SHIFTED chunk cut by the row's ends holds elements of the neighbouring row (or,
// at the tensor's ends, bytes of the 16-byte block beyond it), which are zeroed after the load.
template <typename T, int MODE, int CPT>
__device__ __forceinline__ void load_row(const TileSrc& src, int64_t rb, const ColMap<T, MODE, CPT>& cm,
                                         bool rowvalid, RowRegs<T, MODE, CPT>& r) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        const bool in = rowvalid && cm.any[k];
        const uint32_t off = lane_offset(in, (uint32_t)((rb + cm.col0[k] - src.e0) * (int64_t)sizeof(T)));
        if (MODE == MODE_SCALAR) {
            if constexpr (sizeof(T) == 4)
                r.w[k][0] = __builtin_amdgcn_raw_buffer_load_b32(src.rsrc, off, 0, 0);
            else
                r.w[k][0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(src.rsrc, off, 0, 0);
        } else {
            u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(src.rsrc, off, 0, kNontemporal);
            if (MODE == MODE_SHIFTED) {
#pragma unroll
                for (int w = 0; w < 4; ++w) v[w] &= cm.keep[k][w];
            }
            r.w[k][0] = v[0]; r.w[k][1] = v[1]; r.w[k][2] = v[2]; r.w[k][3] = v[3];
        }
    }
}

// Stores go through the same tile descriptors as the loads (TileSrc of the output tensor).  A
// store whose offset lies past the record count writes nothing, so a masked lane issues its
// stores like every other lane, with no branch around them.  That keeps the number of memory
// operations a wave has issued the same on every path through the loop body, which is what
// lets the compiler wait for the next tile's loads alone: loads and stores share one in-order
// counter, and a store count that differs between paths makes it wait for everything,
// including the stores just issued.

__device__ __forceinline__ void store_b128(const TileSrc& d, bool in, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, d.rsrc, lane_offset(in, off), 0, kNontemporal);
}
__device__ __forceinline__ void store_b64(const TileSrc& d, bool in, uint32_t off, uint32_t lo, uint32_t hi) {
    __builtin_amdgcn_raw_buffer_store_b64((u32x2){lo, hi}, d.rsrc, lane_offset(in, off), 0, 0);
}
__device__ __forceinline__ void store_b32(const TileSrc& d, bool in, uint32_t off, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b32(v, d.rsrc, lane_offset(in, off), 0, 0);
}
__device__ __forceinline__ void store_b16(const TileSrc& d, bool in, uint32_t off, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, d.rsrc, lane_offset(in, off), 0, 0);
}

__device__ __forceinline__ uint32_t word_at(const u32x4& w, int i) {
    return i == 0 ? w[0] : i == 1 ? w[1] : i == 2 ? w[2] : w[3];
}

// V float32 values rounded to T, packed as the 16 bytes of one chunk.
template <typename T>
__device__ __forceinline__ u32x4 pack_chunk(const float* o) {
    if constexpr (sizeof(T) == 4) {
        return (u32x4){__builtin_bit_cast(uint32_t, o[0]), __builtin_bit_cast(uint32_t, o[1]),
                       __builtin_bit_cast(uint32_t, o[2]), __builtin_bit_cast(uint32_t, o[3])};
    } else {
        f32x8 f = {o[0], o[1], o[2], o[3], o[4], o[5], o[6], o[7]};
        if constexpr (std::is_same<T, bf16_t>::value)
            return __builtin_bit_cast(u32x4, __builtin_convertvector(f, bf16x8));
        else
            return __builtin_bit_cast(u32x4, __builtin_convertvector(f, f16x8));
    }
}

// Store chunk k of the row starting at element rb (row_base; N elements) into the tile
// destination d, from V float32 values
// rounded to T; only columns inside the row are written, nothing when `rowvalid` is false.  A
// whole chunk is one nontemporal 16-byte store.  A SHIFTED chunk cut by the row's ends covers
// bytes [a, b) of its aligned 16-byte block (the rest belongs to the neighbouring row); that
// range is written as naturally aligned 2-, 4- and 8-byte pieces: up to three rising from a to
// the next 16-byte boundary and up to three falling from there to b.  Every lane issues all
// of these stores, with out-of-range offsets for the pieces it does not need.
template <typename T, int MODE, int CPT>
__device__ __forceinline__ void store_chunk(const TileSrc& d, int64_t rb, int64_t N,
                                            const ColMap<T, MODE, CPT>& cm, int k, const float* o,
                                            bool rowvalid) {
    constexpr int V = ColMap<T, MODE, CPT>::V;
    constexpr int ES = (int)sizeof(T);
    const uint32_t off = (uint32_t)((rb + cm.col0[k] - d.e0) * (int64_t)ES);
    if constexpr (MODE == MODE_SCALAR) {
        const bool in = rowvalid && cm.any[k];
        if constexpr (ES == 4) store_b32(d, in, off, __builtin_bit_cast(uint32_t, o[0]));
        else store_b16(d, in, off, (uint32_t)__builtin_bit_cast(unsigned short, from_f32<T>(o[0])));
    } else {
        const u32x4 w = pack_chunk<T>(o);
        store_b128(d, rowvalid && (MODE == MODE_ALIGNED ? cm.any[k] : cm.full[k]), off, w);
        if constexpr (MODE == MODE_SHIFTED) {
            const bool cut = rowvalid && cm.any[k] && !cm.full[k];
            const int j0 = cm.col0[k];
            const int lo = j0 < 0 ? -j0 : 0;
            const int hi = (int64_t)j0 + V > N ? (int)(N - j0) : V;
            int a = cut ? lo * ES : 16;
            const int b = cut ? hi * ES : 16;
            if constexpr (ES == 2) {
                const bool p = (a & 2) && a < b;   // high half of word a / 4
                store_b16(d, p, off + a, word_at(w, a >> 2) >> 16);
                a += p ? 2 : 0;
            }
            {
                const bool p = (a & 4) && a + 4 <= b;   // word 1 or 3
                store_b32(d, p, off + a, (a & 8) ? w[3] : w[1]);
                a += p ? 4 : 0;
            }
            {
                const bool p = (a & 8) && a + 8 <= b;   // a == 8: words 2, 3
                store_b64(d, p, off + 8, w[2], w[3]);
                a += p ? 8 : 0;
            }
            {
                const bool p = b - a >= 8;   // only from a == 0: words 0, 1
                store_b64(d, p, off, w[0], w[1]);
                a += p ? 8 : 0;
            }
            {
                const bool p = b - a >= 4;
                store_b32(d, p, off + a, word_at(w, a >> 2));
                a += p ? 4 : 0;
            }
            if constexpr (ES == 2) {
                const bool p = b - a >= 2;   // low half of word a / 4
                store_b16(d, p, off + a, word_at(w, a >> 2) & 0xFFFFu);
            }
        }
    }
}

// Store chunk k of the row of p starting at element rb with global stores under the row mask:
// a whole chunk is one nontemporal 16-byte store, a SHIFTED chunk cut by the row's ends is
// written element by element.
template <typename T, int MODE, int CPT>
__device__ __forceinline__ void store_chunk(T* __restrict__ p, int64_t rb, int64_t N,
                                            const ColMap<T, MODE, CPT>& cm, int k, const float* o,
                                            bool rowvalid) {
    constexpr int V = ColMap<T, MODE, CPT>::V;
    if (!rowvalid || !cm.any[k]) return;
    T* rp = p + rb + cm.col0[k];
    if constexpr (MODE == MODE_SCALAR) {
        *rp = from_f32<T>(o[0]);
    } else if (MODE == MODE_ALIGNED || cm.full[k]) {
        __builtin_nontemporal_store(pack_chunk<T>(o), reinterpret_cast<u32x4*>(rp));
    } else {
#pragma unroll
        for (int v = 0; v < V; ++v)
            if (cm.in_row(k, v)) rp[v] = from_f32<T>(o[v]);
    }
}

// Which of the two store forms a kernel uses (measured): the branch-free buffer stores pay in
// backward kernels over wide aligned rows (two or more chunks per lane), whose loops carry
// the most loads in flight; elsewhere the masked global stores are as fast or faster (their
// descriptors cost scalar work per tile, and SHIFTED cut chunks take six piece stores).
template <int MODE, int CPT, bool BWD>
constexpr bool kBufferStores = BWD && MODE == MODE_ALIGNED && CPT >= 2;

template <typename T, int MODE, int CPT, bool BUF>
__device__ __forceinline__ void put_chunk(T* __restrict__ p, const TileSrc& d, int64_t rb, int64_t N,
                                          const ColMap<T, MODE, CPT>& cm, int k, const float* o,
                                          bool rowvalid) {
    if constexpr (BUF) store_chunk<T, MODE, CPT>(d, rb, N, cm, k, o, rowvalid);
    else store_chunk<T, MODE, CPT>(p, rb, N, cm, k, o, rowvalid);
}


// Load a per-column parameter vector (element stride ps) for this thread's columns (0 outside
// [0, N)).
template <typename T, typename PT, int MODE, int CPT>
__device__ __forceinline__ void load_param(const PT* __restrict__ p, int64_t N, int64_t ps,
                                           const ColMap<T, MODE, CPT>& cm, float* o) {
    constexpr int V = ColMap<T, MODE, CPT>::V;
#pragma unroll
    for (int k = 0; k < CPT; ++k)
#pragma unroll
        for (int v = 0; v < V; ++v) {
            int j = cm.col0[k] + v;
            o[k * V + v] = (j >= 0 && (int64_t)j < N && cm.any[k]) ? to_f32(p[j * ps]) : 0.f;
        }
}

// ------------------------------------------------------------------- row reductions
// All reductions must be called by every lane of the wave (uniform control flow): DPP and
// swizzle read neighbouring lanes.  Each step adds a value and its partner's; since float
// addition is commutative both lanes of a pair get the same bits, so every lane of a group
// ends with the identical sum.

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 CTRL, 0xF, 0xF, false));
}
constexpr int DPP_QUAD_XOR1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

__device__ __forceinline__ float swizzle_xor16(float v) {
    // ds_swizzle bit mode: and_mask 0x1F, or_mask 0, xor_mask 0x10 (within 32-lane halves).
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over aligned groups of `g` lanes (g a power of two, 1..64); result in every lane.
__device__ __forceinline__ float group_sum(float v, int g) {
    if (g >= 2) v += dpp_f<DPP_QUAD_XOR1>(v);
    if (g >= 4) v += dpp_f<DPP_QUAD_XOR2>(v);
    if (g >= 8) v += dpp_f<DPP_ROW_HALF_MIRROR>(v);
    if (g >= 16) v += dpp_f<DPP_ROW_MIRROR>(v);
    if (g >= 32) v += swizzle_xor16(v);
    if (g >= 64) v = readlane_f(v, 0) + readlane_f(v, 32);
    return v;
}

// Most waves a workgroup has (1024 threads).
constexpr int kMaxWaves = 16;

// Row sums for K values per thread.  Rows of up to 64 threads reduce inside their wave; rows
// spanning W = tpr/64 waves add the W wave sums from LDS in wave order.  `red` holds
// 2 * kMaxWaves * K floats; `parity` alternates between the two halves so one barrier per
// reduction is enough.  (The halves are sized by the bound rather than by blockDim, whose
// read is a memory load that would make the wave wait for all of its loads in flight.)
template <int K>
__device__ __forceinline__ void row_sum(float (&v)[K], int tpr, float* red, int& parity) {
    // The group size is uniform: one scalar branch picks a straight-line sum for it, instead
    // of a branch around every step.
    auto sums = [&](auto gc) {
#pragma unroll
        for (int i = 0; i < K; ++i) v[i] = group_sum(v[i], decltype(gc)::value);
    };
    if (tpr >= 64) sums(IC<64>{});
    else if (tpr == 32) sums(IC<32>{});
    else if (tpr == 16) sums(IC<16>{});
    else if (tpr == 8) sums(IC<8>{});
    else if (tpr == 4) sums(IC<4>{});
    else if (tpr == 2) sums(IC<2>{});
    if (tpr > 64) {
        const int wave = threadIdx.x >> 6;
        float* buf = red + parity * kMaxWaves * K;
        if ((threadIdx.x & 63) == 0) {
#pragma unroll
            for (int i = 0; i < K; ++i) buf[wave * K + i] = v[i];
        }
        __syncthreads();
        const int w_per_row = tpr >> 6;
        const int first = (wave / w_per_row) * w_per_row;
#pragma unroll
        for (int i = 0; i < K; ++i) {
            float s = buf[first * K + i];
            for (int w = 1; w < w_per_row; ++w) s += buf[(first + w) * K + i];
            v[i] = s;
        }
        parity ^= 1;
    }
}

// Sum of one value over the whole workgroup, in wave order; valid in thread 0.
__device__ __forceinline__ float block_sum(float v, float* scratch) {
    v = group_sum(v, 64);
    const int nw = blockDim.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
    __syncthreads();
    float s = 0.f;
    if (threadIdx.x == 0) {
        s = scratch[0];
        for (int w = 1; w < nw; ++w) s += scratch[w];
    }
    return s;
}

// ------------------------------------------------------------------- tanh and sech^2
// From e = exp(-2|z|): tanh|z| = (1 - e) / (1 + e) and sech^2 z = 4e / (1 + e)^2, both
// without cancellation except 1 - e near z = 0.  For |z| >= 1/32, 1 - e >= 0.06, so the
// rounding of e (and the exp2 instruction's error) costs at most ~4e-6 relative in tanh.  Below
// that, tanh uses its Taylor series z - z^3/3, whose truncation error (2/15) z^4 is below 1.3e-7
// relative there.  z = +-inf gives e = 0: tanh = +-1, sech^2 = 0 exactly.
struct TanhSech2 { float t, s; };

__device__ __forceinline__ TanhSech2 tanh_sech2(float z) {
    const float az = __builtin_fabsf(z);
    const float e = __builtin_amdgcn_exp2f(-2.8853900817779268f * az);   // 2 * log2(e)
    // q2 = 2 / (1 + e) from the halved denominator: scaling by 2 is exact, so t and s come out
    // bitwise as from q = 1 / (1 + e), with one multiply less for s = e * q2 * q2 = 4e q^2.
    const float q2 = __builtin_amdgcn_rcpf(__builtin_fmaf(0.5f, e, 0.5f));
    const float tb = __builtin_fmaf(-0.5f, e, 0.5f) * q2;
    const float ts = z * __builtin_fmaf(z * z, -0.33333333333333333f, 1.0f);
    TanhSech2 r;
    r.t = az < 0.03125f ? ts : __builtin_copysignf(tb, z);
    r.s = e * q2 * q2;
    return r;
}

__device__ __forceinline__ float tanh_only(float z) {
    const float az = __builtin_fabsf(z);
    const float e = __builtin_amdgcn_exp2f(-2.8853900817779268f * az);
    const float tb = (1.0f - e) * __builtin_amdgcn_rcpf(1.0f + e);
    const float ts = z * __builtin_fmaf(z * z, -0.33333333333333333f, 1.0f);
    return az < 0.03125f ? ts : __builtin_copysignf(tb, z);
}

}  // namespace rwn
