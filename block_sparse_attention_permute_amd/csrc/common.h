// Internal helpers shared by the libbsa sources: status reporting, argument
// checks, fast integer division and bf16 conversions.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "bsa.h"

namespace bsa {

// ---------------------------------------------------------------- status ---

void set_error(const char* fmt, ...);
void clear_error();

#define BSA_FAIL(code, ...)            \
    do {                               \
        ::bsa::set_error(__VA_ARGS__); \
        return (code);                 \
    } while (0)

#define BSA_REQUIRE(cond, ...)                                \
    do {                                                      \
        if (!(cond)) BSA_FAIL(BSA_ERR_INVALID_ARG, __VA_ARGS__); \
    } while (0)

// Status of the most recent launch on this thread.
int check_launch(const char* what);

inline int elem_size(int dtype) { return dtype == BSA_BF16 ? 2 : (dtype == BSA_F32 ? 4 : 0); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ------------------------------------------------------ fast division -----
// Division by a run-time invariant divisor d >= 1 for dividends n < 2^31,
// by multiply-high and shift (Granlund & Montgomery, "Division by invariant
// integers using multiplication", 1994).
struct FastDiv {
    uint32_t d, magic, shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    f.shift = s;
    const uint64_t one = 1;
    f.magic = (uint32_t)(((one << 32) * ((one << s) - d)) / d + 1);
    return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
    uint32_t t = __umulhi(n, f.magic);
    return (t + n) >> f.shift;
}

__device__ __forceinline__ void fdivmod(uint32_t n, const FastDiv& f, uint32_t& q, uint32_t& r) {
    q = fdiv(n, f);
    r = n - q * f.d;
}

// ------------------------------------------------------ lane groups -----

// Sum over the LPT consecutive lanes that share a token row, with DPP lane
// swaps (VALU, no LDS): pairs, then quads (quad permutations), then the two
// quads of each 8-lane half (half-row mirror), then the two halves of a
// 16-lane row (row mirror); across 16-lane rows a shuffle.  Every step reads
// lanes of the same group only.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int LPT>
__device__ __forceinline__ float group_sum(float x) {
    if (LPT >= 2) x += dpp_f32<0xB1>(x);   // quad_perm [1, 0, 3, 2]
    if (LPT >= 4) x += dpp_f32<0x4E>(x);   // quad_perm [2, 3, 0, 1]
    if (LPT >= 8) x += dpp_f32<0x141>(x);  // row_half_mirror
    if (LPT >= 16) x += dpp_f32<0x140>(x); // row_mirror
    if (LPT >= 32) x += __shfl_xor(x, 16);
    return x;
}

// A 16-byte slice of a token row as EPV floats (8 bf16 or 4 fp32 values).
template <int EPV>
__device__ __forceinline__ void unpack(const uint4 raw, float (&v)[EPV]) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    if (EPV == 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < EPV; ++i) v[i] = __uint_as_float(w[i]);
    }
}

// Running elementwise max and min of 16-byte row slices (block summaries).
// bf16 (EPV 8) works on the bits: a pair of bf16 read as two int16 and
// mapped by key(x) = x ^ ((x >> 15) & 0x7fff), which flips the magnitude
// bits of negative values, orders like the values (-0 just below +0) and is
// its own inverse; a pair then costs two packed int16 operations for the key
// and one each for max and min (as floats, each value also needs a
// canonicalisation before a max or min).  fp32 (EPV 4) keeps float max/min.
typedef short s16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_key(uint32_t w) {
    const s16x2 x = __builtin_bit_cast(s16x2, w);
    const s16x2 s = x >> (s16x2){15, 15};
    return __builtin_bit_cast(uint32_t, x ^ (s & (s16x2){0x7fff, 0x7fff}));
}

template <int EPV>
struct RowRange {
    uint32_t hi[4], lo[4];  // EPV 8: keys of bf16 pairs; EPV 4: fp32 bits
    __device__ __forceinline__ void init() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // -inf and +inf: what a row range with nothing added reports
            hi[i] = EPV == 8 ? bf16x2_key(0xff80ff80u) : 0xff800000u;
            lo[i] = EPV == 8 ? bf16x2_key(0x7f807f80u) : 0x7f800000u;
        }
    }
    __device__ __forceinline__ void merge(const uint32_t (&h)[4], const uint32_t (&l)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (EPV == 8) {
                hi[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(s16x2, hi[i]),
                                                                              __builtin_bit_cast(s16x2, h[i])));
                lo[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(s16x2, lo[i]),
                                                                              __builtin_bit_cast(s16x2, l[i])));
            } else {
                hi[i] = __float_as_uint(fmaxf(__uint_as_float(hi[i]), __uint_as_float(h[i])));
                lo[i] = __float_as_uint(fminf(__uint_as_float(lo[i]), __uint_as_float(l[i])));
            }
        }
    }
    __device__ __forceinline__ void add(const uint4 raw) {
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
        uint32_t k[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) k[i] = EPV == 8 ? bf16x2_key(w[i]) : w[i];
        merge(k, k);
    }
    // with the lanes `off` apart (shuffles)
    __device__ __forceinline__ void merge_lanes(int off) {
        uint32_t h[4], l[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            h[i] = __shfl_xor(hi[i], off);
            l[i] = __shfl_xor(lo[i], off);
        }
        merge(h, l);
    }
    __device__ __forceinline__ uint4 max_row() const { return row(hi); }
    __device__ __forceinline__ uint4 min_row() const { return row(lo); }

  private:
    __device__ __forceinline__ static uint4 row(const uint32_t (&v)[4]) {
        if (EPV == 8) return make_uint4(bf16x2_key(v[0]), bf16x2_key(v[1]), bf16x2_key(v[2]), bf16x2_key(v[3]));
        return make_uint4(v[0], v[1], v[2], v[3]);
    }
};

// -------------------------------------------------------- conversions -----

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Round to nearest, ties to even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------- tilings -------
// One candidate tiling (a, b, c) of a T x Hg x Wg grid.  Tiles are numbered
// T-major over the (T/a) x (Hg/b) x (Wg/c) tile grid and cells T-major inside
// a tile, so permuted position p = tile * vol + cell.
struct TileGeo {
    uint32_t a, b, c, nty, ntx, vol;
    FastDiv f_vol, f_ntyx, f_ntx, f_bc, f_c, f_a, f_b;
};

inline TileGeo make_geo(int Hg, int Wg, int a, int b, int c) {
    TileGeo g;
    g.a = a;
    g.b = b;
    g.c = c;
    g.nty = Hg / b;
    g.ntx = Wg / c;
    g.vol = a * b * c;
    g.f_vol = make_fastdiv(g.vol);
    g.f_ntyx = make_fastdiv(g.nty * g.ntx);
    g.f_ntx = make_fastdiv(g.ntx);
    g.f_bc = make_fastdiv(b * c);
    g.f_c = make_fastdiv(c);
    g.f_a = make_fastdiv(a);
    g.f_b = make_fastdiv(b);
    return g;
}

// Every candidate must divide the grid ([Adaptive tiling (SPADE), "Deviations
// and notes": divisible grids only]).
// The same tiling on the grid padded up to a multiple of the tile along every
// axis ([Adaptive tiling (SPADE), "Deviations and notes": pad with zero
// tokens]): the tile grid is ceil(T/a) x ceil(Hg/b) x ceil(Wg/c) and cells
// outside T x Hg x Wg are padding.
inline TileGeo make_geo_padded(int Hg, int Wg, int a, int b, int c) {
    TileGeo g = make_geo(Hg, Wg, a, b, c);
    g.nty = (Hg + b - 1) / b;
    g.ntx = (Wg + c - 1) / c;
    g.f_ntyx = make_fastdiv(g.nty * g.ntx);
    g.f_ntx = make_fastdiv(g.ntx);
    return g;
}

// Padded length T' * Hg' * Wg' of a tiling, or -1 for bad arguments.
inline int64_t padded_length(int T, int Hg, int Wg, int a, int b, int c) {
    if (T <= 0 || Hg <= 0 || Wg <= 0 || a <= 0 || b <= 0 || c <= 0) return -1;
    return (int64_t)((T + a - 1) / a * a) * ((Hg + b - 1) / b * b) * ((Wg + c - 1) / c * c);
}

// Candidates of a padded tiling only need positive extents.
inline int check_tiles_padded(int T, int Hg, int Wg, const int32_t* tiles, int n_tiles) {
    BSA_REQUIRE(tiles != nullptr, "tiles is NULL");
    BSA_REQUIRE(n_tiles >= 1 && n_tiles <= BSA_MAX_TILINGS, "n_tiles=%d must be in [1, %d]", n_tiles,
                BSA_MAX_TILINGS);
    BSA_REQUIRE(T > 0 && Hg > 0 && Wg > 0, "grid must be positive");
    for (int i = 0; i < n_tiles; ++i) {
        const int a = tiles[3 * i], b = tiles[3 * i + 1], c = tiles[3 * i + 2];
        BSA_REQUIRE(a > 0 && b > 0 && c > 0, "tile %d (%d,%d,%d) must be positive", i, a, b, c);
    }
    return BSA_OK;
}

inline int check_tiles(int T, int Hg, int Wg, const int32_t* tiles, int n_tiles) {
    BSA_REQUIRE(tiles != nullptr, "tiles is NULL");
    BSA_REQUIRE(n_tiles >= 1 && n_tiles <= BSA_MAX_TILINGS, "n_tiles=%d must be in [1, %d]", n_tiles,
                BSA_MAX_TILINGS);
    for (int i = 0; i < n_tiles; ++i) {
        const int a = tiles[3 * i], b = tiles[3 * i + 1], c = tiles[3 * i + 2];
        BSA_REQUIRE(a > 0 && b > 0 && c > 0, "tile %d (%d,%d,%d) must be positive", i, a, b, c);
        BSA_REQUIRE(T % a == 0 && Hg % b == 0 && Wg % c == 0,
                    "candidate tile %d (%d,%d,%d) does not divide the grid %dx%dx%d", i, a, b, c, T, Hg, Wg);
    }
    return BSA_OK;
}

// T-major index of the first token of tile `tile`.
__device__ __forceinline__ uint32_t tile_origin(uint32_t tile, const TileGeo& g, uint32_t Hg, uint32_t Wg) {
    uint32_t tt, rem, ty, tx;
    fdivmod(tile, g.f_ntyx, tt, rem);
    fdivmod(rem, g.f_ntx, ty, tx);
    return ((tt * g.a) * Hg + ty * g.b) * Wg + tx * g.c;
}

// T-major offset of cell `cell` (T-major inside the tile) from the tile origin.
__device__ __forceinline__ uint32_t cell_offset(uint32_t cell, const TileGeo& g, uint32_t Hg, uint32_t Wg) {
    uint32_t rt, rem, ry, rx;
    fdivmod(cell, g.f_bc, rt, rem);
    fdivmod(rem, g.f_c, ry, rx);
    return (rt * Hg + ry) * Wg + rx;
}

// Permuted position p -> T-major token s.
__device__ __forceinline__ uint32_t perm_to_tmajor(uint32_t p, const TileGeo& g, uint32_t Hg, uint32_t Wg) {
    uint32_t tid, r, tt, rem, ty, tx, rt, rem2, ry, rx;
    fdivmod(p, g.f_vol, tid, r);
    fdivmod(tid, g.f_ntyx, tt, rem);
    fdivmod(rem, g.f_ntx, ty, tx);
    fdivmod(r, g.f_bc, rt, rem2);
    fdivmod(rem2, g.f_c, ry, rx);
    return ((tt * g.a + rt) * Hg + ty * g.b + ry) * Wg + tx * g.c + rx;
}

// Padded permuted position p -> T-major token of the unpadded grid, or -1
// for a padding cell (g from make_geo_padded).
__device__ __forceinline__ int32_t perm_to_tmajor_padded(uint32_t p, const TileGeo& g, uint32_t T, uint32_t Hg,
                                                         uint32_t Wg) {
    uint32_t tid, r, tt, rem, ty, tx, rt, rem2, ry, rx;
    fdivmod(p, g.f_vol, tid, r);
    fdivmod(tid, g.f_ntyx, tt, rem);
    fdivmod(rem, g.f_ntx, ty, tx);
    fdivmod(r, g.f_bc, rt, rem2);
    fdivmod(rem2, g.f_c, ry, rx);
    const uint32_t t = tt * g.a + rt, y = ty * g.b + ry, x = tx * g.c + rx;
    if (t >= T || y >= Hg || x >= Wg) return -1;
    return (int32_t)((t * Hg + y) * Wg + x);
}

}  // namespace bsa
