// Tile permutation of token rows: bsa_tile_permute and bsa_invert_permute.
//
// [Adaptive tiling (SPADE), "The idea" step 2 and "Recipe"]: q, k and v are
// reordered so that every tile of the chosen tiling is one contiguous run of
// tokens, and outputs are reordered back afterwards.
//
// Design: a pure gather in both directions (the output is written
// sequentially, the input is read in runs of c tokens, c the tile's x extent).
// The source index of every output row comes from integer arithmetic on the
// tile geometry (multiply-high divisions), so no permutation table is read.
// One workgroup covers a slice of one (b, h) row, so the head's tiling choice
// is uniform across the workgroup and is read once with a scalar load.
//
// Padded variants ([Adaptive tiling (SPADE), "Deviations and notes": pad the
// grid to a multiple of the tile with zero tokens]): the permuted side has
// Sp rows per head, Sp >= the padded length of every candidate; padding rows
// are written as zeros (and labelled -1 in an optional int32 label row, real
// rows 0), and the inverse reads only the real rows back.
#include "common.h"

#include <algorithm>

namespace bsa {
namespace {

struct PermParams {
    const char* src;
    char* dst;
    uint32_t S, T, Hg, Wg;
    uint32_t rows_in, rows_out;  // rows per head of src and dst
    uint32_t items_per_head;  // rows_out * vectors per row
    uint32_t vecs_per_row;
    int32_t* labels;          // padded gather only: (B, H, rows_out), or null
    FastDiv f_vecs, f_HgWg, f_Wg;
    const int32_t* head_choice;
    uint32_t n_tiles;
    TileGeo geo[BSA_MAX_TILINGS];
};

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

// T-major token s -> permuted position p.
__device__ __forceinline__ uint32_t tmajor_to_perm(uint32_t s, const TileGeo& g, const PermParams& P) {
    uint32_t t, rem, y, x, tt, rt, ty, ry, tx, rx;
    fdivmod(s, P.f_HgWg, t, rem);
    fdivmod(rem, P.f_Wg, y, x);
    fdivmod(t, g.f_a, tt, rt);
    fdivmod(y, g.f_b, ty, ry);
    fdivmod(x, g.f_c, tx, rx);
    return ((tt * g.nty + ty) * g.ntx + tx) * g.vol + (rt * g.b + ry) * g.c + rx;
}

// Output row `o` of one head reads input row src_row(o).  INVERSE = false:
// output in permuted order; true: output in T-major order.  PAD: the tilings
// are padded (geometry from make_geo_padded).
template <typename VecT, bool INVERSE, bool PAD>
__global__ __launch_bounds__(kThreads) void permute_rows_kernel(const PermParams P) {
    const uint32_t bh = blockIdx.y;
    uint32_t choice = 0;
    if (P.head_choice != nullptr) choice = (uint32_t)__builtin_amdgcn_readfirstlane(P.head_choice[bh]);
    if (choice >= P.n_tiles) choice = 0;  // out-of-range choices are caught by bsa_validate_indices
    const TileGeo& g = P.geo[choice];
    const VecT* __restrict__ src = reinterpret_cast<const VecT*>(P.src) + (size_t)bh * P.rows_in * P.vecs_per_row;
    VecT* __restrict__ dst = reinterpret_cast<VecT*>(P.dst) + (size_t)bh * P.items_per_head;

    const uint32_t first = blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
    VecT buf[kUnroll];
    uint32_t out_idx[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint32_t i = first + u * kThreads;
        out_idx[u] = i;
        if (i < P.items_per_head) {
            uint32_t row, vec;
            fdivmod(i, P.f_vecs, row, vec);
            if (PAD && !INVERSE) {
                const int32_t srow = perm_to_tmajor_padded(row, g, P.T, P.Hg, P.Wg);
                if (srow >= 0)
                    buf[u] = src[(size_t)srow * P.vecs_per_row + vec];
                else
                    buf[u] = VecT{};
                if (P.labels != nullptr && vec == 0) P.labels[(size_t)bh * P.rows_out + row] = srow >= 0 ? 0 : -1;
            } else {
                const uint32_t srow = INVERSE ? tmajor_to_perm(row, g, P) : perm_to_tmajor(row, g, P.Hg, P.Wg);
                buf[u] = src[(size_t)srow * P.vecs_per_row + vec];
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
        if (out_idx[u] < P.items_per_head) dst[out_idx[u]] = buf[u];
}

// Sp = 0: plain tilings (every candidate divides the grid).  Sp > 0: padded
// tilings with Sp rows per head on the permuted side.
template <bool INVERSE>
int launch_permute(const void* in, void* out, int dtype, int64_t B, int64_t H, int T, int Hg, int Wg, int64_t D,
                   const int32_t* tiles, int n_tiles, const int32_t* head_choice, int64_t Sp, int32_t* labels,
                   hipStream_t stream, const char* name) {
    clear_error();
    const int es = elem_size(dtype);
    BSA_REQUIRE(es != 0, "%s: unknown dtype %d", name, dtype);
    BSA_REQUIRE(in != nullptr && out != nullptr, "%s: NULL tensor", name);
    BSA_REQUIRE(B >= 1 && H >= 1 && D >= 1, "%s: B, H, D must be >= 1", name);
    BSA_REQUIRE(T > 0 && Hg > 0 && Wg > 0, "%s: grid must be positive", name);
    const bool pad = Sp > 0;
    int rc = pad ? check_tiles_padded(T, Hg, Wg, tiles, n_tiles) : check_tiles(T, Hg, Wg, tiles, n_tiles);
    if (rc) return rc;
    const int64_t S = (int64_t)T * Hg * Wg;
    if (pad) {
        int64_t need = 0;
        for (int i = 0; i < n_tiles; ++i)
            need = std::max(need, padded_length(T, Hg, Wg, tiles[3 * i], tiles[3 * i + 1], tiles[3 * i + 2]));
        BSA_REQUIRE(Sp >= need, "%s: Sp=%lld is shorter than the longest padded tiling (%lld)", name, (long long)Sp,
                    (long long)need);
        BSA_REQUIRE(Sp < ((int64_t)1 << 31), "%s: Sp too large", name);
    }
    const int64_t rows_perm = pad ? Sp : S;
    const int64_t rows_in = INVERSE ? rows_perm : S, rows_out = INVERSE ? S : rows_perm;
    const int64_t row_bytes = D * es;
    BSA_REQUIRE(B * H <= 65535, "%s: B*H=%lld too large", name, (long long)(B * H));
    const char* src = static_cast<const char*>(in);
    char* dst = static_cast<char*>(out);
    BSA_REQUIRE(dst + B * H * rows_out * row_bytes <= src || src + B * H * rows_in * row_bytes <= dst,
                "%s: input and output overlap", name);

    PermParams P;
    P.src = src;
    P.dst = dst;
    P.S = (uint32_t)S;
    P.T = (uint32_t)T;
    P.Hg = Hg;
    P.Wg = Wg;
    P.rows_in = (uint32_t)rows_in;
    P.rows_out = (uint32_t)rows_out;
    P.labels = (pad && !INVERSE) ? labels : nullptr;
    P.f_HgWg = make_fastdiv((uint32_t)Hg * Wg);
    P.f_Wg = make_fastdiv(Wg);
    P.head_choice = head_choice;
    P.n_tiles = (uint32_t)n_tiles;
    for (int i = 0; i < BSA_MAX_TILINGS; ++i) {
        const int j = i < n_tiles ? i : 0;
        P.geo[i] = pad ? make_geo_padded(Hg, Wg, tiles[3 * j], tiles[3 * j + 1], tiles[3 * j + 2])
                       : make_geo(Hg, Wg, tiles[3 * j], tiles[3 * j + 1], tiles[3 * j + 2]);
    }
    auto fits = [&](int v) {
        return row_bytes % v == 0 && reinterpret_cast<uintptr_t>(src) % v == 0 &&
               reinterpret_cast<uintptr_t>(dst) % v == 0;
    };
    int vec = 16;
    while (vec > 2 && !fits(vec)) vec >>= 1;
    BSA_REQUIRE(fits(vec), "%s: tensors are not 2-byte aligned", name);
    const int64_t vecs = row_bytes / vec;
    const int64_t items = rows_out * vecs;
    BSA_REQUIRE(items < ((int64_t)1 << 31) && rows_in * vecs < ((int64_t)1 << 31),
                "%s: a head has too many elements", name);
    P.vecs_per_row = (uint32_t)vecs;
    P.items_per_head = (uint32_t)items;
    P.f_vecs = make_fastdiv((uint32_t)vecs);

    dim3 grid((unsigned)((items + kThreads * kUnroll - 1) / (kThreads * kUnroll)), (unsigned)(B * H));
#define BSA_PERM(V)                                                                  \
    (pad ? permute_rows_kernel<V, INVERSE, true><<<grid, kThreads, 0, stream>>>(P) \
         : permute_rows_kernel<V, INVERSE, false><<<grid, kThreads, 0, stream>>>(P))
    switch (vec) {
        case 16: BSA_PERM(uint4); break;
        case 8: BSA_PERM(uint2); break;
        case 4: BSA_PERM(uint32_t); break;
        default: BSA_PERM(uint16_t); break;
    }
#undef BSA_PERM
    return check_launch(name);
}

}  // namespace
}  // namespace bsa

using namespace bsa;

extern "C" int bsa_tile_permute(const void* x, void* y, int dtype, int64_t B, int64_t H, int T, int Hg, int Wg,
                                int64_t D, const int32_t* tiles_host, int n_tiles, const int32_t* head_choice,
                                bsa_stream_t stream) {
    return launch_permute<false>(x, y, dtype, B, H, T, Hg, Wg, D, tiles_host, n_tiles, head_choice, 0, nullptr,
                                 (hipStream_t)stream, "bsa_tile_permute");
}

extern "C" int bsa_invert_permute(const void* y, void* x, int dtype, int64_t B, int64_t H, int T, int Hg, int Wg,
                                  int64_t D, const int32_t* tiles_host, int n_tiles, const int32_t* head_choice,
                                  bsa_stream_t stream) {
    return launch_permute<true>(y, x, dtype, B, H, T, Hg, Wg, D, tiles_host, n_tiles, head_choice, 0, nullptr,
                                (hipStream_t)stream, "bsa_invert_permute");
}

extern "C" int bsa_tile_permute_padded(const void* x, void* y, int dtype, int64_t B, int64_t H, int T, int Hg,
                                       int Wg, int64_t D, const int32_t* tiles_host, int n_tiles,
                                       const int32_t* head_choice, int64_t Sp, int32_t* labels_or_null,
                                       bsa_stream_t stream) {
    if (Sp <= 0) {
        clear_error();
        BSA_FAIL(BSA_ERR_INVALID_ARG, "bsa_tile_permute_padded: Sp must be > 0");
    }
    return launch_permute<false>(x, y, dtype, B, H, T, Hg, Wg, D, tiles_host, n_tiles, head_choice, Sp,
                                 labels_or_null, (hipStream_t)stream, "bsa_tile_permute_padded");
}

extern "C" int bsa_invert_permute_padded(const void* y, void* x, int dtype, int64_t B, int64_t H, int T, int Hg,
                                         int Wg, int64_t D, const int32_t* tiles_host, int n_tiles,
                                         const int32_t* head_choice, int64_t Sp, bsa_stream_t stream) {
    if (Sp <= 0) {
        clear_error();
        BSA_FAIL(BSA_ERR_INVALID_ARG, "bsa_invert_permute_padded: Sp must be > 0");
    }
    return launch_permute<true>(y, x, dtype, B, H, T, Hg, Wg, D, tiles_host, n_tiles, head_choice, Sp, nullptr,
                                (hipStream_t)stream, "bsa_invert_permute_padded");
}
