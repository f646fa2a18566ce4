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
#include "common.h"

namespace bsa {
namespace {

struct PermParams {
    const char* src;
    char* dst;
    uint32_t S, Hg, Wg;
    uint32_t items_per_head;  // S * vectors per row
    uint32_t vecs_per_row;
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
// output in permuted order; true: output in T-major order.
template <typename VecT, bool INVERSE>
__global__ __launch_bounds__(kThreads) void permute_rows_kernel(const PermParams P) {
    const uint32_t bh = blockIdx.y;
    uint32_t choice = 0;
    if (P.head_choice != nullptr) choice = (uint32_t)__builtin_amdgcn_readfirstlane(P.head_choice[bh]);
    if (choice >= P.n_tiles) choice = 0;  // out-of-range choices are caught by bsa_validate_indices
    const TileGeo& g = P.geo[choice];
    const size_t head_base = (size_t)bh * P.items_per_head;
    const VecT* __restrict__ src = reinterpret_cast<const VecT*>(P.src) + head_base;
    VecT* __restrict__ dst = reinterpret_cast<VecT*>(P.dst) + head_base;

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
            const uint32_t srow = INVERSE ? tmajor_to_perm(row, g, P) : perm_to_tmajor(row, g, P.Hg, P.Wg);
            buf[u] = src[(size_t)srow * P.vecs_per_row + vec];
        }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
        if (out_idx[u] < P.items_per_head) dst[out_idx[u]] = buf[u];
}

template <bool INVERSE>
int launch_permute(const void* in, void* out, int dtype, int64_t B, int64_t H, int T, int Hg, int Wg, int64_t D,
                   const int32_t* tiles, int n_tiles, const int32_t* head_choice, hipStream_t stream,
                   const char* name) {
    clear_error();
    const int es = elem_size(dtype);
    BSA_REQUIRE(es != 0, "%s: unknown dtype %d", name, dtype);
    BSA_REQUIRE(in != nullptr && out != nullptr, "%s: NULL tensor", name);
    BSA_REQUIRE(B >= 1 && H >= 1 && D >= 1, "%s: B, H, D must be >= 1", name);
    BSA_REQUIRE(T > 0 && Hg > 0 && Wg > 0, "%s: grid must be positive", name);
    int rc = check_tiles(T, Hg, Wg, tiles, n_tiles);
    if (rc) return rc;
    const int64_t S = (int64_t)T * Hg * Wg;
    const int64_t row_bytes = D * es;
    BSA_REQUIRE(B * H <= 65535, "%s: B*H=%lld too large", name, (long long)(B * H));
    const char* src = static_cast<const char*>(in);
    char* dst = static_cast<char*>(out);
    BSA_REQUIRE(dst + B * H * S * row_bytes <= src || src + B * H * S * row_bytes <= dst,
                "%s: input and output overlap", name);

    PermParams P;
    P.src = src;
    P.dst = dst;
    P.S = (uint32_t)S;
    P.Hg = Hg;
    P.Wg = Wg;
    P.f_HgWg = make_fastdiv((uint32_t)Hg * Wg);
    P.f_Wg = make_fastdiv(Wg);
    P.head_choice = head_choice;
    P.n_tiles = (uint32_t)n_tiles;
    for (int i = 0; i < BSA_MAX_TILINGS; ++i) {
        const int j = i < n_tiles ? i : 0;
        P.geo[i] = make_geo(Hg, Wg, tiles[3 * j], tiles[3 * j + 1], tiles[3 * j + 2]);
    }
    auto fits = [&](int v) {
        return row_bytes % v == 0 && reinterpret_cast<uintptr_t>(src) % v == 0 &&
               reinterpret_cast<uintptr_t>(dst) % v == 0;
    };
    int vec = 16;
    while (vec > 2 && !fits(vec)) vec >>= 1;
    BSA_REQUIRE(fits(vec), "%s: tensors are not 2-byte aligned", name);
    const int64_t vecs = row_bytes / vec;
    const int64_t items = S * vecs;
    BSA_REQUIRE(items < ((int64_t)1 << 31), "%s: a head has too many elements", name);
    P.vecs_per_row = (uint32_t)vecs;
    P.items_per_head = (uint32_t)items;
    P.f_vecs = make_fastdiv((uint32_t)vecs);

    dim3 grid((unsigned)((items + kThreads * kUnroll - 1) / (kThreads * kUnroll)), (unsigned)(B * H));
    switch (vec) {
        case 16: permute_rows_kernel<uint4, INVERSE><<<grid, kThreads, 0, stream>>>(P); break;
        case 8: permute_rows_kernel<uint2, INVERSE><<<grid, kThreads, 0, stream>>>(P); break;
        case 4: permute_rows_kernel<uint32_t, INVERSE><<<grid, kThreads, 0, stream>>>(P); break;
        default: permute_rows_kernel<uint16_t, INVERSE><<<grid, kThreads, 0, stream>>>(P); break;
    }
    return check_launch(name);
}

}  // namespace
}  // namespace bsa

using namespace bsa;

extern "C" int bsa_tile_permute(const void* x, void* y, int dtype, int64_t B, int64_t H, int T, int Hg, int Wg,
                                int64_t D, const int32_t* tiles_host, int n_tiles, const int32_t* head_choice,
                                bsa_stream_t stream) {
    return launch_permute<false>(x, y, dtype, B, H, T, Hg, Wg, D, tiles_host, n_tiles, head_choice,
                                 (hipStream_t)stream, "bsa_tile_permute");
}

extern "C" int bsa_invert_permute(const void* y, void* x, int dtype, int64_t B, int64_t H, int T, int Hg, int Wg,
                                  int64_t D, const int32_t* tiles_host, int n_tiles, const int32_t* head_choice,
                                  bsa_stream_t stream) {
    return launch_permute<true>(y, x, dtype, B, H, T, Hg, Wg, D, tiles_host, n_tiles, head_choice,
                                (hipStream_t)stream, "bsa_invert_permute");
}
