// Query cohesion per tile and per-head tiling choice: bsa_block_cohesion and
// bsa_select_tiling.
//
// [Adaptive tiling (SPADE), "The idea" step 1]: each candidate tiling is
// scored per head by the cohesion (SICS) of its tiles, the mean pairwise
// cosine of the queries inside a tile, and the most cohesive tiling is kept.
// [Adaptive tiling (SPADE), "Deviations and notes"]: tokens of zero norm are
// left out and the tiling score is the plain average of the per-tile values.
//
// Design: the mean over ordered pairs i != j of cos(q_i, q_j) equals
// (|sum_i q_i/|q_i||^2 - n) / (n (n - 1)), so a tile costs one pass over its
// tokens (O(vol * D)) instead of O(vol^2 * D).  One wave owns one tile and
// reads its tokens straight from the T-major tensor through the tile
// geometry, so no candidate tiling is ever materialised.  Per-tile values go
// to a caller-provided buffer and a second small kernel averages them per
// (b, h, candidate) in double in a fixed order, so results are deterministic.
//
// bsa_select_tiling_ex adds two variants of the same passes:
//  * padded candidates ([Adaptive tiling (SPADE), "Deviations and notes": pad
//    the grid to a multiple of the tile with zero tokens, left out of the
//    cohesion]): tiles run over the padded tile grid and only their real
//    cells are read, which is the same as reading zero padding and leaving
//    zero-norm tokens out;
//  * SPADE's pooled statistic ([same section, "Selection statistic"]: sum of
//    pair similarities over the number of pairs across the whole tiling,
//    zero-norm tokens counted): a tile contributes |sum u/|u||^2 - n_nonzero
//    to the numerator and n(n - 1) (n = its real tokens) to the denominator.
#include "common.h"

#include <algorithm>
#include <mutex>

namespace bsa {
namespace {

constexpr int kWaves = 4;
constexpr int kBatch = 8;  // tokens loaded per lane before use

struct CohParams {
    const char* x;
    int dtype;
    uint32_t S, T, Hg, Wg, D;
    uint32_t pad, pooled;
    uint32_t vecs_per_row;  // 16-byte vectors per token row
    uint32_t n_tiles, max_nb;
    uint32_t nb[BSA_MAX_TILINGS];
    TileGeo geo[BSA_MAX_TILINGS];
    float* tile_coh;  // [B*H][n_tiles][max_nb]
    // optional: each tile's elementwise max and min of q, in q's dtype,
    // [n_tiles][2][B*H][max_nb][D] (candidates of one volume, no padding)
    char* qsumm;
    uint32_t BH;
};

// 1 / sqrt(x) for x > 0 with the hardware's reciprocal square root (about
// 1 ulp); inputs below 2^-100 are scaled by 2^100 first, since the
// instruction does not take denormal inputs.
__device__ __forceinline__ float rsq(float x) {
    const bool tiny = x < 0x1p-100f;
    return __builtin_amdgcn_rsqf(tiny ? x * 0x1p100f : x) * (tiny ? 0x1p50f : 1.0f);
}

// LPT lanes cooperate on one token (16 bytes each); 64/LPT tokens per step.
// SUMM: also the tile's elementwise max and min of q (the block summaries of
// the tiling, read by the scores pass instead of q itself).
template <int EPV, int LPT, bool PAD, bool SUMM>
__global__ __launch_bounds__(64 * kWaves) void tile_cohesion_kernel(const CohParams P) {
    constexpr int TPI = 64 / LPT;
    const int lane = threadIdx.x & 63;
    // Workgroup order: (head, tile group, candidate), the candidate fastest,
    // and each XCD (workgroup w runs on XCD w % 8) a contiguous range of it.
    // The candidates' tiles of one group cover about the same frames (every
    // candidate has the same number of tiles per frame), so the candidates
    // after the first read q from the XCD's L2.
    uint32_t w = blockIdx.x;
    if (gridDim.x % 8u == 0u) w = (w & 7u) * (gridDim.x >> 3) + (w >> 3);
    const uint32_t cand = w % P.n_tiles;
    w /= P.n_tiles;
    const uint32_t groups = (P.max_nb + kWaves - 1) / kWaves;
    const uint32_t tile = (w % groups) * kWaves + (threadIdx.x >> 6);
    const uint32_t bh = w / groups;
    if (tile >= P.nb[cand]) return;
    const TileGeo& g = P.geo[cand];
    const uint32_t origin = PAD ? 0u : tile_origin(tile, g, P.Hg, P.Wg);
    uint32_t t0 = 0, y0 = 0, x0 = 0;
    if (PAD) {
        uint32_t tt, rem, ty, tx;
        fdivmod(tile, g.f_ntyx, tt, rem);
        fdivmod(rem, g.f_ntx, ty, tx);
        t0 = tt * g.a;
        y0 = ty * g.b;
        x0 = tx * g.c;
    }
    const size_t row_bytes = (size_t)P.vecs_per_row * 16;
    const char* head = P.x + (size_t)bh * P.S * row_bytes;
    const int sub = lane % LPT;   // which 16-byte slice of the row
    const int slot = lane / LPT;  // which token of the step

    float u[EPV];
#pragma unroll
    for (int i = 0; i < EPV; ++i) u[i] = 0.f;
    float n = 0.f;
    RowRange<EPV> range;
    range.init();
    // kBatch tokens per lane are loaded before any is used, so that many
    // loads are in flight per wave; a cell outside the tile or the grid loads
    // the head's first row and is then taken as a zero token.
    // (with the summaries, fewer rows in flight keep the register count down)
    constexpr int NB = SUMM ? kBatch / 2 : kBatch;
    for (uint32_t base = 0; base < g.vol; base += TPI * NB) {
        uint4 raw[NB];
        bool real[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const uint32_t cell = base + j * TPI + slot;
            real[j] = cell < g.vol;
            uint32_t s = 0;
            if (PAD) {
                uint32_t rt, rem, ry, rx;
                fdivmod(real[j] ? cell : 0u, g.f_bc, rt, rem);
                fdivmod(rem, g.f_c, ry, rx);
                real[j] = real[j] && t0 + rt < P.T && y0 + ry < P.Hg && x0 + rx < P.Wg;
                s = real[j] ? ((t0 + rt) * P.Hg + y0 + ry) * P.Wg + x0 + rx : 0u;
            } else {
                // (a cell past the tile reads the tile's first token: a member of the tile, so the
                // summaries may take it in again)
                s = origin + cell_offset(real[j] ? cell : 0u, g, P.Hg, P.Wg);
            }
            raw[j] = *reinterpret_cast<const uint4*>(head + (size_t)s * row_bytes + (size_t)sub * 16);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            float v[EPV];
            unpack<EPV>(raw[j], v);
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < EPV; ++i) ss = fmaf(v[i], v[i], ss);
            ss = group_sum<LPT>(ss);
            if (SUMM) range.add(raw[j]);
            if (real[j] && ss > 0.f) {
                const float inv = rsq(ss);
#pragma unroll
                for (int i = 0; i < EPV; ++i) u[i] = fmaf(v[i], inv, u[i]);
                n += 1.f;
            }
        }
    }
    // sum the normalised vectors over token slots (lanes with equal `sub`)
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
        for (int i = 0; i < EPV; ++i) u[i] += __shfl_xor(u[i], off);
        n += __shfl_xor(n, off);
    }
    if (SUMM) {
#pragma unroll
        for (int off = LPT; off < 64; off <<= 1) range.merge_lanes(off);
        if (slot == 0) {
            const size_t plane = (size_t)P.BH * P.max_nb * row_bytes;
            char* dst = P.qsumm + (size_t)(2 * cand) * plane + ((size_t)bh * P.max_nb + tile) * row_bytes +
                        (size_t)sub * 16;
            *reinterpret_cast<uint4*>(dst) = range.max_row();
            *reinterpret_cast<uint4*>(dst + plane) = range.min_row();
        }
    }
    float uu = 0.f;
#pragma unroll
    for (int i = 0; i < EPV; ++i) uu = fmaf(u[i], u[i], uu);
#pragma unroll
    for (int off = LPT / 2; off >= 1; off >>= 1) uu += __shfl_xor(uu, off);
    if (lane == 0) {
        // after the slot reduction n is the number of non-zero tokens
        const float cnt = n;
        const float sics = cnt >= 2.f ? (uu - cnt) / (cnt * (cnt - 1.f)) : __builtin_nanf("");
        P.tile_coh[((size_t)bh * P.n_tiles + cand) * P.max_nb + tile] = P.pooled ? uu - cnt : sics;
    }
}

struct SelParams {
    const float* tile_coh;
    uint32_t n_tiles, max_nb;
    uint32_t nb[BSA_MAX_TILINGS];
    float* score;
    int32_t* choice;
    uint32_t pooled, T, Hg, Wg;
    TileGeo geo[BSA_MAX_TILINGS];  // pooled: tile extents (padded geometry)
};

// Real tokens of a (possibly clipped) tile.
__device__ __forceinline__ double tile_tokens(uint32_t tile, const TileGeo& g, const SelParams& P) {
    uint32_t tt, rem, ty, tx;
    fdivmod(tile, g.f_ntyx, tt, rem);
    fdivmod(rem, g.f_ntx, ty, tx);
    const uint32_t at = min(g.a, P.T - tt * g.a), bt = min(g.b, P.Hg - ty * g.b), ct = min(g.c, P.Wg - tx * g.c);
    return (double)at * bt * ct;
}

// One wave per (b, h): per candidate the mean over tiles (or the pooled
// ratio), then the argmax.
__global__ __launch_bounds__(64) void select_kernel(const SelParams P) {
    const uint32_t bh = blockIdx.x;
    const int lane = threadIdx.x;
    double best = 0.0;
    int best_i = -1;
    for (uint32_t c = 0; c < P.n_tiles; ++c) {
        const float* row = P.tile_coh + ((size_t)bh * P.n_tiles + c) * P.max_nb;
        double sum = 0.0;
        double cnt = 0.0;
        for (uint32_t t = lane; t < P.nb[c]; t += 64) {
            const float v = row[t];
            if (P.pooled) {
                const double n = tile_tokens(t, P.geo[c], P);
                sum += (double)v;
                cnt += n * (n - 1.0);
            } else if (v == v) {
                sum += (double)v;
                cnt += 1.0;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            sum += __shfl_xor(sum, off);
            cnt += __shfl_xor(cnt, off);
        }
        const double mean = cnt > 0.0 ? sum / cnt : -__builtin_inf();
        if (lane == 0) P.score[(size_t)bh * P.n_tiles + c] = (float)mean;
        if (best_i < 0 || mean > best) {  // strict: ties keep the lower index
            best = mean;
            best_i = (int)c;
        }
    }
    if (lane == 0) P.choice[bh] = best_i;
}

int launch_tile_cohesion(const CohParams& P, uint32_t BH, hipStream_t stream, const char* name) {
    const uint64_t n_wg = (uint64_t)((P.max_nb + kWaves - 1) / kWaves) * P.n_tiles * BH;
    BSA_REQUIRE(n_wg < ((uint64_t)1 << 31), "%s: too many tiles", name);
    const dim3 grid((uint32_t)n_wg);
    const int lpt = (int)P.vecs_per_row;
#define BSA_COH(EPV, LPT)                                                                            \
    (P.pad ? tile_cohesion_kernel<EPV, LPT, true, false><<<grid, 64 * kWaves, 0, stream>>>(P)      \
     : P.qsumm ? tile_cohesion_kernel<EPV, LPT, false, true><<<grid, 64 * kWaves, 0, stream>>>(P) \
               : tile_cohesion_kernel<EPV, LPT, false, false><<<grid, 64 * kWaves, 0, stream>>>(P))
    if (P.dtype == BSA_BF16) {
        switch (lpt) {
            case 1: BSA_COH(8, 1); break;
            case 2: BSA_COH(8, 2); break;
            case 4: BSA_COH(8, 4); break;
            case 8: BSA_COH(8, 8); break;
            case 16: BSA_COH(8, 16); break;
            case 32: BSA_COH(8, 32); break;
            default: BSA_FAIL(BSA_ERR_UNSUPPORTED, "%s: bf16 D=%u unsupported", name, P.D);
        }
    } else {
        switch (lpt) {
            case 1: BSA_COH(4, 1); break;
            case 2: BSA_COH(4, 2); break;
            case 4: BSA_COH(4, 4); break;
            case 8: BSA_COH(4, 8); break;
            case 16: BSA_COH(4, 16); break;
            case 32: BSA_COH(4, 32); break;
            default: BSA_FAIL(BSA_ERR_UNSUPPORTED, "%s: fp32 D=%u unsupported", name, P.D);
        }
    }
#undef BSA_COH
    return check_launch(name);
}

int fill_common(CohParams& P, const void* x, int dtype, int64_t B, int64_t H, int64_t S, int64_t D,
                const char* name) {
    const int es = elem_size(dtype);
    BSA_REQUIRE(es != 0, "%s: unknown dtype %d", name, dtype);
    BSA_REQUIRE(x != nullptr, "%s: NULL tensor", name);
    BSA_REQUIRE(B >= 1 && H >= 1 && S >= 1 && D >= 1, "%s: sizes must be >= 1", name);
    BSA_REQUIRE(B * H <= 65535, "%s: B*H too large", name);
    BSA_REQUIRE(S < ((int64_t)1 << 31), "%s: S too large", name);
    BSA_REQUIRE(aligned16(x), "%s: tensor must be 16-byte aligned", name);
    const int64_t row_bytes = D * es;
    BSA_REQUIRE(row_bytes % 16 == 0, "%s: D*elem_size must be a multiple of 16 bytes", name);
    const int64_t vecs = row_bytes / 16;
    if (!(vecs == 1 || vecs == 2 || vecs == 4 || vecs == 8 || vecs == 16 || vecs == 32))
        BSA_FAIL(BSA_ERR_UNSUPPORTED, "%s: D=%lld unsupported (row of 16..512 bytes, power of two)", name,
                 (long long)D);
    P.x = static_cast<const char*>(x);
    P.dtype = dtype;
    P.S = (uint32_t)S;
    P.D = (uint32_t)D;
    P.vecs_per_row = (uint32_t)vecs;
    return BSA_OK;
}

}  // namespace
}  // namespace bsa

using namespace bsa;

extern "C" int bsa_block_cohesion(const void* x, int dtype, int64_t B, int64_t H, int64_t S, int64_t D, int block,
                                  float* coh, bsa_stream_t stream) {
    clear_error();
    const char* name = "bsa_block_cohesion";
    CohParams P{};
    int rc = fill_common(P, x, dtype, B, H, S, D, name);
    if (rc) return rc;
    BSA_REQUIRE(coh != nullptr, "%s: NULL output", name);
    BSA_REQUIRE(block >= 1 && S % block == 0, "%s: block %d must divide S=%lld", name, block, (long long)S);
    // consecutive runs = tiles (1, 1, block) of a 1 x 1 x S grid
    P.T = 1;
    P.pad = 0;
    P.pooled = 0;
    P.Hg = 1;
    P.Wg = (uint32_t)S;
    P.n_tiles = 1;
    P.max_nb = (uint32_t)(S / block);
    for (int i = 0; i < BSA_MAX_TILINGS; ++i) {
        P.geo[i] = make_geo(1, (int)S, 1, 1, block);
        P.nb[i] = P.max_nb;
    }
    P.tile_coh = coh;
    return launch_tile_cohesion(P, (uint32_t)(B * H), (hipStream_t)stream, name);
}

extern "C" int bsa_select_tiling_ex(const void* q, int dtype, int64_t B, int64_t H, int T, int Hg, int Wg,
                                    int64_t D, const int32_t* tiles_host, int n_tiles, int statistic, int pad,
                                    float* tile_coh, float* score, int32_t* choice, void* q_summaries_or_null,
                                    bsa_stream_t stream) {
    clear_error();
    const char* name = "bsa_select_tiling";
    BSA_REQUIRE(T > 0 && Hg > 0 && Wg > 0, "%s: grid must be positive", name);
    BSA_REQUIRE(statistic == BSA_STAT_MEAN || statistic == BSA_STAT_POOLED, "%s: unknown statistic %d", name,
                statistic);
    BSA_REQUIRE(pad == 0 || pad == 1, "%s: pad must be 0 or 1", name);
    const int64_t S = (int64_t)T * Hg * Wg;
    CohParams P{};
    int rc = fill_common(P, q, dtype, B, H, S, D, name);
    if (rc) return rc;
    rc = pad ? check_tiles_padded(T, Hg, Wg, tiles_host, n_tiles) : check_tiles(T, Hg, Wg, tiles_host, n_tiles);
    if (rc) return rc;
    BSA_REQUIRE(tile_coh != nullptr && score != nullptr && choice != nullptr, "%s: NULL output", name);
    P.T = (uint32_t)T;
    P.Hg = (uint32_t)Hg;
    P.Wg = (uint32_t)Wg;
    P.pad = (uint32_t)pad;
    P.pooled = statistic == BSA_STAT_POOLED ? 1u : 0u;
    P.n_tiles = (uint32_t)n_tiles;
    P.max_nb = 0;
    for (int i = 0; i < BSA_MAX_TILINGS; ++i) {
        const int j = i < n_tiles ? i : 0;
        const int a = tiles_host[3 * j], b = tiles_host[3 * j + 1], c = tiles_host[3 * j + 2];
        P.geo[i] = make_geo_padded(Hg, Wg, a, b, c);  // equals make_geo when the tile divides the grid
        P.nb[i] = (uint32_t)(padded_length(T, Hg, Wg, a, b, c) / ((int64_t)a * b * c));
        if (i < n_tiles && P.nb[i] > P.max_nb) P.max_nb = P.nb[i];
    }
    P.tile_coh = tile_coh;
    P.qsumm = static_cast<char*>(q_summaries_or_null);
    P.BH = (uint32_t)(B * H);
    if (P.qsumm != nullptr) {
        BSA_REQUIRE(!pad, "%s: q summaries need candidates that divide the grid (pad = 0)", name);
        BSA_REQUIRE(aligned16(P.qsumm), "%s: q summaries must be 16-byte aligned", name);
        for (int i = 1; i < n_tiles; ++i)
            BSA_REQUIRE(P.nb[i] == P.nb[0], "%s: q summaries need candidates of one volume", name);
    }
    hipStream_t st = (hipStream_t)stream;
    rc = launch_tile_cohesion(P, (uint32_t)(B * H), st, name);
    if (rc) return rc;
    SelParams Q;
    Q.tile_coh = tile_coh;
    Q.n_tiles = P.n_tiles;
    Q.max_nb = P.max_nb;
    for (int i = 0; i < BSA_MAX_TILINGS; ++i) {
        Q.nb[i] = P.nb[i];
        Q.geo[i] = P.geo[i];
    }
    Q.score = score;
    Q.choice = choice;
    Q.pooled = P.pooled;
    Q.T = P.T;
    Q.Hg = P.Hg;
    Q.Wg = P.Wg;
    select_kernel<<<(unsigned)(B * H), 64, 0, st>>>(Q);
    return check_launch(name);
}

extern "C" int bsa_select_tiling(const void* q, int dtype, int64_t B, int64_t H, int T, int Hg, int Wg, int64_t D,
                                 const int32_t* tiles_host, int n_tiles, float* tile_coh, float* score,
                                 int32_t* choice, bsa_stream_t stream) {
    return bsa_select_tiling_ex(q, dtype, B, H, T, Hg, Wg, D, tiles_host, n_tiles, BSA_STAT_MEAN, 0, tile_coh, score,
                                choice, nullptr, stream);
}

// ------------------------------------------------------ no allocation ---
// bsa_select_tiling_noalloc keeps the per-tile values in this fixed array
// instead of a caller workspace.  Every device the library runs on holds its
// own copy until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device copy: kernels get the address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) float scratch[BSA_NOALLOC_TILE_VALUES];

namespace bsa {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
int scratch_on_current_device(float** out, const char* name) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        BSA_FAIL(BSA_ERR_DEVICE, "%s: no usable current device (%d)", name, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            BSA_FAIL(BSA_ERR_DEVICE, "%s: hipGetSymbolAddress of the scratch array failed on device %d: %s", name,
                     dev, hipGetErrorString(e));
        g_scratch_dev[dev] = static_cast<float*>(p);
    }
    *out = g_scratch_dev[dev];
    return BSA_OK;
}

}  // namespace
}  // namespace bsa

extern "C" int bsa_select_tiling_noalloc(const void* q, int dtype, int64_t B, int64_t H, int T, int Hg, int Wg,
                                         int64_t D, const int32_t* tiles_host, int n_tiles, float* score,
                                         int32_t* choice, bsa_stream_t stream) {
    clear_error();
    const char* name = "bsa_select_tiling_noalloc";
    BSA_REQUIRE(T > 0 && Hg > 0 && Wg > 0, "%s: grid must be positive", name);
    BSA_REQUIRE(B >= 1 && H >= 1, "%s: B and H must be >= 1", name);
    int rc = check_tiles(T, Hg, Wg, tiles_host, n_tiles);
    if (rc) return rc;
    const int64_t S = (int64_t)T * Hg * Wg;
    int64_t max_nb = 0;
    for (int i = 0; i < n_tiles; ++i)
        max_nb = std::max<int64_t>(max_nb, S / ((int64_t)tiles_host[3 * i] * tiles_host[3 * i + 1] *
                                                tiles_host[3 * i + 2]));
    const int64_t need = B * H * n_tiles * max_nb;
    BSA_REQUIRE(need <= (int64_t)BSA_NOALLOC_TILE_VALUES,
                "%s: B*H*n_tiles*max_tiles = %lld per-tile values exceed the fixed scratch of %d (use "
                "bsa_select_tiling with a workspace)",
                name, (long long)need, BSA_NOALLOC_TILE_VALUES);
    float* ws = nullptr;
    rc = scratch_on_current_device(&ws, name);
    if (rc) return rc;
    return bsa_select_tiling_ex(q, dtype, B, H, T, Hg, Wg, D, tiles_host, n_tiles, BSA_STAT_MEAN, 0, ws, score,
                                choice, nullptr, stream);
}
