// Per-row block selection with sink and diagonal blocks: bsa_topk_block_mask
// (a fixed budget) and bsa_top_p_block_mask (a probability-mass budget).
//
// [Adaptive tiling (SPADE), "The idea" step 4]: a fixed budget of k key blocks
// is kept per query block, and the sink blocks and a diagonal band are always
// kept ([Adaptive tiling (SPADE), "Recipe"]: they are ORed into the top-k
// mask; SPADE's Wan configurations use a sink width of 5 and a band width of
// 40).  A band of width w keeps key blocks J with abs(I - J) <= w / 2, so
// width 1 is the diagonal alone.  The top-p variant (named among the
// library's block masks on the same page) keeps the shortest best-ranked
// prefix whose softmax probability mass reaches p.
//
// Design: one wave per row, the row's scores held in registers (element
// e = i*64 + lane).  Scores map to order-preserving unsigned keys (-0.0 as
// +0.0, NaN lowest), the threshold key is found by a 32-step bitwise search
// with wave-wide counts (top-k) or wave-wide probability mass (top-p), and
// ties at the threshold are resolved to the lowest indices with ballots.
// The kept set comes out in ascending index order as a compact list (what
// the attention kernel walks) and, optionally, as a byte mask.  Top-k
// selection is exact: for the same fp32 scores it is bit-identical to a sort
// by (score desc, index asc).  Top-p sums fp32 weights (the butterfly sums
// are identical in every lane), so its cut can differ from a float64 one
// only where the cumulative mass lies within rounding of p.
#include "common.h"

#include <cmath>

namespace bsa {
namespace {

struct TopkParams {
    const float* scores;
    int32_t* kv_idx;
    int32_t* kv_cnt;
    uint8_t* mask;
    uint32_t nq, nk, k, sink, max_kept;
    int32_t diag_half;  // band half-width; -1: no band
    float p, scale_log2;  // top-p only
    uint64_t rows;
    // per-head budget (bsa_topk_block_mask_tiled): k and the head's block
    // count come from the tables at the head's tiling choice
    const int32_t* head_choice;
    uint32_t n_table;
    uint32_t k_table[BSA_MAX_TILINGS], nk_table[BSA_MAX_TILINGS];
};

// Larger score -> larger key.  NaN -> 0, and every number maps above 0.
__device__ __forceinline__ uint32_t order_key(float f) {
    if (f != f) return 0u;
    if (f == 0.0f) f = 0.0f;  // -0.0 ranks as +0.0
    const uint32_t b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

__device__ __forceinline__ uint32_t popc64(uint64_t m) { return (uint32_t)__popcll(m); }

// VPL = values per lane (the row length is at most 64 * VPL).  TOPP selects
// by probability mass instead of by count.
template <int VPL, bool TOPP>
__global__ __launch_bounds__(256) void topk_kernel(const TopkParams P) {
    const int lane = threadIdx.x & 63;
    const uint64_t row = (uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= P.rows) return;
    const uint32_t I = (uint32_t)(row % P.nq);
    const float* s = P.scores + row * P.nk;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    uint32_t k_row = P.k, nk_row = P.nk;
    if (P.head_choice != nullptr) {
        uint32_t c = (uint32_t)__builtin_amdgcn_readfirstlane(P.head_choice[row / P.nq]);
        if (c >= P.n_table) c = 0;  // out-of-range choices are caught by bsa_validate_indices
        k_row = P.k_table[c];
        nk_row = P.nk_table[c];
    }
    const bool row_exists = P.head_choice == nullptr || I < nk_row;

    uint32_t key[VPL];
    bool valid[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const uint32_t e = i * 64 + lane;
        valid[i] = row_exists && e < nk_row;
        key[i] = valid[i] ? order_key(s[e]) : 0u;
    }
    // TOPP: softmax weights w = exp(scale * (s - max)); NaN and -inf weigh 0
    float w[VPL];
    float target = (float)P.k;
    if (TOPP) {
        float m = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (valid[i] && key[i] != 0u) m = fmaxf(m, s[i * 64 + lane]);
        m = wave_max_f(m);
        float z = 0.f;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const float x = valid[i] ? s[i * 64 + lane] : 0.f;
            w[i] = (!valid[i] || key[i] == 0u) ? 0.f : (x == m ? 1.f : __builtin_amdgcn_exp2f((x - m) * P.scale_log2));
            z += w[i];
        }
        target = P.p * wave_sum_f(z);
    }
    // threshold key T: the largest T with count (or mass) of keys >= T reaching the target
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        if (TOPP) {
            float c = 0.f;
#pragma unroll
            for (int i = 0; i < VPL; ++i) c += key[i] >= cand ? w[i] : 0.f;  // w = 0 where not valid
            if (wave_sum_f(c) >= target) T = cand;
        } else {
            // wave-wide count from ballots (scalar popcounts, no cross-lane
            // shuffles); entries that are not valid hold key 0 < cand
            uint32_t c = 0;
#pragma unroll
            for (int i = 0; i < VPL; ++i) c += popc64(__ballot(key[i] >= cand));
            if (c >= k_row) T = cand;
        }
    }
    uint32_t need;  // ties at T to take, lowest index first
    if (TOPP) {
        float gt = 0.f, wt = 0.f;
        uint32_t nt = 0;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            gt += key[i] > T ? w[i] : 0.f;
            if (valid[i] && key[i] == T) { wt = w[i]; ++nt; }
        }
        gt = wave_sum_f(gt);
        wt = wave_max_f(wt);
        nt = wave_sum(nt);
        const float t = wt > 0.f ? ceilf((target - gt) / wt) : 1.f;
        need = (uint32_t)fminf(fmaxf(t, 1.f), (float)nt);
    } else {
        uint32_t gt = 0;
#pragma unroll
        for (int i = 0; i < VPL; ++i) gt += popc64(__ballot(key[i] > T));
        need = row_exists ? k_row - gt : 0u;
    }

    bool keep[VPL];
    uint32_t tie_seen = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const bool tie = valid[i] && key[i] == T;
        const uint64_t m = __ballot(tie);
        const uint32_t rank = tie_seen + popc64(m & lt_mask);
        tie_seen += popc64(m);
        const uint32_t e = i * 64 + lane;
        const int d = (int)e - (int)I;
        keep[i] = valid[i] &&
                  (key[i] > T || (tie && rank < need) || e < P.sink || (d <= P.diag_half && -d <= P.diag_half));
    }
    int32_t* out = P.kv_idx + row * P.max_kept;
    uint32_t pos = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const uint64_t m = __ballot(keep[i]);
        const uint32_t at = pos + popc64(m & lt_mask);
        if (keep[i] && at < P.max_kept) out[at] = (int32_t)(i * 64 + lane);
        pos += popc64(m);
        if (P.mask != nullptr && i * 64 + lane < P.nk) P.mask[row * P.nk + i * 64 + lane] = keep[i] ? 1 : 0;
    }
    for (uint32_t j = pos + lane; j < P.max_kept; j += 64) out[j] = -1;
    if (lane == 0) P.kv_cnt[row] = (int32_t)pos;
}

}  // namespace
}  // namespace bsa

using namespace bsa;

namespace bsa {
namespace {

int band_width(int diag_width) { return diag_width >= 1 ? 2 * (diag_width / 2) + 1 : 0; }

template <bool TOPP>
int launch_select(TopkParams& P, hipStream_t st, const char* name) {
    const uint64_t blocks = (P.rows + 3) / 4;
    BSA_REQUIRE(blocks < ((uint64_t)1 << 31), "%s: too many rows", name);
    const int vpl = ((int)P.nk + 63) / 64;
    if (vpl <= 8)
        topk_kernel<8, TOPP><<<(unsigned)blocks, 256, 0, st>>>(P);
    else if (vpl <= 16)
        topk_kernel<16, TOPP><<<(unsigned)blocks, 256, 0, st>>>(P);
    else if (vpl <= 32)
        topk_kernel<32, TOPP><<<(unsigned)blocks, 256, 0, st>>>(P);
    else
        topk_kernel<64, TOPP><<<(unsigned)blocks, 256, 0, st>>>(P);
    return check_launch(name);
}

}  // namespace
}  // namespace bsa

extern "C" int bsa_topk_block_mask(const float* scores, int64_t B, int64_t H, int Nq, int Nk, int k, int sink_blocks,
                                   int diag_width, int32_t* kv_idx, int32_t* kv_cnt, int max_kept,
                                   uint8_t* mask_or_null, bsa_stream_t stream) {
    clear_error();
    const char* name = "bsa_topk_block_mask";
    BSA_REQUIRE(scores && kv_idx && kv_cnt, "%s: NULL argument", name);
    BSA_REQUIRE(B >= 1 && H >= 1 && Nq >= 1, "%s: B, H, Nq must be >= 1", name);
    BSA_REQUIRE(Nk >= 1 && Nk <= 4096, "%s: Nk=%d must be in [1, 4096]", name, Nk);
    BSA_REQUIRE(k >= 1 && k <= Nk, "%s: k=%d must be in [1, Nk=%d]", name, k, Nk);
    BSA_REQUIRE(sink_blocks >= 0, "%s: sink_blocks must be >= 0", name);
    BSA_REQUIRE(diag_width >= 0, "%s: diag_width must be >= 0", name);
    const int64_t widest = std::min<int64_t>(Nk, (int64_t)k + sink_blocks + band_width(diag_width));
    BSA_REQUIRE(max_kept >= widest, "%s: max_kept=%d < %lld (k + sink + band, at most Nk)", name, max_kept,
                (long long)widest);
    TopkParams P{};
    P.scores = scores;
    P.kv_idx = kv_idx;
    P.kv_cnt = kv_cnt;
    P.mask = mask_or_null;
    P.nq = (uint32_t)Nq;
    P.nk = (uint32_t)Nk;
    P.k = (uint32_t)k;
    P.sink = (uint32_t)std::min(sink_blocks, Nk);
    P.diag_half = diag_width >= 1 ? diag_width / 2 : -1;
    P.max_kept = (uint32_t)max_kept;
    P.rows = (uint64_t)B * H * Nq;
    return launch_select<false>(P, (hipStream_t)stream, name);
}

extern "C" int bsa_top_p_block_mask(const float* scores, int64_t B, int64_t H, int Nq, int Nk, float p, float scale,
                                    int sink_blocks, int diag_width, int32_t* kv_idx, int32_t* kv_cnt, int max_kept,
                                    uint8_t* mask_or_null, bsa_stream_t stream) {
    clear_error();
    const char* name = "bsa_top_p_block_mask";
    BSA_REQUIRE(scores && kv_idx && kv_cnt, "%s: NULL argument", name);
    BSA_REQUIRE(B >= 1 && H >= 1 && Nq >= 1, "%s: B, H, Nq must be >= 1", name);
    BSA_REQUIRE(Nk >= 1 && Nk <= 4096, "%s: Nk=%d must be in [1, 4096]", name, Nk);
    BSA_REQUIRE(p > 0.f && p <= 1.f, "%s: p=%g must be in (0, 1]", name, (double)p);
    BSA_REQUIRE(scale > 0.f && std::isfinite(scale), "%s: scale must be positive and finite", name);
    BSA_REQUIRE(sink_blocks >= 0, "%s: sink_blocks must be >= 0", name);
    BSA_REQUIRE(diag_width >= 0, "%s: diag_width must be >= 0", name);
    BSA_REQUIRE(max_kept >= Nk, "%s: max_kept=%d must be >= Nk=%d (top-p can keep every block)", name, max_kept, Nk);
    TopkParams P{};
    P.scores = scores;
    P.kv_idx = kv_idx;
    P.kv_cnt = kv_cnt;
    P.mask = mask_or_null;
    P.nq = (uint32_t)Nq;
    P.nk = (uint32_t)Nk;
    P.k = 1;
    P.sink = (uint32_t)std::min(sink_blocks, Nk);
    P.diag_half = diag_width >= 1 ? diag_width / 2 : -1;
    P.max_kept = (uint32_t)max_kept;
    P.p = p;
    P.scale_log2 = (float)((double)scale * 1.4426950408889634);
    P.rows = (uint64_t)B * H * Nq;
    return launch_select<true>(P, (hipStream_t)stream, name);
}

extern "C" int bsa_topk_block_mask_tiled(const float* scores, int64_t B, int64_t H, int Nq, int Nk,
                                         const int32_t* head_choice, const int32_t* k_table, const int32_t* nk_table,
                                         int n_table, int sink_blocks, int diag_width, int32_t* kv_idx,
                                         int32_t* kv_cnt, int max_kept, uint8_t* mask_or_null, bsa_stream_t stream) {
    clear_error();
    const char* name = "bsa_topk_block_mask_tiled";
    BSA_REQUIRE(scores && kv_idx && kv_cnt && head_choice && k_table && nk_table, "%s: NULL argument", name);
    BSA_REQUIRE(B >= 1 && H >= 1 && Nq >= 1, "%s: B, H, Nq must be >= 1", name);
    BSA_REQUIRE(Nk >= 1 && Nk <= 4096, "%s: Nk=%d must be in [1, 4096]", name, Nk);
    BSA_REQUIRE(n_table >= 1 && n_table <= BSA_MAX_TILINGS, "%s: n_table=%d must be in [1, %d]", name, n_table,
                BSA_MAX_TILINGS);
    BSA_REQUIRE(sink_blocks >= 0, "%s: sink_blocks must be >= 0", name);
    BSA_REQUIRE(diag_width >= 0, "%s: diag_width must be >= 0", name);
    TopkParams P{};
    int64_t widest = 0;
    for (int c = 0; c < n_table; ++c) {
        BSA_REQUIRE(nk_table[c] >= 1 && nk_table[c] <= Nk, "%s: nk_table[%d]=%d must be in [1, Nk=%d]", name, c,
                    nk_table[c], Nk);
        BSA_REQUIRE(k_table[c] >= 1 && k_table[c] <= nk_table[c], "%s: k_table[%d]=%d must be in [1, %d]", name, c,
                    k_table[c], nk_table[c]);
        widest = std::max<int64_t>(widest, std::min<int64_t>(nk_table[c], (int64_t)k_table[c] + sink_blocks +
                                                                              band_width(diag_width)));
        P.k_table[c] = (uint32_t)k_table[c];
        P.nk_table[c] = (uint32_t)nk_table[c];
    }
    BSA_REQUIRE(max_kept >= widest, "%s: max_kept=%d < %lld (k + sink + band, at most nk)", name, max_kept,
                (long long)widest);
    P.scores = scores;
    P.kv_idx = kv_idx;
    P.kv_cnt = kv_cnt;
    P.mask = mask_or_null;
    P.nq = (uint32_t)Nq;
    P.nk = (uint32_t)Nk;
    P.k = 1;
    P.sink = (uint32_t)std::min(sink_blocks, Nk);
    P.diag_half = diag_width >= 1 ? diag_width / 2 : -1;
    P.max_kept = (uint32_t)max_kept;
    P.rows = (uint64_t)B * H * Nq;
    P.head_choice = head_choice;
    P.n_table = (uint32_t)n_table;
    return launch_select<false>(P, (hipStream_t)stream, name);
}
