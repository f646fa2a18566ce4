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

// Wave-wide fp32 sum for the top-p search, on VALU lane exchanges only (the
// search takes 32 dependent sums per row, and shuffles through the LDS
// crossbar made it latency-bound): within quads by DPP, then across 8 and 16
// lanes by DPP row mirrors (once the smaller groups are uniform, pairing lane
// i with its mirror adds the other half), then across rows by the 16- and
// 32-lane swaps.  Every lane adds the same two values in the same order, so
// the result is identical in all lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float wave_sum_mass(float v) {
    v = dpp_add<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v = dpp_add<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v = dpp_add<0x141>(v);  // row_half_mirror: lane i with 7 - i
    v = dpp_add<0x140>(v);  // row_mirror: lane i with 15 - i
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
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
    // TOPP: softmax weights w = exp(scale * (s - max)) at their limit values:
    // NaN weighs 0, and an entry equal to the row max weighs 1 (so a +inf max,
    // or a row whose numbers are all -inf, shares the mass equally)
    float w[VPL];
    float target = (float)P.k;
    bool no_mass = false;
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
        const float ztot = wave_sum_mass(z);
        target = P.p * ztot;
        no_mass = ztot == 0.f;  // every score NaN: the first-ranked entry is kept
    }
    // threshold key T: the largest T with count (or mass) of keys >= T reaching the target
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        if (TOPP) {
            float c = 0.f;
#pragma unroll
            for (int i = 0; i < VPL; ++i) c += key[i] >= cand ? w[i] : 0.f;  // w = 0 where not valid
            if (wave_sum_mass(c) >= target) T = cand;
        } else {
            // wave-wide count from ballots (scalar popcounts, no cross-lane
            // shuffles); entries that are not valid hold key 0 < cand
            uint32_t c = 0;
#pragma unroll
            for (int i = 0; i < VPL; ++i) c += popc64(__ballot(key[i] >= cand));
            if (c >= k_row) T = cand;
            // exactly k_row keys at or above T: they are the top k_row, and the
            // threshold the remaining bits would reach is their smallest key
            if (c == k_row) {
                uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
                for (int i = 0; i < VPL; ++i) mn = key[i] >= T ? min(mn, key[i]) : mn;
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) mn = min(mn, (uint32_t)__shfl_xor((int)mn, off));
                T = (uint32_t)__builtin_amdgcn_readfirstlane((int)mn);
                break;
            }
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
        gt = wave_sum_mass(gt);
        wt = wave_max_f(wt);
        nt = wave_sum(nt);
        const float t = wt > 0.f ? ceilf((target - gt) / wt) : 1.f;
        need = (uint32_t)fminf(fmaxf(t, 1.f), (float)nt);
        if (no_mass) {  // all keys are 0 (NaN): take the lowest index among them
            T = 0u;
            need = 1u;
        }
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

// Launch plan for block lists whose lengths differ from row to row (the
// top-p budget: one query block may keep hundreds of key blocks while most
// keep a handful).  The attention kernels stream each head's K and V tiles
// through the L2 of the XCD that runs its rows, so a plan keeps a head's
// rows on one XCD (units: whole heads, or 2, 4, 8 equal row ranges of a head
// when there are fewer than 16 heads), balances the XCDs' work and starts
// long rows first:
//  1. unit weight = its rows' kept counts plus a fixed cost per row
//     (kRowCost blocks: the prologue and epilogue of a query block), all
//     weights shifted right by the bits that bring their total under 2^28
//     (none at any size met here), so that loads fit 32-bit keys;
//  2. units, heaviest first, go to the least loaded XCD that holds fewer
//     than ceil(U/8) units (list scheduling, longest processing time first,
//     with equal room on every XCD so that the grid needs almost no empty
//     slots);
//  3. an XCD runs its units in the order they came, each unit's rows in
//     decreasing count (in kPlanBins coarse bins: counts >= kPlanBins - 1
//     rank as one).
// Workgroup w runs on XCD w % 8, so XCD x's j-th row goes to entry 8j + x.
// Three launches: the weights and the sorts run one workgroup per unit, the
// scheduling one workgroup; the weights and placements pass through the last
// 3U entries of the order buffer, which the sorts then leave empty.
constexpr int kPlanThreads = 1024, kPlanWaves = kPlanThreads / 64, kPlanBins = 256, kMaxUnits = 1024;
constexpr int kUnitThreads = 256, kUnitWaves = kUnitThreads / 64;
constexpr uint32_t kRowCost = 5, kEmptySlot = 0xFFFFFFFFu;

struct Plan {
    int64_t units, unit_rows, cap;  // cap: rows per XCD
    int64_t plan_len() const { return 8 * cap; }
    int64_t len() const { return 8 * cap + 3 * units; }  // plus the scratch words
};

Plan plan_shape(int64_t BH, int64_t nq) {
    int64_t r = 1;
    while (r < 8 && BH * r < 16) r *= 2;
    while (nq % r != 0) r /= 2;
    Plan p;
    p.units = BH * r;
    p.unit_rows = nq / r;
    p.cap = p.unit_rows * ((p.units + 7) / 8);
    return p;
}

__device__ __forceinline__ uint32_t plan_count(int c) { return (uint32_t)min(max(c, 0), 65535); }

__device__ __forceinline__ uint32_t plan_key(uint32_t c) {
    // bin of a count: longest first, counts of kPlanBins - 1 or more in bin 0
    return c >= kPlanBins - 1 ? 0u : kPlanBins - 1 - c;
}

// 1. one workgroup per unit: its weight, as two words at scratch[2u]
__global__ __launch_bounds__(kUnitThreads) void plan_weight_kernel(const int32_t* __restrict__ cnt,
                                                                   uint32_t unit_rows, uint32_t* __restrict__ scratch) {
    __shared__ unsigned long long part[kUnitWaves];
    const uint32_t u = blockIdx.x, t = threadIdx.x, lane = t & 63u, wave = t >> 6;
    const int32_t* c = cnt + (size_t)u * unit_rows;
    unsigned long long w = 0;
#pragma unroll 4
    for (uint32_t i = t; i < unit_rows; i += kUnitThreads) w += plan_count(c[i]) + kRowCost;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) w += __shfl_xor(w, off);
    if (lane == 0) part[wave] = w;
    __syncthreads();
    if (t == 0) {
        unsigned long long sum = 0;
#pragma unroll
        for (int i = 0; i < kUnitWaves; ++i) sum += part[i];
        scratch[2 * u] = (uint32_t)sum;
        scratch[2 * u + 1] = (uint32_t)(sum >> 32);
    }
}

// 2. one workgroup: the weights' shift, the units' rank, list scheduling; the
// placement of unit u ((first position on its XCD) << 3 | XCD) goes to
// scratch[2U + u], and the plan's slots past each XCD's rows, and the buffer
// past the scratch words, are emptied
__global__ __launch_bounds__(kPlanThreads) void plan_place_kernel(uint32_t units, uint32_t unit_rows, uint32_t cap,
                                                                  uint32_t len, uint32_t* __restrict__ order) {
    __shared__ unsigned long long weight[kMaxUnits];
    __shared__ uint32_t weight32[kMaxUnits];
    __shared__ uint32_t ranked_weight[kMaxUnits];
    __shared__ uint32_t by_rank[kMaxUnits];
    __shared__ unsigned long long partial[kPlanWaves];
    __shared__ uint32_t fill[8];
    const uint32_t t = threadIdx.x, lane = t & 63u, wave = t >> 6;
    const uint32_t plan_len = 8u * cap;
    uint32_t* scratch = order + plan_len;
    {   // the total weight -> the shift that brings it under 2^28 (one unit per thread: units <= kPlanThreads)
        unsigned long long w = t < units ? ((unsigned long long)scratch[2 * t + 1] << 32) | scratch[2 * t] : 0ull;
        if (t < units) weight[t] = w;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) w += __shfl_xor(w, off);
        if (lane == 0) partial[wave] = w;
        __syncthreads();
        unsigned long long total = 0;
#pragma unroll
        for (int i = 0; i < kPlanWaves; ++i) total += partial[i];
        const int bits = total == 0 ? 0 : 64 - __builtin_clzll(total);
        const int shift = bits > 28 ? bits - 28 : 0;
        if (t < units) weight32[t] = (uint32_t)(weight[t] >> shift);
    }
    __syncthreads();
    // units ranked by weight, heaviest first (ties: lower unit first)
    if (t < units) {
        const uint32_t w = weight32[t];
        uint32_t rank = 0;
        for (uint32_t v = 0; v < units; ++v) {
            const uint32_t x = weight32[v];
            rank += (x > w || (x == w && v < t)) ? 1u : 0u;
        }
        by_rank[rank] = t;
        ranked_weight[rank] = w;
    }
    __syncthreads();
    // list scheduling in wave 0 on wave-uniform values: XCD x's load is kept as the key (load << 3) | x
    // (< 2^31), so the least loaded XCD (ties: lower XCD) is the smallest key of those with room, found
    // without branches; 64 ranked units at a time are read into a VGPR, one per lane, taken out lane by
    // lane, and their placements gathered in a VGPR that is written once
    if (wave == 0) {
        const uint32_t room = cap / unit_rows;   // units an XCD may hold: ceil(U/8)
        uint32_t key[8], held[8];
#pragma unroll
        for (int x = 0; x < 8; ++x) key[x] = (uint32_t)x, held[x] = 0;
        for (uint32_t k0 = 0; k0 < units; k0 += 64) {
            const bool has = k0 + lane < units;
            const uint32_t my_u = has ? by_rank[k0 + lane] : 0u;
            const uint32_t my_w = has ? ranked_weight[k0 + lane] : 0u;
            uint32_t my_place = 0;
            const uint32_t n = min(64u, units - k0);
            for (uint32_t j = 0; j < n; ++j) {
                const uint32_t w8 = (uint32_t)__builtin_amdgcn_readlane((int)my_w, (int)j) << 3;
                uint32_t best = ~0u;
#pragma unroll
                for (int x = 0; x < 8; ++x) best = min(best, held[x] < room ? key[x] : ~0u);
                const uint32_t bx = best & 7u;
                uint32_t first = 0;
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                    const bool hit = (uint32_t)x == bx;
                    first = hit ? held[x] : first;
                    key[x] += hit ? w8 : 0u;
                    held[x] += hit ? 1u : 0u;
                }
                my_place = lane == j ? (((first * unit_rows) << 3) | bx) : my_place;
            }
            if (has) scratch[2 * units + my_u] = my_place;
        }
#pragma unroll
        for (int x = 0; x < 8; ++x)
            if (lane == (uint32_t)x) fill[x] = held[x] * unit_rows;
    }
    __syncthreads();
    for (uint32_t e = t; e < plan_len; e += kPlanThreads)
        if ((e >> 3) >= fill[e & 7u]) order[e] = kEmptySlot;
    for (uint32_t e = plan_len + 3u * units + t; e < len; e += kPlanThreads) order[e] = kEmptySlot;
}

// 3. one workgroup per unit: its rows by decreasing count into its place; its
// scratch words are left empty
__global__ __launch_bounds__(kUnitThreads) void plan_sort_kernel(const int32_t* __restrict__ cnt, uint32_t units,
                                                                 uint32_t unit_rows, uint32_t cap,
                                                                 uint32_t* __restrict__ order) {
    __shared__ uint32_t bins[kPlanBins];
    __shared__ uint32_t wave_total[kUnitWaves];
    const uint32_t u = blockIdx.x, t = threadIdx.x, lane = t & 63u, wave = t >> 6;
    uint32_t* scratch = order + 8u * cap;
    const uint32_t place = (uint32_t)__builtin_amdgcn_readfirstlane(scratch[2 * units + u]);
    const uint32_t x = place & 7u, p0 = place >> 3;
    const uint32_t r0 = u * unit_rows;
    for (uint32_t i = t; i < kPlanBins; i += kUnitThreads) bins[i] = 0;
    __syncthreads();
    // (when every active lane of a wave has the same key, as a head's equal-length top-k lists give, one
    // lane adds them all: 64 lanes on one LDS address would serialise)
    for (uint32_t i = t; i < unit_rows; i += kUnitThreads) {
        const uint32_t key = plan_key(plan_count(cnt[r0 + i]));
        const uint32_t k0 = (uint32_t)__builtin_amdgcn_readfirstlane(key);
        const uint64_t same = __ballot(key == k0), all = __ballot(true);
        if (same == all) {
            if (lane == (uint32_t)__builtin_ctzll(all)) atomicAdd(&bins[k0], (uint32_t)__builtin_popcountll(all));
        } else {
            atomicAdd(&bins[key], 1u);
        }
    }
    __syncthreads();
    // exclusive scan of the bins, one bin per thread
    const uint32_t own = bins[t];
    uint32_t incl = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off);
        if (lane >= (uint32_t)off) incl += y;
    }
    if (lane == 63u) wave_total[wave] = incl;
    __syncthreads();
    uint32_t run = incl - own;
    for (uint32_t i = 0; i < wave; ++i) run += wave_total[i];
    bins[t] = run;
    __syncthreads();
    for (uint32_t i = t; i < unit_rows; i += kUnitThreads) {
        const uint32_t key = plan_key(plan_count(cnt[r0 + i]));
        const uint32_t k0 = (uint32_t)__builtin_amdgcn_readfirstlane(key);
        const uint64_t same = __ballot(key == k0), all = __ballot(true);
        uint32_t rank;
        if (same == all) {
            const uint32_t first = (uint32_t)__builtin_ctzll(all);
            uint32_t base = 0;
            if (lane == first) base = atomicAdd(&bins[k0], (uint32_t)__builtin_popcountll(all));
            base = (uint32_t)__shfl((int)base, (int)first);
            rank = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(all >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)all, 0u));
        } else {
            rank = atomicAdd(&bins[key], 1u);
        }
        order[8u * (p0 + rank) + x] = r0 + i;
    }
    if (t == 0) {
        scratch[2 * u] = kEmptySlot;
        scratch[2 * u + 1] = kEmptySlot;
        scratch[2 * units + u] = kEmptySlot;
    }
}

// Launch order for block lists of (nearly) equal lengths: the rows of a head
// sorted by the middle entry of their kept lists, so that the query blocks an
// XCD runs side by side keep key blocks from the same part of the sequence and
// share more of them through the XCD's L2.  One workgroup per head: a counting
// sort over the Nk key blocks (bins in LDS, rows of one bin in no fixed order),
// then row rank -> slot h*Nq + rank of the plain XCD ranges (XCD x holds slots
// [x*per_xcd, (x+1)*per_xcd), its j-th at order[8j + x]).  With R > 1 XCDs per
// head (R divides Nq, 8/R divides BH) the XCDs form 8/R groups of R, group g
// runs heads g, g + 8/R, ... in turn, and XCD g*R + i takes the i-th of R
// contiguous parts of each head's sorted rows: R times fewer heads are in
// flight at once, while the rows an XCD runs side by side stay as close in
// the sorted order as with whole heads.
constexpr uint32_t kMaxMedianBins = 4096;

__global__ __launch_bounds__(kUnitThreads) void median_order_kernel(const int32_t* __restrict__ kv_idx,
                                                                    const int32_t* __restrict__ kv_cnt, uint32_t nq,
                                                                    uint32_t max_kept, uint32_t nk, uint32_t per_xcd,
                                                                    uint32_t xcds_per_head, uint32_t* __restrict__ order) {
    __shared__ uint32_t bins[kMaxMedianBins];
    __shared__ uint32_t wave_total[kUnitWaves];
    const uint32_t h = blockIdx.x, t = threadIdx.x, lane = t & 63u, wave = t >> 6;
    const size_t r0 = (size_t)h * nq;
    // the key of row i: its middle kept block (lists ascend), 0 for an empty list,
    // out-of-range entries clamped (bsa_validate_block_list reports them)
    auto key_of = [&](uint32_t i) -> uint32_t {
        const int c = min(max(kv_cnt[r0 + i], 0), (int)max_kept);
        if (c == 0) return 0u;
        const int32_t j = kv_idx[(r0 + i) * max_kept + (uint32_t)c / 2u];
        return j < 0 ? 0u : ((uint32_t)j < nk ? (uint32_t)j : nk - 1u);
    };
    for (uint32_t b = t; b < nk; b += kUnitThreads) bins[b] = 0;
    __syncthreads();
    for (uint32_t i = t; i < nq; i += kUnitThreads) atomicAdd(&bins[key_of(i)], 1u);
    __syncthreads();
    // exclusive scan: thread t owns bins [t*per, (t+1)*per)
    const uint32_t per = (nk + kUnitThreads - 1) / kUnitThreads;
    uint32_t own = 0;
    for (uint32_t j = 0; j < per; ++j) {
        const uint32_t b = t * per + j;
        if (b < nk) own += bins[b];
    }
    uint32_t incl = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(incl, off);
        if (lane >= (uint32_t)off) incl += y;
    }
    if (lane == 63u) wave_total[wave] = incl;
    __syncthreads();
    uint32_t run = incl - own;
    for (uint32_t w = 0; w < wave; ++w) run += wave_total[w];
    for (uint32_t j = 0; j < per; ++j) {
        const uint32_t b = t * per + j;
        if (b < nk) {
            const uint32_t c = bins[b];
            bins[b] = run;
            run += c;
        }
    }
    __syncthreads();
    const uint32_t R = xcds_per_head, G = 8u / R, part = nq / R;
    for (uint32_t i = t; i < nq; i += kUnitThreads) {
        const uint32_t rank = atomicAdd(&bins[key_of(i)], 1u);
        uint32_t x, j;
        if (R == 1u) {
            const uint32_t slot = h * nq + rank;
            x = slot / per_xcd;
            j = slot - x * per_xcd;
        } else {
            x = (h % G) * R + rank / part;
            j = (h / G) * part + rank % part;
        }
        order[8u * j + x] = (uint32_t)(r0 + i);
    }
}

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

extern "C" int64_t bsa_row_order_len(int64_t BH, int64_t nq) {
    clear_error();
    if (BH < 1 || nq < 1 || BH * nq >= ((int64_t)1 << 31)) {
        set_error("bsa_row_order_len: BH=%lld and nq=%lld must be >= 1 with BH*nq < 2^31", (long long)BH,
                  (long long)nq);
        return -1;
    }
    const Plan p = plan_shape(BH, nq);
    if (p.units > kMaxUnits) {
        set_error("bsa_row_order_len: more than %d heads", kMaxUnits);
        return -1;
    }
    if (p.len() >= ((int64_t)1 << 31)) {
        set_error("bsa_row_order_len: the plan would exceed 2^31 entries");
        return -1;
    }
    return p.len();
}

extern "C" int bsa_row_order(const int32_t* kv_cnt, int64_t BH, int64_t nq, uint32_t* order, int64_t order_len,
                             bsa_stream_t stream) {
    const char* name = "bsa_row_order";
    const int64_t need = bsa_row_order_len(BH, nq);
    if (need < 0) return BSA_ERR_INVALID_ARG;
    BSA_REQUIRE(kv_cnt && order, "%s: NULL argument", name);
    BSA_REQUIRE(order_len >= need && order_len < ((int64_t)1 << 31), "%s: order_len=%lld must be in [%lld, 2^31)",
                name, (long long)order_len, (long long)need);
    const Plan p = plan_shape(BH, nq);
    hipStream_t st = (hipStream_t)stream;
    uint32_t* scratch = order + p.plan_len();
    const uint32_t units = (uint32_t)p.units, rows = (uint32_t)p.unit_rows, cap = (uint32_t)p.cap;
    plan_weight_kernel<<<units, kUnitThreads, 0, st>>>(kv_cnt, rows, scratch);
    plan_place_kernel<<<1, kPlanThreads, 0, st>>>(units, rows, cap, (uint32_t)order_len, order);
    plan_sort_kernel<<<units, kUnitThreads, 0, st>>>(kv_cnt, units, rows, cap, order);
    return check_launch(name);
}

// Heads whose K and V together exceed this many bytes are split over two
// XCDs (bsa_row_order_by_median_ex).  Measured with host-built orders on the
// same lists at S = 122,880, D = 128 (63 MB per head, 24 heads): 2.0-2.9%
// faster than whole heads per XCD; 4 or 8 XCDs per head 21-40% slower.  At
// S = 30,720 (16 MB per head) two XCDs per head were 0.6% slower.
constexpr int64_t kSplitHeadBytes = 32ll << 20;

extern "C" int bsa_row_order_by_median_ex(const int32_t* kv_idx, const int32_t* kv_cnt, int64_t BH, int64_t nq,
                                          int max_kept, int64_t nk, int64_t head_kv_bytes, uint32_t* order,
                                          int64_t order_len, bsa_stream_t stream) {
    clear_error();
    const char* name = "bsa_row_order_by_median";
    BSA_REQUIRE(kv_idx && kv_cnt && order, "%s: NULL argument", name);
    BSA_REQUIRE(BH >= 1 && nq >= 1 && BH * nq < ((int64_t)1 << 31), "%s: BH=%lld and Nq=%lld must be >= 1 with BH*Nq < 2^31",
                name, (long long)BH, (long long)nq);
    BSA_REQUIRE((BH * nq) % 8 == 0, "%s: BH*Nq=%lld must be a multiple of 8 (one equal range of rows per XCD)", name,
                (long long)(BH * nq));
    BSA_REQUIRE(max_kept >= 1, "%s: max_kept=%d must be >= 1", name, max_kept);
    BSA_REQUIRE(nk >= 1 && nk <= (int64_t)kMaxMedianBins, "%s: Nk=%lld must be in [1, %u]", name, (long long)nk,
                kMaxMedianBins);
    BSA_REQUIRE(order_len >= BH * nq && order_len < ((int64_t)1 << 31), "%s: order_len=%lld must be in [%lld, 2^31)",
                name, (long long)order_len, (long long)(BH * nq));
    BSA_REQUIRE(head_kv_bytes >= 0, "%s: head_kv_bytes=%lld must be >= 0", name, (long long)head_kv_bytes);
    const uint32_t R = (head_kv_bytes > kSplitHeadBytes && BH % 4 == 0 && nq % 2 == 0) ? 2u : 1u;
    median_order_kernel<<<(unsigned)BH, kUnitThreads, 0, (hipStream_t)stream>>>(
        kv_idx, kv_cnt, (uint32_t)nq, (uint32_t)max_kept, (uint32_t)nk, (uint32_t)(BH * nq / 8), R, order);
    return check_launch(name);
}

extern "C" int bsa_row_order_by_median(const int32_t* kv_idx, const int32_t* kv_cnt, int64_t BH, int64_t nq,
                                       int max_kept, int64_t nk, uint32_t* order, int64_t order_len,
                                       bsa_stream_t stream) {
    return bsa_row_order_by_median_ex(kv_idx, kv_cnt, BH, nq, max_kept, nk, 0, order, order_len, stream);
}
