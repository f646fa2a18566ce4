// Min/max block summaries and estimated block scores: bsa_minmax_block_scores.
//
// [Adaptive tiling (SPADE), "The idea" step 3]: each block of tile-contiguous
// queries (keys) is summarised by its elementwise maximum and minimum, and
// the (query block I, key block J) score is estimated as
//   max((qmax_I + qmin_I) . kmax_J, (qmax_I + qmin_I) . kmin_J).
//
// bsa_minmax_block_scores_tiled reads q and k in T-major order, block J of a
// head being tile J of the head's chosen tiling (the permuted copies are
// never formed).  Given q's summaries of every candidate (the tiling choice
// pass forms them while it reads q), it copies the chosen ones and reads
// only k.
//
// bsa_minmax_block_scores_masked leaves out tokens labelled < 0 (the padding
// of a padded tiling, [Adaptive tiling (SPADE), "Deviations and notes"]):
// a partial block is summarised by its real tokens, and a block with none
// scores -inf in its row and its column.  bsa_minmax_block_scores_tiled_padded
// does the same on T-major q and k, block J of a head being tile J of the
// head's tiling on the grid padded along T: cells of the padding frames lie
// past the head and are left out without being read.
//
// Design: pass 1 is an HBM-bound reduction, one wave per block, that keeps
// the summaries in the input dtype (a max or min of bf16 values is a bf16
// value, so they are exact).  Pass 2 is a small product per head, Nb x Nb
// outputs over D: for bf16 on the matrix cores (block_scores_mfma_kernel),
// otherwise in fp32 FMAs tiled 64 x 64 per workgroup through LDS, with the
// two dot products of a score sharing their query operand.
#include "common.h"

#include <algorithm>

namespace bsa {
namespace {

constexpr int kWaves = 4;
constexpr int kBatch = 8;  // token rows loaded per lane before use

struct SumParams {
    const char* q;
    const char* k;
    char* summ;  // 4 x (BH, Nb, D) of the input dtype
    float* knorm;  // (BH, Nb): largest L2 norm of a key row in each block, or null
    uint32_t block, nb, vecs_per_row, BH;
    uint32_t head_len;      // token rows of a head in q and k
    const int32_t* labels;  // (BH, S) or null; tokens labelled < 0 are left out
    // tiled: q, k in T-major order, block = tile of the head's tiling
    const int32_t* head_choice;
    uint32_t n_tiles, Hg, Wg;
    TileGeo geo[BSA_MAX_TILINGS];
    // padded along T (tiled): each candidate's block count on its padded grid
    uint32_t nbt[BSA_MAX_TILINGS];
    // tiled, optional: q's summaries of every candidate, [n_tiles][2][BH][Nb][D]
    // (bsa_select_tiling_ex writes them); the q half then copies the chosen
    // candidate's instead of reading q
    const char* qsumm;
};

// blockIdx: x = group of kWaves blocks, y = 0 (q) / 1 (k), z = b*H + h.
// LABELS: P.labels is set (contiguous blocks only).
// PADT (tiled): the tiling's grid is padded along T; a cell at or past the
// head's end is padding, left out and not read, and blocks past the head's
// own count hold padding only.
template <int EPV, int LPT, bool TILED, bool LABELS, bool PADT = false>
__global__ __launch_bounds__(64 * kWaves) void block_minmax_kernel(const SumParams P) {
    constexpr int TPI = 64 / LPT;
    const int lane = threadIdx.x & 63;
    const uint32_t blk = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (blk >= P.nb) return;
    const uint32_t which = blockIdx.y;
    const uint32_t bh = blockIdx.z;
    const size_t row_bytes = (size_t)P.vecs_per_row * 16;
    uint32_t origin = 0;
    bool block_real = true;  // PADT: the block is a tile of the head's padded grid
    TileGeo g{};  // a copy: indexing the by-value parameter through a pointer puts it in scratch memory
    if (TILED) {
        uint32_t c = P.head_choice != nullptr ? (uint32_t)__builtin_amdgcn_readfirstlane(P.head_choice[bh]) : 0u;
        if (c >= P.n_tiles) c = 0;  // out-of-range choices are caught by bsa_validate_indices
        if (which == 0 && P.qsumm != nullptr) {
            if (lane < LPT) {
                const size_t plane = (size_t)P.BH * P.nb * row_bytes;
                const size_t at = ((size_t)bh * P.nb + blk) * row_bytes + (size_t)lane * 16;
                const char* from = P.qsumm + (size_t)(2 * c) * plane + at;
                *reinterpret_cast<uint4*>(P.summ + at) = *reinterpret_cast<const uint4*>(from);
                *reinterpret_cast<uint4*>(P.summ + plane + at) = *reinterpret_cast<const uint4*>(from + plane);
            }
            return;
        }
        g = P.geo[c];
        if (PADT) block_real = blk < P.nbt[c];
        origin = block_real ? tile_origin(blk, g, P.Hg, P.Wg) : 0u;
    }
    const char* head_src = (which == 0 ? P.q : P.k) + (size_t)bh * P.head_len * row_bytes;
    const char* src = TILED ? head_src + (size_t)origin * row_bytes : head_src + (size_t)blk * P.block * row_bytes;
    const int sub = lane % LPT;
    const int slot = lane / LPT;
    RowRange<EPV> range;
    range.init();
    const int32_t* lab = LABELS ? P.labels + ((size_t)bh * P.nb + blk) * P.block : nullptr;
    // key blocks: also the largest squared row norm (a row's LPT lanes add
    // their squares; every pass of the loop keeps the same lanes together)
    const bool norms = which == 1 && P.knorm != nullptr;
    float n2max = 0.f;
    // kBatch rows per lane are loaded before any is used, so that many loads
    // are in flight per wave; a row past the block loads the block's first
    // row (which the summaries may take in again, but the norms leave out),
    // and a row labelled < 0 is left out.
    for (uint32_t t0 = slot; t0 < P.block; t0 += TPI * kBatch) {
        uint4 raw[kBatch];
        bool use[kBatch], real[kBatch];
        int32_t lv[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const uint32_t t = t0 + j * TPI;
            const uint32_t tc = t < P.block ? t : 0u;
            if (LABELS) lv[j] = lab[tc];
            uint32_t r = TILED ? cell_offset(tc, g, P.Hg, P.Wg) : tc;
            real[j] = !PADT || (block_real && origin + r < P.head_len);
            if (!real[j]) r = 0u;  // padding: the head's first row stands in, and is left out below
            raw[j] = *reinterpret_cast<const uint4*>((real[j] ? src : head_src) + (size_t)r * row_bytes +
                                                     (size_t)sub * 16);
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) use[j] = t0 + j * TPI < P.block && (!LABELS || lv[j] >= 0) && real[j];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            if (!(LABELS || PADT) || use[j]) range.add(raw[j]);
            if (norms) {
                float v[EPV];
                unpack<EPV>(raw[j], v);
                float n2 = 0.f;
#pragma unroll
                for (int i = 0; i < EPV; ++i) n2 = fmaf(v[i], v[i], n2);
                // every lane of the row group takes part in the lane swaps
                const float row = group_sum<LPT>(n2);
                if (use[j]) n2max = fmaxf(n2max, row);
            }
        }
    }
    if (norms) {
#pragma unroll
        for (int off = LPT; off < 64; off <<= 1) n2max = fmaxf(n2max, __shfl_xor(n2max, off));
        if (lane == 0) P.knorm[(size_t)bh * P.nb + blk] = sqrtf(n2max);
    }
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) range.merge_lanes(off);
    if (slot == 0) {
        const size_t plane = (size_t)P.BH * P.nb * row_bytes;
        char* dst = P.summ + (size_t)(2 * which) * plane + ((size_t)bh * P.nb + blk) * row_bytes + (size_t)sub * 16;
        *reinterpret_cast<uint4*>(dst) = range.max_row();
        *reinterpret_cast<uint4*>(dst + plane) = range.min_row();
    }
}

constexpr int kTile = 64;  // output tile (I x J)
constexpr int kDC = 32;    // D chunk staged in LDS

template <bool BF16>
__device__ __forceinline__ float load_elem(const char* base, size_t idx) {
    if (BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[idx]);
    return reinterpret_cast<const float*>(base)[idx];
}

// S[I, J] = max(c_I . kmax_J, c_I . kmin_J), c = qmax + qmin.
// blockIdx: x = J tile, y = I tile, z = b*H + h.  Thread (ty, tx) owns
// I = I0 + ty + 16 r and J = J0 + tx + 16 c for r, c < 4.
template <bool BF16>
__global__ __launch_bounds__(256) void block_scores_kernel(const char* __restrict__ summ, uint32_t BH, uint32_t nb,
                                                           uint32_t D, float* __restrict__ scores) {
    __shared__ float Cs[kDC][kTile + 1];
    __shared__ float Xs[kDC][kTile + 1];
    __shared__ float Ns[kDC][kTile + 1];
    const uint32_t bh = blockIdx.z;
    const uint32_t I0 = blockIdx.y * kTile, J0 = blockIdx.x * kTile;
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const size_t plane = (size_t)BH * nb * D;
    const size_t head = (size_t)bh * nb * D;
    const char* es = summ;
    const int esz = BF16 ? 2 : 4;
    const char* qmax = es;
    const char* qmin = es + plane * esz;
    const char* kmax = es + 2 * plane * esz;
    const char* kmin = es + 3 * plane * esz;
    float ax[4][4], an[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) ax[r][c] = an[r][c] = 0.f;

    for (uint32_t d0 = 0; d0 < D; d0 += kDC) {
        // stage 64 rows x kDC columns of c, kmax and kmin (column-major in LDS)
#pragma unroll
        for (int e = tid; e < kTile * kDC; e += 256) {
            const int row = e / kDC, col = e % kDC;
            const uint32_t d = d0 + col;
            float cv = 0.f, xv = 0.f, nv = 0.f;
            if (d < D) {
                if (I0 + row < nb) {
                    const size_t idx = head + (size_t)(I0 + row) * D + d;
                    cv = load_elem<BF16>(qmax, idx) + load_elem<BF16>(qmin, idx);
                }
                if (J0 + row < nb) {
                    const size_t idx = head + (size_t)(J0 + row) * D + d;
                    xv = load_elem<BF16>(kmax, idx);
                    nv = load_elem<BF16>(kmin, idx);
                }
            }
            Cs[col][row] = cv;
            Xs[col][row] = xv;
            Ns[col][row] = nv;
        }
        __syncthreads();
#pragma unroll 8
        for (int d = 0; d < kDC; ++d) {
            float a[4], bx[4], bn[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) a[r] = Cs[d][ty + 16 * r];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                bx[c] = Xs[d][tx + 16 * c];
                bn[c] = Ns[d][tx + 16 * c];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    ax[r][c] = fmaf(a[r], bx[c], ax[r][c]);
                    an[r][c] = fmaf(a[r], bn[c], an[r][c]);
                }
        }
        __syncthreads();
    }
    // a block without tokens has max = -inf (inputs are finite otherwise)
    bool ok_i[4], ok_j[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t I = I0 + ty + 16 * r, J = J0 + tx + 16 * r;
        ok_i[r] = I < nb && load_elem<BF16>(qmax, head + (size_t)I * D) != -__builtin_inff();
        ok_j[r] = J < nb && load_elem<BF16>(kmax, head + (size_t)J * D) != -__builtin_inff();
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t I = I0 + ty + 16 * r;
        if (I >= nb) continue;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t J = J0 + tx + 16 * c;
            if (J < nb)
                scores[((size_t)bh * nb + I) * nb + J] =
                    (ok_i[r] && ok_j[c]) ? fmaxf(ax[r][c], an[r][c]) : -__builtin_inff();
        }
    }
}

// bf16 summaries, D a multiple of 16: the same scores on the matrix cores.
// c = qmax + qmin is formed in fp32 (as above) and split exactly into three
// bf16 parts, c = c0 + c1 + c2 (8 significant bits each cover fp32's 24), so
// every product c_d * k_d is exact and the MFMAs accumulate in fp32, as the
// FMA chain does.  One wave per 32 x 32 tile of (I, J): S^T-free layout,
// A = parts of c (rows I), B = kmax / kmin (columns J).
typedef __bf16 bf16x8s __attribute__((ext_vector_type(8)));
typedef float f32x16s __attribute__((ext_vector_type(16)));

// c = qmax + qmin over eight dims (a, b: eight bf16 values each), split
// exactly into three bf16 parts c = p0 + p1 + p2, and the six MFMAs of one
// 16-dim step: S_max += c kmax^T, S_min += c kmin^T over the three parts
__device__ __forceinline__ void score_step(const uint4 a, const uint4 b, const uint4 x, const uint4 n, f32x16s& sx,
                                           f32x16s& sn) {
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
    bf16x8s p0, p1, p2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t ha = (e & 1) ? (wa[e / 2] & 0xffff0000u) : (wa[e / 2] << 16);
        const uint32_t hb = (e & 1) ? (wb[e / 2] & 0xffff0000u) : (wb[e / 2] << 16);
        const float c = __uint_as_float(ha) + __uint_as_float(hb);
        const __bf16 c0 = (__bf16)c;
        const float r1 = c - (float)c0;
        const __bf16 c1 = (__bf16)r1;
        p0[e] = c0;
        p1[e] = c1;
        p2[e] = (__bf16)(r1 - (float)c1);
    }
    const bf16x8s bx = __builtin_bit_cast(bf16x8s, x), bn = __builtin_bit_cast(bf16x8s, n);
    sx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p0, bx, sx, 0, 0, 0);
    sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p0, bn, sn, 0, 0, 0);
    sx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p1, bx, sx, 0, 0, 0);
    sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p1, bn, sn, 0, 0, 0);
    sx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p2, bx, sx, 0, 0, 0);
    sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p2, bn, sn, 0, 0, 0);
}

// ND > 0: D = 16 * ND and every step's operands are loaded before the first
// MFMA (one memory latency per tile instead of one per step); ND = 0: any D,
// one step at a time.
template <int ND>
__global__ __launch_bounds__(64) void block_scores_mfma_kernel(const uint16_t* __restrict__ summ, uint32_t BH,
                                                               uint32_t nb, uint32_t D, float* __restrict__ scores) {
    const int lane = threadIdx.x;
    // 1D grid of (head, I tile, J tile), J fastest; each XCD (workgroup w runs
    // on XCD w % 8) takes a contiguous range, so a head's summaries are read
    // by one XCD and stay in its L2 (spread over all eight, they were fetched
    // from beyond L2 about once per output tile)
    uint32_t w = blockIdx.x;
    if (gridDim.x % 8u == 0u) w = (w & 7u) * (gridDim.x >> 3) + (w >> 3);
    const uint32_t n32 = (nb + 31) / 32;
    const uint32_t bh = w / (n32 * n32);
    const uint32_t I0 = (w / n32 % n32) * 32, J0 = (w % n32) * 32;
    const size_t plane = (size_t)BH * nb * D;
    const size_t head = (size_t)bh * nb * D;
    const uint16_t* qmax = summ;
    const uint16_t* qmin = summ + plane;
    const uint16_t* kmax = summ + 2 * plane;
    const uint16_t* kmin = summ + 3 * plane;
    const int r = lane & 31, kg = lane >> 5;
    const uint32_t I = min(I0 + r, nb - 1), J = min(J0 + r, nb - 1);  // rows past nb are computed and dropped
    f32x16s sx, sn;
#pragma unroll
    for (int v = 0; v < 16; ++v) sx[v] = sn[v] = 0.f;
    auto ld = [&](const uint16_t* base, uint32_t row, uint32_t d) {
        return *reinterpret_cast<const uint4*>(base + head + (size_t)row * D + d);
    };
    uint4 a[ND > 0 ? ND : 1], b[ND > 0 ? ND : 1], x[ND > 0 ? ND : 1], n[ND > 0 ? ND : 1];
    if (ND > 0) {
#pragma unroll
        for (int s = 0; s < ND; ++s) {
            const uint32_t d = 16 * s + 8 * kg;
            a[s] = ld(qmax, I, d);
            b[s] = ld(qmin, I, d);
            x[s] = ld(kmax, J, d);
            n[s] = ld(kmin, J, d);
        }
#pragma unroll
        for (int s = 0; s < ND; ++s) score_step(a[s], b[s], x[s], n[s], sx, sn);
    } else {
        for (uint32_t d0 = 0; d0 < D; d0 += 16) {
            const uint32_t d = d0 + 8 * kg;
            score_step(ld(qmax, I, d), ld(qmin, I, d), ld(kmax, J, d), ld(kmin, J, d), sx, sn);
        }
    }
    // value v of lane l: row I0 + 8(v/4) + 4(l/32) + v%4, column J0 + l%32.
    // A block with no token (max -inf) scores -inf: with the operands in
    // registers (ND > 0), lane r < 32 holds element 0 of rows I0 + r and
    // J0 + r, and the other lanes take theirs by shuffles instead of loads.
    const uint32_t Jc = J0 + r;
    bool ok_i[16], ok_j;
    if (ND > 0) {
        const int qf0 = (int)(a[0].x & 0xffffu), kf0 = (int)(x[0].x & 0xffffu);
        ok_j = __shfl(kf0, r) != 0xff80;
#pragma unroll
        for (int v = 0; v < 16; ++v) ok_i[v] = __shfl(qf0, 8 * (v / 4) + 4 * kg + (v % 4)) != 0xff80;
    }
    if (Jc >= nb) return;
    if (ND == 0) {
        ok_j = bf16_to_f32(kmax[head + (size_t)Jc * D]) != -__builtin_inff();
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const uint32_t Ir = min(I0 + 8 * (v / 4) + 4 * kg + (v % 4), nb - 1);
            ok_i[v] = bf16_to_f32(qmax[head + (size_t)Ir * D]) != -__builtin_inff();
        }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const uint32_t Ir = I0 + 8 * (v / 4) + 4 * kg + (v % 4);
        if (Ir >= nb) continue;
        scores[((size_t)bh * nb + Ir) * nb + Jc] = (ok_i[v] && ok_j) ? fmaxf(sx[v], sn[v]) : -__builtin_inff();
    }
}

}  // namespace
}  // namespace bsa

using namespace bsa;

namespace bsa {
namespace {

int minmax_scores(const void* q, const void* k, int dtype, int64_t B, int64_t H, int64_t S, int64_t D, int block,
                  const int32_t* labels, SumParams& P, bool tiled, void* summaries, float* scores, float* key_norms,
                  hipStream_t st, const char* name, bool pad = false, int64_t head_len = 0) {
    const int es = elem_size(dtype);
    BSA_REQUIRE(es != 0, "%s: unknown dtype %d", name, dtype);
    BSA_REQUIRE(q && k && summaries && scores, "%s: NULL argument", name);
    BSA_REQUIRE(B >= 1 && H >= 1 && S >= 1 && D >= 1, "%s: sizes must be >= 1", name);
    BSA_REQUIRE(B * H <= 65535, "%s: B*H too large", name);
    BSA_REQUIRE(block >= 1 && S % block == 0, "%s: block %d must divide S=%lld", name, block, (long long)S);
    BSA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(summaries), "%s: tensors must be 16-byte aligned", name);
    const int64_t row_bytes = D * es;
    BSA_REQUIRE(row_bytes % 16 == 0, "%s: D*elem_size must be a multiple of 16 bytes", name);
    const int64_t vecs = row_bytes / 16;
    const int64_t nb = S / block;
    BSA_REQUIRE(nb <= 65535 * kTile, "%s: too many blocks", name);
    BSA_REQUIRE(B * H * nb * D < ((int64_t)1 << 40), "%s: too large", name);
    P.q = static_cast<const char*>(q);
    P.k = static_cast<const char*>(k);
    P.summ = static_cast<char*>(summaries);
    P.block = (uint32_t)block;
    P.nb = (uint32_t)nb;
    P.vecs_per_row = (uint32_t)vecs;
    P.BH = (uint32_t)(B * H);
    P.labels = labels;
    P.knorm = key_norms;
    P.head_len = (uint32_t)(head_len > 0 ? head_len : S);
    dim3 g1((unsigned)((nb + kWaves - 1) / kWaves), 2, (unsigned)(B * H));
#define BSA_MM(EPV, LPT)                                                                                \
    (pad ? block_minmax_kernel<EPV, LPT, true, false, true><<<g1, 64 * kWaves, 0, st>>>(P)             \
     : tiled ? block_minmax_kernel<EPV, LPT, true, false><<<g1, 64 * kWaves, 0, st>>>(P)               \
     : labels ? block_minmax_kernel<EPV, LPT, false, true><<<g1, 64 * kWaves, 0, st>>>(P)              \
              : block_minmax_kernel<EPV, LPT, false, false><<<g1, 64 * kWaves, 0, st>>>(P))
    const bool bf = dtype == BSA_BF16;
    switch (vecs) {
        case 1: if (bf) BSA_MM(8, 1); else BSA_MM(4, 1); break;
        case 2: if (bf) BSA_MM(8, 2); else BSA_MM(4, 2); break;
        case 4: if (bf) BSA_MM(8, 4); else BSA_MM(4, 4); break;
        case 8: if (bf) BSA_MM(8, 8); else BSA_MM(4, 8); break;
        case 16: if (bf) BSA_MM(8, 16); else BSA_MM(4, 16); break;
        case 32: if (bf) BSA_MM(8, 32); else BSA_MM(4, 32); break;
        default: BSA_FAIL(BSA_ERR_UNSUPPORTED, "%s: D=%lld unsupported", name, (long long)D);
    }
#undef BSA_MM
    int rc = check_launch(name);
    if (rc) return rc;
    if (bf && D % 16 == 0) {
        const uint64_t n32 = (uint64_t)((nb + 31) / 32);
        BSA_REQUIRE(n32 * n32 * (uint64_t)(B * H) < ((uint64_t)1 << 31), "%s: too many score tiles", name);
        const dim3 g3((uint32_t)(n32 * n32 * (uint64_t)(B * H)));
        const uint16_t* summ = static_cast<const uint16_t*>(summaries);
        if (D == 128)
            block_scores_mfma_kernel<8><<<g3, 64, 0, st>>>(summ, P.BH, P.nb, (uint32_t)D, scores);
        else if (D == 64)
            block_scores_mfma_kernel<4><<<g3, 64, 0, st>>>(summ, P.BH, P.nb, (uint32_t)D, scores);
        else
            block_scores_mfma_kernel<0><<<g3, 64, 0, st>>>(summ, P.BH, P.nb, (uint32_t)D, scores);
        return check_launch(name);
    }
    const unsigned nt = (unsigned)((nb + kTile - 1) / kTile);
    dim3 g2(nt, nt, (unsigned)(B * H));
    if (bf)
        block_scores_kernel<true><<<g2, 256, 0, st>>>(static_cast<const char*>(summaries), P.BH, P.nb, (uint32_t)D,
                                                      scores);
    else
        block_scores_kernel<false><<<g2, 256, 0, st>>>(static_cast<const char*>(summaries), P.BH, P.nb, (uint32_t)D,
                                                       scores);
    return check_launch(name);
}

}  // namespace
}  // namespace bsa

extern "C" int bsa_minmax_block_scores_masked(const void* q, const void* k, int dtype, int64_t B, int64_t H,
                                              int64_t S, int64_t D, int block, const int32_t* labels_or_null,
                                              void* summaries, float* scores, float* key_norms_or_null,
                                              bsa_stream_t stream) {
    clear_error();
    SumParams P{};
    return minmax_scores(q, k, dtype, B, H, S, D, block, labels_or_null, P, false, summaries, scores,
                         key_norms_or_null, (hipStream_t)stream, "bsa_minmax_block_scores");
}

extern "C" int bsa_minmax_block_scores_tiled(const void* q, const void* k, int dtype, int64_t B, int64_t H, int T,
                                             int Hg, int Wg, int64_t D, const int32_t* tiles_host, int n_tiles,
                                             const int32_t* head_choice, void* summaries, float* scores,
                                             float* key_norms_or_null, const void* q_summaries_or_null,
                                             bsa_stream_t stream) {
    clear_error();
    const char* name = "bsa_minmax_block_scores_tiled";
    BSA_REQUIRE(T > 0 && Hg > 0 && Wg > 0, "%s: grid must be positive", name);
    int rc = check_tiles(T, Hg, Wg, tiles_host, n_tiles);
    if (rc) return rc;
    SumParams P{};
    const int vol = tiles_host[0] * tiles_host[1] * tiles_host[2];
    for (int i = 0; i < BSA_MAX_TILINGS; ++i) {
        const int j = i < n_tiles ? i : 0;
        const int a = tiles_host[3 * j], b = tiles_host[3 * j + 1], c = tiles_host[3 * j + 2];
        BSA_REQUIRE(a * b * c == vol, "%s: candidate tiles must share one volume", name);
        P.geo[i] = make_geo(Hg, Wg, a, b, c);
    }
    P.head_choice = head_choice;
    P.n_tiles = (uint32_t)n_tiles;
    P.Hg = (uint32_t)Hg;
    P.Wg = (uint32_t)Wg;
    P.qsumm = static_cast<const char*>(q_summaries_or_null);
    BSA_REQUIRE(aligned16(P.qsumm), "%s: q summaries must be 16-byte aligned", name);
    return minmax_scores(q, k, dtype, B, H, (int64_t)T * Hg * Wg, D, vol, nullptr, P, true, summaries, scores,
                         key_norms_or_null, (hipStream_t)stream, name);
}

extern "C" int bsa_minmax_block_scores_tiled_padded(const void* q, const void* k, int dtype, int64_t B, int64_t H,
                                                    int T, int Hg, int Wg, int64_t D, const int32_t* tiles_host,
                                                    int n_tiles, const int32_t* head_choice, void* summaries,
                                                    float* scores, float* key_norms_or_null, bsa_stream_t stream) {
    clear_error();
    const char* name = "bsa_minmax_block_scores_tiled_padded";
    int rc = check_tiles_padded(T, Hg, Wg, tiles_host, n_tiles);
    if (rc) return rc;
    SumParams P{};
    const int vol = tiles_host[0] * tiles_host[1] * tiles_host[2];
    int64_t nb = 0;
    for (int i = 0; i < BSA_MAX_TILINGS; ++i) {
        const int j = i < n_tiles ? i : 0;
        const int a = tiles_host[3 * j], b = tiles_host[3 * j + 1], c = tiles_host[3 * j + 2];
        BSA_REQUIRE(a * b * c == vol, "%s: candidate tiles must share one volume", name);
        if (Hg % b != 0 || Wg % c != 0)
            BSA_FAIL(BSA_ERR_UNSUPPORTED, "%s: padding along T only (tile %d is %dx%dx%d on a %dx%dx%d grid)", name,
                     j, a, b, c, T, Hg, Wg);
        P.geo[i] = make_geo_padded(Hg, Wg, a, b, c);
        const int64_t n = padded_length(T, Hg, Wg, a, b, c) / vol;
        P.nbt[i] = (uint32_t)n;
        nb = std::max<int64_t>(nb, n);
    }
    P.head_choice = head_choice;
    P.n_tiles = (uint32_t)n_tiles;
    P.Hg = (uint32_t)Hg;
    P.Wg = (uint32_t)Wg;
    return minmax_scores(q, k, dtype, B, H, nb * vol, D, vol, nullptr, P, true, summaries, scores, key_norms_or_null,
                         (hipStream_t)stream, name, true, (int64_t)T * Hg * Wg);
}

extern "C" int bsa_minmax_block_scores(const void* q, const void* k, int dtype, int64_t B, int64_t H, int64_t S,
                                       int64_t D, int block, void* summaries, float* scores, float* key_norms_or_null,
                                       bsa_stream_t stream) {
    return bsa_minmax_block_scores_masked(q, k, dtype, B, H, S, D, block, nullptr, summaries, scores,
                                          key_norms_or_null, stream);
}
