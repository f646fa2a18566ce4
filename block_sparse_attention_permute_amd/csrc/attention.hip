// Block-sparse and sliding-window attention: bsa_block_sparse_attention and
// bsa_windowed_attention.
//
// Both compute dense scaled dot-product attention under an additive 0/-inf
// mask while visiting only the key blocks the mask keeps:
//  * block-sparse: query block I attends to the key blocks of its compact
//    list ([Adaptive tiling (SPADE), "Recipe": the block mask expanded to
//    tokens; "Dense by design": skipping masked blocks is where the speed
//    comes from]);
//  * windowed: query i attends to keys with abs(i - j) <= window/2 and to the
//    sinks j < sink, and a query block reads only the key tiles of its local
//    slice and the sink tiles ([FastVideo windowed_attention.py, "Window
//    policy" and "Implementation note (FLOPs)"]).
//
// Kernels:
//  * attn_solo_kernel (bf16, D = 128, blocks of 64): one single-wave
//    workgroup per query block; described at its definition.  Modes: block
//    list, window, labels (a token rule inside kept blocks), and gather on
//    load (q, k, v, out in T-major order, blocks = tiles of a tiling);
//  * attn_mfma_kernel (bf16, D in {64, 128}, blocks of 32 or 64; used for
//    D = 64 and blocks of 32): one workgroup per query block of
//    (BLK/32) x (BLK/32) waves; wave (wr, wk) owns query rows 32*wr..+32 and
//    key columns 32*wk..+32 of every key block, all waves share each K/V tile
//    staged in LDS (double-buffered, one barrier per tile), and the key
//    halves are merged through LDS at the end;
//  * attn_scalar_kernel: one thread per query row, fp32 math, for fp32
//    tensors and every other shape.
// Common to the MFMA kernels:
//  * scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    each lane then holds 16 scores of ONE query row, which is exactly the
//    B-operand layout of O^T = V^T P^T, so P never leaves registers;
//  * V^T fragments come from LDS with the transposing ds_read_b64_tr_b16;
//  * online softmax in fp32 with exp2 (log2 e folded into the scale) and a
//    lazy rescale: the running max is only moved when a row's max grows by
//    more than 2^8, which skips almost every O rescale;
//  * workgroups are remapped so consecutive query blocks of a head run on
//    the same XCD and share its L2 (neighbouring query blocks keep many of
//    the same key blocks).
#include "common.h"

#include <algorithm>
#include <type_traits>

namespace bsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// row sums add the bf16-rounded P two at a time (v_dot2 with ones): exactly
// the weights the P V product uses
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
constexpr float kRescaleSlack = 8.0f;  // log2 units: P may grow to 2^8 before a rescale
constexpr float kSkipSlack = 32.0f;    // log2 units: P may reach 2^32 in a tile that skips the max

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8; a field at its maximum does not wait)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kVmcnt16 = waitcnt_vm(16);  // all but the 16 most recent vector-memory ops
constexpr int kLgkmcnt0 = 0xC07F;         // all LDS / scalar-memory ops
constexpr int kVm16Lgkm0 = kVmcnt16 & ~0x0F00;  // vmcnt(16) and lgkmcnt(0)
static_assert(kVmcnt16 == 0x4F70, "vmcnt(16) encoding");

// kLabels: a block list plus the token rule labels[i] == labels[j] inside
// the kept blocks (padding of a padded tiling, spatial-only attention).
// kGroups: temporal-only attention of T-major tensors; a query tile holds the
// T frames of G = 64 / T spatial positions, read straight from T-major
// memory, and attends to itself under the rule "same position".
enum Mode { kBlockList = 0, kWindow = 1, kLabels = 2, kGroups = 3 };

struct AttnParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* out;
    uint32_t S, nq;        // sequence length, query blocks per head
    uint32_t n_wg;         // workgroups in the grid
    uint32_t xcd_remap;    // 1: spread heads over XCDs in contiguous ranges
    uint32_t xcd_per_head; // single-wave kernel: XCDs that share each head (1, 2, 4 or 8)
    float scale_log2;      // softmax scale * log2(e)
    // block list
    const int32_t* kv_idx;
    const int32_t* kv_cnt;
    uint32_t max_kept;
    // block lists: workgroup w runs row row_order[w] = (b*H + h)*nq + I when
    // not null (entries past the last row are empty slots), in a grid of
    // `grid` workgroups (0: n_wg, one per row)
    const uint32_t* row_order;
    uint32_t grid;
    // window
    int32_t half, sink;
    // block lists: per key block, at least the largest L2 norm of its key rows, or null
    const float* knorm;
    // labels
    const int32_t* labels;
    uint64_t label_stride;  // elements between heads (0: one row for all heads)
    // tiled (gather on load): q, k, v, out stay in T-major order and block J
    // of a head is tile J of the head's tiling
    const int32_t* head_choice;
    uint32_t n_tiles, Hg, Wg;
    // groups: T frames per position, G positions per tile, HW positions per frame
    uint32_t grp_T, grp_G, grp_HW;
    TileGeo geo[BSA_MAX_TILINGS];
    int32_t voff[BSA_MAX_TILINGS][16];   // byte offset of cell 4q (a DMA row group) from the tile origin
    int32_t rdelta[BSA_MAX_TILINGS][4];  // byte offsets of cells 4q + j from cell 4q (the same for every q)
    // padded along T: frames of the grid, and each tiling's block count on its padded grid
    uint32_t T;
    uint32_t nbt[BSA_MAX_TILINGS];
};

template <int D, int BLK>
struct Cfg {
    static constexpr int NWR = BLK / 32, NWK = BLK / 32, NW = NWR * NWK, NT = 64 * NW;
    static constexpr int NCH = D / 8;             // 16-byte chunks per row
    static constexpr int TILE = BLK * D * 2;      // one K or V tile in LDS (swizzled, unpadded)
    static constexpr int STAGE = 2 * TILE;        // K then V
    static constexpr int CH = BLK * NCH / NT;     // 16-byte chunks per thread per tensor
    static constexpr int MERGE = (NW - NWR) * 64 * (D / 2 + 2) * 4;
    static constexpr int SMEM = (2 * STAGE > MERGE) ? 2 * STAGE : MERGE;
    static constexpr int SMEM1 = (STAGE > MERGE) ? STAGE : MERGE;  // one key tile: no second stage
    static_assert(CH >= 1 && (BLK * NCH) % NT == 0, "uneven staging");
};

// LDS rows are stored unpadded with their 16-byte chunks XOR-swizzled per
// row, with a different swizzle for each tile so that both readers are free
// of bank conflicts:
//  * K, chunk ^ (row % 8): a 128-bit K read has 8 consecutive rows reading
//    one chunk, which then land on 8 different 4-bank groups;
//  * V, chunk ^ 2*(row % 4): a transposing read has 4 consecutive rows
//    reading an aligned chunk pair, which then land on 4 different 8-bank
//    groups.
template <int D>
__device__ __forceinline__ int k_lds(int row, int chunk) {
    return row * (D * 2) + ((chunk ^ (row & 7)) << 4);
}
template <int D>
__device__ __forceinline__ int v_lds(int row, int chunk) {
    return row * (D * 2) + ((chunk ^ ((row & 3) << 1)) << 4);
}

// The single-wave kernel's tiles (D = 128: 16 chunks per row) use wider
// swizzles, measured with the LDS bank-conflict counter: the LDS serves 256
// bytes (64 banks) per pass, i.e. 16 lanes of a 128-bit read or 32 lanes of a
// 64-bit read, and the narrower swizzles above repeat within such a pass (a
// 2-way conflict: 4 extra cycles per K read, 2 per V read):
//  * K, chunk ^ (row % 16): the 16 consecutive rows of a 128-bit read's pass
//    land on 16 different 4-bank groups;
//  * V, chunk ^ 4*(row % 4): the 4 rows times 4 chunks of a transposing read's
//    32-lane pass land on 16 different 4-bank groups.
__device__ __forceinline__ int k_lds_solo(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }
__device__ __forceinline__ int v_lds_solo(int row, int chunk) { return row * 256 + ((chunk ^ ((row & 3) << 2)) << 4); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Registers holding one K/V tile on its way from global memory to LDS.
template <int D, int BLK>
struct Staging {
    u32x4 k[Cfg<D, BLK>::CH], v[Cfg<D, BLK>::CH];
};

// Buffer loads of key rows [j0, j0 + BLK): the tile offset is a scalar, the
// per-thread offset a loop invariant, and rows past the end read as zero.
template <int D, int BLK>
__device__ __forceinline__ void stage_load(Staging<D, BLK>& st, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                           int j0, int tid) {
    using C = Cfg<D, BLK>;
    const int soff = j0 * (D * 2);
#pragma unroll
    for (int j = 0; j < C::CH; ++j) {
        const int c = tid + C::NT * j;
        const int voff = (c / C::NCH) * (D * 2) + (c % C::NCH) * 16;
        st.k[j] = __builtin_amdgcn_raw_buffer_load_b128(kr, voff, soff, 0);
        st.v[j] = __builtin_amdgcn_raw_buffer_load_b128(vr, voff, soff, 0);
    }
}

template <int D, int BLK>
__device__ __forceinline__ void stage_store(const Staging<D, BLK>& st, char* stage, int tid) {
    using C = Cfg<D, BLK>;
#pragma unroll
    for (int j = 0; j < C::CH; ++j) {
        const int c = tid + C::NT * j;
        const int row = c / C::NCH, chunk = c % C::NCH;
        *reinterpret_cast<u32x4*>(stage + k_lds<D>(row, chunk)) = st.k[j];
        *reinterpret_cast<u32x4*>(stage + C::TILE + v_lds<D>(row, chunk)) = st.v[j];
    }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int N>
using ic = std::integral_constant<int, N>;

// POS: the softmax scale is positive, so the row max of the raw scores gives
// the max of the scaled ones and exp2(s * c - m) is one FMA and one exp.
// kv_idx / kv_cnt are separate restrict arguments so their uniform reads
// become scalar loads.
template <int D, int BLK, int MODE, bool POS>
__global__ __launch_bounds__((Cfg<D, BLK>::NT), (Cfg<D, BLK>::NT >= 256 ? 2 : 1)) void attn_mfma_kernel(
    const AttnParams P, const int32_t* __restrict__ kv_idx, const int32_t* __restrict__ kv_cnt) {
    using C = Cfg<D, BLK>;
    // groups mode visits one key tile and needs one LDS stage; at D = 128 that
    // makes room for three workgroups per CU instead of two
    __shared__ __attribute__((aligned(16))) char smem[MODE == kGroups ? C::SMEM1 : C::SMEM];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = wave % C::NWR, wk = wave / C::NWR;
    const int half_id = lane >> 5, col = lane & 31;

    uint32_t wg = blockIdx.x;
    if (MODE == kBlockList && P.row_order != nullptr) {
        wg = P.row_order[wg];
        if (wg >= P.n_wg) return;
    } else if (P.xcd_remap) {
        wg = (wg & 7u) * (P.n_wg >> 3) + (wg >> 3);
    }
    const uint32_t bh = wg / P.nq, I = wg % P.nq;
    const size_t head = (size_t)bh * P.S * D;
    const uint32_t head_bytes = P.S * D * 2;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(P.q + head, head_bytes);
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(P.k + head, head_bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(P.v + head, head_bytes);
    const int q0 = (int)I * BLK;

    // ---- key tiles to visit
    int n_iter;
    const int32_t* list = nullptr;
    int n_sink_tiles = 0, local_first = 0;
    if (MODE == kBlockList) {
        const size_t row = (size_t)bh * P.nq + I;
        n_iter = min(kv_cnt[row], (int)P.max_kept);
        list = kv_idx + row * P.max_kept;
    } else if (MODE == kGroups) {
        n_iter = 1;
    } else {
        n_sink_tiles = (P.sink + BLK - 1) / BLK;
        const int lo = max(0, q0 - P.half);
        const int hi = min((int)P.S, q0 + BLK - 1 + P.half + 1);  // exclusive
        const int t_lo = lo / BLK, t_hi = (hi - 1) / BLK;
        local_first = max(t_lo, n_sink_tiles);
        n_iter = n_sink_tiles + max(0, t_hi - local_first + 1);
    }
    // tile index of iteration `it` (wave-uniform: it feeds scalar buffer offsets)
    auto tile_at = [&](int it) -> int {
        if (MODE == kBlockList) return __builtin_amdgcn_readfirstlane(list[it]);
        if (MODE == kGroups) return (int)I;
        return it < n_sink_tiles ? it : local_first + (it - n_sink_tiles);
    };
    // kGroups: tile row r (r < G*T) is frame r % T of position I*G + r / T, at
    // T-major row (r % T) * HW + position; other rows (and positions past the
    // grid) are given an offset past the head, so buffer loads read zeros
    const int oob = (int)head_bytes;
    auto grp_row = [&](int r) -> int {  // T-major row of tile row r, or -1
        const int g = r / (int)P.grp_T, f = r - g * (int)P.grp_T;
        const int pos = (int)I * (int)P.grp_G + g;
        return (g < (int)P.grp_G && pos < (int)P.grp_HW) ? f * (int)P.grp_HW + pos : -1;
    };
    auto row_bytes = [&](int r) -> int {  // byte offset of tile row r from the head
        if (MODE != kGroups) return (q0 + r) * (D * 2);
        const int t = grp_row(r);
        return t >= 0 ? t * (D * 2) : oob;
    };

    // ---- Q fragment (B operand): row q0 + 32*wr + col, D cols 16*s + 8*half_id + 0..7
    bf16x8 qf[D / 16];
    {
        const int voff = row_bytes(32 * wr + col) + half_id * 16;
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            qf[s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, voff + 32 * s, 0, 0));
    }

    f32x16 o[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[t][v] = 0.f;
    float m_used = -1e30f, l_part = 0.f;
    const int my_row = q0 + 32 * wr + col;
    const float c_scale = POS ? P.scale_log2 : 1.0f;

    // loop-invariant LDS byte offsets of this lane's operands (stage 0)
    int k_addr[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) k_addr[s] = k_lds<D>(32 * wk + col, 2 * s + half_id);
    // transposing V reads: lane (g = lane/16, r = lane%16) addresses key
    // 32*wk + 16*m + 8*part + 4*(g/2) + r/4, column 32*t + 16*(g%2) + 4*(r%4);
    // the key offset 16*m + 8*part keeps row % 4, hence the swizzle
    const int g16 = lane >> 4, r16 = lane & 15;
    const int v_key0 = 32 * wk + 4 * (g16 >> 1) + (r16 >> 2);
    const int v_col0 = 16 * (g16 & 1) + 4 * (r16 & 3);
    int v_addr[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
        const int colv = 32 * t + v_col0;
        v_addr[t] = C::TILE + v_lds<D>(v_key0, colv >> 3) + (colv & 7) * 2;
    }

    // Tiles are prefetched two iterations ahead into two register sets, so a
    // tile's global loads have two iterations to land before it is written to
    // LDS; LDS is double-buffered (tile it in stage it % 2).
    Staging<D, BLK> st[2];
    if (MODE == kGroups) {  // one tile: the query tile's own rows, gathered
#pragma unroll
        for (int j = 0; j < C::CH; ++j) {
            const int c = tid + C::NT * j;
            const int voff = row_bytes(c / C::NCH) + (c % C::NCH) * 16;
            st[0].k[j] = __builtin_amdgcn_raw_buffer_load_b128(kr, voff, 0, 0);
            st[0].v[j] = __builtin_amdgcn_raw_buffer_load_b128(vr, voff, 0, 0);
        }
        stage_store<D, BLK>(st[0], smem, tid);
    } else if (n_iter > 0) {
        stage_load<D, BLK>(st[0], kr, vr, tile_at(0) * BLK, tid);
        stage_store<D, BLK>(st[0], smem, tid);
    }
    // Drain every load (the Q fragment included) before the loop, so that the
    // loop's only outstanding loads are the prefetched tiles': otherwise the
    // compiler's wait tracking makes each tile's QK^T wait for the prefetch.
    __builtin_amdgcn_s_waitcnt(0);
    if (MODE != kGroups && n_iter > 0) stage_load<D, BLK>(st[1], kr, vr, tile_at(min(1, n_iter - 1)) * BLK, tid);
    __syncthreads();
    // kGroups: this lane's row group (-1: a padding row, which sees no key)
    int my_grp = -1;
    if (MODE == kGroups) my_grp = grp_row(32 * wr + col) >= 0 ? (32 * wr + col) / (int)P.grp_T : -1;

    // One key tile.  CUR (0 or 1) is the LDS stage holding tile `it` and the
    // register set that receives tile it + 2; it is a compile-time constant so
    // every LDS address is a register plus an immediate offset.
    auto body = [&](auto cur_c, int it) {
        constexpr int CUR = decltype(cur_c)::value;
        // always issued (the last tile again past the end): a conditional load
        // would make the compiler's wait counts assume it was skipped and wait
        // for every outstanding load before the LDS store below
        if (MODE != kGroups) stage_load<D, BLK>(st[CUR], kr, vr, tile_at(min(it + 2, n_iter - 1)) * BLK, tid);
        const char* stage = smem + CUR * C::STAGE;

        // S^T (32 keys x 32 query rows) = K Q^T over D
        f32x16 sacc;
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            const bf16x8 kf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(stage + k_addr[s]));
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc, 0, 0, 0);
        }
        if (!POS) {
#pragma unroll
            for (int v = 0; v < 16; ++v) sacc[v] *= P.scale_log2;
        }
        // value v of this lane is key 8*(v/4) + 4*half_id + v%4 of the wave's half
        if (MODE == kWindow) {
            const int j0 = tile_at(it) * BLK;
            const int kbase = j0 + 32 * wk + 4 * half_id;
            const bool full = (j0 + BLK - 1 < P.sink) ||
                              (q0 + BLK - 1 - j0 <= P.half && j0 + BLK - 1 - q0 <= P.half && j0 + BLK <= (int)P.S);
            if (!full) {
                // branch-free selects: a short-circuit form of this test was
                // miscompiled (the store for v = 0 was dropped)
                const float neg_inf = -__builtin_inff();
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int j = kbase + 8 * (v / 4) + (v % 4);
                    const int d = my_row - j;
                    const bool vis = (j < (int)P.S) & (((d <= P.half) & (-d <= P.half)) | (j < P.sink));
                    sacc[v] = vis ? sacc[v] : neg_inf;
                }
            }
        }
        if (MODE == kGroups) {  // same position: key row j of the tile is in group j / T
            const float neg_inf = -__builtin_inff();
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int j = 32 * wk + 4 * half_id + 8 * (v / 4) + (v % 4);
                sacc[v] = (j / (int)P.grp_T == my_grp) ? sacc[v] : neg_inf;
            }
        }
        float smax = fmaxf(fmaxf(sacc[0], sacc[1]), sacc[2]);
#pragma unroll
        for (int v = 3; v < 15; v += 2) smax = fmaxf(fmaxf(smax, sacc[v]), sacc[v + 1]);
        smax = fmaxf(smax, sacc[15]);
        smax = fmaxf(smax, __shfl_xor(smax, 32));
        const float mloc = smax * c_scale;
        const bool grow = mloc > m_used + kRescaleSlack;
        if (__ballot(grow)) {
            const float m_new = grow ? mloc : m_used;
            const float alpha = __builtin_amdgcn_exp2f(m_used - m_new);
            m_used = m_new;
            l_part *= alpha;
#pragma unroll
            for (int t = 0; t < D / 32; ++t)
#pragma unroll
                for (int v = 0; v < 16; ++v) o[t][v] *= alpha;
        }
        bf16x8 pb[2];
        float psum;
        const float neg_m = -m_used;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sacc[v], c_scale, neg_m));
            psum = v == 0 ? p : psum + p;
            pb[v / 8][v % 8] = (__bf16)p;
        }
        l_part += psum;

        // O^T (D x 32 rows) += V^T P^T; slot jj of MFMA m is key 16m + 8*(jj/4) + 4*half_id + jj%4,
        // delivered by two transposing reads (jj < 4, jj >= 4)
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const char* va = stage + v_addr[t] + (16 * m) * (D * 2);
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)va);
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(va + 8 * (D * 2)));
                const s16x4 a8[2] = {lo, hi};
                o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a8), pb[m], o[t], 0, 0, 0);
            }
        }

        if (MODE != kGroups && it + 1 < n_iter) stage_store<D, BLK>(st[1 - CUR], smem + (1 - CUR) * C::STAGE, tid);
        __syncthreads();
    };
    int it = 0;
    // (groups mode: one tile, stage 0 only)
    for (; MODE != kGroups && it + 1 < n_iter; it += 2) {
        body(ic<0>{}, it);
        body(ic<1>{}, it + 1);
    }
    if (it < n_iter) body(ic<0>{}, it);

    // ---- merge the key halves of each row and write out
    float l_row = l_part + __shfl_xor(l_part, 32);
    float* mbuf = reinterpret_cast<float*>(smem);
    constexpr int REGS = D / 2 + 2;
    if (wk > 0) {
        float* dst = mbuf + ((size_t)((wk - 1) * C::NWR + wr) * REGS) * 64 + lane;
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) dst[(t * 16 + v) * 64] = o[t][v];
        dst[(D / 2) * 64] = m_used;
        dst[(D / 2 + 1) * 64] = l_row;
    }
    __syncthreads();
    if (wk > 0) return;
#pragma unroll
    for (int w = 1; w < C::NWK; ++w) {
        const float* src = mbuf + ((size_t)((w - 1) * C::NWR + wr) * REGS) * 64 + lane;
        const float m2 = src[(D / 2) * 64], l2 = src[(D / 2 + 1) * 64];
        const float mf = fmaxf(m_used, m2);
        const float a1 = exp2f(m_used - mf), a2 = exp2f(m2 - mf);
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) o[t][v] = o[t][v] * a1 + src[(t * 16 + v) * 64] * a2;
        l_row = l_row * a1 + l2 * a2;
        m_used = mf;
    }
    int out_row = my_row;
    if (MODE == kGroups) out_row = grp_row(32 * wr + col);
    if (out_row < 0 || out_row >= (int)P.S) return;
    const float inv = l_row > 0.f ? 1.0f / l_row : 0.f;  // a row that saw no key is written as zeros
    uint16_t* orow = P.out + head + (size_t)out_row * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            // values 4g .. 4g+3 are d = 32t + 8g + 4*half_id + 0..3; the hardware
            // conversion rounds to nearest even
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            bf16x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[t][4 * g + e] * inv);
            *reinterpret_cast<bf16x4*>(orow + 32 * t + 8 * g + 4 * half_id) = w;
        }
}

// ------------------------------------------------------------- one wave ---
// 64-token blocks, D = 128: one single-wave workgroup per query block.  The
// wave owns all 64 query rows (two 32-row tiles) and all 64 keys of each key
// tile (two 32-key halves):
//  * Q is loaded once into registers (the B operand of both row tiles);
//  * K goes global -> LDS with the LDS-destination buffer loads, whole 256-byte
//    rows per instruction (16 per tile, issued one tile ahead), and is read
//    back as A-operand fragments two score steps ahead.  Loading the A
//    fragments straight from global memory instead costs 32 partial cache
//    lines per instruction in the vector-memory path and was 7% slower;
//  * S^T = K Q^T is four independent 8-MFMA chains (key half x row tile), so
//    every K fragment feeds two MFMAs;
//  * V is staged through the wave's own LDS (no barrier: one wave) and read
//    back transposed; each V^T fragment feeds the two row tiles' MFMAs;
//  * nothing is shared between waves, so there are no barriers at all and
//    waves of different query blocks drift freely;
//  * one wave per SIMD has no other wave to hide its LDS latency, so the
//    loop is laid out by hand in steps fenced by scheduling barriers: K
//    fragments are read two score steps ahead, the V DMA is spread over the
//    score steps, and in the P V product the exps of 16-key group m+1 and its
//    V^T reads are issued beside the MFMAs of group m;
//  * block-list entries come one tile ahead through buffer loads (vector
//    memory), so waiting for them never waits on LDS traffic;
//  * EV (early V): the next tile's V DMA is issued beside the last 8 P V
//    MFMAs, once this tile's V^T reads have returned, instead of beside the
//    next tile's score MFMAs; it then has a whole score phase longer to land
//    (2.3% faster at S = 30720, but 8.5% slower at S = 122880, where fewer
//    tile reads hit L2 and the earlier requests only add to its load);
//  * workgroup order: XCD x (workgroup w runs on XCD w % 8) takes a
//    contiguous range of query blocks, so neighbouring query blocks, which
//    keep many of the same key blocks, share its L2.  On padded grids the
//    range is an eighth of all heads' real blocks (heads differ in their
//    block counts there).  With xcd_per_head = R
//    > 1, R XCDs share each head (each takes 1/R of its query blocks): lists
//    whose lengths vary with the data then load the XCDs evenly (top-p at
//    the Wan shape: the heaviest XCD held 1.59x the mean tiles with whole
//    heads per XCD and 1.07x with R = 4).
struct SoloCfg {
    static constexpr int D = 128, BLK = 64;
    static constexpr int TILE = BLK * D * 2;  // one V tile in LDS
};

// PADT (gather on load): the tilings may pad the grid along T.  Cells of a
// padding frame lie past the head, so their loads read zeros; their keys are
// masked and their rows are not stored.  Blocks past the head's own block
// count (the grid covers the largest) have no tile.
// Real cells of tile t of a grid padded along T: a prefix of the tile (cells
// are T-major inside it), all 64 unless the tile reaches into the padding
__device__ __forceinline__ int padded_tile_cells(const TileGeo& geo, uint32_t T, uint32_t t) {
    uint32_t tt, rem;
    fdivmod(t, geo.f_ntyx, tt, rem);
    const int left = (int)T - (int)(tt * geo.a);
    return left >= (int)geo.a ? 64 : left * (int)(geo.b * geo.c);
}

template <int MODE, bool POS, bool TILED, bool BOUND = false, bool PADT = false, bool EV = true>
__global__ __launch_bounds__(64, 1) void attn_solo_kernel(const AttnParams P, const int32_t* __restrict__ kv_idx,
                                                          const int32_t* __restrict__ kv_cnt,
                                                          const float* __restrict__ knorm) {
    using C = SoloCfg;
    constexpr int D = C::D, BLK = C::BLK;
    static_assert(D * 2 == 256, "k_lds_solo / v_lds_solo assume 256-byte rows");
    // Q (64 rows) and one V tile live in the wave's LDS (32 KB: four waves per CU)
    __shared__ __attribute__((aligned(16))) char klds[C::TILE];
    __shared__ __attribute__((aligned(16))) char vlds[C::TILE];
    const int lane = threadIdx.x;
    const int half_id = lane >> 5, col = lane & 31;

    uint32_t wg = blockIdx.x, bh, I;
    if (MODE == kBlockList && P.row_order != nullptr) {
        const uint32_t r = P.row_order[wg];
        if (r >= P.n_wg) return;
        bh = r / P.nq;
        I = r % P.nq;
    } else if (PADT && P.xcd_remap && P.head_choice != nullptr) {
        // heads differ in their block counts (each its own padded grid): the
        // heads' real blocks are taken in order and XCD x runs the x-th eighth
        // of them, so that every XCD gets the same work
        const uint32_t x = wg & 7u, slot = wg >> 3, n_heads = P.n_wg / P.nq;
        auto blocks_of = [&](uint32_t h) -> uint32_t {
            const uint32_t c = (uint32_t)__builtin_amdgcn_readfirstlane(P.head_choice[h]);
            return P.nbt[c < P.n_tiles ? c : 0u];
        };
        uint32_t total = 0;
        for (uint32_t h = 0; h < n_heads; ++h) total += blocks_of(h);
        const uint32_t lo = (uint32_t)((uint64_t)total * x / 8u), hi = (uint32_t)((uint64_t)total * (x + 1u) / 8u);
        if (lo + slot >= hi) return;
        uint32_t p = lo + slot, h = 0;
        for (uint32_t n = blocks_of(0); p >= n; n = blocks_of(++h)) p -= n;
        bh = h;
        I = p;
    } else if (P.xcd_per_head > 1u) {  // XCD x = u + R g shares heads g, g + 8/R, ... with R - 1 others
        const uint32_t R = P.xcd_per_head, x = wg & 7u, slot = wg >> 3, chunk = P.nq / R;
        bh = x / R + (slot / chunk) * (8u / R);
        I = (x % R) * chunk + slot % chunk;
    } else {
        if (P.xcd_remap) wg = (wg & 7u) * (P.n_wg >> 3) + (wg >> 3);
        bh = wg / P.nq;
        I = wg % P.nq;
    }
    // PADT: a query tile whose real cells (a prefix of the tile) fit in its
    // first 32 rows runs one row tile; the other 32 rows are padding, neither
    // computed nor stored
    auto body = [&](auto nr_tag) {
        constexpr int NR = decltype(nr_tag)::value;
        const size_t head = (size_t)bh * P.S * D;
        const uint32_t head_bytes = P.S * D * 2;
        const __amdgpu_buffer_rsrc_t qr = make_rsrc(P.q + head, head_bytes);
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(P.k + head, head_bytes);
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(P.v + head, head_bytes);
        const int q0 = (int)I * BLK;
        // TILED: the head's tiling, the query tile's T-major origin, and each
        // lane's two cells (32c + col) as T-major offsets from a tile origin
        uint32_t tc = 0;
        if (TILED && P.head_choice != nullptr) {
            tc = (uint32_t)__builtin_amdgcn_readfirstlane(P.head_choice[bh]);
            if (tc >= P.n_tiles) tc = 0;  // out-of-range choices are caught by bsa_validate_indices
        }
        if (PADT && I >= P.nbt[tc]) return;
        const TileGeo& geo = P.geo[tc];
        const uint32_t q_origin = TILED ? tile_origin(I, geo, P.Hg, P.Wg) : (uint32_t)q0;
        int kcell[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) kcell[c] = TILED ? (int)cell_offset(32 * c + col, geo, P.Hg, P.Wg) : 32 * c + col;
        auto tile_soff = [&](int t) -> int {  // byte offset of key tile t's first row
            return TILED ? (int)tile_origin((uint32_t)t, geo, P.Hg, P.Wg) * (D * 2) : t * BLK * (D * 2);
        };
        // PADT: key rows of tile t that are real cells, a prefix of the tile (cells are T-major inside it)
        auto tile_keys = [&](int t) -> int { return PADT ? padded_tile_cells(geo, P.T, (uint32_t)t) : BLK; };

        int n_iter;
        const int32_t* list = nullptr;
        int n_sink_tiles = 0, local_first = 0;
        if (MODE != kWindow) {
            const size_t row = (size_t)bh * P.nq + I;
            n_iter = min(kv_cnt[row], (int)P.max_kept);
            list = kv_idx + row * P.max_kept;
        } else {
            n_sink_tiles = (P.sink + BLK - 1) / BLK;
            const int lo = max(0, q0 - P.half);
            const int hi = min((int)P.S, q0 + BLK - 1 + P.half + 1);  // exclusive
            const int t_lo = lo / BLK, t_hi = (hi - 1) / BLK;
            local_first = max(t_lo, n_sink_tiles);
            n_iter = n_sink_tiles + max(0, t_hi - local_first + 1);
        }
        auto tile_at = [&](int it) -> int {
            if (MODE != kWindow) return __builtin_amdgcn_readfirstlane(list[it]);
            return it < n_sink_tiles ? it : local_first + (it - n_sink_tiles);
        };
        // entry it of the list as a vector value (a buffer load, read one tile ahead)
        const __amdgpu_buffer_rsrc_t lr = make_rsrc(list, MODE != kWindow ? 4u * (uint32_t)max(n_iter, 0) : 0u);
        auto tile_ahead = [&](int it) -> int {
            if (MODE != kWindow) return __builtin_amdgcn_raw_buffer_load_b32(lr, 4 * it, 0, 0);
            return it < n_sink_tiles ? it : local_first + (it - n_sink_tiles);
        };

        // fragments: row (or key) 32*x + col, D cols 16*s + 8*half_id + 0..7;
        // koff[x] is that row's byte offset from its tile's origin
        int koff[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) koff[c] = kcell[c] * (D * 2) + half_id * 16;
        // Q stays in registers as the B operand of both row tiles
        bf16x8 qf[2][D / 16];
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int s = 0; s < D / 16; ++s)
                qf[r][s] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qr, koff[r] + 32 * s, TILED ? (int)q_origin * (D * 2) : q0 * (D * 2), 0));
        // LDS address of K fragment (key half 0, step s); key half 1 is 32 rows on
        int k_addr[D / 16];
#pragma unroll
        for (int s = 0; s < D / 16; ++s) k_addr[s] = k_lds_solo(col, 2 * s + half_id);
        // Row group q (rows 4q..4q+3 of a tile) lies goff[q] bytes from the tile's
        // first row: the same for every lane, so it goes into the DMA's scalar
        // offset and only the lane's place within the group stays in a VGPR.
        // TILED: cells 4q..4q+3 are 4 consecutive T-major tokens (tiles with an x
        // extent that is a multiple of 4), P.voff[tc][q] bytes from the origin.
        int goff[C::TILE / 1024];
#pragma unroll
        for (int q = 0; q < C::TILE / 1024; ++q) goff[q] = TILED ? P.voff[tc][q] : 1024 * q;
        // K tile straight into LDS with the K swizzle: instruction q fills rows
        // 4q..4q+3, lane l physical chunk l % 16 of row 4q + l / 16, which holds
        // logical chunk (l % 16) ^ (row % 16), row % 16 = 4(q % 4) + l / 16
        // row lane / 16 of a DMA row group lies rrow bytes after the group's first row
        const int rrow = TILED ? P.rdelta[tc][lane >> 4] : (lane >> 4) * (D * 2);
        int klane[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) klane[p] = rrow + (((lane & 15) ^ (4 * p + (lane >> 4))) << 4);
        auto dma_k = [&](int soff) {
#pragma unroll
            for (int q = 0; q < C::TILE / 1024; ++q)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (__attribute__((address_space(3))) void*)(klds + 1024 * q), 16,
                                                         klane[q & 3], soff + goff[q], 0, 0);
        };
        // V tile straight into LDS (buffer loads with the LDS destination): wave
        // instruction q fills LDS bytes [1024q, 1024q + 1024), i.e. rows 4q..4q+3,
        // lane l landing on physical chunk l % 16 of row 4q + l / 16, which holds
        // logical chunk (l % 16) ^ 4(row % 4) (the V swizzle); row % 4 = l / 16.
        const int vlane = rrow + (((lane & 15) ^ (4 * (lane >> 4))) << 4);
        auto dma_v = [&](char* buf, int soff, int q_lo, int q_hi) {
#pragma unroll
            for (int q = q_lo; q < q_hi; ++q)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (__attribute__((address_space(3))) void*)(buf + 1024 * q), 16,
                                                         vlane, soff + goff[q], 0, 0);
        };

        f32x16 o[2][D / 32];
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int t = 0; t < D / 32; ++t)
#pragma unroll
                for (int v = 0; v < 16; ++v) o[r][t][v] = 0.f;
        float m_used[2] = {-1e30f, -1e30f}, l_part[2] = {0.f, 0.f};
        const float c_scale = POS ? P.scale_log2 : 1.0f;
        // Key norms given (block lists, positive scale): by Cauchy-Schwarz every
        // score of this query block against key tile J, times scale * log2(e), is
        // at most q_lim * knorm[J], q_lim = the largest |q_row| of the block times
        // scale * log2(e).  When that stays within kSkipSlack of the smallest
        // running max of the block's rows, m_min, no softmax weight of the tile
        // can pass 2^kSkipSlack and the tile skips the max.  The test is
        // knorm[J] <= kn_lim = (m_min + kSkipSlack) / q_lim, on scalars; kn_lim
        // only moves when a rescale moves the running max.
        constexpr bool bounded = BOUND && MODE == kBlockList && POS;
        const float* knorm_head = bounded ? knorm + (size_t)bh * P.nq : nullptr;
        float q_lim = 0.f, kn_lim = -__builtin_inff(), kn_cur = 0.f;
        if (bounded) {
            float n2max = 0.f;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                float n2 = 0.f;
#pragma unroll
                for (int s = 0; s < D / 16; ++s)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bf16x2 two = {qf[r][s][2 * e], qf[r][s][2 * e + 1]};
                        n2 = __builtin_amdgcn_fdot2_f32_bf16(two, two, n2, false);
                    }
                // lanes l and l ^ 32 hold the two halves of row 32r + l % 32
                const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(n2), __float_as_uint(n2), false, false);
                n2max = fmaxf(n2max, __uint_as_float(pr[0]) + __uint_as_float(pr[1]));
            }
#pragma unroll
            for (int off = 1; off < 32; off <<= 1) n2max = fmaxf(n2max, __shfl_xor(n2max, off));
            q_lim = sqrtf(__uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(n2max)))) * c_scale;
        }

        const int g16 = lane >> 4, r16 = lane & 15;
        const int v_key0 = 4 * (g16 >> 1) + (r16 >> 2);
        const int v_col0 = 16 * (g16 & 1) + 4 * (r16 & 3);
        int v_addr[D / 32];
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
            const int colv = 32 * t + v_col0;
            v_addr[t] = v_lds_solo(v_key0, colv >> 3) + (colv & 7) * 2;
        }

        // label rule: this lane's two row labels, whether the whole query block
        // shares one label, and the key labels of the next tile (lane l holds
        // key l), fetched with that tile's K
        int qlab[2] = {0, 0}, q_uni = 0, klab = 0, klab_next = 0;
        bool q_uniform = true;
        const int32_t* labs = nullptr;
        if (MODE == kLabels) {
            labs = P.labels + (size_t)bh * P.label_stride;
            qlab[0] = labs[q0 + col];
            qlab[1] = labs[q0 + 32 + col];
            q_uni = __builtin_amdgcn_readfirstlane(qlab[0]);
            q_uniform = __ballot((qlab[0] != q_uni) | (qlab[1] != q_uni)) == 0;
        }

        int soff_cur = 0, v_nxt = 0, kval_cur = BLK;
        if (n_iter > 0) {
            const int t0 = tile_at(0);
            if (bounded) kn_cur = knorm_head[t0];
            soff_cur = tile_soff(t0);
            kval_cur = tile_keys(t0);
            dma_k(soff_cur);
            if (EV) dma_v(vlds, soff_cur, 0, C::TILE / 1024);
            if (MODE == kLabels) klab_next = labs[t0 * BLK + lane];
            v_nxt = tile_ahead(min(1, n_iter - 1));
        }
        __builtin_amdgcn_s_waitcnt(0);

        for (int it = 0; it < n_iter; ++it) {
            const int nxt_tile = __builtin_amdgcn_readfirstlane(v_nxt);
            const int nxt = nxt_tile * BLK;
            const float kn_nxt = bounded ? knorm_head[nxt_tile] : 0.f;
            // this tile's K has landed in LDS (only its V (EV) was issued later) and
            // the previous tile's V reads have completed
            __builtin_amdgcn_s_waitcnt(EV ? kVm16Lgkm0 : 0);
            // Q's fragments are only ever MFMA B operands in the loop: an empty
            // asm with an accumulation-register constraint keeps them in AGPRs,
            // which the MFMAs read directly (no per-tile copies to VGPRs)
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int s = 0; s < D / 16; ++s) asm volatile("" : "+a"(qf[r][s]));

            // PADT: a key tile whose real keys (a prefix) fit in its first 32 rows
            // skips key half 1: its scores stay 0 and are masked to -inf below,
            // and the P V groups of keys 32..63 are not run
            const bool khalf = PADT && __builtin_amdgcn_readfirstlane(kval_cur) <= 32;

            // S^T of (key half c, row tile r) = K_c Q_r^T: four independent chains
            f32x16 sacc[2][2];
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int r = 0; r < NR; ++r) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) sacc[c][r][v] = 0.f;
                }
            // K fragments of the two key halves, read two steps ahead (ring of three)
            bf16x8 kfa[3], kfb[3];
            auto read_k = [&](int s) {
                kfa[s % 3] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(klds + k_addr[s]));
                kfb[s % 3] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(klds + k_addr[s] + 32 * (D * 2)));
            };
            read_k(0);
            read_k(1);
            // (one MFMA per fenced region, with one V DMA or the K reads of step s+2
            // beside it)
#pragma unroll
            for (int s = 0; s < D / 16; ++s) {
                const bf16x8 ka = kfa[s % 3], kb = kfb[s % 3];
                sacc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[0][s], sacc[0][0], 0, 0, 0);
                if (!EV) dma_v(vlds, soff_cur, 2 * s, NR == 2 ? 2 * s + 1 : 2 * s + 2);
                __builtin_amdgcn_sched_barrier(0);
                if (NR == 2) {
                    sacc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[1][s], sacc[0][1], 0, 0, 0);
                    if (!EV) dma_v(vlds, soff_cur, 2 * s + 1, 2 * s + 2);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (!khalf) sacc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, qf[0][s], sacc[1][0], 0, 0, 0);
                if (s + 2 < D / 16) read_k(s + 2);
                __builtin_amdgcn_sched_barrier(0);
                if (NR == 2 && !khalf) {
                    sacc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, qf[1][s], sacc[1][1], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // this tile's K is read: the next tile's K goes into its LDS (the last tile
            // again past the end), with the list entry of the tile after it
            if (MODE == kLabels) klab = klab_next;
            v_nxt = tile_ahead(min(it + 2, n_iter - 1));
            const int soff_nxt = tile_soff(nxt_tile);
            const int kval_nxt = tile_keys(nxt_tile);
            __builtin_amdgcn_s_waitcnt(kLgkmcnt0);  // this tile's K reads are complete
            dma_k(soff_nxt);
            if (MODE == kLabels) klab_next = labs[nxt + lane];
            __builtin_amdgcn_sched_barrier(0);

            // softmax of both row tiles (32 values of one row per lane and tile)
            if (!POS) {
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int r = 0; r < NR; ++r)
#pragma unroll
                        for (int v = 0; v < 16; ++v) sacc[c][r][v] *= P.scale_log2;
            }
            if (PADT && kval_cur < BLK) {  // padding keys of a tile at the end of the padded frames
                const float neg_inf = -__builtin_inff();
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int r = 0; r < NR; ++r)
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int j = 32 * c + 4 * half_id + 8 * (v / 4) + (v % 4);
                            sacc[c][r][v] = j < kval_cur ? sacc[c][r][v] : neg_inf;
                        }
            }
            if (MODE == kWindow) {
                const int j0 = tile_at(it) * BLK;
                const bool full = (j0 + BLK - 1 < P.sink) ||
                                  (q0 + BLK - 1 - j0 <= P.half && j0 + BLK - 1 - q0 <= P.half && j0 + BLK <= (int)P.S);
                if (!full) {
                    const float neg_inf = -__builtin_inff();
                    if (j0 >= P.sink && j0 + BLK <= (int)P.S) {
                        // a tile past the sinks and inside the sequence: only the band
                        // |row - key| <= half.  With base = row - (first key of this
                        // lane's share), key offset k = 8(v / 4) + v % 4 is visible when
                        // base - half <= k <= base + half: two compares against a constant
#pragma unroll
                        for (int c = 0; c < 2; ++c)
#pragma unroll
                            for (int r = 0; r < NR; ++r) {
                                const int base = q0 + 32 * r + col - (j0 + 32 * c + 4 * half_id);
                                const int lo = base - P.half, hi = base + P.half;
#pragma unroll
                                for (int v = 0; v < 16; ++v) {
                                    const int kk = 8 * (v / 4) + (v % 4);
                                    const bool vis = (kk >= lo) & (kk <= hi);
                                    sacc[c][r][v] = vis ? sacc[c][r][v] : neg_inf;
                                }
                            }
                    } else {
#pragma unroll
                        for (int c = 0; c < 2; ++c)
#pragma unroll
                            for (int r = 0; r < NR; ++r) {
                                const int my_row = q0 + 32 * r + col;
#pragma unroll
                                for (int v = 0; v < 16; ++v) {
                                    const int j = j0 + 32 * c + 4 * half_id + 8 * (v / 4) + (v % 4);
                                    const int d = my_row - j;
                                    const bool vis =
                                        (j < (int)P.S) & (((d <= P.half) & (-d <= P.half)) | (j < P.sink));
                                    sacc[c][r][v] = vis ? sacc[c][r][v] : neg_inf;
                                }
                            }
                    }
                }
            }
            if (MODE == kLabels) {
                // a tile whose keys all carry the query block's single label needs no mask
                if (!q_uniform || __ballot(klab != q_uni) != 0) {
                    const float neg_inf = -__builtin_inff();
#pragma unroll
                    for (int c = 0; c < 2; ++c)
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int kl = __shfl(klab, 32 * c + 4 * half_id + 8 * (v / 4) + (v % 4));
#pragma unroll
                            for (int r = 0; r < NR; ++r) sacc[c][r][v] = kl == qlab[r] ? sacc[c][r][v] : neg_inf;
                        }
                }
            }
            // (the ballot keeps the test in a VGPR compare; as a plain scalar branch
            // the compiler allocates the loop's registers far worse)
            const bool skip = bounded && __ballot(kn_cur <= kn_lim) != 0;
            kn_cur = kn_nxt;
            if (__builtin_expect(!skip, !bounded)) {
                float mloc[2];
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    float smax = fmaxf(sacc[0][r][0], sacc[1][r][0]);
#pragma unroll
                    for (int v = 1; v < 16; ++v) smax = fmaxf(fmaxf(smax, sacc[0][r][v]), sacc[1][r][v]);
                    const auto pr =
                        __builtin_amdgcn_permlane32_swap(__float_as_uint(smax), __float_as_uint(smax), false, false);
                    mloc[r] = fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1])) * c_scale;
                }
                const bool grow0 = mloc[0] > m_used[0] + kRescaleSlack;
                const bool grow1 = NR == 2 && mloc[NR - 1] > m_used[NR - 1] + kRescaleSlack;
                if (__ballot(grow0 | grow1)) {
#pragma unroll
                    for (int r = 0; r < NR; ++r) {
                        const bool grow = r == 0 ? grow0 : grow1;
                        const float m_new = grow ? mloc[r] : m_used[r];
                        const float alpha = __builtin_amdgcn_exp2f(m_used[r] - m_new);
                        m_used[r] = m_new;
                        l_part[r] *= alpha;
#pragma unroll
                        for (int t = 0; t < D / 32; ++t)
#pragma unroll
                            for (int v = 0; v < 16; ++v) o[r][t][v] *= alpha;
                    }
                    if (bounded) {
                        float mm = fminf(m_used[0], m_used[NR - 1]);
#pragma unroll
                        for (int off = 1; off < 64; off <<= 1) mm = fminf(mm, __shfl_xor(mm, off));
                        const float m_min = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(mm)));
                        kn_lim = (m_min + kSkipSlack) / q_lim;
                    }
                }
            }
            // P as bf16 B operands, one 16-key group m at a time (pb[r][m] covers keys
            // 16m..16m+15); group m+1's exps and V^T reads are issued beside the
            // MFMAs of group m
            bf16x8 pb[2][4];
            float psum[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
            // piece j (0..3) of group m for row tile r: accumulator values
            // 8(m % 2) + 2j and + 1 of key half m / 2, i.e. two of this lane's share
            // of keys 16m..16m+15
            auto p_piece = [&](int m, int r, int j) {
                const int c = m / 2, v = 8 * (m % 2) + 2 * j;
                const float neg_m = -m_used[r];
                const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[c][r][v], c_scale, neg_m));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[c][r][v + 1], c_scale, neg_m));
                const bf16x2 two = {(__bf16)p0, (__bf16)p1};
                psum[r][m % 2] = __builtin_amdgcn_fdot2_f32_bf16(two, kOnes2, psum[r][m % 2], false);
                pb[r][m][v % 8] = two[0];
                pb[r][m][v % 8 + 1] = two[1];
            };
            // V^T fragment t of group m (keys 16m..16m+15) in two transposing reads of
            // 8 keys each; vfr[m % 2] holds a group's four fragments
            bf16x8 vfr[2][D / 32];
            s16x4 vlo[D / 32];
            auto v_half = [&](int m, int t, int h) {
                const char* va = vlds + v_addr[t] + (16 * m + 8 * h) * (D * 2);
                const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)va);
                if (h == 0) {
                    vlo[t] = x;
                } else {
                    const s16x4 a8[2] = {vlo[t], x};
                    vfr[m % 2][t] = __builtin_bit_cast(bf16x8, a8);
                }
            };
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j) p_piece(0, r, j);
            // O^T += V^T P^T once this tile's V has landed: only the next tile's 16 K
            // loads and (block lists) its list entry were issued after it
            __builtin_amdgcn_s_waitcnt(MODE == kWindow ? kVmcnt16 : waitcnt_vm(17));
#pragma unroll
            for (int t = 0; t < D / 32; ++t) {
                v_half(0, t, 0);
                v_half(0, t, 1);
            }
            __builtin_amdgcn_sched_barrier(0);
            // (one MFMA per fenced region; beside each, the share of group m+1 that
            // falls to it: with two row tiles two exps of one row tile and half of
            // one V^T fragment, with one row tile two exps and a whole fragment; EV:
            // beside the last group's MFMAs, the next tile's V DMA instructions in
            // equal shares, the last tile's again past the end)
            constexpr int kPvPerGroup = NR * (D / 32), kDmaPer = (C::TILE / 1024) / kPvPerGroup;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                if (m >= 2 && khalf) continue;  // keys 32..63 are all padding
                if (EV && m == 3) {  // every V^T read of this tile has returned
                    __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int i = 0; i < kPvPerGroup; ++i) {
                    const int t = NR == 2 ? i / 2 : i, r = NR == 2 ? i % 2 : 0;
                    o[r][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[m % 2][t], pb[r][m], o[r][t], 0, 0, 0);
                    if (m + 1 < 4) {
                        if (m + 1 < 2 || !khalf) {
                            if (NR == 2) {
                                p_piece(m + 1, i / 4, i % 4);
                                v_half(m + 1, t, i % 2);
                            } else {
                                p_piece(m + 1, 0, i);
                                v_half(m + 1, t, 0);
                                v_half(m + 1, t, 1);
                            }
                        }
                    } else if (EV) {
                        dma_v(vlds, soff_nxt, kDmaPer * i, kDmaPer * (i + 1));
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if (EV && khalf) {  // the next tile's V, once this tile's V^T reads (groups 0, 1) have returned
                __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
                __builtin_amdgcn_sched_barrier(0);
                dma_v(vlds, soff_nxt, 0, C::TILE / 1024);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int r = 0; r < NR; ++r) l_part[r] += psum[r][0] + psum[r][1];
            soff_cur = soff_nxt;
            kval_cur = kval_nxt;
        }

        // ---- write out (each lane pair holds one row; their partial sums add up)
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_part[r]), __float_as_uint(l_part[r]), false,
                                                             false);
            const float l = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
            const float inv = l > 0.f ? 1.0f / l : 0.f;  // a row that saw no key is written as zeros
            const int my_row = TILED ? (int)q_origin + kcell[r] : q0 + 32 * r + col;
            if (my_row >= (int)P.S) continue;
            uint16_t* orow = P.out + head + (size_t)my_row * D;
#pragma unroll
            for (int t = 0; t < D / 32; ++t)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                    bf16x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[r][t][4 * g + e] * inv);
                    *reinterpret_cast<bf16x4*>(orow + 32 * t + 8 * g + 4 * half_id) = w;
                }
        }
        // EV: the V DMA issued past the last tile lands before the wave ends
        if (EV) __builtin_amdgcn_s_waitcnt(0);
    };
    if (PADT) {
        uint32_t tc = 0;
        if (P.head_choice != nullptr) {
            tc = (uint32_t)__builtin_amdgcn_readfirstlane(P.head_choice[bh]);
            if (tc >= P.n_tiles) tc = 0;
        }
        if (I < P.nbt[tc] && padded_tile_cells(P.geo[tc], P.T, I) <= 32) {
            body(std::integral_constant<int, 1>{});
            return;
        }
    }
    body(std::integral_constant<int, 2>{});
}

// ----------------------------------------------------------------- scalar ---
// One thread per query row, fp32 math, exact online softmax.  For fp32
// tensors and shapes the MFMA kernel does not cover.

struct ScalarParams {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    uint32_t S, BH, block;
    float scale_log2;
    const int32_t* kv_idx;
    const int32_t* kv_cnt;
    uint32_t max_kept, nq;
    int32_t half, sink;
    const int32_t* labels;
    uint64_t label_stride;
};

template <bool BF16>
__device__ __forceinline__ float ld(const void* base, size_t i) {
    if (BF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
    return static_cast<const float*>(base)[i];
}

template <int D, bool BF16, int MODE>
__global__ __launch_bounds__(64) void attn_scalar_kernel(const ScalarParams P) {
    const uint64_t gid = (uint64_t)blockIdx.x * 64 + threadIdx.x;
    if (gid >= (uint64_t)P.BH * P.S) return;
    const uint32_t bh = (uint32_t)(gid / P.S), i = (uint32_t)(gid % P.S);
    const size_t head = (size_t)bh * P.S * D;
    float qv[D], acc[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        qv[d] = ld<BF16>(P.q, head + (size_t)i * D + d);
        acc[d] = 0.f;
    }
    float m = -__builtin_inff(), l = 0.f;
    auto visit = [&](uint32_t j) {
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) s = fmaf(qv[d], ld<BF16>(P.k, head + (size_t)j * D + d), s);
        s *= P.scale_log2;
        const float mn = fmaxf(m, s);
        const float a = exp2f(m - mn), p = exp2f(s - mn);
        l = l * a + p;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = fmaf(p, ld<BF16>(P.v, head + (size_t)j * D + d), acc[d] * a);
        m = mn;
    };
    if (MODE != kWindow) {
        const size_t row = (size_t)bh * P.nq + i / P.block;
        const int cnt = min(P.kv_cnt[row], (int)P.max_kept);
        const int32_t* labs = MODE == kLabels ? P.labels + (size_t)bh * P.label_stride : nullptr;
        const int32_t my_label = MODE == kLabels ? labs[i] : 0;
        for (int t = 0; t < cnt; ++t) {
            const uint32_t J = (uint32_t)P.kv_idx[row * P.max_kept + t];
            if (J >= P.nq) continue;  // invalid lists are reported by bsa_validate_block_list
            for (uint32_t j = J * P.block; j < (J + 1) * P.block; ++j)
                if (MODE != kLabels || labs[j] == my_label) visit(j);
        }
    } else {
        const uint32_t sink = (uint32_t)P.sink;
        for (uint32_t j = 0; j < sink; ++j) visit(j);
        const int64_t lo = max((int64_t)sink, (int64_t)i - P.half);
        const int64_t hi = min((int64_t)P.S - 1, (int64_t)i + P.half);
        for (int64_t j = lo; j <= hi; ++j) visit((uint32_t)j);
    }
    const float inv = l > 0.f ? 1.0f / l : 0.f;  // a row that saw no key is written as zeros
    for (int d = 0; d < D; ++d) {
        const float r = acc[d] * inv;
        if (BF16)
            static_cast<uint16_t*>(P.out)[head + (size_t)i * D + d] = f32_to_bf16(r);
        else
            static_cast<float*>(P.out)[head + (size_t)i * D + d] = r;
    }
}

template <int MODE>
int launch_scalar(const ScalarParams& P, int dtype, int64_t D, hipStream_t st, const char* name) {
    const uint64_t rows = (uint64_t)P.BH * P.S;
    const unsigned blocks = (unsigned)((rows + 63) / 64);
    const bool bf = dtype == BSA_BF16;
#define BSA_SC(DD) \
    (bf ? attn_scalar_kernel<DD, true, MODE><<<blocks, 64, 0, st>>>(P) : attn_scalar_kernel<DD, false, MODE><<<blocks, 64, 0, st>>>(P))
    switch (D) {
        case 16: BSA_SC(16); break;
        case 32: BSA_SC(32); break;
        case 64: BSA_SC(64); break;
        case 128: BSA_SC(128); break;
        default: BSA_FAIL(BSA_ERR_UNSUPPORTED, "%s: D=%lld unsupported (16, 32, 64, 128)", name, (long long)D);
    }
#undef BSA_SC
    return check_launch(name);
}

uint32_t grid_of(const AttnParams& P) { return P.grid != 0 ? P.grid : P.n_wg; }

template <int MODE, bool TILED, bool PADT, bool EV>
void launch_solo_ev(const AttnParams& P, hipStream_t st) {
    if (MODE == kBlockList && P.scale_log2 > 0.f && P.knorm != nullptr)
        attn_solo_kernel<MODE, true, TILED, true, PADT, EV><<<grid_of(P), 64, 0, st>>>(P, P.kv_idx, P.kv_cnt, P.knorm);
    else if (P.scale_log2 > 0.f)
        attn_solo_kernel<MODE, true, TILED, false, PADT, EV><<<grid_of(P), 64, 0, st>>>(P, P.kv_idx, P.kv_cnt, nullptr);
    else
        attn_solo_kernel<MODE, false, TILED, false, PADT, EV><<<grid_of(P), 64, 0, st>>>(P, P.kv_idx, P.kv_cnt, nullptr);
}

// The early V DMA is used unless a head's K and V exceed kEarlyVBytes (block
// lists; the other modes always use it).
constexpr uint64_t kEarlyVBytes = 32ull << 20;

template <int MODE, bool TILED = false, bool PADT = false>
void launch_solo(const AttnParams& P, hipStream_t st) {
    if constexpr (MODE == kBlockList && !PADT) {
        if ((uint64_t)P.S * (SoloCfg::D * 4) > kEarlyVBytes) {
            launch_solo_ev<MODE, TILED, PADT, false>(P, st);
            return;
        }
    }
    launch_solo_ev<MODE, TILED, PADT, true>(P, st);
}

// Workgroup order of the single-wave kernel: contiguous ranges of (head,
// query block) per XCD, or, for lists that may hold every block (their
// lengths vary with the data), each head shared by 4 XCDs.
// A caller's launch order: row_order_len workgroups, workgroup w running row
// row_order[w] (empty when that is not a row).
int set_row_order(AttnParams& P, const uint32_t* row_order, int64_t row_order_len, const char* name) {
    if (row_order == nullptr) return BSA_OK;
    BSA_REQUIRE(row_order_len >= 1 && row_order_len < ((int64_t)1 << 31), "%s: row_order_len=%lld must be in [1, 2^31)",
                name, (long long)row_order_len);
    P.row_order = row_order;
    P.grid = (uint32_t)row_order_len;
    return BSA_OK;
}

void set_order(AttnParams& P, int64_t BH, int max_kept) {
    P.xcd_remap = (P.n_wg % 8 == 0) ? 1u : 0u;
    P.xcd_per_head = 1;
    constexpr uint32_t R = 4;
    if (P.xcd_remap && (int64_t)max_kept >= (int64_t)P.nq && BH % (8 / R) == 0 && P.nq % R == 0)
        P.xcd_per_head = R;
}

template <int D, int BLK, int MODE>
void launch_mfma(const AttnParams& P, hipStream_t st) {
    if (P.scale_log2 > 0.f)
        attn_mfma_kernel<D, BLK, MODE, true><<<grid_of(P), Cfg<D, BLK>::NT, 0, st>>>(P, P.kv_idx, P.kv_cnt);
    else
        attn_mfma_kernel<D, BLK, MODE, false><<<grid_of(P), Cfg<D, BLK>::NT, 0, st>>>(P, P.kv_idx, P.kv_cnt);
}

int common_checks(const void* q, const void* k, const void* v, void* out, int dtype, int64_t B, int64_t H, int64_t S,
                  int64_t D, const char* name) {
    BSA_REQUIRE(elem_size(dtype) != 0, "%s: unknown dtype %d", name, dtype);
    BSA_REQUIRE(q && k && v && out, "%s: NULL tensor", name);
    BSA_REQUIRE(B >= 1 && H >= 1, "%s: B and H must be >= 1", name);
    BSA_REQUIRE(S >= 1, "%s: sequence length must be > 0", name);
    BSA_REQUIRE(D >= 1, "%s: head dim must be > 0", name);
    BSA_REQUIRE(S < ((int64_t)1 << 30), "%s: S too large", name);
    BSA_REQUIRE(S * D * elem_size(dtype) < ((int64_t)1 << 31), "%s: one head must stay under 2 GiB", name);
    BSA_REQUIRE(B * H * S * D < ((int64_t)1 << 40), "%s: tensor too large", name);
    BSA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(out), "%s: tensors must be 16-byte aligned",
                name);
    return BSA_OK;
}

float resolve_scale_log2(float scale, int64_t D) {
    const double s = std::isnan(scale) ? 1.0 / std::sqrt((double)D) : (double)scale;
    return (float)(s * 1.4426950408889634);
}

}  // namespace
}  // namespace bsa

using namespace bsa;

extern "C" int bsa_block_sparse_attention(const void* q, const void* k, const void* v, void* out, int dtype, int64_t B,
                                          int64_t H, int64_t S, int64_t D, int block, const int32_t* kv_idx,
                                          const int32_t* kv_cnt, int max_kept, float scale,
                                          const float* key_norms_or_null, const uint32_t* row_order_or_null,
                                          int64_t row_order_len, bsa_stream_t stream) {
    clear_error();
    const char* name = "bsa_block_sparse_attention";
    int rc = common_checks(q, k, v, out, dtype, B, H, S, D, name);
    if (rc) return rc;
    BSA_REQUIRE(kv_idx && kv_cnt, "%s: NULL block list", name);
    BSA_REQUIRE(block >= 1 && S % block == 0, "%s: block %d must divide S=%lld", name, block, (long long)S);
    BSA_REQUIRE(max_kept >= 1, "%s: max_kept must be >= 1", name);
    hipStream_t st = (hipStream_t)stream;
    const int64_t nq = S / block;
    const float sl2 = resolve_scale_log2(scale, D);
    const bool mfma = dtype == BSA_BF16 && (D == 64 || D == 128) && (block == 32 || block == 64);
    if (mfma) {
        const int64_t nwg = B * H * nq;
        BSA_REQUIRE(nwg < ((int64_t)1 << 31), "%s: too many blocks", name);
        AttnParams P{};
        P.q = static_cast<const uint16_t*>(q);
        P.k = static_cast<const uint16_t*>(k);
        P.v = static_cast<const uint16_t*>(v);
        P.out = static_cast<uint16_t*>(out);
        P.S = (uint32_t)S;
        P.nq = (uint32_t)nq;
        P.n_wg = (uint32_t)nwg;
        P.xcd_remap = (nwg % 8 == 0) ? 1u : 0u;
        P.scale_log2 = sl2;
        P.kv_idx = kv_idx;
        P.kv_cnt = kv_cnt;
        P.max_kept = (uint32_t)max_kept;
        P.knorm = key_norms_or_null;
        rc = set_row_order(P, row_order_or_null, row_order_len, name);
        if (rc) return rc;
        set_order(P, B * H, max_kept);
        if (D == 128 && block == 64) launch_solo<kBlockList>(P, st);
        else if (D == 128 && block == 32) launch_mfma<128, 32, kBlockList>(P, st);
        else if (D == 64 && block == 64) launch_mfma<64, 64, kBlockList>(P, st);
        else launch_mfma<64, 32, kBlockList>(P, st);
        return check_launch(name);
    }
    ScalarParams P{};
    P.q = q;
    P.k = k;
    P.v = v;
    P.out = out;
    P.S = (uint32_t)S;
    P.BH = (uint32_t)(B * H);
    P.block = (uint32_t)block;
    P.scale_log2 = sl2;
    P.kv_idx = kv_idx;
    P.kv_cnt = kv_cnt;
    P.max_kept = (uint32_t)max_kept;
    P.nq = (uint32_t)nq;
    return launch_scalar<kBlockList>(P, dtype, D, st, name);
}

extern "C" int bsa_windowed_attention(const void* q, const void* k, const void* v, void* out, int dtype, int64_t B,
                                      int64_t H, int64_t S, int64_t D, int window, int sink, float scale, int chunk,
                                      bsa_stream_t stream) {
    clear_error();
    const char* name = "bsa_windowed_attention";
    int rc = common_checks(q, k, v, out, dtype, B, H, S, D, name);
    if (rc) return rc;
    BSA_REQUIRE(window >= 1, "%s: window must be >= 1, got %d", name, window);
    BSA_REQUIRE(sink >= 0, "%s: sink must be >= 0, got %d", name, sink);
    BSA_REQUIRE(sink <= S, "%s: sink (%d) cannot exceed the sequence length (%lld)", name, sink, (long long)S);
    BSA_REQUIRE(chunk >= 0, "%s: chunk must be >= 1 (or 0 for the default), got %d", name, chunk);
    hipStream_t st = (hipStream_t)stream;
    const int32_t half = window / 2;
    const float sl2 = resolve_scale_log2(scale, D);
    const bool mfma = dtype == BSA_BF16 && (D == 64 || D == 128);
    if (mfma) {
        constexpr int BLK = 64;
        const int64_t nq = (S + BLK - 1) / BLK;
        const int64_t nwg = B * H * nq;
        BSA_REQUIRE(nwg < ((int64_t)1 << 31), "%s: too many blocks", name);
        AttnParams P{};
        P.q = static_cast<const uint16_t*>(q);
        P.k = static_cast<const uint16_t*>(k);
        P.v = static_cast<const uint16_t*>(v);
        P.out = static_cast<uint16_t*>(out);
        P.S = (uint32_t)S;
        P.nq = (uint32_t)nq;
        P.n_wg = (uint32_t)nwg;
        P.xcd_remap = (nwg % 8 == 0) ? 1u : 0u;
        P.scale_log2 = sl2;
        P.half = half;
        P.sink = sink;
        if (D == 128) launch_solo<kWindow>(P, st);
        else launch_mfma<64, BLK, kWindow>(P, st);
        return check_launch(name);
    }
    ScalarParams P{};
    P.q = q;
    P.k = k;
    P.v = v;
    P.out = out;
    P.S = (uint32_t)S;
    P.BH = (uint32_t)(B * H);
    P.scale_log2 = sl2;
    P.half = half;
    P.sink = sink;
    return launch_scalar<kWindow>(P, dtype, D, st, name);
}

extern "C" int bsa_block_sparse_attention_labels(const void* q, const void* k, const void* v, void* out, int dtype,
                                                 int64_t B, int64_t H, int64_t S, int64_t D, int block,
                                                 const int32_t* kv_idx, const int32_t* kv_cnt, int max_kept,
                                                 const int32_t* labels, int64_t label_head_stride, float scale,
                                                 bsa_stream_t stream) {
    clear_error();
    const char* name = "bsa_block_sparse_attention_labels";
    int rc = common_checks(q, k, v, out, dtype, B, H, S, D, name);
    if (rc) return rc;
    BSA_REQUIRE(kv_idx && kv_cnt && labels, "%s: NULL block list or labels", name);
    BSA_REQUIRE(block >= 1 && S % block == 0, "%s: block %d must divide S=%lld", name, block, (long long)S);
    BSA_REQUIRE(max_kept >= 1, "%s: max_kept must be >= 1", name);
    BSA_REQUIRE(label_head_stride == 0 || label_head_stride >= S, "%s: label_head_stride must be 0 or >= S", name);
    hipStream_t st = (hipStream_t)stream;
    const int64_t nq = S / block;
    const float sl2 = resolve_scale_log2(scale, D);
    if (dtype == BSA_BF16 && D == 128 && block == 64) {
        const int64_t nwg = B * H * nq;
        BSA_REQUIRE(nwg < ((int64_t)1 << 31), "%s: too many blocks", name);
        AttnParams P{};
        P.q = static_cast<const uint16_t*>(q);
        P.k = static_cast<const uint16_t*>(k);
        P.v = static_cast<const uint16_t*>(v);
        P.out = static_cast<uint16_t*>(out);
        P.S = (uint32_t)S;
        P.nq = (uint32_t)nq;
        P.n_wg = (uint32_t)nwg;
        P.xcd_remap = (nwg % 8 == 0) ? 1u : 0u;
        P.scale_log2 = sl2;
        P.kv_idx = kv_idx;
        P.kv_cnt = kv_cnt;
        P.max_kept = (uint32_t)max_kept;
        P.labels = labels;
        P.label_stride = (uint64_t)label_head_stride;
        set_order(P, B * H, max_kept);
        launch_solo<kLabels>(P, st);
        return check_launch(name);
    }
    ScalarParams P{};
    P.q = q;
    P.k = k;
    P.v = v;
    P.out = out;
    P.S = (uint32_t)S;
    P.BH = (uint32_t)(B * H);
    P.block = (uint32_t)block;
    P.scale_log2 = sl2;
    P.kv_idx = kv_idx;
    P.kv_cnt = kv_cnt;
    P.max_kept = (uint32_t)max_kept;
    P.nq = (uint32_t)nq;
    P.labels = labels;
    P.label_stride = (uint64_t)label_head_stride;
    return launch_scalar<kLabels>(P, dtype, D, st, name);
}

namespace bsa {
namespace {

// Cell offsets of tiling i for the gather-on-load kernel: the T-major offset
// of each DMA row group (cells 4q..4q+3) from the tile origin, and of a
// group's four cells from its first.  A tiling qualifies when it has 64
// cells and every group has the same four offsets (x extent a multiple of 4,
// or smaller extents whose cells still pair up evenly, e.g. (16, 2, 2)).
int fill_tile_rows(AttnParams& P, int i, int Hg, int Wg, int a, int b, int c, int64_t D, const char* name) {
    if (a * b * c != 64)
        BSA_FAIL(BSA_ERR_UNSUPPORTED, "%s: tiles of 64 tokens only (tile %d is %dx%dx%d)", name, i, a, b, c);
    auto off = [&](int cell) -> int64_t {
        const int rt = cell / (b * c), rem = cell % (b * c), ry = rem / c, rx = rem % c;
        return ((int64_t)rt * Hg + ry) * Wg + rx;
    };
    for (int q = 0; q < 16; ++q) {
        for (int j = 0; j < 4; ++j)
            if (off(4 * q + j) - off(4 * q) != off(j) - off(0))
                BSA_FAIL(BSA_ERR_UNSUPPORTED,
                         "%s: tile %d (%dx%dx%d): its cells, taken four at a time, do not share one row pattern",
                         name, i, a, b, c);
        P.voff[i][q] = (int32_t)(off(4 * q) * D * 2);
    }
    for (int j = 0; j < 4; ++j) P.rdelta[i][j] = (int32_t)((off(j) - off(0)) * D * 2);
    return BSA_OK;
}

int tiled_attention(const void* q, const void* k, const void* v, void* out, int dtype, int64_t B, int64_t H, int T,
                    int Hg, int Wg, int64_t D, const int32_t* tiles_host, int n_tiles, const int32_t* head_choice,
                    const int32_t* kv_idx, const int32_t* kv_cnt, int max_kept, float scale, const float* key_norms,
                    const uint32_t* row_order, int64_t row_order_len, bool pad, bsa_stream_t stream,
                    const char* name) {
    BSA_REQUIRE(T > 0 && Hg > 0 && Wg > 0, "%s: grid must be positive", name);
    const int64_t S = (int64_t)T * Hg * Wg;
    int rc = common_checks(q, k, v, out, dtype, B, H, S, D, name);
    if (rc) return rc;
    rc = pad ? check_tiles_padded(T, Hg, Wg, tiles_host, n_tiles) : check_tiles(T, Hg, Wg, tiles_host, n_tiles);
    if (rc) return rc;
    BSA_REQUIRE(kv_idx && kv_cnt, "%s: NULL block list", name);
    BSA_REQUIRE(max_kept >= 1, "%s: max_kept must be >= 1", name);
    if (!(dtype == BSA_BF16 && D == 128))
        BSA_FAIL(BSA_ERR_UNSUPPORTED, "%s: bf16 with D = 128 only (permute and use bsa_block_sparse_attention)",
                 name);
    AttnParams P{};
    int64_t nq = 0, longest = S;
    for (int i = 0; i < BSA_MAX_TILINGS; ++i) {
        const int j = i < n_tiles ? i : 0;
        const int a = tiles_host[3 * j], b = tiles_host[3 * j + 1], c = tiles_host[3 * j + 2];
        if (pad && (Hg % b != 0 || Wg % c != 0))
            BSA_FAIL(BSA_ERR_UNSUPPORTED, "%s: padding along T only (tile %d is %dx%dx%d on a %dx%dx%d grid)", name,
                     j, a, b, c, T, Hg, Wg);
        rc = fill_tile_rows(P, i, Hg, Wg, a, b, c, D, name);
        if (rc) return rc;
        P.geo[i] = pad ? make_geo_padded(Hg, Wg, a, b, c) : make_geo(Hg, Wg, a, b, c);
        const int64_t len = padded_length(T, Hg, Wg, a, b, c);
        P.nbt[i] = (uint32_t)(len / 64);
        nq = std::max<int64_t>(nq, len / 64);
        longest = std::max<int64_t>(longest, len);
    }
    BSA_REQUIRE(longest * D * 2 < ((int64_t)1 << 31), "%s: the padded head must stay under 2 GiB", name);
    const int64_t nwg = B * H * nq;
    BSA_REQUIRE(nwg < ((int64_t)1 << 31), "%s: too many blocks", name);
    P.q = static_cast<const uint16_t*>(q);
    P.k = static_cast<const uint16_t*>(k);
    P.v = static_cast<const uint16_t*>(v);
    P.out = static_cast<uint16_t*>(out);
    P.S = (uint32_t)S;
    P.T = (uint32_t)T;
    P.nq = (uint32_t)nq;
    P.n_wg = (uint32_t)nwg;
    P.xcd_remap = (nwg % 8 == 0) ? 1u : 0u;
    P.scale_log2 = resolve_scale_log2(scale, D);
    P.kv_idx = kv_idx;
    P.kv_cnt = kv_cnt;
    P.max_kept = (uint32_t)max_kept;
    P.knorm = key_norms;
    P.head_choice = head_choice;
    P.n_tiles = (uint32_t)n_tiles;
    P.Hg = (uint32_t)Hg;
    P.Wg = (uint32_t)Wg;
    rc = set_row_order(P, row_order, row_order_len, name);
    if (rc) return rc;
    set_order(P, B * H, max_kept);
    if (pad) launch_solo<kBlockList, true, true>(P, (hipStream_t)stream);
    else launch_solo<kBlockList, true>(P, (hipStream_t)stream);
    return check_launch(name);
}

}  // namespace
}  // namespace bsa

extern "C" int bsa_block_sparse_attention_tiled(const void* q, const void* k, const void* v, void* out, int dtype,
                                                int64_t B, int64_t H, int T, int Hg, int Wg, int64_t D,
                                                const int32_t* tiles_host, int n_tiles, const int32_t* head_choice,
                                                const int32_t* kv_idx, const int32_t* kv_cnt, int max_kept,
                                                float scale, const float* key_norms_or_null,
                                                const uint32_t* row_order_or_null, int64_t row_order_len,
                                                bsa_stream_t stream) {
    clear_error();
    return tiled_attention(q, k, v, out, dtype, B, H, T, Hg, Wg, D, tiles_host, n_tiles, head_choice, kv_idx, kv_cnt,
                           max_kept, scale, key_norms_or_null, row_order_or_null, row_order_len, false, stream,
                           "bsa_block_sparse_attention_tiled");
}

extern "C" int bsa_block_sparse_attention_tiled_padded(const void* q, const void* k, const void* v, void* out,
                                                       int dtype, int64_t B, int64_t H, int T, int Hg, int Wg,
                                                       int64_t D, const int32_t* tiles_host, int n_tiles,
                                                       const int32_t* head_choice, const int32_t* kv_idx,
                                                       const int32_t* kv_cnt, int max_kept, float scale,
                                                       const float* key_norms_or_null,
                                                       const uint32_t* row_order_or_null, int64_t row_order_len,
                                                       bsa_stream_t stream) {
    clear_error();
    return tiled_attention(q, k, v, out, dtype, B, H, T, Hg, Wg, D, tiles_host, n_tiles, head_choice, kv_idx, kv_cnt,
                           max_kept, scale, key_norms_or_null, row_order_or_null, row_order_len, true, stream,
                           "bsa_block_sparse_attention_tiled_padded");
}

extern "C" int bsa_tiled_attention_supported(int dtype, int64_t D, int T, int Hg, int Wg, const int32_t* tiles_host,
                                             int n_tiles, int pad) {
    clear_error();
    const char* name = "bsa_tiled_attention_supported";
    if (!(dtype == BSA_BF16 && D == 128) || T <= 0 || Hg <= 0 || Wg <= 0) return 0;
    if ((pad ? check_tiles_padded(T, Hg, Wg, tiles_host, n_tiles) : check_tiles(T, Hg, Wg, tiles_host, n_tiles)) !=
        BSA_OK)
        return 0;
    AttnParams P{};
    for (int i = 0; i < n_tiles; ++i) {
        const int a = tiles_host[3 * i], b = tiles_host[3 * i + 1], c = tiles_host[3 * i + 2];
        if (pad && (Hg % b != 0 || Wg % c != 0)) return 0;
        if (fill_tile_rows(P, i, Hg, Wg, a, b, c, D, name) != BSA_OK) return 0;
    }
    clear_error();
    return 1;
}

extern "C" int bsa_temporal_only_attention(const void* q, const void* k, const void* v, void* out, int dtype,
                                           int64_t B, int64_t H, int T, int Hg, int Wg, int64_t D, float scale,
                                           bsa_stream_t stream) {
    clear_error();
    const char* name = "bsa_temporal_only_attention";
    BSA_REQUIRE(T > 0 && Hg > 0 && Wg > 0, "%s: grid must be positive", name);
    const int64_t S = (int64_t)T * Hg * Wg;
    int rc = common_checks(q, k, v, out, dtype, B, H, S, D, name);
    if (rc) return rc;
    if (!(dtype == BSA_BF16 && (D == 64 || D == 128) && T <= 64))
        BSA_FAIL(BSA_ERR_UNSUPPORTED,
                 "%s: bf16 with D in {64, 128} and T <= 64 only (bsa_video_labels + bsa_block_sparse_attention_labels "
                 "cover the rest)",
                 name);
    const int64_t hw = (int64_t)Hg * Wg, g = 64 / T, nq = (hw + g - 1) / g;
    const int64_t nwg = B * H * nq;
    BSA_REQUIRE(nwg < ((int64_t)1 << 31), "%s: too many tiles", name);
    AttnParams P{};
    P.q = static_cast<const uint16_t*>(q);
    P.k = static_cast<const uint16_t*>(k);
    P.v = static_cast<const uint16_t*>(v);
    P.out = static_cast<uint16_t*>(out);
    P.S = (uint32_t)S;
    P.nq = (uint32_t)nq;
    P.n_wg = (uint32_t)nwg;
    P.xcd_remap = (nwg % 8 == 0) ? 1u : 0u;
    P.scale_log2 = resolve_scale_log2(scale, D);
    P.grp_T = (uint32_t)T;
    P.grp_G = (uint32_t)g;
    P.grp_HW = (uint32_t)hw;
    if (D == 128) launch_mfma<128, 64, kGroups>(P, (hipStream_t)stream);
    else launch_mfma<64, 64, kGroups>(P, (hipStream_t)stream);
    return check_launch(name);
}
