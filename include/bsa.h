/*
 * bsa.h - block-sparse attention over T-major video token sequences, MI355X (gfx950).
 *
 * C ABI of libbsa.so.  Every call takes plain pointers and sizes.
 *
 * Conventions shared by all calls
 * -------------------------------
 *  Tokens.   A video latent of T x Hg x Wg positions is flattened T-major,
 *            s = (t*Hg + y)*Wg + x  [ADR-0001 "Sparse-attention roadmap for
 *            video DiTs", shared conventions: token order].  S = T*Hg*Wg.
 *  Tensors.  q, k, v and outputs are contiguous row-major (B, H, S, D)
 *            device arrays of one element type (bsa_dtype), 16-byte aligned
 *            [FastVideo windowed_attention.py, `_validate_qkv`: q, k, v share
 *            one (B, H, S, D) shape].
 *  Memory.   The caller owns every buffer and allocates it on the current
 *            HIP device; "device" below means a device pointer, "host" a
 *            host pointer.  The library keeps no pointer after a call
 *            returns.  Device calls are asynchronous on `stream` (0 = the
 *            null stream) unless marked synchronous.
 *  Status.   Every call returns a bsa_status.  Bad arguments give
 *            BSA_ERR_INVALID_ARG and violated invariants BSA_ERR_INVARIANT,
 *            mirroring the ValueError / RuntimeError split of [ADR-0001,
 *            shared conventions: validation].  On any error nothing is
 *            launched and bsa_last_error() returns a message (thread-local).
 *            Asynchronous calls check their arguments on the host only; they
 *            trust device-resident indices, which bsa_validate_block_list /
 *            bsa_validate_indices check on request.
 *  Masks.    Additive 0 / -inf semantics [ADR-0001, shared conventions: mask
 *            format]: a key is either seen with its plain score or not at all.
 */
#ifndef BSA_H
#define BSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* bsa_stream_t; /* a hipStream_t */

typedef enum {
    BSA_OK = 0,
    BSA_ERR_INVALID_ARG = 1, /* bad shape, size or option (a ValueError in Python) */
    BSA_ERR_INVARIANT = 2,   /* a checked invariant does not hold (a RuntimeError) */
    BSA_ERR_UNSUPPORTED = 3, /* valid request this build has no kernel for */
    BSA_ERR_DEVICE = 4       /* a HIP runtime call or launch failed */
} bsa_status;

typedef enum {
    BSA_F32 = 0,  /* IEEE binary32 */
    BSA_BF16 = 1  /* bfloat16 */
} bsa_dtype;

typedef enum {
    BSA_STAT_MEAN = 0,   /* mean over tiles of the per-tile cohesion */
    BSA_STAT_POOLED = 1  /* sum of pair similarities over the number of pairs */
} bsa_statistic;

#define BSA_MAX_TILINGS 8

/* Message of the last failed call on this thread ("" if none). */
const char* bsa_last_error(void);

/* ABI version: (major << 16) | minor. */
int bsa_version(void);

/* ------------------------------------------------------------------------
 * Host helpers (no GPU involved)
 * ------------------------------------------------------------------------ */

/* Tile-contiguous order of a T x Hg x Wg grid under tiles of a x b x c.
 * [Adaptive tiling (SPADE), "Recipe": the order is the argsort of the tile
 * labels]; tiles are numbered T-major over the tile grid and tokens keep
 * T-major order inside a tile.  Writes perm_host[p] = source token of
 * permuted position p, for p < T*Hg*Wg (host array, caller-owned).
 * INVALID_ARG if a size is <= 0 or the tile does not divide the grid
 * [Adaptive tiling (SPADE), "Deviations and notes": divisible grids only]. */
int bsa_tile_permutation(int T, int Hg, int Wg, int a, int b, int c, int32_t* perm_host);

/* inv[perm[p]] = p for p < S (host arrays).  INVALID_ARG unless perm is a
 * permutation of 0..S-1.  [Adaptive tiling (SPADE), "Recipe": the inverse
 * order is the argsort of the order.] */
int bsa_invert_permutation(const int32_t* perm_host, int64_t S, int32_t* inv_host);

/* Key blocks kept per query block: max(1, floor(frac * n_blocks)), with the
 * product formed in double precision.  [Adaptive tiling (SPADE), "The idea"
 * step 4 (a fixed budget, 17% on Wan 2.1, 10% on HunyuanVideo) and "Recipe"
 * (floored, at least one).]  Returns k >= 1, or -1 if frac is not in (0, 1]
 * or n_blocks < 1. */
int bsa_budget(double frac, int n_blocks);

/* Sliding-tile block lists over an nt x nh x nw grid of tiles (tiles
 * numbered T-major): query tile I keeps key tile J when their tile
 * coordinates differ by at most (rt, rh, rw) on each axis; neighbours
 * outside the grid do not exist [ADR-0001, "Décision" step 1,
 * sliding_tile_block_mask, read as a clipped 3x3x3 neighbourhood for radius
 * 1].  Writes kv_idx_host[I*max_kept + i] (ascending, -1 padded) and
 * kv_cnt_host[I].  INVALID_ARG on sizes <= 0, radii < 0, or max_kept smaller
 * than the largest row. */
int bsa_sliding_tile_block_list(int nt, int nh, int nw, int rt, int rh, int rw,
                                int32_t* kv_idx_host, int32_t* kv_cnt_host, int max_kept);

/* Length T'*Hg'*Wg' of the grid padded up to a multiple of the tile along
 * every axis [Adaptive tiling (SPADE), "Deviations and notes": a grid the
 * candidate tiles do not divide is padded with zero tokens].  Returns -1 if
 * a size is <= 0. */
int64_t bsa_padded_length(int T, int Hg, int Wg, int a, int b, int c);

/* Tile order of the padded grid: writes perm_host[p] for p < the padded
 * length, the T-major index (in the unpadded grid) of the token at padded
 * permuted position p, or -1 for padding.  Tiles are numbered T-major over
 * the padded tile grid, cells T-major inside a tile (so a dividing tile
 * gives bsa_tile_permutation).  INVALID_ARG if a size is <= 0. */
int bsa_tile_permutation_padded(int T, int Hg, int Wg, int a, int b, int c, int32_t* perm_host);

typedef enum {
    BSA_LABEL_SPATIAL = 0,  /* spatial-only attention: a token sees its own frame */
    BSA_LABEL_TEMPORAL = 1  /* temporal-only attention: a token sees its own (y, x) in every frame */
} bsa_label_kind;

/* Token labels of spatial-only or temporal-only attention [ADR-0001,
 * "Décision" step 1: spatial_only_mask, temporal_only_mask; the pages give
 * the names only].  Reading: spatial-only lets token i see token j exactly
 * when they lie in one frame, temporal-only exactly when they sit at one
 * spatial position; both are the rule labels[i] == labels[j].  The labels
 * are written in the order the matching attention call runs in:
 *  BSA_LABEL_SPATIAL:  T-major order; labels_host[s] = t = s / (Hg*Wg), the
 *                      frame index (frames are contiguous runs of Hg*Wg);
 *  BSA_LABEL_TEMPORAL: the order of the tiling (T, 1, 1), where position
 *                      p = (y*Wg + x)*T + t holds token (t*Hg + y)*Wg + x;
 *                      labels_host[p] = y*Wg + x = p / T, the spatial
 *                      position (each position's T frames are contiguous).
 * labels_host: T*Hg*Wg int32 (host, caller-owned).  INVALID_ARG if a size
 * is <= 0, T*Hg*Wg exceeds 2^31 - 1, or kind is unknown. */
int bsa_video_labels(int T, int Hg, int Wg, int kind, int32_t* labels_host);

/* Block lists of the "same label" rule: key block J is kept for query block
 * I when some token of I and some token of J carry the same label (labels
 * < 0 never match).  With the frame index as label this is the block
 * structure of spatial-only attention, with the spatial position (in an
 * order that groups positions, e.g. tiles (T, 1, 1)) that of temporal-only
 * attention [ADR-0001, "Décision" step 1: spatial_only_mask,
 * temporal_only_mask].  labels_host: S int32 (host); block divides S.
 * Writes kv_idx_host[I*max_kept + i] (ascending, -1 padded) and
 * kv_cnt_host[I] for I < S/block.  INVALID_ARG on bad sizes or if a row does
 * not fit in max_kept. */
int bsa_label_block_list(const int32_t* labels_host, int64_t S, int block, int32_t* kv_idx_host,
                         int32_t* kv_cnt_host, int max_kept);

/* ------------------------------------------------------------------------
 * Device calls
 * ------------------------------------------------------------------------ */

/* Permute tokens so every tile is contiguous:
 *   y[b,h,p,:] = x[b,h,perm_c[p],:],  c = head_choice[b*H + h] (0 if NULL),
 * where perm_c is bsa_tile_permutation of the grid under candidate tile c
 * [Adaptive tiling (SPADE), "The idea" step 2 and "Recipe"].  tiles_host is
 * a host array of n_tiles (a, b, c) triples, 1 <= n_tiles <= BSA_MAX_TILINGS,
 * each dividing the grid.  head_choice: device int32[B*H] or NULL; values
 * must lie in [0, n_tiles) (trusted; see bsa_validate_indices).
 * x and y: device (B, H, S, D) of `dtype`, S = T*Hg*Wg, must not overlap.
 * The index math is done in-kernel; no permutation table is read. */
int bsa_tile_permute(const void* x, void* y, int dtype, int64_t B, int64_t H,
                     int T, int Hg, int Wg, int64_t D, const int32_t* tiles_host, int n_tiles,
                     const int32_t* head_choice, bsa_stream_t stream);

/* Inverse of bsa_tile_permute: x[b,h,perm_c[p],:] = y[b,h,p,:] (back to
 * T-major order) [Adaptive tiling (SPADE), "Recipe": outputs are taken back
 * with the inverse order].  Same arguments, with y the input and x the output. */
int bsa_invert_permute(const void* y, void* x, int dtype, int64_t B, int64_t H,
                       int T, int Hg, int Wg, int64_t D, const int32_t* tiles_host, int n_tiles,
                       const int32_t* head_choice, bsa_stream_t stream);

/* bsa_tile_permute over padded tilings (candidates need not divide the
 * grid): y is device (B, H, Sp, D) with Sp >= bsa_padded_length of every
 * candidate; y[b,h,p,:] = x[b,h,perm_c[p],:] with perm_c from
 * bsa_tile_permutation_padded, and zero rows where perm_c[p] = -1 or p is
 * past the padded length of candidate c [Adaptive tiling (SPADE),
 * "Deviations and notes": pad with zero tokens].  labels_or_null: device
 * int32 (B, H, Sp), written 0 for real rows and -1 for padding (the labels
 * of bsa_minmax_block_scores_masked and bsa_block_sparse_attention_labels),
 * or NULL.  INVALID_ARG if a tile extent is <= 0 or Sp is too short. */
int bsa_tile_permute_padded(const void* x, void* y, int dtype, int64_t B, int64_t H, int T, int Hg,
                            int Wg, int64_t D, const int32_t* tiles_host, int n_tiles,
                            const int32_t* head_choice, int64_t Sp, int32_t* labels_or_null,
                            bsa_stream_t stream);

/* Inverse of bsa_tile_permute_padded: x[b,h,perm_c[p],:] = y[b,h,p,:] for
 * the real rows (padding rows are dropped); y (B, H, Sp, D), x (B, H, S, D). */
int bsa_invert_permute_padded(const void* y, void* x, int dtype, int64_t B, int64_t H, int T, int Hg,
                              int Wg, int64_t D, const int32_t* tiles_host, int n_tiles,
                              const int32_t* head_choice, int64_t Sp, bsa_stream_t stream);

/* Cohesion (SICS) of every run of `block` consecutive tokens:
 *   coh[b,h,i] = mean over ordered pairs u != w of non-zero-norm tokens of
 *                cos(x_u, x_w), NaN when the run has fewer than two such tokens.
 * [Adaptive tiling (SPADE), "The idea" step 1 (mean pairwise cosine of the
 * queries in a tile) and "Deviations and notes" (zero-norm tokens excluded).]
 * Computed in fp32 from the normalised sum, (|sum u/|u||^2 - n) / (n(n-1)).
 * x: device (B, H, S, D); coh: device float[B*H*(S/block)].
 * INVALID_ARG unless block divides S. */
int bsa_block_cohesion(const void* x, int dtype, int64_t B, int64_t H, int64_t S, int64_t D,
                       int block, float* coh, bsa_stream_t stream);

/* Choose a tiling per (b, h): the candidate whose tiles have the highest mean
 * cohesion, ties to the lowest candidate index [Adaptive tiling (SPADE), "The
 * idea" step 1; "Deviations and notes": the average of per-tile mean
 * cosines, tiles without a pair left out, -inf if no tile has one].
 * q: device (B, H, S, D), S = T*Hg*Wg.  tiles_host: host (a, b, c) triples.
 * tile_coh: device float[B*H*n_tiles*maxNb] workspace that receives the
 * per-tile cohesion (maxNb = max over candidates of S/(a*b*c)); score:
 * device float[B*H*n_tiles]; choice: device int32[B*H].
 * INVALID_ARG if a candidate does not divide the grid or n_tiles is out of range. */
int bsa_select_tiling(const void* q, int dtype, int64_t B, int64_t H, int T, int Hg, int Wg,
                      int64_t D, const int32_t* tiles_host, int n_tiles, float* tile_coh,
                      float* score, int32_t* choice, bsa_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * bsa_select_tiling without the tile_coh workspace.  The per-tile cohesion
 * goes to a fixed array inside the library, BSA_NOALLOC_TILE_VALUES floats
 * (4 MiB) in the memory of each device the library runs on, held until the
 * process ends; its address is looked up once per device, on the first call
 * with that device current (make that first call outside graph capture).
 * Nothing is allocated, and nothing needs clearing: every per-tile value a
 * call reads is written earlier in the same call.  Calls that overlap on one
 * device (two streams or two threads) share the array and race: serialise
 * them.  Arguments, outputs and errors as bsa_select_tiling, plus
 * INVALID_ARG when B*H*n_tiles*maxNb exceeds BSA_NOALLOC_TILE_VALUES and
 * BSA_ERR_DEVICE when the array's address cannot be found. */
#define BSA_NOALLOC_TILE_VALUES (1 << 20)
int bsa_select_tiling_noalloc(const void* q, int dtype, int64_t B, int64_t H, int T, int Hg, int Wg,
                              int64_t D, const int32_t* tiles_host, int n_tiles, float* score,
                              int32_t* choice, bsa_stream_t stream);

/* bsa_select_tiling with a choice of statistic and padded candidates.
 * statistic BSA_STAT_MEAN is bsa_select_tiling's rule; BSA_STAT_POOLED is
 * SPADE's engine rule [Adaptive tiling (SPADE), "Deviations and notes",
 * selection statistic]: per candidate, the sum over tiles of the sum over
 * ordered pairs i != j of cos(q_i, q_j) divided by the number of such pairs,
 * every token counted (a pair with a zero-norm token has similarity 0).
 * pad = 1 accepts candidates that do not divide the grid and scores them on
 * the zero-padded grid: padding is left out of the mean rule and is not
 * counted by the pooled rule; pad = 0 rejects them like bsa_select_tiling.
 * tile_coh: device float[B*H*n_tiles*maxNb], maxNb = max over candidates of
 * bsa_padded_length/(a*b*c) (per-tile values: the cohesion, or for the
 * pooled rule its numerator).
 * q_summaries_or_null: device, 2*n_tiles*B*H*Nb*D elements of `dtype`, or
 * NULL.  When given, the same pass over q also writes every candidate's block
 * summaries of q [Adaptive tiling (SPADE), "The idea" step 3: elementwise max
 * and min of each block], in the order (candidate, max/min, B, H, Nb, D), so
 * that bsa_minmax_block_scores_tiled need not read q again.  It needs pad = 0
 * and candidates of one volume (Nb = S / volume).
 * INVALID_ARG on an unknown statistic, pad not in {0, 1}, a bad candidate,
 * or q summaries with pad = 1 or candidates of different volumes. */
int bsa_select_tiling_ex(const void* q, int dtype, int64_t B, int64_t H, int T, int Hg, int Wg,
                         int64_t D, const int32_t* tiles_host, int n_tiles, int statistic, int pad,
                         float* tile_coh, float* score, int32_t* choice, void* q_summaries_or_null,
                         bsa_stream_t stream);

/* Min/max block summaries and estimated block scores of tile-contiguous q, k:
 *   qmax_I = elementwise max over block I of q, qmin_I the min (and kmax, kmin),
 *   scores[b,h,I,J] = max((qmax_I + qmin_I) . kmax_J, (qmax_I + qmin_I) . kmin_J)
 * [Adaptive tiling (SPADE), "The idea" step 3].  Summaries are exact (each is
 * an input value); the sum and dot products are fp32.  Inputs must be finite.
 * q, k: device (B, H, S, D).  summaries: device, 4*B*H*Nb*D elements of
 * `dtype` in the order qmax, qmin, kmax, kmin, each (B, H, Nb, D); it is
 * written.  scores: device float (B, H, Nb, Nb).  Nb = S/block.
 * key_norms_or_null: device float (B, H, Nb) or NULL; when given, entry
 * (b, h, J) is set to the largest L2 norm of a key row of block J (fp32;
 * not part of the method: it lets bsa_block_sparse_attention bound a block's
 * scores by Cauchy-Schwarz).
 * INVALID_ARG unless block divides S. */
int bsa_minmax_block_scores(const void* q, const void* k, int dtype, int64_t B, int64_t H,
                            int64_t S, int64_t D, int block, void* summaries, float* scores,
                            float* key_norms_or_null, bsa_stream_t stream);

/* bsa_minmax_block_scores on T-major q and k: block J of head (b, h) is tile
 * J of candidate c = head_choice[b*H + h] (0 if NULL), read in place through
 * the tile geometry, so the permuted copies of q and k are never formed
 * (the summaries fused with the permutation [Adaptive tiling (SPADE),
 * "The idea" steps 2 and 3]).  Candidates must divide the grid and share one
 * volume, the block size.  Outputs as bsa_minmax_block_scores.
 * q_summaries_or_null: NULL, or the q summaries bsa_select_tiling_ex wrote
 * for the same q and candidates; the chosen candidate's are then copied into
 * `summaries` and q itself is not read (trusted to match q). */
int bsa_minmax_block_scores_tiled(const void* q, const void* k, int dtype, int64_t B, int64_t H,
                                  int T, int Hg, int Wg, int64_t D, const int32_t* tiles_host,
                                  int n_tiles, const int32_t* head_choice, void* summaries,
                                  float* scores, float* key_norms_or_null,
                                  const void* q_summaries_or_null, bsa_stream_t stream);

/* bsa_minmax_block_scores_tiled on each head's grid padded along T (the
 * candidates need not divide T): block J of head (b, h) is tile J of the
 * padded grid of candidate c = head_choice[b*H + h] (0 if NULL), tiles
 * numbered T-major as bsa_tile_permutation_padded.  Cells of the padding
 * frames lie past the head; they are left out of the summaries and the key
 * norms without being read, so the result equals
 * bsa_tile_permute_padded -> bsa_minmax_block_scores_masked (labels 0 for
 * real, -1 for padding) bit for bit, without the padded copies
 * [Adaptive tiling (SPADE), "Deviations and notes": pad with zero tokens and
 * mask them; "The idea" steps 2 and 3].  Nb = the largest padded block
 * count over the candidates; blocks past a head's own count hold padding
 * only (scores -inf, key norm 0).  Outputs as bsa_minmax_block_scores with
 * that Nb.  UNSUPPORTED when a candidate would pad along y or x (b must
 * divide Hg and c divide Wg); INVALID_ARG as bsa_minmax_block_scores_tiled
 * otherwise. */
int bsa_minmax_block_scores_tiled_padded(const void* q, const void* k, int dtype, int64_t B, int64_t H,
                                         int T, int Hg, int Wg, int64_t D, const int32_t* tiles_host,
                                         int n_tiles, const int32_t* head_choice, void* summaries,
                                         float* scores, float* key_norms_or_null, bsa_stream_t stream);

/* bsa_minmax_block_scores over labelled tokens only: tokens with
 * labels[b,h,s] < 0 (padding) are left out of the summaries, so a partial
 * block is summarised by its real tokens [Adaptive tiling (SPADE),
 * "Deviations and notes": padded grids].  A block with no such token scores
 * -inf in its whole row and column.  labels_or_null: device int32 (B, H, S)
 * (NULL: every token counts); key norms over the labelled key rows. */
int bsa_minmax_block_scores_masked(const void* q, const void* k, int dtype, int64_t B, int64_t H,
                                   int64_t S, int64_t D, int block, const int32_t* labels_or_null,
                                   void* summaries, float* scores, float* key_norms_or_null,
                                   bsa_stream_t stream);

/* Per-row block selection: keep the k best key blocks of each (b, h, I) row,
 * ranked by score (higher first) and then by index (lower first), then add
 * key blocks 0 .. sink_blocks-1 and the diagonal band abs(J - I) <= diag_width/2
 * (integer division; diag_width 1 = block J = I alone, 0 = no band)
 * [Adaptive tiling (SPADE), "The idea" step 4 and "Recipe": top-k budget,
 * sink blocks and a diagonal band ORed into the mask; SPADE's Wan widths are
 * 5 and 40].  -0.0 ranks as +0.0 and NaN below every number.
 * scores: device float (B, H, Nq, Nk).  kv_idx: device int32
 * (B, H, Nq, max_kept): kept indices ascending, then -1.  kv_cnt: device int32
 * (B, H, Nq).  mask_or_null: device uint8 (B, H, Nq, Nk), 1 = kept, or NULL.
 * INVALID_ARG unless 1 <= k <= Nk, 1 <= Nk <= 4096, sink_blocks >= 0,
 * diag_width >= 0 and max_kept >= min(Nk, k + sink_blocks + band), where
 * band = 2*(diag_width/2) + 1 (0 when diag_width = 0). */
int bsa_topk_block_mask(const float* scores, int64_t B, int64_t H, int Nq, int Nk, int k,
                        int sink_blocks, int diag_width, int32_t* kv_idx, int32_t* kv_cnt,
                        int max_kept, uint8_t* mask_or_null, bsa_stream_t stream);

/* Per-row block selection by probability mass (top-p; the pages name
 * top_p_block_mask among the block masks [Adaptive tiling (SPADE), "What
 * mlx-arsenal ships"] without defining it; the nucleus rule is used): the
 * row's block probabilities are softmax(scale * scores[b,h,I,:]); blocks are
 * ranked as in bsa_topk_block_mask and the shortest prefix whose cumulative
 * probability reaches p is kept (at least one block), then the sink blocks
 * and the diagonal band are added.  Weights and sums are fp32 and take the
 * softmax's limit values: NaN scores weigh 0; a +inf row max (or a row whose
 * numbers are all -inf) shares the mass equally among the entries equal to
 * it; a row of NaNs keeps its lowest index.  Arguments and outputs as
 * bsa_topk_block_mask.
 * INVALID_ARG unless 0 < p <= 1, scale > 0, 1 <= Nk <= 4096, sink_blocks >= 0,
 * diag_width >= 0 and max_kept >= Nk. */
int bsa_top_p_block_mask(const float* scores, int64_t B, int64_t H, int Nq, int Nk, float p,
                         float scale, int sink_blocks, int diag_width, int32_t* kv_idx,
                         int32_t* kv_cnt, int max_kept, uint8_t* mask_or_null,
                         bsa_stream_t stream);

/* Launch plan for block lists whose lengths differ from row to row, as the
 * top-p lists above do: a scheduling aid that is no step of the method and
 * changes no result (the attention calls take it as row_order).  The
 * attention kernels read each head's K and V tiles through the L2 cache of
 * the XCD that runs the head's rows (workgroup w runs on XCD w % 8), so the
 * plan keeps each unit's rows on one XCD, where a unit is a head (B*H >= 16)
 * or 2, 4 or 8 equal ranges of a head's rows (fewer heads; a count that
 * divides Nq).  Each unit weighs the sum over its rows of c + 5, with c the
 * row's kv_cnt clamped to [0, 65535], shifted right by the bits that bring
 * the total of all weights under 2^28 (none unless that total reaches it);
 * units, heaviest first (ties: lower unit first), go to the least loaded
 * XCD (ties: lower XCD first) among those holding fewer than ceil(U/8) of
 * the U units.  An XCD runs its units in the order they came, each unit's
 * rows in decreasing c (values of 255 or more rank as one; rows of one rank
 * come in no fixed order).  order[8j + x] is the j-th row (b*H + h)*Nq + I
 * of XCD x, and 0xFFFFFFFF an empty slot.
 * kv_cnt: device int32 (BH * Nq); order: device uint32 (order_len).  The
 * last 3U entries of the plan serve the call as scratch and are left empty.
 * Three launches: the weights and the per-unit sorts one workgroup per unit,
 * the scheduling one workgroup; kv_cnt is read twice.
 * INVALID_ARG unless order_len >= bsa_row_order_len(BH, Nq) > 0 and
 * order_len < 2^31. */
int bsa_row_order(const int32_t* kv_cnt, int64_t BH, int64_t Nq, uint32_t* order, int64_t order_len,
                  bsa_stream_t stream);

/* Host: the length of bsa_row_order's plan for BH heads of Nq rows,
 * 8 * ceil(U/8) * (rows per unit) + 3U >= BH * Nq, or -1 (and bsa_last_error) unless
 * BH, Nq >= 1, BH * Nq < 2^31, the plan has at most 1024 units and fewer
 * than 2^31 entries.  Nothing is launched. */
int64_t bsa_row_order_len(int64_t BH, int64_t Nq);

/* Launch order for block lists of (nearly) equal lengths, as top-k lists
 * are: like bsa_row_order a scheduling aid that is no step of the method and
 * changes no result (the attention calls take it as row_order, with
 * row_order_len = BH * Nq).  The rows keep the plain split over the 8 XCDs
 * (XCD x runs rows x*BH*Nq/8 .. (x+1)*BH*Nq/8 - 1 of the order below, so a
 * head stays on one XCD when 8 divides BH), but each head's rows come sorted
 * by the middle entry of their kept list, kv_idx[row][kv_cnt[row] / 2] (0 for
 * an empty row; rows with one key come in no fixed order).  Query blocks that
 * an XCD runs side by side then keep key blocks from the same part of the
 * sequence and share more of them through the XCD's L2.  order[8j + x] is the
 * j-th row (b*H + h)*Nq + I of XCD x; every slot is filled.
 * kv_idx, kv_cnt: device int32 as bsa_topk_block_mask writes them (kept
 * indices ascending, kv_cnt clamped to [0, max_kept], entries outside
 * [0, Nk) clamped); order: device uint32 (order_len).  One launch, one
 * workgroup per head.  INVALID_ARG unless BH, Nq >= 1, BH * Nq < 2^31 is a
 * multiple of 8, max_kept >= 1, 1 <= Nk <= 4096 and
 * BH * Nq <= order_len < 2^31. */
int bsa_row_order_by_median(const int32_t* kv_idx, const int32_t* kv_cnt, int64_t BH, int64_t Nq,
                            int max_kept, int64_t Nk, uint32_t* order, int64_t order_len,
                            bsa_stream_t stream);

/* bsa_row_order_by_median for heads of head_kv_bytes bytes of K and V
 * (2 * S * D * element size; 0 when unknown, which gives exactly
 * bsa_row_order_by_median).  Heads above 32 MiB, when 4 divides BH and Nq
 * is even, are split over two XCDs: XCDs 2g and 2g + 1 run heads g, g + 4,
 * g + 8, ... in turn, XCD 2g + i taking the i-th half of each head's rows in
 * the same sorted order, so that half as many heads are in flight at once
 * (order[8j + x] is the j-th row of XCD x; every slot is filled).  A
 * scheduling aid like bsa_row_order_by_median: no step of the method, no
 * change to any result.  INVALID_ARG as bsa_row_order_by_median, or when
 * head_kv_bytes < 0. */
int bsa_row_order_by_median_ex(const int32_t* kv_idx, const int32_t* kv_cnt, int64_t BH, int64_t Nq,
                               int max_kept, int64_t Nk, int64_t head_kv_bytes, uint32_t* order,
                               int64_t order_len, bsa_stream_t stream);

/* bsa_topk_block_mask with a per-head budget and block count: head (b, h)
 * uses k = k_table[c] and nk = nk_table[c], c = head_choice[b*H + h]
 * (device int32, trusted to lie in [0, n_table)).  Only key blocks J < nk
 * exist for the head (the sink blocks and the band are clipped to them) and
 * query rows I >= nk keep nothing (count 0).  This is the padded recipe,
 * where every candidate tiling has its own padded block count and the
 * budget is floor(frac * that count) [Adaptive tiling (SPADE), "Recipe" and
 * "Deviations and notes"].  k_table, nk_table: host int32[n_table],
 * 1 <= k <= nk <= Nk.  max_kept >= min(max nk, max k + sink + band). */
int bsa_topk_block_mask_tiled(const float* scores, int64_t B, int64_t H, int Nq, int Nk,
                              const int32_t* head_choice, const int32_t* k_table_host,
                              const int32_t* nk_table_host, int n_table, int sink_blocks,
                              int diag_width, int32_t* kv_idx, int32_t* kv_cnt, int max_kept,
                              uint8_t* mask_or_null, bsa_stream_t stream);

/* Block-sparse attention: for every query block I of `block` tokens,
 *   out_I = softmax(scale * q_I k_K^T) v_K,  K = the tokens of the key blocks
 *           kv_idx[b,h,I,0..kv_cnt[b,h,I])
 * which equals dense attention under the additive mask expanded from the
 * block mask [Adaptive tiling (SPADE), "Recipe": expand the block mask to
 * tokens and run dense attention; "Dense by design": a block-sparse kernel
 * skips the masked blocks instead].  scale NaN means D^-1/2
 * [FastVideo windowed_attention.py, `_default_scale`].
 * q, k, v, out: device (B, H, S, D) in the tile-contiguous order the blocks
 * refer to; out has q's dtype.  kv_idx: device int32 (B, H, S/block,
 * max_kept), ascending without repeats; kv_cnt: device int32 (B, H, S/block)
 * in [1, max_kept] (both trusted; see bsa_validate_block_list, which reports a
 * count of 0 as an invariant violation; the kernels write such a row as zeros).
 * bf16: D in {64, 128} and block in {32, 64} run on MFMA; other bf16 / fp32
 * shapes with D <= 128 use a scalar kernel.  Accumulation and softmax are
 * fp32; bf16 outputs are rounded to nearest even once.
 * key_norms_or_null: device float (B, H, S/block) or NULL, each at least the
 * largest L2 norm of a key row of its block (bsa_minmax_block_scores writes
 * them).  It changes only the work, not the result beyond rounding: for
 * bf16, D = 128, block 64 and scale > 0, a key block whose scores cannot
 * pass the smallest running row max of the query block by more than 32 in
 * log2 units (max_i |q_i| * norm_J * scale * log2(e), Cauchy-Schwarz; so no
 * weight exceeds 2^32) skips the running-max update, so its
 * softmax weights are taken relative to an older max (an exact shift of the
 * softmax; the weights are rounded to bf16 at a different scale).
 * row_order_or_null, row_order_len: a launch order (as bsa_row_order or
 * bsa_row_order_by_median writes it) or NULL, 0.  Given one, the bf16 kernels run row_order_len workgroups,
 * workgroup w taking row row_order[w] = (b*H + h)*(S/block) + I; entries
 * past the last row are empty slots, each row must appear exactly once
 * (a row left out is not written).  NULL keeps the library's own order.  The
 * result does not depend on the order; the fp32 / scalar kernel ignores it.
 * INVALID_ARG unless block divides S, max_kept >= 1 and, with an order,
 * 1 <= row_order_len < 2^31. */
int bsa_block_sparse_attention(const void* q, const void* k, const void* v, void* out, int dtype,
                               int64_t B, int64_t H, int64_t S, int64_t D, int block,
                               const int32_t* kv_idx, const int32_t* kv_cnt, int max_kept,
                               float scale, const float* key_norms_or_null,
                               const uint32_t* row_order_or_null, int64_t row_order_len,
                               bsa_stream_t stream);

/* Block-sparse attention on T-major q, k, v, out: query/key block J of head
 * (b, h) is tile J of candidate c = head_choice[b*H + h] (0 if NULL), and the
 * kernel gathers tile rows on load and scatters output rows on store, so
 * the result equals bsa_tile_permute -> bsa_block_sparse_attention ->
 * bsa_invert_permute without the three permuted copies and the inverse pass
 * [Adaptive tiling (SPADE), "The idea" step 2 and "Recipe": attention in
 * tile order, results taken back to T-major order].  kv_idx / kv_cnt and
 * key_norms_or_null (per tile, as bsa_minmax_block_scores_tiled writes them)
 * as in bsa_block_sparse_attention with S/64 blocks per head.
 * UNSUPPORTED unless dtype is bf16, D = 128 and every candidate has 64
 * cells that, taken four at a time in tile order, all sit at the same four
 * T-major offsets from the group's first cell (one row pattern per LDS-DMA
 * row group): an x extent that is a multiple of 4, or e.g. (16, 2, 2),
 * (8, 8, 1); bsa_tiled_attention_supported answers on the host.
 * row_order_or_null, row_order_len: as in bsa_block_sparse_attention, over
 * the S/64 tiles of each head.
 * INVALID_ARG if a candidate does not divide the grid. */
int bsa_block_sparse_attention_tiled(const void* q, const void* k, const void* v, void* out,
                                     int dtype, int64_t B, int64_t H, int T, int Hg, int Wg,
                                     int64_t D, const int32_t* tiles_host, int n_tiles,
                                     const int32_t* head_choice, const int32_t* kv_idx,
                                     const int32_t* kv_cnt, int max_kept, float scale,
                                     const float* key_norms_or_null,
                                     const uint32_t* row_order_or_null, int64_t row_order_len,
                                     bsa_stream_t stream);

/* bsa_block_sparse_attention_tiled on the zero-padded grids of candidates
 * that do not divide T [Adaptive tiling (SPADE), "Deviations and notes": pad
 * the grid with zero tokens, mask the padded keys].  Each head works on the
 * padded grid of its own candidate (tiles numbered T-major over it, as
 * bsa_tile_permutation_padded): cells of a padding frame read as zeros, are
 * masked as keys and are not written as rows, so the result equals
 * bsa_tile_permute_padded -> bsa_block_sparse_attention_labels (labels 0 for
 * real, -1 for padding) -> bsa_invert_permute_padded.  kv_idx / kv_cnt
 * (and key_norms_or_null) have Nq = the largest padded block count over the
 * candidates; rows of blocks past a head's own count are ignored.
 * row_order_or_null, row_order_len: as in bsa_block_sparse_attention, over
 * the Nq rows of each head (rows past a head's own count run empty).
 * UNSUPPORTED as bsa_block_sparse_attention_tiled, and when a candidate would
 * pad along y or x (b must divide Hg and c divide Wg). */
int bsa_block_sparse_attention_tiled_padded(const void* q, const void* k, const void* v, void* out,
                                            int dtype, int64_t B, int64_t H, int T, int Hg, int Wg,
                                            int64_t D, const int32_t* tiles_host, int n_tiles,
                                            const int32_t* head_choice, const int32_t* kv_idx,
                                            const int32_t* kv_cnt, int max_kept, float scale,
                                            const float* key_norms_or_null,
                                            const uint32_t* row_order_or_null, int64_t row_order_len,
                                            bsa_stream_t stream);

/* Host: 1 if bsa_block_sparse_attention_tiled (pad = 0) or its _padded form
 * (pad = 1) has a kernel for these arguments, else 0.  Nothing is launched. */
int bsa_tiled_attention_supported(int dtype, int64_t D, int T, int Hg, int Wg, const int32_t* tiles_host,
                                  int n_tiles, int pad);

/* bsa_block_sparse_attention with a token label rule inside the kept
 * blocks: query i sees key j when j's block is kept for i's block AND
 * labels[i] == labels[j].  Padding of a padded tiling is labelled -1 and
 * real tokens 0, so padded keys are masked out of every real row
 * [Adaptive tiling (SPADE), "Deviations and notes": mask the padded keys];
 * frame indices give spatial-only and spatial positions temporal-only
 * attention [ADR-0001, "Décision" step 1].  labels: device int32 with
 * element (b, h, s) at labels[(b*H + h)*label_head_stride + s]
 * (label_head_stride 0: one row shared by every head, else >= S).  A query
 * row that sees no key is written as zeros.  Other arguments as
 * bsa_block_sparse_attention (kv_cnt may be 0 for rows that keep nothing). */
int bsa_block_sparse_attention_labels(const void* q, const void* k, const void* v, void* out,
                                      int dtype, int64_t B, int64_t H, int64_t S, int64_t D,
                                      int block, const int32_t* kv_idx, const int32_t* kv_cnt,
                                      int max_kept, const int32_t* labels,
                                      int64_t label_head_stride, float scale,
                                      bsa_stream_t stream);

/* Temporal-only attention of T-major q, k, v, out [ADR-0001, "Décision"
 * step 1: temporal_only_mask; reading: token i sees token j exactly when
 * both sit at one spatial position (y, x), i.e. the same position in every
 * frame].  Equals bsa_block_sparse_attention_labels on the tiling (T, 1, 1)
 * with BSA_LABEL_TEMPORAL labels and their block lists, followed by the
 * inverse permutation, without forming a permuted copy: each 64-row tile
 * holds the T frames of floor(64 / T) positions, gathered from T-major
 * memory (its remaining rows are padding and are not written).
 * Scale as bsa_block_sparse_attention; out has q's shape and dtype.
 * UNSUPPORTED unless bf16 with D in {64, 128} and T <= 64 (the label call
 * covers the rest); INVALID_ARG on bad sizes. */
int bsa_temporal_only_attention(const void* q, const void* k, const void* v, void* out, int dtype,
                                int64_t B, int64_t H, int T, int Hg, int Wg, int64_t D, float scale,
                                bsa_stream_t stream);

/* Symmetric sliding-window attention with sinks: query i sees key j when
 * abs(i - j) <= window/2 (integer division) or j < sink
 * [FastVideo windowed_attention.py, module docstring "Window policy" and
 * `windowed_attention`].  The kernel visits only the key tiles of the local
 * slice and the sinks.  `chunk` is the query chunk of the page's loop; it
 * does not change the result (0 = the default min(window, 512)).  The policy
 * is applied at every window size (no unmasked shortcut when window >= S).
 * q, k, v, out: device (B, H, S, D) in T-major order.  scale NaN means D^-1/2.
 * INVALID_ARG unless window >= 1, 0 <= sink <= S and chunk >= 0 (argument
 * checks as on the page). */
int bsa_windowed_attention(const void* q, const void* k, const void* v, void* out, int dtype,
                           int64_t B, int64_t H, int64_t S, int64_t D, int window, int sink,
                           float scale, int chunk, bsa_stream_t stream);

/* Synchronous check of device-resident block lists: every count in
 * [1, max_kept] and every row ascending, without repeats, inside [0, Nk).
 * An empty row is the "no visible key" case [FastVideo windowed_attention.py,
 * `windowed_attention`: RuntimeError for a query block without keys].
 * Returns BSA_ERR_INVARIANT on the first violation found. */
int bsa_validate_block_list(const int32_t* kv_idx, const int32_t* kv_cnt, int64_t B, int64_t H,
                            int Nq, int Nk, int max_kept, bsa_stream_t stream);

/* Synchronous check that every device int32 v[0..n) lies in [lo, hi).
 * Returns BSA_ERR_INVARIANT otherwise. */
int bsa_validate_indices(const int32_t* v, int64_t n, int lo, int hi, bsa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
