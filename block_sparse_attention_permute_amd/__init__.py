"""Block-sparse attention over T-major video token sequences for MI355X (gfx950).

The compute lives in libbsa.so (HIP, C ABI declared in include/bsa.h); this
package holds its build script, a ctypes binding with the same function names
(``bsa``, re-exported here: every C entry point, the pipeline compositions and
the status / dtype codes) and the seeded synthetic inputs (``synth``).
"""
from .bsa import (  # noqa: F401
    BSA_BF16, BSA_F32, BSA_LABEL_SPATIAL, BSA_LABEL_TEMPORAL, BSA_MAX_TILINGS, BSA_NOALLOC_TILE_VALUES,
    BSA_STAT_MEAN, BSA_STAT_POOLED,
    EXPORTED, AdaptiveBlockSparse, UnsupportedError, VideoLabelAttention, bsa_block_cohesion,
    bsa_block_sparse_attention, bsa_block_sparse_attention_labels, bsa_block_sparse_attention_tiled,
    bsa_block_sparse_attention_tiled_padded, bsa_budget,
    bsa_invert_permutation, bsa_invert_permute, bsa_invert_permute_padded, bsa_label_block_list,
    bsa_minmax_block_scores, bsa_minmax_block_scores_tiled, bsa_minmax_block_scores_tiled_padded, bsa_padded_length, bsa_row_order, bsa_row_order_len, bsa_row_order_by_median, bsa_select_tiling,
    bsa_select_tiling_noalloc, bsa_sliding_tile_block_list, bsa_tile_permutation, bsa_tile_permutation_padded, bsa_tile_permute,
    bsa_tile_permute_padded, bsa_top_p_block_mask, bsa_topk_block_mask, bsa_topk_block_mask_tiled,
    bsa_temporal_only_attention, bsa_validate_block_list, bsa_validate_indices, bsa_version, bsa_video_labels,
    bsa_windowed_attention, lib,
    padded_rows, tiled_attention_supported, video_label_attention,
)
