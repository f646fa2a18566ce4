"""Block-sparse attention over T-major video token sequences for MI355X (gfx950).

The compute lives in libbsa.so (HIP, C ABI declared in include/bsa.h); this
package holds its build script, a ctypes binding with the same function names
(``bsa``) and the seeded synthetic inputs (``synth``).
"""
from .bsa import (  # noqa: F401
    AdaptiveBlockSparse, UnsupportedError, bsa_block_cohesion, bsa_block_sparse_attention, bsa_budget,
    bsa_invert_permutation, bsa_invert_permute, bsa_minmax_block_scores, bsa_select_tiling,
    bsa_sliding_tile_block_list, bsa_tile_permutation, bsa_tile_permute, bsa_topk_block_mask,
    bsa_validate_block_list, bsa_validate_indices, bsa_version, bsa_windowed_attention, lib,
)
