"""Oracle: the adaptive-tiling block-sparse recipe end to end (TEST INFRASTRUCTURE ONLY).

Follows the steps of [Adaptive tiling (SPADE), "The idea" and "Recipe"] in
their order, with the "drop skipped blocks" variant of the recipe (expand the
block mask to tokens, dense attention) and the sink and diagonal blocks ORed
into the top-k mask.
"""
from __future__ import annotations

import numpy as np

from . import attention, blocks, tiling


def adaptive_block_sparse(q, k, v, grid, tiles, frac: float, scale=None,
                          sink_blocks: int = 1, keep_diag: bool = True):
    """Per head: choose a tiling, permute, score, keep top-k (+sink, +diag), attend, un-permute.

    q, k, v: float64 (B, H, S, D).  Every candidate must have the same volume
    so that all heads share one block count.  Returns a dict with the
    T-major output and every intermediate (choice, tiling scores, per-head
    permutation, block scores, kept mask).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, S, D = attention.validate_qkv(q, k, v)
    vols = {a * b * c for a, b, c in tiles}
    if len(vols) != 1:
        raise ValueError("candidate tilings must share one volume")
    block = vols.pop()
    nb = S // block
    sc = attention.default_scale(D, scale)
    choice, tscore = tiling.select_tiling(q, grid, tiles)
    kk = blocks.budget(frac, nb)
    out = np.empty_like(q)
    perms = np.empty((B, H, S), dtype=np.int64)
    scores = np.empty((B, H, nb, nb))
    keep = np.empty((B, H, nb, nb), dtype=bool)
    for b in range(B):
        for h in range(H):
            perm = tiling.tile_permutation(grid, tiles[int(choice[b, h])])
            perms[b, h] = perm
            qp, kp, vp = (tiling.permute_tokens(x[b, h], perm) for x in (q, k, v))
            scores[b, h] = blocks.minmax_block_scores(qp, kp, block)
            keep[b, h] = blocks.topk_block_mask(scores[b, h], kk, sink_blocks, keep_diag)
            mask = attention.block_keep_to_token_mask(keep[b, h], block)
            op = attention.masked_attention(qp, kp, vp, mask, sc)
            out[b, h] = tiling.unpermute_tokens(op, perm)
    return dict(out=out, choice=choice, tiling_score=tscore, perm=perms,
                scores=scores, keep=keep, k=kk, block=block)


def label_mask_attention(q_head, k_head, v_head, labels, keep_head, scale: float):
    """Second form of block-sparse attention, with no permutation at all.

    In T-major order, query i sees key j exactly when the block mask keeps
    (label(i), label(j)).  Agrees with attending in permuted order and
    un-permuting, because attention is equivariant under a common
    permutation of its rows and keys.
    """
    labels = np.asarray(labels)
    allowed = np.asarray(keep_head, dtype=bool)[labels][:, labels]
    mask = np.where(allowed, 0.0, -np.inf)
    return attention.masked_attention(q_head, k_head, v_head, mask, scale)
