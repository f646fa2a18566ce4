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
                          sink_blocks: int = 1, keep_diag=True, statistic: str = "mean",
                          top_p=None, p_scale: float = 1.0):
    """Per head: choose a tiling, permute, score, keep top-k (+sink, +diag), attend, un-permute.

    q, k, v: float64 (B, H, S, D).  Every candidate must have the same volume
    so that all heads share one block count.  ``keep_diag`` is the diagonal
    band width (True = the diagonal alone), ``statistic`` the tiling-choice
    rule, and ``top_p`` (if given) replaces the top-k budget with the
    nucleus rule of blocks.top_p_count.  Returns a dict with the T-major
    output and every intermediate (choice, tiling scores, per-head
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
    choice, tscore = tiling.select_tiling(q, grid, tiles, statistic=statistic)
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
            if top_p is None:
                keep[b, h] = blocks.topk_block_mask(scores[b, h], kk, sink_blocks, keep_diag)
            else:
                keep[b, h] = blocks.top_p_block_mask(scores[b, h], top_p, sink_blocks, int(keep_diag), p_scale)
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


def padded_adaptive_block_sparse(q, k, v, grid, tiles, frac: float, scale=None,
                                 sink_blocks: int = 1, keep_diag=True, statistic: str = "mean"):
    """The recipe on grids the candidate tiles need not divide.

    [Adaptive tiling (SPADE), "Deviations and notes"]: pad the grid to a
    multiple of the tile with zero tokens, leave them out of the cohesion,
    and mask the padded keys.  Per head, on the padded grid of its chosen
    tiling: the block summaries cover real tokens only (block_minmax_valid),
    the budget is floor(frac * padded block count), padded keys are masked
    out of every row, and padded query rows are dropped when the result
    returns to T-major order.  Candidates must share one volume.  Returns a
    dict with the T-major output and, per head, the padded permutation,
    block scores and kept mask (lists, since padded lengths differ).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, S, D = attention.validate_qkv(q, k, v)
    vols = {a * b * c for a, b, c in tiles}
    if len(vols) != 1:
        raise ValueError("candidate tilings must share one volume")
    block = vols.pop()
    sc = attention.default_scale(D, scale)
    choice, tscore = tiling.select_tiling(q, grid, tiles, statistic=statistic, pad=True)
    out = np.empty_like(q)
    perms, scores, keeps, ks = [], [], [], []
    for b in range(B):
        for h in range(H):
            tile = tiles[int(choice[b, h])]
            perm = tiling.padded_tile_permutation(grid, tile)
            valid = perm >= 0
            src = np.where(valid, perm, 0)

            def gather(x):
                return np.where(valid[:, None], x[b, h][src], 0.0)

            qp, kp, vp = gather(q), gather(k), gather(v)
            nb = perm.shape[0] // block
            kk = blocks.budget(frac, nb)
            sc_bh = blocks.minmax_block_scores_valid(qp, kp, valid, block)
            keep = blocks.topk_block_mask(sc_bh, kk, sink_blocks, keep_diag)
            mask = attention.block_keep_to_token_mask(keep, block)
            mask = np.where(valid[None, :], mask, -np.inf)
            rows = np.flatnonzero(valid)
            op = attention.masked_attention(qp[rows], kp, vp, mask[rows], sc)
            out[b, h, perm[rows]] = op
            perms.append(perm)
            scores.append(sc_bh)
            keeps.append(keep)
            ks.append(kk)
    return dict(out=out, choice=choice, tiling_score=tscore, perm=perms, scores=scores, keep=keeps, k=ks,
                block=block)


def label_equal_attention(q_head, k_head, v_head, labels, scale: float, keep_head=None, block: int = 0):
    """Attention where query i sees key j exactly when labels[i] == labels[j].

    With ``keep_head`` (a block mask over runs of ``block`` tokens) the label
    rule is applied inside the kept blocks only.  The spatial-only and
    temporal-only masks of [ADR-0001, "Décision" step 1] are this rule with
    the frame index, or the spatial position, as the label (see
    attention.spatial_only_mask / temporal_only_mask).
    """
    labels = np.asarray(labels)
    allowed = labels[:, None] == labels[None, :]
    if keep_head is not None:
        allowed &= attention.block_keep_to_token_mask(keep_head, block) == 0.0
    mask = np.where(allowed, 0.0, -np.inf)
    return attention.masked_attention(q_head, k_head, v_head, mask, scale)


def label_rows_gathered(q_head, k_head, v_head, labels, rows, scale: float):
    """Rows ``rows`` of :func:`label_equal_attention` (no block mask), over the keys of their own label.

    The same result as the dense form: a key of another label adds exact
    zeros.  Rows are taken one label at a time, against that label's keys.
    """
    labels = np.asarray(labels)
    rows = np.asarray(rows)
    out = np.empty((rows.size, q_head.shape[1]))
    for lab in np.unique(labels[rows]):
        sel = np.flatnonzero(labels[rows] == lab)
        keys = np.flatnonzero(labels == lab)
        out[sel] = attention.masked_attention(q_head[rows[sel]], k_head[keys], v_head[keys], 0.0, scale)
    return out


def label_block_keep(labels, block: int) -> np.ndarray:
    """Block mask keeping (I, J) exactly when blocks I and J share some label (brute force)."""
    labels = np.asarray(labels)
    s = labels.shape[0]
    if block <= 0 or s % block:
        raise ValueError(f"block {block} must divide S={s}")
    nb = s // block
    keep = np.zeros((nb, nb), dtype=bool)
    for i in range(nb):
        li = set(labels[i * block:(i + 1) * block].tolist())
        for j in range(nb):
            keep[i, j] = bool(li & set(labels[j * block:(j + 1) * block].tolist()))
    return keep
