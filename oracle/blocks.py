"""Oracle: min/max block scores and the top-k block budget (TEST INFRASTRUCTURE ONLY)."""
from __future__ import annotations

import math

import numpy as np


def block_minmax(x, block: int):
    """Element-wise max and min over each run of ``block`` consecutive tokens.

    [Adaptive tiling (SPADE), "The idea" step 3]: the per-block summaries are
    the element-wise maximum and minimum of the block's vectors.  x: (S, D)
    -> (xmax, xmin), each (S // block, D).  Exact: each entry is an input value.
    """
    x = np.asarray(x, dtype=np.float64)
    s, d = x.shape
    if block <= 0 or s % block:
        raise ValueError(f"block {block} must divide S={s}")
    xb = x.reshape(s // block, block, d)
    return xb.max(axis=1), xb.min(axis=1)


def minmax_block_scores(qp, kp, block: int):
    """Estimated block scores S[I, J] = max(c_I . kmax_J, c_I . kmin_J), c = qmax + qmin.

    [Adaptive tiling (SPADE), "The idea" step 3; "What mlx-arsenal ships",
    minmax_block_scores], on tile-contiguous (permuted) q and k of one head:
    (S, D) each -> (Nq, Nk) float64.  The literal formula: no softmax scale.
    """
    qmax, qmin = block_minmax(qp, block)
    kmax, kmin = block_minmax(kp, block)
    c = qmax + qmin
    return np.maximum(c @ kmax.T, c @ kmin.T)


def block_minmax_valid(x, valid, block: int):
    """block_minmax over the valid tokens of each block only (padding left out).

    Used on padded grids ([Adaptive tiling (SPADE), "Deviations and notes":
    pad with zero tokens]); reading: a partial edge tile is summarised by its
    real tokens, as SPADE's kernel treats partial tiles.  Every block must
    hold at least one valid token.
    """
    x = np.asarray(x, dtype=np.float64)
    valid = np.asarray(valid, dtype=bool)
    s, d = x.shape
    if block <= 0 or s % block:
        raise ValueError(f"block {block} must divide S={s}")
    xb = x.reshape(s // block, block, d)
    vb = valid.reshape(s // block, block)[:, :, None]
    if not vb.any(axis=1).all():
        raise ValueError("a block holds no valid token")
    return np.where(vb, xb, -np.inf).max(axis=1), np.where(vb, xb, np.inf).min(axis=1)


def minmax_block_scores_valid(qp, kp, valid, block: int):
    """minmax_block_scores with the summaries taken over valid tokens only."""
    qmax, qmin = block_minmax_valid(qp, valid, block)
    kmax, kmin = block_minmax_valid(kp, valid, block)
    c = qmax + qmin
    return np.maximum(c @ kmax.T, c @ kmin.T)


def budget(frac: float, n_blocks: int) -> int:
    """Kept key blocks per query block: max(1, floor(frac * n)).

    [Adaptive tiling (SPADE), "Recipe"]: the budget fraction times the number
    of key blocks, floored, at least one.  ValueError unless 0 < frac <= 1 and
    n_blocks >= 1.
    """
    if not (0.0 < frac <= 1.0):
        raise ValueError(f"budget fraction must be in (0, 1], got {frac}")
    if n_blocks < 1:
        raise ValueError(f"n_blocks must be >= 1, got {n_blocks}")
    return max(1, int(math.floor(float(frac) * float(n_blocks))))


def topk_row(scores_row, k: int) -> np.ndarray:
    """Indices of the k best key blocks of one row, ranked (score desc, index asc).

    [Adaptive tiling (SPADE), "The idea" step 4: a fixed per-row budget].
    Readings: equal scores go to the lower index; -0.0 equals +0.0; NaN ranks
    below every number.
    """
    s = np.asarray(scores_row, dtype=np.float64)
    n = s.shape[0]
    if not (1 <= k <= n):
        raise ValueError(f"k={k} must be in [1, {n}]")
    order = np.lexsort((np.arange(n), -s))   # primary: -score ascending (NaN last)
    return np.sort(order[:k])


def static_blocks(nq: int, nk: int, sink_blocks: int = 1, diag_width: int = 1) -> np.ndarray:
    """Blocks every row keeps whatever the scores: sinks and a diagonal band.

    [Adaptive tiling (SPADE), "Recipe" note]: SPADE always keeps a few sink
    key blocks and a diagonal band (its Wan configurations use widths 5 and
    40) and these are ORed into the estimated mask.  Readings: the sinks are
    key blocks 0 .. sink_blocks-1; a band of width w keeps J with
    abs(I - J) <= w // 2, the same rule as the windowed-attention policy
    ([FastVideo windowed_attention, "Window policy"]), so width 1 is the
    diagonal alone and width 0 keeps no band.
    """
    if sink_blocks < 0 or diag_width < 0:
        raise ValueError("sink_blocks and diag_width must be >= 0")
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    keep = j < sink_blocks
    if diag_width >= 1:
        keep = keep | (np.abs(i - j) <= diag_width // 2)
    return np.broadcast_to(keep, (nq, nk)).copy()


def topk_block_mask(scores, k: int, sink_blocks: int = 1, keep_diag=True) -> np.ndarray:
    """Boolean (Nq, Nk) block mask: top-k per row, OR the sink and diagonal blocks.

    [Adaptive tiling (SPADE), "The idea" step 4 and "Recipe"]: a fixed top-k
    budget per query block, and the sink key blocks and the diagonal are
    always kept, ORed in after the top-k.  ``keep_diag`` is a diagonal band
    width (True = 1, the diagonal alone; False = 0); see ``static_blocks``.
    """
    scores = np.asarray(scores, dtype=np.float64)
    nq, nk = scores.shape
    keep = static_blocks(nq, nk, sink_blocks, int(keep_diag))
    for i in range(nq):
        keep[i, topk_row(scores[i], k)] = True
    return keep


def top_p_ranked_mass(scores_row, scale: float = 1.0):
    """Ranking and unnormalised softmax weights of one row, for the nucleus rule.

    Returns (order, w): order ranks the blocks (score desc, index asc, NaN
    last, as topk_row) and w[i] is the weight of block order[i], i.e.
    exp(scale * (s - max)).  Non-finite scores take the softmax's limit
    values: NaN carries no weight; when the row's largest score is +inf (or
    every number in it is -inf) the weight is shared equally by the entries
    equal to it; otherwise -inf weighs 0.  A row of NaNs has no weight at all.
    scale must be positive and finite.
    """
    if not (math.isfinite(scale) and scale > 0.0):
        raise ValueError(f"scale must be positive and finite, got {scale}")
    s = np.asarray(scores_row, dtype=np.float64) * float(scale)
    n = s.shape[0]
    order = np.lexsort((np.arange(n), -s))   # NaN last
    z = s[order]
    top = z[0]                                # the row's largest score (NaN only if all are)
    if np.isnan(top):
        return order, np.zeros(n)
    if np.isinf(top):
        return order, np.where(z == top, 1.0, 0.0)
    return order, np.where(np.isnan(z), 0.0, np.exp(z - top))


def top_p_count(scores_row, p: float, scale: float = 1.0) -> int:
    """Smallest number of best-ranked blocks whose softmax mass reaches p.

    The pages name top_p_block_mask without defining it ([Adaptive tiling
    (SPADE), "What mlx-arsenal ships"]).  Reading (the nucleus rule): the
    row's block probabilities are softmax(scale * S_I.) over all key blocks
    (top_p_ranked_mass, with its limit values for NaN and infinite scores);
    blocks are ranked (score desc, index asc) and the shortest prefix with
    cumulative probability >= p is kept (at least one block).  p in (0, 1].
    A row with no mass at all (every score NaN) keeps its first-ranked
    block, the lowest index.
    """
    if not (0.0 < p <= 1.0):
        raise ValueError(f"p must be in (0, 1], got {p}")
    _, w = top_p_ranked_mass(scores_row, scale)
    n = w.shape[0]
    if w.sum() == 0.0:
        return 1
    cum = np.cumsum(w) / w.sum()
    m = int(np.searchsorted(cum, p, side="left")) + 1
    return min(max(m, 1), n)


def top_p_block_mask(scores, p: float, sink_blocks: int = 1, diag_width: int = 1, scale: float = 1.0):
    """Boolean (Nq, Nk) block mask: per row the top-p prefix, OR the static blocks."""
    scores = np.asarray(scores, dtype=np.float64)
    nq, nk = scores.shape
    keep = static_blocks(nq, nk, sink_blocks, diag_width)
    for i in range(nq):
        keep[i, topk_row(scores[i], top_p_count(scores[i], p, scale))] = True
    return keep


def keep_to_lists(keep):
    """Ascending kept-index lists and counts from a boolean block mask (..., Nq, Nk)."""
    keep = np.asarray(keep, dtype=bool)
    cnt = keep.sum(axis=-1)
    return [np.flatnonzero(r) for r in keep.reshape(-1, keep.shape[-1])], cnt


def near_tie_ok(scores_row, k: int, idx: int, rel: float = 1e-5) -> bool:
    """True when block ``idx`` is within ``rel`` (relative) of the row's k-th score.

    Used to allow a top-k membership difference only for near ties.  The
    k-th score is the k-th entry in topk_row's ranking (NaN last), so a row
    with NaN scores ranks them below every number; a NaN entry or a NaN k-th
    score is never a near tie.
    """
    s = np.asarray(scores_row, dtype=np.float64)
    n = s.shape[0]
    order = np.lexsort((np.arange(n), -s))
    kth = s[order[k - 1]]
    return bool(abs(s[idx] - kth) < rel * abs(kth))
