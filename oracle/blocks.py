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


def topk_block_mask(scores, k: int, sink_blocks: int = 1, keep_diag: bool = True) -> np.ndarray:
    """Boolean (Nq, Nk) block mask: top-k per row, OR the sink and diagonal blocks.

    [Adaptive tiling (SPADE), "The idea" step 4 and "Recipe"]: a fixed top-k
    budget per query block, and the sink key blocks and the diagonal are
    always kept, ORed in after the top-k (so a row keeps between k and
    k + sink_blocks + 1 blocks).  Reading: sink blocks are key blocks
    0 .. sink_blocks-1 and the diagonal is key block J = I.
    """
    scores = np.asarray(scores, dtype=np.float64)
    nq, nk = scores.shape
    if sink_blocks < 0:
        raise ValueError("sink_blocks must be >= 0")
    keep = np.zeros((nq, nk), dtype=bool)
    for i in range(nq):
        keep[i, topk_row(scores[i], k)] = True
        keep[i, :min(sink_blocks, nk)] = True
        if keep_diag and i < nk:
            keep[i, i] = True
    return keep


def keep_to_lists(keep):
    """Ascending kept-index lists and counts from a boolean block mask (..., Nq, Nk)."""
    keep = np.asarray(keep, dtype=bool)
    cnt = keep.sum(axis=-1)
    return [np.flatnonzero(r) for r in keep.reshape(-1, keep.shape[-1])], cnt


def near_tie_ok(scores_row, k: int, idx: int, rel: float = 1e-5) -> bool:
    """True when block ``idx`` is within ``rel`` (relative) of the row's k-th score.

    Used to allow a top-k membership difference only for near ties.
    """
    s = np.asarray(scores_row, dtype=np.float64)
    kth = np.sort(s)[::-1][k - 1]
    return abs(s[idx] - kth) < rel * abs(kth)
