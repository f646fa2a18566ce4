"""Oracle: attention by definition (TEST INFRASTRUCTURE ONLY; see package doc).

All arithmetic is float64.  Inputs are the exact float64 values of the stored
bf16 / fp32 tensors.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def default_scale(head_dim: int, scale: float | None = None) -> float:
    """Softmax scale: the explicit value, else head_dim ** -1/2.

    [FastVideo windowed_attention.py, `_default_scale`]: an explicit scale is
    used as given; otherwise the inverse square root of the head dimension,
    which must be positive (ValueError otherwise).
    """
    if scale is not None:
        return float(scale)
    if head_dim <= 0:
        raise ValueError(f"head_dim must be positive, got {head_dim}")
    return float(head_dim) ** -0.5


def validate_qkv(q, k, v):
    """Rank-4 (B, H, S, D) tensors of identical shape with S > 0 and D > 0.

    [FastVideo windowed_attention.py, `_validate_qkv`]; bad arguments are a
    ValueError [ADR-0001, shared conventions: validation].
    """
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError(f"q/k/v must be rank 4 (B, H, S, D); got {q.shape}, {k.shape}, {v.shape}")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"q/k/v shapes differ: {q.shape}, {k.shape}, {v.shape}")
    b, h, s, d = q.shape
    if s == 0:
        raise ValueError("sequence length must be > 0")
    if d == 0:
        raise ValueError("head dim must be > 0")
    return b, h, s, d


def masked_attention(q, k, v, mask, scale: float):
    """softmax(scale * q k^T + M) v with an additive 0 / -inf mask.

    The defining result of every attention call on the path: dense scaled
    dot-product attention under an additive mask [ADR-0001, shared
    conventions: mask format; FastVideo windowed_attention.py,
    `full_attention`].  ``mask`` broadcasts against (B, H, S, S).  A query
    row whose mask hides every key has no defined output: RuntimeError
    [FastVideo windowed_attention.py, `windowed_attention`, raises].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    logits = scale * (q @ np.swapaxes(k, -1, -2)) + mask
    row_max = logits.max(axis=-1, keepdims=True)
    if not np.all(np.isfinite(row_max)):
        raise RuntimeError("a query row has no visible key")
    e = np.exp(logits - row_max)
    p = e / e.sum(axis=-1, keepdims=True)
    return p @ v


def masked_attention_rows(q_rows, k, v, mask_rows, scale: float):
    """The rows ``q_rows`` (n, D) of :func:`masked_attention` for one head.

    Same definition, evaluated for a subset of query rows against every key
    (``k``, ``v``: (S, D); ``mask_rows``: (n, S) additive).  Used where the
    full S x S problem does not fit in memory.
    """
    return masked_attention(q_rows, k, v, mask_rows, scale)


def full_attention(q, k, v, scale: float | None = None):
    """Dense attention with the default scale [FastVideo windowed_attention.py, `full_attention`]."""
    _, _, _, d = validate_qkv(q, k, v)
    return masked_attention(q, k, v, 0.0, default_scale(d, scale))


def window_mask(S: int, window: int, sink: int = 0):
    """Additive (S, S) mask of the symmetric sliding window with sinks.

    [FastVideo windowed_attention.py, module docstring "Window policy"]:
    query i sees key j when abs(i - j) <= window // 2, and every query sees
    the sink keys j < sink.  Arguments as validated in `windowed_attention`:
    window >= 1, 0 <= sink <= S.
    """
    if window < 1:
        raise ValueError(f"window must be >= 1, got {window}")
    if sink < 0:
        raise ValueError(f"sink must be >= 0, got {sink}")
    if sink > S:
        raise ValueError(f"sink ({sink}) exceeds sequence length ({S})")
    half = window // 2
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    allowed = (np.abs(i - j) <= half) | (j < sink)
    return np.where(allowed, 0.0, NEG_INF)


def windowed_attention(q, k, v, window: int, sink: int = 0, scale: float | None = None,
                       chunk: int | None = None):
    """Symmetric sliding-window attention with sinks, by definition.

    Dense masked attention under :func:`window_mask`.  The query chunk of
    [FastVideo windowed_attention.py, `windowed_attention`] only decides
    which key slices are loaded; it is validated (>= 1) and otherwise has no
    effect on the result.  Reading of the page: the window policy is the
    definition at every window size, including window >= S, where the page's
    shortcut to unmasked attention agrees with the policy only when
    window // 2 >= S - 1 or sink == S.
    """
    _, _, s, d = validate_qkv(q, k, v)
    mask = window_mask(s, window, sink)
    if chunk is not None and chunk < 1:
        raise ValueError(f"chunk must be >= 1, got {chunk}")
    return masked_attention(q, k, v, mask, default_scale(d, scale))


def block_keep_to_token_mask(keep, block_q: int, block_k: int | None = None):
    """Expand a boolean (Nq, Nk) block mask to an additive token mask.

    [Adaptive tiling (SPADE), "Recipe"]: to drop the skipped blocks, the block
    mask is repeated by the block size along both axes and given to dense
    attention.  ``keep`` may carry leading (B, H) axes.
    """
    block_k = block_q if block_k is None else block_k
    keep = np.asarray(keep, dtype=bool)
    tok = np.repeat(np.repeat(keep, block_q, axis=-2), block_k, axis=-1)
    return np.where(tok, 0.0, NEG_INF)


def block_sparse_attention(q, k, v, keep, block: int, scale: float | None = None):
    """Block-sparse attention over permuted tokens, by definition.

    ``keep``: bool (B, H, Nq, Nk), Nq = Nk = S / block.  The result is dense
    masked attention under the expanded block mask (see
    :func:`block_keep_to_token_mask`).
    """
    _, _, s, d = validate_qkv(q, k, v)
    if s % block:
        raise ValueError(f"block {block} does not divide S={s}")
    mask = block_keep_to_token_mask(keep, block)
    return masked_attention(q, k, v, mask, default_scale(d, scale))


def block_sparse_rows(q_head, k_head, v_head, keep_head, block: int, rows, scale: float):
    """Rows ``rows`` of one head's block-sparse attention, by definition.

    Each sampled query row p sees key q' exactly when the block mask keeps
    (p // block, q' // block); evaluated against all S keys with an explicit
    additive mask row.
    """
    rows = np.asarray(rows)
    s = k_head.shape[0]
    kb = np.arange(s) // block
    keep_head = np.asarray(keep_head, dtype=bool)
    mask_rows = np.where(keep_head[rows // block][:, kb], 0.0, NEG_INF)
    return masked_attention_rows(q_head[rows], k_head, v_head, mask_rows, scale)


def window_rows(q_head, k_head, v_head, rows, window: int, sink: int, scale: float):
    """Rows ``rows`` of one head's windowed attention, by definition."""
    rows = np.asarray(rows)
    s = k_head.shape[0]
    half = window // 2
    j = np.arange(s)[None, :]
    allowed = (np.abs(rows[:, None] - j) <= half) | (j < sink)
    mask_rows = np.where(allowed, 0.0, NEG_INF)
    return masked_attention_rows(q_head[rows], k_head, v_head, mask_rows, scale)


def block_sparse_rows_gathered(q_head, k_head, v_head, keep_head, block: int, rows, scale: float, key_valid=None):
    """Rows ``rows`` of one head's block-sparse attention over the kept key blocks only.

    The same result as :func:`block_sparse_rows`: a masked key adds exp(-inf)
    = 0 to the softmax sum and 0 * v to the output, so leaving it out changes
    nothing but the order of the additions.  For each query block holding
    sampled rows, the keys of its kept blocks are gathered and dense
    attention runs over them with no mask.  ``key_valid`` (bool (S,), or
    None) leaves further keys out, the padding of a padded grid
    ([Adaptive tiling (SPADE), "Deviations and notes": padded keys are
    masked]).  A query block that sees no key has no defined output:
    RuntimeError.
    """
    rows = np.asarray(rows)
    keep_head = np.asarray(keep_head, dtype=bool)
    out = np.empty((rows.size, q_head.shape[1]))
    qb = rows // block
    for i in np.unique(qb):
        sel = np.flatnonzero(qb == i)
        kept = np.flatnonzero(keep_head[i])
        keys = (kept[:, None] * block + np.arange(block)[None, :]).ravel()
        if key_valid is not None:
            keys = keys[np.asarray(key_valid, dtype=bool)[keys]]
        if keys.size == 0:
            raise RuntimeError("a query row has no visible key")
        out[sel] = masked_attention(q_head[rows[sel]], k_head[keys], v_head[keys], 0.0, scale)
    return out


def window_rows_gathered(q_head, k_head, v_head, rows, window: int, sink: int, scale: float, span: int = 64):
    """Rows ``rows`` of one head's windowed attention over the keys a row can see.

    The same result as :func:`window_rows`: rows are taken ``span``
    consecutive positions at a time, and each group is evaluated against the
    sink keys plus the union of its members' windows, with the window mask
    of :func:`window_mask` on that key set (keys outside it are masked for
    every row of the group, so leaving them out changes only the order of
    the additions).
    """
    rows = np.asarray(rows)
    s = k_head.shape[0]
    half = window // 2
    out = np.empty((rows.size, q_head.shape[1]))
    grp = rows // span
    for g in np.unique(grp):
        sel = np.flatnonzero(grp == g)
        r = rows[sel]
        lo, hi = max(0, int(r.min()) - half), min(s, int(r.max()) + half + 1)
        keys = np.union1d(np.arange(min(sink, s)), np.arange(lo, hi))
        allowed = (np.abs(r[:, None] - keys[None, :]) <= half) | (keys[None, :] < sink)
        out[sel] = masked_attention(q_head[r], k_head[keys], v_head[keys], np.where(allowed, 0.0, NEG_INF), scale)
    return out


def kept_block_flops(kv_cnt, block_q: int, block_k: int, D: int) -> int:
    """Algorithmic FLOPs of block-sparse attention: 4 * Bq * Bk * D per kept block."""
    return int(np.asarray(kv_cnt, dtype=np.int64).sum()) * 4 * block_q * block_k * D


def spatial_only_mask(grid) -> np.ndarray:
    """Additive (S, S) mask: token i sees token j exactly when both are in one frame.

    [ADR-0001, "Décision" step 1] names spatial_only_mask; the pages give no
    definition.  Reading: spatial-only attention stays inside a frame,
    t(i) == t(j), T-major tokens s = (t * Hg + y) * Wg + x.
    """
    T, Hg, Wg = (int(g) for g in grid)
    t = np.arange(T * Hg * Wg) // (Hg * Wg)
    return np.where(t[:, None] == t[None, :], 0.0, NEG_INF)


def temporal_only_mask(grid) -> np.ndarray:
    """Additive (S, S) mask: token i sees token j exactly when both sit at one (y, x).

    [ADR-0001, "Décision" step 1] names temporal_only_mask; reading:
    temporal-only attention links the same spatial position across frames.
    """
    T, Hg, Wg = (int(g) for g in grid)
    pos = np.arange(T * Hg * Wg) % (Hg * Wg)
    return np.where(pos[:, None] == pos[None, :], 0.0, NEG_INF)
