"""Oracle: tiles, permutations, cohesion and tiling choice (TEST INFRASTRUCTURE ONLY).

Tokens are in T-major order, s = (t * Hg + y) * Wg + x [ADR-0001, shared
conventions: token order].
"""
from __future__ import annotations

import numpy as np


def check_tile(grid, tile):
    """A candidate tile must divide the grid [Adaptive tiling (SPADE), "Deviations and notes"]."""
    T, Hg, Wg = (int(g) for g in grid)
    a, b, c = (int(t) for t in tile)
    if min(T, Hg, Wg) <= 0 or min(a, b, c) <= 0:
        raise ValueError(f"grid {grid} and tile {tile} must be positive")
    if T % a or Hg % b or Wg % c:
        raise ValueError(f"tile {tile} does not divide grid {grid}")
    return T, Hg, Wg, a, b, c


def tile_labels(grid, tile) -> np.ndarray:
    """Tile id of every T-major token.

    [Adaptive tiling (SPADE), "What mlx-arsenal ships" / "Recipe"]: tokens
    are labelled by the tile that holds them; tiles are numbered in T-major
    order over the tile grid (reading: the pages do not fix the numbering).
    """
    T, Hg, Wg, a, b, c = check_tile(grid, tile)
    t, y, x = np.meshgrid(np.arange(T), np.arange(Hg), np.arange(Wg), indexing="ij")
    lab = ((t // a) * (Hg // b) + (y // b)) * (Wg // c) + (x // c)
    return lab.ravel().astype(np.int64)


def tile_permutation(grid, tile) -> np.ndarray:
    """perm with y[p] = x[perm[p]] making every tile contiguous.

    [Adaptive tiling (SPADE), "Recipe"]: argsort of the tile labels.  Reading:
    the sort is stable, so tokens keep T-major order inside their tile.
    """
    return np.argsort(tile_labels(grid, tile), kind="stable").astype(np.int64)


def padded_grid(grid, tile):
    """The grid rounded up, axis by axis, to a multiple of the tile.

    [Adaptive tiling (SPADE), "Deviations and notes"]: a grid the tile does not
    divide is padded to a multiple of the tile with zero tokens.
    """
    T, Hg, Wg = (int(g) for g in grid)
    a, b, c = (int(t) for t in tile)
    if min(T, Hg, Wg) <= 0 or min(a, b, c) <= 0:
        raise ValueError(f"grid {grid} and tile {tile} must be positive")
    return -(-T // a) * a, -(-Hg // b) * b, -(-Wg // c) * c


def pad_tokens(x, grid, tile):
    """Zero tokens appended along every axis: (..., T*Hg*Wg, D) -> (..., T'*H'*W', D), T-major."""
    x = np.asarray(x)
    T, Hg, Wg = grid
    Tp, Hp, Wp = padded_grid(grid, tile)
    lead, d = x.shape[:-2], x.shape[-1]
    g = x.reshape(*lead, T, Hg, Wg, d)
    out = np.zeros((*lead, Tp, Hp, Wp, d), dtype=x.dtype)
    out[..., :T, :Hg, :Wg, :] = g
    return out.reshape(*lead, Tp * Hp * Wp, d)


def padded_tile_permutation(grid, tile) -> np.ndarray:
    """Tile order over the padded grid, as indices into the real tokens (-1 = padding).

    The padded grid is labelled and stably sorted exactly like a dividing
    grid (tile_permutation of the padded grid); each position is then mapped
    back to its T-major index in the unpadded grid, or -1 if it is padding.
    """
    T, Hg, Wg = (int(g) for g in grid)
    pg = padded_grid(grid, tile)
    pperm = tile_permutation(pg, tile)
    _, Hp, Wp = pg
    t, rem = np.divmod(pperm, Hp * Wp)
    y, x = np.divmod(rem, Wp)
    real = (t < T) & (y < Hg) & (x < Wg)
    return np.where(real, (t * Hg + y) * Wg + x, -1).astype(np.int64)


def invert_permutation(perm) -> np.ndarray:
    """inv with inv[perm[p]] = p; ValueError unless perm is a bijection of 0..S-1.

    [Adaptive tiling (SPADE), "Recipe"]: the inverse order is argsort(order).
    """
    perm = np.asarray(perm, dtype=np.int64)
    s = perm.shape[0]
    if perm.ndim != 1 or not np.array_equal(np.sort(perm), np.arange(s)):
        raise ValueError("perm is not a permutation of 0..S-1")
    return np.argsort(perm, kind="stable").astype(np.int64)


def permute_tokens(x, perm):
    """y[..., p, :] = x[..., perm[p], :] (tiles become contiguous)."""
    return np.asarray(x)[..., np.asarray(perm), :]


def unpermute_tokens(y, perm):
    """x[..., perm[p], :] = y[..., p, :] (back to T-major order)."""
    y = np.asarray(y)
    out = np.empty_like(y)
    out[..., np.asarray(perm), :] = y
    return out


def tile_cohesion(tokens) -> float:
    """SICS of one tile: mean cosine over distinct pairs of non-zero tokens.

    [Adaptive tiling (SPADE), "The idea" step 1 and "Deviations and notes"]:
    cohesion is the mean pairwise cosine similarity of the queries in a tile;
    zero-norm tokens are left out.  Computed by brute force over every
    ordered pair i != j.  Reading: a tile with fewer than two non-zero tokens
    has no pair and returns NaN (it is excluded from the tiling average).
    The n x n matrix of pair cosines is formed explicitly (one product of the
    tile with itself) and its off-diagonal entries are averaged.
    """
    x = np.asarray(tokens, dtype=np.float64)
    norms = np.sqrt((x * x).sum(axis=1))
    keep = norms > 0
    n = int(keep.sum())
    if n < 2:
        return float("nan")
    xs, ns = x[keep], norms[keep]
    cos = (xs @ xs.T) / np.outer(ns, ns)
    return float((cos.sum() - np.trace(cos)) / (n * (n - 1)))


def block_self_similarity(x, block: int) -> np.ndarray:
    """SICS of each run of ``block`` consecutive tokens of x (S, D) -> (S // block,).

    [Adaptive tiling (SPADE), "What mlx-arsenal ships", block_self_similarity].
    """
    x = np.asarray(x, dtype=np.float64)
    s = x.shape[0]
    if block <= 0 or s % block:
        raise ValueError(f"block {block} must divide S={s}")
    return np.array([tile_cohesion(x[i:i + block]) for i in range(0, s, block)])


def tiling_score(q_head, grid, tile) -> float:
    """Mean SICS over the tiles of one tiling (tiles with no pair excluded).

    [Adaptive tiling (SPADE), "Deviations and notes", selection statistic]:
    the average of the per-tile mean cosines.  -inf if no tile has a pair.
    """
    perm = tile_permutation(grid, tile)
    a, b, c = tile
    coh = block_self_similarity(permute_tokens(q_head, perm), a * b * c)
    coh = coh[~np.isnan(coh)]
    return float(coh.mean()) if coh.size else float("-inf")


def tiling_score_padded(q_head, grid, tile) -> float:
    """tiling_score on the zero-padded grid (padding has zero norm, so it is left out)."""
    pg = padded_grid(grid, tile)
    return tiling_score(pad_tokens(q_head, grid, tile), pg, tile)


def pooled_tiling_score(q_head, grid, tile, pad: bool = False) -> float:
    """SPADE engine's pooled statistic: sum of pair cosines over sum of pairs.

    [Adaptive tiling (SPADE), "Deviations and notes", selection statistic]:
    SPADE's cossim kernel pools the pairwise similarities over the whole
    tiling (sum of pair similarities / number of pairs) and counts every
    token, zero-norm ones included.  Readings: a pair with a zero-norm token
    has similarity 0; on a padded grid the padding positions are not tokens
    and are not counted (tiles then differ in size).  Brute force over the
    ordered pairs i != j of every tile.
    """
    q = np.asarray(q_head, dtype=np.float64)
    if pad:
        perm = padded_tile_permutation(grid, tile)
    else:
        perm = tile_permutation(grid, tile)
    a, b, c = tile
    vol = a * b * c
    num, den = 0.0, 0
    for start in range(0, perm.shape[0], vol):
        idx = perm[start:start + vol]
        idx = idx[idx >= 0]
        x = q[idx]
        n = x.shape[0]
        norms = np.sqrt((x * x).sum(axis=1))
        unit = np.divide(x, norms[:, None], out=np.zeros_like(x), where=norms[:, None] > 0)
        cos = unit @ unit.T
        num += float(cos.sum() - np.trace(cos))
        den += n * (n - 1)
    return num / den if den else float("-inf")


def select_tiling(q, grid, tiles, statistic: str = "mean", pad: bool = False):
    """Per (b, h): index of the most cohesive candidate tiling, and all scores.

    [Adaptive tiling (SPADE), "The idea" step 1; "What mlx-arsenal ships",
    select_tiling].  Ties go to the lowest candidate index (np.argmax takes
    the first maximum).  statistic "mean" averages per-tile SICS (the
    library's rule); "pooled" is SPADE's engine rule (pooled_tiling_score).
    pad=True accepts candidates that do not divide the grid and scores them
    on the zero-padded grid.  Returns (choice int64 (B, H), score float64 (B, H, n)).
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, S, _ = q.shape
    T, Hg, Wg = grid
    if T * Hg * Wg != S:
        raise ValueError(f"grid {grid} does not match S={S}")
    if len(tiles) < 1:
        raise ValueError("need at least one candidate tiling")
    if statistic not in ("mean", "pooled"):
        raise ValueError(f"unknown statistic {statistic!r}")
    for t in tiles:
        if pad:
            padded_grid(grid, t)
        else:
            check_tile(grid, t)
    score = np.empty((B, H, len(tiles)))
    for bi in range(B):
        for hi in range(H):
            for ci, t in enumerate(tiles):
                if statistic == "pooled":
                    score[bi, hi, ci] = pooled_tiling_score(q[bi, hi], grid, t, pad)
                elif pad:
                    score[bi, hi, ci] = tiling_score_padded(q[bi, hi], grid, t)
                else:
                    score[bi, hi, ci] = tiling_score(q[bi, hi], grid, t)
    return np.argmax(score, axis=-1), score


def sliding_tile_keep(tile_grid, radius=(1, 1, 1)) -> np.ndarray:
    """Sliding-tile block mask over a grid of tiles, clipped at the edges.

    Query tile I keeps key tile J when their tile coordinates differ by at
    most ``radius`` along every axis (a 3x3x3 tile neighbourhood for radius
    1).  Tiles are numbered T-major over the tile grid; neighbours that would
    fall outside the grid do not exist.  [ADR-0001, "Décision" step 1,
    sliding_tile_block_mask; the pages name the mask, this is its plainest
    reading.]  Returns bool (N, N), N = nt * nh * nw.
    """
    nt, nh, nw = tile_grid
    t, y, x = np.meshgrid(np.arange(nt), np.arange(nh), np.arange(nw), indexing="ij")
    coords = np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1)
    d = np.abs(coords[:, None, :] - coords[None, :, :])
    return np.all(d <= np.asarray(radius)[None, None, :], axis=-1)
