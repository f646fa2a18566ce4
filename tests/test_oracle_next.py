"""Pins for the oracle's widened rows: static widths, top-p, the pooled
statistic, padded grids, and the spatial-only / temporal-only label masks.

Each check reaches the oracle's result by another route: a closed form, a
brute-force loop over small inputs, or a special case that reduces to an
already pinned function.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import attention as OA
from oracle import blocks as OB
from oracle import pipeline as OP
from oracle import tiling as OT


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------ static widths
def test_static_blocks_brute_force():
    for nq, nk, sink, w in [(5, 6, 1, 3), (7, 7, 0, 1), (9, 9, 2, 4), (6, 6, 3, 0), (4, 9, 5, 40)]:
        want = np.zeros((nq, nk), bool)
        for i in range(nq):
            for j in range(nk):
                want[i, j] = j < sink or (w >= 1 and 2 * abs(i - j) <= 2 * (w // 2))
        assert np.array_equal(OB.static_blocks(nq, nk, sink, w), want)


def test_band_width_counts_closed_form():
    nb, w = 100, 40
    keep = OB.static_blocks(nb, nb, 0, w)
    interior = keep[50]
    assert interior.sum() == 2 * (w // 2) + 1 == 41
    assert keep[0].sum() == w // 2 + 1
    keep = OB.static_blocks(nb, nb, 5, w)
    assert keep[:, :5].all() and keep[99].sum() == 5 + 21


def test_topk_with_widths_is_union_of_parts():
    s = _rng(1).standard_normal((60, 60))
    k = 7
    keep = OB.topk_block_mask(s, k, 5, 40)
    for i in range(60):
        want = set(OB.topk_row(s[i], k)) | set(range(5)) | {j for j in range(60) if abs(i - j) <= 20}
        assert set(np.flatnonzero(keep[i])) == want
    # width 1 is the old diagonal-only rule
    a = OB.topk_block_mask(s, k, 1, True)
    b = OB.topk_block_mask(s, k, 1, 1)
    assert np.array_equal(a, b)


# -------------------------------------------------------------------- top-p
def test_top_p_uniform_closed_form():
    for n, p in [(10, 0.35), (480, 0.17), (7, 0.99), (5, 0.01)]:
        assert OB.top_p_count(np.zeros(n), p) == math.ceil(p * n)


def test_top_p_two_levels_closed_form():
    # two blocks at log(3), four at 0: probabilities 0.3, 0.3, 0.1 x 4
    s = np.array([0.0, np.log(3.0), 0.0, np.log(3.0), 0.0, 0.0])
    assert OB.top_p_count(s, 0.25) == 1
    assert OB.top_p_count(s, 0.5) == 2
    assert OB.top_p_count(s, 0.65) == 3
    assert OB.top_p_count(s, 0.95) == 6
    keep = OB.top_p_block_mask(s[None, :], 0.5, 0, 0)
    assert list(np.flatnonzero(keep[0])) == [1, 3]
    # the third block goes to the lowest index among the equal ones
    keep = OB.top_p_block_mask(s[None, :], 0.65, 0, 0)
    assert list(np.flatnonzero(keep[0])) == [0, 1, 3]


def test_top_p_limits_and_scale():
    s = _rng(2).standard_normal(50) * 3
    assert OB.top_p_count(s, 1.0) == 50
    assert OB.top_p_count(s, 1e-9) == 1
    for sc in (0.1, 0.5, 2.0):
        assert OB.top_p_count(s, 0.7, sc) == OB.top_p_count(sc * s, 0.7)
    with pytest.raises(ValueError):
        OB.top_p_count(s, 0.0)


def test_top_p_brute_force_cumulative():
    r = _rng(3)
    for _ in range(20):
        s = r.standard_normal(30) * 2
        p = float(r.uniform(0.05, 0.95))
        m = OB.top_p_count(s, p)
        e = [math.exp(x) for x in s]
        z = sum(e)
        ranked = sorted(range(30), key=lambda j: (-s[j], j))
        cum = [sum(e[j] for j in ranked[:c]) / z for c in range(1, 31)]
        want = next(c for c in range(1, 31) if cum[c - 1] >= p)
        assert m == want


def _top_p_brute(row, p):
    """Count of the nucleus by a plain loop: NaN entries removed, softmax of what is left."""
    fin = [(x, j) for j, x in enumerate(row) if not math.isnan(x)]
    if not fin:
        return 1
    ranked = sorted(fin, key=lambda t: (-t[0], t[1]))
    top = ranked[0][0]
    if math.isinf(top):
        e = [1.0 if x == top else 0.0 for x, _ in ranked]
    else:
        e = [math.exp(x - top) for x, _ in ranked]
    z = sum(e)
    acc = 0.0
    for c, w in enumerate(e, start=1):
        acc += w
        if acc / z >= p:
            return c
    return len(e)


def test_top_p_nan_scores_carry_no_mass():
    """NaN scores: the count equals that of the row with the NaNs removed (a plain loop), and a NaN block
    is never kept while a number is left out."""
    r = _rng(31)
    for trial in range(40):
        n = int(r.integers(4, 40))
        s = r.standard_normal(n) * 2
        nan_at = r.random(n) < 0.3
        nan_at[int(r.integers(0, n))] = False              # keep at least one number
        s[nan_at] = np.nan
        p = float(r.uniform(0.05, 0.95))
        m = OB.top_p_count(s, p)
        assert m == _top_p_brute(s.tolist(), p), trial
        assert m == OB.top_p_count(s[~nan_at], p), trial
        keep = OB.top_p_block_mask(s[None, :], p, 0, 0)[0]
        assert keep.sum() == m
        if keep[nan_at].any():
            assert keep[~nan_at].all()
    # NaN ahead of the numbers in index order changes nothing: the numbers rank first
    s = np.array([np.nan, np.nan, 1.0, 0.0])
    keep = OB.top_p_block_mask(s[None, :], 0.99, 0, 0)[0]
    assert list(np.flatnonzero(keep)) == [2, 3]


def test_top_p_all_nan_row_keeps_lowest_index():
    s = np.full(7, np.nan)
    for p in (0.01, 0.5, 1.0):
        assert OB.top_p_count(s, p) == 1
        assert list(np.flatnonzero(OB.top_p_block_mask(s[None, :], p, 0, 0)[0])) == [0]


def test_top_p_infinities_take_the_softmax_limit():
    # two +inf scores share all the mass: 0.5 each
    s = np.array([1.0, np.inf, 3.0, np.inf, np.nan])
    assert OB.top_p_count(s, 0.5) == 1
    assert OB.top_p_count(s, 0.51) == 2
    assert OB.top_p_count(s, 1.0) == 2
    assert list(np.flatnonzero(OB.top_p_block_mask(s[None, :], 0.5, 0, 0)[0])) == [1]
    # only -inf numbers: uniform over them (NaN still weighs nothing)
    s = np.array([-np.inf, np.nan, -np.inf, -np.inf])
    assert OB.top_p_count(s, 0.5) == 2
    assert OB.top_p_count(s, 0.7) == 3
    # -inf beside a finite maximum weighs 0: probabilities 0.25, 0, 0.75
    s = np.array([0.0, -np.inf, np.log(3.0)])
    assert OB.top_p_count(s, 0.75) == 1
    assert OB.top_p_count(s, 0.8) == 2
    assert OB.top_p_count(s, 1.0) == 2
    for row in ([1.0, np.inf, 3.0, np.inf, np.nan], [-np.inf, np.nan, -np.inf, -np.inf], [0.0, -np.inf, 2.0]):
        for p in (0.2, 0.5, 0.9):
            assert OB.top_p_count(np.array(row), p) == _top_p_brute(row, p)


def test_top_p_rejects_bad_scale():
    for sc in (0.0, -1.0, float("inf"), float("nan")):
        with pytest.raises(ValueError):
            OB.top_p_count(np.zeros(4), 0.5, sc)


# ---------------------------------------------------------- pooled statistic
def _pooled_brute(q, grid, tile):
    T, Hg, Wg = grid
    a, b, c = tile
    num, den = 0.0, 0
    for t0 in range(0, T, a):
        for y0 in range(0, Hg, b):
            for x0 in range(0, Wg, c):
                toks = [q[(t * Hg + y) * Wg + x] for t in range(t0, min(T, t0 + a))
                        for y in range(y0, min(Hg, y0 + b)) for x in range(x0, min(Wg, x0 + c))]
                for i, j in itertools.permutations(range(len(toks)), 2):
                    ni, nj = np.linalg.norm(toks[i]), np.linalg.norm(toks[j])
                    num += 0.0 if ni == 0 or nj == 0 else float(toks[i] @ toks[j]) / (ni * nj)
                    den += 1
    return num / den


def test_pooled_statistic_brute_force_with_zero_tokens():
    grid, tile = (2, 4, 4), (2, 2, 2)
    q = _rng(4).standard_normal((32, 5))
    q[[0, 7, 13]] = 0.0
    assert OT.pooled_tiling_score(q, grid, tile) == pytest.approx(_pooled_brute(q, grid, tile), abs=1e-12)
    # padded: (3, 4, 4) with tile (2, 2, 2) pads T to 4; padding positions are not tokens
    q3 = _rng(5).standard_normal((48, 5))
    assert OT.pooled_tiling_score(q3, (3, 4, 4), tile, pad=True) == pytest.approx(
        _pooled_brute(q3, (3, 4, 4), tile), abs=1e-12)


def test_pooled_equals_mean_for_equal_tiles_without_zeros():
    # the pages: equal tile volumes and no zero tokens make both rules agree
    grid = (4, 8, 8)
    tiles = [(1, 4, 8), (4, 2, 4), (2, 4, 4)]
    q = _rng(6).standard_normal((1, 2, 256, 6))
    for h in range(2):
        for t in tiles:
            assert OT.pooled_tiling_score(q[0, h], grid, t) == pytest.approx(OT.tiling_score(q[0, h], grid, t),
                                                                              abs=1e-12)
    assert np.array_equal(OT.select_tiling(q, grid, tiles, "pooled")[0], OT.select_tiling(q, grid, tiles)[0])


# ------------------------------------------------------------------ padding
def test_padded_grid_and_permutation_reduce_to_dividing_case():
    assert OT.padded_grid((20, 32, 48), (16, 2, 2)) == (32, 32, 48)
    assert OT.padded_grid((16, 45, 80), (1, 8, 8)) == (16, 48, 80)
    for grid, tile in [((4, 8, 8), (2, 4, 4)), ((2, 4, 4), (1, 2, 2))]:
        assert np.array_equal(OT.padded_tile_permutation(grid, tile), OT.tile_permutation(grid, tile))


def test_padded_permutation_is_tile_order_of_real_tokens():
    grid, tile = (3, 5, 6), (2, 2, 4)
    perm = OT.padded_tile_permutation(grid, tile)
    Tp, Hp, Wp = OT.padded_grid(grid, tile)
    assert perm.shape[0] == Tp * Hp * Wp and (perm < 0).sum() == Tp * Hp * Wp - 90
    real = perm[perm >= 0]
    assert np.array_equal(np.sort(real), np.arange(90))
    # brute force: walk the padded tile grid in T-major tile order, T-major inside each tile
    want = []
    for tt in range(Tp // 2):
        for ty in range(Hp // 2):
            for tx in range(Wp // 4):
                for t in range(2 * tt, 2 * tt + 2):
                    for y in range(2 * ty, 2 * ty + 2):
                        for x in range(4 * tx, 4 * tx + 4):
                            want.append((t * 5 + y) * 6 + x if (t < 3 and y < 5 and x < 6) else -1)
    assert np.array_equal(perm, np.array(want))


def test_padded_tiling_score_is_mean_over_clipped_tiles():
    grid, tile = (3, 5, 6), (2, 2, 4)
    q = _rng(7).standard_normal((90, 4))
    q[11] = 0.0
    want = []
    for t0 in range(0, 3, 2):
        for y0 in range(0, 5, 2):
            for x0 in range(0, 6, 4):
                idx = [(t * 5 + y) * 6 + x for t in range(t0, min(3, t0 + 2)) for y in range(y0, min(5, y0 + 2))
                       for x in range(x0, min(6, x0 + 4))]
                c = OT.tile_cohesion(q[idx])
                if not np.isnan(c):
                    want.append(c)
    assert OT.tiling_score_padded(q, grid, tile) == pytest.approx(np.mean(want), abs=1e-12)
    # a dividing tile scores the same padded or not
    assert OT.tiling_score_padded(q, grid, (1, 5, 6)) == pytest.approx(OT.tiling_score(q, grid, (1, 5, 6)))


def test_valid_summaries_ignore_padding():
    x = _rng(8).standard_normal((8, 3))
    valid = np.array([1, 1, 0, 1, 0, 0, 0, 1], bool)
    mx, mn = OB.block_minmax_valid(x, valid, 4)
    assert np.array_equal(mx[0], x[[0, 1, 3]].max(0)) and np.array_equal(mn[1], x[[7]].min(0))
    assert np.array_equal(OB.block_minmax_valid(x, np.ones(8, bool), 4)[0], OB.block_minmax(x, 4)[0])
    with pytest.raises(ValueError):
        OB.block_minmax_valid(x, np.array([1, 1, 1, 1, 0, 0, 0, 0], bool), 4)


def test_padded_pipeline_reduces_to_dividing_pipeline():
    grid, tiles = (4, 8, 8), [(1, 4, 8), (4, 2, 4), (2, 4, 4)]
    q, k, v = (_rng(9 + i).standard_normal((1, 2, 256, 8)) for i in range(3))
    a = OP.adaptive_block_sparse(q, k, v, grid, tiles, 0.25)
    b = OP.padded_adaptive_block_sparse(q, k, v, grid, tiles, 0.25)
    assert np.array_equal(a["choice"], b["choice"])
    assert np.allclose(a["out"], b["out"], atol=1e-12)
    assert np.array_equal(a["keep"][0, 1], b["keep"][1])


def test_padded_pipeline_second_form_without_padding():
    """Padded attention equals attention over the real tokens under the block
    mask read through each real token's padded-tile position."""
    grid, tiles = (3, 6, 5), [(2, 2, 2), (1, 4, 2)]
    q, k, v = (_rng(20 + i).standard_normal((1, 2, 90, 8)) for i in range(3))
    r = OP.padded_adaptive_block_sparse(q, k, v, grid, tiles, 0.3, sink_blocks=1, keep_diag=3)
    for h in range(2):
        perm, keep = r["perm"][h], r["keep"][h]
        blk = np.empty(90, np.int64)
        pos = np.flatnonzero(perm >= 0)
        blk[perm[pos]] = pos // 8
        want = OP.label_mask_attention(q[0, h], k[0, h], v[0, h], blk, keep, 8 ** -0.5)
        assert np.allclose(r["out"][0, h], want, atol=1e-12)
        nb = perm.shape[0] // 8
        assert r["k"][h] == max(1, int(0.3 * nb))


# -------------------------------------------------- spatial / temporal masks
def test_spatial_only_is_attention_per_frame():
    grid = (3, 4, 4)
    q, k, v = (_rng(30 + i).standard_normal((48, 8)) for i in range(3))
    t = np.arange(48) // 16
    got = OP.label_equal_attention(q, k, v, t, 0.3)
    assert np.allclose(got, OA.masked_attention(q, k, v, OA.spatial_only_mask(grid), 0.3), atol=1e-12)
    for f in range(3):
        sl = slice(16 * f, 16 * f + 16)
        assert np.allclose(got[sl], OA.full_attention(q[sl][None, None], k[sl][None, None], v[sl][None, None], 0.3)[0, 0], atol=1e-12)


def test_temporal_only_is_attention_per_position():
    grid = (5, 2, 3)
    q, k, v = (_rng(40 + i).standard_normal((30, 8)) for i in range(3))
    pos = np.arange(30) % 6
    got = OP.label_equal_attention(q, k, v, pos, 0.5)
    assert np.allclose(got, OA.masked_attention(q, k, v, OA.temporal_only_mask(grid), 0.5), atol=1e-12)
    for s in range(6):
        idx = np.arange(s, 30, 6)
        assert np.allclose(got[idx], OA.full_attention(q[idx][None, None], k[idx][None, None], v[idx][None, None], 0.5)[0, 0], atol=1e-12)


def test_label_rows_gathered_matches_dense_label_rule():
    grid = (5, 3, 4)
    S = 60
    r = _rng(41)
    q, k, v = (r.standard_normal((S, 8)) for _ in range(3))
    for labels in (np.arange(S) % 12, np.arange(S) // 12, r.integers(0, 4, S)):
        want = OP.label_equal_attention(q, k, v, labels, 0.4)
        rows = np.arange(S)
        np.testing.assert_allclose(OP.label_rows_gathered(q, k, v, labels, rows, 0.4), want, atol=1e-12)
        some = np.array([59, 3, 17, 17, 40])
        np.testing.assert_allclose(OP.label_rows_gathered(q, k, v, labels, some, 0.4), want[some], atol=1e-12)
    # temporal-only labels (position of a T-major token) give the oracle's temporal-only mask
    pos = np.arange(S) % (grid[1] * grid[2])
    want = OA.masked_attention(q, k, v, OA.temporal_only_mask(grid), 0.4)
    np.testing.assert_allclose(OP.label_rows_gathered(q, k, v, pos, np.arange(S), 0.4), want, atol=1e-12)


def test_label_block_list_covers_the_label_mask():
    grid = (5, 4, 4)
    T, Hg, Wg = grid
    # temporal labels in (T,1,1)-tile order: runs of T tokens per position
    perm = OT.tile_permutation(grid, (T, 1, 1))
    lab = perm % (Hg * Wg)
    keep = OP.label_block_keep(lab, 16)
    q, k, v = (_rng(50 + i).standard_normal((80, 4)) for i in range(3))
    qp, kp, vp = (x[perm] for x in (q, k, v))
    a = OP.label_equal_attention(qp, kp, vp, lab, 0.4, keep, 16)
    b = OP.label_equal_attention(qp, kp, vp, lab, 0.4)
    assert np.allclose(a, b, atol=1e-12)
    # back in T-major order it is the temporal-only mask
    c = OT.unpermute_tokens(a, perm)
    assert np.allclose(c, OA.masked_attention(q, k, v, OA.temporal_only_mask(grid), 0.4), atol=1e-12)
    # spatial labels with frames of 16 tokens and blocks of 8: block-diagonal by frame
    sp = np.arange(80) // 16
    ks = OP.label_block_keep(sp, 8)
    i = np.arange(10)
    assert np.array_equal(ks, (i[:, None] // 2) == (i[None, :] // 2))
