"""Pins of the oracle's tiling, permutation and cohesion definitions (CPU only)."""
import os

import numpy as np
import pytest

from oracle import tiling as T

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_ints(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return np.array([int(t) for line in f if not line.startswith("#") for t in line.split()])


def test_permutation_golden_hand_derived():
    assert np.array_equal(T.tile_permutation((2, 4, 4), (1, 2, 2)), _golden_ints("tile_perm_T2H4W4_tile1x2x2.txt"))


@pytest.mark.parametrize("grid,tile", [((2, 4, 4), (1, 2, 2)), ((8, 16, 16), (2, 4, 4)),
                                       ((20, 32, 48), (1, 8, 8)), ((20, 32, 48), (4, 4, 4)),
                                       ((4, 6, 10), (2, 3, 5))])
def test_permutation_invariants(grid, tile):
    perm = T.tile_permutation(grid, tile)
    S = int(np.prod(grid))
    a, b, c = tile
    vol = a * b * c
    assert np.array_equal(np.sort(perm), np.arange(S))                   # bijection
    inv = T.invert_permutation(perm)
    x = np.arange(S * 2).reshape(S, 2)
    assert np.array_equal(T.unpermute_tokens(T.permute_tokens(x, perm), perm), x)
    assert np.array_equal(T.permute_tokens(T.permute_tokens(x, perm), inv), x)
    labels = T.tile_labels(grid, tile)[perm]
    assert np.all(np.diff(labels) >= 0)                                 # tiles contiguous, in order
    _, Hg, Wg = grid
    t, rem = np.divmod(perm, Hg * Wg)
    y, xx = np.divmod(rem, Wg)
    for blk in range(S // vol):                                         # each block is one box
        sl = slice(blk * vol, (blk + 1) * vol)
        for coord, ext in ((t[sl], a), (y[sl], b), (xx[sl], c)):
            assert coord.min() % ext == 0 and coord.max() - coord.min() == ext - 1
        assert len(set(zip(t[sl], y[sl], xx[sl]))) == vol
    assert np.all(np.diff(perm.reshape(-1, vol), axis=1) > 0)           # T-major inside a tile


def test_permutation_closed_form():
    """Permuted position p = tile * vol + within-tile offset, both counted T-major."""
    grid, tile = (6, 8, 12), (3, 2, 4)
    T_, Hg, Wg = grid
    a, b, c = tile
    perm = T.tile_permutation(grid, tile)
    nty, ntx = Hg // b, Wg // c
    for p in range(0, T_ * Hg * Wg, 7):
        tid, r = divmod(p, a * b * c)
        tt, rem = divmod(tid, nty * ntx)
        ty, tx = divmod(rem, ntx)
        rt, rem = divmod(r, b * c)
        ry, rx = divmod(rem, c)
        assert perm[p] == ((tt * a + rt) * Hg + ty * b + ry) * Wg + tx * c + rx


def test_identity_tilings_and_errors():
    assert np.array_equal(T.tile_permutation((3, 4, 5), (1, 1, 1)), np.arange(60))
    assert np.array_equal(T.tile_permutation((3, 4, 5), (3, 4, 5)), np.arange(60))
    assert np.array_equal(T.tile_permutation((3, 4, 5), (1, 1, 5)), np.arange(60))
    with pytest.raises(ValueError):
        T.tile_labels((20, 32, 48), (16, 2, 2))     # 16 does not divide 20
    with pytest.raises(ValueError):
        T.invert_permutation(np.array([0, 0, 1]))


def test_cohesion_closed_forms():
    rng = np.random.default_rng(0)
    u = rng.standard_normal(16)
    assert T.tile_cohesion(np.outer(rng.random(10) + 0.1, u)) == pytest.approx(1.0, abs=1e-14)
    assert T.tile_cohesion(np.eye(16)[:9] * 3.0) == pytest.approx(0.0, abs=1e-15)
    assert T.tile_cohesion(np.stack([u, -2 * u])) == pytest.approx(-1.0, abs=1e-15)
    assert np.isnan(T.tile_cohesion(np.stack([u, 0 * u, 0 * u])))      # one non-zero token: no pair
    assert np.isnan(T.tile_cohesion(np.zeros((4, 16))))
    # two clusters of m identical unit vectors with cosine c between them
    w = rng.standard_normal(16)
    cu, cw = u / np.linalg.norm(u), w / np.linalg.norm(w)
    c, m = float(cu @ cw), 5
    x = np.concatenate([np.tile(cu, (m, 1)), np.tile(cw, (m, 1))])
    n = 2 * m
    want = (2 * m * (m - 1) + 2 * m * m * c) / (n * (n - 1))
    assert T.tile_cohesion(x) == pytest.approx(want, abs=1e-14)


def test_cohesion_invariances_and_normalised_sum_identity():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((12, 8))
    base = T.tile_cohesion(x)
    y = x * rng.uniform(0.1, 10.0, (12, 1))                              # positive rescaling
    assert T.tile_cohesion(y) == pytest.approx(base, abs=1e-13)
    assert T.tile_cohesion(x[rng.permutation(12)]) == pytest.approx(base, abs=1e-13)
    z = np.concatenate([x, np.zeros((3, 8))])                           # zero tokens excluded
    assert T.tile_cohesion(z) == pytest.approx(base, abs=1e-15)
    xh = x / np.linalg.norm(x, axis=1, keepdims=True)
    n = 12
    assert base == pytest.approx((np.sum(xh.sum(0) ** 2) - n) / (n * (n - 1)), abs=1e-13)


def test_block_self_similarity_is_per_block():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((24, 4))
    got = T.block_self_similarity(x, 8)
    assert got.shape == (3,)
    for i in range(3):
        assert got[i] == T.tile_cohesion(x[8 * i:8 * i + 8])
    with pytest.raises(ValueError):
        T.block_self_similarity(x, 5)


def test_select_tiling_constructed():
    grid = (2, 4, 4)
    tiles = [(2, 1, 1), (1, 2, 2), (1, 1, 4), (1, 2, 2)]
    rng = np.random.default_rng(3)
    vecs = rng.standard_normal((8, 32))
    lab = T.tile_labels(grid, (1, 2, 2))
    q = np.empty((1, 2, 32, 32))
    q[0, 0] = vecs[lab] * rng.uniform(0.5, 2.0, (32, 1))               # constant direction per 1x2x2 tile
    q[0, 1] = vecs[T.tile_labels(grid, (1, 1, 4))]
    choice, score = T.select_tiling(q, grid, tiles)
    assert score[0, 0, 1] == pytest.approx(1.0, abs=1e-14) and score[0, 0, 3] == score[0, 0, 1]
    assert choice[0, 0] == 1                                            # the tie with index 3 goes low
    assert choice[0, 1] == 2 and score[0, 1, 2] == pytest.approx(1.0, abs=1e-14)
    assert np.all(score[0, 0, [0, 2]] < 1.0 - 1e-3)
    with pytest.raises(ValueError):
        T.select_tiling(q, grid, [(2, 3, 1)])


def test_tiling_score_excludes_pairless_tiles():
    grid, tile = (1, 2, 4), (1, 1, 2)
    q = np.zeros((8, 3))
    q[0], q[1] = [1, 0, 0], [1, 1, 0]          # tile 0: cos 1/sqrt2
    q[2] = [0, 0, 1]                           # tile 1: one token, excluded
    q[4], q[5] = [1, 0, 0], [-1, 0, 0]         # tile 2: -1
    assert T.tiling_score(q, grid, tile) == pytest.approx((2 ** -0.5 - 1.0) / 2, abs=1e-15)
    assert T.tiling_score(np.zeros((8, 3)), grid, tile) == float("-inf")


def test_sliding_tile_counts():
    keep = T.sliding_tile_keep((4, 4, 4))
    assert keep.sum() == 1000                  # (4 + 2*3)^3 pairs within distance 1 per axis
    assert np.array_equal(keep, keep.T)
    counts = keep.sum(axis=1)
    assert counts.min() == 8 and counts.max() == 27
    assert counts[0] == 8 and counts[(1 * 4 + 1) * 4 + 1] == 27
    assert np.all(np.diag(keep))
    assert T.sliding_tile_keep((3, 1, 1), (0, 0, 0)).sum() == 3
