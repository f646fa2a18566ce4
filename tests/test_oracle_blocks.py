"""Pins of the oracle's block-score, budget, top-k and pipeline definitions (CPU only)."""
import os

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import blocks as K
from oracle import pipeline as P
from oracle import tiling as T

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_block_minmax_and_scores_brute_force():
    rng = np.random.default_rng(0)
    S, D, blk = 12, 3, 4
    q, k = rng.standard_normal((S, D)), rng.standard_normal((S, D))
    qmax, qmin = K.block_minmax(q, blk)
    sc = K.minmax_block_scores(q, k, blk)
    nb = S // blk
    for I in range(nb):
        for d in range(D):
            col = [q[I * blk + i][d] for i in range(blk)]
            assert qmax[I][d] == max(col) and qmin[I][d] == min(col)
    for I in range(nb):
        for J in range(nb):
            c = [max(q[I * blk + i][d] for i in range(blk)) + min(q[I * blk + i][d] for i in range(blk))
                 for d in range(D)]
            kx = [max(k[J * blk + i][d] for i in range(blk)) for d in range(D)]
            kn = [min(k[J * blk + i][d] for i in range(blk)) for d in range(D)]
            a = sum(c[d] * kx[d] for d in range(D))
            b = sum(c[d] * kn[d] for d in range(D))
            assert sc[I, J] == pytest.approx(max(a, b), abs=1e-13)


def test_scores_block1_closed_form_and_within_block_invariance():
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal((10, 5)), rng.standard_normal((10, 5))
    np.testing.assert_allclose(K.minmax_block_scores(q, k, 1), 2.0 * q @ k.T, atol=1e-13)
    perm = np.concatenate([rng.permutation(5), 5 + rng.permutation(5)])
    np.testing.assert_array_equal(K.minmax_block_scores(q[perm], k[perm], 5),
                                  K.minmax_block_scores(q, k, 5))
    with pytest.raises(ValueError):
        K.minmax_block_scores(q, k, 3)


def test_budget_golden():
    with open(os.path.join(GOLDEN, "budgets.txt")) as f:
        rows = [line.split() for line in f if line.strip() and not line.startswith("#")]
    for frac, n, k in rows:
        assert K.budget(float(frac), int(n)) == int(k)
    for bad in (0.0, -0.1, 1.01, float("nan")):
        with pytest.raises(ValueError):
            K.budget(bad, 10)


def test_topk_row_matches_library_sort():
    rng = np.random.default_rng(2)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        s = rng.integers(-3, 4, n).astype(np.float64)      # many exact ties
        if trial % 3 == 0:
            s = rng.standard_normal(n)
        k = int(rng.integers(1, n + 1))
        want = sorted(sorted(range(n), key=lambda j: (-s[j], j))[:k])
        assert list(K.topk_row(s, k)) == want


def test_topk_tie_zero_nan_rules():
    assert list(K.topk_row([1.0, 3.0, 3.0, 2.0, 3.0], 2)) == [1, 2]
    assert list(K.topk_row([-0.0, 0.0, -1.0], 1)) == [0]
    assert list(K.topk_row([0.0, -0.0, -1.0], 1)) == [0]
    assert list(K.topk_row([np.nan, -5.0, np.nan], 2)) == [0, 1]
    assert list(K.topk_row([np.inf, 1.0, np.nan], 1)) == [0]
    assert list(K.topk_row(np.arange(6.0), 6)) == list(range(6))
    with pytest.raises(ValueError):
        K.topk_row([1.0, 2.0], 3)


def test_topk_block_mask_sink_and_diagonal():
    rng = np.random.default_rng(3)
    s = rng.standard_normal((16, 16))
    keep = K.topk_block_mask(s, 3, sink_blocks=1, keep_diag=True)
    cnt = keep.sum(1)
    assert np.all((cnt >= 3) & (cnt <= 5))
    assert np.all(keep[:, 0]) and np.all(np.diag(keep))
    for i in range(16):
        extra = set(np.flatnonzero(keep[i])) - set(K.topk_row(s[i], 3))
        assert extra <= {0, i}
    assert np.all(K.topk_block_mask(s, 16))                  # k = Nk keeps everything
    keep0 = K.topk_block_mask(s, 2, sink_blocks=0, keep_diag=False)
    assert np.all(keep0.sum(1) == 2)
    lists, cnts = K.keep_to_lists(keep[None])
    assert all(np.all(np.diff(li) > 0) for li in lists) and np.array_equal(cnts[0], cnt)


def test_near_tie_rule():
    s = np.array([10.0, 9.99999999, 5.0, 1.0])
    assert K.near_tie_ok(s, 1, 1) and not K.near_tie_ok(s, 1, 2)
    # the bound is relative to the k-th score, strict, and two-sided
    s = np.array([4.0, 2.0, 2.0 - 1.9e-5, 2.0 - 2.1e-5, 1.0])
    assert K.near_tie_ok(s, 2, 2) and not K.near_tie_ok(s, 2, 3)      # below the k-th score
    assert K.near_tie_ok(s, 3, 1) and not K.near_tie_ok(s, 3, 0)      # above it
    # negative k-th score: the magnitude sets the bound
    s = np.array([-1.0, -1.000001, -1.0001, -5.0])
    assert K.near_tie_ok(s, 1, 1) and not K.near_tie_ok(s, 1, 2)
    # a k-th score of 0 admits no difference at all (the bound is 0)
    s = np.array([3.0, 0.0, 0.0, 1e-30, -2.0])
    assert not K.near_tie_ok(s, 3, 2) and not K.near_tie_ok(s, 3, 3)
    # NaN ranks last: it is never the k-th score of a row that has k numbers, and never a near tie
    s = np.array([np.nan, 5.0, 4.99999999, 1.0])
    assert K.near_tie_ok(s, 1, 2) and not K.near_tie_ok(s, 1, 0)
    assert not K.near_tie_ok(np.array([1.0, np.nan]), 2, 1)


def test_near_tie_rule_brute_force():
    """Against a plain loop: the k-th largest by sorted(), then the relative gap."""
    r = np.random.default_rng(17)
    for _ in range(30):
        s = np.round(r.standard_normal(25) * 4, 3)           # rounding makes exact ties common
        k = int(r.integers(1, 26))
        kth = sorted(s.tolist(), reverse=True)[k - 1]
        for j in range(25):
            assert K.near_tie_ok(s, k, j, 1e-3) == (abs(s[j] - kth) < 1e-3 * abs(kth))


def _sdpa(q, k, v):
    t = [torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v)]
    return torch.nn.functional.scaled_dot_product_attention(*t).numpy()


def test_pipeline_forms_agree_and_full_budget_is_dense():
    rng = np.random.default_rng(4)
    grid, tiles = (2, 4, 4), [(1, 2, 2), (2, 2, 1), (1, 1, 4)]
    q, k, v = (rng.standard_normal((1, 3, 32, 8)) for _ in range(3))
    r = P.adaptive_block_sparse(q, k, v, grid, tiles, frac=0.25)
    assert r["k"] == 2 and r["block"] == 4
    for h in range(3):
        lab = T.tile_labels(grid, tiles[int(r["choice"][0, h])])
        alt = P.label_mask_attention(q[0, h], k[0, h], v[0, h], lab, r["keep"][0, h], 8 ** -0.5)
        np.testing.assert_allclose(r["out"][0, h], alt, atol=1e-12)
        assert np.array_equal(r["perm"][0, h], T.tile_permutation(grid, tiles[int(r["choice"][0, h])]))
    dense = P.adaptive_block_sparse(q, k, v, grid, tiles, frac=1.0)
    np.testing.assert_allclose(dense["out"], _sdpa(q, k, v), atol=1e-12)


def test_pipeline_insensitive_to_within_tile_order():
    """Summaries and block masks ignore the order inside a tile, so the output does too."""
    rng = np.random.default_rng(5)
    grid, tile = (2, 4, 4), (1, 2, 2)
    q, k, v = (rng.standard_normal((32, 8)) for _ in range(3))
    perm = T.tile_permutation(grid, tile)
    alt = perm.reshape(-1, 4)[:, ::-1].ravel()               # reversed inside every tile
    outs = []
    for pm in (perm, alt):
        qp, kp, vp = (T.permute_tokens(x, pm) for x in (q, k, v))
        keep = K.topk_block_mask(K.minmax_block_scores(qp, kp, 4), 2)
        op = A.masked_attention(qp, kp, vp, A.block_keep_to_token_mask(keep, 4), 0.3)
        outs.append(T.unpermute_tokens(op, pm))
    np.testing.assert_allclose(outs[0], outs[1], atol=1e-12)


def test_pipeline_rejects_mixed_volumes():
    x = np.zeros((1, 1, 32, 4))
    with pytest.raises(ValueError):
        P.adaptive_block_sparse(x, x, x, (2, 4, 4), [(1, 2, 2), (1, 1, 2)], 0.5)
