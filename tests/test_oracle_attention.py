"""Pins of the oracle's attention definitions (CPU only).

Each test checks the oracle against something other than itself: PyTorch's
float64 CPU scaled_dot_product_attention (a library routine), closed forms,
or the window policy enumerated from its range form.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _torch_sdpa(q, k, v, allowed=None, scale=None):
    t = [torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v)]
    m = None if allowed is None else torch.from_numpy(np.ascontiguousarray(allowed))
    return torch.nn.functional.scaled_dot_product_attention(*t, attn_mask=m, scale=scale).numpy()


def test_full_attention_matches_library_sdpa():
    q, k, v = (_rand((2, 3, 17, 8), s) for s in (1, 2, 3))
    np.testing.assert_allclose(A.full_attention(q, k, v), _torch_sdpa(q, k, v), rtol=0, atol=1e-12)
    np.testing.assert_allclose(A.full_attention(q, k, v, scale=0.3),
                               _torch_sdpa(q, k, v, scale=0.3), rtol=0, atol=1e-12)


def test_masked_attention_matches_library_sdpa_with_boolean_mask():
    q, k, v = (_rand((1, 2, 23, 5), s) for s in (4, 5, 6))
    rng = np.random.default_rng(7)
    allowed = rng.random((23, 23)) < 0.3
    allowed[np.arange(23), rng.integers(0, 23, 23)] = True   # every row sees a key
    mask = np.where(allowed, 0.0, -np.inf)
    got = A.masked_attention(q, k, v, mask, 5 ** -0.5)
    np.testing.assert_allclose(got, _torch_sdpa(q, k, v, allowed), rtol=0, atol=1e-12)


def test_softmax_rows_sum_to_one_and_masked_weights_are_zero():
    # with v = identity the output is the probability matrix itself
    S = 12
    q, k = _rand((1, 1, S, 4), 8), _rand((1, 1, S, 4), 9)
    v = np.eye(S)[None, None]
    allowed = np.random.default_rng(10).random((S, S)) < 0.5
    allowed[np.arange(S), np.arange(S)] = True
    p = A.masked_attention(q, k, v, np.where(allowed, 0.0, -np.inf), 0.5)[0, 0]
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p[~allowed] == 0.0) and np.all(p[allowed] > 0.0)


def test_closed_forms():
    S, D = 9, 6
    q = _rand((1, 1, S, D), 11)
    v = _rand((1, 1, S, D), 12)
    # all keys equal -> uniform weights over the visible keys -> mean of visible v
    k_same = np.broadcast_to(_rand((D,), 13), (1, 1, S, D)).copy()
    allowed = np.zeros((S, S), bool)
    allowed[:, [1, 4, 5]] = True
    out = A.masked_attention(q, k_same, v, np.where(allowed, 0.0, -np.inf), 1.0)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(v[0, 0, [1, 4, 5]].mean(0), (S, D)), atol=1e-12)
    # constant v -> the constant
    v_c = np.full((1, 1, S, D), 2.5)
    np.testing.assert_allclose(A.full_attention(q, _rand((1, 1, S, D), 14), v_c), 2.5, atol=1e-12)
    # a single visible key j -> v_j
    one = np.full((S, S), -np.inf)
    one[np.arange(S), (np.arange(S) * 4) % S] = 0.0
    out = A.masked_attention(q, _rand((1, 1, S, D), 15), v, one, 1.0)
    np.testing.assert_allclose(out[0, 0], v[0, 0, (np.arange(S) * 4) % S], atol=0)


def test_row_with_no_visible_key_raises():
    q = _rand((1, 1, 4, 2), 16)
    mask = np.zeros((4, 4))
    mask[2] = -np.inf
    with pytest.raises(RuntimeError):
        A.masked_attention(q, q, q, mask, 1.0)


def test_default_scale_and_validation():
    assert A.default_scale(64) == 0.125
    assert A.default_scale(64, 0.3) == 0.3
    with pytest.raises(ValueError):
        A.default_scale(0)
    x = np.zeros((1, 1, 4, 2))
    with pytest.raises(ValueError):
        A.validate_qkv(x[0], x, x)
    with pytest.raises(ValueError):
        A.validate_qkv(x, np.zeros((1, 1, 5, 2)), x)
    empty = np.zeros((1, 1, 0, 2))
    with pytest.raises(ValueError):
        A.validate_qkv(empty, empty, empty)


def _policy_allowed(S, window, sink):
    """Allowed keys from the range form of the window policy."""
    half = window // 2
    allowed = np.zeros((S, S), bool)
    for i in range(S):
        for j in range(max(0, i - half), min(S, i + half + 1)):
            allowed[i, j] = True
        for j in range(0, sink):
            allowed[i, j] = True
    return allowed


@pytest.mark.parametrize("S,window,sink", [(32, 8, 2), (32, 7, 0), (20, 1, 3), (16, 40, 0), (17, 5, 17)])
def test_windowed_matches_policy_enumeration(S, window, sink):
    q, k, v = (_rand((1, 2, S, 16), 20 + i) for i in range(3))
    want = _torch_sdpa(q, k, v, _policy_allowed(S, window, sink), scale=0.25)
    got = A.windowed_attention(q, k, v, window, sink, scale=0.25, chunk=8)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_windowed_special_cases():
    S = 16
    q, k, v = (_rand((1, 1, S, 4), 30 + i) for i in range(3))
    full = _torch_sdpa(q, k, v)
    # window >= 2S - 1 (half >= S - 1), no sink: every key visible -> dense
    np.testing.assert_allclose(A.windowed_attention(q, k, v, 2 * S - 1), full, atol=1e-12)
    # sink == S: every key is a sink -> dense
    np.testing.assert_allclose(A.windowed_attention(q, k, v, 1, sink=S), full, atol=1e-12)
    # window 1 (half 0), no sink: each query sees itself only -> v
    np.testing.assert_allclose(A.windowed_attention(q, k, v, 1), v, atol=0)
    # reading of the dense shortcut: window == S is NOT dense under the policy
    assert np.max(np.abs(A.windowed_attention(q, k, v, S) - full)) > 1e-3


def test_windowed_validation():
    x = _rand((1, 1, 8, 2), 40)
    for kw in (dict(window=0), dict(window=4, sink=-1), dict(window=4, sink=9), dict(window=4, chunk=0)):
        with pytest.raises(ValueError):
            A.windowed_attention(x, x, x, **kw)


def test_block_sparse_all_kept_equals_dense_and_diag_only_block1_is_v():
    q, k, v = (_rand((1, 2, 24, 8), 50 + i) for i in range(3))
    keep = np.ones((1, 2, 3, 3), bool)
    np.testing.assert_allclose(A.block_sparse_attention(q, k, v, keep, 8), _torch_sdpa(q, k, v), atol=1e-12)
    eye = np.broadcast_to(np.eye(24, dtype=bool), (1, 2, 24, 24))
    np.testing.assert_allclose(A.block_sparse_attention(q, k, v, eye, 1), v, atol=0)


def test_block_sparse_matches_library_with_expanded_mask_and_rows_agree():
    q, k, v = (_rand((1, 1, 32, 8), 60 + i) for i in range(3))
    rng = np.random.default_rng(61)
    keep = rng.random((4, 4)) < 0.4
    keep[np.arange(4), np.arange(4)] = True
    allowed = np.kron(keep, np.ones((8, 8), bool)).astype(bool)
    want = _torch_sdpa(q, k, v, allowed, scale=0.4)
    got = A.block_sparse_attention(q, k, v, keep[None, None], 8, scale=0.4)
    np.testing.assert_allclose(got, want, atol=1e-12)
    rows = np.array([0, 5, 17, 31])
    np.testing.assert_allclose(A.block_sparse_rows(q[0, 0], k[0, 0], v[0, 0], keep, 8, rows, 0.4),
                               want[0, 0, rows], atol=1e-12)
    wrows = A.window_rows(q[0, 0], k[0, 0], v[0, 0], rows, 6, 2, 0.4)
    np.testing.assert_allclose(wrows, A.windowed_attention(q, k, v, 6, 2, scale=0.4)[0, 0, rows], atol=1e-12)


def test_gathered_forms_match_the_library_on_all_rows():
    """The kept-block and window-slice forms against torch's SDPA with the full boolean mask."""
    S, D, block = 96, 8, 8
    q, k, v = (_rand((1, 1, S, D), 70 + i) for i in range(3))
    rng = np.random.default_rng(71)
    nb = S // block
    keep = rng.random((nb, nb)) < 0.35
    keep[np.arange(nb), np.arange(nb)] = True
    keep[3] = False
    keep[3, nb - 1] = True                          # a one-block row at the far end
    keep[5] = True                                  # a full row
    allowed = np.kron(keep, np.ones((block, block), bool)).astype(bool)
    want = _torch_sdpa(q, k, v, allowed, scale=0.3)[0, 0]
    rows = np.arange(S)
    got = A.block_sparse_rows_gathered(q[0, 0], k[0, 0], v[0, 0], keep, block, rows, 0.3)
    np.testing.assert_allclose(got, want, atol=1e-12)
    some = np.array([95, 0, 17, 40, 41, 3])         # unsorted, several per block
    got = A.block_sparse_rows_gathered(q[0, 0], k[0, 0], v[0, 0], keep, block, some, 0.3)
    np.testing.assert_allclose(got, want[some], atol=1e-12)
    # key validity: the same as masking those keys in the expanded block mask
    valid = np.random.default_rng(72).random(S) < 0.7
    allowed = np.kron(keep, np.ones((block, block), bool)).astype(bool) & valid[None, :]
    want = _torch_sdpa(q, k, v, allowed, scale=0.3)[0, 0]
    got = A.block_sparse_rows_gathered(q[0, 0], k[0, 0], v[0, 0], keep, block, rows, 0.3, key_valid=valid)
    np.testing.assert_allclose(got, want, atol=1e-12)
    keep[2] = False
    with pytest.raises(RuntimeError):
        A.block_sparse_rows_gathered(q[0, 0], k[0, 0], v[0, 0], keep, block, np.array([16]), 0.3)
    for window, sink, span in [(9, 3, 8), (30, 0, 16), (2, 96, 5), (400, 7, 64)]:
        i, j = np.arange(S)[:, None], np.arange(S)[None, :]
        allowed = (np.abs(i - j) <= window // 2) | (j < sink)
        want = _torch_sdpa(q, k, v, allowed, scale=0.3)[0, 0]
        got = A.window_rows_gathered(q[0, 0], k[0, 0], v[0, 0], rows, window, sink, 0.3, span)
        np.testing.assert_allclose(got, want, atol=1e-12)


def test_kept_block_flops():
    assert A.kept_block_flops(np.array([[81, 83]]), 64, 64, 128) == 164 * 4 * 64 * 64 * 128
