"""libbsa on the CPU: exported symbols, host helpers against the oracle, and
argument validation of the device calls (rejected before any launch).

No compute kernel is launched here.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import blocks as OB
from oracle import pipeline as OP
from oracle import tiling as OT

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")

bsa = pytest.importorskip("block_sparse_attention_permute_amd.bsa")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bsa.LIB_PATH):
        pytest.fail("libbsa.so is not built (run __graft_entry__.build())")
    return bsa.lib()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|int64_t|int)\s+(bsa_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) >= 16
    for n in names:
        assert hasattr(L, n), n
    assert sorted(bsa.EXPORTED) == names


def test_version_and_empty_error(L):
    assert bsa.bsa_version() >> 16 == bsa.ABI_MAJOR == 2
    assert isinstance(L.bsa_last_error(), bytes)


@pytest.mark.parametrize("grid,tile", [((2, 4, 4), (1, 2, 2)), ((8, 16, 16), (2, 4, 4)), ((20, 32, 48), (1, 8, 8)),
                                       ((20, 32, 48), (4, 4, 4)), ((32, 48, 80), (4, 4, 4)), ((3, 5, 7), (3, 1, 7)),
                                       ((1, 1, 9), (1, 1, 1))])
def test_tile_permutation_bit_exact(L, grid, tile):
    got = bsa.bsa_tile_permutation(*grid, tile)
    assert got.dtype == np.int32
    assert np.array_equal(got, OT.tile_permutation(grid, tile))
    assert np.array_equal(bsa.bsa_invert_permutation(got), OT.invert_permutation(got))


def test_tile_permutation_rejects(L):
    with pytest.raises(ValueError, match="does not divide"):
        bsa.bsa_tile_permutation(20, 32, 48, (16, 2, 2))
    with pytest.raises(ValueError):
        bsa.bsa_tile_permutation(0, 4, 4, (1, 1, 1))
    with pytest.raises(ValueError):
        bsa.bsa_invert_permutation(np.array([0, 2, 2], np.int32))
    with pytest.raises(ValueError):
        bsa.bsa_invert_permutation(np.array([0, 3, 1], np.int32))


def test_budget_matches_oracle(L):
    rng = np.random.default_rng(0)
    cases = [(0.17, 480), (0.10, 1920), (0.01, 10), (1.0, 7), (0.5, 1)]
    cases += [(float(rng.uniform(1e-4, 1.0)), int(rng.integers(1, 5000))) for _ in range(300)]
    for frac, n in cases:
        assert bsa.bsa_budget(frac, n) == OB.budget(frac, n), (frac, n)
    for bad in (0.0, -1.0, 1.5, float("nan")):
        with pytest.raises(ValueError):
            bsa.bsa_budget(bad, 10)
    with pytest.raises(ValueError):
        bsa.bsa_budget(0.5, 0)


@pytest.mark.parametrize("tg,rad", [((4, 4, 4), (1, 1, 1)), ((3, 5, 2), (1, 2, 0)), ((1, 1, 1), (1, 1, 1)),
                                    ((10, 16, 12), (1, 1, 1))])
def test_sliding_tile_lists_bit_exact(L, tg, rad):
    idx, cnt = bsa.bsa_sliding_tile_block_list(tg, rad)
    keep = OT.sliding_tile_keep(tg, rad)
    lists, ocnt = OB.keep_to_lists(keep)
    assert np.array_equal(cnt, ocnt)
    for i, li in enumerate(lists):
        assert np.array_equal(idx[i, :cnt[i]], li)
        assert np.all(idx[i, cnt[i]:] == -1)
    with pytest.raises(ValueError):
        bsa.bsa_sliding_tile_block_list(tg, rad, max_kept=int(cnt.max()) - 1)


@pytest.mark.parametrize("grid,tile", [((20, 32, 48), (16, 2, 2)), ((16, 45, 80), (1, 8, 8)), ((3, 5, 6), (2, 2, 4)),
                                       ((4, 8, 8), (2, 4, 4)), ((1, 1, 5), (2, 2, 2))])
def test_padded_permutation_bit_exact(L, grid, tile):
    got = bsa.bsa_tile_permutation_padded(*grid, tile)
    want = OT.padded_tile_permutation(grid, tile)
    assert bsa.bsa_padded_length(*grid, tile) == want.size == int(np.prod(OT.padded_grid(grid, tile)))
    assert np.array_equal(got, want)
    with pytest.raises(ValueError):
        bsa.bsa_padded_length(0, 4, 4, tile)


@pytest.mark.parametrize("grid,block,kind", [((5, 4, 4), 16, "temporal"), ((3, 4, 4), 8, "spatial"),
                                             ((20, 32, 48), 64, "temporal"), ((20, 32, 48), 64, "spatial"),
                                             ((3, 6, 5), 8, "padded")])
def test_label_block_lists_bit_exact(L, grid, block, kind):
    T, Hg, Wg = grid
    if kind == "spatial":
        lab = np.arange(T * Hg * Wg) // (Hg * Wg)
    elif kind == "temporal":
        lab = OT.tile_permutation(grid, (T, 1, 1)) % (Hg * Wg)
    else:   # padding labelled -1 never matches
        perm = OT.padded_tile_permutation(grid, (2, 2, 2))
        lab = np.where(perm >= 0, 0, -1)
    idx, cnt = bsa.bsa_label_block_list(lab, block)
    if lab.size <= 4096:
        keep = OP.label_block_keep(lab, block)
    else:   # the oracle's brute force over 480^2 block pairs, on the structure it must have
        nb = lab.size // block
        sets = [set(lab[i * block:(i + 1) * block].tolist()) for i in range(nb)]
        keep = np.array([[bool(sets[i] & sets[j]) for j in range(nb)] for i in range(nb)])
    lists, ocnt = OB.keep_to_lists(keep)
    assert np.array_equal(cnt, ocnt)
    for i, li in enumerate(lists):
        assert np.array_equal(idx[i, :cnt[i]], li)
    with pytest.raises(ValueError):
        bsa.bsa_label_block_list(lab, block, max_kept=int(cnt.max()) - 1)


@pytest.mark.parametrize("grid", [(2, 4, 4), (5, 4, 4), (3, 6, 5), (1, 7, 3), (6, 1, 1), (20, 32, 48)])
def test_video_labels_bit_exact(L, grid):
    """bsa_video_labels against the oracle's spatial-only and temporal-only masks: spatial labels in T-major
    order, temporal labels in the order of the tiling (T, 1, 1); equal labels exactly where the mask keeps."""
    from oracle import attention as OA
    T, Hg, Wg = grid
    S = T * Hg * Wg
    perm = OT.tile_permutation(grid, (T, 1, 1))
    sp = bsa.bsa_video_labels(grid, "spatial")
    tp = bsa.bsa_video_labels(grid, "temporal")
    assert sp.dtype == np.int32 and tp.dtype == np.int32 and sp.shape == tp.shape == (S,)
    if S <= 4096:
        ms = OA.spatial_only_mask(grid) == 0.0
        mt = (OA.temporal_only_mask(grid) == 0.0)[perm][:, perm]
        assert np.array_equal(sp[:, None] == sp[None, :], ms)
        assert np.array_equal(tp[:, None] == tp[None, :], mt)
        for lab in (sp, tp):                  # and their block lists equal the brute-force block rule
            for block in (b for b in (4, 8, 16) if S % b == 0):
                idx, cnt = bsa.bsa_label_block_list(lab, block)
                lists, ocnt = OB.keep_to_lists(OP.label_block_keep(lab, block))
                assert np.array_equal(cnt, ocnt)
                assert all(np.array_equal(idx[i, :cnt[i]], li) for i, li in enumerate(lists))
    else:                                     # the masks are S x S: compare with the rule they are built on
        assert np.array_equal(sp, np.arange(S) // (Hg * Wg))
        assert np.array_equal(tp, perm % (Hg * Wg))
    with pytest.raises(ValueError):
        bsa.bsa_video_labels(grid, "diagonal")
    assert L.bsa_video_labels(T, Hg, Wg, 2, (ctypes.c_int32 * S)()) == bsa.BSA_ERR_INVALID_ARG
    assert L.bsa_video_labels(0, Hg, Wg, 0, (ctypes.c_int32 * S)()) == bsa.BSA_ERR_INVALID_ARG


# --- argument validation of device calls: all rejected on the host --------

FAKE = ctypes.c_void_p(4096)  # never dereferenced: every case below fails validation first
TILES = (ctypes.c_int32 * 6)(1, 8, 8, 4, 4, 4)
BAD_TILES = (ctypes.c_int32 * 3)(16, 2, 2)
MIXED_TILES = (ctypes.c_int32 * 6)(1, 8, 8, 2, 4, 4)
K_TAB = (ctypes.c_int32 * 2)(81, 130)
NK_TAB = (ctypes.c_int32 * 2)(480, 768)
NK_BAD = (ctypes.c_int32 * 2)(480, 769)


def _rc(L, name, *args):
    rc = getattr(L, name)(*args)
    return rc, L.bsa_last_error().decode()


def test_device_calls_reject_bad_arguments(L):
    F, BF = bsa.BSA_F32, bsa.BSA_BF16
    cases = [
        ("bsa_tile_permute", (FAKE, ctypes.c_void_p(1 << 20), BF, 1, 40, 20, 32, 48, 128, BAD_TILES, 1, None, None),
         "does not divide"),
        ("bsa_tile_permute", (FAKE, ctypes.c_void_p(1 << 20), BF, 1, 40, 20, 32, 48, 128, TILES, 0, None, None),
         "n_tiles"),
        ("bsa_tile_permute", (FAKE, FAKE, BF, 1, 1, 8, 8, 8, 8, TILES, 1, None, None), "overlap"),
        ("bsa_invert_permute", (FAKE, ctypes.c_void_p(1 << 20), 7, 1, 1, 20, 32, 48, 128, TILES, 2, None, None),
         "dtype"),
        ("bsa_block_cohesion", (FAKE, BF, 1, 2, 100, 64, 64, FAKE, None), "divide"),
        ("bsa_select_tiling", (FAKE, BF, 1, 40, 20, 32, 48, 128, BAD_TILES, 1, FAKE, FAKE, FAKE, None), "divide"),
        ("bsa_minmax_block_scores", (FAKE, FAKE, BF, 1, 2, 100, 128, 64, FAKE, FAKE, None, None), "divide"),
        ("bsa_topk_block_mask", (FAKE, 1, 1, 480, 480, 0, 1, 1, FAKE, FAKE, 83, None, None), "k=0"),
        ("bsa_topk_block_mask", (FAKE, 1, 1, 480, 480, 481, 1, 1, FAKE, FAKE, 483, None, None), "k=481"),
        ("bsa_topk_block_mask", (FAKE, 1, 1, 480, 480, 81, 1, 1, FAKE, FAKE, 82, None, None), "max_kept"),
        ("bsa_topk_block_mask", (FAKE, 1, 1, 4, 5000, 81, 1, 1, FAKE, FAKE, 83, None, None), "Nk"),
        ("bsa_topk_block_mask", (FAKE, 1, 1, 480, 480, 81, 5, 40, FAKE, FAKE, 126, None, None), "max_kept"),
        ("bsa_topk_block_mask", (FAKE, 1, 1, 480, 480, 81, 1, -1, FAKE, FAKE, 83, None, None), "diag_width"),
        ("bsa_top_p_block_mask", (FAKE, 1, 1, 480, 480, ctypes.c_float(0.0), ctypes.c_float(1.0), 1, 1, FAKE, FAKE,
                                  480, None, None), "p="),
        ("bsa_top_p_block_mask", (FAKE, 1, 1, 480, 480, ctypes.c_float(1.5), ctypes.c_float(1.0), 1, 1, FAKE, FAKE,
                                  480, None, None), "p="),
        ("bsa_top_p_block_mask", (FAKE, 1, 1, 480, 480, ctypes.c_float(0.5), ctypes.c_float(0.0), 1, 1, FAKE, FAKE,
                                  480, None, None), "scale"),
        ("bsa_top_p_block_mask", (FAKE, 1, 1, 480, 480, ctypes.c_float(0.5), ctypes.c_float(1.0), 1, 1, FAKE, FAKE,
                                  479, None, None), "max_kept"),
        ("bsa_block_sparse_attention",
         (FAKE, FAKE, FAKE, FAKE, BF, 1, 1, 100, 128, 64, FAKE, FAKE, 8, ctypes.c_float(0.1), None, None, 0, None),
         "divide"),
        ("bsa_block_sparse_attention",
         (FAKE, FAKE, FAKE, FAKE, BF, 1, 1, 0, 128, 64, FAKE, FAKE, 8, ctypes.c_float(0.1), None, None, 0, None),
         "> 0"),
        ("bsa_block_sparse_attention",
         (FAKE, FAKE, FAKE, FAKE, BF, 1, 1, 128, 128, 64, FAKE, FAKE, 2, ctypes.c_float(0.1), None, FAKE, 0, None),
         "row_order_len"),
        ("bsa_block_sparse_attention_tiled",
         (FAKE, FAKE, FAKE, FAKE, BF, 1, 2, 20, 32, 48, 128, TILES, 2, None, FAKE, FAKE, 82, ctypes.c_float(0.1),
          None, FAKE, 1 << 31, None), "row_order_len"),
        ("bsa_row_order", (FAKE, 40, 480, FAKE, 19319, None), "order_len"),
        ("bsa_row_order", (None, 40, 480, FAKE, 19320, None), "NULL"),
        ("bsa_row_order", (FAKE, 0, 480, FAKE, 19320, None), "BH"),
        ("bsa_row_order_by_median", (FAKE, FAKE, 3, 5, 4, 5, FAKE, 15, None), "multiple of 8"),
        ("bsa_row_order_by_median", (None, FAKE, 1, 8, 4, 8, FAKE, 8, None), "NULL"),
        ("bsa_row_order_by_median", (FAKE, FAKE, 1, 8, 4, 4097, FAKE, 8, None), "Nk"),
        ("bsa_row_order_by_median", (FAKE, FAKE, 1, 8, 4, 8, FAKE, 7, None), "order_len"),
        ("bsa_row_order_by_median", (FAKE, FAKE, 1, 8, 0, 8, FAKE, 8, None), "max_kept"),
        ("bsa_row_order_by_median_ex", (FAKE, FAKE, 1, 8, 4, 8, -1, FAKE, 8, None), "head_kv_bytes"),
        ("bsa_row_order_by_median_ex", (FAKE, None, 1, 8, 4, 8, 0, FAKE, 8, None), "NULL"),
        ("bsa_row_order_by_median_ex", (FAKE, FAKE, 3, 5, 4, 5, 1 << 30, FAKE, 15, None), "multiple of 8"),
        ("bsa_windowed_attention", (FAKE, FAKE, FAKE, FAKE, F, 1, 1, 32, 16, 0, 2, ctypes.c_float(0.25), 8, None),
         "window"),
        ("bsa_windowed_attention", (FAKE, FAKE, FAKE, FAKE, F, 1, 1, 32, 16, 8, -1, ctypes.c_float(0.25), 8, None),
         "sink"),
        ("bsa_windowed_attention", (FAKE, FAKE, FAKE, FAKE, F, 1, 1, 32, 16, 8, 33, ctypes.c_float(0.25), 8, None),
         "exceed"),
        ("bsa_windowed_attention", (FAKE, FAKE, FAKE, FAKE, F, 1, 1, 32, 16, 8, 2, ctypes.c_float(0.25), -1, None),
         "chunk"),
        ("bsa_windowed_attention", (None, FAKE, FAKE, FAKE, F, 1, 1, 32, 16, 8, 2, ctypes.c_float(0.25), 8, None),
         "NULL"),
        ("bsa_validate_block_list", (FAKE, FAKE, 1, 1, 0, 4, 4, None), ">= 1"),
        ("bsa_select_tiling_ex", (FAKE, BF, 1, 40, 20, 32, 48, 128, TILES, 2, 7, 0, FAKE, FAKE, FAKE, None, None),
         "statistic"),
        ("bsa_select_tiling_ex", (FAKE, BF, 1, 40, 20, 32, 48, 128, BAD_TILES, 1, 0, 0, FAKE, FAKE, FAKE, None,
                                  None),
         "divide"),
        ("bsa_select_tiling_ex", (FAKE, BF, 1, 40, 20, 32, 48, 128, TILES, 2, 0, 2, FAKE, FAKE, FAKE, None, None),
         "pad"),
        ("bsa_select_tiling_ex", (FAKE, BF, 1, 40, 20, 32, 48, 128, TILES, 2, 0, 1, FAKE, FAKE, FAKE, FAKE, None),
         "pad = 0"),
        ("bsa_select_tiling_ex", (FAKE, BF, 1, 40, 20, 32, 48, 128, MIXED_TILES, 2, 0, 0, FAKE, FAKE, FAKE, FAKE,
                                  None), "one volume"),
        ("bsa_tile_permute_padded", (FAKE, ctypes.c_void_p(1 << 30), BF, 1, 40, 20, 32, 48, 128, BAD_TILES, 1, None,
                                     30720, None, None), "shorter"),
        ("bsa_tile_permute_padded", (FAKE, ctypes.c_void_p(1 << 30), BF, 1, 40, 20, 32, 48, 128, BAD_TILES, 1, None,
                                     0, None, None), "Sp"),
        ("bsa_invert_permute_padded", (FAKE, ctypes.c_void_p(1 << 30), BF, 1, 40, 20, 32, 48, 128, BAD_TILES, 1,
                                       None, 40000, None), "shorter"),
        ("bsa_minmax_block_scores_masked", (FAKE, FAKE, BF, 1, 2, 100, 128, 64, FAKE, FAKE, FAKE, None, None),
         "divide"),
        ("bsa_topk_block_mask_tiled", (FAKE, 1, 1, 768, 768, FAKE, K_TAB, NK_BAD, 2, 1, 1, FAKE, FAKE, 140, None,
                                       None), "nk_table"),
        ("bsa_topk_block_mask_tiled", (FAKE, 1, 1, 768, 768, FAKE, K_TAB, NK_TAB, 2, 1, 1, FAKE, FAKE, 100, None,
                                       None), "max_kept"),
        ("bsa_block_sparse_attention_labels",
         (FAKE, FAKE, FAKE, FAKE, BF, 1, 1, 128, 128, 64, FAKE, FAKE, 2, FAKE, 5, ctypes.c_float(0.1), None),
         "stride"),
        ("bsa_block_sparse_attention_labels",
         (FAKE, FAKE, FAKE, FAKE, BF, 1, 1, 128, 128, 64, FAKE, FAKE, 2, None, 0, ctypes.c_float(0.1), None),
         "NULL"),
        ("bsa_validate_indices", (None, 4, 0, 3, None), "NULL"),
    ]
    for name, args, needle in cases:
        rc, msg = _rc(L, name, *args)
        assert rc == bsa.BSA_ERR_INVALID_ARG, (name, rc, msg)
        assert needle in msg, (name, msg)


def test_row_order_len(L):
    """Plan length = 8 XCDs x ceil(U/8) units of U x rows per unit, plus 3U scratch words."""
    assert bsa.bsa_row_order_len(40, 480) == 8 * 5 * 480 + 3 * 40    # whole heads: no empty slot
    assert bsa.bsa_row_order_len(24, 1920) == 8 * 3 * 1920 + 3 * 24
    assert bsa.bsa_row_order_len(6, 64) == 8 * 3 * 16 + 3 * 24       # 24 units: a quarter head each
    assert bsa.bsa_row_order_len(1, 480) == 8 * 1 * 60 + 3 * 8       # 8 units of 60 rows
    assert bsa.bsa_row_order_len(2, 7) == 8 * 1 * 7 + 3 * 2          # 7 rows do not split: whole heads
    assert bsa.bsa_row_order_len(1024, 3) == 8 * 128 * 3 + 3 * 1024
    assert bsa.bsa_row_order_len(5, 12) == 8 * 3 * 3 + 3 * 20        # 20 units of 3 rows
    for bh, nq in [(40, 480), (6, 64), (1, 1), (3, 5), (41, 480)]:
        assert bsa.bsa_row_order_len(bh, nq) >= bh * nq
    for bh, nq in [(0, 4), (4, 0), (1025, 1), (1 << 16, 1 << 15)]:
        with pytest.raises(ValueError):
            bsa.bsa_row_order_len(bh, nq)


def test_unaligned_tensors_rejected(L):
    rc, msg = _rc(L, "bsa_windowed_attention", ctypes.c_void_p(4098), FAKE, FAKE, FAKE, bsa.BSA_F32, 1, 1, 32, 16, 8,
                  2, ctypes.c_float(0.25), 8, None)
    assert rc == bsa.BSA_ERR_INVALID_ARG and "aligned" in msg


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(bsa, "_lib", None)
    monkeypatch.setattr(bsa, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        bsa.bsa_budget(0.5, 10)
