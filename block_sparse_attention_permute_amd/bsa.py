"""Python binding of libbsa (ctypes): argument marshalling only.

Every function has the name of the C entry point it calls.  Tensors are torch
tensors on the current HIP device (torch provides device memory and the
stream); every step of the computation runs in libbsa's kernels.  Status codes
map to exceptions: BSA_ERR_INVALID_ARG -> ValueError, BSA_ERR_INVARIANT ->
RuntimeError, BSA_ERR_UNSUPPORTED -> UnsupportedError (a ValueError),
BSA_ERR_DEVICE -> RuntimeError.

The library must be built (``python -m block_sparse_attention_permute_amd.build``);
there is no fallback: without libbsa.so every call raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsa.so")

BSA_OK, BSA_ERR_INVALID_ARG, BSA_ERR_INVARIANT, BSA_ERR_UNSUPPORTED, BSA_ERR_DEVICE = range(5)
BSA_F32, BSA_BF16 = 0, 1
BSA_STAT_MEAN, BSA_STAT_POOLED = 0, 1
BSA_LABEL_SPATIAL, BSA_LABEL_TEMPORAL = 0, 1
BSA_MAX_TILINGS = 8
BSA_NOALLOC_TILE_VALUES = 1 << 20

EXPORTED = (
    "bsa_last_error", "bsa_version", "bsa_tile_permutation", "bsa_invert_permutation", "bsa_budget",
    "bsa_sliding_tile_block_list", "bsa_tile_permute", "bsa_invert_permute", "bsa_block_cohesion",
    "bsa_select_tiling", "bsa_minmax_block_scores", "bsa_topk_block_mask", "bsa_top_p_block_mask",
    "bsa_block_sparse_attention", "bsa_padded_length", "bsa_tile_permutation_padded", "bsa_label_block_list",
    "bsa_tile_permute_padded", "bsa_invert_permute_padded", "bsa_select_tiling_ex",
    "bsa_minmax_block_scores_masked", "bsa_topk_block_mask_tiled", "bsa_block_sparse_attention_labels",
    "bsa_minmax_block_scores_tiled", "bsa_block_sparse_attention_tiled",
    "bsa_windowed_attention", "bsa_validate_block_list", "bsa_validate_indices", "bsa_video_labels",
    "bsa_select_tiling_noalloc", "bsa_temporal_only_attention", "bsa_block_sparse_attention_tiled_padded",
    "bsa_tiled_attention_supported", "bsa_row_order", "bsa_row_order_len", "bsa_row_order_by_median", "bsa_minmax_block_scores_tiled_padded",
    "bsa_row_order_by_median_ex",
)


class UnsupportedError(ValueError):
    """A valid request that libbsa has no kernel for."""


_lib = None

_P, _I, _I64, _F, _D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double
_SIGS = {
    "bsa_last_error": (ctypes.c_char_p, []),
    "bsa_version": (_I, []),
    "bsa_tile_permutation": (_I, [_I, _I, _I, _I, _I, _I, _P]),
    "bsa_invert_permutation": (_I, [_P, _I64, _P]),
    "bsa_budget": (_I, [_D, _I]),
    "bsa_sliding_tile_block_list": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _I]),
    "bsa_tile_permute": (_I, [_P, _P, _I, _I64, _I64, _I, _I, _I, _I64, _P, _I, _P, _P]),
    "bsa_invert_permute": (_I, [_P, _P, _I, _I64, _I64, _I, _I, _I, _I64, _P, _I, _P, _P]),
    "bsa_block_cohesion": (_I, [_P, _I, _I64, _I64, _I64, _I64, _I, _P, _P]),
    "bsa_select_tiling": (_I, [_P, _I, _I64, _I64, _I, _I, _I, _I64, _P, _I, _P, _P, _P, _P]),
    "bsa_select_tiling_noalloc": (_I, [_P, _I, _I64, _I64, _I, _I, _I, _I64, _P, _I, _P, _P, _P]),
    "bsa_minmax_block_scores": (_I, [_P, _P, _I, _I64, _I64, _I64, _I64, _I, _P, _P, _P, _P]),
    "bsa_topk_block_mask": (_I, [_P, _I64, _I64, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P]),
    "bsa_top_p_block_mask": (_I, [_P, _I64, _I64, _I, _I, _F, _F, _I, _I, _P, _P, _I, _P, _P]),
    "bsa_block_sparse_attention": (_I, [_P, _P, _P, _P, _I, _I64, _I64, _I64, _I64, _I, _P, _P, _I, _F, _P, _P,
                                        _I64, _P]),
    "bsa_windowed_attention": (_I, [_P, _P, _P, _P, _I, _I64, _I64, _I64, _I64, _I, _I, _F, _I, _P]),
    "bsa_temporal_only_attention": (_I, [_P, _P, _P, _P, _I, _I64, _I64, _I, _I, _I, _I64, _F, _P]),
    "bsa_validate_block_list": (_I, [_P, _P, _I64, _I64, _I, _I, _I, _P]),
    "bsa_validate_indices": (_I, [_P, _I64, _I, _I, _P]),
    "bsa_padded_length": (_I64, [_I, _I, _I, _I, _I, _I]),
    "bsa_tile_permutation_padded": (_I, [_I, _I, _I, _I, _I, _I, _P]),
    "bsa_label_block_list": (_I, [_P, _I64, _I, _P, _P, _I]),
    "bsa_video_labels": (_I, [_I, _I, _I, _I, _P]),
    "bsa_tile_permute_padded": (_I, [_P, _P, _I, _I64, _I64, _I, _I, _I, _I64, _P, _I, _P, _I64, _P, _P]),
    "bsa_invert_permute_padded": (_I, [_P, _P, _I, _I64, _I64, _I, _I, _I, _I64, _P, _I, _P, _I64, _P]),
    "bsa_select_tiling_ex": (_I, [_P, _I, _I64, _I64, _I, _I, _I, _I64, _P, _I, _I, _I, _P, _P, _P, _P, _P]),
    "bsa_minmax_block_scores_masked": (_I, [_P, _P, _I, _I64, _I64, _I64, _I64, _I, _P, _P, _P, _P, _P]),
    "bsa_topk_block_mask_tiled": (_I, [_P, _I64, _I64, _I, _I, _P, _P, _P, _I, _I, _I, _P, _P, _I, _P, _P]),
    "bsa_block_sparse_attention_labels": (_I, [_P, _P, _P, _P, _I, _I64, _I64, _I64, _I64, _I, _P, _P, _I, _P,
                                               _I64, _F, _P]),
    "bsa_minmax_block_scores_tiled": (_I, [_P, _P, _I, _I64, _I64, _I, _I, _I, _I64, _P, _I, _P, _P, _P, _P, _P,
                                           _P]),
    "bsa_block_sparse_attention_tiled": (_I, [_P, _P, _P, _P, _I, _I64, _I64, _I, _I, _I, _I64, _P, _I, _P, _P, _P,
                                              _I, _F, _P, _P, _I64, _P]),
    "bsa_block_sparse_attention_tiled_padded": (_I, [_P, _P, _P, _P, _I, _I64, _I64, _I, _I, _I, _I64, _P, _I, _P,
                                                     _P, _P, _I, _F, _P, _P, _I64, _P]),
    "bsa_tiled_attention_supported": (_I, [_I, _I64, _I, _I, _I, _P, _I, _I]),
    "bsa_row_order": (_I, [_P, _I64, _I64, _P, _I64, _P]),
    "bsa_minmax_block_scores_tiled_padded": (_I, [_P, _P, _I, _I64, _I64, _I, _I, _I, _I64, _P, _I, _P, _P, _P, _P,
                                                  _P]),
    "bsa_row_order_len": (_I64, [_I64, _I64]),
    "bsa_row_order_by_median": (_I, [_P, _P, _I64, _I64, _I, _I64, _P, _I64, _P]),
    "bsa_row_order_by_median_ex": (_I, [_P, _P, _I64, _I64, _I, _I64, _I64, _P, _I64, _P]),
}

# libbsa's ABI major version these signatures are written for
ABI_MAJOR = 2


def lib() -> ctypes.CDLL:
    """Load libbsa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_attention_permute_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        if L.bsa_version() >> 16 != ABI_MAJOR:
            raise RuntimeError(f"{LIB_PATH} has ABI {L.bsa_version() >> 16}, this binding needs {ABI_MAJOR}: rebuild it")
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc == BSA_OK:
        return
    msg = lib().bsa_last_error().decode(errors="replace")
    if rc == BSA_ERR_INVALID_ARG:
        raise ValueError(msg)
    if rc == BSA_ERR_UNSUPPORTED:
        raise UnsupportedError(msg)
    if rc == BSA_ERR_INVARIANT:
        raise RuntimeError(msg)
    raise RuntimeError(f"device error: {msg}")


# ----------------------------------------------------------------- helpers --

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BSA_BF16
    if t.dtype == torch.float32:
        return BSA_F32
    raise ValueError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _dev(t, name="tensor"):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _bhsd(t, name="tensor"):
    if t.dim() != 4:
        raise ValueError(f"{name} must be rank 4 (B, H, S, D); got {tuple(t.shape)}")
    return tuple(int(s) for s in t.shape)


def _stream(t):
    return _torch().cuda.current_stream(t.device).cuda_stream


def _tiles_arr(tiles):
    tiles = [tuple(int(v) for v in t) for t in tiles]
    if not tiles or any(len(t) != 3 for t in tiles):
        raise ValueError("tiles must be a non-empty list of (a, b, c)")
    arr = (ctypes.c_int32 * (3 * len(tiles)))(*[v for t in tiles for v in t])
    return arr, len(tiles)


def _scale(scale):
    return float("nan") if scale is None else float(scale)


# ------------------------------------------------------------ host calls ---

def bsa_version() -> int:
    return int(lib().bsa_version())


def bsa_tile_permutation(T: int, Hg: int, Wg: int, tile) -> np.ndarray:
    """Host: tile-contiguous order, perm[p] = source token of position p."""
    a, b, c = (int(v) for v in tile)
    S = max(int(T) * int(Hg) * int(Wg), 1)
    out = np.empty(S, dtype=np.int32)
    _check(lib().bsa_tile_permutation(int(T), int(Hg), int(Wg), a, b, c, out.ctypes.data))
    return out


def bsa_invert_permutation(perm) -> np.ndarray:
    perm = np.ascontiguousarray(perm, dtype=np.int32)
    inv = np.empty_like(perm)
    _check(lib().bsa_invert_permutation(perm.ctypes.data, perm.size, inv.ctypes.data))
    return inv


def bsa_budget(frac: float, n_blocks: int) -> int:
    k = int(lib().bsa_budget(float(frac), int(n_blocks)))
    if k < 0:
        raise ValueError(lib().bsa_last_error().decode())
    return k


def bsa_sliding_tile_block_list(tile_grid, radius=(1, 1, 1), max_kept: int | None = None):
    """Host: (kv_idx int32 (N, max_kept), kv_cnt int32 (N,)) of the clipped sliding-tile mask."""
    nt, nh, nw = (int(v) for v in tile_grid)
    rt, rh, rw = (int(v) for v in radius)
    if max_kept is None:
        max_kept = min(nt, 2 * rt + 1) * min(nh, 2 * rh + 1) * min(nw, 2 * rw + 1)
    n = max(nt * nh * nw, 1)
    idx = np.empty((n, max(int(max_kept), 1)), dtype=np.int32)
    cnt = np.empty(n, dtype=np.int32)
    _check(lib().bsa_sliding_tile_block_list(nt, nh, nw, rt, rh, rw, idx.ctypes.data, cnt.ctypes.data,
                                             int(max_kept)))
    return idx, cnt


def bsa_padded_length(T: int, Hg: int, Wg: int, tile) -> int:
    """Host: length of the grid padded up to a multiple of the tile."""
    a, b, c = (int(v) for v in tile)
    n = int(lib().bsa_padded_length(int(T), int(Hg), int(Wg), a, b, c))
    if n < 0:
        raise ValueError(lib().bsa_last_error().decode())
    return n


def bsa_tile_permutation_padded(T: int, Hg: int, Wg: int, tile) -> np.ndarray:
    """Host: tile order of the padded grid, the real token of each position or -1."""
    a, b, c = (int(v) for v in tile)
    out = np.empty(max(bsa_padded_length(T, Hg, Wg, tile), 1), dtype=np.int32)
    _check(lib().bsa_tile_permutation_padded(int(T), int(Hg), int(Wg), a, b, c, out.ctypes.data))
    return out


def bsa_video_labels(grid, kind: str) -> np.ndarray:
    """Host: int32 (S,) labels of spatial-only ("spatial", T-major order) or temporal-only ("temporal",
    the order of the tiling (T, 1, 1)) attention."""
    T, Hg, Wg = (int(g) for g in grid)
    codes = {"spatial": BSA_LABEL_SPATIAL, "temporal": BSA_LABEL_TEMPORAL}
    if kind not in codes:
        raise ValueError(f"kind must be 'spatial' or 'temporal', got {kind!r}")
    out = np.empty(max(T * Hg * Wg, 1), dtype=np.int32)
    _check(lib().bsa_video_labels(T, Hg, Wg, codes[kind], out.ctypes.data))
    return out


def bsa_label_block_list(labels, block: int, max_kept: int | None = None):
    """Host: (kv_idx int32 (Nb, max_kept), kv_cnt int32 (Nb,)) keeping blocks that share a label."""
    lab = np.ascontiguousarray(labels, dtype=np.int32).ravel()
    S = lab.size
    if block < 1 or S % block:
        raise ValueError(f"block {block} must divide S={S}")
    nb = S // block
    mk = nb if max_kept is None else int(max_kept)
    idx = np.empty((nb, max(mk, 1)), dtype=np.int32)
    cnt = np.empty(nb, dtype=np.int32)
    _check(lib().bsa_label_block_list(lab.ctypes.data, S, int(block), idx.ctypes.data, cnt.ctypes.data, mk))
    if max_kept is None:
        idx = np.ascontiguousarray(idx[:, :max(int(cnt.max()), 1)])
    return idx, cnt


# ---------------------------------------------------------- device calls ---

def _permute(fn, x, grid, tiles, head_choice, out):
    torch = _torch()
    B, H, S, D = _bhsd(x, "x")
    T, Hg, Wg = (int(g) for g in grid)
    if T * Hg * Wg != S:
        raise ValueError(f"grid {tuple(grid)} does not match S={S}")
    arr, n = _tiles_arr(tiles)
    y = torch.empty_like(x) if out is None else out
    if y.shape != x.shape or y.dtype != x.dtype:
        raise ValueError("out must match x")
    hc = None
    if head_choice is not None:
        if head_choice.dtype != torch.int32 or head_choice.numel() != B * H:
            raise ValueError("head_choice must be int32 with B*H entries")
        hc = _dev(head_choice, "head_choice")
    _check(fn(_dev(x, "x"), _dev(y, "out"), _dtype_code(x), B, H, T, Hg, Wg, D, arr, n, hc, _stream(x)))
    return y


def bsa_tile_permute(x, grid, tiles, head_choice=None, out=None):
    """y[b,h,p,:] = x[b,h,perm_c[p],:] with c = head_choice[b,h] (0 if None)."""
    return _permute(lib().bsa_tile_permute, x, grid, tiles, head_choice, out)


def bsa_invert_permute(y, grid, tiles, head_choice=None, out=None):
    """x[b,h,perm_c[p],:] = y[b,h,p,:] (back to T-major order)."""
    return _permute(lib().bsa_invert_permute, y, grid, tiles, head_choice, out)


def padded_rows(grid, tiles) -> int:
    """Rows per head of a padded permutation covering every candidate."""
    T, Hg, Wg = (int(g) for g in grid)
    return max(bsa_padded_length(T, Hg, Wg, t) for t in tiles)


def bsa_tile_permute_padded(x, grid, tiles, head_choice=None, Sp=None, out=None, labels=True):
    """Padded tile order -> (y (B, H, Sp, D) with zero padding rows, labels int32 (B, H, Sp) or None)."""
    torch = _torch()
    B, H, S, D = _bhsd(x, "x")
    T, Hg, Wg = (int(g) for g in grid)
    if T * Hg * Wg != S:
        raise ValueError(f"grid {tuple(grid)} does not match S={S}")
    arr, n = _tiles_arr(tiles)
    Sp = padded_rows(grid, tiles) if Sp is None else int(Sp)
    if out is None:
        y = torch.empty((B, H, Sp, D), dtype=x.dtype, device=x.device)
        lab = torch.empty((B, H, Sp), dtype=torch.int32, device=x.device) if labels else None
    else:
        y, lab = out
    if tuple(y.shape) != (B, H, Sp, D) or y.dtype != x.dtype:
        raise ValueError("out must be (B, H, Sp, D) of x's dtype")
    hc = None
    if head_choice is not None:
        if head_choice.dtype != torch.int32 or head_choice.numel() != B * H:
            raise ValueError("head_choice must be int32 with B*H entries")
        hc = _dev(head_choice, "head_choice")
    _check(lib().bsa_tile_permute_padded(_dev(x, "x"), _dev(y, "out"), _dtype_code(x), B, H, T, Hg, Wg, D, arr, n,
                                         hc, Sp, None if lab is None else _dev(lab, "labels"), _stream(x)))
    return y, lab


def bsa_invert_permute_padded(y, grid, tiles, head_choice=None, out=None):
    """Back to T-major order, padding rows dropped -> (B, H, S, D)."""
    torch = _torch()
    B, H, Sp, D = _bhsd(y, "y")
    T, Hg, Wg = (int(g) for g in grid)
    arr, n = _tiles_arr(tiles)
    x = torch.empty((B, H, T * Hg * Wg, D), dtype=y.dtype, device=y.device) if out is None else out
    hc = None
    if head_choice is not None:
        if head_choice.dtype != torch.int32 or head_choice.numel() != B * H:
            raise ValueError("head_choice must be int32 with B*H entries")
        hc = _dev(head_choice, "head_choice")
    _check(lib().bsa_invert_permute_padded(_dev(y, "y"), _dev(x, "out"), _dtype_code(y), B, H, T, Hg, Wg, D, arr, n,
                                           hc, Sp, _stream(y)))
    return x


def bsa_block_cohesion(x, block: int):
    """Cohesion of each run of `block` tokens -> float32 (B, H, S // block)."""
    torch = _torch()
    B, H, S, D = _bhsd(x, "x")
    if block < 1 or S % block:
        raise ValueError(f"block {block} must divide S={S}")
    coh = torch.empty((B, H, S // block), dtype=torch.float32, device=x.device)
    _check(lib().bsa_block_cohesion(_dev(x, "x"), _dtype_code(x), B, H, S, D, int(block), _dev(coh), _stream(x)))
    return coh


def bsa_select_tiling(q, grid, tiles, workspace=None, statistic: str = "mean", pad: bool = False,
                      q_summaries=None):
    """Per-head tiling choice -> (choice int32 (B, H), score float32 (B, H, n), tile_coh).

    statistic "mean" (per-tile cohesion averaged) or "pooled" (SPADE's engine
    rule); pad=True scores candidates that do not divide the grid on the
    zero-padded grid.  q_summaries: None, or a (n, 2, B, H, S // volume, D)
    tensor of q's dtype that receives every candidate's block max and min of
    q (candidates of one volume, pad=False), for bsa_minmax_block_scores_tiled."""
    torch = _torch()
    B, H, S, D = _bhsd(q, "q")
    T, Hg, Wg = (int(g) for g in grid)
    if T * Hg * Wg != S:
        raise ValueError(f"grid {tuple(grid)} does not match S={S}")
    if statistic not in ("mean", "pooled"):
        raise ValueError(f"unknown statistic {statistic!r}")
    arr, n = _tiles_arr(tiles)
    if pad:
        max_nb = max(bsa_padded_length(T, Hg, Wg, t) // max(t[0] * t[1] * t[2], 1) for t in tiles)
    else:
        max_nb = max(S // max(a * b * c, 1) for a, b, c in tiles)
    if workspace is None:
        tile_coh = torch.empty((B, H, n, max_nb), dtype=torch.float32, device=q.device)
        score = torch.empty((B, H, n), dtype=torch.float32, device=q.device)
        choice = torch.empty((B, H), dtype=torch.int32, device=q.device)
    else:
        tile_coh, score, choice = workspace
        if tile_coh.numel() < B * H * n * max_nb:
            raise ValueError("tile_coh workspace too small")
    stat = BSA_STAT_POOLED if statistic == "pooled" else BSA_STAT_MEAN
    qs = None if q_summaries is None else _q_summaries_arg(q_summaries, q, tiles, S, "q_summaries")
    _check(lib().bsa_select_tiling_ex(_dev(q, "q"), _dtype_code(q), B, H, T, Hg, Wg, D, arr, n, stat, int(bool(pad)),
                                      _dev(tile_coh), _dev(score), _dev(choice), qs, _stream(q)))
    return choice, score, tile_coh


def bsa_select_tiling_noalloc(q, grid, tiles, out):
    """bsa_select_tiling with no workspace and no allocation: out = (choice int32 (B, H), score float32
    (B, H, n)), both caller-allocated, are written and returned.  The per-tile values live in a fixed
    array inside libbsa (BSA_NOALLOC_TILE_VALUES floats per device); calls that overlap on one device race."""
    torch = _torch()
    B, H, S, D = _bhsd(q, "q")
    T, Hg, Wg = (int(g) for g in grid)
    if T * Hg * Wg != S:
        raise ValueError(f"grid {tuple(grid)} does not match S={S}")
    arr, n = _tiles_arr(tiles)
    choice, score = out
    if choice.dtype != torch.int32 or choice.numel() != B * H:
        raise ValueError("choice must be int32 with B*H entries")
    if score.dtype != torch.float32 or score.numel() != B * H * n:
        raise ValueError("score must be float32 with B*H*n entries")
    _check(lib().bsa_select_tiling_noalloc(_dev(q, "q"), _dtype_code(q), B, H, T, Hg, Wg, D, arr, n,
                                           _dev(score, "score"), _dev(choice, "choice"), _stream(q)))
    return choice, score


def _q_summaries_arg(t, q, tiles, S, what):
    """Device pointer of a (n, 2, B, H, S // volume, D) q-summary tensor of q's dtype and device."""
    B, H, _, D = (int(x) for x in q.shape)
    vol = int(tiles[0][0]) * int(tiles[0][1]) * int(tiles[0][2])
    want = (len(tiles), 2, B, H, S // max(vol, 1), D)
    if tuple(t.shape) != want or t.dtype != q.dtype or t.device != q.device or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous {q.dtype} tensor of shape {want} on {q.device}")
    return _dev(t, what)


def _norms_out(key_norms, B, H, nb, like):
    """Pointer of an optional float32 (B, H, nb) key-norm tensor (None: not written / not used)."""
    if key_norms is None:
        return None
    torch = _torch()
    if key_norms.dtype != torch.float32 or tuple(key_norms.shape) != (B, H, nb):
        raise ValueError(f"key_norms must be float32 {(B, H, nb)}")
    if key_norms.device != like.device:
        raise ValueError("key_norms must be on the tensors' device")
    return _dev(key_norms, "key_norms")


def bsa_minmax_block_scores(q, k, block: int, out=None, labels=None, key_norms=None):
    """-> (scores float32 (B, H, Nb, Nb), summaries (4, B, H, Nb, D): qmax, qmin, kmax, kmin).

    labels: int32 (B, H, S) or None; tokens labelled < 0 are left out.
    key_norms: float32 (B, H, Nb) or None; when given it receives each key
    block's largest row L2 norm (for bsa_block_sparse_attention)."""
    torch = _torch()
    B, H, S, D = _bhsd(q, "q")
    if _bhsd(k, "k") != (B, H, S, D) or k.dtype != q.dtype:
        raise ValueError("q and k must match")
    if block < 1 or S % block:
        raise ValueError(f"block {block} must divide S={S}")
    nb = S // block
    if out is None:
        scores = torch.empty((B, H, nb, nb), dtype=torch.float32, device=q.device)
        summ = torch.empty((4, B, H, nb, D), dtype=q.dtype, device=q.device)
    else:
        scores, summ = out
    kn = _norms_out(key_norms, B, H, nb, q)
    if labels is None:
        _check(lib().bsa_minmax_block_scores(_dev(q, "q"), _dev(k, "k"), _dtype_code(q), B, H, S, D, int(block),
                                             _dev(summ), _dev(scores), kn, _stream(q)))
    else:
        if labels.dtype != torch.int32 or tuple(labels.shape) != (B, H, S):
            raise ValueError("labels must be int32 (B, H, S)")
        _check(lib().bsa_minmax_block_scores_masked(_dev(q, "q"), _dev(k, "k"), _dtype_code(q), B, H, S, D,
                                                    int(block), _dev(labels, "labels"), _dev(summ), _dev(scores),
                                                    kn, _stream(q)))
    return scores, summ


def bsa_minmax_block_scores_tiled(q, k, grid, tiles, head_choice=None, out=None, key_norms=None, q_summaries=None):
    """Min/max block scores of T-major q, k, block J = tile J of each head's tiling (key_norms as in
    bsa_minmax_block_scores).  q_summaries: None, or what bsa_select_tiling(..., q_summaries=) wrote for
    the same q and tiles; q is then not read again."""
    torch = _torch()
    B, H, S, D = _bhsd(q, "q")
    if _bhsd(k, "k") != (B, H, S, D) or k.dtype != q.dtype:
        raise ValueError("q and k must match")
    T, Hg, Wg = (int(g) for g in grid)
    if T * Hg * Wg != S:
        raise ValueError(f"grid {tuple(grid)} does not match S={S}")
    arr, n = _tiles_arr(tiles)
    block = tiles[0][0] * tiles[0][1] * tiles[0][2]
    nb = S // block
    if out is None:
        scores = torch.empty((B, H, nb, nb), dtype=torch.float32, device=q.device)
        summ = torch.empty((4, B, H, nb, D), dtype=q.dtype, device=q.device)
    else:
        scores, summ = out
    hc = None if head_choice is None else _dev(head_choice, "head_choice")
    kn = _norms_out(key_norms, B, H, nb, q)
    qs = None if q_summaries is None else _q_summaries_arg(q_summaries, q, tiles, S, "q_summaries")
    _check(lib().bsa_minmax_block_scores_tiled(_dev(q, "q"), _dev(k, "k"), _dtype_code(q), B, H, T, Hg, Wg, D, arr,
                                               n, hc, _dev(summ), _dev(scores), kn, qs, _stream(q)))
    return scores, summ


def bsa_minmax_block_scores_tiled_padded(q, k, grid, tiles, head_choice=None, out=None, key_norms=None):
    """Min/max block scores of T-major q, k on each head's grid padded along T (block J = tile J of the head's
    padded tiling; padding cells left out, unread) -> (scores (B, H, Nb, Nb), summaries (4, B, H, Nb, D)), Nb =
    the largest padded block count (padded_rows(grid, tiles) // block).  key_norms as in bsa_minmax_block_scores."""
    torch = _torch()
    B, H, S, D = _bhsd(q, "q")
    if _bhsd(k, "k") != (B, H, S, D) or k.dtype != q.dtype:
        raise ValueError("q and k must match")
    T, Hg, Wg = (int(g) for g in grid)
    if T * Hg * Wg != S:
        raise ValueError(f"grid {tuple(grid)} does not match S={S}")
    arr, n = _tiles_arr(tiles)
    block = tiles[0][0] * tiles[0][1] * tiles[0][2]
    nb = padded_rows(grid, tiles) // block
    if out is None:
        scores = torch.empty((B, H, nb, nb), dtype=torch.float32, device=q.device)
        summ = torch.empty((4, B, H, nb, D), dtype=q.dtype, device=q.device)
    else:
        scores, summ = out
    hc = None if head_choice is None else _dev(head_choice, "head_choice")
    kn = _norms_out(key_norms, B, H, nb, q)
    _check(lib().bsa_minmax_block_scores_tiled_padded(_dev(q, "q"), _dev(k, "k"), _dtype_code(q), B, H, T, Hg, Wg, D,
                                                      arr, n, hc, _dev(summ), _dev(scores), kn, _stream(q)))
    return scores, summ


def _band(diag_width) -> int:
    """Diagonal band width: True/False mean 1/0 (the diagonal alone / none)."""
    w = int(diag_width)
    if w < 0:
        raise ValueError(f"diag_width must be >= 0, got {diag_width}")
    return w


def _band_blocks(w: int) -> int:
    return 2 * (w // 2) + 1 if w >= 1 else 0


def _select_out(scores, max_kept, return_mask, out):
    torch = _torch()
    B, H, Nq, Nk = (int(s) for s in scores.shape)
    if out is None:
        kv_idx = torch.empty((B, H, Nq, max_kept), dtype=torch.int32, device=scores.device)
        kv_cnt = torch.empty((B, H, Nq), dtype=torch.int32, device=scores.device)
        mask = torch.empty((B, H, Nq, Nk), dtype=torch.uint8, device=scores.device) if return_mask else None
        return kv_idx, kv_cnt, mask
    return out


def bsa_topk_block_mask(scores, k: int, sink_blocks: int = 1, keep_diag=True,
                        max_kept: int | None = None, return_mask: bool = False, out=None):
    """-> (kv_idx int32 (B, H, Nq, max_kept), kv_cnt int32 (B, H, Nq)[, mask uint8 (B, H, Nq, Nk)]).

    ``keep_diag`` is the diagonal band width (True = 1, the diagonal alone)."""
    torch = _torch()
    if scores.dim() != 4 or scores.dtype != torch.float32:
        raise ValueError("scores must be float32 (B, H, Nq, Nk)")
    B, H, Nq, Nk = (int(s) for s in scores.shape)
    w = _band(keep_diag)
    if max_kept is None:
        max_kept = min(Nk, int(k) + int(sink_blocks) + _band_blocks(w))
    kv_idx, kv_cnt, mask = _select_out(scores, max_kept, return_mask, out)
    _check(lib().bsa_topk_block_mask(_dev(scores, "scores"), B, H, Nq, Nk, int(k), int(sink_blocks), w,
                                     _dev(kv_idx), _dev(kv_cnt), int(max_kept),
                                     None if mask is None else _dev(mask), _stream(scores)))
    return (kv_idx, kv_cnt, mask) if return_mask else (kv_idx, kv_cnt)


def bsa_top_p_block_mask(scores, p: float, scale: float = 1.0, sink_blocks: int = 1, diag_width=1,
                         return_mask: bool = False, out=None):
    """Top-p (nucleus) block selection -> (kv_idx (B, H, Nq, Nk), kv_cnt[, mask])."""
    torch = _torch()
    if scores.dim() != 4 or scores.dtype != torch.float32:
        raise ValueError("scores must be float32 (B, H, Nq, Nk)")
    B, H, Nq, Nk = (int(s) for s in scores.shape)
    kv_idx, kv_cnt, mask = _select_out(scores, Nk, return_mask, out)
    _check(lib().bsa_top_p_block_mask(_dev(scores, "scores"), B, H, Nq, Nk, float(p), float(scale),
                                      int(sink_blocks), _band(diag_width), _dev(kv_idx), _dev(kv_cnt),
                                      int(kv_idx.shape[-1]), None if mask is None else _dev(mask),
                                      _stream(scores)))
    return (kv_idx, kv_cnt, mask) if return_mask else (kv_idx, kv_cnt)


def bsa_topk_block_mask_tiled(scores, head_choice, k_table, nk_table, sink_blocks: int = 1, diag_width=1,
                              max_kept: int | None = None, return_mask: bool = False, out=None):
    """Top-k with a per-head budget k_table[c] over the head's nk_table[c] blocks, c = head_choice[b, h]."""
    torch = _torch()
    if scores.dim() != 4 or scores.dtype != torch.float32:
        raise ValueError("scores must be float32 (B, H, Nq, Nk)")
    B, H, Nq, Nk = (int(s) for s in scores.shape)
    if head_choice.dtype != torch.int32 or head_choice.numel() != B * H:
        raise ValueError("head_choice must be int32 with B*H entries")
    kt = np.ascontiguousarray(k_table, dtype=np.int32)
    nt = np.ascontiguousarray(nk_table, dtype=np.int32)
    if kt.shape != nt.shape or kt.ndim != 1:
        raise ValueError("k_table and nk_table must be 1-D of equal length")
    w = _band(diag_width)
    if max_kept is None:
        max_kept = int(max(min(int(n), int(k) + int(sink_blocks) + _band_blocks(w)) for k, n in zip(kt, nt)))
    kv_idx, kv_cnt, mask = _select_out(scores, max_kept, return_mask, out)
    _check(lib().bsa_topk_block_mask_tiled(_dev(scores, "scores"), B, H, Nq, Nk, _dev(head_choice, "head_choice"),
                                           kt.ctypes.data, nt.ctypes.data, int(kt.size), int(sink_blocks), w,
                                           _dev(kv_idx), _dev(kv_cnt), int(kv_idx.shape[-1]),
                                           None if mask is None else _dev(mask), _stream(scores)))
    return (kv_idx, kv_cnt, mask) if return_mask else (kv_idx, kv_cnt)


def _qkv(q, k, v):
    shp = _bhsd(q, "q")
    if _bhsd(k, "k") != shp or _bhsd(v, "v") != shp:
        raise ValueError(f"q/k/v shapes must match exactly; got {tuple(q.shape)}, {tuple(k.shape)}, "
                         f"{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q/k/v dtypes must match")
    return shp


def bsa_block_sparse_attention(q, k, v, kv_idx, kv_cnt, block: int, scale=None, out=None, key_norms=None,
                               row_order=None):
    """Attention of every query block over its kept key blocks -> (B, H, S, D) like q.

    key_norms: float32 (B, H, S // block) or None, at least each key block's largest row L2 norm (as
    bsa_minmax_block_scores writes them); it lets the kernel skip the running-max update of key blocks
    that cannot pass it, which changes the result only by rounding.
    row_order: a launch order as bsa_row_order writes it (1-D int32 / uint32: workgroup w runs row
    row_order[w] = (b*H + h)*Nq + I, entries past the last row are empty slots), or None: the bf16 kernels
    start the rows in that order (the result does not depend on it)."""
    torch = _torch()
    B, H, S, D = _qkv(q, k, v)
    if kv_idx.dtype != torch.int32 or kv_cnt.dtype != torch.int32 or kv_idx.dim() != 4:
        raise ValueError("kv_idx must be int32 (B, H, Nq, max_kept) and kv_cnt int32 (B, H, Nq)")
    if block < 1 or S % block:
        raise ValueError(f"block {block} must divide S={S}")
    if tuple(kv_idx.shape[:3]) != (B, H, S // block) or tuple(kv_cnt.shape) != (B, H, S // block):
        raise ValueError("block lists do not match (B, H, S // block)")
    o = torch.empty_like(q) if out is None else out
    _check(lib().bsa_block_sparse_attention(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "out"),
                                            _dtype_code(q), B, H, S, D, int(block), _dev(kv_idx), _dev(kv_cnt),
                                            int(kv_idx.shape[3]), _scale(scale),
                                            _norms_out(key_norms, B, H, S // block, q),
                                            *_order_args(row_order, B * H * (S // block)), _stream(q)))
    return o


def _order_args(row_order, rows: int):
    """(pointer, length) of an optional launch order over `rows` rows."""
    if row_order is None:
        return None, 0
    torch = _torch()
    if row_order.dtype not in (torch.int32, torch.uint32) or row_order.dim() != 1 or row_order.numel() < rows:
        raise ValueError(f"row_order must be a 1-D int32 / uint32 tensor of at least {rows} entries")
    return _dev(row_order, "row_order"), int(row_order.numel())


def bsa_row_order_len(BH: int, nq: int) -> int:
    """Length of bsa_row_order's launch plan for BH heads of nq rows (asked of libbsa, nothing launched)."""
    n = int(lib().bsa_row_order_len(int(BH), int(nq)))
    if n < 0:
        raise ValueError(lib().bsa_last_error().decode())
    return n


def bsa_row_order(kv_cnt, out=None):
    """Launch plan for the block lists of kv_cnt (B, H, Nq) -> int32 (bsa_row_order_len(B*H, Nq),): each XCD
    gets whole heads (or head ranges) of balanced work, long rows first; empty slots read -1."""
    torch = _torch()
    if kv_cnt.dtype != torch.int32 or kv_cnt.dim() != 3:
        raise ValueError("kv_cnt must be int32 (B, H, Nq)")
    B, H, nq = (int(s) for s in kv_cnt.shape)
    n = bsa_row_order_len(B * H, nq)
    o = torch.empty(n, dtype=torch.int32, device=kv_cnt.device) if out is None else out
    if o.dtype not in (torch.int32, torch.uint32) or o.dim() != 1 or o.numel() < n:
        raise ValueError(f"out must be a 1-D int32 / uint32 tensor of at least {n} entries")
    _check(lib().bsa_row_order(_dev(kv_cnt, "kv_cnt"), B * H, nq, _dev(o, "out"), int(o.numel()), _stream(kv_cnt)))
    return o


def bsa_row_order_by_median(kv_idx, kv_cnt, nk: int = None, out=None, head_kv_bytes: int = 0):
    """Launch order for top-k block lists kv_idx (B, H, Nq, max_kept) / kv_cnt (B, H, Nq) -> int32 (B*H*Nq,): the
    plain split of the rows over the 8 XCDs, each head's rows sorted by the middle entry of their kept list
    (nk: key blocks per row, default Nq).  head_kv_bytes: bytes of one head's K and V; libbsa splits heads
    above 32 MiB over two XCDs (bsa_row_order_by_median_ex)."""
    torch = _torch()
    if kv_cnt.dtype != torch.int32 or kv_cnt.dim() != 3:
        raise ValueError("kv_cnt must be int32 (B, H, Nq)")
    if kv_idx.dtype != torch.int32 or kv_idx.dim() != 4 or tuple(kv_idx.shape[:3]) != tuple(kv_cnt.shape):
        raise ValueError("kv_idx must be int32 (B, H, Nq, max_kept) over kv_cnt's rows")
    B, H, nq = (int(s) for s in kv_cnt.shape)
    n = B * H * nq
    o = torch.empty(n, dtype=torch.int32, device=kv_cnt.device) if out is None else out
    if o.dtype not in (torch.int32, torch.uint32) or o.dim() != 1 or o.numel() < n:
        raise ValueError(f"out must be a 1-D int32 / uint32 tensor of at least {n} entries")
    _check(lib().bsa_row_order_by_median_ex(_dev(kv_idx, "kv_idx"), _dev(kv_cnt, "kv_cnt"), B * H, nq,
                                            int(kv_idx.shape[3]), nq if nk is None else int(nk), int(head_kv_bytes),
                                            _dev(o, "out"), int(o.numel()), _stream(kv_cnt)))
    return o


def tiled_attention_supported(dtype, D, tiles, grid, pad: bool = False) -> bool:
    """Whether bsa_block_sparse_attention_tiled (or, with pad, its _padded form) has a kernel for these tilings
    of the grid (asked of libbsa, nothing launched)."""
    torch = _torch()
    T, Hg, Wg = (int(g) for g in grid)
    arr, n = _tiles_arr(tiles)
    code = BSA_BF16 if dtype == torch.bfloat16 else BSA_F32
    return bool(lib().bsa_tiled_attention_supported(code, int(D), T, Hg, Wg, arr, n, int(bool(pad))))


def bsa_block_sparse_attention_tiled(q, k, v, grid, tiles, kv_idx, kv_cnt, head_choice=None, scale=None, out=None,
                                     key_norms=None, row_order=None):
    """Block-sparse attention of T-major tensors, blocks = tiles (gather on load) -> T-major (B, H, S, D).

    key_norms and row_order: per tile of each head's tiling, as in bsa_block_sparse_attention."""
    torch = _torch()
    B, H, S, D = _qkv(q, k, v)
    T, Hg, Wg = (int(g) for g in grid)
    if T * Hg * Wg != S:
        raise ValueError(f"grid {tuple(grid)} does not match S={S}")
    arr, n = _tiles_arr(tiles)
    if kv_idx.dtype != torch.int32 or kv_cnt.dtype != torch.int32 or kv_idx.dim() != 4:
        raise ValueError("kv_idx must be int32 (B, H, Nq, max_kept) and kv_cnt int32 (B, H, Nq)")
    if tuple(kv_idx.shape[:3]) != (B, H, S // 64) or tuple(kv_cnt.shape) != (B, H, S // 64):
        raise ValueError("block lists do not match (B, H, S // 64)")
    o = torch.empty_like(q) if out is None else out
    hc = None if head_choice is None else _dev(head_choice, "head_choice")
    _check(lib().bsa_block_sparse_attention_tiled(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "out"),
                                                  _dtype_code(q), B, H, T, Hg, Wg, D, arr, n, hc, _dev(kv_idx),
                                                  _dev(kv_cnt), int(kv_idx.shape[3]), _scale(scale),
                                                  _norms_out(key_norms, B, H, S // 64, q),
                                                  *_order_args(row_order, B * H * (S // 64)), _stream(q)))
    return o


def bsa_block_sparse_attention_tiled_padded(q, k, v, grid, tiles, kv_idx, kv_cnt, head_choice=None, scale=None,
                                            out=None, key_norms=None, row_order=None):
    """bsa_block_sparse_attention_tiled on each head's zero-padded grid (candidates may leave T undivided):
    kv lists over the largest padded block count Nq; padding keys are masked and padding rows not written.
    row_order: a launch order over the Nq rows of each head, as in bsa_block_sparse_attention."""
    torch = _torch()
    B, H, S, D = _qkv(q, k, v)
    T, Hg, Wg = (int(g) for g in grid)
    if T * Hg * Wg != S:
        raise ValueError(f"grid {tuple(grid)} does not match S={S}")
    arr, n = _tiles_arr(tiles)
    nq = padded_rows(grid, tiles) // 64
    if kv_idx.dtype != torch.int32 or kv_cnt.dtype != torch.int32 or kv_idx.dim() != 4:
        raise ValueError("kv_idx must be int32 (B, H, Nq, max_kept) and kv_cnt int32 (B, H, Nq)")
    if tuple(kv_idx.shape[:3]) != (B, H, nq) or tuple(kv_cnt.shape) != (B, H, nq):
        raise ValueError(f"block lists do not match (B, H, {nq})")
    o = torch.empty_like(q) if out is None else out
    hc = None if head_choice is None else _dev(head_choice, "head_choice")
    _check(lib().bsa_block_sparse_attention_tiled_padded(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "out"),
                                                         _dtype_code(q), B, H, T, Hg, Wg, D, arr, n, hc, _dev(kv_idx),
                                                         _dev(kv_cnt), int(kv_idx.shape[3]), _scale(scale),
                                                         _norms_out(key_norms, B, H, nq, q),
                                                         *_order_args(row_order, B * H * nq), _stream(q)))
    return o


def bsa_block_sparse_attention_labels(q, k, v, kv_idx, kv_cnt, block: int, labels, scale=None, out=None):
    """Block-sparse attention with the token rule labels[i] == labels[j] inside kept blocks.

    labels: int32 (S,) shared by every head, or (B, H, S)."""
    torch = _torch()
    B, H, S, D = _qkv(q, k, v)
    if kv_idx.dtype != torch.int32 or kv_cnt.dtype != torch.int32 or kv_idx.dim() != 4:
        raise ValueError("kv_idx must be int32 (B, H, Nq, max_kept) and kv_cnt int32 (B, H, Nq)")
    if block < 1 or S % block:
        raise ValueError(f"block {block} must divide S={S}")
    if tuple(kv_idx.shape[:3]) != (B, H, S // block) or tuple(kv_cnt.shape) != (B, H, S // block):
        raise ValueError("block lists do not match (B, H, S // block)")
    if labels.dtype != torch.int32:
        raise ValueError("labels must be int32")
    if tuple(labels.shape) == (S,):
        stride = 0
    elif tuple(labels.shape) == (B, H, S):
        stride = S
    else:
        raise ValueError("labels must be (S,) or (B, H, S)")
    o = torch.empty_like(q) if out is None else out
    _check(lib().bsa_block_sparse_attention_labels(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "out"),
                                                   _dtype_code(q), B, H, S, D, int(block), _dev(kv_idx),
                                                   _dev(kv_cnt), int(kv_idx.shape[3]), _dev(labels, "labels"), stride,
                                                   _scale(scale), _stream(q)))
    return o


def bsa_windowed_attention(q, k, v, window: int, sink: int = 0, scale=None, chunk=None, out=None):
    """Symmetric sliding-window attention with sinks -> (B, H, S, D) like q."""
    torch = _torch()
    B, H, S, D = _qkv(q, k, v)
    o = torch.empty_like(q) if out is None else out
    _check(lib().bsa_windowed_attention(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "out"), _dtype_code(q),
                                        B, H, S, D, int(window), int(sink), _scale(scale),
                                        0 if chunk is None else int(chunk), _stream(q)))
    return o


def bsa_temporal_only_attention(q, k, v, grid, scale=None, out=None):
    """Temporal-only attention of T-major (B, H, S, D) tensors: token i sees token j exactly when they sit
    at one (y, x).  UnsupportedError outside bf16, D in {64, 128}, T <= 64."""
    torch = _torch()
    B, H, S, D = _qkv(q, k, v)
    T, Hg, Wg = (int(g) for g in grid)
    if T * Hg * Wg != S:
        raise ValueError(f"grid {tuple(grid)} does not match S={S}")
    o = torch.empty_like(q) if out is None else out
    _check(lib().bsa_temporal_only_attention(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "out"),
                                             _dtype_code(q), B, H, T, Hg, Wg, D, _scale(scale), _stream(q)))
    return o


def bsa_validate_block_list(kv_idx, kv_cnt, Nk: int) -> None:
    """Synchronous: RuntimeError unless every row is a non-empty ascending list inside [0, Nk)."""
    B, H, Nq, max_kept = (int(s) for s in kv_idx.shape)
    _check(lib().bsa_validate_block_list(_dev(kv_idx), _dev(kv_cnt), B, H, Nq, int(Nk), max_kept,
                                         _stream(kv_idx)))


def bsa_validate_indices(v, lo: int, hi: int) -> None:
    """Synchronous: RuntimeError unless lo <= v < hi everywhere."""
    _check(lib().bsa_validate_indices(_dev(v), v.numel(), int(lo), int(hi), _stream(v)))


# ----------------------------------------------------------- composition ---

class AdaptiveBlockSparse:
    """The adaptive-tiling pipeline as a sequence of libbsa launches on one stream.

    select tiling -> permute q, k, v -> min/max scores -> top-k (+sink, +diag)
    -> block-sparse attention -> inverse permute.  Buffers are allocated once
    (torch) and reused, so a call allocates nothing and never synchronises.
    ``keep_diag`` is the diagonal band width (True = the diagonal alone);
    ``top_p`` replaces the top-k budget with the top-p rule (softmax of
    ``p_scale`` * scores); ``statistic`` is the tiling-choice rule ("mean" or
    SPADE's "pooled").  ``pad=True`` accepts candidates that do not divide
    the grid: every head works on the zero-padded grid of its own choice
    (padding left out of the cohesion and the summaries, masked as keys,
    dropped from the output), with the budget floor(frac * that grid's block
    count.  ``fused`` (default: whenever the kernels cover the tilings, see
    tiled_attention_supported) reads q, k, v in place through the tile
    geometry for the scores and the attention and writes the output in
    T-major order, so no pass forms a permuted copy (with padding, the cells
    of the padding frames are left out unread).  ``validate=True`` checks the device-resident tiling choices and (without
    padding) block lists (bsa_validate_indices, bsa_validate_block_list)
    before the attention runs; each check synchronises the stream and raises
    RuntimeError on a violation.
    """

    def __init__(self, B, H, grid, D, tiles, frac, dtype, device, sink_blocks=1, keep_diag=True, scale=None,
                 top_p=None, p_scale=1.0, statistic="mean", pad=False, fused=None, validate=False):
        torch = _torch()
        self.grid = tuple(int(g) for g in grid)
        self.tiles = [tuple(int(v) for v in t) for t in tiles]
        vols = {a * b * c for a, b, c in self.tiles}
        if len(vols) != 1:
            raise ValueError("candidate tilings must share one volume")
        self.block = vols.pop()
        T, Hg, Wg = self.grid
        self.S = T * Hg * Wg
        self.pad, self.statistic = bool(pad), statistic
        if self.pad and top_p is not None:
            raise ValueError("top_p is not supported together with pad")
        self.Sp = padded_rows(self.grid, self.tiles) if self.pad else self.S
        self.nb = self.Sp // self.block
        self.sink_blocks, self.keep_diag, self.scale = int(sink_blocks), _band(keep_diag), scale
        self.top_p, self.p_scale = top_p, float(p_scale)
        self.validate = bool(validate)
        can_fuse = tiled_attention_supported(dtype, D, self.tiles, self.grid, self.pad)
        if fused and not can_fuse:
            raise ValueError("the fused path needs bf16, D = 128 and tilings tiled_attention_supported accepts")
        self.fused = can_fuse if fused is None else bool(fused)
        if self.pad:
            self.nk_table = [bsa_padded_length(T, Hg, Wg, t) // self.block for t in self.tiles]
            self.k_table = [bsa_budget(frac, n) for n in self.nk_table]
            self.k = max(self.k_table)
            self.max_kept = max(min(n, k + self.sink_blocks + _band_blocks(self.keep_diag))
                                for k, n in zip(self.k_table, self.nk_table))
        else:
            self.k = bsa_budget(frac, self.nb)
            if top_p is None:
                self.max_kept = min(self.nb, self.k + self.sink_blocks + _band_blocks(self.keep_diag))
            else:
                self.max_kept = self.nb
        f = dict(device=device)
        n = len(self.tiles)
        self.ws_select = (torch.empty((B, H, n, self.nb), dtype=torch.float32, **f),
                          torch.empty((B, H, n), dtype=torch.float32, **f),
                          torch.empty((B, H), dtype=torch.int32, **f))
        if self.fused:     # every pass reads q, k, v in place through the tile geometry
            self.qp = self.kp = self.vp = self.op = None
        else:
            self.qp, self.kp, self.vp, self.op = (torch.empty((B, H, self.Sp, D), dtype=dtype, **f)
                                                  for _ in range(4))
        self.labels = torch.empty((B, H, self.Sp), dtype=torch.int32, **f) if self.pad and not self.fused else None
        self.ws_scores = (torch.empty((B, H, self.nb, self.nb), dtype=torch.float32, **f),
                          torch.empty((4, B, H, self.nb, D), dtype=dtype, **f))
        self.ws_topk = (torch.empty((B, H, self.nb, self.max_kept), dtype=torch.int32, **f),
                        torch.empty((B, H, self.nb), dtype=torch.int32, **f), None)
        # top-p lists differ in length from row to row, and padded candidates give heads different block
        # counts and budgets: a launch plan balances the XCDs by work and starts long rows first (the fused
        # attention takes it).  Top-k lists have (nearly) equal lengths: their launch order keeps the plain
        # XCD ranges and sorts each head's rows by where their kept key blocks lie, so that the query blocks an
        # XCD runs side by side share more key blocks through its L2
        self.order_by_median = top_p is None and not self.pad and (B * H * self.nb) % 8 == 0
        if top_p is not None or (self.pad and self.fused):
            self.ws_order = torch.empty(bsa_row_order_len(B * H, self.nb), dtype=torch.int32, **f)
        elif self.order_by_median:
            self.ws_order = torch.empty(B * H * self.nb, dtype=torch.int32, **f)
        else:
            self.ws_order = None
        # each key block's largest row norm, written by the scores pass: the attention kernel skips the
        # running-max update of the key blocks it proves cannot pass it
        self.ws_knorm = (torch.empty((B, H, self.nb), dtype=torch.float32, **f) if self.fused or not self.pad
                         else None)
        # fused path: the tiling choice pass also forms q's block summaries of every candidate, so the scores
        # pass reads only k
        self.ws_qsumm = (torch.empty((n, 2, B, H, self.nb, D), dtype=dtype, **f) if self.fused and not self.pad
                         else None)

    @property
    def choice(self):
        return self.ws_select[2]

    @property
    def kv(self):
        return self.ws_topk[0], self.ws_topk[1]

    def __call__(self, q, k, v, out=None, attention_hook=None):
        choice, _, _ = bsa_select_tiling(q, self.grid, self.tiles, workspace=self.ws_select, statistic=self.statistic,
                                         pad=self.pad, q_summaries=self.ws_qsumm)
        if self.validate:
            bsa_validate_indices(choice, 0, len(self.tiles))
        if self.pad:
            if self.fused:
                scores, _ = bsa_minmax_block_scores_tiled_padded(q, k, self.grid, self.tiles, head_choice=choice,
                                                                 out=self.ws_scores, key_norms=self.ws_knorm)
            else:
                for src, dst, lab in ((q, self.qp, self.labels), (k, self.kp, None), (v, self.vp, None)):
                    bsa_tile_permute_padded(src, self.grid, self.tiles, head_choice=choice, Sp=self.Sp,
                                            out=(dst, lab))
                scores, _ = bsa_minmax_block_scores(self.qp, self.kp, self.block, out=self.ws_scores,
                                                    labels=self.labels, key_norms=self.ws_knorm)
            kv_idx, kv_cnt = bsa_topk_block_mask_tiled(scores, choice, self.k_table, self.nk_table, self.sink_blocks,
                                                       self.keep_diag, max_kept=self.max_kept, out=self.ws_topk)
            if self.ws_order is not None:
                bsa_row_order(kv_cnt, out=self.ws_order)
        else:
            if self.fused:
                scores, _ = bsa_minmax_block_scores_tiled(q, k, self.grid, self.tiles, head_choice=choice,
                                                          out=self.ws_scores, key_norms=self.ws_knorm,
                                                          q_summaries=self.ws_qsumm)
            else:
                for src, dst in ((q, self.qp), (k, self.kp), (v, self.vp)):
                    bsa_tile_permute(src, self.grid, self.tiles, head_choice=choice, out=dst)
                scores, _ = bsa_minmax_block_scores(self.qp, self.kp, self.block, out=self.ws_scores,
                                                    key_norms=self.ws_knorm)
            if self.top_p is None:
                kv_idx, kv_cnt, _ = bsa_topk_block_mask(scores, self.k, self.sink_blocks, self.keep_diag,
                                                        max_kept=self.max_kept, return_mask=True, out=self.ws_topk)
                if self.order_by_median:
                    bsa_row_order_by_median(kv_idx, kv_cnt, out=self.ws_order,
                                            head_kv_bytes=2 * k.shape[2] * k.shape[3] * k.element_size())
            else:
                kv_idx, kv_cnt, _ = bsa_top_p_block_mask(scores, self.top_p, self.p_scale, self.sink_blocks,
                                                         self.keep_diag, return_mask=True, out=self.ws_topk)
                bsa_row_order(kv_cnt, out=self.ws_order)
        if self.validate and not self.pad:
            bsa_validate_block_list(kv_idx, kv_cnt, self.nb)
        if self.fused:
            if attention_hook is not None:
                attention_hook(True)
            if self.pad:
                o = bsa_block_sparse_attention_tiled_padded(q, k, v, self.grid, self.tiles, kv_idx, kv_cnt,
                                                            head_choice=choice, scale=self.scale, out=out,
                                                            key_norms=self.ws_knorm, row_order=self.ws_order)
            else:
                o = bsa_block_sparse_attention_tiled(q, k, v, self.grid, self.tiles, kv_idx, kv_cnt,
                                                     head_choice=choice, scale=self.scale, out=out,
                                                     key_norms=self.ws_knorm, row_order=self.ws_order)
            if attention_hook is not None:
                attention_hook(False)
            return o
        if attention_hook is not None:
            attention_hook(True)
        if self.pad:
            bsa_block_sparse_attention_labels(self.qp, self.kp, self.vp, kv_idx, kv_cnt, self.block, self.labels,
                                              self.scale, out=self.op)
        else:
            bsa_block_sparse_attention(self.qp, self.kp, self.vp, kv_idx, kv_cnt, self.block, self.scale,
                                       out=self.op, key_norms=self.ws_knorm, row_order=self.ws_order)
        if attention_hook is not None:
            attention_hook(False)
        if self.pad:
            return bsa_invert_permute_padded(self.op, self.grid, self.tiles, head_choice=choice, out=out)
        return bsa_invert_permute(self.op, self.grid, self.tiles, head_choice=choice, out=out)


class VideoLabelAttention:
    """Spatial-only or temporal-only attention of T-major (B, H, S, D) tensors.

    kind "spatial": a token sees the tokens of its own frame (labels = frame
    index, T-major order, block lists of the frames' blocks).  kind
    "temporal": a token sees the tokens at its own (y, x) in every frame.
    With bf16, D in {64, 128} and T <= 64 (``dtype``, ``D`` given) that is one
    bsa_temporal_only_attention call, which gathers each position's frames
    on load; otherwise the tokens are permuted with tiles (T, 1, 1) so that
    each position's frames are contiguous, labelled by position, attended,
    and permuted back.  [ADR-0001, "Décision" step 1: spatial_only_mask,
    temporal_only_mask.]  Block lists and labels are built once (host, then
    copied to the device); a call is a sequence of libbsa launches on the
    current stream.
    """

    def __init__(self, B, H, grid, kind: str, device, block: int = 64, dtype=None, D: int = 128):
        torch = _torch()
        self.grid = tuple(int(g) for g in grid)
        T, Hg, Wg = self.grid
        S = T * Hg * Wg
        lab = bsa_video_labels(self.grid, kind)
        self.tiles = [(T, 1, 1)] if kind == "temporal" else None
        # temporal-only: one call that gathers each position's frames on load, where it has a kernel
        self.direct = kind == "temporal" and dtype == _torch().bfloat16 and int(D) in (64, 128) and T <= 64
        if S % block:
            raise ValueError(f"block {block} must divide S={S}")
        self.kind, self.block, self.S = kind, int(block), S
        idx, cnt = bsa_label_block_list(lab, self.block)
        nb = S // self.block
        self.kv_idx = torch.from_numpy(np.broadcast_to(idx, (B, H) + idx.shape).copy()).to(device)
        self.kv_cnt = torch.from_numpy(np.broadcast_to(cnt, (B, H, nb)).copy()).to(device)
        self.labels = torch.from_numpy(lab).to(device)

    def __call__(self, q, k, v, scale=None, out=None):
        if self.tiles is not None and self.direct:
            return bsa_temporal_only_attention(q, k, v, self.grid, scale, out=out)
        if self.tiles is None:
            return bsa_block_sparse_attention_labels(q, k, v, self.kv_idx, self.kv_cnt, self.block, self.labels, scale,
                                                     out=out)
        qp, kp, vp = (bsa_tile_permute(x, self.grid, self.tiles) for x in (q, k, v))
        op = bsa_block_sparse_attention_labels(qp, kp, vp, self.kv_idx, self.kv_cnt, self.block, self.labels, scale)
        return bsa_invert_permute(op, self.grid, self.tiles, out=out)


def video_label_attention(q, k, v, grid, kind: str, block: int = 64, scale=None, out=None):
    """One-shot VideoLabelAttention (builds the block lists on every call)."""
    B, H, _, D = _bhsd(q, "q")
    return VideoLabelAttention(B, H, grid, kind, q.device, block, q.dtype, D)(q, k, v, scale, out)
