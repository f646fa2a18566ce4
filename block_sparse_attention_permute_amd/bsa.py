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
import math
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsa.so")

BSA_OK, BSA_ERR_INVALID_ARG, BSA_ERR_INVARIANT, BSA_ERR_UNSUPPORTED, BSA_ERR_DEVICE = range(5)
BSA_F32, BSA_BF16 = 0, 1
BSA_MAX_TILINGS = 8

EXPORTED = (
    "bsa_last_error", "bsa_version", "bsa_tile_permutation", "bsa_invert_permutation", "bsa_budget",
    "bsa_sliding_tile_block_list", "bsa_tile_permute", "bsa_invert_permute", "bsa_block_cohesion",
    "bsa_select_tiling", "bsa_minmax_block_scores", "bsa_topk_block_mask", "bsa_top_p_block_mask",
    "bsa_block_sparse_attention",
    "bsa_windowed_attention", "bsa_validate_block_list", "bsa_validate_indices",
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
    "bsa_minmax_block_scores": (_I, [_P, _P, _I, _I64, _I64, _I64, _I64, _I, _P, _P, _P]),
    "bsa_topk_block_mask": (_I, [_P, _I64, _I64, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P]),
    "bsa_top_p_block_mask": (_I, [_P, _I64, _I64, _I, _I, _F, _F, _I, _I, _P, _P, _I, _P, _P]),
    "bsa_block_sparse_attention": (_I, [_P, _P, _P, _P, _I, _I64, _I64, _I64, _I64, _I, _P, _P, _I, _F, _P]),
    "bsa_windowed_attention": (_I, [_P, _P, _P, _P, _I, _I64, _I64, _I64, _I64, _I, _I, _F, _I, _P]),
    "bsa_validate_block_list": (_I, [_P, _P, _I64, _I64, _I, _I, _I, _P]),
    "bsa_validate_indices": (_I, [_P, _I64, _I, _I, _P]),
}


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


def bsa_block_cohesion(x, block: int):
    """Cohesion of each run of `block` tokens -> float32 (B, H, S // block)."""
    torch = _torch()
    B, H, S, D = _bhsd(x, "x")
    if block < 1 or S % block:
        raise ValueError(f"block {block} must divide S={S}")
    coh = torch.empty((B, H, S // block), dtype=torch.float32, device=x.device)
    _check(lib().bsa_block_cohesion(_dev(x, "x"), _dtype_code(x), B, H, S, D, int(block), _dev(coh), _stream(x)))
    return coh


def bsa_select_tiling(q, grid, tiles, workspace=None):
    """Per-head tiling choice -> (choice int32 (B, H), score float32 (B, H, n), tile_coh)."""
    torch = _torch()
    B, H, S, D = _bhsd(q, "q")
    T, Hg, Wg = (int(g) for g in grid)
    if T * Hg * Wg != S:
        raise ValueError(f"grid {tuple(grid)} does not match S={S}")
    arr, n = _tiles_arr(tiles)
    max_nb = max(S // max(a * b * c, 1) for a, b, c in tiles)
    if workspace is None:
        tile_coh = torch.empty((B, H, n, max_nb), dtype=torch.float32, device=q.device)
        score = torch.empty((B, H, n), dtype=torch.float32, device=q.device)
        choice = torch.empty((B, H), dtype=torch.int32, device=q.device)
    else:
        tile_coh, score, choice = workspace
    _check(lib().bsa_select_tiling(_dev(q, "q"), _dtype_code(q), B, H, T, Hg, Wg, D, arr, n, _dev(tile_coh),
                                   _dev(score), _dev(choice), _stream(q)))
    return choice, score, tile_coh


def bsa_minmax_block_scores(q, k, block: int, out=None):
    """-> (scores float32 (B, H, Nb, Nb), summaries (4, B, H, Nb, D): qmax, qmin, kmax, kmin)."""
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
    _check(lib().bsa_minmax_block_scores(_dev(q, "q"), _dev(k, "k"), _dtype_code(q), B, H, S, D, int(block),
                                         _dev(summ), _dev(scores), _stream(q)))
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


def _qkv(q, k, v):
    shp = _bhsd(q, "q")
    if _bhsd(k, "k") != shp or _bhsd(v, "v") != shp:
        raise ValueError(f"q/k/v shapes must match exactly; got {tuple(q.shape)}, {tuple(k.shape)}, "
                         f"{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q/k/v dtypes must match")
    return shp


def bsa_block_sparse_attention(q, k, v, kv_idx, kv_cnt, block: int, scale=None, out=None):
    """Attention of every query block over its kept key blocks -> (B, H, S, D) like q."""
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
                                            int(kv_idx.shape[3]), _scale(scale), _stream(q)))
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


def bsa_validate_block_list(kv_idx, kv_cnt, Nk: int) -> None:
    """Synchronous: RuntimeError unless every row is a non-empty ascending list inside [0, Nk)."""
    B, H, Nq, max_kept = (int(s) for s in kv_idx.shape)
    _check(lib().bsa_validate_block_list(_dev(kv_idx), _dev(kv_cnt), B, H, Nq, int(Nk), max_kept,
                                         _stream(kv_idx)))


def bsa_validate_indices(v, lo: int, hi: int) -> None:
    """Synchronous: RuntimeError unless lo <= v < hi everywhere."""
    _check(lib().bsa_validate_indices(_dev(v), v.numel(), int(lo), int(hi), _stream(v)))


# ----------------------------------------------------------- composition ---

def default_scale(D: int, scale=None) -> float:
    return float(scale) if scale is not None else 1.0 / math.sqrt(D)


class AdaptiveBlockSparse:
    """The adaptive-tiling pipeline as a sequence of libbsa launches on one stream.

    select tiling -> permute q, k, v -> min/max scores -> top-k (+sink, +diag)
    -> block-sparse attention -> inverse permute.  Buffers are allocated once
    (torch) and reused, so a call allocates nothing and never synchronises.
    ``keep_diag`` is the diagonal band width (True = the diagonal alone);
    ``top_p`` replaces the top-k budget with the top-p rule (softmax of
    ``p_scale`` * scores).
    """

    def __init__(self, B, H, grid, D, tiles, frac, dtype, device, sink_blocks=1, keep_diag=True, scale=None,
                 top_p=None, p_scale=1.0):
        torch = _torch()
        self.grid = tuple(int(g) for g in grid)
        self.tiles = [tuple(int(v) for v in t) for t in tiles]
        vols = {a * b * c for a, b, c in self.tiles}
        if len(vols) != 1:
            raise ValueError("candidate tilings must share one volume")
        self.block = vols.pop()
        T, Hg, Wg = self.grid
        self.S = T * Hg * Wg
        self.nb = self.S // self.block
        self.k = bsa_budget(frac, self.nb)
        self.sink_blocks, self.keep_diag, self.scale = int(sink_blocks), _band(keep_diag), scale
        self.top_p, self.p_scale = top_p, float(p_scale)
        if top_p is None:
            self.max_kept = min(self.nb, self.k + self.sink_blocks + _band_blocks(self.keep_diag))
        else:
            self.max_kept = self.nb
        f = dict(device=device)
        n = len(self.tiles)
        self.ws_select = (torch.empty((B, H, n, self.nb), dtype=torch.float32, **f),
                          torch.empty((B, H, n), dtype=torch.float32, **f),
                          torch.empty((B, H), dtype=torch.int32, **f))
        self.qp, self.kp, self.vp, self.op = (torch.empty((B, H, self.S, D), dtype=dtype, **f) for _ in range(4))
        self.ws_scores = (torch.empty((B, H, self.nb, self.nb), dtype=torch.float32, **f),
                          torch.empty((4, B, H, self.nb, D), dtype=dtype, **f))
        self.ws_topk = (torch.empty((B, H, self.nb, self.max_kept), dtype=torch.int32, **f),
                        torch.empty((B, H, self.nb), dtype=torch.int32, **f), None)

    @property
    def choice(self):
        return self.ws_select[2]

    @property
    def kv(self):
        return self.ws_topk[0], self.ws_topk[1]

    def __call__(self, q, k, v, out=None, attention_hook=None):
        choice, _, _ = bsa_select_tiling(q, self.grid, self.tiles, workspace=self.ws_select)
        for src, dst in ((q, self.qp), (k, self.kp), (v, self.vp)):
            bsa_tile_permute(src, self.grid, self.tiles, head_choice=choice, out=dst)
        scores, _ = bsa_minmax_block_scores(self.qp, self.kp, self.block, out=self.ws_scores)
        if self.top_p is None:
            kv_idx, kv_cnt, _ = bsa_topk_block_mask(scores, self.k, self.sink_blocks, self.keep_diag,
                                                    max_kept=self.max_kept, return_mask=True, out=self.ws_topk)
        else:
            kv_idx, kv_cnt, _ = bsa_top_p_block_mask(scores, self.top_p, self.p_scale, self.sink_blocks,
                                                     self.keep_diag, return_mask=True, out=self.ws_topk)
        if attention_hook is not None:
            attention_hook(True)
        bsa_block_sparse_attention(self.qp, self.kp, self.vp, kv_idx, kv_cnt, self.block, self.scale, out=self.op)
        if attention_hook is not None:
            attention_hook(False)
        return bsa_invert_permute(self.op, self.grid, self.tiles, head_choice=choice, out=out)
