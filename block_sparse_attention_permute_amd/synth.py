"""Seeded synthetic inputs for the five workloads.

This module is shared by the CPU oracle's tests and by the GPU path (tests,
smoke run, benchmark).  It holds no attention arithmetic at all: only random
draws, the input recipe for video-like queries and keys, and exact rounding
of float64 draws to bfloat16.

Seeding: every tensor of every head comes from its own PCG64 stream keyed by
``SeedSequence([2026, cfg, role, head])`` with role q=0, k=1, v=2 and
features=3, so results are platform-stable and any head can be regenerated on
its own.

Workloads (all batch 1, tokens in T-major order ``s = (t*Hg + y)*Wg + x``):

  1. fp32, H=2, grid 2x4x4 (S=32), D=16; q, k, v ~ N(0, 1).
  2. bf16, H=8, grid 8x16x16 (S=2048), D=64; q, k, v ~ N(0, 1).
  3. bf16, H=24, grid 16x32x32 (S=16384), D=128; q, k ~ N(0, 1/2), v ~ N(0, 1).
  4. bf16, H=40, grid 20x32x48 (S=30720), D=128; q, k from the Fourier recipe.
  5. bf16, H=24, grid 32x48x80 (S=122880), D=128; q, k from the Fourier recipe.

Fourier recipe (workloads 4 and 5), per head h, from the features stream:
  a_h ~ U{temporal, spatial}          the head's axis preference
  l = (8, 2, 2) for a temporal head,  length scales (t, y, x) in grid units:
      (2, 8, 8) for a spatial head    long along time, or along both axes of a frame
  z_f ~ N(0, I_3), w_f = z_f / l      16 random Fourier frequencies
  phi_f ~ U[0, 2*pi)
  A_f ~ N(0, (2/16) I_D)
  F(p) = sum_f A_f cos(w_f . p + phi_f)   (unit variance per dimension)
  q = F + 0.3 N(0, 1)  (q stream),  k = F + 0.3 N(0, 1)  (k stream)
q and k share F, so every head has smooth structure that is longer along its
preferred axes: a temporal head is coherent across frames at one position and
a spatial head across a frame, the two kinds of heads that adaptive tiling
serves with different tiles.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

ROLE_Q, ROLE_K, ROLE_V, ROLE_FEAT = 0, 1, 2, 3
HEAD_TEMPORAL, HEAD_SPATIAL = 0, 1
SEED_ROOT = 2026


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    dtype: str          # "f32" or "bf16"
    H: int
    grid: tuple         # (T, Hg, Wg)
    D: int
    B: int = 1

    @property
    def S(self) -> int:
        T, Hg, Wg = self.grid
        return T * Hg * Wg


WORKLOADS = {
    1: Workload(1, "tiny windowed fp32 (H=2, grid 2x4x4, D=16)", "f32", 2, (2, 4, 4), 16),
    2: Workload(2, "sliding-tile block-sparse bf16 (H=8, grid 8x16x16, D=64)", "bf16", 8, (8, 16, 16), 64),
    3: Workload(3, "windowed w=2048 sink=64 bf16 (H=24, grid 16x32x32, D=128)", "bf16", 24, (16, 32, 32), 128),
    4: Workload(4, "adaptive-tiling block-sparse at the Wan 2.1 latent shape bf16 "
                   "(H=40, grid 20x32x48, D=128, 17% budget)", "bf16", 40, (20, 32, 48), 128),
    5: Workload(5, "long-sequence block-sparse bf16 (H=24, grid 32x48x80, D=128, 10% budget)",
                "bf16", 24, (32, 48, 80), 128),
}


def rng_for(cfg: int, role: int, head: int) -> np.random.Generator:
    """The PCG64 stream of one (workload, role, head)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, cfg, role, head])))


# ---------------------------------------------------------------------------
# exact rounding helpers
# ---------------------------------------------------------------------------

def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (round to nearest, ties to even).

    Rounds once, directly from float64, to 8 significant bits; returns the
    raw 16-bit patterns as uint16.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    y = np.ldexp(np.rint(m * 256.0), e - 8)  # np.rint rounds half to even
    tiny = np.abs(x) < 2.0 ** -126          # bf16 subnormal range: fixed quantum
    if np.any(tiny):
        y = np.where(tiny, np.rint(x * 2.0 ** 133) * 2.0 ** -133, y)
    return (y.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bfloat16 bit patterns to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def round_to_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


# ---------------------------------------------------------------------------
# per-head draws
# ---------------------------------------------------------------------------

def grid_positions(grid) -> np.ndarray:
    """(S, 3) float64 positions (t, y, x) of the T-major tokens."""
    T, Hg, Wg = grid
    t, y, x = np.meshgrid(np.arange(T), np.arange(Hg), np.arange(Wg), indexing="ij")
    return np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1).astype(np.float64)


def fourier_field(cfg: int, head: int, grid, D: int, n_feat: int = 16) -> np.ndarray:
    """The shared smooth field F of one head, (S, D) float64."""
    g = rng_for(cfg, ROLE_FEAT, head)
    ell = np.array([8.0, 2.0, 2.0]) if int(g.integers(0, 2)) == HEAD_TEMPORAL else np.array([2.0, 8.0, 8.0])
    w = g.standard_normal((n_feat, 3)) / ell
    phi = g.uniform(0.0, 2.0 * np.pi, n_feat)
    amp = g.standard_normal((n_feat, D)) * np.sqrt(2.0 / n_feat)
    pos = grid_positions(grid)
    return np.cos(pos @ w.T + phi) @ amp


def head_kind(cfg: int, head: int) -> int:
    """HEAD_TEMPORAL or HEAD_SPATIAL: the axis preference the Fourier recipe drew for a head."""
    return int(rng_for(cfg, ROLE_FEAT, head).integers(0, 2))


def head_f64(cfg: int, role: int, head: int) -> np.ndarray:
    """Unrounded float64 draw of one head's q, k or v: (S, D)."""
    wl = WORKLOADS[cfg]
    S, D = wl.S, wl.D
    g = rng_for(cfg, role, head)
    if cfg in (4, 5) and role in (ROLE_Q, ROLE_K):
        return fourier_field(cfg, head, wl.grid, D) + 0.3 * g.standard_normal((S, D))
    if cfg == 3 and role in (ROLE_Q, ROLE_K):
        return g.standard_normal((S, D)) / np.sqrt(2.0)
    return g.standard_normal((S, D))


def tensor_bits(cfg: int, role: int, heads=None, workers: int | None = None) -> np.ndarray:
    """A (1, H', S, D) tensor of one role as stored bits.

    bf16 workloads return uint16 bit patterns; workload 1 returns float32.
    ``heads`` selects a subset of heads (default: all).  Heads are drawn from
    independent streams, so they are generated in parallel threads with no
    effect on the values.
    """
    import concurrent.futures as cf
    import os

    wl = WORKLOADS[cfg]
    heads = list(range(wl.H)) if heads is None else list(heads)
    f32 = wl.dtype == "f32"
    out = np.empty((1, len(heads), wl.S, wl.D), dtype=np.float32 if f32 else np.uint16)

    def one(i):
        x = head_f64(cfg, role, heads[i])
        out[0, i] = round_to_f32(x) if f32 else round_to_bf16_bits(x)

    n = workers or min(16, os.cpu_count() or 1, len(heads))
    if n <= 1:
        for i in range(len(heads)):
            one(i)
    else:
        with cf.ThreadPoolExecutor(max_workers=n) as ex:
            list(ex.map(one, range(len(heads))))
    return out


def stored_to_f64(arr: np.ndarray) -> np.ndarray:
    """Exact float64 view of what :func:`tensor_bits` returned."""
    if arr.dtype == np.uint16:
        return bf16_bits_to_f64(arr)
    return np.asarray(arr, dtype=np.float64)


def qkv(cfg: int, heads=None):
    """(q, k, v) as stored bits for a workload."""
    return tuple(tensor_bits(cfg, r, heads) for r in (ROLE_Q, ROLE_K, ROLE_V))


def normal_bits(shape, seed: int, scale: float = 1.0, dtype: str = "bf16") -> np.ndarray:
    """Small ad-hoc N(0, scale^2) tensors for edge-case tests (own seed space)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, 1000, seed])))
    x = g.standard_normal(shape) * scale
    if dtype == "f32":
        return round_to_f32(x)
    return round_to_bf16_bits(x)


def to_torch(arr: np.ndarray, device="cuda"):
    """Stored bits -> torch tensor of the workload dtype on ``device``."""
    import torch
    if arr.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


def from_torch(t) -> np.ndarray:
    """torch tensor -> stored-bits numpy array (uint16 for bf16)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
