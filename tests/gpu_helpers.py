"""Shared helpers of the GPU parity tests (inputs, conversions, tolerances)."""
import numpy as np
import pytest

from block_sparse_attention_permute_amd import synth

BF16_ATOL = 2e-2   # max-abs error allowed on bf16 attention outputs
F32_ATOL = 1e-4    # max-abs error allowed on fp32 attention outputs
TOPK_REL = 1e-5    # relative score gap under which a top-k membership may differ


def torch_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("a GPU is required for the gpu-marked tests")
    return torch


def gpu(bits):
    return synth.to_torch(bits, "cuda")


def f64(t):
    """GPU tensor -> exact float64 numpy."""
    return synth.stored_to_f64(synth.from_torch(t))


def bits(t):
    return synth.from_torch(t)


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


TOPP_REL = 1e-5    # relative distance of the cumulative mass from p under which a top-p cut may differ


def top_p_row_ok(gpu_row, scores_row, p, scale, static_row, rel=TOPP_REL):
    """True if the GPU's kept row equals the oracle's top-p row, or differs
    only by moving the cut where the oracle's cumulative mass is within
    ``rel`` of p.  gpu_row, static_row: bool (Nk,); scores_row: float64."""
    from oracle import blocks as OB
    nk = scores_row.shape[0]
    want = OB.top_p_block_mask(scores_row[None, :], p, 0, 0, scale)[0] | static_row
    if np.array_equal(gpu_row, want):
        return True
    order, w = OB.top_p_ranked_mass(scores_row, scale)
    if w.sum() == 0.0:
        return False
    cum = np.cumsum(w) / w.sum()
    cuts = [c for c in range(1, nk + 1) if np.array_equal(np.isin(np.arange(nk), order[:c]) | static_row, gpu_row)]
    if not cuts:
        return False
    mo = OB.top_p_count(scores_row, p, scale)
    c = min(cuts, key=lambda x: abs(x - mo))
    return abs(cum[min(c, mo) - 1] - p) <= rel * p
