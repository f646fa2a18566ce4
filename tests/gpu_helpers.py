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
