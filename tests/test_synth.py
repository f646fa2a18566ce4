"""The seeded input generators: exact bf16 rounding and reproducibility (CPU only)."""
import numpy as np
import torch

from block_sparse_attention_permute_amd import synth


def test_bf16_rounding_matches_torch_on_float32_values():
    # torch's float32 -> bfloat16 conversion rounds to nearest even; on values
    # that are exact in float32 a single rounding from float64 must agree.
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    x = np.concatenate([x, np.float32([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0, 65504.0])])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.round_to_bf16_bits(x.astype(np.float64)), want)


def test_bf16_rounding_ties_and_roundtrip():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0
    assert synth.bf16_bits_to_f64(synth.round_to_bf16_bits(np.array([1.0 + 2 ** -8]))) == 1.0
    assert synth.bf16_bits_to_f64(synth.round_to_bf16_bits(np.array([1.0 + 3 * 2 ** -8]))) == 1.0 + 2 ** -6
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    vals = synth.bf16_bits_to_f64(bits)
    finite = np.isfinite(vals)
    back = synth.round_to_bf16_bits(vals[finite])
    same = (back == bits[finite]) | (vals[finite] == 0)
    assert np.all(same)


def test_generators_are_seeded_and_per_head():
    a = synth.tensor_bits(2, synth.ROLE_Q, heads=[3])
    b = synth.tensor_bits(2, synth.ROLE_Q, heads=[1, 3])
    assert np.array_equal(a[0, 0], b[0, 1])
    assert not np.array_equal(b[0, 0], b[0, 1])
    q = synth.stored_to_f64(synth.tensor_bits(1, synth.ROLE_Q))
    assert q.shape == (1, 2, 32, 16) and abs(q.std() - 1.0) < 0.2


def test_fourier_recipe_has_unit_scale_and_locality():
    wl = synth.WORKLOADS[4]
    f = synth.fourier_field(4, 0, wl.grid, wl.D)
    assert 0.5 < f.std() < 1.6
    q = synth.stored_to_f64(synth.tensor_bits(4, synth.ROLE_Q, heads=[0]))[0, 0]
    k = synth.stored_to_f64(synth.tensor_bits(4, synth.ROLE_K, heads=[0]))[0, 0]
    # q and k share the field: strongly correlated, not identical
    c = np.corrcoef(q.ravel(), k.ravel())[0, 1]
    assert 0.8 < c < 0.99
