"""Tile permutation kernels against the oracle: bit-exact."""
import numpy as np
import pytest

from block_sparse_attention_permute_amd import bsa, synth
from oracle import tiling as OT
from tests.gpu_helpers import bits, gpu, torch_gpu

CASES = [
    # grid, tiles, D, dtype, H
    ((8, 16, 16), [(2, 4, 4)], 64, "bf16", 8),                      # sliding-tile workload
    ((20, 32, 48), [(1, 8, 8), (4, 4, 4)], 128, "bf16", 40),         # Wan 2.1 shape, per-head choice
    ((32, 48, 80), [(4, 4, 4)], 128, "bf16", 24),                    # long sequence
    ((2, 4, 4), [(1, 2, 2), (2, 1, 4), (1, 1, 1)], 16, "f32", 3),    # fp32, three candidates
    ((3, 5, 7), [(3, 1, 7), (1, 5, 1)], 6, "bf16", 2),               # 12-byte rows
    ((4, 6, 10), [(2, 3, 5)], 3, "f32", 2),                          # 12-byte rows, odd tile
    ((2, 2, 6), [(1, 2, 3)], 1, "bf16", 5),                          # 2-byte rows
]


def _random_bits(shape, dtype, seed):
    g = np.random.default_rng(seed)
    if dtype == "bf16":
        return g.integers(0, 1 << 16, size=shape, dtype=np.uint16)    # any pattern: a pure copy
    return g.standard_normal(shape).astype(np.float32)


@pytest.mark.gpu
@pytest.mark.parametrize("grid,tiles,D,dtype,H", CASES)
def test_permute_and_invert_bit_exact(grid, tiles, D, dtype, H):
    torch = torch_gpu()
    S = int(np.prod(grid))
    x = _random_bits((1, H, S, D), dtype, seed=S + D)
    choice = (np.arange(H) * 7 % len(tiles)).astype(np.int32)
    hc = torch.from_numpy(choice).cuda() if len(tiles) > 1 else None
    xg = gpu(x)
    y = bsa.bsa_tile_permute(xg, grid, tiles, head_choice=hc)
    z = bsa.bsa_invert_permute(y, grid, tiles, head_choice=hc)
    torch.cuda.synchronize()
    yb, zb = bits(y), bits(z)
    perms = [OT.tile_permutation(grid, t) for t in tiles]
    for h in range(H):
        c = int(choice[h]) if hc is not None else 0
        assert np.array_equal(yb[0, h], OT.permute_tokens(x[0, h], perms[c])), h
    assert np.array_equal(zb, x)


@pytest.mark.gpu
def test_permute_batch_two_and_null_choice_uses_first_tiling():
    torch = torch_gpu()
    grid, tiles = (4, 8, 8), [(2, 4, 4), (1, 8, 8)]
    x = _random_bits((2, 3, 256, 64), "bf16", seed=5)
    y = bits(bsa.bsa_tile_permute(gpu(x), grid, tiles))
    perm = OT.tile_permutation(grid, tiles[0])
    assert np.array_equal(y, x[:, :, perm])
    choice = torch.tensor([[1, 0, 1], [0, 1, 1]], dtype=torch.int32, device="cuda")
    y2 = bits(bsa.bsa_tile_permute(gpu(x), grid, tiles, head_choice=choice))
    p1 = OT.tile_permutation(grid, tiles[1])
    for b in range(2):
        for h in range(3):
            want = x[b, h, p1] if int(choice[b, h]) == 1 else x[b, h, perm]
            assert np.array_equal(y2[b, h], want)
    bsa.bsa_validate_indices(choice.view(-1), 0, 2)
    with pytest.raises(RuntimeError):
        bsa.bsa_validate_indices(choice.view(-1), 0, 1)
