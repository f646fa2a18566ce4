"""bsa_select_tiling_noalloc, the entry point for callers that cannot allocate, against bsa_select_tiling.

Through the C ABI: the same choices and scores bit for bit on two calls in a row, the second smaller (the
fixed scratch keeps the first call's values, which the second must not read); sizes past the fixed scratch
are rejected on the host before any launch.
"""
import ctypes

import pytest

from block_sparse_attention_permute_amd import bsa, synth
from tests.gpu_helpers import gpu, torch_gpu


def _both(torch, q, grid, tiles):
    choice, score, _ = bsa.bsa_select_tiling(q, grid, tiles)
    B, H = q.shape[:2]
    c2 = torch.full((B, H), -7, dtype=torch.int32, device="cuda")
    s2 = torch.full((B, H, len(tiles)), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    bsa.bsa_select_tiling_noalloc(q, grid, tiles, out=(c2, s2))
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return choice, score, c2, s2


@pytest.mark.gpu
def test_select_tiling_noalloc_matches_workspace_call():
    torch = torch_gpu()
    # first call: the Wan shape, all 40 heads, two candidates (38,400 per-tile values)
    q = gpu(synth.tensor_bits(4, synth.ROLE_Q))
    c1, s1, c2, s2 = _both(torch, q, (20, 32, 48), [(1, 8, 8), (4, 4, 4)])
    assert torch.equal(c1, c2) and torch.equal(s1, s2)
    assert set(c2.cpu().numpy().ravel().tolist()) == {0, 1}
    # second call, smaller: B = 2, three candidates of 32 tokens, D = 64, one all-zero head (-inf scores)
    qb = synth.normal_bits((2, 3, 256, 64), seed=950)
    qb[1, 2] = 0
    c1, s1, c2, s2 = _both(torch, gpu(qb), (4, 8, 8), [(1, 4, 8), (4, 2, 4), (2, 4, 4)])
    assert torch.equal(c1, c2) and torch.equal(s1, s2)
    assert bool(torch.isinf(s2[1, 2]).all())
    # and the first shape again after the smaller one
    c1, s1, c2, s2 = _both(torch, q[:, :7].contiguous(), (20, 32, 48), [(4, 4, 4), (1, 8, 8)])
    assert torch.equal(c1, c2) and torch.equal(s1, s2)


def test_select_tiling_noalloc_rejects_sizes_past_the_scratch():
    if not __import__("os").path.exists(bsa.LIB_PATH):
        pytest.fail("libbsa.so is not built")
    L = bsa.lib()
    fake = ctypes.c_void_p(4096)                    # never dereferenced: the call fails validation first
    one = (ctypes.c_int32 * 3)(1, 1, 1)
    # 2048 heads x 1024 tiles = 2^21 per-tile values > 2^20
    rc = L.bsa_select_tiling_noalloc(fake, bsa.BSA_BF16, 1, 2048, 1, 1, 1024, 16, one, 1, fake, fake, None)
    assert rc == bsa.BSA_ERR_INVALID_ARG
    assert "scratch" in L.bsa_last_error().decode()
    bad = (ctypes.c_int32 * 3)(3, 1, 1)               # does not divide T = 1
    assert L.bsa_select_tiling_noalloc(fake, bsa.BSA_BF16, 1, 1, 1, 1, 64, 16, bad, 1, fake, fake,
                                       None) == bsa.BSA_ERR_INVALID_ARG
