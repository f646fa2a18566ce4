"""Key-block norms: the summary passes' optional output, and block-sparse
attention given those norms, which skips the running-max update of the key
blocks whose scores provably cannot pass it.  The result must match the
oracle within the bf16 tolerance whatever the norms let the kernel skip."""
import numpy as np
import pytest

from block_sparse_attention_permute_amd import bsa, synth
from oracle import attention as OA
from oracle import tiling as OT
from tests.gpu_helpers import BF16_ATOL, f64, gpu, max_abs, torch_gpu

GRID, TILES = (4, 16, 16), [(1, 8, 8), (4, 4, 4)]


def _block_norm_max(x, block):
    """Largest row L2 norm of each block of consecutive rows, float64: x (H, S, D) -> (H, S // block)."""
    H, S, D = x.shape
    return np.linalg.norm(x.reshape(H, S // block, block, D), axis=-1).max(-1)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,D,block,S", [("bf16", 128, 64, 1024), ("bf16", 64, 32, 512), ("f32", 16, 8, 64),
                                             ("bf16", 128, 5, 200)])
def test_key_norms_from_summaries(dtype, D, block, S):
    torch = torch_gpu()
    H = 2
    q, k = (synth.normal_bits((1, H, S, D), seed=700 + i + S + D, dtype=dtype, scale=1.0 + i) for i in range(2))
    nb = S // block
    kn = torch.full((1, H, nb), -1.0, dtype=torch.float32, device="cuda")
    scores, _ = bsa.bsa_minmax_block_scores(gpu(q), gpu(k), block, key_norms=kn)
    want = _block_norm_max(synth.stored_to_f64(k)[0], block)
    assert np.allclose(kn.cpu().numpy()[0], want, rtol=1e-5, atol=0.0)
    # the scores are unchanged by the extra output
    s2, _ = bsa.bsa_minmax_block_scores(gpu(q), gpu(k), block)
    assert torch.equal(scores, s2)


@pytest.mark.gpu
def test_key_norms_tiled_and_masked():
    torch = torch_gpu()
    H, D, S = 2, 128, 1024
    nb = S // 64
    q, k = (synth.normal_bits((1, H, S, D), seed=730 + i) for i in range(2))
    kf = synth.stored_to_f64(k)[0]
    choice = torch.tensor([[0, 1]], dtype=torch.int32).cuda()
    kn = torch.full((1, H, nb), -1.0, dtype=torch.float32, device="cuda")
    bsa.bsa_minmax_block_scores_tiled(gpu(q), gpu(k), GRID, TILES, head_choice=choice, key_norms=kn)
    for h in range(H):
        perm = OT.tile_permutation(GRID, TILES[h])
        want = _block_norm_max(kf[h][perm][None], 64)[0]
        assert np.allclose(kn.cpu().numpy()[0, h], want, rtol=1e-5, atol=0.0), h
    # labelled tokens only: rows labelled < 0 are left out of the norms
    lab = np.zeros((1, H, S), np.int32)
    lab[..., 1::3] = -1
    kn2 = torch.full((1, H, nb), -1.0, dtype=torch.float32, device="cuda")
    bsa.bsa_minmax_block_scores(gpu(q), gpu(k), 64, labels=torch.from_numpy(lab).cuda(), key_norms=kn2)
    kz = np.where(lab[0][..., None] < 0, 0.0, kf)
    assert np.allclose(kn2.cpu().numpy()[0], _block_norm_max(kz, 64), rtol=1e-5, atol=0.0)


def _lists(keep):
    torch = torch_gpu()
    H, nq, nk = keep.shape
    cnt = keep.sum(-1).astype(np.int32)
    idx = np.full((1, H, nq, int(cnt.max())), -1, np.int32)
    for h in range(H):
        for i in range(nq):
            li = np.flatnonzero(keep[h, i])
            idx[0, h, i, :li.size] = li
    return torch.from_numpy(idx).cuda(), torch.from_numpy(cnt[None]).cuda()


def _case(seed, H=2, S=1024, D=128, hot=(3, 9), big=()):
    """q, k, v bits and a keep mask whose rows hold block 0, the diagonal and random blocks; key block J of
    `hot` repeats query block J (scores ~ |q|^2, far above the first block's: the running max grows), and
    the key blocks in `big` are scaled by 64 (their norm bound is far too large to skip)."""
    q, k, v = (synth.stored_to_f64(synth.normal_bits((1, H, S, D), seed=seed + i)) for i in range(3))
    nb = S // 64
    for J in hot:
        k[0, :, J * 64:(J + 1) * 64] = q[0, :, J * 64:(J + 1) * 64]
    for J in big:
        k[0, :, J * 64:(J + 1) * 64] *= 64.0
    rng = np.random.default_rng(seed)
    keep = rng.random((H, nb, nb)) < 0.3
    keep[:, :, 0] = True
    keep[:, np.arange(nb), np.arange(nb)] = True
    bits = [synth.round_to_bf16_bits(x) for x in (q, k, v)]
    return bits, keep


@pytest.mark.gpu
@pytest.mark.parametrize("big", [(), (2, 7)])
def test_attention_with_key_norms_matches_oracle(big):
    torch = torch_gpu()
    (q, k, v), keep = _case(900 + len(big), big=big)
    H, S, D = 2, 1024, 128
    nb = S // 64
    kv_idx, kv_cnt = _lists(keep)
    kn = torch.empty((1, H, nb), dtype=torch.float32, device="cuda")
    bsa.bsa_minmax_block_scores(gpu(q), gpu(k), 64, key_norms=kn)
    with_n = bsa.bsa_block_sparse_attention(gpu(q), gpu(k), gpu(v), kv_idx, kv_cnt, 64, key_norms=kn)
    without = bsa.bsa_block_sparse_attention(gpu(q), gpu(k), gpu(v), kv_idx, kv_cnt, 64)
    qf, kf, vf = (synth.stored_to_f64(x)[0] for x in (q, k, v))
    got = f64(with_n)[0]
    rows = np.arange(S)
    for h in range(H):
        want = OA.block_sparse_rows(qf[h], kf[h], vf[h], keep[h], 64, rows, D ** -0.5)
        assert max_abs(got[h], want) <= BF16_ATOL, h
    # the query blocks that meet a repeated key block take the skip where the plain kernel moves its max, so
    # the two differ by rounding somewhere (with scaled blocks, those dominate the rows that meet them and the
    # results may agree exactly)
    if not big:
        assert not torch.equal(with_n, without)
    # norms that prove nothing (NaN) leave the plain kernel's result, bit for bit
    nan = torch.full_like(kn, float("nan"))
    assert torch.equal(bsa.bsa_block_sparse_attention(gpu(q), gpu(k), gpu(v), kv_idx, kv_cnt, 64, key_norms=nan),
                       without)


@pytest.mark.gpu
def test_tiled_attention_with_key_norms_matches_permuted():
    """The gather-on-load kernel with the tiled summaries' norms equals the permuted kernel with the permuted
    summaries' norms, bit for bit, and both match the oracle."""
    torch = torch_gpu()
    (q, k, v), keep = _case(950)
    H, S, D = 2, 1024, 128
    nb = S // 64
    kv_idx, kv_cnt = _lists(keep)
    choice = torch.tensor([[0, 1]], dtype=torch.int32).cuda()
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    kn_t = torch.empty((1, H, nb), dtype=torch.float32, device="cuda")
    bsa.bsa_minmax_block_scores_tiled(qg, kg, GRID, TILES, head_choice=choice, key_norms=kn_t)
    out_t = bsa.bsa_block_sparse_attention_tiled(qg, kg, vg, GRID, TILES, kv_idx, kv_cnt, head_choice=choice,
                                                 key_norms=kn_t)
    qp, kp, vp = (bsa.bsa_tile_permute(x, GRID, TILES, head_choice=choice) for x in (qg, kg, vg))
    kn_p = torch.empty((1, H, nb), dtype=torch.float32, device="cuda")
    bsa.bsa_minmax_block_scores(qp, kp, 64, key_norms=kn_p)
    assert torch.equal(kn_t, kn_p)
    out_p = bsa.bsa_block_sparse_attention(qp, kp, vp, kv_idx, kv_cnt, 64, key_norms=kn_p)
    assert torch.equal(bsa.bsa_invert_permute(out_p, GRID, TILES, head_choice=choice), out_t)
    qf, kf, vf, of = (synth.stored_to_f64(x)[0] for x in (q, k, v, synth.from_torch(out_t)))
    for h in range(H):
        perm = OT.tile_permutation(GRID, TILES[h])
        want = OA.block_sparse_rows(qf[h][perm], kf[h][perm], vf[h][perm], keep[h], 64, np.arange(S), D ** -0.5)
        assert max_abs(of[h][perm], want) <= BF16_ATOL, h


@pytest.mark.gpu
def test_key_norms_shape_checked():
    torch = torch_gpu()
    (q, k, v), keep = _case(990, H=1, S=256)
    kv_idx, kv_cnt = _lists(keep)
    bad = torch.zeros((1, 1, 3), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="key_norms"):
        bsa.bsa_block_sparse_attention(gpu(q), gpu(k), gpu(v), kv_idx, kv_cnt, 64, key_norms=bad)
    with pytest.raises(ValueError, match="key_norms"):
        bsa.bsa_minmax_block_scores(gpu(q), gpu(k), 64, key_norms=bad.double())
