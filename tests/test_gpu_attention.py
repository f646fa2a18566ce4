"""Block-sparse and windowed attention kernels against the oracle."""
import numpy as np
import pytest

from block_sparse_attention_permute_amd import bsa, synth
from oracle import attention as OA
from oracle import blocks as OB
from oracle import pipeline as OP
from oracle import tiling as OT
from tests.gpu_helpers import BF16_ATOL, F32_ATOL, f64, gpu, max_abs, torch_gpu


def _lists_to_keep(idx, cnt, nk):
    B, H, Nq, _ = idx.shape
    keep = np.zeros((B, H, Nq, nk), bool)
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                keep[b, h, i, idx[b, h, i, :cnt[b, h, i]]] = True
    return keep


def _keep_to_gpu_lists(keep):
    torch = torch_gpu()
    B, H, Nq, Nk = keep.shape
    cnt = keep.sum(-1).astype(np.int32)
    mk = max(int(cnt.max()), 1)
    idx = np.full((B, H, Nq, mk), -1, np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                li = np.flatnonzero(keep[b, h, i])
                idx[b, h, i, :li.size] = li
    return torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()


def _random_keep(B, H, nb, rng, density=0.3):
    keep = rng.random((B, H, nb, nb)) < density
    keep[..., np.arange(nb), np.arange(nb)] = True
    keep[:, :, 0] = True                                     # a full row
    if nb > 2:
        keep[:, :, 1] = False
        keep[:, :, 1, nb - 1] = True                         # a single-block row
    return keep


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,D,block,S,H", [("bf16", 128, 64, 1024, 3), ("bf16", 64, 64, 512, 2),
                                               ("bf16", 128, 32, 512, 2), ("bf16", 64, 32, 640, 3),
                                               ("f32", 16, 8, 64, 2), ("bf16", 16, 16, 128, 2),
                                               ("f32", 128, 64, 256, 1)])
def test_block_sparse_random_lists(dtype, D, block, S, H):
    torch_gpu()
    rng = np.random.default_rng(S + D + block)
    q, k, v = (synth.normal_bits((1, H, S, D), seed=100 + i + S, dtype=dtype) for i in range(3))
    keep = _random_keep(1, H, S // block, rng)
    kv_idx, kv_cnt = _keep_to_gpu_lists(keep)
    bsa.bsa_validate_block_list(kv_idx, kv_cnt, S // block)
    scale = None if D != 16 else 0.3
    out = bsa.bsa_block_sparse_attention(gpu(q), gpu(k), gpu(v), kv_idx, kv_cnt, block, scale=scale)
    want = OA.block_sparse_attention(*(synth.stored_to_f64(x) for x in (q, k, v)), keep, block, scale)
    tol = BF16_ATOL if dtype == "bf16" else F32_ATOL
    assert max_abs(f64(out), want) <= tol


@pytest.mark.gpu
@pytest.mark.parametrize("nb", [200, 260])
def test_block_sparse_long_lists(nb):
    """Lists longer than 64, 128 and 192 entries (and past 256, where another
    kernel takes over), checked on the rows of the longest-list blocks."""
    torch_gpu()
    block, D, H = 64, 128, 1
    S = nb * block
    rng = np.random.default_rng(nb)
    keep = rng.random((1, H, nb, nb)) < 0.8
    keep[..., np.arange(nb), np.arange(nb)] = True
    keep[:, :, 0] = True                                     # nb entries
    keep[:, :, 1] = False
    keep[:, :, 1, [0, 63, 64, 127, 128, 191, nb - 1]] = True  # the chunk edges
    q, k, v = (synth.normal_bits((1, H, S, D), seed=300 + i + nb) for i in range(3))
    kv_idx, kv_cnt = _keep_to_gpu_lists(keep)
    out = f64(bsa.bsa_block_sparse_attention(gpu(q), gpu(k), gpu(v), kv_idx, kv_cnt, block))
    qf, kf, vf = (synth.stored_to_f64(x)[0, 0] for x in (q, k, v))
    for qb in [0, 1, 2, nb // 2, nb - 1]:
        rows = np.arange(qb * block, (qb + 1) * block)
        want = OA.block_sparse_rows(qf, kf, vf, keep[0, 0], block, rows, D ** -0.5)
        assert max_abs(out[0, 0, rows], want) <= BF16_ATOL, qb


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,D,block", [("bf16", 128, 64), ("bf16", 64, 32), ("f32", 16, 32)])
def test_block_sparse_all_kept_equals_dense(dtype, D, block):
    torch_gpu()
    S, H = (32, 2) if dtype == "f32" else (512, 2)
    if dtype == "f32":
        q, k, v = synth.qkv(1)                               # the tiny fp32 workload, dense variant
    else:
        q, k, v = (synth.normal_bits((1, H, S, D), seed=200 + i) for i in range(3))
    keep = np.ones((1, H, S // block, S // block), bool)
    kv_idx, kv_cnt = _keep_to_gpu_lists(keep)
    out = bsa.bsa_block_sparse_attention(gpu(q), gpu(k), gpu(v), kv_idx, kv_cnt, block)
    want = OA.full_attention(*(synth.stored_to_f64(x) for x in (q, k, v)))
    assert max_abs(f64(out), want) <= (BF16_ATOL if dtype == "bf16" else F32_ATOL)


@pytest.mark.gpu
def test_sliding_tile_workload_end_to_end():
    """grid 8x16x16, tiles 2x4x4 (block 32), 3x3x3 tile neighbourhood, D=64, H=8: every output checked."""
    torch_gpu()
    grid, tile, block = (8, 16, 16), (2, 4, 4), 32
    q, k, v = synth.qkv(2)
    tg = (8 // 2, 16 // 4, 16 // 4)
    idx, cnt = bsa.bsa_sliding_tile_block_list(tg)
    H, nb = 8, 64
    torch = torch_gpu()
    kv_idx = torch.from_numpy(np.broadcast_to(idx, (1, H) + idx.shape).copy()).cuda()
    kv_cnt = torch.from_numpy(np.broadcast_to(cnt, (1, H, nb)).copy()).cuda()
    bsa.bsa_validate_block_list(kv_idx, kv_cnt, nb)
    qp, kp, vp = (bsa.bsa_tile_permute(gpu(x), grid, [tile]) for x in (q, k, v))
    op = bsa.bsa_block_sparse_attention(qp, kp, vp, kv_idx, kv_cnt, block)
    out = f64(bsa.bsa_invert_permute(op, grid, [tile]))
    keep = OT.sliding_tile_keep(tg)
    labels = OT.tile_labels(grid, tile)
    qf, kf, vf = (synth.stored_to_f64(x) for x in (q, k, v))
    assert int(keep.sum()) == 1000
    for h in range(H):
        want = OP.label_mask_attention(qf[0, h], kf[0, h], vf[0, h], labels, keep, 64 ** -0.5)
        assert max_abs(out[0, h], want) <= BF16_ATOL, h


# --------------------------------------------------------------- windowed ---

@pytest.mark.gpu
def test_windowed_tiny_fp32_workload():
    torch_gpu()
    q, k, v = synth.qkv(1)
    out = bsa.bsa_windowed_attention(gpu(q), gpu(k), gpu(v), window=8, sink=2, scale=0.25, chunk=8)
    want = OA.windowed_attention(*(synth.stored_to_f64(x) for x in (q, k, v)), 8, 2, scale=0.25, chunk=8)
    assert max_abs(f64(out), want) <= F32_ATOL


@pytest.mark.gpu
@pytest.mark.parametrize("S,D,window,sink", [(1000, 128, 130, 3), (512, 64, 64, 0), (512, 128, 8, 100),
                                             (700, 64, 1, 0), (333, 128, 2 * 333 - 1, 0), (256, 128, 3, 256),
                                             (100, 128, 500, 7), (64, 64, 64, 64), (1, 128, 1, 0)])
def test_windowed_small_against_dense_masked(S, D, window, sink):
    torch_gpu()
    H = 2
    q, k, v = (synth.normal_bits((1, H, S, D), seed=300 + i + S + window) for i in range(3))
    out = bsa.bsa_windowed_attention(gpu(q), gpu(k), gpu(v), window=window, sink=sink)
    want = OA.windowed_attention(*(synth.stored_to_f64(x) for x in (q, k, v)), window, sink)
    assert max_abs(f64(out), want) <= BF16_ATOL


@pytest.mark.gpu
def test_windowed_chunk_does_not_change_result_and_dense_limits():
    torch = torch_gpu()
    S, D = 1024, 128
    q, k, v = (gpu(synth.normal_bits((1, 2, S, D), seed=400 + i)) for i in range(3))
    outs = [bsa.bsa_windowed_attention(q, k, v, 256, 16, chunk=c) for c in (None, 1, 8, 512, S)]
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    dense = f64(bsa.bsa_windowed_attention(q, k, v, 2 * S - 1, 0))
    want = OA.full_attention(*(f64(x) for x in (q, k, v)))
    assert max_abs(dense, want) <= BF16_ATOL
    assert max_abs(f64(bsa.bsa_windowed_attention(q, k, v, 1, S)), want) <= BF16_ATOL


@pytest.mark.gpu
def test_windowed_workload_sampled_rows():
    """S=16384, window 2048, sink 64, D=128, H=24 in one launch; sampled rows of a few heads."""
    torch_gpu()
    q, k, v = synth.qkv(3)
    out = f64(bsa.bsa_windowed_attention(gpu(q), gpu(k), gpu(v), window=2048, sink=64, scale=128 ** -0.5,
                                         chunk=512))
    rows = np.array([0, 1, 63, 64, 65, 1023, 1024, 1087, 1088, 1089, 1150, 5000, 8191, 16000, 16383])
    for h in (0, 11, 23):
        qf, kf, vf = (synth.stored_to_f64(x[0, h]) for x in (q, k, v))
        want = OA.window_rows(qf, kf, vf, rows, 2048, 64, 128 ** -0.5)
        assert max_abs(out[0, h, rows], want) <= BF16_ATOL, h


@pytest.mark.gpu
@pytest.mark.parametrize("tiled", [False, True])
def test_block_sparse_short_and_empty_lists(tiled):
    """Lists of 0 to 4 key blocks, on the permuted and the gather-on-load
    paths: a query block with an empty list is written as zeros, every other
    row matches the oracle."""
    torch = torch_gpu()
    grid, tiles = (4, 16, 16), [(1, 8, 8), (4, 4, 4)]
    H, D, block = 2, 128, 64
    S = 4 * 16 * 16
    nb = S // block
    rng = np.random.default_rng(31 + tiled)
    keep = np.zeros((1, H, nb, nb), bool)
    for h in range(H):
        for I in range(nb):
            n = I % 5                                       # 0, 1, 2, 3, 4 blocks
            keep[0, h, I, rng.choice(nb, size=n, replace=False)] = True
    q, k, v = (synth.normal_bits((1, H, S, D), seed=520 + i + 10 * tiled) for i in range(3))
    kv_idx, kv_cnt = _keep_to_gpu_lists(keep)
    choice = torch.tensor([[0, 1]], dtype=torch.int32).cuda()
    if tiled:
        out = f64(bsa.bsa_block_sparse_attention_tiled(gpu(q), gpu(k), gpu(v), grid, tiles, kv_idx, kv_cnt,
                                                       head_choice=choice))
    else:
        out = f64(bsa.bsa_block_sparse_attention(gpu(q), gpu(k), gpu(v), kv_idx, kv_cnt, block))
    qf, kf, vf = (synth.stored_to_f64(x)[0] for x in (q, k, v))
    for h in range(H):
        # rows of the head in block order: the tile order of its tiling (tiled), or T-major
        perm = OT.tile_permutation(grid, tiles[h]) if tiled else np.arange(S)
        qh, kh, vh, oh = qf[h][perm], kf[h][perm], vf[h][perm], out[0, h][perm]
        empty = np.flatnonzero(~keep[0, h].any(-1))
        assert empty.size > 0
        for I in empty:
            assert np.all(oh[I * block:(I + 1) * block] == 0.0), (h, I)
        rows = np.concatenate([np.arange(I * block, (I + 1) * block) for I in range(nb) if keep[0, h, I].any()])
        want = OA.block_sparse_rows(qh, kh, vh, keep[0, h], block, rows, D ** -0.5)
        assert max_abs(oh[rows], want) <= BF16_ATOL, h


@pytest.mark.gpu
@pytest.mark.parametrize("D,block,S", [(64, 32, 640), (128, 32, 512), (64, 64, 512), (32, 32, 256)])
def test_block_sparse_empty_lists_other_kernels(D, block, S):
    """Lists of 0 to 3 key blocks on the four-wave MFMA kernel (D = 64 or blocks of 32) and the scalar
    kernel (D = 32): a query block with an empty list is written as zeros, every other row matches."""
    torch_gpu()
    H = 2
    nb = S // block
    rng = np.random.default_rng(41 + D + block)
    keep = np.zeros((1, H, nb, nb), bool)
    for h in range(H):
        for I in range(nb):
            keep[0, h, I, rng.choice(nb, size=I % 4, replace=False)] = True
    q, k, v = (synth.normal_bits((1, H, S, D), seed=540 + i + D + block) for i in range(3))
    kv_idx, kv_cnt = _keep_to_gpu_lists(keep)
    out = f64(bsa.bsa_block_sparse_attention(gpu(q), gpu(k), gpu(v), kv_idx, kv_cnt, block))
    assert np.all(np.isfinite(out))
    qf, kf, vf = (synth.stored_to_f64(x)[0] for x in (q, k, v))
    for h in range(H):
        empty = np.flatnonzero(~keep[0, h].any(-1))
        assert empty.size > 0
        for I in empty:
            assert np.all(out[0, h, I * block:(I + 1) * block] == 0.0), (h, I)
        rows = np.concatenate([np.arange(I * block, (I + 1) * block) for I in range(nb) if keep[0, h, I].any()])
        want = OA.block_sparse_rows_gathered(qf[h], kf[h], vf[h], keep[0, h], block, rows, D ** -0.5)
        assert max_abs(out[0, h, rows], want) <= BF16_ATOL, h


@pytest.mark.gpu
@pytest.mark.parametrize("scale", [0.0, -0.06, -0.2])
@pytest.mark.parametrize("D,block", [(128, 64), (64, 32), (64, 64)])
def test_block_sparse_non_positive_scale(scale, D, block):
    """An explicit scale is used as given, also when it is 0 (uniform weights over the visible keys) or
    negative; the kernels' non-positive-scale paths, with and without key norms."""
    torch = torch_gpu()
    H, S = 2, 1024
    rng = np.random.default_rng(int(D + block - 100 * scale))
    q, k, v = (synth.normal_bits((1, H, S, D), seed=560 + i + D) for i in range(3))
    keep = _random_keep(1, H, S // block, rng)
    kv_idx, kv_cnt = _keep_to_gpu_lists(keep)
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    out = bsa.bsa_block_sparse_attention(qg, kg, vg, kv_idx, kv_cnt, block, scale=scale)
    want = OA.block_sparse_attention(*(synth.stored_to_f64(x) for x in (q, k, v)), keep, block, scale)
    assert max_abs(f64(out), want) <= BF16_ATOL
    if scale == 0.0:                                  # uniform weights: the mean of the visible values
        vf = synth.stored_to_f64(v)[0, 0]
        I = 0
        keys = np.concatenate([np.arange(J * block, (J + 1) * block) for J in np.flatnonzero(keep[0, 0, I])])
        assert max_abs(f64(out)[0, 0, :block], np.broadcast_to(vf[keys].mean(0), (block, D))) <= BF16_ATOL
    norms = torch.full((1, H, S // block), 1e3, dtype=torch.float32, device="cuda")
    out2 = bsa.bsa_block_sparse_attention(qg, kg, vg, kv_idx, kv_cnt, block, scale=scale, key_norms=norms)
    assert torch.equal(out, out2)                     # the key-norm bound only applies to positive scales


@pytest.mark.gpu
@pytest.mark.parametrize("scale", [0.0, -0.08])
@pytest.mark.parametrize("D", [128, 64])
def test_windowed_non_positive_scale(scale, D):
    torch_gpu()
    H, S, window, sink = 2, 700, 130, 5
    q, k, v = (synth.normal_bits((1, H, S, D), seed=580 + i + D) for i in range(3))
    out = bsa.bsa_windowed_attention(gpu(q), gpu(k), gpu(v), window=window, sink=sink, scale=scale)
    want = OA.windowed_attention(*(synth.stored_to_f64(x) for x in (q, k, v)), window, sink, scale=scale)
    assert max_abs(f64(out), want) <= BF16_ATOL


@pytest.mark.gpu
def test_windowed_workload_every_row_of_one_head():
    """S=16384, window 2048, sink 64, D=128, H=24 in one launch: every output row of head 5 against the
    oracle (window-slice form), and sampled rows of two more heads."""
    torch_gpu()
    q, k, v = synth.qkv(3)
    out = f64(bsa.bsa_windowed_attention(gpu(q), gpu(k), gpu(v), window=2048, sink=64, scale=128 ** -0.5,
                                         chunk=512))
    S = 16384
    for h, rows in ((5, np.arange(S)), (0, np.arange(0, S, 97)), (23, np.arange(40, S, 131))):
        qf, kf, vf = (synth.stored_to_f64(x[0, h]) for x in (q, k, v))
        want = OA.window_rows_gathered(qf, kf, vf, rows, 2048, 64, 128 ** -0.5)
        assert max_abs(out[0, h, rows], want) <= BF16_ATOL, h


def _lists_full_width(keep):
    """Compact lists of width Nk (a list may hold every block), entries past the count -1."""
    torch = torch_gpu()
    B, H, Nq, Nk = keep.shape
    cnt = keep.sum(-1).astype(np.int32)
    idx = np.full((B, H, Nq, Nk), -1, np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                li = np.flatnonzero(keep[b, h, i])
                idx[b, h, i, :li.size] = li
    return torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()


@pytest.mark.gpu
def test_lists_of_any_length_every_output():
    """Lists as wide as the key-block count (their lengths vary with the data, as top-p's do): the kernel
    then spreads each head over four XCDs.  Lengths 0 to Nq, with and without key norms, on permuted and
    T-major tensors (equal bit for bit), every output against the oracle."""
    torch = torch_gpu()
    grid, tiles, H, D = (4, 32, 32), [(1, 8, 8), (4, 4, 4)], 4, 128
    S, nb = 4096, 64
    rng = np.random.default_rng(4242)
    dens = rng.random((1, H, nb, 1)) ** 3                    # rows from nearly empty to full
    keep = rng.random((1, H, nb, nb)) < dens
    keep[0, 0, 3] = False                                    # an empty list
    keep[0, 1, 5] = True                                     # a full list
    q, k, v = (synth.normal_bits((1, H, S, D), seed=4300 + i) for i in range(3))
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    kv_idx, kv_cnt = _lists_full_width(keep)
    assert kv_idx.shape[-1] == nb
    kn = torch.full((1, H, nb), -1.0, dtype=torch.float32, device="cuda")
    bsa.bsa_minmax_block_scores(qg, kg, 64, key_norms=kn)
    qf, kf, vf = (synth.stored_to_f64(x) for x in (q, k, v))

    def check(o, h, q_h, k_h, v_h, perm=None):
        """Rows of query blocks with keys against the oracle; an empty list's rows are zeros."""
        seen = keep[0, h].any(-1)
        rows = np.flatnonzero(np.repeat(seen, 64))
        want = OA.block_sparse_rows_gathered(q_h, k_h, v_h, keep[0, h], 64, rows, D ** -0.5)
        got = o[0, h] if perm is None else o[0, h, perm]
        assert max_abs(got[rows], want) <= BF16_ATOL, h
        assert np.all(got[np.repeat(~seen, 64)] == 0.0), h

    assert not keep[0, 0, 3].any()
    for norms in (None, kn):
        out = f64(bsa.bsa_block_sparse_attention(qg, kg, vg, kv_idx, kv_cnt, 64, key_norms=norms))
        for h in range(H):
            check(out, h, qf[0, h], kf[0, h], vf[0, h])
    choice = torch.tensor([[0, 1, 1, 0]], dtype=torch.int32, device="cuda")
    out_t = bsa.bsa_block_sparse_attention_tiled(qg, kg, vg, grid, tiles, kv_idx, kv_cnt, head_choice=choice)
    qp, kp, vp = (bsa.bsa_tile_permute(x, grid, tiles, head_choice=choice) for x in (qg, kg, vg))
    ref = bsa.bsa_invert_permute(bsa.bsa_block_sparse_attention(qp, kp, vp, kv_idx, kv_cnt, 64), grid, tiles,
                                 head_choice=choice)
    assert torch.equal(out_t, ref)
    o = f64(out_t)
    for h in range(H):
        perm = OT.tile_permutation(grid, tiles[int(choice[0, h])])
        check(o, h, *(OT.permute_tokens(x[0, h], perm) for x in (qf, kf, vf)), perm=perm)


@pytest.mark.gpu
@pytest.mark.parametrize("norms", [False, True])
def test_long_head_late_v_schedule(norms):
    """A head whose K and V exceed 32 MB (S = 69632, D = 128) takes the schedule that issues each tile's V
    DMA beside its own score MFMAs: T-major (17x64x64 grid, tiles 1x8x8) equals permuted bit for bit, and
    the first and last row of every 16th query block, plus all rows of three blocks, match the oracle."""
    torch = torch_gpu()
    grid, tiles, H, D = (17, 64, 64), [(1, 8, 8)], 1, 128
    S = 17 * 64 * 64
    nb = S // 64
    assert S * D * 4 > (32 << 20)
    rng = np.random.default_rng(6969)
    keep = rng.random((1, H, nb, nb)) < 0.02
    keep[..., np.arange(nb), np.arange(nb)] = True
    keep[..., 0] = True
    q, k, v = (synth.normal_bits((1, H, S, D), seed=6970 + i) for i in range(3))
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    kv_idx, kv_cnt = _keep_to_gpu_lists(keep)
    qp, kp, vp = (bsa.bsa_tile_permute(x, grid, tiles) for x in (qg, kg, vg))
    kn = None
    if norms:
        kn = torch.full((1, H, nb), -1.0, dtype=torch.float32, device="cuda")
        bsa.bsa_minmax_block_scores(qp, kp, 64, key_norms=kn)
    outp = bsa.bsa_block_sparse_attention(qp, kp, vp, kv_idx, kv_cnt, 64, key_norms=kn)
    out_t = bsa.bsa_block_sparse_attention_tiled(qg, kg, vg, grid, tiles, kv_idx, kv_cnt, key_norms=kn)
    assert torch.equal(out_t, bsa.bsa_invert_permute(outp, grid, tiles))
    perm = OT.tile_permutation(grid, tiles[0])
    qf, kf, vf = (OT.permute_tokens(synth.stored_to_f64(x)[0, 0], perm) for x in (q, k, v))
    blocks = np.arange(0, nb, 16)
    rows = np.concatenate([np.stack([blocks * 64, blocks * 64 + 63], 1).ravel(),
                           np.arange(64), np.arange(nb // 2 * 64, nb // 2 * 64 + 64), np.arange(S - 64, S)])
    rows = np.unique(rows)
    want = OA.block_sparse_rows_gathered(qf, kf, vf, keep[0, 0], 64, rows, D ** -0.5)
    assert max_abs(f64(outp)[0, 0, rows], want) <= BF16_ATOL
