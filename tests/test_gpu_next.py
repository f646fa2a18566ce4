"""Padded grids, the pooled statistic, per-head budgets, label-masked
attention and the spatial-only / temporal-only masks, against the oracle."""
import numpy as np
import pytest

from block_sparse_attention_permute_amd import bsa, synth
from oracle import attention as OA
from oracle import blocks as OB
from oracle import pipeline as OP
from oracle import tiling as OT
from tests.gpu_helpers import BF16_ATOL, F32_ATOL, TOPK_REL, f64, gpu, max_abs, torch_gpu

WAN_GRID = (20, 32, 48)


def _gather_padded(x_head, perm):
    valid = perm >= 0
    return np.where(valid[:, None], x_head[np.where(valid, perm, 0)], 0.0)


# --------------------------------------------------------------- permutes ---

@pytest.mark.gpu
@pytest.mark.parametrize("dtype,grid,tiles", [("bf16", (3, 5, 6), [(2, 2, 4), (1, 4, 8)]),
                                              ("f32", (5, 3, 7), [(2, 2, 2), (4, 1, 3), (5, 3, 7)]),
                                              ("bf16", (20, 32, 48), [(16, 2, 2), (1, 8, 8)])])
def test_padded_permute_roundtrip(dtype, grid, tiles):
    torch = torch_gpu()
    T, Hg, Wg = grid
    S, H = T * Hg * Wg, 4
    D = 128 if S > 10000 else 16
    x = synth.normal_bits((1, H, S, D), seed=S + D, dtype=dtype)
    choice = torch.tensor([[h % len(tiles) for h in range(H)]], dtype=torch.int32).cuda()
    y, lab = bsa.bsa_tile_permute_padded(gpu(x), grid, tiles, head_choice=choice)
    Sp = max(int(np.prod(OT.padded_grid(grid, t))) for t in tiles)
    assert tuple(y.shape) == (1, H, Sp, D)
    yb, lb = f64(y), lab.cpu().numpy()
    xf = synth.stored_to_f64(x)
    for h in range(H):
        perm = OT.padded_tile_permutation(grid, tiles[h % len(tiles)])
        perm = np.concatenate([perm, -np.ones(Sp - perm.size, np.int64)])
        assert np.array_equal(yb[0, h], _gather_padded(xf[0, h], perm))
        assert np.array_equal(lb[0, h], np.where(perm >= 0, 0, -1))
    back = bsa.bsa_invert_permute_padded(y, grid, tiles, head_choice=choice)
    assert np.array_equal(synth.from_torch(back), x)


# ------------------------------------------------------ tiling selection ---

@pytest.mark.gpu
@pytest.mark.parametrize("statistic,pad", [("pooled", False), ("mean", True), ("pooled", True)])
def test_select_tiling_pooled_and_padded(statistic, pad):
    torch = torch_gpu()
    grid = (4, 8, 8) if not pad else (5, 9, 10)
    tiles = [(1, 4, 8), (4, 2, 4), (2, 4, 4)]
    S = int(np.prod(grid))
    q = synth.normal_bits((1, 4, S, 64), seed=700 + int(pad))
    q[0, 1, :40] = 0                                        # zero-norm tokens: counted by pooled, not by mean
    choice, score, _ = bsa.bsa_select_tiling(gpu(q), grid, tiles, statistic=statistic, pad=pad)
    oc, osc = OT.select_tiling(synth.stored_to_f64(q), grid, tiles, statistic=statistic, pad=pad)
    got = score.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got - osc)) < 2e-5
    ch = choice.cpu().numpy()
    for h in range(4):
        if ch[0, h] != oc[0, h]:
            a, b = osc[0, h, ch[0, h]], osc[0, h, oc[0, h]]
            assert abs(a - b) < TOPK_REL * abs(b)


@pytest.mark.gpu
def test_select_tiling_wan_shape_with_padded_candidate():
    """Wan 2.1 grid with all three SPADE candidates; (16, 2, 2) scored on the padded grid."""
    torch = torch_gpu()
    heads = [0, 3, 9, 21]
    tiles = [(1, 8, 8), (4, 4, 4), (16, 2, 2)]
    q = synth.tensor_bits(4, synth.ROLE_Q, heads=heads)
    for statistic in ("mean", "pooled"):
        choice, score, _ = bsa.bsa_select_tiling(gpu(q), WAN_GRID, tiles, statistic=statistic, pad=True)
        oc, osc = OT.select_tiling(synth.stored_to_f64(q), WAN_GRID, tiles, statistic=statistic, pad=True)
        assert np.max(np.abs(score.cpu().numpy() - osc)) < 2e-5
        ch = choice.cpu().numpy()
        for h in range(len(heads)):
            if ch[0, h] != oc[0, h]:
                a, b = osc[0, h, ch[0, h]], osc[0, h, oc[0, h]]
                assert abs(a - b) < TOPK_REL * abs(b)


# ------------------------------------------------------- masked summaries ---

@pytest.mark.gpu
def test_minmax_scores_masked():
    torch = torch_gpu()
    S, D, block = 640, 128, 64
    q, k = (synth.normal_bits((1, 2, S, D), seed=710 + i) for i in range(2))
    rng = np.random.default_rng(3)
    lab = np.where(rng.random((1, 2, S)) < 0.2, -1, 0).astype(np.int32)
    lab[0, 0, 128:192] = -1                                   # a block with no real token
    scores, summ = bsa.bsa_minmax_block_scores(gpu(q), gpu(k), block, labels=torch.from_numpy(lab).cuda())
    got = scores.cpu().numpy().astype(np.float64)[0]
    qf, kf = synth.stored_to_f64(q), synth.stored_to_f64(k)
    for h in range(2):
        valid = lab[0, h] >= 0
        nb = S // block
        ok = np.array([valid[i * block:(i + 1) * block].any() for i in range(nb)])
        want = np.full((nb, nb), -np.inf)
        vq = np.where(ok.repeat(block), valid, True)        # the oracle needs a token per block
        sub = OB.minmax_block_scores_valid(qf[0, h], kf[0, h], vq, block)
        want[np.ix_(ok, ok)] = sub[np.ix_(ok, ok)]
        assert np.array_equal(np.isinf(got[h]), np.isinf(want))
        fin = np.isfinite(want)
        # fp32 dot products of length D: error <= (D + 2) u sum_d |c_d| max(|kmax_d|, |kmin_d|)
        qmax, qmin = OB.block_minmax_valid(qf[0, h], vq, block)
        kmax, kmin = OB.block_minmax_valid(kf[0, h], vq, block)
        bound = np.abs(qmax + qmin) @ np.maximum(np.abs(kmax), np.abs(kmin)).T
        err = np.abs(got[h] - np.where(fin, want, 0.0))
        assert np.all(err[fin] <= (D + 2) * 2.0 ** -24 * bound[fin] + 1e-30)


# ------------------------------------------------------- per-head budgets ---

@pytest.mark.gpu
def test_topk_tiled_per_head_budgets():
    torch = torch_gpu()
    rng = np.random.default_rng(5)
    B, H, N = 1, 4, 300
    s = (rng.standard_normal((B, H, N, N)) * 10).astype(np.float32)
    choice = np.array([[0, 1, 2, 1]], np.int32)
    k_tab, nk_tab = [40, 12, 70], [300, 100, 250]
    kv_idx, kv_cnt, mask = bsa.bsa_topk_block_mask_tiled(torch.from_numpy(s).cuda(), torch.from_numpy(choice).cuda(),
                                                         k_tab, nk_tab, 5, 40, return_mask=True)
    idx, cnt, m = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy(), mask.cpu().numpy().astype(bool)
    for h in range(H):
        c = choice[0, h]
        nk, k = nk_tab[c], k_tab[c]
        keep = OB.topk_block_mask(s[0, h, :nk, :nk].astype(np.float64), k, 5, 40)
        assert np.array_equal(m[0, h, :nk, :nk], keep)
        assert not m[0, h, :, nk:].any() and not m[0, h, nk:].any()
        assert np.all(cnt[0, h, nk:] == 0)
        for I in range(nk):
            li = np.flatnonzero(keep[I])
            assert cnt[0, h, I] == li.size and np.array_equal(idx[0, h, I, :li.size], li)


# ------------------------------------------------- label-masked attention ---

@pytest.mark.gpu
@pytest.mark.parametrize("dtype,D,block,shared", [("bf16", 128, 64, True), ("bf16", 128, 64, False),
                                                  ("bf16", 64, 32, False), ("f32", 16, 16, True)])
def test_block_sparse_attention_labels(dtype, D, block, shared):
    torch = torch_gpu()
    S, H = 512, 2
    rng = np.random.default_rng(D + block)
    q, k, v = (synth.normal_bits((1, H, S, D), seed=720 + i, dtype=dtype) for i in range(3))
    nb = S // block
    keep = rng.random((1, H, nb, nb)) < 0.5
    keep[..., np.arange(nb), np.arange(nb)] = True
    lab = rng.integers(0, 3, (1, H, S)).astype(np.int32)
    lab[:, :, 5] = -1                                   # a padding token
    lab[:, :, 7] = 9                                    # a label found nowhere else: its row sees only itself
    if shared:
        lab[:, 1] = lab[:, 0]
    cnt = keep.sum(-1).astype(np.int32)
    idx = np.full((1, H, nb, nb), -1, np.int32)
    for h in range(H):
        for I in range(nb):
            li = np.flatnonzero(keep[0, h, I])
            idx[0, h, I, :li.size] = li
    lt = torch.from_numpy(lab[0, 0] if shared else lab).cuda()
    out = bsa.bsa_block_sparse_attention_labels(gpu(q), gpu(k), gpu(v), torch.from_numpy(idx).cuda(),
                                                torch.from_numpy(cnt).cuda(), block, lt)
    got = f64(out)
    qf, kf, vf = (synth.stored_to_f64(x) for x in (q, k, v))
    tol = BF16_ATOL if dtype == "bf16" else F32_ATOL
    for h in range(H):
        want = OP.label_equal_attention(qf[0, h], kf[0, h], vf[0, h], lab[0, h], D ** -0.5, keep[0, h], block)
        assert max_abs(got[0, h], want) <= tol, h


@pytest.mark.gpu
def test_labels_row_without_keys_is_zero():
    torch = torch_gpu()
    S, D = 128, 128
    q, k, v = (synth.normal_bits((1, 1, S, D), seed=730 + i) for i in range(3))
    lab = np.zeros(S, np.int32)
    lab[:64] = 1                       # block 0 only keeps block 1, whose keys carry label 0
    idx = torch.tensor([[[[1, -1], [0, 1]]]], dtype=torch.int32).cuda()
    cnt = torch.tensor([[[1, 2]]], dtype=torch.int32).cuda()
    out = f64(bsa.bsa_block_sparse_attention_labels(gpu(q), gpu(k), gpu(v), idx, cnt, 64, torch.from_numpy(lab).cuda()))
    assert np.all(out[0, 0, :64] == 0.0)
    qf, kf, vf = (synth.stored_to_f64(x)[0, 0] for x in (q, k, v))
    rows = np.arange(64, 128)
    allowed = lab[rows][:, None] == lab[None, :]          # block 1 keeps blocks 0 and 1
    want = OA.masked_attention_rows(qf[rows], kf, vf, np.where(allowed, 0.0, -np.inf), D ** -0.5)
    assert max_abs(out[0, 0, rows], want) <= BF16_ATOL


# ------------------------------------------------ spatial / temporal masks ---

@pytest.mark.gpu
@pytest.mark.parametrize("kind,D", [("spatial", 128), ("temporal", 128), ("spatial", 64), ("temporal", 64)])
def test_spatial_temporal_attention_small(kind, D):
    torch_gpu()
    grid = (4, 8, 16)
    S = 512
    q, k, v = (synth.normal_bits((1, 2, S, D), seed=740 + i) for i in range(3))
    out = f64(bsa.video_label_attention(gpu(q), gpu(k), gpu(v), grid, kind))
    mask = OA.spatial_only_mask(grid) if kind == "spatial" else OA.temporal_only_mask(grid)
    qf, kf, vf = (synth.stored_to_f64(x) for x in (q, k, v))
    for h in range(2):
        want = OA.masked_attention(qf[0, h], kf[0, h], vf[0, h], mask, D ** -0.5)
        assert max_abs(out[0, h], want) <= BF16_ATOL, h


@pytest.mark.gpu
@pytest.mark.parametrize("kind", ["spatial", "temporal"])
def test_spatial_temporal_attention_wan_shape(kind):
    """Wan 2.1 grid (S = 30720), two heads; sampled rows against the dense definition."""
    torch = torch_gpu()
    heads = [0, 1]
    q, k, v = (synth.tensor_bits(4, role, heads=heads) for role in (synth.ROLE_Q, synth.ROLE_K, synth.ROLE_V))
    out = bsa.video_label_attention(gpu(q), gpu(k), gpu(v), WAN_GRID, kind)
    T, Hg, Wg = WAN_GRID
    S = T * Hg * Wg
    rng = np.random.default_rng(1)
    rows = np.concatenate([[0, 1535, 1536, S - 1], rng.integers(0, S, 12)])
    got = f64(out[:, :, torch.from_numpy(rows).cuda()])
    j = np.arange(S)
    for h in range(2):
        qf, kf, vf = (synth.stored_to_f64(x[0, h]) for x in (q, k, v))
        if kind == "spatial":
            allowed = (rows[:, None] // (Hg * Wg)) == (j[None, :] // (Hg * Wg))
        else:
            allowed = (rows[:, None] % (Hg * Wg)) == (j[None, :] % (Hg * Wg))
        want = OA.masked_attention_rows(qf[rows], kf, vf, np.where(allowed, 0.0, -np.inf), 128 ** -0.5)
        assert max_abs(got[0, h], want) <= BF16_ATOL, h


@pytest.mark.gpu
@pytest.mark.parametrize("grid,D,B", [((5, 4, 4), 128, 1), ((3, 6, 5), 64, 2), ((1, 8, 8), 128, 1),
                                      ((64, 2, 2), 64, 1), ((7, 3, 5), 128, 1), ((20, 2, 5), 128, 2),
                                      ((20, 4, 6), 64, 1)])
def test_temporal_only_gathered_small(grid, D, B):
    """bsa_temporal_only_attention (each position's frames gathered on load): every output against the
    oracle's temporal-only mask, including partial last tiles (positions % (64 // T) != 0), T = 1 and T = 64,
    and against the permute + label-attention + inverse path."""
    torch = torch_gpu()
    T, Hg, Wg = grid
    S, H = T * Hg * Wg, 2
    q, k, v = (synth.normal_bits((B, H, S, D), seed=860 + i + S + D) for i in range(3))
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    out = f64(bsa.bsa_temporal_only_attention(qg, kg, vg, grid))
    mask = OA.temporal_only_mask(grid)
    qf, kf, vf = (synth.stored_to_f64(x) for x in (q, k, v))
    for b in range(B):
        for h in range(H):
            want = OA.masked_attention(qf[b, h], kf[b, h], vf[b, h], mask, D ** -0.5)
            assert max_abs(out[b, h], want) <= BF16_ATOL, (b, h)
    if T == 1:                                   # one key per row: the output is v itself
        assert np.array_equal(out, vf)
    if S % 64 == 0:
        ref = bsa.VideoLabelAttention(B, H, grid, "temporal", qg.device)   # no dtype: the permuted path
        assert not ref.direct
        assert max_abs(out, f64(ref(qg, kg, vg))) <= BF16_ATOL


@pytest.mark.gpu
def test_temporal_only_gathered_wan_shape_and_scales():
    """Wan grid, 40 heads in one launch: every row of head 3 and sampled rows of two more against the
    oracle (rows over the keys of their own position); explicit scales 0 and < 0; unsupported shapes."""
    torch = torch_gpu()
    q, k, v = synth.qkv(4)
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    T, Hg, Wg = WAN_GRID
    S = T * Hg * Wg
    pos = np.arange(S) % (Hg * Wg)
    out = f64(bsa.bsa_temporal_only_attention(qg, kg, vg, WAN_GRID))
    rng = np.random.default_rng(5)
    for h, rows in ((3, np.arange(S)), (0, rng.integers(0, S, 300)), (39, rng.integers(0, S, 300))):
        qf, kf, vf = (synth.stored_to_f64(x[0, h]) for x in (q, k, v))
        want = OP.label_rows_gathered(qf, kf, vf, pos, rows, 128 ** -0.5)
        assert max_abs(out[0, h, rows], want) <= BF16_ATOL, h
    sub = [x[:, :2].contiguous() for x in (qg, kg, vg)]
    for scale in (0.0, -0.05):
        got = f64(bsa.bsa_temporal_only_attention(*sub, WAN_GRID, scale=scale))
        rows = rng.integers(0, S, 200)
        for h in range(2):
            qf, kf, vf = (synth.stored_to_f64(x[0, h]) for x in (q, k, v))
            want = OP.label_rows_gathered(qf, kf, vf, pos, rows, scale)
            assert max_abs(got[0, h, rows], want) <= BF16_ATOL, (scale, h)
    with pytest.raises(bsa.UnsupportedError):
        bsa.bsa_temporal_only_attention(*(x.float() for x in sub), WAN_GRID)
    x = torch.zeros((1, 1, 65 * 4, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bsa.UnsupportedError):
        bsa.bsa_temporal_only_attention(x, x, x, (65, 2, 2))


# ---------------------------------------------------------- padded recipe ---

@pytest.mark.gpu
@pytest.mark.parametrize("statistic", ["mean", "pooled"])
def test_padded_pipeline_small_grid_every_output(statistic):
    """The recipe on a grid no candidate divides; every output against the oracle."""
    torch = torch_gpu()
    grid, tiles = (5, 10, 12), [(4, 4, 4), (1, 8, 8)]
    H, D = 3, 128
    S = 600
    q, k, v = (synth.normal_bits((1, H, S, D), seed=750 + i) for i in range(3))
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    pipe = bsa.AdaptiveBlockSparse(1, H, grid, D, tiles, 0.3, qg.dtype, qg.device, sink_blocks=1, keep_diag=3,
                                   statistic=statistic, pad=True)
    out = f64(pipe(qg, kg, vg))
    qf, kf, vf = (synth.stored_to_f64(x) for x in (q, k, v))
    ref = OP.padded_adaptive_block_sparse(qf, kf, vf, grid, tiles, 0.3, sink_blocks=1, keep_diag=3,
                                          statistic=statistic)
    choice = pipe.choice.cpu().numpy()
    kv_idx, kv_cnt = pipe.kv
    idx, cnt = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    checked = 0
    for h in range(H):
        if choice[0, h] != ref["choice"][0, h]:
            a, b = ref["tiling_score"][0, h, choice[0, h]], ref["tiling_score"][0, h, ref["choice"][0, h]]
            assert abs(a - b) < TOPK_REL * abs(b)
            continue
        keep = ref["keep"][h]
        nb = keep.shape[0]
        gkeep = np.zeros_like(keep)
        for I in range(nb):
            gkeep[I, idx[0, h, I, :cnt[0, h, I]]] = True
        for I, J in zip(*np.nonzero(gkeep != keep)):
            assert OB.near_tie_ok(ref["scores"][h][I], ref["k"][h], J, TOPK_REL), (h, I, J)
        if np.array_equal(gkeep, keep):
            assert max_abs(out[0, h], ref["out"][0, h]) <= BF16_ATOL, h
            checked += 1
    assert checked >= 1


@pytest.mark.gpu
def test_padded_pipeline_wan_shape_with_16_2_2():
    """Wan 2.1 grid with all three SPADE candidates, (16, 2, 2) padded to T = 32.
    Sampled heads: choice, kept lists (near ties aside) and sampled output rows."""
    torch = torch_gpu()
    wl = synth.WORKLOADS[4]
    tiles = [(1, 8, 8), (4, 4, 4), (16, 2, 2)]
    q, k, v = synth.qkv(4)
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    pipe = bsa.AdaptiveBlockSparse(1, wl.H, wl.grid, wl.D, tiles, 0.17, qg.dtype, qg.device, pad=True)
    out = pipe(qg, kg, vg)
    torch.cuda.synchronize()
    assert pipe.k_table == [81, 81, 130] and pipe.Sp == 49152
    choice = pipe.choice.cpu().numpy()
    kv_idx, kv_cnt = pipe.kv
    idx, cnt = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    rng = np.random.default_rng(4)
    heads = [0, 11, 25, 38]
    qs = synth.stored_to_f64(q[:, heads])
    oc, osc = OT.select_tiling(qs, wl.grid, tiles, pad=True)
    for n, h in enumerate(heads):
        c = int(choice[0, h])
        if c != oc[0, n]:
            a, b = osc[0, n, c], osc[0, n, oc[0, n]]
            assert abs(a - b) < TOPK_REL * abs(b)
        perm = OT.padded_tile_permutation(wl.grid, tiles[c])
        valid = perm >= 0
        qp, kp, vp = (_gather_padded(synth.stored_to_f64(x[0, h]), perm) for x in (q, k, v))
        nb = perm.size // 64
        scores = OB.minmax_block_scores_valid(qp, kp, valid, 64)
        kk = OB.budget(0.17, nb)
        okeep = OB.topk_block_mask(scores, kk, 1, True)
        gkeep = np.zeros((nb, nb), bool)
        for I in range(nb):
            gkeep[I, idx[0, h, I, :cnt[0, h, I]]] = True
        for I, J in zip(*np.nonzero(okeep != gkeep)):
            assert J != 0 and J != I
            assert OB.near_tie_ok(scores[I], kk, J, TOPK_REL), (h, I, J)
        # sampled real rows, attended over the GPU's lists with padded keys masked
        real_pos = np.flatnonzero(valid)
        rows_p = np.sort(rng.choice(real_pos, 12, replace=False))
        allowed = gkeep[rows_p // 64][:, np.arange(perm.size) // 64] & valid[None, :]
        want = OA.masked_attention_rows(qp[rows_p], kp, vp, np.where(allowed, 0.0, -np.inf), 128 ** -0.5)
        got = f64(out[0, h, torch.from_numpy(perm[rows_p]).cuda()])
        assert max_abs(got, want) <= BF16_ATOL, h


# ------------------------------------------------------ gather on load ---

@pytest.mark.gpu
def test_tiled_scores_and_attention_equal_the_permuted_path():
    """Reading q, k, v through the tile geometry gives the same bits as the
    permute -> scores / attention -> inverse permute sequence."""
    torch = torch_gpu()
    grid, tiles = (4, 16, 16), [(1, 8, 8), (4, 4, 4), (2, 8, 4)]
    H, D, S = 5, 128, 1024
    q, k, v = (gpu(synth.normal_bits((1, H, S, D), seed=760 + i)) for i in range(3))
    choice = torch.tensor([[0, 1, 2, 1, 0]], dtype=torch.int32).cuda()
    s_t, _ = bsa.bsa_minmax_block_scores_tiled(q, k, grid, tiles, head_choice=choice)
    qp, kp, vp = (bsa.bsa_tile_permute(x, grid, tiles, head_choice=choice) for x in (q, k, v))
    s_p, _ = bsa.bsa_minmax_block_scores(qp, kp, 64)
    assert torch.equal(s_t, s_p)
    kv_idx, kv_cnt = bsa.bsa_topk_block_mask(s_p, 4, 1, 3)
    o_t = bsa.bsa_block_sparse_attention_tiled(q, k, v, grid, tiles, kv_idx, kv_cnt, head_choice=choice)
    o_p = bsa.bsa_invert_permute(bsa.bsa_block_sparse_attention(qp, kp, vp, kv_idx, kv_cnt, 64), grid, tiles,
                                 head_choice=choice)
    assert torch.equal(o_t, o_p)
    # and against the oracle for one head
    qf, kf, vf = (f64(x)[0, 3] for x in (q, k, v))
    perm = OT.tile_permutation(grid, tiles[1])
    keep = np.zeros((16, 16), bool)
    idx, cnt = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    for I in range(16):
        keep[I, idx[0, 3, I, :cnt[0, 3, I]]] = True
    lab = np.empty(S, np.int64)
    lab[perm] = np.arange(S) // 64
    want = OP.label_mask_attention(qf, kf, vf, lab, keep, D ** -0.5)
    assert max_abs(f64(o_t)[0, 3], want) <= BF16_ATOL


@pytest.mark.gpu
def test_tiled_attention_rejects_uncovered_tilings():
    torch = torch_gpu()
    q = gpu(synth.normal_bits((1, 1, 1024, 128), seed=770))
    idx = torch.zeros((1, 1, 16, 1), dtype=torch.int32).cuda()
    cnt = torch.ones((1, 1, 16), dtype=torch.int32).cuda()
    with pytest.raises(bsa.UnsupportedError):
        bsa.bsa_block_sparse_attention_tiled(q, q, q, (4, 16, 16), [(2, 4, 4)], idx, cnt)    # 32 tokens
    assert not bsa.tiled_attention_supported(torch.bfloat16, 128, [(2, 4, 4)], (4, 16, 16))
    assert bsa.tiled_attention_supported(torch.bfloat16, 128, [(4, 8, 2), (4, 16, 1)], (4, 16, 16))
    # padding along y (10 rows, tiles 8 high) has no gather-on-load kernel; along T it has
    q10 = gpu(synth.normal_bits((1, 1, 4 * 10 * 16, 128), seed=772))
    i10 = torch.zeros((1, 1, 16, 1), dtype=torch.int32).cuda()      # the grid padded to 4x16x16: 16 blocks
    c10 = torch.ones((1, 1, 16), dtype=torch.int32).cuda()
    with pytest.raises(bsa.UnsupportedError):
        bsa.bsa_block_sparse_attention_tiled_padded(q10, q10, q10, (4, 10, 16), [(1, 8, 8)], i10, c10)
    assert not bsa.tiled_attention_supported(torch.bfloat16, 128, [(1, 8, 8)], (4, 10, 16), pad=True)
    assert bsa.tiled_attention_supported(torch.bfloat16, 128, [(16, 2, 2)], (20, 32, 48), pad=True)
    assert not bsa.tiled_attention_supported(torch.bfloat16, 128, [(16, 2, 2)], (20, 32, 48), pad=False)
    q64 = gpu(synth.normal_bits((1, 1, 1024, 64), seed=771))
    with pytest.raises(bsa.UnsupportedError):
        bsa.bsa_block_sparse_attention_tiled(q64, q64, q64, (4, 16, 16), [(1, 8, 8)], idx, cnt)
    with pytest.raises(ValueError):
        bsa.bsa_block_sparse_attention_tiled(q, q, q, (4, 16, 16), [(3, 4, 4)], idx, cnt)    # does not divide


@pytest.mark.gpu
@pytest.mark.parametrize("cfg", [4, 5])
def test_fused_pipeline_equals_unfused_full_size(cfg):
    torch = torch_gpu()
    wl = synth.WORKLOADS[cfg]
    tiles = [(1, 8, 8), (4, 4, 4)] if cfg == 4 else [(4, 4, 4)]
    frac = 0.17 if cfg == 4 else 0.10
    q, k, v = (gpu(x) for x in synth.qkv(cfg))
    fused = bsa.AdaptiveBlockSparse(1, wl.H, wl.grid, wl.D, tiles, frac, q.dtype, q.device)
    assert fused.fused
    a = fused(q, k, v)
    b = bsa.AdaptiveBlockSparse(1, wl.H, wl.grid, wl.D, tiles, frac, q.dtype, q.device, fused=False)(q, k, v)
    assert torch.equal(a, b)


# ------------------------------------------------------------- batch > 1 ---

@pytest.mark.gpu
def test_batch_two_fused_and_padded_pipelines():
    """B = 2 through the fused pipeline and the padded pipeline, every output
    against the oracle (rows attended over the GPU's kept lists)."""
    torch = torch_gpu()
    H, D = 2, 128
    for grid, tiles, pad in [((4, 16, 16), [(1, 8, 8), (4, 4, 4)], False), ((5, 10, 12), [(4, 4, 4), (1, 8, 8)], True)]:
        S = int(np.prod(grid))
        q, k, v = (synth.normal_bits((2, H, S, D), seed=780 + i + S) for i in range(3))
        qg, kg, vg = gpu(q), gpu(k), gpu(v)
        pipe = bsa.AdaptiveBlockSparse(2, H, grid, D, tiles, 0.3, qg.dtype, qg.device, pad=pad)
        assert pipe.fused == (not pad)
        out = f64(pipe(qg, kg, vg))
        choice = pipe.choice.cpu().numpy()
        kv_idx, kv_cnt = pipe.kv
        idx, cnt = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
        qf, kf, vf = (synth.stored_to_f64(x) for x in (q, k, v))
        oc, osc = OT.select_tiling(qf, grid, tiles, pad=pad)
        for b in range(2):
            for h in range(H):
                c = int(choice[b, h])
                if c != oc[b, h]:
                    a_, b_ = osc[b, h, c], osc[b, h, oc[b, h]]
                    assert abs(a_ - b_) < TOPK_REL * abs(b_)
                perm = (OT.padded_tile_permutation if pad else OT.tile_permutation)(grid, tiles[c])
                valid = perm >= 0
                nb = perm.size // 64
                gkeep = np.zeros((nb, nb), bool)
                for I in range(nb):
                    gkeep[I, idx[b, h, I, :cnt[b, h, I]]] = True
                qp, kp, vp = (_gather_padded(x[b, h], perm) for x in (qf, kf, vf))
                rows = np.flatnonzero(valid)
                allowed = gkeep[rows // 64][:, np.arange(perm.size) // 64] & valid[None, :]
                want = OA.masked_attention_rows(qp[rows], kp, vp, np.where(allowed, 0.0, -np.inf), D ** -0.5)
                assert max_abs(out[b, h, perm[rows]], want) <= BF16_ATOL, (grid, b, h)


@pytest.mark.gpu
def test_padded_pipeline_scalar_path_fp32():
    """fp32 and D = 64 take the scalar label kernel on the padded path."""
    torch = torch_gpu()
    grid, tiles = (3, 5, 6), [(2, 2, 4), (1, 4, 4)]
    H = 2
    for dtype, D in (("f32", 16), ("bf16", 64)):
        S = 90
        q, k, v = (synth.normal_bits((1, H, S, D), seed=790 + i, dtype=dtype) for i in range(3))
        qg, kg, vg = gpu(q), gpu(k), gpu(v)
        pipe = bsa.AdaptiveBlockSparse(1, H, grid, D, tiles, 0.5, qg.dtype, qg.device, pad=True)
        out = f64(pipe(qg, kg, vg))
        ref = OP.padded_adaptive_block_sparse(*(synth.stored_to_f64(x) for x in (q, k, v)), grid, tiles, 0.5)
        choice = pipe.choice.cpu().numpy()
        kv_idx, kv_cnt = pipe.kv
        idx, cnt = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
        tol = BF16_ATOL if dtype == "bf16" else F32_ATOL
        qf, kf, vf = (synth.stored_to_f64(x) for x in (q, k, v))
        same = 0
        for h in range(H):
            assert choice[0, h] == ref["choice"][0, h]
            keep = ref["keep"][h]
            nb = keep.shape[0]
            gkeep = np.zeros_like(keep)
            for I in range(nb):
                gkeep[I, idx[0, h, I, :cnt[0, h, I]]] = True
            # list differences only at near ties of the oracle's scores
            for I, J in zip(*np.nonzero(gkeep != keep)):
                assert OB.near_tie_ok(ref["scores"][h][I], ref["k"][h], J, TOPK_REL), (dtype, h, I, J)
            # every output row against the oracle attending over the GPU's own lists
            perm = ref["perm"][h]
            valid = perm >= 0
            qp, kp, vp = (_gather_padded(x[0, h], perm) for x in (qf, kf, vf))
            rows = np.flatnonzero(valid)
            blk = ref["block"]
            allowed = gkeep[rows // blk][:, np.arange(perm.size) // blk] & valid[None, :]
            want = OA.masked_attention_rows(qp[rows], kp, vp, np.where(allowed, 0.0, -np.inf), D ** -0.5)
            assert max_abs(out[0, h, perm[rows]], want) <= tol, (dtype, h)
            if np.array_equal(gkeep, keep):
                assert max_abs(out[0, h], ref["out"][0, h]) <= tol, (dtype, h)
                same += 1
        assert same >= 1, dtype


# ------------------------------------- gather on load: row patterns, padding ---

@pytest.mark.gpu
@pytest.mark.parametrize("tiles", [[(2, 16, 2), (4, 16, 1)], [(8, 8, 1), (4, 8, 2)], [(1, 8, 8), (8, 2, 4)]])
def test_tiled_attention_row_patterns(tiles):
    """Tiles whose x extent is 2 or 1 (four cells of a DMA row group on two or four T-major rows): the
    gather-on-load attention equals permute -> attention -> inverse bit for bit, and the oracle's rows."""
    torch = torch_gpu()
    grid, H, D = (8, 16, 16), 2, 128
    S, nb = 2048, 32
    assert bsa.tiled_attention_supported(torch.bfloat16, D, tiles, grid)
    q, k, v = (synth.normal_bits((1, H, S, D), seed=880 + i) for i in range(3))
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    rng = np.random.default_rng(88)
    keep = rng.random((1, H, nb, nb)) < 0.3
    keep[..., np.arange(nb), np.arange(nb)] = True
    cnt = keep.sum(-1).astype(np.int32)
    idx = np.full((1, H, nb, int(cnt.max())), -1, np.int32)
    for h in range(H):
        for I in range(nb):
            li = np.flatnonzero(keep[0, h, I])
            idx[0, h, I, :li.size] = li
    kv_idx, kv_cnt = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    choice = torch.tensor([[0, 1]], dtype=torch.int32, device="cuda")
    out = bsa.bsa_block_sparse_attention_tiled(qg, kg, vg, grid, tiles, kv_idx, kv_cnt, head_choice=choice)
    qp, kp, vp = (bsa.bsa_tile_permute(x, grid, tiles, head_choice=choice) for x in (qg, kg, vg))
    ref = bsa.bsa_invert_permute(bsa.bsa_block_sparse_attention(qp, kp, vp, kv_idx, kv_cnt, 64), grid, tiles,
                                 head_choice=choice)
    assert torch.equal(out, ref)
    qf, kf, vf = (synth.stored_to_f64(x) for x in (q, k, v))
    o = f64(out)
    for h in range(H):
        perm = OT.tile_permutation(grid, tiles[h])
        want = OA.block_sparse_rows_gathered(*(OT.permute_tokens(x[0, h], perm) for x in (qf, kf, vf)),
                                             keep[0, h], 64, np.arange(S), D ** -0.5)
        assert max_abs(o[0, h, perm], want) <= BF16_ATOL, h


def _padded_lists_check_rows(out, q, k, v, grid, tiles, choice, idx, cnt, heads, full_head=None, rng=None):
    """Every real row (full_head) or a sample of rows of `heads`, against the oracle over the GPU's lists on
    the head's padded grid, padding keys left out."""
    torch = torch_gpu()
    qf, kf, vf = (synth.stored_to_f64(x) for x in (q, k, v))
    D = q.shape[-1]
    for h in heads:
        perm = OT.padded_tile_permutation(grid, tiles[int(choice[0, h])])
        valid = perm >= 0
        nb = perm.size // 64
        gkeep = np.zeros((nb, nb), bool)
        for I in range(nb):
            gkeep[I, idx[0, h, I, :cnt[0, h, I]]] = True
        real = np.flatnonzero(valid)
        rows = real if h == full_head else np.sort(rng.choice(real, 200, replace=False))
        qp, kp, vp = (_gather_padded(x[0, h], perm) for x in (qf, kf, vf))
        want = OA.block_sparse_rows_gathered(qp, kp, vp, gkeep, 64, rows, D ** -0.5, key_valid=valid)
        got = f64(out[0, h, torch.from_numpy(perm[rows]).cuda()])
        assert max_abs(got, want) <= BF16_ATOL, h


@pytest.mark.gpu
@pytest.mark.parametrize("grid,tiles,H,choices", [
    ((20, 8, 8), [(1, 8, 8), (4, 4, 4), (16, 2, 2)], 4, [0, 2, 1, 2]),      # T = 20 padded to 32 for (16, 2, 2)
    ((6, 16, 16), [(1, 8, 8), (4, 4, 4)], 3, [1, 0, 1]),                   # T = 6 padded to 8 for (4, 4, 4)
    ((5, 8, 16), [(1, 8, 8), (2, 4, 8), (4, 4, 4)], 2, [2, 1]),           # every candidate pads but (1, 8, 8)
])
def test_padded_scores_gather_on_load_equal_masked_copies(grid, tiles, H, choices):
    """bsa_minmax_block_scores_tiled_padded on T-major q, k equals bsa_tile_permute_padded followed by
    bsa_minmax_block_scores_masked bit for bit: summaries, scores (-inf rows and columns of padding-only blocks
    included) and key norms; B = 2 with different choices per batch."""
    torch = torch_gpu()
    B, D = 2, 128
    S = grid[0] * grid[1] * grid[2]
    q, k = (synth.normal_bits((B, H, S, D), seed=8100 + i) for i in range(2))
    qg, kg = gpu(q), gpu(k)
    choice = torch.tensor([choices, choices[::-1]], dtype=torch.int32, device="cuda")
    Sp = bsa.padded_rows(grid, tiles)
    nb = Sp // 64
    kn_t = torch.full((B, H, nb), -7.0, dtype=torch.float32, device="cuda")
    sc_t, sm_t = bsa.bsa_minmax_block_scores_tiled_padded(qg, kg, grid, tiles, head_choice=choice, key_norms=kn_t)
    qp, lab = bsa.bsa_tile_permute_padded(qg, grid, tiles, head_choice=choice, Sp=Sp)
    kp, _ = bsa.bsa_tile_permute_padded(kg, grid, tiles, head_choice=choice, Sp=Sp, labels=False)
    kn_p = torch.full((B, H, nb), -7.0, dtype=torch.float32, device="cuda")
    sc_p, sm_p = bsa.bsa_minmax_block_scores(qp, kp, 64, labels=lab, key_norms=kn_p)
    assert torch.equal(sm_t, sm_p)
    assert torch.equal(kn_t, kn_p)
    assert torch.equal(sc_t.isneginf(), sc_p.isneginf()) and sc_t.isneginf().any()
    assert torch.equal(sc_t, sc_p)


@pytest.mark.gpu
def test_padded_pipeline_gather_on_load_small():
    """Candidates (1,8,8), (4,4,4), (16,2,2) on a 20x8x8 grid (T padded to 32 for (16,2,2)): the padded
    pipeline with attention on T-major tensors gives the same lists as the permuted-copy pipeline, outputs
    within tolerance of it, and every output within tolerance of the oracle's padded recipe on its lists."""
    torch = torch_gpu()
    grid, tiles, H, D = (20, 8, 8), [(1, 8, 8), (4, 4, 4), (16, 2, 2)], 4, 128
    S = 1280
    q, k, v = (synth.normal_bits((1, H, S, D), seed=890 + i) for i in range(3))
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    fused = bsa.AdaptiveBlockSparse(1, H, grid, D, tiles, 0.25, qg.dtype, qg.device, pad=True)
    plain = bsa.AdaptiveBlockSparse(1, H, grid, D, tiles, 0.25, qg.dtype, qg.device, pad=True, fused=False)
    assert fused.fused and not plain.fused
    a, b = fused(qg, kg, vg), plain(qg, kg, vg)
    assert torch.equal(fused.choice, plain.choice)
    assert torch.equal(fused.kv[1], plain.kv[1]) and torch.equal(fused.kv[0], plain.kv[0])
    assert max_abs(f64(a), f64(b)) <= BF16_ATOL
    choice = fused.choice.cpu().numpy()
    forced = torch.full((1, H), 2, dtype=torch.int32, device="cuda")     # every head on (16, 2, 2)
    idx, cnt = fused.kv[0].cpu().numpy(), fused.kv[1].cpu().numpy()
    _padded_lists_check_rows(a, q, k, v, grid, tiles, choice, idx, cnt, range(H), full_head=0,
                             rng=np.random.default_rng(0))
    for h in range(1, H):
        _padded_lists_check_rows(a, q, k, v, grid, tiles, choice, idx, cnt, [h], full_head=h)
    # forced (16, 2, 2) on every head through the ABI call directly, against the label kernel on the same lists
    qp, lab = bsa.bsa_tile_permute_padded(qg, grid, tiles, head_choice=forced)
    kp, _ = bsa.bsa_tile_permute_padded(kg, grid, tiles, head_choice=forced, labels=False)
    vp, _ = bsa.bsa_tile_permute_padded(vg, grid, tiles, head_choice=forced, labels=False)
    scores, _ = bsa.bsa_minmax_block_scores(qp, kp, 64, labels=lab)
    nbt = [bsa.bsa_padded_length(*grid, t) // 64 for t in tiles]
    kt = [bsa.bsa_budget(0.25, n) for n in nbt]
    kv_idx, kv_cnt = bsa.bsa_topk_block_mask_tiled(scores, forced, kt, nbt, 1, 1)
    got = bsa.bsa_block_sparse_attention_tiled_padded(qg, kg, vg, grid, tiles, kv_idx, kv_cnt, head_choice=forced)
    op = bsa.bsa_block_sparse_attention_labels(qp, kp, vp, kv_idx, kv_cnt, 64, lab)
    want = bsa.bsa_invert_permute_padded(op, grid, tiles, head_choice=forced)
    assert max_abs(f64(got), f64(want)) <= BF16_ATOL
    _padded_lists_check_rows(got, q, k, v, grid, tiles, np.full((1, H), 2), kv_idx.cpu().numpy(),
                             kv_cnt.cpu().numpy(), [1], full_head=1)


@pytest.mark.gpu
def test_padded_pipeline_gather_on_load_wan_shape():
    """The Wan grid with (1,8,8), (4,4,4) and (16,2,2) (T padded from 20 to 32): the temporal heads pick
    (16,2,2); every row of one such head and sampled rows of others against the oracle on the GPU's lists,
    which equal the oracle's top-k on the padded summaries except at near ties."""
    torch = torch_gpu()
    wl = synth.WORKLOADS[4]
    tiles = [(1, 8, 8), (4, 4, 4), (16, 2, 2)]
    q, k, v = synth.qkv(4)
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    pipe = bsa.AdaptiveBlockSparse(1, wl.H, wl.grid, wl.D, tiles, 0.17, qg.dtype, qg.device, pad=True)
    assert pipe.fused
    out = pipe(qg, kg, vg)
    choice = pipe.choice.cpu().numpy()
    assert set(choice[0].tolist()) == {0, 2}
    idx, cnt = pipe.kv[0].cpu().numpy(), pipe.kv[1].cpu().numpy()
    temporal = [h for h in range(wl.H) if choice[0, h] == 2]
    spatial = [h for h in range(wl.H) if choice[0, h] == 0]
    qf, kf = synth.stored_to_f64(q), synth.stored_to_f64(k)
    for h in (temporal[0], spatial[0]):            # lists: the oracle's top-k on the padded summaries
        perm = OT.padded_tile_permutation(wl.grid, tiles[int(choice[0, h])])
        valid = perm >= 0
        nb = perm.size // 64
        sc = OB.minmax_block_scores_valid(_gather_padded(qf[0, h], perm), _gather_padded(kf[0, h], perm), valid, 64)
        okeep = OB.topk_block_mask(sc, OB.budget(0.17, nb), 1, True)
        gkeep = np.zeros((nb, nb), bool)
        for I in range(nb):
            gkeep[I, idx[0, h, I, :cnt[0, h, I]]] = True
        for I, J in zip(*np.nonzero(okeep != gkeep)):
            assert OB.near_tie_ok(sc[I], OB.budget(0.17, nb), J, TOPK_REL), (h, I, J)
    _padded_lists_check_rows(out, q, k, v, wl.grid, tiles, choice, idx, cnt,
                             [temporal[0], temporal[-1], spatial[0]], full_head=temporal[0],
                             rng=np.random.default_rng(3))


@pytest.mark.gpu
def test_padded_gather_on_load_batch_of_two_mixed_choices():
    """B = 2, H = 3 with every (b, h) on its own candidate of (1,8,8), (4,4,4) and the padded (16,2,2): the
    padded gather-on-load attention (whose workgroups walk all heads' real blocks in order) equals the label
    kernel on padded permuted copies within tolerance, and the oracle's padded recipe on every real row of
    two heads."""
    torch = torch_gpu()
    grid, tiles, B, H, D = (20, 8, 8), [(1, 8, 8), (4, 4, 4), (16, 2, 2)], 2, 3, 128
    S = 1280
    q, k, v = (synth.normal_bits((B, H, S, D), seed=930 + i) for i in range(3))
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    choice_np = np.array([[0, 2, 1], [2, 0, 2]], np.int32)
    choice = torch.from_numpy(choice_np).cuda()
    qp, lab = bsa.bsa_tile_permute_padded(qg, grid, tiles, head_choice=choice)
    kp, _ = bsa.bsa_tile_permute_padded(kg, grid, tiles, head_choice=choice, labels=False)
    vp, _ = bsa.bsa_tile_permute_padded(vg, grid, tiles, head_choice=choice, labels=False)
    scores, _ = bsa.bsa_minmax_block_scores(qp, kp, 64, labels=lab)
    nbt = [bsa.bsa_padded_length(*grid, t) // 64 for t in tiles]
    assert (B * H * max(nbt)) % 8 == 0 and len(set(nbt)) > 1
    kt = [bsa.bsa_budget(0.25, n) for n in nbt]
    kv_idx, kv_cnt = bsa.bsa_topk_block_mask_tiled(scores, choice, kt, nbt, 1, 1)
    got = bsa.bsa_block_sparse_attention_tiled_padded(qg, kg, vg, grid, tiles, kv_idx, kv_cnt, head_choice=choice)
    op = bsa.bsa_block_sparse_attention_labels(qp, kp, vp, kv_idx, kv_cnt, 64, lab)
    want = bsa.bsa_invert_permute_padded(op, grid, tiles, head_choice=choice)
    assert max_abs(f64(got), f64(want)) <= BF16_ATOL
    idx, cnt = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    for b, h in ((0, 1), (1, 0)):
        sel = (slice(b, b + 1),)
        _padded_lists_check_rows(got[sel], q[sel], k[sel], v[sel], grid, tiles, choice_np[sel], idx[sel], cnt[sel],
                                 [h], full_head=h)
