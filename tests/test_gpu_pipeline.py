"""The adaptive-tiling block-sparse pipeline end to end, at full workload sizes.

Launch configuration as in the benchmark: one AdaptiveBlockSparse call over all
heads.  Checked per sampled head: the tiling choice, the kept block lists
(exact except near ties) and output rows against the oracle: every row of one
head at the Wan shape, the first and last row of every query block of one head
at the long-sequence shape, and sampled rows of the other heads.
"""
import numpy as np
import pytest

from block_sparse_attention_permute_amd import bsa, synth
from oracle import attention as OA
from oracle import blocks as OB
from oracle import pipeline as OP
from oracle import tiling as OT
from tests.gpu_helpers import BF16_ATOL, TOPK_REL, f64, gpu, max_abs, top_p_row_ok, torch_gpu

SETUPS = {
    4: dict(tiles=[(1, 8, 8), (4, 4, 4)], frac=0.17, heads=[0, 7, 22, 39], full_head=0),
    5: dict(tiles=[(4, 4, 4)], frac=0.10, heads=[0, 13, 23], full_head=13),
}


def _sample_rows(cnt_row, nb, block, rng):
    blocks = {0, nb - 1, int(np.argmax(cnt_row)), int(np.argmin(cnt_row))}
    blocks |= set(rng.integers(0, nb, 2).tolist())
    rows = []
    for I in sorted(blocks):
        rows += [I * block, I * block + block // 2, I * block + block - 1]
    return np.array(rows)


def _gpu_keep(idx, cnt, nb):
    keep = np.zeros((nb, nb), bool)
    for I in range(nb):
        keep[I, idx[I, :cnt[I]]] = True
    return keep


def _lists_near_ties_only(gkeep, scores, k, sink, width, what):
    """The GPU's kept lists equal the oracle's top-k (+ static blocks) on the oracle's scores, except
    for members within TOPK_REL of the row's k-th score."""
    nb = scores.shape[0]
    okeep = OB.topk_block_mask(scores, k, sink, width)
    static = OB.static_blocks(nb, nb, sink, width)
    for I, J in zip(*np.nonzero(okeep != gkeep)):
        assert not static[I, J], (what, I, J)
        assert OB.near_tie_ok(scores[I], k, J, TOPK_REL), (what, I, J)
    return int((okeep != gkeep).sum())


@pytest.mark.gpu
@pytest.mark.parametrize("cfg,sink,width", [(4, 1, 1), (5, 1, 1), (4, 5, 40)])
def test_adaptive_pipeline_full_size(cfg, sink, width):
    """(4, 5, 40): SPADE's static widths for Wan (sink 5, diagonal band 40)."""
    torch = torch_gpu()
    wl, st = synth.WORKLOADS[cfg], SETUPS[cfg]
    q, k, v = synth.qkv(cfg)
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    pipe = bsa.AdaptiveBlockSparse(1, wl.H, wl.grid, wl.D, st["tiles"], st["frac"], qg.dtype, qg.device,
                                   sink_blocks=sink, keep_diag=width, validate=True)
    out = pipe(qg, kg, vg)
    torch.cuda.synchronize()
    kv_idx, kv_cnt = pipe.kv
    choice = pipe.choice.cpu().numpy()
    idx, cnt = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    assert pipe.k == OB.budget(st["frac"], pipe.nb) == (81 if cfg == 4 else 192)
    band = 2 * (width // 2) + 1
    assert cnt.min() >= pipe.k and cnt.max() <= pipe.k + sink + band
    rng = np.random.default_rng(cfg)
    scale = wl.D ** -0.5
    nb, blk = pipe.nb, pipe.block
    for h in st["heads"]:
        qf, kf, vf = (synth.stored_to_f64(x[0, h]) for x in (q, k, v))
        # tiling choice
        if len(st["tiles"]) > 1:
            oc, osc = OT.select_tiling(qf[None, None], wl.grid, st["tiles"])
            if oc[0, 0] != choice[0, h]:
                a, b = osc[0, 0, choice[0, h]], osc[0, 0, oc[0, 0]]
                assert abs(a - b) < TOPK_REL * abs(b), (h, a, b)
        perm = OT.tile_permutation(wl.grid, st["tiles"][int(choice[0, h])])
        qp, kp, vp = (OT.permute_tokens(x, perm) for x in (qf, kf, vf))
        # kept lists: oracle top-k on oracle scores, differences only at near ties
        gkeep = _gpu_keep(idx[0, h], cnt[0, h], nb)
        _lists_near_ties_only(gkeep, OB.minmax_block_scores(qp, kp, blk), pipe.k, sink, width, h)
        # output rows (T-major), attended over the GPU's kept lists: every row of one head (every
        # query block's first and last row at the long sequence), sampled rows of the others
        if h == st["full_head"] and sink == 1:
            rows_p = np.arange(wl.S) if cfg == 4 else np.sort(np.r_[np.arange(0, wl.S, blk),
                                                                    np.arange(blk - 1, wl.S, blk)])
        else:
            rows_p = _sample_rows(cnt[0, h], nb, blk, rng)
        want_p = OA.block_sparse_rows_gathered(qp, kp, vp, gkeep, blk, rows_p, scale)
        got = f64(out[0, h, torch.from_numpy(perm[rows_p]).cuda()])
        assert max_abs(got, want_p) <= BF16_ATOL, (h, rows_p.size)


@pytest.mark.gpu
def test_fused_pipeline_forced_mixed_choice_full_size():
    """Wan shape with head_choice forced to alternate (1, 8, 8) and (4, 4, 4) over the 40 heads: the
    gather-on-load stages equal the permuted-copy stages bit for bit (scores, key norms, lists, output),
    with and without the tiling pass's q summaries; every row of one head of each tiling and sampled rows
    of two more against the oracle."""
    torch = torch_gpu()
    wl = synth.WORKLOADS[4]
    tiles, grid, blk, nb, kk = [(1, 8, 8), (4, 4, 4)], wl.grid, 64, 480, 81
    q, k, v = synth.qkv(4)
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    forced = torch.tensor([[h % 2 for h in range(wl.H)]], dtype=torch.int32, device="cuda")
    nrm_t = torch.empty((1, wl.H, nb), dtype=torch.float32, device="cuda")
    nrm_u = torch.empty_like(nrm_t)
    qs = torch.empty((2, 2, 1, wl.H, nb, wl.D), dtype=qg.dtype, device="cuda")
    bsa.bsa_select_tiling(qg, grid, tiles, q_summaries=qs)
    sc_t, _ = bsa.bsa_minmax_block_scores_tiled(qg, kg, grid, tiles, head_choice=forced, key_norms=nrm_t)
    sc_q, _ = bsa.bsa_minmax_block_scores_tiled(qg, kg, grid, tiles, head_choice=forced, q_summaries=qs)
    idx_t, cnt_t = bsa.bsa_topk_block_mask(sc_t, kk, 1, True)
    out_t = bsa.bsa_block_sparse_attention_tiled(qg, kg, vg, grid, tiles, idx_t, cnt_t, head_choice=forced,
                                                 key_norms=nrm_t)
    qp, kp, vp = (bsa.bsa_tile_permute(x, grid, tiles, head_choice=forced) for x in (qg, kg, vg))
    sc_u, _ = bsa.bsa_minmax_block_scores(qp, kp, blk, key_norms=nrm_u)
    idx_u, cnt_u = bsa.bsa_topk_block_mask(sc_u, kk, 1, True)
    op = bsa.bsa_block_sparse_attention(qp, kp, vp, idx_u, cnt_u, blk, key_norms=nrm_u)
    out_u = bsa.bsa_invert_permute(op, grid, tiles, head_choice=forced)
    torch.cuda.synchronize()
    assert torch.equal(sc_t, sc_u) and torch.equal(sc_q, sc_u) and torch.equal(nrm_t, nrm_u)
    assert torch.equal(idx_t, idx_u) and torch.equal(cnt_t, cnt_u)
    assert torch.equal(out_t, out_u)
    idx, cnt = idx_t.cpu().numpy(), cnt_t.cpu().numpy()
    rng = np.random.default_rng(44)
    for h in (0, 1, 20, 33):
        qf, kf, vf = (synth.stored_to_f64(x[0, h]) for x in (q, k, v))
        perm = OT.tile_permutation(grid, tiles[h % 2])
        qp_, kp_, vp_ = (OT.permute_tokens(x, perm) for x in (qf, kf, vf))
        gkeep = _gpu_keep(idx[0, h], cnt[0, h], nb)
        _lists_near_ties_only(gkeep, OB.minmax_block_scores(qp_, kp_, blk), kk, 1, 1, h)
        rows_p = np.arange(wl.S) if h in (0, 1) else _sample_rows(cnt[0, h], nb, blk, rng)
        want = OA.block_sparse_rows_gathered(qp_, kp_, vp_, gkeep, blk, rows_p, 128 ** -0.5)
        got = f64(out_t[0, h, torch.from_numpy(perm[rows_p]).cuda()])
        assert max_abs(got, want) <= BF16_ATOL, h


@pytest.mark.gpu
def test_adaptive_pipeline_small_grid_every_output():
    """The whole recipe on a small grid, every head and every output: the choice equals the oracle's (or
    is a near tie), the lists differ only at near ties, and the output matches the oracle attending over
    the GPU's own choice and lists."""
    torch_gpu()
    grid, tiles = (4, 8, 8), [(1, 4, 8), (4, 2, 4), (2, 4, 4)]
    H, D, blk = 4, 64, 32
    q, k, v = (synth.normal_bits((1, H, 256, D), seed=500 + i) for i in range(3))
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    pipe = bsa.AdaptiveBlockSparse(1, H, grid, D, tiles, 0.25, qg.dtype, qg.device)
    out = f64(pipe(qg, kg, vg))
    qf, kf, vf = (synth.stored_to_f64(x) for x in (q, k, v))
    ref = OP.adaptive_block_sparse(qf, kf, vf, grid, tiles, 0.25)
    choice = pipe.choice.cpu().numpy()
    kv_idx, kv_cnt = pipe.kv
    idx, cnt = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    same = 0
    for h in range(H):
        c = int(choice[0, h])
        if c != ref["choice"][0, h]:
            a, b = ref["tiling_score"][0, h, c], ref["tiling_score"][0, h, ref["choice"][0, h]]
            assert abs(a - b) < TOPK_REL * abs(b), h
        perm = OT.tile_permutation(grid, tiles[c])
        qp, kp, vp = (OT.permute_tokens(x[0, h], perm) for x in (qf, kf, vf))
        gkeep = _gpu_keep(idx[0, h], cnt[0, h], 8)
        _lists_near_ties_only(gkeep, OB.minmax_block_scores(qp, kp, blk), ref["k"], 1, 1, h)
        want = OT.unpermute_tokens(OA.block_sparse_rows_gathered(qp, kp, vp, gkeep, blk, np.arange(256),
                                                                 D ** -0.5), perm)
        assert max_abs(out[0, h], want) <= BF16_ATOL, h
        if c == ref["choice"][0, h] and np.array_equal(gkeep, ref["keep"][0, h]):
            assert max_abs(out[0, h], ref["out"][0, h]) <= BF16_ATOL, h
            same += 1
    assert same >= 1                          # the oracle's own end-to-end result is met on some head


@pytest.mark.gpu
def test_adaptive_pipeline_top_p_small_grid():
    """Top-p instead of top-k (p = 0.9 of the softmax of scores / sqrt(D)),
    with SPADE-style static blocks, on a grid the oracle runs whole."""
    torch = torch_gpu()
    grid, tiles = (4, 16, 16), [(1, 8, 8), (4, 4, 4)]
    H, D, p = 3, 128, 0.9
    q, k, v = (synth.normal_bits((1, H, 1024, D), seed=600 + i) for i in range(3))
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    pipe = bsa.AdaptiveBlockSparse(1, H, grid, D, tiles, 0.25, qg.dtype, qg.device, sink_blocks=2, keep_diag=3,
                                   top_p=p, p_scale=D ** -0.5)
    out = f64(pipe(qg, kg, vg))
    qf, kf, vf = (synth.stored_to_f64(x) for x in (q, k, v))
    ref = OP.adaptive_block_sparse(qf, kf, vf, grid, tiles, 0.25, sink_blocks=2, keep_diag=3, top_p=p,
                                   p_scale=D ** -0.5)
    choice = pipe.choice.cpu().numpy()
    kv_idx, kv_cnt = pipe.kv
    idx, cnt = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    static = OB.static_blocks(16, 16, 2, 3)
    for h in range(H):
        assert choice[0, h] == ref["choice"][0, h]
        gkeep = np.zeros((16, 16), bool)
        for I in range(16):
            gkeep[I, idx[0, h, I, :cnt[0, h, I]]] = True
        # GPU scores (fp32) against the oracle's: the kept rows agree up to the cut tolerance
        for I in range(16):
            assert top_p_row_ok(gkeep[I], ref["scores"][0, h, I], p, D ** -0.5, static[I]), (h, I)
        perm = ref["perm"][0, h]
        qp, kp, vp = (OT.permute_tokens(x[0, h], perm) for x in (qf, kf, vf))
        want = OT.unpermute_tokens(OA.block_sparse_attention(qp[None, None], kp[None, None], vp[None, None],
                                                             gkeep[None, None], 64, D ** -0.5)[0, 0], perm)
        assert max_abs(out[0, h], want) <= BF16_ATOL, h
