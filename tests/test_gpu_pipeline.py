"""The adaptive-tiling block-sparse pipeline end to end, at full workload sizes.

Launch configuration as in the benchmark: one AdaptiveBlockSparse call over all
heads.  Checked per sampled head: the tiling choice, the kept block lists
(exact except near ties) and sampled output rows, against the oracle.
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
    4: dict(tiles=[(1, 8, 8), (4, 4, 4)], frac=0.17, heads=[0, 7, 22, 39]),
    5: dict(tiles=[(4, 4, 4)], frac=0.10, heads=[0, 13, 23]),
}


def _sample_rows(cnt_row, nb, block, rng):
    blocks = {0, nb - 1, int(np.argmax(cnt_row)), int(np.argmin(cnt_row))}
    blocks |= set(rng.integers(0, nb, 2).tolist())
    rows = []
    for I in sorted(blocks):
        rows += [I * block, I * block + block // 2, I * block + block - 1]
    return np.array(rows)


@pytest.mark.gpu
@pytest.mark.parametrize("cfg,sink,width", [(4, 1, 1), (5, 1, 1), (4, 5, 40)])
def test_adaptive_pipeline_full_size(cfg, sink, width):
    """(4, 5, 40): SPADE's static widths for Wan (sink 5, diagonal band 40)."""
    torch = torch_gpu()
    wl, st = synth.WORKLOADS[cfg], SETUPS[cfg]
    q, k, v = synth.qkv(cfg)
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    pipe = bsa.AdaptiveBlockSparse(1, wl.H, wl.grid, wl.D, st["tiles"], st["frac"], qg.dtype, qg.device,
                                   sink_blocks=sink, keep_diag=width)
    out = pipe(qg, kg, vg)
    torch.cuda.synchronize()
    kv_idx, kv_cnt = pipe.kv
    bsa.bsa_validate_block_list(kv_idx, kv_cnt, pipe.nb)
    choice = pipe.choice.cpu().numpy()
    idx, cnt = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    assert pipe.k == OB.budget(st["frac"], pipe.nb) == (81 if cfg == 4 else 192)
    band = 2 * (width // 2) + 1
    assert cnt.min() >= pipe.k and cnt.max() <= pipe.k + sink + band
    outf = None
    rng = np.random.default_rng(cfg)
    scale = wl.D ** -0.5
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
        scores = OB.minmax_block_scores(qp, kp, pipe.block)
        okeep = OB.topk_block_mask(scores, pipe.k, sink, width)
        static = OB.static_blocks(pipe.nb, pipe.nb, sink, width)
        gkeep = np.zeros_like(okeep)
        for I in range(pipe.nb):
            gkeep[I, idx[0, h, I, :cnt[0, h, I]]] = True
        for I, J in zip(*np.nonzero(okeep != gkeep)):
            assert not static[I, J]
            assert OB.near_tie_ok(scores[I], pipe.k, J, TOPK_REL), (h, I, J)
        # sampled rows of the output (T-major), attended over the GPU's kept lists
        rows_p = _sample_rows(cnt[0, h], pipe.nb, pipe.block, rng)
        want_p = OA.block_sparse_rows(qp, kp, vp, gkeep, pipe.block, rows_p, scale)
        if outf is None:
            outf = out
        got = f64(outf[0, h, torch.from_numpy(perm[rows_p]).cuda()])
        assert max_abs(got, want_p) <= BF16_ATOL, h


@pytest.mark.gpu
def test_adaptive_pipeline_small_grid_every_output():
    """The whole recipe on a small grid: every output against the oracle pipeline."""
    torch = torch_gpu()
    grid, tiles = (4, 8, 8), [(1, 4, 8), (4, 2, 4), (2, 4, 4)]
    H, D = 4, 64
    q, k, v = (synth.normal_bits((1, H, 256, D), seed=500 + i) for i in range(3))
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    pipe = bsa.AdaptiveBlockSparse(1, H, grid, D, tiles, 0.25, qg.dtype, qg.device)
    out = f64(pipe(qg, kg, vg))
    ref = OP.adaptive_block_sparse(*(synth.stored_to_f64(x) for x in (q, k, v)), grid, tiles, 0.25)
    choice = pipe.choice.cpu().numpy()
    kv_idx, kv_cnt = pipe.kv
    idx, cnt = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    for h in range(H):
        if choice[0, h] != ref["choice"][0, h]:
            a, b = ref["tiling_score"][0, h, choice[0, h]], ref["tiling_score"][0, h, ref["choice"][0, h]]
            assert abs(a - b) < TOPK_REL * abs(b)
            continue
        gkeep = np.zeros((8, 8), bool)
        for I in range(8):
            gkeep[I, idx[0, h, I, :cnt[0, h, I]]] = True
        if np.array_equal(gkeep, ref["keep"][0, h]):
            assert max_abs(out[0, h], ref["out"][0, h]) <= BF16_ATOL, h


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
