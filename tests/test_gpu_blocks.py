"""Cohesion, tiling choice, min/max block scores and top-k against the oracle."""
import numpy as np
import pytest

from block_sparse_attention_permute_amd import bsa, synth
from oracle import blocks as OB
from oracle import tiling as OT
from tests.gpu_helpers import TOPK_REL, bits, f64, gpu, top_p_row_ok, torch_gpu

WAN_GRID, WAN_TILES = (20, 32, 48), [(1, 8, 8), (4, 4, 4)]


# ------------------------------------------------------------- cohesion ---

@pytest.mark.gpu
@pytest.mark.parametrize("dtype,D,block", [("bf16", 64, 16), ("bf16", 128, 64), ("f32", 16, 8), ("bf16", 8, 5)])
def test_block_cohesion(dtype, D, block):
    torch_gpu()
    S = block * 24
    x = synth.normal_bits((1, 3, S, D), seed=D + block, dtype=dtype)
    if dtype == "bf16":
        x[0, 0, :block] = 0                         # empty block -> NaN
        x[0, 0, block + 1:2 * block] = 0            # one non-zero token -> NaN
        x[0, 1, 3 * block:3 * block + 2] = 0        # two zero tokens are left out
    got = bsa.bsa_block_cohesion(gpu(x), block).cpu().numpy().astype(np.float64)
    xf = synth.stored_to_f64(x)
    for h in range(3):
        want = OT.block_self_similarity(xf[0, h], block)
        assert np.array_equal(np.isnan(got[0, h]), np.isnan(want))
        ok = ~np.isnan(want)
        assert np.max(np.abs(got[0, h][ok] - want[ok])) < 2e-5


@pytest.mark.gpu
def test_select_tiling_wan_shape_against_oracle():
    """Full Wan 2.1 grid, all 40 heads: scores within 1e-5 and every choice equal to the oracle's (a
    different choice only at a near tie).  The inputs' temporal heads pick (4, 4, 4) and their spatial
    heads (1, 8, 8), so both candidates occur."""
    torch = torch_gpu()
    q = synth.tensor_bits(4, synth.ROLE_Q)
    choice, score, _ = bsa.bsa_select_tiling(gpu(q), WAN_GRID, WAN_TILES)
    torch.cuda.synchronize()
    ochoice, oscore = OT.select_tiling(synth.stored_to_f64(q), WAN_GRID, WAN_TILES)
    s = score.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(s - oscore)) < 1e-5
    c = choice.cpu().numpy()
    differ = 0
    for h in range(40):
        if c[0, h] != ochoice[0, h]:
            a, b = oscore[0, h, c[0, h]], oscore[0, h, ochoice[0, h]]
            assert abs(a - b) < TOPK_REL * abs(b), (h, a, b)
            differ += 1
    assert differ == 0                        # no near tie at this workload: every choice is the oracle's
    assert set(ochoice[0].tolist()) == {0, 1}
    spatial = [h for h in range(40) if synth.head_kind(4, h) == synth.HEAD_SPATIAL]
    assert 0 < len(spatial) < 40 and all(ochoice[0, h] == 0 for h in spatial)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,D,grid,tiles", [("bf16", 128, (4, 16, 16), [(1, 8, 8), (4, 4, 4)]),
                                                ("f32", 16, (4, 8, 8), [(1, 4, 8), (2, 4, 4), (4, 2, 4)])])
def test_select_tiling_q_summaries(dtype, D, grid, tiles):
    """The tiling choice pass's q summaries equal the oracle's block max / min of the permuted q for every
    candidate (exact), leave the choice unchanged, and give the tiled scores pass the same result as reading
    q itself."""
    torch = torch_gpu()
    H = 3
    S = grid[0] * grid[1] * grid[2]
    vol = tiles[0][0] * tiles[0][1] * tiles[0][2]
    nb, n = S // vol, len(tiles)
    q, k = (synth.normal_bits((1, H, S, D), seed=1500 + i + D, dtype=dtype) for i in range(2))
    q[0, 1, 5:40] = 0                                  # zero tokens count in the summaries
    qg, kg = gpu(q), gpu(k)
    qs = torch.full((n, 2, 1, H, nb, D), float("nan"), dtype=qg.dtype, device="cuda")
    choice, score, coh = bsa.bsa_select_tiling(qg, grid, tiles, q_summaries=qs)
    choice0, score0, _ = bsa.bsa_select_tiling(qg, grid, tiles)
    assert torch.equal(choice, choice0) and torch.equal(score, score0)
    got = f64(qs)
    qf = synth.stored_to_f64(q)
    for c, t in enumerate(tiles):
        perm = OT.tile_permutation(grid, t)
        for h in range(H):
            mx, mn = OB.block_minmax(OT.permute_tokens(qf[0, h], perm), vol)
            assert np.array_equal(got[c, 0, 0, h], mx), (c, h)
            assert np.array_equal(got[c, 1, 0, h], mn), (c, h)
    kn = torch.empty((1, H, nb), dtype=torch.float32, device="cuda")
    kn0 = torch.empty_like(kn)
    sc, summ = bsa.bsa_minmax_block_scores_tiled(qg, kg, grid, tiles, head_choice=choice, key_norms=kn,
                                                 q_summaries=qs)
    sc0, summ0 = bsa.bsa_minmax_block_scores_tiled(qg, kg, grid, tiles, head_choice=choice, key_norms=kn0)
    assert torch.equal(sc, sc0) and torch.equal(summ, summ0) and torch.equal(kn, kn0)
    with pytest.raises(ValueError, match="q_summaries"):
        bsa.bsa_select_tiling(qg, grid, tiles, q_summaries=qs[:, :, :, :, :-1])


@pytest.mark.gpu
def test_select_tiling_ties_and_constructed_choice():
    torch = torch_gpu()
    grid = (2, 4, 4)
    tiles = [(2, 1, 1), (1, 2, 2), (1, 1, 4), (1, 2, 2)]
    rng = np.random.default_rng(3)
    vecs = rng.standard_normal((8, 32))
    lab = OT.tile_labels(grid, (1, 2, 2))
    q = np.empty((1, 2, 32, 32))
    q[0, 0] = vecs[lab]
    q[0, 1] = vecs[OT.tile_labels(grid, (1, 1, 4))]
    qb = synth.round_to_bf16_bits(q)
    choice, score, _ = bsa.bsa_select_tiling(gpu(qb), grid, tiles)
    c = choice.cpu().numpy()
    assert c[0, 0] == 1 and c[0, 1] == 2                # exact ties go to the lower index
    ochoice, oscore = OT.select_tiling(synth.stored_to_f64(qb), grid, tiles)
    assert np.array_equal(c, ochoice)
    assert np.max(np.abs(score.cpu().numpy() - oscore)) < 1e-5


# ----------------------------------------------------------- block scores ---

def _score_bound(qp, kp, block):
    """|c| . max(|kmax|, |kmin|) per (I, J): scale of the rounding error of a score."""
    qmax, qmin = OB.block_minmax(qp, block)
    kmax, kmin = OB.block_minmax(kp, block)
    c = np.abs(qmax + qmin)
    return c @ np.maximum(np.abs(kmax), np.abs(kmin)).T


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,S,D,block", [("bf16", 30720, 128, 64), ("bf16", 2048, 64, 32), ("f32", 96, 16, 8),
                                             ("bf16", 200, 128, 5)])
def test_minmax_block_scores(dtype, S, D, block):
    torch_gpu()
    H = 2
    if S == 30720:
        grid = WAN_GRID
        q = synth.tensor_bits(4, synth.ROLE_Q, heads=[0, 5])
        k = synth.tensor_bits(4, synth.ROLE_K, heads=[0, 5])
        perm = OT.tile_permutation(grid, (4, 4, 4))
        q, k = q[:, :, perm], k[:, :, perm]
    else:
        q = synth.normal_bits((1, H, S, D), seed=11 + S, dtype=dtype)
        k = synth.normal_bits((1, H, S, D), seed=12 + S, dtype=dtype)
    scores, summ = bsa.bsa_minmax_block_scores(gpu(q), gpu(k), block)
    sc = scores.cpu().numpy().astype(np.float64)
    sm = synth.stored_to_f64(bits(summ))
    qf, kf = synth.stored_to_f64(q), synth.stored_to_f64(k)
    for h in range(H):
        qmax, qmin = OB.block_minmax(qf[0, h], block)
        kmax, kmin = OB.block_minmax(kf[0, h], block)
        for got, want in zip(sm[:, 0, h], (qmax, qmin, kmax, kmin)):
            assert np.array_equal(got, want)                # summaries are exact
        want = OB.minmax_block_scores(qf[0, h], kf[0, h], block)
        err = np.abs(sc[0, h] - want)
        # fp32 dot products of length D: |error| <= (D + 2) u sum|c_d k_d|, u = 2^-24
        assert np.all(err <= (D + 2) * 2.0 ** -24 * _score_bound(qf[0, h], kf[0, h], block) + 1e-30)


# ------------------------------------------------------------------ top-k ---

def _check_topk(scores_np, k, sink, diag, max_kept=None):
    torch = torch_gpu()
    s = torch.from_numpy(scores_np.astype(np.float32)).cuda()
    kv_idx, kv_cnt, mask = bsa.bsa_topk_block_mask(s, k, sink, diag, max_kept=max_kept, return_mask=True)
    idx, cnt, m = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy(), mask.cpu().numpy().astype(bool)
    B, H, Nq, Nk = scores_np.shape
    for b in range(B):
        for h in range(H):
            keep = OB.topk_block_mask(scores_np[b, h].astype(np.float32).astype(np.float64), k, sink, diag)
            assert np.array_equal(m[b, h], keep), (b, h)
            for I in range(Nq):
                li = np.flatnonzero(keep[I])
                assert cnt[b, h, I] == li.size
                assert np.array_equal(idx[b, h, I, :li.size], li)
                assert np.all(idx[b, h, I, li.size:] == -1)
    return idx, cnt


@pytest.mark.gpu
def test_topk_random_and_tie_heavy_rows():
    rng = np.random.default_rng(0)
    _check_topk(rng.standard_normal((1, 3, 37, 100)), 17, 1, True)
    _check_topk(rng.integers(-3, 4, (2, 2, 20, 70)).astype(np.float64), 9, 1, True)   # many exact ties
    _check_topk(rng.integers(0, 2, (1, 1, 8, 64)).astype(np.float64), 20, 0, False)
    _check_topk(rng.standard_normal((1, 2, 16, 16)), 16, 1, True)                    # k = Nk keeps all


@pytest.mark.gpu
def test_topk_special_values():
    s = np.array([[[[np.nan, -0.0, 0.0, -np.inf, np.inf, 1.0, np.nan, -1.0, 0.0, 2.0]]]])
    for k in range(1, 11):
        _check_topk(np.broadcast_to(s, (1, 1, 3, 10)).copy(), k, 0, False)
        _check_topk(np.broadcast_to(s, (1, 1, 3, 10)).copy(), k, 2, True)


@pytest.mark.gpu
@pytest.mark.parametrize("Nq,Nk,k,sink", [(480, 480, 81, 1), (64, 1920, 192, 1), (8, 4096, 1, 3), (70, 33, 5, 1),
                                          (33, 70, 70, 0)])
def test_topk_workload_widths(Nq, Nk, k, sink):
    rng = np.random.default_rng(Nk)
    s = rng.standard_normal((1, 2, Nq, Nk)) * 100
    s[..., ::7] = np.round(s[..., ::7])                      # sprinkle exact ties
    idx, cnt = _check_topk(s, k, sink, True)
    assert cnt.min() >= k and cnt.max() <= min(Nk, k + sink + 1)


@pytest.mark.gpu
@pytest.mark.parametrize("sink,width", [(5, 40), (0, 0), (2, 2), (1, 3), (0, 1000)])
def test_topk_sink_and_band_widths(sink, width):
    """SPADE's static widths (sink 5, band 40 at the Wan shape) and edge widths, bit-exact."""
    rng = np.random.default_rng(width + 7)
    s = rng.standard_normal((1, 2, 480, 480)) * 50
    idx, cnt = _check_topk(s, 81, sink, width)
    band = 2 * (width // 2) + 1 if width else 0
    assert cnt.max() <= min(480, 81 + sink + band)


# ------------------------------------------------------------------ top-p ---

def _check_top_p(scores_np, p, scale, sink, width):
    """GPU top-p against the oracle, row by row (tests.gpu_helpers.top_p_row_ok)."""
    torch = torch_gpu()
    s32 = scores_np.astype(np.float32)
    s = torch.from_numpy(s32).cuda()
    kv_idx, kv_cnt, mask = bsa.bsa_top_p_block_mask(s, p, scale, sink, width, return_mask=True)
    idx, cnt, m = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy(), mask.cpu().numpy().astype(bool)
    B, H, Nq, Nk = scores_np.shape
    for b in range(B):
        for h in range(H):
            sf = s32[b, h].astype(np.float64)
            static = OB.static_blocks(Nq, Nk, sink, width)
            for I in range(Nq):
                li = np.flatnonzero(m[b, h, I])
                assert cnt[b, h, I] == li.size and np.array_equal(idx[b, h, I, :li.size], li)
                assert np.all(idx[b, h, I, li.size:] == -1)
                assert top_p_row_ok(m[b, h, I], sf[I], p, scale, static[I]), (b, h, I)


@pytest.mark.gpu
@pytest.mark.parametrize("p,scale", [(0.5, 1.0), (0.9, 1.0), (0.99, 0.3), (0.2, 3.0)])
def test_top_p_random_rows(p, scale):
    rng = np.random.default_rng(int(p * 100))
    s = rng.standard_normal((1, 2, 40, 200)) * 3
    _check_top_p(s, p, scale, 1, 1)


@pytest.mark.gpu
def test_top_p_ties_uniform_and_special_values():
    rng = np.random.default_rng(11)
    _check_top_p(rng.integers(-2, 3, (1, 1, 30, 64)).astype(np.float64), 0.6, 1.0, 0, 0)   # many exact ties
    _check_top_p(np.zeros((1, 1, 4, 10)), 0.35, 1.0, 0, 0)                               # uniform: ceil(p n)
    _check_top_p(np.zeros((1, 1, 4, 10)), 1.0, 1.0, 0, 0)                                # p = 1 keeps all
    s = np.array([[[[np.nan, 0.5, -np.inf, 2.0, 2.0, -1.0, np.nan, 0.0]]]])
    for p in (0.1, 0.5, 0.8, 0.999):
        _check_top_p(np.broadcast_to(s, (1, 1, 3, 8)).copy(), p, 1.0, 1, 1)
    # the softmax's limit values: +inf maxima share the mass, only -inf numbers share it equally,
    # and a row of NaNs keeps its lowest index (no static blocks, so that block is the whole row)
    rows = np.array([[np.nan] * 8,
                     [1.0, np.inf, 3.0, np.inf, np.nan, -np.inf, 0.0, np.inf],
                     [-np.inf, np.nan, -np.inf, -np.inf, np.nan, -np.inf, -np.inf, np.nan],
                     [np.nan, np.nan, np.nan, -np.inf, np.nan, np.nan, np.nan, np.nan]])
    for p in (0.1, 0.34, 0.5, 0.7, 1.0):
        _check_top_p(rows[None, None], p, 1.0, 0, 0)
    torch = torch_gpu()
    _, cnt = bsa.bsa_top_p_block_mask(torch.full((1, 1, 2, 130), float("nan"), device="cuda"), 0.5, 1.0, 0, 0)
    assert cnt.cpu().numpy().tolist() == [[[1, 1]]]


@pytest.mark.gpu
def test_top_p_wan_shape_scores():
    """Min/max scores of the Wan-shape inputs (a sample of heads) under the
    softmax scale: counts vary per row and include the static blocks."""
    torch = torch_gpu()
    heads = [0, 5]
    q = synth.tensor_bits(4, synth.ROLE_Q, heads=heads)
    k = synth.tensor_bits(4, synth.ROLE_K, heads=heads)
    qp, kp = (bsa.bsa_tile_permute(gpu(x), WAN_GRID, [(4, 4, 4)]) for x in (q, k))
    scores, _ = bsa.bsa_minmax_block_scores(qp, kp, 64)
    s = scores.cpu().numpy().astype(np.float64)
    _check_top_p(s[:, :, :48], 0.9, 128 ** -0.5, 5, 40)
