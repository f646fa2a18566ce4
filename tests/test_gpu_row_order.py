"""Launch plans: bsa_row_order for block lists of varying length, bsa_row_order_by_median for top-k lists.

A plan only decides which workgroup runs which query block, so attention under a plan must equal attention
without one bit for bit.  Each plan is checked against the rule bsa.h states, written out here on the host:
for bsa_row_order unit placement exactly, and inside each unit the rows as a set with non-increasing counts
(rows of one count may come in any order); for bsa_row_order_by_median the plain XCD ranges over a sequence in
which each head's rows fill their own slots with non-decreasing middle kept blocks (rows of one key may come in
any order).
"""
import numpy as np
import pytest

from block_sparse_attention_permute_amd import bsa, synth
from oracle import attention as OA
from tests.gpu_helpers import BF16_ATOL, f64, gpu, max_abs, torch_gpu

EMPTY = -1          # an empty slot, 0xFFFFFFFF read as int32
ROW_COST = 5        # fixed cost of a row in the unit weights, in blocks
BINS = 256          # counts of BINS - 1 or more rank as one


def plan_rule(cnt):
    """(units of each XCD in run order, rows per unit, rows per XCD) for counts cnt of shape (BH, Nq)."""
    BH, nq = cnt.shape
    r = 1
    while r < 8 and BH * r < 16:
        r *= 2
    while nq % r:
        r //= 2
    ur, U = nq // r, BH * r
    flat = np.clip(cnt.reshape(-1).astype(np.int64), 0, 65535)
    weight = [int(flat[u * ur:(u + 1) * ur].sum()) + ROW_COST * ur for u in range(U)]
    shift = max(0, sum(weight).bit_length() - 28)
    weight = [w >> shift for w in weight]
    room = -(-U // 8)
    load, units = [0] * 8, [[] for _ in range(8)]
    for u in sorted(range(U), key=lambda u: (-weight[u], u)):
        x = min((x for x in range(8) if len(units[x]) < room), key=lambda x: (load[x], x))
        units[x].append(u)
        load[x] += weight[u]
    return units, ur, room * ur


def check_plan(order, cnt):
    units, ur, cap = plan_rule(cnt)
    n_units = sum(len(us) for us in units)
    o = order.cpu().numpy().astype(np.int64)
    assert o.size >= 8 * cap + 3 * n_units == bsa.bsa_row_order_len(*cnt.shape)
    assert np.all(o[8 * cap:] == EMPTY)          # the scratch words and anything past the plan read as empty
    key = np.clip(cnt.reshape(-1), 0, BINS - 1)
    for x in range(8):
        lane = o[:8 * cap][x::8]
        assert np.all(lane[len(units[x]) * ur:] == EMPTY), x
        for j, u in enumerate(units[x]):
            seg = lane[j * ur:(j + 1) * ur]
            assert np.array_equal(np.sort(seg), np.arange(u * ur, (u + 1) * ur)), (x, u)
            assert np.all(np.diff(key[seg]) <= 0), (x, u)


def skewed_counts(shape, rng, top):
    """Mostly short lists and a few long ones (the top-p shape), with 0, negative and > 255 entries mixed in."""
    c = np.minimum(top, (rng.pareto(1.1, shape) * 4).astype(np.int64) + 1)
    c[rng.random(shape) < 0.02] = 0
    c[rng.random(shape) < 0.01] = -3
    c[rng.random(shape) < 0.01] = 300
    return c.astype(np.int32)


@pytest.mark.gpu
@pytest.mark.parametrize("B,H,nq", [(1, 40, 480), (2, 3, 64), (1, 1, 7), (1, 5, 12), (1, 1024, 2), (1, 1, 1),
                                    (3, 8, 40), (1, 4, 16384), (1, 16, 4096)])
def test_plan_follows_its_rule(B, H, nq):
    """(1, 4, 16384): more rows than the LDS cache holds; (1, 16, 4096): counts near 65535, so that the total
    weight passes 2^28 and the weights are shifted."""
    torch = torch_gpu()
    rng = np.random.default_rng(B * 1000 + H * 10 + nq)
    cnt = skewed_counts((B, H, nq), rng, 5000)
    if H == 16:
        cnt = rng.integers(60000, 70000, (B, H, nq)).astype(np.int32)
        assert int(np.clip(cnt, 0, 65535).sum()) + 5 * cnt.size >= 1 << 28
    cg = torch.from_numpy(cnt).cuda()
    check_plan(bsa.bsa_row_order(cg), cnt.reshape(B * H, nq))
    n = bsa.bsa_row_order_len(B * H, nq)
    longer = torch.full((n + 37,), 7, dtype=torch.int32, device="cuda")     # a longer buffer: the rest is empty
    check_plan(bsa.bsa_row_order(cg, out=longer), cnt.reshape(B * H, nq))


@pytest.mark.gpu
@pytest.mark.parametrize("case", ["zeros", "one_heavy_head", "equal"])
def test_plan_edge_weights(case):
    """All counts 0 (equal weights: units in index order round the XCDs), one head holding nearly all the work
    (it gets an XCD of its own share while the others fill the rest), and equal top-k counts."""
    torch = torch_gpu()
    B, H, nq = 1, 24, 96
    if case == "zeros":
        cnt = np.zeros((B, H, nq), np.int32)
    elif case == "one_heavy_head":
        cnt = np.ones((B, H, nq), np.int32)
        cnt[0, 7] = 4000
    else:
        cnt = np.full((B, H, nq), 17, np.int32)
    order = bsa.bsa_row_order(torch.from_numpy(cnt).cuda())
    check_plan(order, cnt.reshape(B * H, nq))
    units, _, _ = plan_rule(cnt.reshape(B * H, nq))
    if case != "one_heavy_head":
        assert [len(us) for us in units] == [3] * 8
    else:
        heavy = next(x for x in range(8) if 7 in units[x])
        assert units[heavy][0] == 7


def _varying_lists(B, H, nb, rng):
    """Full-width lists whose lengths run from 0 to nb (density per row cubed), the diagonal kept."""
    torch = torch_gpu()
    dens = rng.random((B, H, nb, 1)) ** 3
    keep = rng.random((B, H, nb, nb)) < dens
    keep[..., np.arange(nb), np.arange(nb)] |= rng.random((B, H, nb)) < 0.9
    keep[0, 0, 1] = False                                        # an empty list: written as zeros
    cnt = keep.sum(-1).astype(np.int32)
    idx = np.full((B, H, nb, nb), -1, np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                li = np.flatnonzero(keep[b, h, i])
                idx[b, h, i, :li.size] = li
    return keep, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()


def _any_order(rows, rng):
    """A random permutation of the rows with empty slots strewn among them."""
    torch = torch_gpu()
    o = np.concatenate([rng.permutation(rows), np.full(rows // 3 + 5, EMPTY)]).astype(np.int32)
    return torch.from_numpy(rng.permutation(o)).cuda()


@pytest.mark.gpu
@pytest.mark.parametrize("D,block", [(128, 64), (64, 64), (128, 32), (64, 32)])
def test_block_list_attention_under_a_plan(D, block):
    """bf16 block lists of every length on each MFMA kernel (B = 2, H = 3): the planned launch and a random
    padded order give the unplanned result bit for bit; rows of head (1, 2) under the plan match the oracle."""
    torch = torch_gpu()
    B, H, S = 2, 3, 2048
    nb = S // block
    rng = np.random.default_rng(D + block)
    keep, kv_idx, kv_cnt = _varying_lists(B, H, nb, rng)
    q, k, v = (synth.normal_bits((B, H, S, D), seed=7100 + D + block + i) for i in range(3))
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    ref = bsa.bsa_block_sparse_attention(qg, kg, vg, kv_idx, kv_cnt, block)
    plan = bsa.bsa_row_order(kv_cnt)
    check_plan(plan, kv_cnt.cpu().numpy().reshape(B * H, nb))
    out = bsa.bsa_block_sparse_attention(qg, kg, vg, kv_idx, kv_cnt, block, row_order=plan)
    assert torch.equal(out, ref)
    out2 = bsa.bsa_block_sparse_attention(qg, kg, vg, kv_idx, kv_cnt, block, row_order=_any_order(B * H * nb, rng))
    assert torch.equal(out2, ref)
    o = f64(out)[1, 2]
    seen = keep[1, 2].any(-1)
    rows = np.flatnonzero(np.repeat(seen, block))
    qf, kf, vf = (synth.stored_to_f64(x)[1, 2] for x in (q, k, v))
    want = OA.block_sparse_rows_gathered(qf, kf, vf, keep[1, 2], block, rows, D ** -0.5)
    assert max_abs(o[rows], want) <= BF16_ATOL
    assert np.all(o[np.repeat(~seen, block)] == 0.0)


@pytest.mark.gpu
def test_f32_attention_ignores_the_plan():
    torch = torch_gpu()
    B, H, S, D, block = 1, 2, 256, 32, 32
    rng = np.random.default_rng(77)
    _, kv_idx, kv_cnt = _varying_lists(B, H, S // block, rng)
    q, k, v = (synth.normal_bits((B, H, S, D), seed=7700 + i, dtype="f32") for i in range(3))
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    ref = bsa.bsa_block_sparse_attention(qg, kg, vg, kv_idx, kv_cnt, block)
    out = bsa.bsa_block_sparse_attention(qg, kg, vg, kv_idx, kv_cnt, block, row_order=bsa.bsa_row_order(kv_cnt))
    assert torch.equal(out, ref)


@pytest.mark.gpu
def test_tiled_attention_under_a_plan():
    """T-major tensors, two tilings, five heads (not a multiple of 8), lists of every length: the planned
    launch equals the unplanned one and the permuted path bit for bit; so does a random padded order."""
    torch = torch_gpu()
    grid, tiles, H, D = (4, 32, 32), [(1, 8, 8), (4, 4, 4)], 5, 128
    S, nb = 4096, 64
    rng = np.random.default_rng(5151)
    _, kv_idx, kv_cnt = _varying_lists(1, H, nb, rng)
    q, k, v = (synth.normal_bits((1, H, S, D), seed=5200 + i) for i in range(3))
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    choice = torch.tensor([[0, 1, 1, 0, 1]], dtype=torch.int32, device="cuda")
    kn = torch.full((1, H, nb), -1.0, dtype=torch.float32, device="cuda")
    bsa.bsa_minmax_block_scores_tiled(qg, kg, grid, tiles, head_choice=choice, key_norms=kn)
    for norms in (None, kn):
        ref = bsa.bsa_block_sparse_attention_tiled(qg, kg, vg, grid, tiles, kv_idx, kv_cnt, head_choice=choice,
                                                   key_norms=norms)
        for order in (bsa.bsa_row_order(kv_cnt), _any_order(H * nb, rng)):
            out = bsa.bsa_block_sparse_attention_tiled(qg, kg, vg, grid, tiles, kv_idx, kv_cnt, head_choice=choice,
                                                       key_norms=norms, row_order=order)
            assert torch.equal(out, ref)
    qp, kp, vp = (bsa.bsa_tile_permute(x, grid, tiles, head_choice=choice) for x in (qg, kg, vg))
    perm = bsa.bsa_invert_permute(bsa.bsa_block_sparse_attention(qp, kp, vp, kv_idx, kv_cnt, 64), grid, tiles,
                                  head_choice=choice)
    assert torch.equal(ref, perm)


@pytest.mark.gpu
def test_padded_attention_under_a_plan():
    """Padded candidates (heads with different block counts and budgets): the padded pipeline plans its launch,
    and its output equals the unplanned padded attention bit for bit; so does a random padded order."""
    torch = torch_gpu()
    grid, tiles, H, D = (6, 16, 16), [(1, 8, 8), (4, 4, 4)], 5, 128          # (4,4,4) pads T from 6 to 8
    q, k, v = (synth.normal_bits((1, H, 1536, D), seed=5400 + i) for i in range(3))
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    pipe = bsa.AdaptiveBlockSparse(1, H, grid, D, tiles, 0.3, qg.dtype, qg.device, pad=True)
    out = pipe(qg, kg, vg)
    kv_idx, kv_cnt = pipe.kv
    assert pipe.ws_order is not None
    check_plan(pipe.ws_order, kv_cnt.cpu().numpy().reshape(H, -1))
    ref = bsa.bsa_block_sparse_attention_tiled_padded(qg, kg, vg, grid, tiles, kv_idx, kv_cnt,
                                                      head_choice=pipe.choice, key_norms=pipe.ws_knorm)
    assert torch.equal(out, ref)
    rng = np.random.default_rng(5401)
    out2 = bsa.bsa_block_sparse_attention_tiled_padded(qg, kg, vg, grid, tiles, kv_idx, kv_cnt,
                                                       head_choice=pipe.choice, key_norms=pipe.ws_knorm,
                                                       row_order=_any_order(kv_cnt.numel(), rng))
    assert torch.equal(out2, ref)


@pytest.mark.gpu
def test_top_p_pipeline_plans_its_launch():
    """The top-p pipeline plans its attention launch: the plan follows the rule for the pipeline's own lists,
    and the pipeline's output equals the unplanned attention on the same lists bit for bit."""
    torch = torch_gpu()
    grid, tiles, H, D = (4, 32, 32), [(1, 8, 8), (4, 4, 4)], 6, 128
    q, k, v = (synth.normal_bits((1, H, 4096, D), seed=5300 + i) for i in range(3))
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    pipe = bsa.AdaptiveBlockSparse(1, H, grid, D, tiles, 0.25, qg.dtype, qg.device, top_p=0.7, p_scale=D ** -0.5)
    out = pipe(qg, kg, vg)
    kv_idx, kv_cnt = pipe.kv
    assert pipe.ws_order is not None
    check_plan(pipe.ws_order, kv_cnt.cpu().numpy().reshape(H, -1))
    ref = bsa.bsa_block_sparse_attention_tiled(qg, kg, vg, grid, tiles, kv_idx, kv_cnt, head_choice=pipe.choice,
                                               key_norms=pipe.ws_knorm)
    assert torch.equal(out, ref)


def check_median_order(order, kv_idx, kv_cnt, nk, xcds_per_head=1):
    """order follows bsa_row_order_by_median's rule for the lists kv_idx (B, H, Nq, max_kept) / kv_cnt (B, H, Nq);
    xcds_per_head = 2: bsa_row_order_by_median_ex's split of each head over XCDs 2g and 2g + 1."""
    idx, cnt = kv_idx.cpu().numpy(), kv_cnt.cpu().numpy()
    B, H, nq = cnt.shape
    BH, max_kept = B * H, idx.shape[-1]
    n = BH * nq
    per = n // 8
    o = order.cpu().numpy().astype(np.int64)
    assert o.size >= n
    seq = np.empty(n, dtype=np.int64)            # the rows of head h at seq[h*nq : (h+1)*nq], in order
    if xcds_per_head == 1:                       # slot x*per + j holds order[8j + x]
        for x in range(8):
            seq[x * per:(x + 1) * per] = o[:n][x::8]
    else:                                        # head h = g + 4*hl: XCD 2g's slots of that head, then XCD 2g+1's
        assert xcds_per_head == 2 and BH % 4 == 0 and nq % 2 == 0
        part = nq // 2
        for h in range(BH):
            g, hl = h % 4, h // 4
            for i in range(2):
                x = 2 * g + i
                seq[h * nq + i * part:h * nq + (i + 1) * part] = o[:n][x::8][hl * part:(hl + 1) * part]
    assert np.array_equal(np.sort(seq), np.arange(n))
    idx2, cnt2 = idx.reshape(BH, nq, max_kept), np.clip(cnt.reshape(BH, nq), 0, max_kept)

    def key(r):
        h, i = divmod(int(r), nq)
        c = cnt2[h, i]
        return 0 if c == 0 else int(min(max(idx2[h, i, c // 2], 0), nk - 1))

    for h in range(BH):
        seg = seq[h * nq:(h + 1) * nq]
        assert np.array_equal(np.sort(seg), np.arange(h * nq, (h + 1) * nq)), h
        keys = [key(r) for r in seg]
        assert all(a <= b for a, b in zip(keys, keys[1:])), h


def _sorted_lists(B, H, nq, nk, max_kept, rng, empty_share=0.1):
    """Ascending kept lists of random length (some empty), padded with -1, as bsa_topk_block_mask writes them."""
    cnt = rng.integers(1, max_kept + 1, (B, H, nq))
    cnt[rng.random((B, H, nq)) < empty_share] = 0
    idx = np.full((B, H, nq, max_kept), -1, dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nq):
                c = int(cnt[b, h, i])
                idx[b, h, i, :c] = np.sort(rng.choice(nk, c, replace=False))
    return idx, cnt.astype(np.int32)


@pytest.mark.gpu
@pytest.mark.parametrize("B,H,nq,nk,max_kept", [(1, 40, 480, 480, 83), (1, 3, 8, 8, 4), (2, 3, 12, 12, 5),
                                                (1, 1, 8, 4096, 300), (1, 24, 64, 64, 7)])
def test_median_order_follows_its_rule(B, H, nq, nk, max_kept):
    """Random ascending lists, empty rows among them; heads that straddle XCD ranges (3 heads of 8 rows over
    8 ranges of 3), Nk at its 4096 limit."""
    torch = torch_gpu()
    rng = np.random.default_rng(7100 + B * H * nq + nk)
    idx, cnt = _sorted_lists(B, H, nq, nk, max_kept, rng)
    kv_idx, kv_cnt = (torch.from_numpy(a).to("cuda") for a in (idx, cnt))
    order = bsa.bsa_row_order_by_median(kv_idx, kv_cnt, nk=nk)
    check_median_order(order, kv_idx, kv_cnt, nk)


@pytest.mark.gpu
@pytest.mark.parametrize("BH,nq,head_bytes,split", [(8, 64, 64 << 20, True), (24, 40, (32 << 20) + 1, True),
                                                    (8, 64, 32 << 20, False), (6, 8, 64 << 20, False),
                                                    (8, 9, 64 << 20, False), (8, 64, 0, False)])
def test_median_order_split_over_two_xcds(BH, nq, head_bytes, split):
    """Heads of more than 32 MiB of K and V go to two XCDs, each taking one half of the head's sorted rows,
    when 4 divides BH and Nq is even; otherwise (and at 32 MiB or with the size unknown) the plain rule."""
    torch = torch_gpu()
    rng = np.random.default_rng(7150 + BH * nq)
    idx, cnt = _sorted_lists(1, BH, nq, nq, 7, rng)
    kv_idx, kv_cnt = (torch.from_numpy(a).to("cuda") for a in (idx, cnt))
    order = bsa.bsa_row_order_by_median(kv_idx, kv_cnt, head_kv_bytes=head_bytes)
    check_median_order(order, kv_idx, kv_cnt, nq, 2 if split else 1)
    plain = bsa.bsa_row_order_by_median(kv_idx, kv_cnt)
    assert torch.equal(order, plain) != split


@pytest.mark.gpu
def test_attention_under_a_split_median_order():
    """Block-sparse attention under the two-XCD order equals it without one, bit for bit."""
    torch = torch_gpu()
    rng = np.random.default_rng(7350)
    B, H, S, D, block = 1, 8, 1024, 128, 64
    nb = S // block
    idx, cnt = _sorted_lists(B, H, nb, nb, 6, rng)
    kv_idx, kv_cnt = (torch.from_numpy(a).to("cuda") for a in (idx, cnt))
    q, k, v = (gpu(synth.normal_bits((B, H, S, D), seed=7360 + i)) for i in range(3))
    order = bsa.bsa_row_order_by_median(kv_idx, kv_cnt, head_kv_bytes=1 << 30)
    check_median_order(order, kv_idx, kv_cnt, nb, 2)
    got = bsa.bsa_block_sparse_attention(q, k, v, kv_idx, kv_cnt, block, row_order=order)
    ref = bsa.bsa_block_sparse_attention(q, k, v, kv_idx, kv_cnt, block)
    assert torch.equal(got, ref)


@pytest.mark.gpu
def test_median_order_clamps_bad_entries():
    """Middle entries outside [0, Nk) and counts outside [0, max_kept] are clamped, not read past."""
    torch = torch_gpu()
    rng = np.random.default_rng(7200)
    B, H, nq, nk, max_kept = 1, 2, 16, 16, 5
    idx, cnt = _sorted_lists(B, H, nq, nk, max_kept, rng, empty_share=0.0)
    cnt[0, 0, :4] = [7, -3, 99, 5]                 # clamped to max_kept, 0, max_kept, 5
    idx[0, 1, :4, 2] = [-5, 16, 1000, 3]           # middle entries of 5-long lists: clamped to 0 or Nk - 1
    cnt[0, 1, :4] = 5
    kv_idx, kv_cnt = (torch.from_numpy(a).to("cuda") for a in (idx, cnt))
    order = bsa.bsa_row_order_by_median(kv_idx, kv_cnt, nk=nk)
    check_median_order(order, kv_idx, kv_cnt, nk)


@pytest.mark.gpu
def test_attention_under_a_median_order():
    """Block-sparse attention on permuted copies under the order equals it without one, bit for bit."""
    torch = torch_gpu()
    rng = np.random.default_rng(7300)
    B, H, S, D, block = 1, 4, 1024, 128, 64
    nb = S // block
    idx, cnt = _sorted_lists(B, H, nb, nb, 6, rng)
    kv_idx, kv_cnt = (torch.from_numpy(a).to("cuda") for a in (idx, cnt))
    q, k, v = (gpu(synth.normal_bits((B, H, S, D), seed=7310 + i)) for i in range(3))
    order = bsa.bsa_row_order_by_median(kv_idx, kv_cnt)
    got = bsa.bsa_block_sparse_attention(q, k, v, kv_idx, kv_cnt, block, row_order=order)
    ref = bsa.bsa_block_sparse_attention(q, k, v, kv_idx, kv_cnt, block)
    assert torch.equal(got, ref)


@pytest.mark.gpu
@pytest.mark.parametrize("fused", [True, False])
def test_top_k_pipeline_orders_its_launch(fused):
    """The top-k pipeline orders its attention launch by the lists' middle blocks: the order follows its rule
    for the pipeline's own lists, and the output equals the unordered attention on the same lists bit for bit
    (fused: gather on load; unfused: permuted copies, compared after the inverse permutation)."""
    torch = torch_gpu()
    grid, tiles, H, D = (4, 32, 32), [(1, 8, 8), (4, 4, 4)], 6, 128
    q, k, v = (synth.normal_bits((1, H, 4096, D), seed=7400 + i) for i in range(3))
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    pipe = bsa.AdaptiveBlockSparse(1, H, grid, D, tiles, 0.25, qg.dtype, qg.device, fused=fused)
    out = pipe(qg, kg, vg)
    kv_idx, kv_cnt = pipe.kv
    assert pipe.ws_order is not None and pipe.order_by_median
    check_median_order(pipe.ws_order, kv_idx, kv_cnt, pipe.nb)
    if fused:
        ref = bsa.bsa_block_sparse_attention_tiled(qg, kg, vg, grid, tiles, kv_idx, kv_cnt,
                                                   head_choice=pipe.choice, key_norms=pipe.ws_knorm)
    else:
        op = bsa.bsa_block_sparse_attention(pipe.qp, pipe.kp, pipe.vp, kv_idx, kv_cnt, pipe.block,
                                            key_norms=pipe.ws_knorm)
        ref = bsa.bsa_invert_permute(op, grid, tiles, head_choice=pipe.choice)
    assert torch.equal(out, ref)
