"""Benchmark: adaptive-tiling block-sparse attention at the Wan 2.1 latent shape.

One step = the whole hot path over one batch already resident in HBM:
  select tiling (cohesion of q under (1,8,8) and (4,4,4)) -> min/max block
  scores of the tiles -> top-k (81 of 480, + sink + diagonal) -> block-sparse
  attention over the kept tiles -> output in T-major order.
The tile permutation is applied on load (scores and attention read q, k, v
in place through the tile geometry and the attention writes its rows back
in T-major order); the same step with permuted copies and the inverse pass
is timed beside it (`unfused_step_ms`) and must give identical bits.
Workload: B=1, H=40, grid 20x32x48 (S=30720), D=128, bf16, seeded synthetic
inputs (the Fourier-feature q/k recipe, v ~ N(0, 1)).

Prints ONE JSON line.  `value` is kept-block attention FLOPs per step
(4 * 64 * 64 * 128 per kept block, from the step's own kv_cnt) divided by the
whole step time.  `roofline` reports the attention kernel alone, timed with
HIP events on its stream.  `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
TILES = [(1, 8, 8), (4, 4, 4)]
DROPPED_TILES = [(16, 2, 2)]  # 16 does not divide T=20
FRAC = 0.17
CFG = 4
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_wan_traffic.json")
ATTN_SRC = os.path.join(ROOT, "block_sparse_attention_permute_amd", "csrc", "attention.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def attention_source_hash() -> str:
    """sha256 (16 hex digits) of the attention source, comments and blank lines removed, and its extra flags."""
    from block_sparse_attention_permute_amd.build import SOURCE_FLAGS
    with open(ATTN_SRC, encoding="utf-8") as f:
        lines = [re.sub(r"//.*$", "", line).rstrip() for line in f.read().splitlines()]
    lines.append(" ".join(SOURCE_FLAGS.get(os.path.basename(ATTN_SRC), [])))
    return hashlib.sha256("\n".join(line for line in lines if line).encode()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per attention launch from the committed counter runs, if still current."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("attention_source_sha256_16") != attention_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def host_description() -> dict:
    """The host the CPU oracle runs on: logical CPUs, CPU model and numpy's BLAS."""
    import subprocess

    import numpy as np
    from threadpoolctl import threadpool_info

    model = ""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        model = next((ln.split(":", 1)[1].strip() for ln in out.splitlines() if ln.startswith("Model name")), "")
    except (OSError, subprocess.SubprocessError):
        pass
    if not model:
        try:
            with open("/proc/cpuinfo") as f:
                model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
        except OSError:
            pass
    blas = np.show_config(mode="dicts").get("Build Dependencies", {}).get("blas", {})
    pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
    return {
        "cpu_count": os.cpu_count(),
        "cpu_model": model or "unknown",
        "blas": f"{blas.get('name', '?')} {blas.get('version', '')}".strip(),
        "blas_threads": max([i.get("num_threads", 1) for i in pools] or [1]),
    }


def cpu_baseline(q, k, v, wl, block, kk, budget_s=12.0):
    """Time the oracle, untuned, on whole heads of the same inputs: per head its tiling choice, permutation,
    min/max scores and top-k, then every output row in the oracle's gathered kept-block form (the same
    float64 math as the dense masked definition: masked keys contribute exact zeros).  Heads are taken in
    order until about `budget_s` seconds have passed (at least one head)."""
    import numpy as np

    from block_sparse_attention_permute_amd import synth
    from oracle import attention as OA
    from oracle import blocks as OB
    from oracle import tiling as OT

    host = host_description()
    scale = wl.D ** -0.5
    rows = np.arange(wl.S)
    heads, flops, t_total = 0, 0, 0.0
    while heads < wl.H and (heads == 0 or t_total < budget_s):
        qf, kf, vf = (synth.stored_to_f64(x[0, heads]) for x in (q, k, v))
        t0 = time.perf_counter()
        choice, _ = OT.select_tiling(qf[None, None], wl.grid, TILES)
        perm = OT.tile_permutation(wl.grid, TILES[int(choice[0, 0])])
        qp, kp, vp = (OT.permute_tokens(x, perm) for x in (qf, kf, vf))
        keep = OB.topk_block_mask(OB.minmax_block_scores(qp, kp, block), kk, 1, True)
        OA.block_sparse_rows_gathered(qp, kp, vp, keep, block, rows, scale)
        t_total += time.perf_counter() - t0
        flops += int(keep.sum()) * 4 * block * block * wl.D
        heads += 1
    return {
        "value": flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": host["blas_threads"],
        "kind": "oracle",
        "sample": (f"heads 0..{heads - 1} of {wl.H} of the same inputs, whole heads: tiling choice, scores, "
                   f"top-k and all {wl.S} output rows in the gathered kept-block form (float64, {t_total:.1f} s; "
                   f"kept-block FLOPs / time)"),
        "wall_s": round(t_total, 2),
        "wall_s_per_call_est": round(t_total / heads * wl.H, 1),
        "cpu_count": host["cpu_count"],
        "cpu_model": host["cpu_model"],
        "blas": host["blas"],
    }


def attention_call(bsa, pipe, q, k, v, out):
    """The pipeline's attention launch alone, on its current block lists."""
    kv_idx, kv_cnt = pipe.kv
    if pipe.fused and pipe.pad:
        return lambda: bsa.bsa_block_sparse_attention_tiled_padded(q, k, v, pipe.grid, pipe.tiles, kv_idx, kv_cnt,
                                                                   head_choice=pipe.choice, scale=pipe.scale,
                                                                   out=out, key_norms=pipe.ws_knorm,
                                                                   row_order=pipe.ws_order)
    if pipe.fused:
        return lambda: bsa.bsa_block_sparse_attention_tiled(q, k, v, pipe.grid, pipe.tiles, kv_idx, kv_cnt,
                                                            head_choice=pipe.choice, scale=pipe.scale, out=out,
                                                            key_norms=pipe.ws_knorm, row_order=pipe.ws_order)
    if pipe.pad:
        return lambda: bsa.bsa_block_sparse_attention_labels(pipe.qp, pipe.kp, pipe.vp, kv_idx, kv_cnt, pipe.block,
                                                             pipe.labels, pipe.scale, out=pipe.op)
    return lambda: bsa.bsa_block_sparse_attention(pipe.qp, pipe.kp, pipe.vp, kv_idx, kv_cnt, pipe.block, pipe.scale,
                                                  out=pipe.op, key_norms=pipe.ws_knorm, row_order=pipe.ws_order)


def _time(torch, fn, steps, warmup):
    """Average ms of fn() over `steps` calls, HIP events on the current stream."""
    for _ in range(warmup):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def _time_steady(torch, fn, warm_ms=150.0, min_ms=60.0, min_steps=5):
    """Average ms of fn() at a steady clock: calls run back to back for at least warm_ms of wall time (the GPU
    clock ramps up over the first tens of milliseconds of load), then enough calls to fill min_ms are timed
    with HIP events on the current stream."""
    torch.cuda.synchronize()
    t0, n = time.perf_counter(), 0
    while True:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= warm_ms:
                break
    per_ms = (time.perf_counter() - t0) * 1e3 / n
    return _time(torch, fn, max(min_steps, int(min_ms / max(per_ms, 1e-3)) + 1), 0)


def oracle_wall(fn, units, total_units):
    """Run fn(u) for u in units; -> (wall s of the sample, the same scaled to total_units)."""
    t0 = time.perf_counter()
    for u in units:
        fn(u)
    dt = time.perf_counter() - t0
    return round(dt, 3), round(dt * total_units / max(len(units), 1), 2)


def sweep(args, torch, np, bsa, synth):
    """Kernel timings on the sliding-tile, windowed and long-sequence workloads, each at a steady clock."""
    dev = torch.device("cuda:0")

    from oracle import attention as OA
    from oracle import blocks as OB
    from oracle import pipeline as OP
    from oracle import tiling as OT

    host = host_description()
    print(json.dumps({"host": host}), flush=True)

    # tiny windowed fp32: H=2, grid 2x4x4, D=16, window 8, sink 2, scale 1/4
    wl = synth.WORKLOADS[1]
    qb, kb, vb = synth.qkv(1)
    q, k, v = (synth.to_torch(x, dev) for x in (qb, kb, vb))
    out = torch.empty_like(q)
    ms = _time_steady(torch, lambda: bsa.bsa_windowed_attention(q, k, v, 8, 2, 0.25, 8, out=out))
    qf, kf, vf = (synth.stored_to_f64(x) for x in (qb, kb, vb))
    wall, _ = oracle_wall(lambda _: OA.windowed_attention(qf, kf, vf, 8, 2, scale=0.25, chunk=8), [0], 1)
    print(json.dumps({"workload": wl.name, "attention_ms": round(ms, 4), "oracle_wall_s": wall,
                      "oracle_sample": "the whole call (dense masked float64)"}), flush=True)

    # sliding tile: grid 8x16x16, tiles 2x4x4 (block 32), 3x3x3 neighbourhood, D=64, H=8
    wl = synth.WORKLOADS[2]
    qb, kb, vb = synth.qkv(2)
    q, k, v = (synth.to_torch(x, dev) for x in (qb, kb, vb))
    tile = [(2, 4, 4)]
    idx, cnt = bsa.bsa_sliding_tile_block_list((4, 4, 4))
    kv_idx = torch.from_numpy(np.broadcast_to(idx, (1, wl.H) + idx.shape).copy()).to(dev)
    kv_cnt = torch.from_numpy(np.broadcast_to(cnt, (1, wl.H, 64)).copy()).to(dev)
    qp, kp, vp = (bsa.bsa_tile_permute(x, wl.grid, tile) for x in (q, k, v))
    out = torch.empty_like(qp)
    ms = _time_steady(torch, lambda: bsa.bsa_block_sparse_attention(qp, kp, vp, kv_idx, kv_cnt, 32, out=out))
    fl = int(kv_cnt.sum().item()) * 4 * 32 * 32 * wl.D

    def step2():
        for x, y in ((q, qp), (k, kp), (v, vp)):
            bsa.bsa_tile_permute(x, wl.grid, tile, out=y)
        bsa.bsa_block_sparse_attention(qp, kp, vp, kv_idx, kv_cnt, 32, out=out)
        bsa.bsa_invert_permute(out, wl.grid, tile)
    ms_step = _time_steady(torch, step2)
    qf, kf, vf = (synth.stored_to_f64(x) for x in (qb, kb, vb))
    keep, labels = OT.sliding_tile_keep((4, 4, 4)), OT.tile_labels(wl.grid, tile[0])
    wall, _ = oracle_wall(lambda h: OP.label_mask_attention(qf[0, h], kf[0, h], vf[0, h], labels, keep, wl.D ** -0.5),
                          range(wl.H), wl.H)
    print(json.dumps({"workload": wl.name, "attention_ms": round(ms, 4), "attention_tflops": round(fl / ms / 1e9, 2),
                      "step_ms": round(ms_step, 4), "kept_block_flops": fl, "oracle_wall_s": wall,
                      "oracle_sample": "the whole call, all 8 heads (dense masked float64, T-major label form)"}),
          flush=True)

    # windowed: S=16384, window 2048 (half 1024), sink 64, D=128, H=24
    wl = synth.WORKLOADS[3]
    qb, kb, vb = synth.qkv(3)
    q, k, v = (synth.to_torch(x, dev) for x in (qb, kb, vb))
    out = torch.empty_like(q)
    ms = _time_steady(torch, lambda: bsa.bsa_windowed_attention(q, k, v, 2048, 64, 128 ** -0.5, 512, out=out))
    S, half, sink = wl.S, 1024, 64
    i = np.arange(S)
    local = np.minimum(S - 1, i + half) - np.maximum(0, i - half) + 1
    extra = np.maximum(0, np.minimum(sink, np.maximum(0, i - half)))      # sinks left of the window
    pairs = int((local + extra).sum())
    fl_tok = pairs * 4 * wl.D * wl.H
    qf, kf, vf = (synth.stored_to_f64(x[0, 0]) for x in (qb, kb, vb))
    wall, full = oracle_wall(lambda _: OA.window_rows_gathered(qf, kf, vf, np.arange(S), 2048, 64, 128 ** -0.5),
                             [0], wl.H)
    print(json.dumps({"workload": wl.name, "attention_ms": round(ms, 4),
                      "attention_tflops_token_exact": round(fl_tok / ms / 1e9, 2), "visible_pairs_per_head": pairs,
                      "oracle_wall_s": wall, "oracle_wall_s_per_call_est": full,
                      "oracle_sample": "head 0, every row (window-slice form, float64), scaled to 24 heads"}),
          flush=True)

    # Wan shape variants: SPADE's static widths, top-p, the pooled statistic, padded (16, 2, 2),
    # spatial-only and temporal-only attention
    wl = synth.WORKLOADS[4]
    q, k, v = (synth.to_torch(x, dev) for x in synth.qkv(4))
    variants = [
        ("wan sink 5 + band 40", dict(tiles=[(1, 8, 8), (4, 4, 4)], sink_blocks=5, keep_diag=40)),
        ("wan top-p 0.9 (scores / sqrt(D))", dict(tiles=[(1, 8, 8), (4, 4, 4)], top_p=0.9, p_scale=wl.D ** -0.5)),
        ("wan pooled statistic", dict(tiles=[(1, 8, 8), (4, 4, 4)], statistic="pooled")),
        ("wan padded, candidates (1,8,8) (4,4,4) (16,2,2), gather on load",
         dict(tiles=[(1, 8, 8), (4, 4, 4), (16, 2, 2)], pad=True)),
        ("wan padded, candidates (1,8,8) (4,4,4) (16,2,2), permuted copies and label kernel",
         dict(tiles=[(1, 8, 8), (4, 4, 4), (16, 2, 2)], pad=True, fused=False)),
    ]
    out = torch.empty_like(q)
    for name, kw in variants:
        tiles = kw.pop("tiles")
        pipe = bsa.AdaptiveBlockSparse(1, wl.H, wl.grid, wl.D, tiles, 0.17, q.dtype, dev, **kw)
        ms_step = _time_steady(torch, lambda: pipe(q, k, v, out=out))
        kv_idx, kv_cnt = pipe.kv
        ms = _time_steady(torch, attention_call(bsa, pipe, q, k, v, out))
        kept = int(kv_cnt.sum().item())
        fl = kept * 4 * 64 * 64 * wl.D
        choice = np.bincount(pipe.choice.cpu().numpy().ravel(), minlength=len(tiles)).tolist()
        print(json.dumps({"workload": name, "attention_ms": round(ms, 4), "attention_tflops": round(fl / ms / 1e9, 2),
                          "step_ms": round(ms_step, 4), "step_tflops": round(fl / ms_step / 1e9, 2),
                          "kept_blocks": kept, "heads_per_candidate": choice}), flush=True)
    S, HW = wl.S, wl.grid[1] * wl.grid[2]
    for kind, pairs, direct in (("spatial", S * HW, True), ("temporal", S * wl.grid[0], True),
                                ("temporal", S * wl.grid[0], False)):
        att = bsa.VideoLabelAttention(1, wl.H, wl.grid, kind, dev, dtype=q.dtype if direct else None, D=wl.D)
        ms = _time_steady(torch, lambda: att(q, k, v, out=out))
        fl_tok = pairs * 4 * wl.D * wl.H
        how = ("label attention on T-major tokens" if kind == "spatial" else
               "frames gathered on load" if direct else "permute + label attention + inverse")
        print(json.dumps({"workload": f"wan {kind}-only attention ({how})",
                          "ms": round(ms, 4), "tflops_token_exact": round(fl_tok / ms / 1e9, 2),
                          "visible_pairs_per_head": pairs}), flush=True)

    # long sequence: grid 32x48x80 (S=122880), tiles 4x4x4, 10% budget, D=128, H=24
    wl = synth.WORKLOADS[5]
    qb, kb, vb = synth.qkv(5)
    q, k, v = (synth.to_torch(x, dev) for x in (qb, kb, vb))
    pipe = bsa.AdaptiveBlockSparse(1, wl.H, wl.grid, wl.D, [(4, 4, 4)], 0.10, q.dtype, dev)
    out = torch.empty_like(q)
    ms_step = _time_steady(torch, lambda: pipe(q, k, v, out=out))
    kv_idx, kv_cnt = pipe.kv
    ms = _time_steady(torch, attention_call(bsa, pipe, q, k, v, out))
    fl = int(kv_cnt.sum().item()) * 4 * 64 * 64 * wl.D
    # the oracle on head 0: permutation, scores and top-k of the head, then 32 query blocks spread over it
    qf, kf, vf = (synth.stored_to_f64(x[0, 0]) for x in (qb, kb, vb))
    nb = wl.S // 64
    t0 = time.perf_counter()
    perm = OT.tile_permutation(wl.grid, (4, 4, 4))
    qp, kp, vp = (OT.permute_tokens(x, perm) for x in (qf, kf, vf))
    keep = OB.topk_block_mask(OB.minmax_block_scores(qp, kp, 64), OB.budget(0.10, nb), 1, True)
    t_pre = time.perf_counter() - t0
    blocks = np.linspace(0, nb - 1, 32).astype(int)
    wall, full = oracle_wall(lambda I: OA.block_sparse_rows_gathered(qp, kp, vp, keep, 64, np.arange(64 * I, 64 * I + 64),
                                                                     wl.D ** -0.5), blocks, nb)
    print(json.dumps({"workload": wl.name, "attention_ms": round(ms, 4), "attention_tflops": round(fl / ms / 1e9, 2),
                      "step_ms": round(ms_step, 4), "step_tflops": round(fl / ms_step / 1e9, 2),
                      "kept_block_flops": fl, "oracle_wall_s": round(t_pre + wall, 3),
                      "oracle_wall_s_per_call_est": round((t_pre + full) * wl.H, 1),
                      "oracle_sample": (f"head 0: scores and top-k ({t_pre:.1f} s), then 32 of {nb} query blocks in "
                                        f"the gathered kept-block form; scaled to all blocks and 24 heads")}),
          flush=True)


def kernel_only(args, torch, bsa, synth):
    """The hot kernel of one workload alone, --warmup + --steps calls, one line of timing (for profilers)."""
    cfg = args.kernel_only
    wl = synth.WORKLOADS[cfg]
    dev = torch.device("cuda:0")
    log(f"generating inputs: {wl.name}")
    q, k, v = (synth.to_torch(x, dev) for x in synth.qkv(cfg))
    out = torch.empty_like(q)
    if cfg == 3:
        def call():
            bsa.bsa_windowed_attention(q, k, v, 2048, 64, 128 ** -0.5, 512, out=out)
        name = "attn_solo_kernel<window, positive scale>"
    else:
        tiles, frac = (TILES, FRAC) if cfg == 4 else ([(4, 4, 4)], 0.10)
        pipe = bsa.AdaptiveBlockSparse(1, wl.H, wl.grid, wl.D, tiles, frac, q.dtype, dev)
        pipe(q, k, v, out=out)
        call = attention_call(bsa, pipe, q, k, v, out)
        name = "attn_solo_kernel<block list, positive scale, gather on load, key-norm bound>"
    ms = _time(torch, call, max(args.steps, 1), args.warmup)
    print(json.dumps({"kernel_only": wl.name, "kernel": name, "calls": args.warmup + max(args.steps, 1),
                      "ms_per_call": round(ms, 4)}), flush=True)


def variant_pipeline(args, torch, bsa, synth):
    """One Wan-shape variant step, --warmup + --steps calls, one line of timing (for profilers): top-p 0.9
    (tiling choice, scores, top-p lists, launch plan, attention) or the padded candidates (1,8,8) (4,4,4)
    (16,2,2) (tiling choice, padded copies of q and k, masked scores, per-head top-k, launch plan, attention)."""
    wl = synth.WORKLOADS[4]
    dev = torch.device("cuda:0")
    log(f"generating inputs: {wl.name}")
    q, k, v = (synth.to_torch(x, dev) for x in synth.qkv(4))
    out = torch.empty_like(q)
    if args.top_p_pipeline:
        name = "top_p_pipeline"
        pipe = bsa.AdaptiveBlockSparse(1, wl.H, wl.grid, wl.D, TILES, FRAC, q.dtype, dev, top_p=0.9,
                                       p_scale=wl.D ** -0.5)
    else:
        name = "padded_pipeline"
        pipe = bsa.AdaptiveBlockSparse(1, wl.H, wl.grid, wl.D, TILES + [(16, 2, 2)], FRAC, q.dtype, dev, pad=True)
    ms = _time(torch, lambda: pipe(q, k, v, out=out), max(args.steps, 1), args.warmup)
    print(json.dumps({name: wl.name, "calls": args.warmup + max(args.steps, 1), "ms_per_step": round(ms, 4)}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the benchmark line, time the hot-path kernels on the other workloads "
                         "(sliding tile, windowed, long sequence) and print one JSON line per workload")
    ap.add_argument("--kernel-only", type=int, choices=(3, 4, 5), default=None,
                    help="only run the hot kernel of one workload (3: windowed attention; 4, 5: block-sparse attention "
                         "on the pipeline's lists) --warmup + --steps times, for profilers")
    ap.add_argument("--top-p-pipeline", action="store_true",
                    help="only run the Wan-shape top-p step (p = 0.9) --warmup + --steps times, for profilers")
    ap.add_argument("--padded-pipeline", action="store_true",
                    help="only run the Wan-shape padded step (candidates (1,8,8) (4,4,4) (16,2,2)) --warmup + "
                         "--steps times, for profilers")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (reference for HBM counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the path shards by heads with no communication, so a multi-GPU figure is the per-GPU "
              "figure at H/N heads and is not measured here.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_sparse_attention_permute_amd import bsa, synth

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30, "calls": 5}))
        return

    if args.sweep:
        sweep(args, torch, np, bsa, synth)
        return

    if args.kernel_only is not None:
        kernel_only(args, torch, bsa, synth)
        return
    if args.top_p_pipeline or args.padded_pipeline:
        variant_pipeline(args, torch, bsa, synth)
        return

    wl = synth.WORKLOADS[CFG]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"generating inputs: {wl.name}")
    q, k, v = synth.qkv(CFG)
    qg, kg, vg = (synth.to_torch(x, dev) for x in (q, k, v))
    pipe = bsa.AdaptiveBlockSparse(1, wl.H, wl.grid, wl.D, TILES, FRAC, qg.dtype, dev)
    out = torch.empty_like(qg)
    block = pipe.block

    ev = []

    def hook(start):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        ev.append(e)

    for _ in range(args.warmup):
        pipe(qg, kg, vg, out=out)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps); timing {args.steps} steps")

    kept_blocks = []
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        pipe(qg, kg, vg, out=out, attention_hook=hook)
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    attn_ms = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(args.steps)]
    attn_ms_avg = float(np.mean(attn_ms))
    kv_cnt = pipe.kv[1]
    kept = int(kv_cnt.sum().item())
    flops = kept * 4 * block * block * wl.D
    log(f"step {ms_step:.3f} ms, attention {attn_ms_avg:.3f} ms, kept blocks {kept}")

    # per-stage breakdown (separate, untimed pass)
    stages = {}
    marks = []

    def mark(name):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        marks.append((name, e))

    # the clock ramps up again over the first few calls after the syncs: the
    # median is taken over the last 5 of 12 passes
    for _ in range(12):
        marks.clear()
        mark("start")
        choice, _, _ = bsa.bsa_select_tiling(qg, wl.grid, TILES, workspace=pipe.ws_select, q_summaries=pipe.ws_qsumm)
        mark("select_tiling")
        scores, _ = bsa.bsa_minmax_block_scores_tiled(qg, kg, wl.grid, TILES, head_choice=choice, out=pipe.ws_scores,
                                                      key_norms=pipe.ws_knorm, q_summaries=pipe.ws_qsumm)
        mark("minmax_block_scores (gather on load)")
        kv_idx, kv_cnt2 = bsa.bsa_topk_block_mask(scores, pipe.k, 1, True, max_kept=pipe.max_kept,
                                                  out=pipe.ws_topk)[:2]
        mark("topk_block_mask")
        bsa.bsa_block_sparse_attention_tiled(qg, kg, vg, wl.grid, TILES, kv_idx, kv_cnt2, head_choice=choice, out=out,
                                             key_norms=pipe.ws_knorm)
        mark("block_sparse_attention (gather on load, T-major out)")
        torch.cuda.synchronize()
        for (_, a), (name, b) in zip(marks[:-1], marks[1:]):
            stages.setdefault(name, []).append(a.elapsed_time(b))
    stage_ms = {n: round(float(np.median(t[-5:])), 4) for n, t in stages.items()}

    # the same step with permuted copies (permute q, k, v -> scores -> top-k -> attention -> inverse)
    unfused = bsa.AdaptiveBlockSparse(1, wl.H, wl.grid, wl.D, TILES, FRAC, qg.dtype, dev, fused=False)
    ms_unfused = _time(torch, lambda: unfused(qg, kg, vg, out=out), max(args.steps // 2, 5), 3)
    same = bool(torch.equal(unfused(qg, kg, vg), pipe(qg, kg, vg)))
    del unfused

    # cold attention: a 512 MB write between calls evicts q, k, v from L2 and MALL
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    attn = attention_call(bsa, pipe, qg, kg, vg, out)
    cold = []
    for _ in range(max(5, min(args.steps, 20))):
        flush.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        attn()
        b.record()
        b.synchronize()
        cold.append(a.elapsed_time(b))
    cold_ms = float(np.median(cold))
    del flush

    achieved = flops / (attn_ms_avg * 1e-3) / 1e12
    result = {
        "metric": "block-sparse attn effective TFLOP/s + ms/call at Wan2.1 shape, % bf16 MFMA peak",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "adaptive-tiling block-sparse attention, Wan 2.1 latent shape",
            "B": 1, "H": wl.H, "grid": list(wl.grid), "S": wl.S, "D": wl.D, "block": block,
            "tiles": [list(t) for t in TILES], "tiles_dropped_not_dividing": [list(t) for t in DROPPED_TILES],
            "budget_frac": FRAC, "k": pipe.k, "sink_blocks": 1, "diagonal": True,
            "kept_blocks_per_step": kept, "kept_fraction": round(kept / (wl.H * pipe.nb * pipe.nb), 4),
            "fused": pipe.fused,
        },
        "unfused_step_ms": round(ms_unfused, 4),
        "fused_equals_unfused": same,
        "attention": {
            "ms_per_call": round(attn_ms_avg, 4),
            "tflops": round(achieved, 2),
            "frac_of_bf16_peak": round(achieved / PEAK_BF16_TFLOPS, 4),
            "kernel": "attn_solo_kernel<block list, positive scale, gather on load, key-norm bound>",
            "cold_ms_per_call": round(cold_ms, 4),
            "cold_tflops": round(flops / (cold_ms * 1e-3) / 1e12, 2),
        },
        "stage_ms": stage_ms,
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(),
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(q, k, v, wl, block, pipe.k)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
