#!/usr/bin/env python3
"""Benchmark of the TriAttention eviction pass on one MI355X.

One step = one whole pass (score -> aggregate/select -> in-place compaction)
over a synthetic cache resident in HBM.  Between steps the cache is restored
from a pristine device copy and the 256 MB Infinity Cache is flushed; neither
is timed.  Each stage is timed with HIP events recorded on the stream the
kernels are launched on.  Prints one JSON line.

Default workload: the full Qwen3-8B-shaped cache at 32K context (36 layers x
8 KV / 32 query heads, head_dim 128, q8_0 K / fp16 V, budget 25%, window 512).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_8b_full_32k_q8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=8,
                    help="layers of the workload the CPU oracle is timed on")
    ap.add_argument("--no-flush", action="store_true")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: every (layer, KV head) unit is independent, so a "
              "multi-GPU run is the same kernels on each GPU's share; --gpus %d is not supported"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from kv_cache_eviction_tria_amd import synth, tria

    wl = synth.WORKLOADS[args.workload]
    if wl.n_seq:
        print("paged workloads are benchmarked by bench_paged.py", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    n, B, S, W, G = wl.n, wl.budget, wl.sink, wl.window, wl.G
    print("# workload %s: generating on the device" % wl.name, file=sys.stderr, flush=True)
    stats = synth.gen_stats(wl.L, wl.Hq, wl.hd, wl.seed)
    k, v, pos = synth.gen_cache(wl.L, wl.Hkv, wl.hd, n, n, wl.k_type, wl.v_type, wl.seed, dev)
    k0, v0, p0 = k.clone(), v.clone(), pos.clone()
    ctx = tria.tria_load_stats(wl.L, wl.Hkv, wl.Hq, wl.hd, wl.k_type, wl.v_type, wl.theta,
                               list(wl.offsets), *stats)
    K = tria.tria_kept_count(n, B, S, W)
    raw = torch.empty(wl.L, wl.Hkv, n, G, dtype=torch.float32, device=dev)
    keep = torch.empty(wl.L, wl.Hkv, K, dtype=torch.int32, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def restore():
        k.copy_(k0)
        v.copy_(v0)
        pos.copy_(p0)
        if not args.no_flush:
            flush.fill_(1)

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

    def step():
        ev[0].record(stream)
        tria.tria_score(ctx, k, v, pos, n, raw, stream)
        ev[1].record(stream)
        tria.tria_select(ctx, raw, n, B, S, W, keep, None, stream)
        ev[2].record(stream)
        tria.tria_compact(ctx, k, v, pos, n, keep, K, stream)
        ev[3].record(stream)

    print("# warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        restore()
        step()
    torch.cuda.synchronize()

    # algorithmic bytes: read K once + read and write every moved K/V/pos row
    moved = int((keep != torch.arange(K, device=dev, dtype=torch.int32)).sum().item())
    kb, vb = synth.row_bytes(wl.k_type, wl.hd), synth.row_bytes(wl.v_type, wl.hd)
    score_bytes = wl.L * wl.Hkv * n * kb
    compact_bytes = moved * 2 * (kb + vb + 4)

    print("# timing %d steps" % args.steps, file=sys.stderr, flush=True)
    t_stage = np.zeros((args.steps, 3))
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    for i in range(args.steps):
        restore()
        step()
        ev[3].synchronize()
        t_stage[i] = [ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2]),
                      ev[2].elapsed_time(ev[3])]
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0

    pass_ms = t_stage.sum(axis=1)
    ms = float(np.median(pass_ms))
    stage_ms = t_stage.mean(axis=0)
    rows = wl.L * wl.Hkv * n
    names = ["score", "select", "compact"]
    dom = int(np.argmax(stage_ms))
    alg = {"score": score_bytes, "select": None, "compact": compact_bytes}
    dom_bytes = alg[names[dom]]
    achieved = dom_bytes / (stage_ms[dom] * 1e-3) / 1e9 if dom_bytes else None
    pass_bytes = score_bytes + compact_bytes

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_layers)

    out = {
        "metric": "KV tokens scored+compacted/sec and eviction-pass ms at 32K ctx; % of HBM peak",
        "value": rows / (ms * 1e-3),
        "unit": "KV rows/s (layer x KV-head x token, scored + compacted)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "q8_0/f16 in, f32 accumulate" if wl.k_type == synth.KV_Q8_0 else "f16 in, f32 accumulate",
        "data": "synthetic (seeded N(0,1) K/V with lognormal channel scales; lognormal/uniform-phase stats)",
        "config": {"workload": wl.name, "layers": wl.L, "kv_heads": wl.Hkv, "q_heads": wl.Hq,
                   "head_dim": wl.hd, "tokens": n, "budget": B, "sink": S, "window": W,
                   "kept": K, "k_type": "q8_0" if wl.k_type else "f16",
                   "v_type": "q8_0" if wl.v_type else "f16", "parallelism": "single GPU"},
        "pass_ms_p10_p90": [float(np.percentile(pass_ms, 10)), float(np.percentile(pass_ms, 90))],
        "stage_ms": {nm: float(x) for nm, x in zip(names, stage_ms)},
        "tokens_per_s": n / (ms * 1e-3),
        "pass_alg_bytes": pass_bytes,
        "pass_alg_GBs": pass_bytes / (ms * 1e-3) / 1e9,
        "pass_frac_hbm": pass_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "moved_rows": moved,
        "wall_s_timed_loop_incl_restore": t_wall,
        "roofline": {"kernel": names[dom], "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": (achieved / HBM_PEAK_GBS) if achieved else None,
                     "traffic": None, "alg_bytes_per_launch": dom_bytes,
                     "avg_launch_ms": float(stage_ms[dom])},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    ctx.close()


def cpu_baseline(wl, layers):
    """The CPU oracle on a bounded sample of the same workload (its first `layers` layers)."""
    import oracle
    from kv_cache_eviction_tria_amd import synth
    layers = max(1, min(layers, wl.L))
    print("# cpu baseline: oracle on %d of %d layers" % (layers, wl.L), file=sys.stderr, flush=True)
    case = synth.make_case(wl, device="cpu", L=layers)
    k, v, pos = case["k"].numpy().copy(), case["v"].numpy().copy(), case["pos"].numpy().copy()
    t = time.perf_counter()
    oracle.evict(wl.k_type, wl.v_type, layers, wl.Hkv, wl.Hq, wl.hd, wl.theta, list(wl.offsets),
                 k, v, pos, wl.n, wl.budget, wl.sink, wl.window, case["q_re"], case["q_im"],
                 case["w"], want_raw=False, want_agg=False)
    dt = time.perf_counter() - t
    rows = layers * wl.Hkv * wl.n
    return {"value": rows / dt, "unit": "KV rows/s (layer x KV-head x token, scored + compacted)",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%d of %d layers (%d units x %d tokens), %.2f s" % (
                layers, wl.L, layers * wl.Hkv, wl.n, dt)}


if __name__ == "__main__":
    main()
