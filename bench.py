#!/usr/bin/env python3
"""Benchmark of the TriAttention eviction pass on one MI355X.

One step = one call of tria_evict (score -> aggregate/select -> in-place
compaction of every layer and KV head) over a synthetic cache resident in
HBM, timed with HIP events recorded on the caller's stream around the call
(every kernel of the pass runs on that stream).  Between steps the cache is restored from a pristine device copy and the
256 MB Infinity Cache is flushed by reading 512 MB of another buffer; neither
is timed.  The read leaves the Infinity Cache holding clean lines of that
buffer, as after decode steps that only read the cache.  (Writing the 512 MB
instead, `--flush write`, leaves them dirty, and the first timed kernel then
writes them back to HBM: a cost of the flush, not of the pass.)

Per-kernel durations come from the library's own timing events (recorded on
the stream each kernel runs on) over as many steps again, run after the timed
ones: events between the kernels of a pass lengthen it, so the timed steps
run without them (the pass time with them is reported beside); the kernel with
the largest total time is reported against the HBM roofline with its
algorithmic bytes:  score = every cached K row read once; compaction = every
moved row (keep_idx[d] != d) read and written (K + V + pos).  A sequential
breakdown (the three stages one after another) is reported beside it, and,
after the steps, a plain device-to-device copy of 1 GiB (`copy_reference`):
the bandwidth a kernel that reads and writes every byte once reaches on the
same GPU in the same run.

Default workload: the full Qwen3-8B-shaped cache at 32K context (36 layers x
8 KV / 32 query heads, head_dim 128, q8_0 K / fp16 V, budget 25%, window 512).
The paged workload (16 sequences of 8K..64K tokens in shuffled 16-row blocks)
runs one initial pass, then rounds of "append 128 rows to every sequence,
evict back to its budget"; a step is one such batched round.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "KV tokens scored+compacted/sec and eviction-pass ms at 32K ctx; % of HBM peak"
UNIT = "KV rows/s (layer x KV-head x token, scored + compacted)"
def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_8b_full_32k_q8")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU work the oracle baseline aims for (whole passes, at least one)")
    ap.add_argument("--staged-steps", type=int, default=5)
    ap.add_argument("--seq-rounds", type=int, default=-1,
                    help="paged workload: rounds of per-sequence passes after the batched "
                         "rounds (default: as many as --steps; 0: none)")
    ap.add_argument("--flush", choices=("read", "write", "none"), default="read",
                    help="between steps, read (default) or write 512 MB to evict the Infinity "
                         "Cache, or leave it as the restore left it")
    ap.add_argument("--copy-reference-bytes", type=int, default=1 << 30,
                    help="after the timed steps, time a plain device-to-device copy of this "
                         "many bytes as the reference a data-moving kernel can reach (0: skip)")
    ap.add_argument("--calibrate-bytes", type=int, default=0,
                    help="run one plain streaming kernel (uint8 xor) over this many bytes before "
                         "the timed steps, as the byte reference for profiler counters")
    ap.add_argument("--keep-mode", choices=sorted(KEEP_MODES), default="per_unit",
                    help="tria_set_keep_mode: who shares a keep set")
    ap.add_argument("--compaction", choices=sorted(COMPACTIONS), default="ordered",
                    help="tria_set_compaction: order-preserving gather or hole filling")
    ap.add_argument("--decode", action="store_true",
                    help="decode loop on a contiguous workload: per step one appended row per "
                         "unit and attention over the cache, with the threshold policy's passes "
                         "(budget = the workload's, divide length 128) vs without eviction")
    return ap.parse_args()


# --keep-mode -> (library mode, oracle mode)
KEEP_MODES = {"per_unit": (0, 0), "per_kv_head": (1, 1), "global": (2, 2)}
# --compaction -> (library mode, oracle mode, profile key of its kernels)
COMPACTIONS = {"ordered": (0, 0, "compact"), "hole_fill": (1, 1, "holefill")}


def measured_traffic(stage, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel sources; None otherwise."""
    from kv_cache_eviction_tria_amd.profile_summary import sources_digest
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.txt" % (stage, workload))
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("sources_sha256_16") != sources_digest(stage):
        return None
    return float(t["bytes_per_launch"])


def traffic_key_fn(args):
    """Profile key of each stage's kernels under the chosen compaction."""
    return lambda stage: COMPACTIONS[args.compaction][2] if stage == "compact" else stage


def roofline(stage, ms_total, launches, alg_bytes_total, workload, traffic_key=None):
    """Roofline entry for one stage from its summed launch durations (traffic_key: the
    profile the stage's counters are stored under, the stage's own name by default)."""
    avg_ms = ms_total / max(launches, 1)
    per_launch = alg_bytes_total / max(launches, 1) if alg_bytes_total else None
    achieved = per_launch / (avg_ms * 1e-3) / 1e9 if per_launch else None
    return {"kernel": stage, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": (achieved / HBM_PEAK_GBS) if achieved else None,
            "traffic": measured_traffic(traffic_key or stage, workload),
            "alg_bytes_per_launch": per_launch,
            "launches_per_step": launches, "avg_launch_ms": avg_ms}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: every (layer, KV head) unit is independent, so a "
              "multi-GPU run is the same kernels on each GPU's share; --gpus %d is not supported"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    from kv_cache_eviction_tria_amd import synth
    if args.calibrate_bytes > 0:
        calibrate(args.calibrate_bytes)
    if args.workload in synth.CALIB_WORKLOADS:
        out = bench_calib(args, args.workload)
    elif args.decode:
        out = bench_decode(args, synth.WORKLOADS[args.workload])
    else:
        wl = synth.WORKLOADS[args.workload]
        out = bench_paged(args, wl) if wl.n_seq else bench_contiguous(args, wl)
    print(json.dumps(out), flush=True)


def calibrate(nbytes):
    """One streaming kernel that reads and writes exactly nbytes (untimed)."""
    import torch
    src = torch.full((nbytes,), 7, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.bitwise_xor(src, 0x5A, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def log(msg):
    print("# " + msg, file=sys.stderr, flush=True)


def copy_reference(nbytes, reps=10):
    """A plain device-to-device copy (torch's copy_ of one uint8 buffer into another)
    of nbytes, median of reps, untimed relative to the pass: the bandwidth a kernel
    that reads and writes every byte once reaches on this GPU, counted like the
    pass's algorithmic bytes (bytes read + bytes written)."""
    if nbytes <= 0:
        return None
    import numpy as np
    import torch
    src = torch.full((nbytes,), 3, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for i in range(reps + 2):
        torch.cuda.synchronize()
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        if i >= 2:
            ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    del src, dst
    torch.cuda.empty_cache()
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    return {"what": "torch copy_ of one device buffer into another", "bytes": nbytes, "ms": ms,
            "GB_s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS}


def dtype_of(wl):
    """The number formats the pass computes in."""
    from kv_cache_eviction_tria_amd import synth
    v = "q8_0" if wl.v_type == synth.KV_Q8_0 else "f16"
    if wl.k_type == synth.KV_Q8_0 and wl.hd % 128 == 0:
        k = ("q8_0 K: trig term int8 values (exact in fp16) x fp16 hi/lo coefficients on MFMA "
             "(fp32 accumulate)")
    elif wl.k_type == synth.KV_Q8_0:
        k = ("q8_0 K: trig term int8 x 32-bit coefficient digits on MFMA (i32 accumulate, "
             "fp32 combine)")
    else:
        k = ("f16 K: trig and norm sums on f16 MFMA with hi/lo fp16 coefficient splits "
             "(fp32 accumulate)")
    return "%s; norm term |K_f| in fp32; z-norm statistics fp64; %s V moved as bytes" % (k, v)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def bench_contiguous(args, wl):
    tkey = traffic_key_fn(args)
    import numpy as np
    import torch

    from kv_cache_eviction_tria_amd import synth, tria

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    n, B, S, W, G = wl.n, wl.budget, wl.sink, wl.window, wl.G
    log("workload %s: generating on the device" % wl.name)
    stats = synth.gen_stats(wl.L, wl.Hq, wl.hd, wl.seed)
    k, v, pos = synth.gen_cache(wl.L, wl.Hkv, wl.hd, n, n, wl.k_type, wl.v_type, wl.seed, dev)
    k0, v0, p0 = k.clone(), v.clone(), pos.clone()
    ctx = tria.tria_load_stats(wl.L, wl.Hkv, wl.Hq, wl.hd, wl.k_type, wl.v_type, wl.theta,
                               list(wl.offsets), *stats)
    tria.tria_set_keep_mode(ctx, KEEP_MODES[args.keep_mode][0])
    tria.tria_set_compaction(ctx, COMPACTIONS[args.compaction][0])
    K = tria.tria_kept_count(n, B, S, W)
    flush = torch.ones(64 << 20, dtype=torch.int64, device=dev)  # 512 MB

    def restore():
        k.copy_(k0)
        v.copy_(v0)
        pos.copy_(p0)
        if args.flush == "read":
            flush.sum()
        elif args.flush == "write":
            flush.fill_(1)

    # the kept rows of this input, for the algorithmic byte count (untimed)
    raw = torch.empty(wl.L, wl.Hkv, n, G, dtype=torch.float32, device=dev)
    keep = torch.empty(wl.L, wl.Hkv, K, dtype=torch.int32, device=dev)
    tria.tria_score(ctx, k, v, pos, n, raw, stream)
    tria.tria_select(ctx, raw, n, B, S, W, keep, None, stream)
    moved = int((keep != torch.arange(K, device=dev, dtype=torch.int32)).sum().item())
    kb, vb = synth.row_bytes(wl.k_type, wl.hd), synth.row_bytes(wl.v_type, wl.hd)
    alg = {"score": wl.L * wl.Hkv * n * kb, "select": 0, "compact": moved * 2 * (kb + vb + 4)}
    pass_bytes = alg["score"] + alg["compact"]

    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        restore()
        tria.tria_evict(ctx, k, v, pos, n, B, S, W, stream)
    torch.cuda.synchronize()

    log("timing %d steps" % args.steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_pass = np.zeros(args.steps)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    for i in range(args.steps):
        restore()
        e0.record(stream)
        kept = tria.tria_evict(ctx, k, v, pos, n, B, S, W, stream)
        e1.record(stream)
        e1.synchronize()
        t_pass[i] = e0.elapsed_time(e1)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    assert kept == K

    # Per-kernel durations from the library's own events, over the same number
    # of steps run again: recorded between the kernels of a pass, those events
    # lengthen it (by about 20 us on the 36-layer cache), so the steps above,
    # which give the pass time, run without them.
    log("per-kernel events over %d more steps" % args.steps)
    st_ms = {s: 0.0 for s in tria.STAGES}
    st_n = {s: 0 for s in tria.STAGES}
    untimed = 0
    tria.tria_timing_enable(ctx, True)
    t_inst = np.zeros(args.steps)
    for i in range(args.steps):
        restore()
        e0.record(stream)
        tria.tria_evict(ctx, k, v, pos, n, B, S, W, stream)
        e1.record(stream)
        e1.synchronize()
        t_inst[i] = e0.elapsed_time(e1)
        ms_i, n_i, u = tria.tria_timing_read(ctx)
        for s in tria.STAGES:
            st_ms[s] += ms_i[s]
            st_n[s] += n_i[s]
        untimed += u
    torch.cuda.synchronize()
    tria.tria_timing_enable(ctx, False)
    tria.tria_device_status(ctx)  # raises if a compaction gave up a wait

    # the same pass as three sequential calls (kernels isolated from each other)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    t_seq = np.zeros((max(args.staged_steps, 0), 3))
    for i in range(args.staged_steps):
        restore()
        ev[0].record(stream)
        tria.tria_score(ctx, k, v, pos, n, raw, stream)
        ev[1].record(stream)
        tria.tria_select(ctx, raw, n, B, S, W, keep, None, stream)
        ev[2].record(stream)
        tria.tria_compact(ctx, k, v, pos, n, keep, K, stream)
        ev[3].record(stream)
        ev[3].synchronize()
        t_seq[i] = [ev[j].elapsed_time(ev[j + 1]) for j in range(3)]
    torch.cuda.synchronize()

    ms = float(np.median(t_pass))
    steps = args.steps
    per_step_ms = {s: st_ms[s] / steps for s in tria.STAGES}
    per_step_n = {s: st_n[s] // steps for s in tria.STAGES}
    dom = max(tria.STAGES, key=lambda s: per_step_ms[s])
    rows = wl.L * wl.Hkv * n
    seq_ms = {s: float(np.median(t_seq[:, j])) for j, s in enumerate(tria.STAGES)} \
        if args.staged_steps > 0 else None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, stats, k0.cpu().numpy(), v0.cpu().numpy(), p0.cpu().numpy(),
                           args.cpu_seconds, KEEP_MODES[args.keep_mode][1],
                           COMPACTIONS[args.compaction][1])

    out = {
        "metric": METRIC,
        "value": rows / (ms * 1e-3),
        "unit": UNIT,
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_of(wl),
        "data": "synthetic (seeded N(0,1) K/V with lognormal channel scales; "
                "lognormal/uniform-phase statistics)",
        "config": {"workload": wl.name, "layers": wl.L, "kv_heads": wl.Hkv, "q_heads": wl.Hq,
                   "head_dim": wl.hd, "tokens": n, "budget": B, "sink": S, "window": W,
                   "kept": K, "k_type": "q8_0" if wl.k_type else "f16",
                   "v_type": "q8_0" if wl.v_type else "f16", "parallelism": "single GPU",
                   "keep_mode": args.keep_mode,
                   "compaction": args.compaction},
        "pass_ms_p10_p90": [float(np.percentile(t_pass, 10)), float(np.percentile(t_pass, 90))],
        "tokens_per_s": n / (ms * 1e-3),
        "pass_alg_bytes": pass_bytes,
        "pass_alg_GBs": pass_bytes / (ms * 1e-3) / 1e9,
        "pass_frac_hbm": pass_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "moved_rows": moved,
        "kernel_ms_per_step": per_step_ms,
        "launches_per_step": per_step_n,
        "untimed_launches": untimed,
        "sequential_stage_ms": seq_ms,
        "sequential_pass_ms": float(sum(seq_ms.values())) if seq_ms else None,
        "wall_s_timed_loop_incl_restore": t_wall,
        "pass_ms_with_kernel_events": float(np.median(t_inst)),
        "cache_flush_between_steps": args.flush,
        "roofline": roofline(dom, per_step_ms[dom], per_step_n[dom], alg[dom], wl.name,
                             tkey(dom)),
        "roofline_all": {s: roofline(s, per_step_ms[s], per_step_n[s], alg[s], wl.name, tkey(s))
                         for s in tria.STAGES},
        "cpu_baseline": cpu,
    }
    ctx.close()
    out["copy_reference"] = copy_reference(args.copy_reference_bytes)
    return out


def bench_paged(args, wl):
    tkey = traffic_key_fn(args)
    import numpy as np
    import torch

    from kv_cache_eviction_tria_amd import synth, tria

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    lens = synth.paged_lengths(wl)
    budgets = [int(wl.budget_frac * x) for x in lens]
    m = wl.append
    log("workload %s: %d sequences, %d..%d tokens; generating on the device" % (
        wl.name, wl.n_seq, min(lens), max(lens)))
    stats = synth.gen_stats(wl.L, wl.Hq, wl.hd, wl.seed)
    pg = synth.gen_paged(wl.L, wl.Hkv, wl.hd, wl.k_type, wl.v_type, lens, wl.seed, dev)
    ctx = tria.tria_load_stats(wl.L, wl.Hkv, wl.Hq, wl.hd, wl.k_type, wl.v_type, wl.theta,
                               list(wl.offsets), *stats)
    tria.tria_set_keep_mode(ctx, KEEP_MODES[args.keep_mode][0])
    tria.tria_set_compaction(ctx, COMPACTIONS[args.compaction][0])
    pools = [pg[x] for x in ("k_pool", "v_pool", "pos_pool", "block_table")]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    log("initial pass")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    kept = tria.tria_evict_paged_batch(ctx, *pools, lens, budgets, wl.sink, wl.window, stream)
    torch.cuda.synchronize()
    first_ms = (time.perf_counter() - t0) * 1e3
    assert kept == budgets, (kept, budgets)
    n_now = list(budgets)

    def append(r):
        for s in range(wl.n_seq):
            row = synth.paged_rows(pg["pos_pool"][:1, :, :1], pg["block_table"][s], n_now[s])
            last = int(row[0, 0, n_now[s] - 1])
            synth.append_paged(pg, s, n_now[s], m, last + 1, wl.L, wl.Hkv, wl.hd, wl.k_type,
                               wl.v_type, wl.seed * 100003 + r * 64 + s)
            n_now[s] += m

    st_ms = {s: 0.0 for s in tria.STAGES}
    st_n = {s: 0 for s in tria.STAGES}
    t_round = []
    t_event = []
    total = args.warmup + args.steps
    log("rounds: %d warmup + %d timed" % (args.warmup, args.steps))
    def kept_positions():
        # positions of every sequence's first B rows (all units); positions are unique
        # within a unit, so row d moved in a pass iff its position changed
        return [synth.paged_rows(pg["pos_pool"], pg["block_table"][s], budgets[s]).clone()
                for s in range(wl.n_seq)]

    moved_total = 0
    for r in range(total):
        append(r)
        torch.cuda.synchronize()
        before = kept_positions() if r >= args.warmup else None
        if r == args.warmup:
            tria.tria_timing_enable(ctx, True)
        # A round is timed on the host, idle device to idle device (it includes
        # the enqueue, ~0.2 ms): events recorded around this call on an idle
        # stream were found to read up to 2x the host-observed time of the same
        # round, so they are only reported alongside.
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        kept = tria.tria_evict_paged_batch(ctx, *pools, n_now, budgets, wl.sink, wl.window,
                                           stream)
        e1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        if r >= args.warmup:
            t_round.append((t1 - t0) * 1e3)
            t_event.append(e0.elapsed_time(e1))
            ms_i, n_i, _ = tria.tria_timing_read(ctx)
            for s in tria.STAGES:
                st_ms[s] += ms_i[s]
                st_n[s] += n_i[s]
        assert kept == budgets
        n_now = list(kept)
        if before is not None:
            after = kept_positions()
            moved_total += sum(int((a != b_).sum().item()) for a, b_ in zip(after, before))
    tria.tria_timing_enable(ctx, False)
    tria.tria_device_status(ctx)  # raises if a compaction gave up a wait

    # Per-sequence passes: after its 128 appends each sequence is evicted on its own (a
    # one-sequence batch), as a loop serving the sequences one at a time would; the
    # steady-state pass latency per sequence, timed like the rounds.
    seq_rounds = args.steps if args.seq_rounds < 0 else args.seq_rounds
    log("per-sequence rounds: %d" % seq_rounds)
    t_seq = [[] for _ in range(wl.n_seq)]
    for r in range(seq_rounds):
        append(total + r)
        for s in range(wl.n_seq):
            bt_s = pg["block_table"][s:s + 1]
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            k_s = tria.tria_evict_paged_batch(ctx, pg["k_pool"], pg["v_pool"], pg["pos_pool"],
                                              bt_s, [n_now[s]], [budgets[s]], wl.sink,
                                              wl.window, stream)
            torch.cuda.synchronize()
            t_seq[s].append((time.perf_counter() - t0) * 1e3)
            assert k_s == [budgets[s]]
            n_now[s] = budgets[s]
    tria.tria_device_status(ctx)
    seq_all = [t for ts in t_seq for t in ts] or [float("nan")]
    seq_rows = [wl.L * wl.Hkv * (b + m) for b in budgets]

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_paged(wl, stats, pg, n_now, budgets, m, args.cpu_seconds,
                                 KEEP_MODES[args.keep_mode][1], COMPACTIONS[args.compaction][1],
                                 total + seq_rounds)

    ms = float(np.median(t_round))
    rows = sum(wl.L * wl.Hkv * (b + m) for b in budgets)
    per_step_ms = {s: st_ms[s] / args.steps for s in tria.STAGES}
    per_step_n = {s: st_n[s] // args.steps for s in tria.STAGES}
    dom = max(tria.STAGES, key=lambda s: per_step_ms[s])
    kb, vb = synth.row_bytes(wl.k_type, wl.hd), synth.row_bytes(wl.v_type, wl.hd)
    moved = moved_total / args.steps
    alg = {"score": rows * kb, "select": 0, "compact": moved * 2 * (kb + vb + 4)}
    out = {
        "metric": METRIC,
        "value": rows / (ms * 1e-3),
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_of(wl),
        "data": "synthetic (seeded N(0,1) K/V with lognormal channel scales; "
                "lognormal/uniform-phase statistics; shuffled block order)",
        "config": {"workload": wl.name, "sequences": wl.n_seq, "lengths": lens,
                   "budgets": budgets, "append": m, "sink": wl.sink, "window": wl.window,
                   "layers": wl.L, "kv_heads": wl.Hkv, "q_heads": wl.Hq, "head_dim": wl.hd,
                   "parallelism": "single GPU", "keep_mode": args.keep_mode,
                   "compaction": args.compaction},
        "round_ms_p10_p90": [float(np.percentile(t_round, 10)), float(np.percentile(t_round, 90))],
        "round_timing": "host clock, synchronised device on both sides, enqueue included",
        "round_ms_events_median": float(np.median(t_event)),
        "initial_pass_ms": first_ms,
        "initial_pass_rows_per_s": sum(wl.L * wl.Hkv * x for x in lens) / (first_ms * 1e-3),
        "kernel_ms_per_step": per_step_ms,
        "launches_per_step": per_step_n,
        "moved_rows_per_round": moved,
        "round_alg_bytes": alg["score"] + alg["compact"],
        "round_frac_hbm": (alg["score"] + alg["compact"]) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline": roofline(dom, per_step_ms[dom], per_step_n[dom], alg[dom], wl.name,
                             tkey(dom)),
        "roofline_all": {s: roofline(s, per_step_ms[s], per_step_n[s], alg[s], wl.name, tkey(s))
                         for s in tria.STAGES},
        "seq_pass_ms_median": float(np.median(seq_all)),
        "seq_pass_ms_p10_p90": [float(np.percentile(seq_all, 10)),
                                float(np.percentile(seq_all, 90))],
        "seq_pass_ms_by_sequence": [float(np.median(ts)) if ts else None for ts in t_seq],
        "seq_pass_rows_per_s": float(np.median([r_ / (np.median(ts) * 1e-3)
                                                for r_, ts in zip(seq_rows, t_seq)]))
        if seq_rounds else None,
        "seq_pass_timing": "each sequence's own pass (n = budget + 128 -> budget), "
                           "%d rounds after the batched ones; host clock, device synchronised "
                           "on both sides, enqueue included" % seq_rounds,
        "cpu_baseline": cpu,
    }
    ctx.close()
    out["copy_reference"] = copy_reference(args.copy_reference_bytes)
    return out


def cpu_baseline_paged(wl, stats, pg, n_now, budgets, m, seconds, keep_mode, compact_mode,
                       round0):
    """The oracle on sequence passes of the same steady state: sequence by sequence, 128
    rows are appended on the device, the logical rows (n = budget + 128) are copied to
    the host and the oracle runs the whole pass on them; until about `seconds`."""
    import numpy as np

    import oracle
    from kv_cache_eviction_tria_amd import synth
    log("cpu baseline: oracle on sequence passes, about %.0f s" % seconds)
    times, stages, rows, done = [], [], 0, []
    for s in range(wl.n_seq):
        if times and sum(times) >= seconds:
            break
        n = n_now[s]
        row = synth.paged_rows(pg["pos_pool"][:1, :, :1], pg["block_table"][s], n)
        synth.append_paged(pg, s, n, m, int(row[0, 0, n - 1]) + 1, wl.L, wl.Hkv, wl.hd,
                           wl.k_type, wl.v_type, wl.seed * 100003 + round0 * 64 + s)
        n += m
        host = [np.ascontiguousarray(synth.paged_rows(pg[x], pg["block_table"][s], n).cpu()
                                     .numpy()) for x in ("k_pool", "v_pool", "pos_pool")]
        t = time.perf_counter()
        oracle.evict(wl.k_type, wl.v_type, wl.L, wl.Hkv, wl.Hq, wl.hd, wl.theta,
                     list(wl.offsets), *host, n, budgets[s], wl.sink, wl.window, *stats,
                     want_raw=False, want_agg=False, keep_mode=keep_mode,
                     compact_mode=compact_mode)
        times.append(time.perf_counter() - t)
        stages.append(oracle.last_stage_seconds())
        rows += wl.L * wl.Hkv * n
        done.append(s)
    st = np.median(np.array(stages), axis=0) * 1e3
    return {"value": rows / sum(times), "unit": UNIT, "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "seq_pass_ms_median": float(np.median(times)) * 1e3,
            "stage_ms_median": {"score_and_aggregate": float(st[0]), "select": float(st[1]),
                                "compact": float(st[2])},
            "sample": "%d sequence passes (sequences %s, n = budget + %d each), %.1f s of CPU "
                      "time" % (len(times), done, m, sum(times))}


def bench_decode(args, wl):
    """Decode loop: each step appends one fresh row to every (layer, KV head) unit and
    computes one decode step's attention over the cache.  'tria': tria_decode_step with
    a threshold policy (budget = the workload's kept count, divide length 128, nothing
    protected beyond sink/window) before the attention; 'dense': no eviction.  Timed per
    step with events around tria_decode_step + tria_decode_attention (the appends, the
    model's own KV writes, are not timed)."""
    import numpy as np
    import torch

    from kv_cache_eviction_tria_amd import synth, tria

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    n0, steps, warm = wl.n, max(args.steps, 1) * 32, max(args.warmup, 1) * 32
    cap = n0 + steps + warm + 1
    log("decode loop %s: %d rows, %d warm-up + %d timed steps" % (wl.name, n0, warm, steps))
    stats = synth.gen_stats(wl.L, wl.Hq, wl.hd, wl.seed)
    k0, v0, p0 = synth.gen_cache(wl.L, wl.Hkv, wl.hd, cap, n0, wl.k_type, wl.v_type, wl.seed, dev)
    fresh = synth.gen_cache(wl.L, wl.Hkv, wl.hd, 256, 256, wl.k_type, wl.v_type, wl.seed + 99, dev)
    q = torch.randn(wl.L, wl.Hq, wl.hd, dtype=torch.float32, device=dev,
                    generator=torch.Generator(device=dev).manual_seed(5))
    res = {}
    for mode in ("dense", "tria"):
        k, v, pos = k0.clone(), v0.clone(), p0.clone()
        ctx = tria.tria_load_stats(wl.L, wl.Hkv, wl.Hq, wl.hd, wl.k_type, wl.v_type, wl.theta,
                                   list(wl.offsets), *stats)
        tria.tria_set_compaction(ctx, COMPACTIONS[args.compaction][0])
        pol = tria.Policy(trigger=tria.TRIA_TRIGGER_THRESHOLD, protect_prefill=0,
                          budget=wl.budget, divide_length=128, interval=1, sink=wl.sink,
                          window=wl.window)
        st = tria.DecodeState(n_rows=n0, n_prompt=0, steps=0, passes=0)
        out = torch.empty_like(q)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts, rows = [], []
        for t in range(warm + steps):
            n = st.n_rows
            j = t % 256
            k[:, :, n] = fresh[0][:, :, j]
            v[:, :, n] = fresh[1][:, :, j]
            pos[:, :, n] = n0 + t
            st.n_rows += 1
            e0.record(stream)
            if mode == "tria":
                tria.tria_decode_step(ctx, k, v, pos, pol, st, stream)
            tria.tria_decode_attention(ctx, k, v, pos, st.n_rows, q, out=out, stream=stream)
            e1.record(stream)
            if t >= warm:
                e1.synchronize()
                ts.append(e0.elapsed_time(e1))
                rows.append(st.n_rows)
        torch.cuda.synchronize()
        tria.tria_device_status(ctx)
        res[mode] = {"ms_per_step": float(np.mean(ts)), "ms_median": float(np.median(ts)),
                     "mean_rows": float(np.mean(rows)), "passes": int(st.passes)}
        ctx.close()
    kb, vb = synth.row_bytes(wl.k_type, wl.hd), synth.row_bytes(wl.v_type, wl.hd)
    units = wl.L * wl.Hkv
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline: oracle decode attention over whole units of the dense cache")
        G, spent, nu = wl.Hq // wl.Hkv, 0.0, 0
        scale = 1.0 / float(wl.hd) ** 0.5
        while nu < units and (nu == 0 or spent < min(args.cpu_seconds, 10.0)):
            l, g = divmod(nu, wl.Hkv)
            kr, vr = k0[l, g, :n0].cpu().numpy(), v0[l, g, :n0].cpu().numpy()
            qq = q[l, g * G:(g + 1) * G].double().cpu().numpy()
            t0 = time.perf_counter()
            oracle.decode_attention_unit(wl.k_type, wl.v_type, kr, vr, wl.hd, qq, scale)
            spent += time.perf_counter() - t0
            nu += 1
        cpu = {"value": nu / (spent * units), "unit": "decode steps/s (dense attention, all layers)",
               "cores": 1, "kind": "oracle", "cpu_model": cpu_model(),
               "sample": "attention of %d of %d (layer, KV head) units over %d rows each, "
                         "%.1f s; compare with dense.steps_per_s" % (nu, units, n0, spent)}
    res["dense"]["steps_per_s"] = 1e3 / res["dense"]["ms_median"]
    dense_bytes = res["dense"]["mean_rows"] * units * (kb + vb)
    d_ms, t_ms = res["dense"]["ms_median"], res["tria"]["ms_per_step"]
    achieved = dense_bytes / (d_ms * 1e-3) / 1e9
    return {
        "metric": "decode steps/s (attention over the cache + eviction passes, all layers)",
        "value": 1e3 / t_ms,
        "unit": "decode steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": t_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_of(wl),
        "data": "synthetic (seeded N(0,1) K/V with lognormal channel scales)",
        "config": {"workload": wl.name, "layers": wl.L, "kv_heads": wl.Hkv, "q_heads": wl.Hq,
                   "head_dim": wl.hd, "start_rows": n0, "budget": wl.budget,
                   "divide_length": 128, "compaction": args.compaction,
                   "parallelism": "single GPU"},
        "dense": res["dense"],
        "tria": res["tria"],
        "speedup_vs_dense": d_ms / t_ms if t_ms > 0 else None,
        "roofline": {"kernel": "decode_attention (dense)", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None, "alg_bytes_per_launch": dense_bytes,
                     "launches_per_step": 1, "avg_launch_ms": d_ms},
        "cpu_baseline": cpu,
    }


def bench_calib(args, name):
    """Calibration statistics: one step = every layer's query rows of one sample added
    and the statistics finished.  The line times one tria_calib_add_layers call over
    all layers (the sample's queries held as one [L, T, Hq*hd] tensor); the same
    step as one tria_calib_add per layer, as a model's forward hands the layers
    over one at a time, is reported beside it."""
    import numpy as np
    import torch

    from kv_cache_eviction_tria_amd import synth, tria

    L, Hq, hd, T, dtype = synth.CALIB_WORKLOADS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    log("calibration stream %s: generating on the device" % name)
    qs = synth.gen_query_stream(L, Hq, hd, T, dtype, 7, dev)
    cal = tria.TriaCalib(L, Hq, hd)

    def step():
        for l in range(L):
            cal.add(l, qs[l], stream)
        return cal.finish(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(args.steps):
        torch.cuda._sleep(1_000_000)  # the start event follows real work (see bench_paged)
        e0.record(stream)
        step()
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    alg = T * L * Hq * hd * torch.tensor([], dtype=dtype).element_size()
    # the same rows added in one call for all layers (tria_calib_add_layers)
    q_all = torch.stack(qs)
    cal_b = tria.TriaCalib(L, Hq, hd)

    def step_batched():
        cal_b.add_layers(0, q_all, stream)
        return cal_b.finish(stream)

    for _ in range(args.warmup):
        step_batched()
    tb = []
    for _ in range(args.steps):
        torch.cuda._sleep(1_000_000)
        e0.record(stream)
        step_batched()
        e1.record(stream)
        e1.synchronize()
        tb.append(e0.elapsed_time(e1))
    ms_b = float(np.median(tb))
    diff = max(float((x - y).abs().max()) for x, y in zip(step(), step_batched()))
    cal_b.close()
    del q_all
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("cpu baseline: oracle statistics of a few layers")
        t0 = time.perf_counter()
        nl = 0
        while nl < L and (nl == 0 or time.perf_counter() - t0 < min(args.cpu_seconds, 10.0)):
            q = qs[nl].float().cpu().numpy().reshape(T, Hq, hd)
            oracle.calib_stats(q)
            nl += 1
        dt = time.perf_counter() - t0
        cpu = {"value": nl * T / dt, "unit": "query tokens/s per layer", "cores": 1,
               "kind": "oracle", "sample": "%d of %d layers, %d tokens each, %.1f s" % (
                   nl, L, T, dt)}
    cal.close()
    achieved = alg / (ms_b * 1e-3) / 1e9
    return {
        "metric": "calibration query rows accumulated/sec (layer x token)",
        "value": L * T / (ms_b * 1e-3),
        "unit": "layer-token query rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_b,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": str(dtype).replace("torch.", "") + " in, f64 sums",
        "data": "synthetic (per-(head, pair) lognormal/uniform-phase mean plus N(0,1) noise)",
        "config": {"workload": name, "layers": L, "q_heads": Hq, "head_dim": hd, "tokens": T,
                   "parallelism": "single GPU"},
        "roofline": {"kernel": "calib (add_layers + finish)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "alg_bytes_per_launch": alg, "launches_per_step": 1,
                     "avg_launch_ms": ms_b},
        "per_layer_adds": {"call": "tria_calib_add per layer, then finish",
                           "ms_per_step": ms, "value": L * T / (ms * 1e-3),
                           "GB_s": alg / (ms * 1e-3) / 1e9,
                           "frac_hbm": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           "max_abs_diff_vs_one_launch": diff},
        "cpu_baseline": cpu,
    }


def cpu_baseline(wl, stats, k0, v0, p0, seconds, keep_mode=0, compact_mode=0):
    """The CPU oracle, as it stands, on whole passes over the same input (host copies of
    the device-generated cache), repeated until about `seconds` of CPU work."""
    import numpy as np

    import oracle
    log("cpu baseline: oracle on whole passes, about %.0f s" % seconds)
    times, stages = [], []
    spent = 0.0
    while len(times) < 3 or (spent < seconds and len(times) < 50):
        k, v, pos = k0.copy(), v0.copy(), p0.copy()
        t = time.perf_counter()
        oracle.evict(wl.k_type, wl.v_type, wl.L, wl.Hkv, wl.Hq, wl.hd, wl.theta,
                     list(wl.offsets), k, v, pos, wl.n, wl.budget, wl.sink, wl.window, *stats,
                     want_raw=False, want_agg=False, keep_mode=keep_mode,
                     compact_mode=compact_mode)
        dt = time.perf_counter() - t
        times.append(dt)
        stages.append(oracle.last_stage_seconds())
        spent += dt
    rows = wl.L * wl.Hkv * wl.n
    med = float(np.median(times))
    st = np.median(np.array(stages), axis=0) * 1e3
    return {"value": rows / med, "unit": UNIT, "cores": oracle.num_threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "pass_ms_median": med * 1e3,
            "stage_ms_median": {"score_and_aggregate": float(st[0]), "select": float(st[1]),
                                "compact": float(st[2])},
            "sample": "%d whole passes (%d units x %d tokens each), %.1f s of CPU time; "
                      "median pass %.3f s" % (len(times), wl.L * wl.Hkv, wl.n, spent, med)}


if __name__ == "__main__":
    main()
