"""GPU parity: the HIP library (through the C ABI) against the CPU oracle on the
same seeded inputs, element by element, to the bar in parity_util."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import parity_util as pu
from kv_cache_eviction_tria_amd import synth, tria

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
F16, Q8 = synth.KV_F16, synth.KV_Q8_0
WL = synth.WORKLOADS


def variant(base, **kw):
    return dataclasses.replace(base, **kw)


def run_case(wl, n, budget, sink, window, cap=None, mutate=None, where=""):
    pu.say("case %s: L%d Hkv%d Hq%d hd%d k%d v%d n%d cap%s B%d S%d W%d" % (
        where or wl.name, wl.L, wl.Hkv, wl.Hq, wl.hd, wl.k_type, wl.v_type, n, cap, budget, sink,
        window))
    case = synth.make_case(wl, device="cpu", n=n, cap=cap)
    if mutate is not None:
        mutate(case)
    stats = (case["q_re"], case["q_im"], case["w"])
    k0, v0, p0 = case["k"].numpy().copy(), case["v"].numpy().copy(), case["pos"].numpy().copy()
    k, v, pos = case["k"].to(DEV), case["v"].to(DEV), case["pos"].to(DEV)
    ctx = pu.make_ctx(wl, stats)
    g = pu.gpu_pass(ctx, k, v, pos, n, budget, sink, window, wl.G)
    tria.tria_device_status(ctx)
    o = oracle.evict(wl.k_type, wl.v_type, wl.L, wl.Hkv, wl.Hq, wl.hd, wl.theta,
                     list(wl.offsets), k0.copy(), v0.copy(), p0.copy(), n, budget, sink, window,
                     *stats, compact=False)
    nd = pu.compare_pass(g, o, n, budget, sink, window, where or wl.name)
    ka, va, pa = pu.host(k), pu.host(v), pu.host(pos)
    K = g["K"]
    for l in range(wl.L):
        for h in range(wl.Hkv):
            keep = g["keep"][l, h]
            pu.check_gather(k0[l, h], ka[l, h], keep, K, "K")
            pu.check_gather(v0[l, h], va[l, h], keep, K, "V")
            pu.check_gather(p0[l, h], pa[l, h], keep, K, "pos")
    ctx.close()
    pu.say("  ok: kept %d, %d rows in the cutoff band differ" % (K, nd))
    return g, o


def test_workload_tiny_1x1_4k():
    wl = WL["tiny_1x1_4k_f16"]
    run_case(wl, wl.n, wl.budget, wl.sink, wl.window)


def test_workload_qwen3_8b_layer_32k():
    wl = WL["qwen3_8b_layer_32k_f16"]
    run_case(wl, wl.n, wl.budget, wl.sink, wl.window)


SHAPES = [
    # hd, Hkv, Hq, k_type, v_type, n, budget, sink, window
    (128, 2, 8, Q8, F16, 1000, 300, 4, 64),
    (128, 1, 4, Q8, Q8, 4097, 1024, 0, 512),
    (96, 1, 3, Q8, F16, 777, 200, 0, 100),
    (96, 2, 6, F16, F16, 513, 100, 2, 50),
    (32, 1, 1, F16, F16, 300, 50, 1, 10),
    (32, 2, 2, Q8, F16, 257, 70, 0, 9),
    (64, 1, 2, Q8, F16, 4095, 1000, 4, 512),
    (256, 2, 8, F16, F16, 2000, 300, 4, 128),
    (256, 1, 16, Q8, F16, 1500, 400, 0, 256),
    (160, 1, 5, Q8, F16, 999, 222, 3, 33),
    (224, 1, 7, F16, Q8, 600, 100, 0, 0),
    (192, 2, 24, Q8, F16, 700, 350, 8, 16),
    # q8_0 keys on the fp16 matrix-core trig path (hd 128, 256): head sub-groups of
    # 8, 4, 2 and 1
    (128, 1, 8, Q8, F16, 1234, 300, 4, 64),
    (128, 2, 6, Q8, Q8, 900, 250, 0, 100),
    (256, 1, 3, Q8, F16, 800, 200, 2, 32),
    # fp16 keys on the matrix-core scorer: head chunks of 4 within a launch of up
    # to 16 heads (G 3 and 5 leave partial chunks), and G 20 takes two launches
    (128, 1, 3, F16, F16, 1100, 300, 2, 64),
    (192, 2, 10, F16, F16, 777, 200, 1, 50),
    (128, 1, 12, F16, Q8, 2049, 512, 0, 128),
    (64, 1, 20, F16, F16, 1300, 333, 3, 100),
    # the largest GQA ratio a model may have (64 query heads per KV head)
    (128, 1, 64, Q8, F16, 700, 200, 2, 64),
    (256, 2, 128, F16, F16, 500, 100, 0, 32),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "hd%d_g%d_%d_k%d_n%d" % (s[0], s[1], s[2], s[3], s[5]))
def test_shapes(shape):
    hd, Hkv, Hq, kt, vt, n, budget, sink, window = shape
    wl = variant(WL["tiny_1x1_4k_f16"], name="shape", L=2, Hkv=Hkv, Hq=Hq, hd=hd, k_type=kt,
                 v_type=vt, seed=hd + Hq + n)
    run_case(wl, n, budget, sink, window, cap=n + 37)


@pytest.mark.parametrize("seed", range(16))
def test_random_configurations(seed):
    """Seeded random configurations across every kernel variant: head dims 32-256
    (matrix-core and row-per-lane scorers, every compaction chunk width), GQA
    ratios 1-16, fp16/q8_0 K and V, row counts with ragged tails, and budgets,
    sinks and windows from empty to covering."""
    rng = np.random.default_rng(1000 + seed)
    hd = int(rng.choice([32, 64, 96, 128, 160, 192, 224, 256]))
    G = int(rng.integers(1, 17))
    Hkv = int(rng.integers(1, 3))
    kt, vt = int(rng.choice([F16, Q8])), int(rng.choice([F16, Q8]))
    n = int(rng.integers(1, 2600))
    budget = int(rng.integers(0, n + 2))
    sink = int(rng.integers(0, 9))
    window = int(rng.choice([0, int(rng.integers(0, n + 1)), int(rng.integers(0, 300))]))
    wl = variant(WL["tiny_1x1_4k_f16"], name="random%d" % seed, L=int(rng.integers(1, 3)),
                 Hkv=Hkv, Hq=Hkv * G, hd=hd, k_type=kt, v_type=vt, seed=seed + 50)
    run_case(wl, n, budget, sink, window, cap=n + int(rng.integers(0, 40)))


@pytest.mark.parametrize("n,budget,sink,window", [
    (1, 0, 0, 0), (1, 0, 0, 1), (2, 1, 0, 0), (5, 0, 0, 0), (300, 0, 0, 0), (300, 10, 200, 200),
    (300, 299, 0, 0), (300, 5, 3, 4), (1025, 1024, 0, 1), (1024, 1, 0, 0), (700, 600, 650, 0),
])
@pytest.mark.parametrize("k_type", [Q8, F16], ids=["q8", "f16"])
def test_edge_budgets(n, budget, sink, window, k_type):
    wl = variant(WL["tiny_1x1_4k_f16"], name="edge", L=1, Hkv=2, Hq=4, k_type=k_type, seed=n + 3)
    run_case(wl, n, budget, sink, window, cap=n + 1)


def test_budget_covers_all_is_a_no_op():
    wl = variant(WL["tiny_1x1_4k_f16"], name="noop", L=2, Hkv=2, Hq=8)
    case = synth.make_case(wl, device="cpu", n=500, cap=600)
    k, v, pos = case["k"].to(DEV), case["v"].to(DEV), case["pos"].to(DEV)
    k0, v0, p0 = k.clone(), v.clone(), pos.clone()
    ctx = pu.make_ctx(wl, (case["q_re"], case["q_im"], case["w"]))
    assert tria.tria_evict(ctx, k, v, pos, 500, 500, 4, 16) == 500
    assert tria.tria_evict(ctx, k, v, pos, 500, 10_000, 0, 0) == 500
    assert tria.tria_evict(ctx, k, v, pos, 0, 0, 0, 0) == 0
    torch.cuda.synchronize()
    assert torch.equal(k, k0) and torch.equal(v, v0) and torch.equal(pos, p0)
    ctx.close()


def test_nonfinite_rows_and_flat_heads():
    """Rows holding inf/NaN score -inf (evicted unless protected) and are left out of
    the statistics; a q8_0 block scale of inf does the same; constant heads give
    sigma = 0 (z = 0) and every tie goes to the lowest row."""
    wl = variant(WL["tiny_1x1_4k_f16"], name="nonfinite", L=1, Hkv=2, Hq=4)

    def poison(case):
        k = case["k"].view(torch.float16)
        k[0, 0, 10, 3] = float("inf")
        k[0, 0, 20, 70] = float("nan")
        k[0, 0, 399, 0] = float("-inf")  # protected by the window
        k[0, 1] = k[0, 1, 0:1]  # every row of KV head 1 identical: flat heads
    run_case(wl, 400, 100, 2, 8, mutate=poison)

    wl8 = variant(wl, k_type=Q8)

    def poison8(case):
        case["k"][0, 0, 33, 0:2] = torch.tensor([0x00, 0x7C], dtype=torch.uint8)  # scale = +inf
    run_case(wl8, 400, 100, 2, 8, mutate=poison8)


def test_f16_magnitudes_past_the_half_range():
    """Key pairs whose |K_f| exceeds the fp16 range (both halves near 6e4) and
    per-head statistics six orders of magnitude apart: the matrix-core scorer's
    hi/lo splits and per-head scales keep every raw score within the bar."""
    wl = variant(WL["tiny_1x1_4k_f16"], name="magnitudes", L=1, Hkv=2, Hq=8, hd=128)

    def big(case):
        k = case["k"].view(torch.float16)
        k[0, 0, 5:40, :] = 60000.0 * torch.sign(k[0, 0, 5:40, :].float()).half()
        k[0, 1, 100:110, 0:64] = 65000.0
        k[0, 1, 100:110, 64:128] = -65000.0
        case["q_re"][0, 0] *= 1e5
        case["q_im"][0, 0] *= 1e5
        case["w"][0, 0] *= 1e5
        case["q_re"][0, 5] *= 1e-5
        case["q_im"][0, 5] *= 1e-5
        case["w"][0, 5] *= 1e-5
    run_case(wl, 600, 150, 4, 32, mutate=big)


def _wide_block(case, hd, pair, key_ratio):
    """One frequency pair's mean query 1e4 times the others of its 32-dim blocks (every
    query head), and, with key_ratio > 1, keys key_ratio times larger on the other
    dimensions of those blocks than on the pair's own two dimensions (outlier key
    channels where the coefficients are small)."""
    F = hd // 2
    for x in ("q_re", "q_im", "w"):
        case[x][:, :, pair] *= 1e4
    if key_ratio > 1.0:
        L, Hkv, cap = case["pos"].shape
        n = case["n"]
        g = torch.Generator().manual_seed(31)
        scale = torch.ones(hd)
        for d0 in ((pair // 32) * 32, F + (pair // 32) * 32):
            scale[d0:d0 + 32] = key_ratio
        scale[pair] = 1.0
        scale[F + pair] = 1.0
        x = torch.randn(L, Hkv, n, hd, generator=g) * scale
        k_type = synth.KV_Q8_0 if case["k"].shape[-1] != 2 * hd else synth.KV_F16
        case["k"][:, :, :n] = synth.encode(x, k_type)


@pytest.mark.parametrize("key_ratio", [1.0, 1e3], ids=["big_pair", "big_keys_on_small_pairs"])
@pytest.mark.parametrize("k_type,hd,Hq", [(Q8, 128, 8), (Q8, 256, 16), (Q8, 96, 6), (Q8, 64, 2),
                                          (F16, 128, 8)],
                         ids=["q8_hd128", "q8_hd256", "q8_hd96", "q8_hd64", "f16_hd128"])
def test_coefficients_across_a_wide_block_range(k_type, hd, Hq, key_ratio):
    """Trig coefficients 1e4 apart inside one 32-dim block (one pair's mean query much
    larger than the rest), alone and with the keys large exactly where the coefficients
    are small: each coefficient must keep its own precision, not the block maximum's,
    for the raw scores to stay within the bar.  q8_0 at hd 128 and 256 takes the
    fp16 matrix-core trig path, at hd 96 and 64 the 32-bit integer digits."""
    wl = variant(WL["tiny_1x1_4k_f16"], name="wide_block", L=2, Hkv=2, Hq=Hq, hd=hd,
                 k_type=k_type, seed=11)
    pair = min(40, hd // 2 - 3)
    run_case(wl, 3000, 900, 4, 128, mutate=lambda c: _wide_block(c, wl.hd, pair, key_ratio),
             where="wide_block k%d hd%d keys x%g" % (k_type, hd, key_ratio))


def test_second_pass_uses_absolute_position():
    """After a compaction the newest row's position exceeds the row count; a second
    pass on the compacted cache plus appended rows must match the oracle."""
    wl = variant(WL["tiny_1x1_4k_f16"], name="second", L=2, Hkv=2, Hq=8, k_type=Q8)
    n, B = 3200, 3072
    case = synth.make_case(wl, device="cpu", n=n, cap=n)
    k, v, pos = case["k"].to(DEV), case["v"].to(DEV), case["pos"].to(DEV)
    stats = (case["q_re"], case["q_im"], case["w"])
    ctx = pu.make_ctx(wl, stats)
    assert tria.tria_evict(ctx, k, v, pos, n, B, 0, 512) == B
    # append 128 new rows at positions continuing after the newest one
    fresh = synth.make_case(variant(wl, seed=99), device="cpu", n=128, cap=128)
    k[:, :, B:B + 128] = fresh["k"].to(DEV)
    v[:, :, B:B + 128] = fresh["v"].to(DEV)
    pos[:, :, B:B + 128] = pos[:, :, B - 1:B] + 1 + torch.arange(128, device=DEV, dtype=torch.int32)
    torch.cuda.synchronize()
    assert int(pos[0, 0, B + 127]) == n + 127  # absolute position, not the row count
    k0, v0, p0 = pu.host(k).copy(), pu.host(v).copy(), pu.host(pos).copy()
    g = pu.gpu_pass(ctx, k, v, pos, n, B, 0, 512, wl.G)
    o = oracle.evict(wl.k_type, wl.v_type, wl.L, wl.Hkv, wl.Hq, wl.hd, wl.theta,
                     list(wl.offsets), k0.copy(), v0.copy(), p0.copy(), n, B, 0, 512, *stats,
                     compact=False)
    pu.compare_pass(g, o, n, B, 0, 512, "second pass")
    ctx.close()


@pytest.mark.parametrize("L", [2, 14])
def test_evict_equals_the_three_stages(L):
    """tria_evict leaves the same cache as score -> select -> compact run one after
    the other."""
    wl = variant(WL["qwen3_8b_layer_32k_f16"], name="stages", L=L, Hkv=4, Hq=16, k_type=Q8)
    n, B, S, W = 9000, 2000, 4, 512
    case = synth.make_case(wl, device="cpu", n=n, cap=n + 5)
    stats = (case["q_re"], case["q_im"], case["w"])
    ctx = pu.make_ctx(wl, stats)
    a = [case[x].to(DEV) for x in ("k", "v", "pos")]
    b = [t.clone() for t in a]
    assert tria.tria_evict(ctx, *a, n, B, S, W) == B
    g = pu.gpu_pass(ctx, *b, n, B, S, W, wl.G)
    tria.tria_device_status(ctx)
    for x, y in zip(a, b):
        assert torch.equal(x[:, :, :B], y[:, :, :B])
    ctx.close()


@pytest.mark.parametrize("pattern", ["alternate", "tail", "head_run", "random", "invalid"])
@pytest.mark.parametrize("hd,n,v_type", [(96, 5000, F16), (160, 4999, Q8), (32, 3001, F16)],
                         ids=["hd96", "hd160_q8v_odd_cap", "hd32_odd_cap"])
def test_compaction_patterns(pattern, hd, n, v_type):
    """Adversarial keep patterns for the in-place gather, K/V/pos of several row sizes.
    q8_0 rows at these widths (102, 170, 34 bytes) move in aligned 4-byte words; an
    odd row count per unit puts every other unit's rows on 2-byte offsets."""
    rng = np.random.default_rng(7)
    L, Hkv = 2, 3
    wl = variant(WL["tiny_1x1_4k_f16"], name="compact", L=L, Hkv=Hkv, Hq=Hkv, hd=hd, k_type=Q8,
                 v_type=v_type)
    kb, vb = synth.row_bytes(Q8, hd), synth.row_bytes(v_type, hd)
    k = torch.from_numpy(rng.integers(0, 256, size=(L, Hkv, n, kb), dtype=np.uint8))
    v = torch.from_numpy(rng.integers(0, 256, size=(L, Hkv, n, vb), dtype=np.uint8))
    pos = torch.from_numpy(np.broadcast_to(np.arange(n, dtype=np.int32), (L, Hkv, n)).copy())
    if pattern == "alternate":
        keep1 = np.arange(1, n, 2)
    elif pattern == "tail":
        keep1 = np.arange(n - 1500, n)
    elif pattern == "head_run":
        keep1 = np.concatenate([np.arange(0, 900), np.arange(1000, n, 3)])
    else:
        keep1 = np.sort(rng.choice(n, size=1234, replace=False))
    pu.say("case compaction %s hd %d n %d v%d" % (pattern, hd, n, v_type))
    K = len(keep1)
    keep = np.broadcast_to(keep1.astype(np.int32), (L, Hkv, K)).copy()
    if pattern == "invalid":
        # still ascending, but outside [d, n): skipped
        keep[0, 0, 0] = -3       # below its destination
        keep[1, 2, K - 1] = n + 50   # past n
    stats = synth.gen_stats(L, Hkv, hd, 1)
    ctx = pu.make_ctx(wl, stats)
    k0, v0, p0 = k.numpy().copy(), v.numpy().copy(), pos.numpy().copy()
    kd, vd, pd, keepd = k.to(DEV), v.to(DEV), pos.to(DEV), torch.from_numpy(keep).to(DEV)
    tria.tria_compact(ctx, kd, vd, pd, n, keepd, K)
    torch.cuda.synchronize()
    ka, va, pa = pu.host(kd), pu.host(vd), pu.host(pd)
    for l in range(L):
        for h in range(Hkv):
            ki = keep[l, h].copy()
            if pattern == "invalid":
                bad = (ki < np.arange(K)) | (ki >= n)
                ki[bad] = np.arange(K)[bad]  # skipped rows keep their own bytes
            pu.check_gather(k0[l, h], ka[l, h], ki, K, "K")
            pu.check_gather(v0[l, h], va[l, h], ki, K, "V")
            pu.check_gather(p0[l, h], pa[l, h], ki, K, "pos")
    ctx.close()


@pytest.mark.parametrize("entry", ["evict", "noalloc"])
def test_captured_pass_replays(entry):
    """A whole pass captured in a HIP graph (after one eager call, so that nothing is
    allocated while capturing) and replayed several times, the cache restored by eager
    copies between replays: every replay leaves the eager pass's cache.  The epoch the
    compaction stamps its flags with advances on the device, so a replay never takes
    the flags of the replay before it for its own."""
    wl = variant(WL["qwen3_8b_full_32k_q8"], name="graph", L=4)
    n, B, S, W = wl.n, wl.budget, wl.sink, wl.window
    stats = synth.gen_stats(wl.L, wl.Hq, wl.hd, 31)
    k, v, pos = synth.gen_cache(wl.L, wl.Hkv, wl.hd, n, n, wl.k_type, wl.v_type, 31, DEV)
    k0, v0, p0 = k.clone(), v.clone(), pos.clone()
    ctx = pu.make_ctx(wl, stats)
    fn = tria.tria_evict if entry == "evict" else tria.tria_evict_noalloc
    assert fn(ctx, k, v, pos, n, B, S, W) == B
    torch.cuda.synchronize()
    want = [t[:, :, :B].clone() for t in (k, v, pos)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(ctx, k, v, pos, n, B, S, W)
    for rep in range(4):
        pu.say("case graph %s replay %d" % (entry, rep))
        k.copy_(k0)
        v.copy_(v0)
        pos.copy_(p0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        tria.tria_device_status(ctx)
        for t, w, name in zip((k, v, pos), want, ("k", "v", "pos")):
            assert torch.equal(t[:, :, :B], w), (entry, rep, name)
    del g
    ctx.close()


def test_captured_paged_batch_replays():
    """A batched pass over a paged cache captured in a HIP graph after one eager call
    and replayed with the pools restored between replays: every replay leaves the
    eager pass's pools (in both compaction modes)."""
    wl = variant(WL["paged16_qwen3_8b_q8"], name="graph_paged", L=4, Hkv=4, Hq=16, hd=128)
    lens = [4000, 1500, 2600, 700]
    budgets = [1200, 500, 800, 700]
    stats = synth.gen_stats(wl.L, wl.Hq, wl.hd, 12)
    pg = synth.gen_paged(wl.L, wl.Hkv, wl.hd, wl.k_type, wl.v_type, lens, 12, DEV)
    names = ("k_pool", "v_pool", "pos_pool")
    pristine = {x: pg[x].clone() for x in names}
    for mode in (tria.TRIA_COMPACT_ORDERED, tria.TRIA_COMPACT_HOLE_FILL):
        ctx = pu.make_ctx(wl, stats)
        tria.tria_set_compaction(ctx, mode)
        for x in names:
            pg[x].copy_(pristine[x])
        args = (ctx, pg["k_pool"], pg["v_pool"], pg["pos_pool"], pg["block_table"], lens, budgets,
                wl.sink, wl.window)
        kept = [tria.tria_kept_count(n, bgt, wl.sink, wl.window) for n, bgt in zip(lens, budgets)]
        assert tria.tria_evict_paged_batch(*args) == kept
        torch.cuda.synchronize()
        want = {x: pg[x].clone() for x in names}
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            tria.tria_evict_paged_batch(*args)
        for rep in range(3):
            pu.say("case graph paged mode %d replay %d" % (mode, rep))
            for x in names:
                pg[x].copy_(pristine[x])
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            tria.tria_device_status(ctx)
            for s, n in enumerate(lens):
                for x in names:
                    got = synth.paged_rows(pg[x], pg["block_table"][s], kept[s])
                    exp = synth.paged_rows(want[x], pg["block_table"][s], kept[s])
                    assert torch.equal(got, exp), (mode, rep, s, x)
        del g
        ctx.close()


def test_two_contexts_on_two_streams():
    """Two contexts, each on its own stream, run passes over their own caches at the
    same time (one ordered, one hole-filling; their persistent compaction grids then
    share the device): both leave the caches a pass alone on one stream leaves."""
    wl = variant(WL["qwen3_8b_full_32k_q8"], name="streams", L=6)
    n, B, S, W = wl.n, wl.budget, wl.sink, wl.window
    caches, ctxs, want = [], [], []
    for i, mode in enumerate((tria.TRIA_COMPACT_ORDERED, tria.TRIA_COMPACT_HOLE_FILL)):
        stats = synth.gen_stats(wl.L, wl.Hq, wl.hd, 40 + i)
        c = list(synth.gen_cache(wl.L, wl.Hkv, wl.hd, n, n, wl.k_type, wl.v_type, 40 + i, DEV))
        ctx = pu.make_ctx(wl, stats)
        tria.tria_set_compaction(ctx, mode)
        ref = [t.clone() for t in c]
        assert tria.tria_evict(ctx, *ref, n, B, S, W) == B
        torch.cuda.synchronize()
        caches.append(c)
        ctxs.append(ctx)
        want.append([t[:, :, :B].clone() for t in ref])
        del ref
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    work = [[t.clone() for t in c] for c in caches]
    torch.cuda.synchronize()
    for rep in range(3):
        pu.say("case two streams rep %d" % rep)
        for i in (0, 1):
            with torch.cuda.stream(streams[i]):
                for t, t0 in zip(work[i], caches[i]):
                    t.copy_(t0)
                assert tria.tria_evict(ctxs[i], *work[i], n, B, S, W, streams[i]) == B
        torch.cuda.synchronize()
        for i in (0, 1):
            tria.tria_device_status(ctxs[i])
            for t, w, name in zip(work[i], want[i], ("k", "v", "pos")):
                assert torch.equal(t[:, :, :B], w), (i, rep, name)
    for ctx in ctxs:
        ctx.close()


@pytest.mark.parametrize("pattern", ["selected", "alternate", "tail", "random"])
def test_serial_compaction_reference(pattern):
    """The ordered compaction run by one workgroup (every chunk task in order, so no
    task waits for another) and by the full grid leave byte-identical caches: the
    forced serial path as the reference of the parallel in-place rule, on a 4 x 8 x 32K
    q8_0 cache with the selector's kept rows and with adversarial patterns."""
    wl = variant(WL["qwen3_8b_full_32k_q8"], name="serial", L=4)
    n, B, S, W = wl.n, wl.budget, wl.sink, wl.window
    stats = synth.gen_stats(wl.L, wl.Hq, wl.hd, 21)
    a = list(synth.gen_cache(wl.L, wl.Hkv, wl.hd, n, n, wl.k_type, wl.v_type, 21, DEV))
    b = [t.clone() for t in a]
    ctx = pu.make_ctx(wl, stats)
    pu.say("case serial compaction %s" % pattern)
    if pattern == "selected":
        tria.tria_set_compaction_workgroups(ctx, 1)
        Ka = tria.tria_evict(ctx, *a, n, B, S, W)
        tria.tria_set_compaction_workgroups(ctx, 0)
        Kb = tria.tria_evict(ctx, *b, n, B, S, W)
    else:
        rng = np.random.default_rng(5)
        if pattern == "alternate":
            keep1 = np.arange(1, n, 2)
        elif pattern == "tail":
            keep1 = np.arange(n - 3000, n)
        else:
            keep1 = np.sort(rng.choice(n, size=10000, replace=False))
        Ka = Kb = len(keep1)
        keep = torch.from_numpy(np.broadcast_to(keep1.astype(np.int32),
                                                (wl.L, wl.Hkv, Ka)).copy()).to(DEV)
        tria.tria_set_compaction_workgroups(ctx, 1)
        tria.tria_compact(ctx, *a, n, keep, Ka)
        tria.tria_set_compaction_workgroups(ctx, 0)
        tria.tria_compact(ctx, *b, n, keep, Kb)
    tria.tria_device_status(ctx)
    assert Ka == Kb
    for x, y, name in zip(a, b, ("k", "v", "pos")):
        assert torch.equal(x[:, :, :Ka], y[:, :, :Ka]), name
    ctx.close()


@pytest.mark.parametrize("groups", [1, 3])
def test_paged_batch_compaction_on_a_small_grid(groups):
    """A paged batch whose sequences move different numbers of chunks (one moves
    none): the compaction's densely numbered tasks, taken by 1 or 3 workgroups,
    leave the pools byte-identical to the full grid's."""
    wl = variant(WL["paged16_qwen3_8b_q8"], name="paged_grid", L=5, Hkv=2, Hq=8, hd=128)
    lens = [3000, 517, 1200, 64, 2048, 4100]
    budgets = [900, 150, 1200, 70, 600, 1000]  # seq 3 keeps everything
    S, W = 0, 128
    pg = synth.gen_paged(wl.L, wl.Hkv, wl.hd, wl.k_type, wl.v_type, lens, 91)
    stats = synth.gen_stats(wl.L, wl.Hq, wl.hd, 9)
    pu.say("case paged compaction on %d workgroups" % groups)
    outs = []
    for g in (groups, 0):
        ctx = pu.make_ctx(wl, stats)
        tria.tria_set_compaction_workgroups(ctx, g)
        dev = {k: pg[k].to(DEV) for k in ("k_pool", "v_pool", "pos_pool", "block_table")}
        kept = tria.tria_evict_paged_batch(ctx, dev["k_pool"], dev["v_pool"], dev["pos_pool"],
                                           dev["block_table"], lens, budgets, S, W)
        tria.tria_device_status(ctx)
        outs.append((kept, [dev[k].cpu() for k in ("k_pool", "v_pool", "pos_pool")]))
        ctx.close()
    (ka, a), (kb, b) = outs
    assert ka == kb
    for x, y, name in zip(a, b, ("k", "v", "pos")):
        assert torch.equal(x, y), name


def _oracle_layers(wl, stats, k0, p0, l0, nl):
    """The oracle's scores, aggregates and kept rows for layers [l0, l0 + nl) of a
    device cache, from host copies of just those layers (bounds host memory)."""
    kk = pu.host(k0[l0:l0 + nl]).copy()
    pp = pu.host(p0[l0:l0 + nl]).copy()
    sl = [x[l0:l0 + nl] for x in stats]
    vv = np.zeros((1,), np.uint8)  # V is not read without compaction
    return oracle.evict(wl.k_type, wl.v_type, nl, wl.Hkv, wl.Hq, wl.hd, wl.theta,
                        list(wl.offsets), kk, vv, pp, wl.n, wl.budget, wl.sink, wl.window, *sl,
                        compact=False)


def _full_size(wl, layers_per_check):
    """Full-size pass in the launch configuration the benchmark times.  Every unit's raw
    scores, aggregates and kept rows are compared with the oracle's (a few layers at a
    time), and every unit's compaction is checked as an exact gather on the device."""
    pu.say("full-size case %s" % wl.name)
    stats = synth.gen_stats(wl.L, wl.Hq, wl.hd, wl.seed)
    k, v, pos = synth.gen_cache(wl.L, wl.Hkv, wl.hd, wl.n, wl.n, wl.k_type, wl.v_type, wl.seed,
                                DEV)
    k0, v0, p0 = k.clone(), v.clone(), pos.clone()
    ctx = pu.make_ctx(wl, stats)
    n, B, S, W, G = wl.n, wl.budget, wl.sink, wl.window, wl.G
    K = tria.tria_kept_count(n, B, S, W)
    raw = torch.empty(wl.L, wl.Hkv, n, G, dtype=torch.float32, device=DEV)
    agg = torch.empty(wl.L, wl.Hkv, n, dtype=torch.float32, device=DEV)
    keep = torch.empty(wl.L, wl.Hkv, K, dtype=torch.int32, device=DEV)
    tria.tria_score(ctx, k, v, pos, n, raw)
    assert tria.tria_select(ctx, raw, n, B, S, W, keep, agg) == K
    tria.tria_compact(ctx, k, v, pos, n, keep, K)
    torch.cuda.synchronize()
    # every unit: exact gather, ascending, protected rows kept
    li = torch.arange(wl.L, device=DEV)[:, None, None]
    hi = torch.arange(wl.Hkv, device=DEV)[None, :, None]
    kl = keep.long()
    assert torch.equal(k[:, :, :K], k0[li, hi, kl])
    assert torch.equal(v[:, :, :K], v0[li, hi, kl])
    assert torch.equal(pos[:, :, :K], p0[li, hi, kl])
    assert bool((kl[:, :, 1:] > kl[:, :, :-1]).all())
    if S:
        assert torch.equal(kl[:, :, :S].cpu(), torch.arange(S).expand(wl.L, wl.Hkv, S))
    assert torch.equal(kl[:, :, K - W:].cpu(), torch.arange(n - W, n).expand(wl.L, wl.Hkv, W))
    # every unit against the oracle
    st = {}
    nd = 0
    for l0 in range(0, wl.L, layers_per_check):
        nl = min(layers_per_check, wl.L - l0)
        o = _oracle_layers(wl, stats, k0, p0, l0, nl)
        g = dict(raw=pu.host(raw[l0:l0 + nl]), agg=pu.host(agg[l0:l0 + nl]),
                 keep=pu.host(keep[l0:l0 + nl]))
        nd += pu.compare_pass(g, o, n, B, S, W, "%s layers %d..%d" % (wl.name, l0, l0 + nl - 1),
                              st)
        del o, g
        pu.say("  layers %d..%d: every unit within the bar" % (l0, l0 + nl - 1))
    pu.say("  all %d units: worst raw rel err %.3g, worst agg err %.3g of the 1e-3 bound, "
           "%d kept rows differ (all in the cutoff band, worst %.3g of max(|tau|,1), %d outside "
           "the strict 1e-3 band)" % (wl.L * wl.Hkv, st.get("worst_raw", 0.0),
                                      st.get("worst_agg", 0.0), nd, st.get("worst_band", 0.0),
                                      st.get("outside_strict", 0)))
    # The whole pass as the benchmark times it (tria_evict), several times in a row:
    # the same cache as the staged calls, and no compaction wait given up.
    kk, vv, pp = k[:, :, :K].clone(), v[:, :, :K].clone(), pos[:, :, :K].clone()
    for rep in range(3):
        k.copy_(k0)
        v.copy_(v0)
        pos.copy_(p0)
        assert tria.tria_evict(ctx, k, v, pos, n, B, S, W) == K
        tria.tria_device_status(ctx)
        assert torch.equal(k[:, :, :K], kk) and torch.equal(v[:, :, :K], vv)
        assert torch.equal(pos[:, :, :K], pp)
        pu.say("  tria_evict rep %d identical" % rep)
    ctx.close()
    del k, v, pos, k0, v0, p0, raw, agg, keep, kk, vv, pp
    torch.cuda.empty_cache()


def test_full_qwen3_8b_32k_q8():
    _full_size(WL["qwen3_8b_full_32k_q8"], 12)


def test_full_hd256_48x4_128k():
    _full_size(WL["hd256_48x4_128k_f16"], 4)


@pytest.mark.parametrize("n,k_type", [(131073, Q8), (tria.TRIA_MAX_ROWS, F16)],
                         ids=["128k+1_q8", "max_f16"])
def test_units_past_the_register_bins(n, k_type):
    """Units of more than 128K rows, up to the largest a pass takes: the selector
    keeps their keys in a global scratch array instead of registers."""
    wl = variant(WL["tiny_1x1_4k_f16"], name="long", L=1, Hkv=2, Hq=4, hd=64, k_type=k_type,
                 seed=n % 1000 + 7)
    run_case(wl, n, n // 10, 4, 1024, cap=n + 5)


def test_rows_past_the_maximum_are_refused():
    """One row more than the largest unit a pass takes is refused before anything
    is enqueued: the cache is left as it was."""
    wl = variant(WL["tiny_1x1_4k_f16"], name="too_long", L=1, Hkv=1, Hq=1, hd=32, seed=5)
    n = tria.TRIA_MAX_ROWS + 1
    pu.say("case too_long: n %d" % n)
    case = synth.make_case(wl, device="cpu", n=n, cap=n)
    ctx = pu.make_ctx(wl, (case["q_re"], case["q_im"], case["w"]))
    k, v, pos = case["k"].to(DEV), case["v"].to(DEV), case["pos"].to(DEV)
    k0, v0, p0 = k.clone(), v.clone(), pos.clone()
    raw = torch.empty(1, 1, n, 1, dtype=torch.float32, device=DEV)
    keep = torch.empty(1, 1, n, dtype=torch.int32, device=DEV)
    for call in (lambda: tria.tria_evict(ctx, k, v, pos, n, 1000, 0, 16),
                 lambda: tria.tria_score(ctx, k, v, pos, n, raw),
                 lambda: tria.tria_select(ctx, raw, n, 1000, 0, 16, keep)):
        with pytest.raises(tria.TriaError) as e:
            call()
        assert e.value.code == tria.TRIA_E_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.equal(k, k0) and torch.equal(v, v0) and torch.equal(pos, p0)
    ctx.close()


@pytest.mark.parametrize("k_type,hd,v_type", [(Q8, 128, F16), (F16, 128, F16), (Q8, 96, Q8)],
                         ids=["q8", "f16", "q8_hd96_q8v"])
def test_paged_batch(k_type, hd, v_type):
    """Paged cache, 16-row blocks in shuffled physical order, several sequences of
    different lengths (one with nothing to evict) in one batched pass; every
    sequence checked against the oracle on its logical rows (q8_0 rows of 102 bytes
    move in aligned 4-byte words)."""
    wl = variant(WL["paged16_qwen3_8b_q8"], name="paged", L=7, Hkv=2, Hq=8, hd=hd,
                 k_type=k_type, v_type=v_type)
    lens = [3000, 517, 1200, 64, 2048]
    budgets = [900, 150, 1200, 70, 600]  # seq 3: budget >= n keeps everything
    S, W = 0, 128
    pg = synth.gen_paged(wl.L, wl.Hkv, wl.hd, wl.k_type, wl.v_type, lens, 77)
    stats = synth.gen_stats(wl.L, wl.Hq, wl.hd, 5)
    before = [(synth.paged_rows(pg["k_pool"], pg["block_table"][s], n).numpy().copy(),
               synth.paged_rows(pg["v_pool"], pg["block_table"][s], n).numpy().copy(),
               synth.paged_rows(pg["pos_pool"], pg["block_table"][s], n).numpy().copy())
              for s, n in enumerate(lens)]
    pu.say("case paged k%d lens %s" % (k_type, lens))
    ctx = pu.make_ctx(wl, stats)
    dev = {k: pg[k].to(DEV) for k in ("k_pool", "v_pool", "pos_pool", "block_table")}
    kept = tria.tria_evict_paged_batch(ctx, dev["k_pool"], dev["v_pool"], dev["pos_pool"],
                                       dev["block_table"], lens, budgets, S, W)
    tria.tria_device_status(ctx)
    bt = dev["block_table"].cpu()
    for s, n in enumerate(lens):
        K = oracle.kept_count(n, budgets[s], S, W)
        assert kept[s] == K
        k0, v0, p0 = before[s]
        o = oracle.evict(wl.k_type, wl.v_type, wl.L, wl.Hkv, wl.Hq, wl.hd, wl.theta,
                         list(wl.offsets), k0.copy(), v0.copy(), p0.copy(), n, budgets[s], S, W,
                         *stats, compact=False)
        ka = synth.paged_rows(dev["k_pool"].cpu(), bt[s], n).numpy()
        va = synth.paged_rows(dev["v_pool"].cpu(), bt[s], n).numpy()
        pa = synth.paged_rows(dev["pos_pool"].cpu(), bt[s], n).numpy()
        for l in range(wl.L):
            for h in range(wl.Hkv):
                keep = pa[l, h, :K]  # positions were 0..n-1: the kept rows
                where = "paged seq %d unit (%d,%d)" % (s, l, h)
                pu.check_kept(keep, o["keep_idx"][l, h], o["agg"][l, h], n, budgets[s], S, W,
                              where)
                pu.check_gather(k0[l, h], ka[l, h], keep, K, where + " K")
                pu.check_gather(v0[l, h], va[l, h], keep, K, where + " V")
    ctx.close()


def test_paged_batch_of_the_most_sequences():
    """The largest batch one call takes (TRIA_MAX_SEQ sequences), with an empty
    sequence, a one-row sequence and one whose budget covers it among seeded ragged
    lengths; every sequence checked against the oracle on its logical rows."""
    rng = np.random.default_rng(64)
    n_seq = tria.TRIA_MAX_SEQ
    lens = [int(x) for x in rng.integers(2, 700, size=n_seq)]
    lens[5], lens[17] = 0, 1
    budgets = [int(0.3 * n) for n in lens]
    budgets[40] = lens[40] + 3  # keeps everything
    S, W = 2, 32
    wl = variant(WL["paged16_qwen3_8b_q8"], name="paged64", L=2, Hkv=2, Hq=6, hd=64,
                 k_type=Q8, v_type=F16)
    pg = synth.gen_paged(wl.L, wl.Hkv, wl.hd, wl.k_type, wl.v_type, lens, 64)
    stats = synth.gen_stats(wl.L, wl.Hq, wl.hd, 9)
    before = [(synth.paged_rows(pg["k_pool"], pg["block_table"][s], n).numpy().copy(),
               synth.paged_rows(pg["v_pool"], pg["block_table"][s], n).numpy().copy(),
               synth.paged_rows(pg["pos_pool"], pg["block_table"][s], n).numpy().copy())
              for s, n in enumerate(lens)]
    pu.say("case paged batch of %d sequences" % n_seq)
    ctx = pu.make_ctx(wl, stats)
    dev = {k: pg[k].to(DEV) for k in ("k_pool", "v_pool", "pos_pool", "block_table")}
    kept = tria.tria_evict_paged_batch(ctx, dev["k_pool"], dev["v_pool"], dev["pos_pool"],
                                       dev["block_table"], lens, budgets, S, W)
    tria.tria_device_status(ctx)
    bt = dev["block_table"].cpu()
    for s, n in enumerate(lens):
        K = oracle.kept_count(n, budgets[s], S, W)
        assert kept[s] == K, s
        if n == 0:
            continue
        k0, v0, p0 = before[s]
        o = oracle.evict(wl.k_type, wl.v_type, wl.L, wl.Hkv, wl.Hq, wl.hd, wl.theta,
                         list(wl.offsets), k0.copy(), v0.copy(), p0.copy(), n, budgets[s], S, W,
                         *stats, compact=False)
        ka = synth.paged_rows(dev["k_pool"].cpu(), bt[s], n).numpy()
        va = synth.paged_rows(dev["v_pool"].cpu(), bt[s], n).numpy()
        pa = synth.paged_rows(dev["pos_pool"].cpu(), bt[s], n).numpy()
        for l in range(wl.L):
            for h in range(wl.Hkv):
                keep = pa[l, h, :K]
                where = "paged64 seq %d unit (%d,%d)" % (s, l, h)
                pu.check_kept(keep, o["keep_idx"][l, h], o["agg"][l, h], n, budgets[s], S, W,
                              where)
                pu.check_gather(k0[l, h], ka[l, h], keep, K, where + " K")
                pu.check_gather(v0[l, h], va[l, h], keep, K, where + " V")
    ctx.close()


def _pre_rows_of(post_pos, pre_pos):
    """Row of the pre-pass cache that holds each position (positions are unique within
    a unit): [..., K] positions, [..., n] pre-pass positions -> [..., K] rows."""
    out = np.empty(post_pos.shape, np.int64)
    for u in np.ndindex(*post_pos.shape[:-1]):
        order = np.argsort(pre_pos[u], kind="stable")
        sp = pre_pos[u][order]
        j = np.searchsorted(sp, post_pos[u])
        assert np.all(j < len(sp)) and np.array_equal(sp[j], post_pos[u]), \
            "unit %s holds a position the pass did not start with" % (u,)
        out[u] = order[j]
    return out


@pytest.mark.parametrize("compaction", ["ordered", "hole_fill"])
def test_full_paged16_rounds(compaction):
    """The paged workload at its stated size: 16 sequences of 8K..64K rows (36 layers x
    8 KV / 32 query heads, hd 128, q8_0 K / fp16 V) in 16-row blocks in shuffled physical
    order, budget 30 %, window 512, one batched call per pass.  The initial pass and
    two steady-state rounds of 128 appended rows per sequence are each checked against
    the oracle sequence by sequence on the logical rows: every unit's kept rows within
    the cutoff band of the oracle's, and its compacted K, V and positions exactly the
    rule's rearrangement of the pre-pass rows (the ordered gather, or the hole fill of
    the GPU's own kept rows)."""
    wl = WL["paged16_qwen3_8b_q8"]
    paged_rounds(wl, synth.paged_lengths(wl), compaction, 3, DEV)


def paged_rounds(wl, lens, compaction, rounds, dev):
    """Initial pass plus rounds - 1 steady-state rounds over a paged cache, each checked
    against the oracle sequence by sequence (see test_full_paged16_rounds)."""
    budgets = [int(wl.budget_frac * x) for x in lens]
    S, W, m = wl.sink, wl.window, wl.append
    L, Hkv = wl.L, wl.Hkv
    pu.say("case paged16 %s: lengths %s" % (compaction, lens))
    stats = synth.gen_stats(L, wl.Hq, wl.hd, wl.seed)
    pg = synth.gen_paged(L, Hkv, wl.hd, wl.k_type, wl.v_type, lens, wl.seed, dev)
    ctx = pu.make_ctx(wl, stats)
    if compaction == "hole_fill":
        tria.tria_set_compaction(ctx, tria.TRIA_COMPACT_HOLE_FILL)
    names = ("k_pool", "v_pool", "pos_pool")
    bt = pg["block_table"]
    li = torch.arange(L, device=dev)[:, None, None]
    hi = torch.arange(Hkv, device=dev)[None, :, None]
    vdummy = np.zeros((1,), np.uint8)  # V is not read without compaction
    n_now = list(lens)
    st = {}
    for r in range(rounds):
        if r > 0:
            for s in range(len(lens)):
                row = synth.paged_rows(pg["pos_pool"][:1, :, :1], bt[s], n_now[s])
                last = int(row[0, 0, n_now[s] - 1])
                synth.append_paged(pg, s, n_now[s], m, last + 1, L, Hkv, wl.hd, wl.k_type,
                                   wl.v_type, 4100 + 64 * r + s)
                n_now[s] += m
        snap = {x: pg[x].clone() for x in names}
        torch.cuda.synchronize()
        pu.say("  round %d: rows %s" % (r, n_now))
        kept = tria.tria_evict_paged_batch(ctx, pg["k_pool"], pg["v_pool"], pg["pos_pool"], bt,
                                           n_now, budgets, S, W)
        tria.tria_device_status(ctx)
        nd = 0
        for s in range(len(lens)):
            n, b = n_now[s], budgets[s]
            K = oracle.kept_count(n, b, S, W)
            assert kept[s] == K
            kh = np.ascontiguousarray(pu.host(synth.paged_rows(snap["k_pool"], bt[s], n)))
            ph = np.ascontiguousarray(pu.host(synth.paged_rows(snap["pos_pool"], bt[s], n)))
            o = oracle.evict(wl.k_type, wl.v_type, L, Hkv, wl.Hq, wl.hd, wl.theta,
                             list(wl.offsets), kh, vdummy, ph, n, b, S, W, *stats,
                             want_raw=False, compact=False)
            del kh
            post = pu.host(synth.paged_rows(pg["pos_pool"], bt[s], n)[:, :, :K])
            rows = _pre_rows_of(post, ph)
            gkeep = np.sort(rows, axis=-1)
            for l in range(L):
                for h in range(Hkv):
                    nd += pu.check_kept(gkeep[l, h], o["keep_idx"][l, h], o["agg"][l, h], n, b,
                                        S, W, "round %d seq %d unit (%d,%d)" % (r, s, l, h), st)
            if compaction == "ordered":
                src = gkeep
                assert np.array_equal(rows, gkeep), "seq %d: kept rows out of order" % s
            else:
                ids = np.arange(n, dtype=np.int32)
                src = np.empty_like(gkeep)
                for l in range(L):
                    for h in range(Hkv):
                        src[l, h] = oracle.compact_holefill(ids, gkeep[l, h], n)[0][:K]
            src_t = torch.from_numpy(src).to(dev)
            for x in names:
                pre = synth.paged_rows(snap[x], bt[s], n)
                now = synth.paged_rows(pg[x], bt[s], n)[:, :, :K]
                assert torch.equal(now, pre[li, hi, src_t]), \
                    "round %d seq %d: %s is not the rule's rearrangement" % (r, s, x)
            del o, post, rows, gkeep, src, src_t
            n_now[s] = K
        del snap
        torch.cuda.empty_cache()
        pu.say("  round %d: all %d units of %d sequences within the bar; %d kept rows differ "
               "(in the cutoff band, worst %.3g of max(|tau|,1), %d outside the strict 1e-3 "
               "band)" % (r, L * Hkv * len(lens), len(lens), nd, st.get("worst_band", 0.0),
                          st.get("outside_strict", 0)))
    ctx.close()
    del pg
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# Shared keep sets (one per KV head across layers; one for the whole cache)
# ---------------------------------------------------------------------------

MODES = {oracle.KEEP_KV_HEAD: tria.TRIA_KEEP_PER_KV_HEAD, oracle.KEEP_GLOBAL: tria.TRIA_KEEP_GLOBAL}


@pytest.mark.parametrize("mode", sorted(MODES), ids=["per_kv_head", "global"])
@pytest.mark.parametrize("k_type,G", [(Q8, 4), (F16, 4), (Q8, 3)], ids=["q8_g4", "f16_g4", "q8_g3"])
def test_shared_keep_modes(mode, k_type, G):
    """Staged score -> select -> compact with a shared keep mode against the oracle's
    same mode: raw scores, group scores, kept sets (cutoff band), exact gathers; every
    member of a group holds the same kept rows; tria_evict leaves the same cache."""
    wl = variant(WL["qwen3_8b_layer_32k_f16"], name="shared", L=5, Hkv=3, Hq=3 * G,
                 k_type=k_type)
    n, B, S, W = 3000, 700, 4, 256
    pu.say("case shared mode %d k%d G%d" % (mode, k_type, G))
    case = synth.make_case(wl, device="cpu", n=n, cap=n + 3)
    stats = (case["q_re"], case["q_im"], case["w"])
    k0, v0, p0 = case["k"].numpy().copy(), case["v"].numpy().copy(), case["pos"].numpy().copy()
    ctx = pu.make_ctx(wl, stats)
    tria.tria_set_keep_mode(ctx, MODES[mode])
    a = [case[x].to(DEV) for x in ("k", "v", "pos")]
    b = [t.clone() for t in a]
    g = pu.gpu_pass(ctx, *a, n, B, S, W, wl.G)
    assert tria.tria_evict(ctx, *b, n, B, S, W) == g["K"]
    tria.tria_device_status(ctx)
    o = oracle.evict(wl.k_type, wl.v_type, wl.L, wl.Hkv, wl.Hq, wl.hd, wl.theta,
                     list(wl.offsets), k0.copy(), v0.copy(), p0.copy(), n, B, S, W, *stats,
                     compact=False, keep_mode=mode)
    nd = pu.compare_pass(g, o, n, B, S, W, "shared mode %d" % mode)
    K = g["K"]
    ka, va, pa = pu.host(a[0]), pu.host(a[1]), pu.host(a[2])
    for l in range(wl.L):
        for h in range(wl.Hkv):
            ref = g["keep"][0, h if mode == oracle.KEEP_KV_HEAD else 0]
            assert np.array_equal(g["keep"][l, h], ref), "group members differ"
            assert np.array_equal(g["agg"][l, h], g["agg"][0, h if mode == oracle.KEEP_KV_HEAD else 0])
            pu.check_gather(k0[l, h], ka[l, h], ref, K, "K")
            pu.check_gather(v0[l, h], va[l, h], ref, K, "V")
            pu.check_gather(p0[l, h], pa[l, h], ref, K, "pos")
    for x, y in zip(a, b):
        assert torch.equal(x[:, :, :K], y[:, :, :K]), "tria_evict differs from the stages"
    ctx.close()
    pu.say("  ok: kept %d, %d rows in the cutoff band differ" % (K, nd))


def test_shared_mode_one_layer_is_the_per_unit_pass():
    """With one layer the per-KV-head mode must leave exactly the per-unit result."""
    wl = variant(WL["qwen3_8b_layer_32k_f16"], name="shared1", L=1, Hkv=8, Hq=32, k_type=Q8)
    n, B, S, W = 20000, 5000, 4, 512
    case = synth.make_case(wl, device="cpu", n=n)
    stats = (case["q_re"], case["q_im"], case["w"])
    a = [case[x].to(DEV) for x in ("k", "v", "pos")]
    b = [t.clone() for t in a]
    ctx = pu.make_ctx(wl, stats)
    assert tria.tria_evict(ctx, *a, n, B, S, W) == B
    tria.tria_set_keep_mode(ctx, tria.TRIA_KEEP_PER_KV_HEAD)
    assert tria.tria_evict(ctx, *b, n, B, S, W) == B
    tria.tria_device_status(ctx)
    for x, y in zip(a, b):
        assert torch.equal(x[:, :, :B], y[:, :, :B])
    ctx.close()


def test_shared_mode_paged_batch():
    """Per-KV-head keep sets over a paged batch of sequences of different lengths."""
    wl = variant(WL["paged16_qwen3_8b_q8"], name="paged_shared", L=4, Hkv=2, Hq=8, hd=128)
    lens = [2500, 700, 64, 1800]
    budgets = [800, 200, 100, 500]
    S, W = 0, 128
    pg = synth.gen_paged(wl.L, wl.Hkv, wl.hd, wl.k_type, wl.v_type, lens, 78)
    stats = synth.gen_stats(wl.L, wl.Hq, wl.hd, 6)
    before = [(synth.paged_rows(pg["k_pool"], pg["block_table"][s], n).numpy().copy(),
               synth.paged_rows(pg["v_pool"], pg["block_table"][s], n).numpy().copy(),
               synth.paged_rows(pg["pos_pool"], pg["block_table"][s], n).numpy().copy())
              for s, n in enumerate(lens)]
    pu.say("case paged shared lens %s" % lens)
    ctx = pu.make_ctx(wl, stats)
    tria.tria_set_keep_mode(ctx, tria.TRIA_KEEP_PER_KV_HEAD)
    dev = {k: pg[k].to(DEV) for k in ("k_pool", "v_pool", "pos_pool", "block_table")}
    kept = tria.tria_evict_paged_batch(ctx, dev["k_pool"], dev["v_pool"], dev["pos_pool"],
                                       dev["block_table"], lens, budgets, S, W)
    tria.tria_device_status(ctx)
    bt = dev["block_table"].cpu()
    for s, n in enumerate(lens):
        K = oracle.kept_count(n, budgets[s], S, W)
        assert kept[s] == K
        k0, v0, p0 = before[s]
        o = oracle.evict(wl.k_type, wl.v_type, wl.L, wl.Hkv, wl.Hq, wl.hd, wl.theta,
                         list(wl.offsets), k0.copy(), v0.copy(), p0.copy(), n, budgets[s], S, W,
                         *stats, compact=False, keep_mode=oracle.KEEP_KV_HEAD)
        ka = synth.paged_rows(dev["k_pool"].cpu(), bt[s], n).numpy()
        pa = synth.paged_rows(dev["pos_pool"].cpu(), bt[s], n).numpy()
        for h in range(wl.Hkv):
            ref = pa[0, h, :K]
            for l in range(wl.L):
                keep = pa[l, h, :K]
                where = "paged shared seq %d unit (%d,%d)" % (s, l, h)
                assert np.array_equal(keep, ref), where + ": layers differ"
                pu.check_kept(keep, o["keep_idx"][l, h], o["agg"][l, h], n, budgets[s], S, W,
                              where)
                pu.check_gather(k0[l, h], ka[l, h], keep, K, where + " K")
    ctx.close()


# ---------------------------------------------------------------------------
# Hole-filling compaction (variant)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("pattern", ["random", "window_run", "all_tail", "one_hole", "invalid"])
def test_holefill_compaction_patterns(pattern):
    """tria_compact with TRIA_COMPACT_HOLE_FILL against the oracle's hole fill on the
    same kept indices, every unit, K, V and positions, bit-exact (rows >= kept are
    not compared)."""
    wl = variant(WL["qwen3_8b_layer_32k_f16"], name="hole", L=3, Hkv=2, Hq=8, k_type=Q8)
    n = 5000
    K = 1300
    rng = np.random.default_rng(hash(pattern) % 1000)
    keep = np.zeros((wl.L, wl.Hkv, K), np.int32)
    for l in range(wl.L):
        for h in range(wl.Hkv):
            if pattern == "random":
                kk = np.sort(rng.choice(n, K, replace=False))
            elif pattern == "window_run":
                kk = np.concatenate([np.sort(rng.choice(n - 500, K - 500, replace=False)),
                                     np.arange(n - 500, n)])
            elif pattern == "all_tail":
                kk = np.arange(n - K, n)
            elif pattern == "one_hole":
                kk = np.concatenate([np.arange(0, 700), np.arange(701, K + 1)])
            else:  # ascending but with entries outside [0, n) at both ends
                kk = np.sort(rng.choice(n, K, replace=False))
                kk[0] = -7
                kk[-1] = n + 40
            keep[l, h] = kk
    pu.say("case holefill pattern %s" % pattern)
    case = synth.make_case(wl, device="cpu", n=n)
    stats = (case["q_re"], case["q_im"], case["w"])
    k0, v0, p0 = case["k"].numpy().copy(), case["v"].numpy().copy(), case["pos"].numpy().copy()
    k, v, pos = case["k"].to(DEV), case["v"].to(DEV), case["pos"].to(DEV)
    ctx = pu.make_ctx(wl, stats)
    tria.tria_set_compaction(ctx, tria.TRIA_COMPACT_HOLE_FILL)
    tria.tria_compact(ctx, k, v, pos, n, torch.from_numpy(keep).to(DEV), K)
    tria.tria_device_status(ctx)
    ka, va, pa = pu.host(k), pu.host(v), pu.host(pos)
    for l in range(wl.L):
        for h in range(wl.Hkv):
            kk = keep[l, h]
            if pattern == "invalid":
                # unspecified layout, but nothing from outside the unit: every row
                # below the kept count is one of the unit's own rows, intact
                for d in range(K):
                    p = int(pa[l, h, d])
                    assert 0 <= p < n
                    assert np.array_equal(ka[l, h, d], k0[l, h, p])
                    assert np.array_equal(va[l, h, d], v0[l, h, p])
                continue
            for arr0, arr, name in ((k0, ka, "K"), (v0, va, "V"), (p0, pa, "pos")):
                want, _ = oracle.compact_holefill(arr0[l, h, :n], kk, n)
                assert np.array_equal(arr[l, h, :K], want[:K]), "%s unit (%d,%d)" % (name, l, h)
    ctx.close()


def test_holefill_paged_rounds():
    """Rounds of 'append 64 rows to every sequence, evict' on a paged batch with
    hole-filling compaction: every round the GPU's kept rows match the oracle's (cutoff
    band), and the compacted logical rows are exactly the oracle's hole fill of the
    GPU's own kept rows; the rows that moved are few once in steady state."""
    wl = variant(WL["paged16_qwen3_8b_q8"], name="paged_hole", L=3, Hkv=2, Hq=8, hd=128)
    lens = [2000, 900, 64, 1500]
    pct = 30
    S, W, m_app = 0, 128, 64
    budgets = [max(1, n * pct // 100) for n in lens]
    rounds = 4
    pg = synth.gen_paged(wl.L, wl.Hkv, wl.hd, wl.k_type, wl.v_type, lens, 79,
                         extra_blocks=(rounds * m_app) // 16 + 1)
    stats = synth.gen_stats(wl.L, wl.Hq, wl.hd, 7)
    ctx = pu.make_ctx(wl, stats)
    tria.tria_set_compaction(ctx, tria.TRIA_COMPACT_HOLE_FILL)
    dev = {k: pg[k].to(DEV) for k in ("k_pool", "v_pool", "pos_pool", "block_table")}
    n_now = list(lens)
    next_pos = list(lens)
    bt = dev["block_table"].cpu()
    moved_last = None
    for r in range(rounds):
        if r > 0:
            for s in range(len(lens)):
                synth.append_paged(dev, s, n_now[s], m_app, next_pos[s], wl.L, wl.Hkv, wl.hd,
                                   wl.k_type, wl.v_type, 900 + 10 * r + s)
                n_now[s] += m_app
                next_pos[s] += m_app
        pu.say("case paged holefill round %d n %s" % (r, n_now))
        before = []
        for s, n in enumerate(n_now):
            before.append(tuple(synth.paged_rows(dev[x].cpu(), bt[s], n).numpy().copy()
                                for x in ("k_pool", "v_pool", "pos_pool")))
        kept = tria.tria_evict_paged_batch(ctx, dev["k_pool"], dev["v_pool"], dev["pos_pool"],
                                           dev["block_table"], n_now, budgets, S, W)
        tria.tria_device_status(ctx)
        moved = 0
        for s, n in enumerate(n_now):
            K = oracle.kept_count(n, budgets[s], S, W)
            assert kept[s] == K
            k0, v0, p0 = before[s]
            o = oracle.evict(wl.k_type, wl.v_type, wl.L, wl.Hkv, wl.Hq, wl.hd, wl.theta,
                             list(wl.offsets), k0.copy(), v0.copy(), p0.copy(), n, budgets[s],
                             S, W, *stats, compact=False)
            ka = synth.paged_rows(dev["k_pool"].cpu(), bt[s], n).numpy()
            va = synth.paged_rows(dev["v_pool"].cpu(), bt[s], n).numpy()
            pa = synth.paged_rows(dev["pos_pool"].cpu(), bt[s], n).numpy()
            for l in range(wl.L):
                for h in range(wl.Hkv):
                    where = "round %d seq %d unit (%d,%d)" % (r, s, l, h)
                    row_of = {int(p): i for i, p in enumerate(p0[l, h])}
                    gkeep = np.array(sorted(row_of[int(p)] for p in pa[l, h, :K]), np.int32)
                    pu.check_kept(gkeep, o["keep_idx"][l, h], o["agg"][l, h], n, budgets[s], S,
                                  W, where)
                    if K < n:
                        for arr0, arr, name in ((k0, ka, "K"), (v0, va, "V"), (p0, pa, "pos")):
                            want, mv = oracle.compact_holefill(arr0[l, h], gkeep, n)
                            assert np.array_equal(arr[l, h, :K], want[:K]), where + " " + name
                        moved += mv
            n_now[s] = K
        pu.say("  moved rows %d" % moved)
        moved_last = moved
    # steady state: each unit moves its appended rows (in the run) plus at most as many
    # tails as holes -- far below the kept rows
    units = wl.L * wl.Hkv * sum(1 for b_, n in zip(budgets, lens) if b_ < n)
    assert moved_last <= units * (W + 4 * m_app)
    ctx.close()


def test_holefill_evict_equals_the_stages():
    wl = variant(WL["qwen3_8b_layer_32k_f16"], name="hole_stages", L=4, Hkv=4, Hq=16, k_type=Q8)
    n, B, S, W = 9000, 2000, 4, 512
    case = synth.make_case(wl, device="cpu", n=n, cap=n + 5)
    stats = (case["q_re"], case["q_im"], case["w"])
    ctx = pu.make_ctx(wl, stats)
    tria.tria_set_compaction(ctx, tria.TRIA_COMPACT_HOLE_FILL)
    a = [case[x].to(DEV) for x in ("k", "v", "pos")]
    b = [t.clone() for t in a]
    assert tria.tria_evict(ctx, *a, n, B, S, W) == B
    pu.gpu_pass(ctx, *b, n, B, S, W, wl.G)
    tria.tria_device_status(ctx)
    for x, y in zip(a, b):
        assert torch.equal(x[:, :, :B], y[:, :, :B])
    ctx.close()


# ---------------------------------------------------------------------------
# Calibration statistics
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.float32, torch.float16, torch.bfloat16],
                         ids=["f32", "f16", "bf16"])
def test_calib_stats_match_the_oracle(dtype):
    """Three layers, the tokens of each added in uneven batches from a fused buffer
    (row stride larger than the query slice); every statistic against the oracle on
    the same values.  Bar: |g - o| <= 1e-6 * max(q_abs, 1e-3) per pair (the pair
    magnitude is formed in fp32, sums in fp64, outputs rounded to fp32)."""
    L, Hq, hd = 3, 6, 64
    T = [300, 1, 517]
    rng = np.random.default_rng(60)
    pu.say("case calib %s" % dtype)
    cal = tria.TriaCalib(L, Hq, hd)
    for l in range(L):
        mean = rng.standard_normal((Hq, hd)) * 0.7
        x = (mean + rng.standard_normal((T[l], Hq, hd))).astype(np.float32)
        fused = torch.zeros(T[l], Hq * hd + 96, dtype=dtype)
        fused[:, :Hq * hd] = torch.from_numpy(x.reshape(T[l], -1)).to(dtype)
        qv = fused[:, :Hq * hd].float().numpy().reshape(T[l], Hq, hd)  # the values added
        dev = fused.to(DEV)
        cut = [0, T[l] // 3, T[l] // 3 + 1, T[l]]
        for a, b in zip(cut[:-1], cut[1:]):
            if b > a:
                cal.add(l, dev[a:b])
        assert cal.tokens(l) == T[l]
        re, im, ab, w = (pu.host(t)[l] for t in cal.finish())
        o = oracle.calib_stats(qv)
        scale = np.maximum(o[2], 1e-3)
        for g, oo, name in zip((re, im, ab, w), o, ("q_re", "q_im", "q_abs", "w")):
            err = np.abs(g.astype(np.float64) - oo)
            assert np.all(err <= 1e-6 * scale), "%s layer %d: max err %g" % (name, l, err.max())
    cal.close()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("hd,layout", [(64, "dense"), (64, "padded"), (64, "odd_layer_stride"),
                                       (36, "padded"), (128, "many_layers")])
def test_calib_add_layers_equals_per_layer_adds(dtype, hd, layout):
    """One tria_calib_add_layers call over four layers (and a two-call split of
    them) gives the statistics of four tria_calib_add calls, whatever the
    strides: dense [L, T, Hq*hd], rows and layers padded, a layer stride that is
    not a multiple of 4 elements (the element-wise kernel), and a head_dim whose
    pair count is not a multiple of 4.  The many-layer call may group the tokens
    into fewer accumulator slots, so the bar is the oracle's (1e-6 * q_abs); the
    same calls repeated give the same bits, and every layer is checked against
    the oracle."""
    # many_layers: 12 layers of 32 heads x 128, enough workgroups that the one
    # call uses fewer accumulator slots than the per-layer calls
    L, Hq, T = (12, 32, 2000) if layout == "many_layers" else (4, 6, 700)
    row = Hq * hd
    rng = np.random.default_rng(62)
    pu.say("case calib_add_layers %s hd%d %s" % (dtype, hd, layout))
    x = (rng.standard_normal((L, 1, Hq * hd)) * 0.7 +
         rng.standard_normal((L, T, Hq * hd))).astype(np.float32)
    dense = layout in ("dense", "many_layers")
    rs = row if dense else row + 40
    ls = T * rs if dense else (T + 3) * rs + (1 if layout == "odd_layer_stride" else 0)
    flat = torch.zeros(L * ls + 64, dtype=dtype)
    q = torch.as_strided(flat, (L, T, row), (ls, rs, 1))
    q.copy_(torch.from_numpy(x).to(dtype))
    qv = q.float().numpy().reshape(L, T, Hq, hd)  # the values added
    dev = flat.to(DEV)
    qd = torch.as_strided(dev, (L, T, row), (ls, rs, 1))
    per, one, split, again = (tria.TriaCalib(L, Hq, hd) for _ in range(4))
    for l in range(L):
        per.add(l, qd[l])
    one.add_layers(0, qd)
    again.add_layers(0, qd)
    split.add_layers(0, qd[:1])
    split.add_layers(1, qd[1:])
    assert [one.tokens(l) for l in range(L)] == [T] * L == [split.tokens(l) for l in range(L)]
    outs = [[pu.host(t) for t in cal.finish()] for cal in (per, one, split)]
    assert all(torch.equal(x, y) for x, y in zip(one.finish(), again.finish()))
    for l in range(L):
        o = oracle.calib_stats(qv[l])
        scale = np.maximum(o[2], 1e-3)
        for which, out in zip(("per-layer", "one call", "split"), outs):
            for g, oo, name in zip((t[l] for t in out), o, ("q_re", "q_im", "q_abs", "w")):
                err = np.abs(g.astype(np.float64) - oo)
                assert np.all(err <= 1e-6 * scale), "%s %s layer %d: max err %g" % (
                    which, name, l, err.max())
    for cal in (per, one, split, again):
        cal.close()


def test_calib_feeds_the_eviction_pass():
    """Statistics accumulated on the GPU load into a context and drive a pass that
    matches the oracle run with the same statistics."""
    wl = variant(WL["tiny_1x1_4k_f16"], name="calib_pass", L=2, Hkv=2, Hq=8, hd=128)
    rng = np.random.default_rng(61)
    cal = tria.TriaCalib(wl.L, wl.Hq, wl.hd)
    for l in range(wl.L):
        q = torch.from_numpy((rng.standard_normal((256, wl.Hq * wl.hd)) +
                              np.repeat(rng.standard_normal((1, wl.Hq * wl.hd)), 256, 0))
                             .astype(np.float32)).to(DEV)
        cal.add(l, q)
    re, im, _, w = cal.finish()
    stats = tuple(pu.host(t).astype(np.float32) for t in (re, im, w))
    n, B, S, W = 3000, 1000, 4, 256
    case = synth.make_case(wl, device="cpu", n=n)
    k0, v0, p0 = case["k"].numpy().copy(), case["v"].numpy().copy(), case["pos"].numpy().copy()
    ctx = pu.make_ctx(wl, stats)
    k, v, pos = case["k"].to(DEV), case["v"].to(DEV), case["pos"].to(DEV)
    g = pu.gpu_pass(ctx, k, v, pos, n, B, S, W, wl.G)
    o = oracle.evict(wl.k_type, wl.v_type, wl.L, wl.Hkv, wl.Hq, wl.hd, wl.theta,
                     list(wl.offsets), k0.copy(), v0.copy(), p0.copy(), n, B, S, W, *stats,
                     compact=False)
    pu.compare_pass(g, o, n, B, S, W, "calibrated stats")
    ctx.close()
    cal.close()


# ---------------------------------------------------------------------------
# Decode attention over the (compacted) cache
# ---------------------------------------------------------------------------

def _att_check(g, o, where):
    """Bar: |g - o| <= 1e-4 * max(max|o|, 1e-2) per head (fp32 scores, softmax and
    sums over up to 10^5 rows against fp64)."""
    tol = 1e-4 * max(float(np.abs(o).max()), 1e-2)
    err = float(np.abs(g.astype(np.float64) - o).max())
    assert err <= tol, "%s: max err %g > %g" % (where, err, tol)


@pytest.mark.parametrize("k_type,hd,G,n", [(Q8, 128, 4, 3000), (F16, 128, 4, 2500),
                                           (F16, 256, 4, 700), (Q8, 64, 1, 129),
                                           (F16, 96, 12, 65), (Q8, 128, 4, 1), (F16, 128, 4, 0)],
                         ids=lambda x: str(x))
def test_decode_attention_matches_the_oracle(k_type, hd, G, n):
    wl = variant(WL["qwen3_8b_layer_32k_f16"], name="att", L=2, Hkv=2, Hq=2 * G, hd=hd,
                 k_type=k_type)
    pu.say("case attention k%d hd%d G%d n%d" % (k_type, hd, G, n))
    case = synth.make_case(wl, device="cpu", n=max(n, 1))
    stats = (case["q_re"], case["q_im"], case["w"])
    rng = np.random.default_rng(80 + hd + G)
    q = rng.standard_normal((wl.L, wl.Hq, hd)).astype(np.float32)
    ctx = pu.make_ctx(wl, stats)
    k, v, pos = case["k"].to(DEV), case["v"].to(DEV), case["pos"].to(DEV)
    scale = 1.0 / np.sqrt(hd)
    out = pu.host(tria.tria_decode_attention(ctx, k, v, pos, n, torch.from_numpy(q).to(DEV)))
    kk, vv = case["k"].numpy(), case["v"].numpy()
    for l in range(wl.L):
        for g in range(wl.Hkv):
            hs = slice(g * G, g * G + G)
            if n == 0:
                assert np.all(out[l, hs] == 0.0)
                continue
            o = oracle.decode_attention_unit(k_type, wl.v_type, kk[l, g, :n], vv[l, g, :n], hd,
                                             q[l, hs], scale)
            _att_check(out[l, hs], o, "unit (%d,%d)" % (l, g))
    ctx.close()


@pytest.mark.parametrize("compaction", ["ordered", "hole_fill"])
def test_decode_attention_after_eviction(compaction):
    """Attention over the rows an eviction pass keeps equals the oracle's attention over
    exactly those rows (any order)."""
    wl = variant(WL["qwen3_8b_layer_32k_f16"], name="att_evict", L=3, Hkv=2, Hq=8, k_type=Q8)
    n, B, S, W = 6000, 1500, 4, 256
    case = synth.make_case(wl, device="cpu", n=n)
    stats = (case["q_re"], case["q_im"], case["w"])
    ctx = pu.make_ctx(wl, stats)
    if compaction == "hole_fill":
        tria.tria_set_compaction(ctx, tria.TRIA_COMPACT_HOLE_FILL)
    k, v, pos = case["k"].to(DEV), case["v"].to(DEV), case["pos"].to(DEV)
    K = tria.tria_evict(ctx, k, v, pos, n, B, S, W)
    q = np.random.default_rng(81).standard_normal((wl.L, wl.Hq, wl.hd)).astype(np.float32)
    out = pu.host(tria.tria_decode_attention(ctx, k, v, pos, K, torch.from_numpy(q).to(DEV)))
    kept = pu.host(pos)[:, :, :K]
    kk, vv = case["k"].numpy(), case["v"].numpy()
    for l in range(wl.L):
        for g in range(wl.Hkv):
            rows = kept[l, g]  # positions were 0..n-1: the kept original rows
            o = oracle.decode_attention_unit(wl.k_type, wl.v_type, kk[l, g, rows], vv[l, g, rows],
                                             wl.hd, q[l, g * wl.G:(g + 1) * wl.G],
                                             1.0 / np.sqrt(wl.hd))
            _att_check(out[l, g * wl.G:(g + 1) * wl.G], o, "%s unit (%d,%d)" % (compaction, l, g))
    ctx.close()


def test_decode_attention_paged_batch():
    wl = variant(WL["paged16_qwen3_8b_q8"], name="att_paged", L=2, Hkv=2, Hq=8, hd=128)
    lens = [1000, 17, 2100]
    pg = synth.gen_paged(wl.L, wl.Hkv, wl.hd, wl.k_type, wl.v_type, lens, 82)
    stats = synth.gen_stats(wl.L, wl.Hq, wl.hd, 8)
    ctx = pu.make_ctx(wl, stats)
    dev = {k: pg[k].to(DEV) for k in ("k_pool", "v_pool", "pos_pool", "block_table")}
    q = np.random.default_rng(83).standard_normal((len(lens), wl.L, wl.Hq, wl.hd)).astype(np.float32)
    out = pu.host(tria.tria_decode_attention_paged_batch(
        ctx, dev["k_pool"], dev["v_pool"], dev["pos_pool"], dev["block_table"], lens,
        torch.from_numpy(q).to(DEV)))
    for s, n in enumerate(lens):
        kk = synth.paged_rows(pg["k_pool"], pg["block_table"][s], n).numpy()
        vv = synth.paged_rows(pg["v_pool"], pg["block_table"][s], n).numpy()
        for l in range(wl.L):
            for g in range(wl.Hkv):
                o = oracle.decode_attention_unit(wl.k_type, wl.v_type, kk[l, g], vv[l, g], wl.hd,
                                                 q[s, l, g * wl.G:(g + 1) * wl.G],
                                                 1.0 / np.sqrt(wl.hd))
                _att_check(out[s, l, g * wl.G:(g + 1) * wl.G], o, "seq %d unit (%d,%d)" % (s, l, g))
    ctx.close()


# ---------------------------------------------------------------------------
# Decode loop: policy + passes + attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("compaction", ["ordered", "hole_fill"])
def test_decode_loop(compaction):
    """A prompt of 300 rows, then 700 decode steps appending one fresh row each with a
    threshold policy (budget 400, divide length 64, prompt protected): every pass runs
    when the policy says, keeps the rows the oracle keeps on the same input (cutoff band)
    with exact gathers, never touches the prompt rows; attention after the last step
    matches the oracle over the rows held."""
    wl = variant(WL["qwen3_8b_layer_32k_f16"], name="loop", L=2, Hkv=2, Hq=8, k_type=Q8)
    P, steps, cap = 300, 700, 1200
    pol = tria.Policy(trigger=tria.TRIA_TRIGGER_THRESHOLD, protect_prefill=1, budget=400,
                      divide_length=64, interval=1, sink=0, window=48)
    assert tria.tria_policy_peak_rows(pol, P) <= cap
    full = synth.make_case(wl, device="cpu", n=P + steps, cap=P + steps)
    stats = (full["q_re"], full["q_im"], full["w"])
    ctx = pu.make_ctx(wl, stats)
    if compaction == "hole_fill":
        tria.tria_set_compaction(ctx, tria.TRIA_COMPACT_HOLE_FILL)
    k = torch.zeros(wl.L, wl.Hkv, cap, full["k"].shape[-1], dtype=torch.uint8, device=DEV)
    v = torch.zeros(wl.L, wl.Hkv, cap, full["v"].shape[-1], dtype=torch.uint8, device=DEV)
    pos = torch.zeros(wl.L, wl.Hkv, cap, dtype=torch.int32, device=DEV)
    src = [full[x].to(DEV) for x in ("k", "v", "pos")]
    k[:, :, :P], v[:, :, :P], pos[:, :, :P] = src[0][:, :, :P], src[1][:, :, :P], src[2][:, :, :P]
    st = tria.DecodeState(n_rows=P, n_prompt=P, steps=0, passes=0)
    prompt_k = pu.host(k)[:, :, :P].copy()
    n_pass = 0
    for t in range(steps):
        n = st.n_rows
        k[:, :, n], v[:, :, n], pos[:, :, n] = src[0][:, :, P + t], src[1][:, :, P + t], src[2][:, :, P + t]
        st.n_rows += 1
        probe = tria.DecodeState(n_rows=st.n_rows, n_prompt=P, steps=st.steps + 1, passes=0)
        due = tria.tria_policy_due(pol, probe)
        before = [pu.host(x)[:, :, :st.n_rows].copy() for x in (k, v, pos)] if due else None
        rows = tria.tria_decode_step(ctx, k, v, pos, pol, st)
        if due is None:
            assert rows == probe.n_rows
            continue
        n_pass += 1
        b, s, w = due
        assert (b, s) == (400 + P, P)
        K = tria.tria_kept_count(probe.n_rows, b, s, w)
        assert rows == K == st.n_rows
        k0, v0, p0 = before
        o = oracle.evict(wl.k_type, wl.v_type, wl.L, wl.Hkv, wl.Hq, wl.hd, wl.theta,
                         list(wl.offsets), k0.copy(), v0.copy(), p0.copy(), probe.n_rows, b, s, w,
                         *stats, compact=False)
        ka, pa = pu.host(k), pu.host(pos)
        for l in range(wl.L):
            for g in range(wl.Hkv):
                row_of = {int(p): i for i, p in enumerate(p0[l, g])}
                gkeep = np.array(sorted(row_of[int(p)] for p in pa[l, g, :K]), np.int32)
                pu.check_kept(gkeep, o["keep_idx"][l, g], o["agg"][l, g], probe.n_rows, b, s, w,
                              "%s pass %d unit (%d,%d)" % (compaction, n_pass, l, g))
                assert np.array_equal(ka[l, g, :P], prompt_k[l, g])
    assert n_pass == st.passes == 1 + (steps - (400 + 64)) // 64
    q = np.random.default_rng(90).standard_normal((wl.L, wl.Hq, wl.hd)).astype(np.float32)
    out = pu.host(tria.tria_decode_attention(ctx, k, v, pos, st.n_rows, torch.from_numpy(q).to(DEV)))
    kk, vv = pu.host(k), pu.host(v)
    for l in range(wl.L):
        for g in range(wl.Hkv):
            o = oracle.decode_attention_unit(wl.k_type, wl.v_type, kk[l, g, :st.n_rows],
                                             vv[l, g, :st.n_rows], wl.hd,
                                             q[l, g * wl.G:(g + 1) * wl.G], 1.0 / np.sqrt(wl.hd))
            _att_check(out[l, g * wl.G:(g + 1) * wl.G], o, "loop attention (%d,%d)" % (l, g))
    ctx.close()


@pytest.mark.parametrize("k_type,v_type,hd", [(Q8, Q8, 128), (Q8, F16, 32), (F16, Q8, 160)],
                         ids=["q8v_hd128", "q8k_hd32", "q8v_hd160"])
def test_decode_attention_row_types(k_type, v_type, hd):
    """q8_0 values (the element-by-element V path) and the 2-byte q8_0 key path."""
    wl = variant(WL["qwen3_8b_layer_32k_f16"], name="att_types", L=1, Hkv=2, Hq=6, hd=hd,
                 k_type=k_type, v_type=v_type)
    n = 900
    pu.say("case attention types k%d v%d hd%d" % (k_type, v_type, hd))
    case = synth.make_case(wl, device="cpu", n=n)
    stats = (case["q_re"], case["q_im"], case["w"])
    q = np.random.default_rng(84 + hd).standard_normal((wl.L, wl.Hq, hd)).astype(np.float32)
    ctx = pu.make_ctx(wl, stats)
    out = pu.host(tria.tria_decode_attention(ctx, case["k"].to(DEV), case["v"].to(DEV),
                                             case["pos"].to(DEV), n, torch.from_numpy(q).to(DEV)))
    kk, vv = case["k"].numpy(), case["v"].numpy()
    for g in range(wl.Hkv):
        o = oracle.decode_attention_unit(k_type, v_type, kk[0, g, :n], vv[0, g, :n], hd,
                                         q[0, g * wl.G:(g + 1) * wl.G], 1.0 / np.sqrt(hd))
        _att_check(out[0, g * wl.G:(g + 1) * wl.G], o, "unit (0,%d)" % g)
    ctx.close()


@pytest.mark.parametrize("mode", sorted(MODES), ids=["per_kv_head", "global"])
def test_shared_keep_mode_with_hole_fill(mode):
    """Shared keep sets compacted by hole filling: every member holds the same rows in
    the same order, and the rows are exactly the oracle's hole fill of the group's kept
    rows."""
    wl = variant(WL["qwen3_8b_layer_32k_f16"], name="shared_hole", L=3, Hkv=2, Hq=8, k_type=Q8)
    n, B, S, W = 4000, 1000, 4, 128
    case = synth.make_case(wl, device="cpu", n=n)
    stats = (case["q_re"], case["q_im"], case["w"])
    k0, v0, p0 = case["k"].numpy().copy(), case["v"].numpy().copy(), case["pos"].numpy().copy()
    ctx = pu.make_ctx(wl, stats)
    tria.tria_set_keep_mode(ctx, MODES[mode])
    tria.tria_set_compaction(ctx, tria.TRIA_COMPACT_HOLE_FILL)
    k, v, pos = case["k"].to(DEV), case["v"].to(DEV), case["pos"].to(DEV)
    K = tria.tria_evict(ctx, k, v, pos, n, B, S, W)
    tria.tria_device_status(ctx)
    o = oracle.evict(wl.k_type, wl.v_type, wl.L, wl.Hkv, wl.Hq, wl.hd, wl.theta,
                     list(wl.offsets), k0.copy(), v0.copy(), p0.copy(), n, B, S, W, *stats,
                     compact=False, keep_mode=mode)
    ka, pa = pu.host(k), pu.host(pos)
    for l in range(wl.L):
        for g in range(wl.Hkv):
            ref = pa[0, g if mode == oracle.KEEP_KV_HEAD else 0, :K]
            assert np.array_equal(pa[l, g, :K], ref), "members differ"
            gkeep = np.sort(pa[l, g, :K]).astype(np.int32)  # positions were 0..n-1
            pu.check_kept(gkeep, o["keep_idx"][l, g], o["agg"][l, g], n, B, S, W,
                          "unit (%d,%d)" % (l, g))
            want, _ = oracle.compact_holefill(k0[l, g, :n], gkeep, n)
            assert np.array_equal(ka[l, g, :K], want[:K])
    ctx.close()
