"""tria_evict_noalloc (the pass on the library's fixed per-GPU scratch) against
tria_evict on the same inputs: the same kept counts and byte-identical caches,
on two calls in a row, the second with a smaller input."""
import dataclasses

import pytest
import torch

import parity_util as pu
from kv_cache_eviction_tria_amd import synth, tria

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _both(ctx, case_dev, n, B, S, W):
    """tria_evict on one copy, tria_evict_noalloc on another; compare kept rows."""
    a = [t.clone() for t in case_dev]
    b = [t.clone() for t in case_dev]
    ka = tria.tria_evict(ctx, *a, n, B, S, W)
    kb = tria.tria_evict_noalloc(ctx, *b, n, B, S, W)
    tria.tria_device_status(ctx)
    assert ka == kb == tria.tria_kept_count(n, B, S, W)
    for x, y, name in zip(a, b, ("k", "v", "pos")):
        assert torch.equal(x[:, :, :ka], y[:, :, :ka]), name
    return ka


def test_noalloc_matches_evict_on_two_calls():
    """The 36 x 8 x 32K q8_0 cache (several layer groups in the fixed scratch), then
    a smaller cache on the same context (one group)."""
    wl = synth.WORKLOADS["qwen3_8b_full_32k_q8"]
    stats = synth.gen_stats(wl.L, wl.Hq, wl.hd, wl.seed)
    ctx = pu.make_ctx(wl, stats)
    pu.say("case noalloc 36x8x32K")
    big = synth.gen_cache(wl.L, wl.Hkv, wl.hd, wl.n, wl.n, wl.k_type, wl.v_type, wl.seed, DEV)
    K = _both(ctx, big, wl.n, wl.budget, wl.sink, wl.window)
    pu.say("  kept %d, identical" % K)
    del big
    torch.cuda.empty_cache()
    pu.say("case noalloc 36x8x9000")
    small = synth.gen_cache(wl.L, wl.Hkv, wl.hd, 9100, 9000, wl.k_type, wl.v_type, 7, DEV)
    K = _both(ctx, small, 9000, 2000, 4, 256)
    pu.say("  kept %d, identical" % K)
    ctx.close()


def test_noalloc_hole_fill_and_limits():
    """Hole-filling compaction through the fixed scratch; a pass whose single layer does
    not fit, and a shared keep mode, are refused before anything is enqueued."""
    wl = dataclasses.replace(synth.WORKLOADS["qwen3_8b_full_32k_q8"], L=3)
    stats = synth.gen_stats(wl.L, wl.Hq, wl.hd, 3)
    ctx = pu.make_ctx(wl, stats)
    tria.tria_set_compaction(ctx, tria.TRIA_COMPACT_HOLE_FILL)
    pu.say("case noalloc hole fill")
    case = synth.gen_cache(wl.L, wl.Hkv, wl.hd, 5000, 5000, wl.k_type, wl.v_type, 3, DEV)
    _both(ctx, case, 5000, 1500, 0, 128)
    _both(ctx, case, 3000, 1000, 2, 64)
    tria.tria_set_compaction(ctx, tria.TRIA_COMPACT_ORDERED)
    tria.tria_set_keep_mode(ctx, tria.TRIA_KEEP_PER_KV_HEAD)
    k, v, pos = [t.clone() for t in case]
    with pytest.raises(tria.TriaError) as e:
        tria.tria_evict_noalloc(ctx, k, v, pos, 5000, 1500, 0, 128)
    assert e.value.code == tria.TRIA_E_UNSUPPORTED
    ctx.close()
    # one layer of 8 KV heads x 64 query heads x 256K rows needs 64 MiB of raw scores alone
    wl2 = dataclasses.replace(wl, L=1, Hq=64)
    n = tria.TRIA_MAX_ROWS
    pu.say("case noalloc too large: n %d G %d" % (n, wl2.G))
    ctx = pu.make_ctx(wl2, synth.gen_stats(1, 64, wl.hd, 4))
    k, v, pos = synth.gen_cache(1, wl.Hkv, wl.hd, n, n, wl.k_type, wl.v_type, 4, DEV)
    k0, v0, p0 = k.clone(), v.clone(), pos.clone()
    with pytest.raises(tria.TriaError) as e:
        tria.tria_evict_noalloc(ctx, k, v, pos, n, n // 4, 0, 512)
    assert e.value.code == tria.TRIA_E_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.equal(k, k0) and torch.equal(v, v0) and torch.equal(pos, p0)
    ctx.close()
