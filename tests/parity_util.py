"""Helpers shared by the GPU parity tests: run the HIP library and the CPU
oracle on the same seeded bytes and compare them to the stated bar.

Bar (from the method's parity requirements):
  raw scores : |g - o| <= 1e-3 * max(|o|, rms_o)   (rms over the head's rows)
  agg        : |g - o| <= 1e-3 * max(|o|, 1); -inf exactly where the oracle has -inf
  kept sets  : same size; every row in the symmetric difference has
               |agg_o - tau| <= 2e-3 * max(|tau|, 1), tau = the oracle's cutoff
  compaction : bit-exact gather given the GPU's own kept indices
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

RAW_RTOL = 1e-3
AGG_TOL = 1e-3
CUT_TOL = 2e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    return t.detach().to("cpu").numpy()


def check_raw(g, o, where=""):
    """g: fp32 [..., n, G]; o: fp64 same shape."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    fin = np.isfinite(o)
    assert np.array_equal(np.isfinite(g), fin), where + ": non-finite pattern differs"
    oz = np.where(fin, o, 0.0)
    gz = np.where(fin, g, 0.0)
    rms = np.sqrt(np.mean(oz * oz, axis=-2, keepdims=True))
    scale = np.maximum(np.abs(oz), rms)
    err = np.abs(gz - oz)
    bad = err > RAW_RTOL * scale
    worst = float(np.max(err / np.maximum(scale, 1e-300))) if err.size else 0.0
    assert not bad.any(), "%s: %d raw scores off (worst rel %.3g)" % (where, int(bad.sum()), worst)
    return worst


def check_agg(g, o, where=""):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    ninf = np.isneginf(o)
    assert np.array_equal(np.isneginf(g), ninf), where + ": -inf pattern differs"
    fin = ~ninf
    err = np.abs(g[fin] - o[fin])
    tol = AGG_TOL * np.maximum(np.abs(o[fin]), 1.0)
    assert np.all(err <= tol), "%s: agg off by %.3g" % (where, float(np.max(err - tol)))
    return float(np.max(err / tol)) if err.size else 0.0


def cutoff(agg_o, n, budget, sink, window):
    """The oracle's cutoff score (lowest kept candidate), or None if no cut inside candidates."""
    K = oracle.kept_count(n, budget, sink, window)
    if budget >= n:
        return None
    s_end = min(sink, n)
    w_start = max(n - window, s_end)
    k = K - (s_end + n - w_start)
    cand = np.asarray(agg_o[s_end:w_start], np.float64)
    if k <= 0 or k >= len(cand):
        return None
    order = np.lexsort((np.arange(len(cand)), -cand))
    return float(cand[order[k - 1]])


def check_kept(g_keep, o_keep, agg_o, n, budget, sink, window, where="", stats=None):
    """Kept sets: same size, strictly ascending; rows in the symmetric difference lie
    inside the cutoff band.  Returns the number of differing rows.  `stats`, a dict,
    collects the worst |agg_o - tau| / max(|tau|, 1) over differing rows ("worst_band")
    and how many of them lie outside the strict band 1e-3 * max(|tau|, 1)
    ("outside_strict"): the bar's band is twice the score tolerance, and this shows how
    much of that width was used."""
    gk = np.asarray(g_keep)
    ok = np.asarray(o_keep)
    assert len(gk) == len(ok), where + ": kept size differs"
    assert np.all(np.diff(gk) > 0), where + ": kept rows not strictly ascending"
    if np.array_equal(gk, ok):
        return 0
    diff = np.setxor1d(gk, ok, assume_unique=True)
    tau = cutoff(agg_o, n, budget, sink, window)
    assert tau is not None, where + ": kept sets differ with no cutoff band"
    a = np.asarray(agg_o, np.float64)[diff]
    rel = np.abs(a - tau) / max(abs(tau), 1.0)
    worst = int(np.argmax(rel))
    assert rel[worst] <= CUT_TOL, "%s: row %d (agg %.6g) differs, cutoff %.6g" % (
        where, int(diff[worst]), float(a[worst]), tau)
    if stats is not None:
        stats["worst_band"] = max(stats.get("worst_band", 0.0), float(rel[worst]))
        stats["outside_strict"] = stats.get("outside_strict", 0) + int(np.sum(rel > AGG_TOL))
        stats["differing"] = stats.get("differing", 0) + len(diff)
    return len(diff)


def check_gather(before, after, keep, K, where=""):
    """after[:K] must equal before[keep] byte for byte (numpy uint8/int32 rows)."""
    exp = before[np.asarray(keep)]
    assert np.array_equal(after[:K], exp), where + ": compaction is not the exact gather"


def make_ctx(wl, stats, k_type=None, v_type=None, L=None, offsets=None, theta=None):
    from kv_cache_eviction_tria_amd import tria
    q_re, q_im, w = stats
    return tria.tria_load_stats(wl.L if L is None else L, wl.Hkv, wl.Hq, wl.hd,
                                wl.k_type if k_type is None else k_type,
                                wl.v_type if v_type is None else v_type,
                                wl.theta if theta is None else theta,
                                list(wl.offsets) if offsets is None else offsets, q_re, q_im, w)


def gpu_pass(ctx, k, v, pos, n, budget, sink, window, G):
    """score -> select (with agg) -> compact on device tensors; returns host results."""
    from kv_cache_eviction_tria_amd import tria
    L, Hkv = pos.shape[0], pos.shape[1]
    raw = torch.empty(L, Hkv, max(n, 1), G, dtype=torch.float32, device=pos.device)
    agg = torch.empty(L, Hkv, max(n, 1), dtype=torch.float32, device=pos.device)
    K = tria.tria_kept_count(n, budget, sink, window)
    keep = torch.empty(L, Hkv, max(K, 1), dtype=torch.int32, device=pos.device)
    tria.tria_score(ctx, k, v, pos, n, raw)
    K2 = tria.tria_select(ctx, raw, n, budget, sink, window, keep, agg)
    assert K2 == K
    # without the aggregate output the selector takes its own histogram loop where
    # every owned row exists (n a multiple of its 1024 threads): the same rows
    keep_noagg = torch.empty_like(keep)
    assert tria.tria_select(ctx, raw, n, budget, sink, window, keep_noagg) == K
    tria.tria_compact(ctx, k, v, pos, n, keep, K)
    torch.cuda.synchronize()
    assert torch.equal(keep_noagg[:, :, :K], keep[:, :, :K]), \
        "kept rows differ without the aggregate output"
    return dict(raw=host(raw)[:, :, :n], agg=host(agg)[:, :, :n], keep=host(keep)[:, :, :K], K=K)


def oracle_pass(wl, stats, k, v, pos, n, budget, sink, window, k_type=None, v_type=None,
                L=None, offsets=None, theta=None):
    q_re, q_im, w = stats
    kk, vv, pp = host(k).copy(), host(v).copy(), host(pos).copy()
    out = oracle.evict(wl.k_type if k_type is None else k_type,
                       wl.v_type if v_type is None else v_type,
                       kk.shape[0] if L is None else L, wl.Hkv, wl.Hq, wl.hd,
                       wl.theta if theta is None else theta,
                       list(wl.offsets) if offsets is None else offsets, kk, vv, pp, n, budget,
                       sink, window, q_re, q_im, w, compact=False)
    return out


def compare_pass(g, o, n, budget, sink, window, where="", stats=None):
    L, Hkv = g["raw"].shape[0], g["raw"].shape[1]
    wr = check_raw(g["raw"], o["raw"], where)
    wa = check_agg(g["agg"], o["agg"], where)
    if stats is not None:
        stats["worst_raw"] = max(stats.get("worst_raw", 0.0), wr)
        stats["worst_agg"] = max(stats.get("worst_agg", 0.0), wa)
    nd = 0
    for l in range(L):
        for h in range(Hkv):
            nd += check_kept(g["keep"][l, h], o["keep_idx"][l, h], o["agg"][l, h], n, budget,
                             sink, window, "%s unit (%d,%d)" % (where, l, h), stats)
    return nd
