"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a closed form, an independent
formulation (explicit RoPE rotation matrices), brute force over tiny inputs,
an invariant, or a hand-worked fixture under tests/golden/ -- chosen so that
a dropped term, a wrong sign, a swapped pairing or a wrong reference position
fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f, parse_constant=lambda c: float(c))


def _num(x):
    return float(x) if not isinstance(x, str) else float(x.replace("inf", "inf"))


def f16_rows(x):
    return np.ascontiguousarray(np.asarray(x, np.float16)).view(np.uint8).reshape(np.shape(x)[0], -1)


# ---------------------------------------------------------------------------
# Independent formulation: explicit RoPE rotation matrices (rotate-half layout)
# ---------------------------------------------------------------------------

def rope_matrix(hd, t, theta):
    """hd x hd rotation for position t; pair f rotates (x[f], x[f+hd/2])."""
    F = hd // 2
    R = np.zeros((hd, hd))
    for f in range(F):
        ang = (theta ** (-2.0 * f / hd)) * t
        c, s = math.cos(ang), math.sin(ang)
        R[f, f] = c
        R[f, f + F] = -s
        R[f + F, f] = s
        R[f + F, f + F] = c
    return R


def explicit_trig(qbar_vec, k_rot, p, offsets, theta):
    """mean over offsets of RoPE_{p+delta}(qbar) . k_rot, as real hd-vectors."""
    hd = len(qbar_vec)
    return float(np.mean([rope_matrix(hd, p + d, theta) @ qbar_vec @ k_rot for d in offsets]))


def random_unit(rng, hd, n, G):
    F = hd // 2
    k = rng.standard_normal((n, hd)).astype(np.float16)
    q_re = rng.standard_normal((G, F)).astype(np.float32)
    q_im = rng.standard_normal((G, F)).astype(np.float32)
    w = np.abs(rng.standard_normal((G, F))).astype(np.float32)
    return k, q_re, q_im, w


# ---------------------------------------------------------------------------
# Decoding
# ---------------------------------------------------------------------------

def test_half_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.decode_rows(oracle.KV_F16, bits.view(np.uint8).reshape(1, -1), 65536)[0]
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(np.isinf(got) & (got > 0), np.isinf(ref) & (ref > 0))


def test_q8_0_decode_hand_block():
    # scale 0.5 (fp16 0x3800), q = -16..15 -> values 0.5*q
    q = np.arange(-16, 16, dtype=np.int8)
    blk = np.concatenate([np.array([0x00, 0x38], np.uint8), q.view(np.uint8)])
    got = oracle.decode_rows(oracle.KV_Q8_0, blk.reshape(1, -1), 32)[0]
    assert np.array_equal(got, 0.5 * np.arange(-16, 16))


def test_q8_0_and_f16_same_values_same_scores():
    """Values d*q with d a power of two and |q| <= 127 are exact in both encodings."""
    rng = np.random.default_rng(5)
    hd, n, G = 64, 9, 3
    q = rng.integers(-127, 128, size=(n, hd)).astype(np.int8)
    d = 2.0 ** -3
    x = d * q.astype(np.float64)
    f16 = f16_rows(x)
    q8 = np.zeros((n, 34 * hd // 32), np.uint8)
    for r in range(n):
        for b in range(hd // 32):
            q8[r, 34 * b:34 * b + 2] = np.array([d], np.float16).view(np.uint8)
            q8[r, 34 * b + 2:34 * b + 34] = q[r, 32 * b:32 * b + 32].view(np.uint8)
    _, q_re, q_im, w = random_unit(rng, hd, n, G)
    offs = [1, 2, 4, 8]
    a = oracle.raw_scores_unit(oracle.KV_F16, f16, hd, q_re, q_im, w, 1e6, 77, offs)
    b = oracle.raw_scores_unit(oracle.KV_Q8_0, q8, hd, q_re, q_im, w, 1e6, 77, offs)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# Score
# ---------------------------------------------------------------------------

def test_score_golden_2pair():
    g = _gold("score_2pair.json")
    row = f16_rows(np.array([g["row_f16"]]))
    for name, c in g["cases"].items():
        s = oracle.raw_scores_unit(oracle.KV_F16, row, g["hd"], np.array([c["q_re"]]),
                                   np.array([c["q_im"]]), np.array([c["w"]]), g["theta"], g["p"],
                                   g["offsets"])
        assert abs(s[0, 0] - c["expected"]) <= 1e-12 * max(1.0, abs(c["expected"])), name


@pytest.mark.parametrize("hd,G,n_off,theta", [(8, 1, 1, 1e4), (16, 3, 4, 1e6), (32, 4, 6, 5e5)])
def test_trig_series_equals_explicit_rope_mean(hd, G, n_off, theta):
    """Closed form: the series equals the mean over offsets of the explicitly
    RoPE-rotated mean query dotted with the stored rotated key."""
    rng = np.random.default_rng(hd + G)
    n = 13
    k, q_re, q_im, _ = random_unit(rng, hd, n, G)
    w = np.zeros_like(q_re)
    offs = sorted(rng.choice(np.arange(1, 5000), size=n_off, replace=False).tolist())
    p = 12345
    got = oracle.raw_scores_unit(oracle.KV_F16, f16_rows(k), hd, q_re, q_im, w, theta, p, offs)
    kd = k.astype(np.float64)
    for j in range(G):
        qv = np.concatenate([q_re[j], q_im[j]]).astype(np.float64)
        for r in range(n):
            ref = explicit_trig(qv, kd[r], p, offs, theta)
            assert abs(got[r, j] - ref) <= 1e-10 * max(1.0, abs(ref)), (j, r)


def test_single_offset_single_pair_is_a_cosine():
    """D={delta}, one active pair, w=0: s = |qbar||K| cos(omega(p+delta) + phi - psi)."""
    hd, theta, p, delta, f = 16, 1e6, 4000, 64, 3
    F = hd // 2
    q_re = np.zeros((1, F), np.float32)
    q_im = np.zeros((1, F), np.float32)
    q_re[0, f], q_im[0, f] = 0.75, -1.25
    row = np.zeros((1, hd))
    row[0, f], row[0, f + F] = -2.0, 0.5
    s = oracle.raw_scores_unit(oracle.KV_F16, f16_rows(row), hd, q_re, q_im, np.zeros_like(q_re),
                               theta, p, [delta])[0, 0]
    om = theta ** (-2.0 * f / hd)
    phi = math.atan2(-1.25, 0.75)
    psi = math.atan2(0.5, -2.0)
    ref = math.hypot(0.75, 1.25) * math.hypot(2.0, 0.5) * math.cos(om * (p + delta) + phi - psi)
    assert abs(s - ref) < 1e-12


def test_offset_mean_geometric_closed_form():
    """D = {1..N}: the geometric sum e^{iwp}(1/N) sum_d e^{iwd} in its stable
    Dirichlet-kernel form e^{iw(p+(N+1)/2)} sin(wN/2) / (N sin(w/2))."""
    hd, theta, p, N = 32, 1e6, 777, 50
    A = oracle.offset_mean(theta, hd, p, list(range(1, N + 1)))
    for f in range(hd // 2):
        om = theta ** (-2.0 * f / hd)
        ang = om * (p + (N + 1) / 2.0)
        mag = math.sin(om * N / 2.0) / (N * math.sin(om / 2.0))
        ref = complex(math.cos(ang), math.sin(ang)) * mag
        assert abs(A[f] - ref) < 1e-13, f


def test_shift_invariance():
    """Rotating every stored key by delta and moving p by delta leaves scores unchanged."""
    rng = np.random.default_rng(11)
    hd, G, n, theta, delta = 16, 2, 7, 1e6, 321
    k, q_re, q_im, w = random_unit(rng, hd, n, G)
    kd = k.astype(np.float64)
    R = rope_matrix(hd, delta, theta)
    k_shift = (R @ kd.T).T
    offs = [1, 3, 9]
    # Rotated keys are not exactly representable in fp16, so the oracle scores the
    # original keys at p and the explicit form scores the rotated keys at p + delta.
    base = oracle.raw_scores_unit(oracle.KV_F16, f16_rows(kd), hd, q_re, q_im, w, theta, 1000,
                                  offs)
    for j in range(G):
        qv = np.concatenate([q_re[j], q_im[j]]).astype(np.float64)
        for r in range(n):
            trig = explicit_trig(qv, k_shift[r], 1000 + delta, offs, theta)
            norm = float(np.sum(w[j] * np.hypot(k_shift[r, :hd // 2], k_shift[r, hd // 2:])))
            assert abs(base[r, j] - (trig + norm)) < 1e-10 * max(1, abs(base[r, j]))


def test_unrotate_formulation_matches_direct():
    """Older form: unrotate each key by its own position t, then apply the relative
    phase (p + delta - t) -- identical to the direct K_rot score when positions are exact."""
    rng = np.random.default_rng(3)
    hd, G, n, theta = 16, 2, 9, 1e6
    k, q_re, q_im, w = random_unit(rng, hd, n, G)
    kd = k.astype(np.float64)
    pos = np.sort(rng.choice(np.arange(0, 3000), size=n, replace=False))
    p = int(pos[-1])
    offs = [1, 2, 4, 8, 16]
    got = oracle.raw_scores_unit(oracle.KV_F16, f16_rows(kd), hd, q_re, q_im, w, theta, p, offs)
    for j in range(G):
        qv = np.concatenate([q_re[j], q_im[j]]).astype(np.float64)
        for r in range(n):
            t = int(pos[r])
            k_pre = rope_matrix(hd, -t, theta) @ kd[r]
            trig = float(np.mean([rope_matrix(hd, p + d - t, theta) @ qv @ k_pre for d in offs]))
            norm = float(np.sum(w[j] * np.hypot(kd[r, :hd // 2], kd[r, hd // 2:])))
            assert abs(got[r, j] - (trig + norm)) < 1e-9 * max(1, abs(got[r, j]))


def test_evict_uses_absolute_position_not_row_count():
    """After a compaction the newest row's position exceeds the row count; the pass must
    phase with pos[n-1] (the worklog's later-compaction fix), which differs from n-1."""
    rng = np.random.default_rng(8)
    L, Hkv, Hq, hd, n = 1, 1, 2, 16, 12
    k, q_re, q_im, w = random_unit(rng, hd, n, Hq)
    pos = np.sort(rng.choice(np.arange(0, 500), size=n, replace=False)).astype(np.int32)
    offs = [1, 2, 4]
    kb = f16_rows(k).reshape(L, Hkv, n, -1).copy()
    vb = kb.copy()
    out = oracle.evict(oracle.KV_F16, oracle.KV_F16, L, Hkv, Hq, hd, 1e6, offs, kb, vb,
                       pos.reshape(L, Hkv, n).copy(), n, 6, 0, 2, q_re.reshape(1, Hq, -1),
                       q_im.reshape(1, Hq, -1), w.reshape(1, Hq, -1), compact=False)
    kd = k.astype(np.float64)
    wrong_differs = False
    for j in range(Hq):
        qv = np.concatenate([q_re[j], q_im[j]]).astype(np.float64)
        for r in range(n):
            norm = float(np.sum(w[j] * np.hypot(kd[r, :hd // 2], kd[r, hd // 2:])))
            good = explicit_trig(qv, kd[r], int(pos[-1]), offs, 1e6) + norm
            bad = explicit_trig(qv, kd[r], n - 1, offs, 1e6) + norm
            assert abs(out["raw"][0, 0, r, j] - good) < 1e-9 * max(1, abs(good))
            wrong_differs |= abs(bad - good) > 1e-3
    assert wrong_differs


def test_evict_head_grouping_and_layer_offsets():
    """Query head h = g*G + j scores KV head g of the same layer."""
    rng = np.random.default_rng(21)
    L, Hkv, Hq, hd, n = 2, 3, 6, 16, 5
    G = Hq // Hkv
    F = hd // 2
    kd = rng.standard_normal((L, Hkv, n, hd)).astype(np.float16)
    q_re = rng.standard_normal((L, Hq, F)).astype(np.float32)
    q_im = rng.standard_normal((L, Hq, F)).astype(np.float32)
    w = np.abs(rng.standard_normal((L, Hq, F))).astype(np.float32)
    kb = np.ascontiguousarray(kd).view(np.uint8).reshape(L, Hkv, n, 2 * hd).copy()
    pos = np.broadcast_to(np.arange(n, dtype=np.int32), (L, Hkv, n)).copy()
    offs = [1, 8]
    out = oracle.evict(oracle.KV_F16, oracle.KV_F16, L, Hkv, Hq, hd, 1e6, offs, kb, kb.copy(),
                       pos, n, n, 0, 0, q_re, q_im, w, compact=False)
    for l in range(L):
        for g in range(Hkv):
            for j in range(G):
                h = g * G + j
                qv = np.concatenate([q_re[l, h], q_im[l, h]]).astype(np.float64)
                for r in range(n):
                    k_r = kd[l, g, r].astype(np.float64)
                    ref = explicit_trig(qv, k_r, n - 1, offs, 1e6) + float(
                        np.sum(w[l, h] * np.hypot(k_r[:F], k_r[F:])))
                    assert abs(out["raw"][l, g, r, j] - ref) < 1e-9 * max(1, abs(ref))


# ---------------------------------------------------------------------------
# Aggregation
# ---------------------------------------------------------------------------

def test_aggregate_golden():
    g = _gold("aggregate_small.json")
    for c in g["cases"]:
        raw = np.array([[_num(x) for x in row] for row in c["raw"]], np.float64)
        agg, _, _ = oracle.aggregate_unit(raw)
        exp = np.array([_num(x) for x in c["agg"]])
        assert np.array_equal(np.isneginf(agg), np.isneginf(exp)), c["name"]
        fin = np.isfinite(exp)
        assert np.allclose(agg[fin], exp[fin], rtol=0, atol=1e-12), c["name"]


def test_aggregate_head_scale_invariance():
    """z-normalisation is invariant to scaling one head's scores by c > 0 and to a shift."""
    rng = np.random.default_rng(2)
    raw = rng.standard_normal((200, 4)) * [1, 2, 3, 4] + [5, -1, 0, 2]
    a0, _, _ = oracle.aggregate_unit(raw)
    raw2 = raw.copy()
    raw2[:, 2] = raw2[:, 2] * 7.5 - 3.0
    a1, _, _ = oracle.aggregate_unit(raw2)
    assert np.allclose(a0, a1, atol=1e-12)


def test_aggregate_population_moments():
    raw = np.array([[2.0], [4.0], [4.0], [4.0], [5.0], [5.0], [7.0], [9.0]])
    _, mu, sg = oracle.aggregate_unit(raw)
    assert mu[0] == 5.0 and sg[0] == 2.0  # textbook population example


# ---------------------------------------------------------------------------
# Selection
# ---------------------------------------------------------------------------

def brute_keep(agg, budget, sink, window):
    """Independent rank-count definition (no sorting)."""
    n = len(agg)
    if budget >= n:
        return list(range(n))
    prot = [r < sink or r >= n - window for r in range(n)]
    K = max(budget, sum(prot))
    k = K - sum(prot)
    cand = [r for r in range(n) if not prot[r]]
    keep = []
    for r in range(n):
        if prot[r]:
            keep.append(r)
            continue
        better = sum(1 for c in cand if agg[c] > agg[r] or (agg[c] == agg[r] and c < r))
        if better < k:
            keep.append(r)
    return keep


def test_select_golden():
    g = _gold("select_small.json")
    for c in g["cases"]:
        agg = np.array([_num(x) for x in c["agg"]])
        got = oracle.select_unit(agg, c["budget"], c["sink"], c["window"])
        assert got.tolist() == c["keep"], c["name"]


def test_kept_count_matches_worklog_schedule():
    g = _gold("schedule_worklog.json")
    for c in g["cases"]:
        assert oracle.kept_count(c["n"], c["budget"], c["sink"], c["window"]) == c["kept"]
    # every later pass sees the same row count (budget + divide length) again
    assert g["rows_before_each"] == g["cases"][0]["kept"] + 128


def test_select_brute_force_all_small_n():
    rng = np.random.default_rng(0)
    for n in range(0, 13):
        for _ in range(40):
            agg = rng.integers(0, 4, size=n).astype(np.float64)  # many ties
            if n and rng.random() < 0.3:
                agg[rng.integers(0, n)] = -np.inf
            budget = int(rng.integers(0, n + 2))
            sink = int(rng.integers(0, 4))
            window = int(rng.integers(0, 5))
            got = oracle.select_unit(agg, budget, sink, window)
            assert got.tolist() == brute_keep(agg.tolist(), budget, sink, window)


def test_select_invariants():
    rng = np.random.default_rng(1)
    n = 300
    agg = rng.standard_normal(n)
    prev = None
    for budget in range(0, n + 3):
        keep = oracle.select_unit(agg, budget, 4, 17)
        prot = set(range(4)) | set(range(n - 17, n))
        assert prot <= set(keep.tolist())
        assert len(keep) == min(n, max(budget, len(prot)))
        assert np.all(np.diff(keep) > 0)
        if prev is not None:
            assert set(prev.tolist()) <= set(keep.tolist())  # nested in the budget
        prev = keep
    assert oracle.select_unit(agg, n, 0, 0).tolist() == list(range(n))


def test_g1_keeps_topk_of_raw():
    """With one query head, z-normalisation is monotone: keep = top-k of the raw score."""
    rng = np.random.default_rng(4)
    raw = rng.standard_normal((100, 1)) * 3 + 1
    agg, _, _ = oracle.aggregate_unit(raw)
    keep = oracle.select_unit(agg, 30, 0, 0)
    order = sorted(range(100), key=lambda r: (-raw[r, 0], r))[:30]
    assert keep.tolist() == sorted(order)


def test_scaling_one_heads_stats_keeps_the_same_rows():
    rng = np.random.default_rng(6)
    hd, G, n = 32, 4, 64
    k, q_re, q_im, w = random_unit(rng, hd, n, G)
    offs = [1, 2, 4, 8]
    raw0 = oracle.raw_scores_unit(oracle.KV_F16, f16_rows(k), hd, q_re, q_im, w, 1e6, 63, offs)
    q_re2, q_im2, w2 = q_re.copy(), q_im.copy(), w.copy()
    q_re2[1] *= 3.0
    q_im2[1] *= 3.0
    w2[1] *= 3.0
    raw1 = oracle.raw_scores_unit(oracle.KV_F16, f16_rows(k), hd, q_re2, q_im2, w2, 1e6, 63, offs)
    a0, _, _ = oracle.aggregate_unit(raw0)
    a1, _, _ = oracle.aggregate_unit(raw1)
    assert oracle.select_unit(a0, 20, 2, 8).tolist() == oracle.select_unit(a1, 20, 2, 8).tolist()


# ---------------------------------------------------------------------------
# Compaction
# ---------------------------------------------------------------------------

def test_compaction_is_exact_gather():
    rng = np.random.default_rng(9)
    rows = rng.integers(0, 256, size=(50, 136), dtype=np.uint8)
    keep = np.sort(rng.choice(50, size=17, replace=False)).astype(np.int32)
    out = oracle.compact_rows(rows, keep)
    assert np.array_equal(out[:17], rows[keep])
    assert np.array_equal(out[17:], rows[17:])


def test_evict_end_to_end_small():
    """Whole pass on a small contiguous cache: keep sets from the composed unit steps,
    compacted rows are the exact gather, positions stay strictly ascending."""
    rng = np.random.default_rng(10)
    L, Hkv, Hq, hd, n = 2, 2, 4, 32, 40
    F = hd // 2
    kd = rng.standard_normal((L, Hkv, n, hd)).astype(np.float16)
    kb = np.ascontiguousarray(kd).view(np.uint8).reshape(L, Hkv, n, 2 * hd).copy()
    vb = rng.integers(0, 256, size=(L, Hkv, n, 2 * hd), dtype=np.uint8)
    pos = np.broadcast_to(np.arange(n, dtype=np.int32) * 3, (L, Hkv, n)).copy()
    q_re = rng.standard_normal((L, Hq, F)).astype(np.float32)
    q_im = rng.standard_normal((L, Hq, F)).astype(np.float32)
    w = np.abs(rng.standard_normal((L, Hq, F))).astype(np.float32)
    offs = [1, 2, 4]
    k0, v0, p0 = kb.copy(), vb.copy(), pos.copy()
    out = oracle.evict(oracle.KV_F16, oracle.KV_F16, L, Hkv, Hq, hd, 1e6, offs, kb, vb, pos, n,
                       15, 2, 5, q_re, q_im, w)
    K = out["kept"]
    assert K == 15
    for l in range(L):
        for g in range(Hkv):
            G = Hq // Hkv
            st = slice(g * G, g * G + G)
            raw = oracle.raw_scores_unit(oracle.KV_F16, k0[l, g], hd, q_re[l, st], q_im[l, st],
                                         w[l, st], 1e6, int(p0[l, g, -1]), offs)
            agg, _, _ = oracle.aggregate_unit(raw)
            keep = oracle.select_unit(agg, 15, 2, 5)
            assert keep.tolist() == out["keep_idx"][l, g].tolist()
            assert np.array_equal(kb[l, g, :K], k0[l, g, keep])
            assert np.array_equal(vb[l, g, :K], v0[l, g, keep])
            assert np.array_equal(pos[l, g, :K], p0[l, g, keep])
            assert np.all(np.diff(pos[l, g, :K]) > 0)


# ---------------------------------------------------------------------------
# Shared keep sets (one per KV head across layers; one for the whole cache)
# ---------------------------------------------------------------------------

def _shared_case(seed, L, Hkv, Hq, hd, n):
    rng = np.random.default_rng(seed)
    F = hd // 2
    kd = rng.standard_normal((L, Hkv, n, hd)).astype(np.float16)
    kb = np.ascontiguousarray(kd).view(np.uint8).reshape(L, Hkv, n, 2 * hd).copy()
    vb = rng.integers(0, 256, size=(L, Hkv, n, 2 * hd), dtype=np.uint8)
    pos = np.broadcast_to(np.arange(n, dtype=np.int32), (L, Hkv, n)).copy()
    q_re = rng.standard_normal((L, Hq, F)).astype(np.float32)
    q_im = rng.standard_normal((L, Hq, F)).astype(np.float32)
    w = np.abs(rng.standard_normal((L, Hq, F))).astype(np.float32)
    return kb, vb, pos, q_re, q_im, w


def _shared_evict(case, L, Hkv, Hq, hd, n, budget, sink, window, mode, compact=True):
    kb, vb, pos, q_re, q_im, w = (x.copy() for x in case)
    out = oracle.evict(oracle.KV_F16, oracle.KV_F16, L, Hkv, Hq, hd, 1e6, [1, 4, 16], kb, vb, pos,
                       n, budget, sink, window, q_re, q_im, w, compact=compact, keep_mode=mode)
    return out, kb, vb, pos


def test_shared_modes_reduce_to_per_unit():
    """One layer: the per-KV-head mode is the per-unit mode.  One KV head: the global
    mode is the per-KV-head mode.  One unit: all three agree."""
    case = _shared_case(31, 1, 3, 6, 16, 60)
    a, *ca = _shared_evict(case, 1, 3, 6, 16, 60, 20, 2, 6, oracle.KEEP_UNIT)
    b, *cb = _shared_evict(case, 1, 3, 6, 16, 60, 20, 2, 6, oracle.KEEP_KV_HEAD)
    assert np.array_equal(a["keep_idx"], b["keep_idx"]) and np.array_equal(a["agg"], b["agg"])
    assert all(np.array_equal(x, y) for x, y in zip(ca, cb))
    case = _shared_case(32, 3, 1, 2, 16, 60)
    b, *cb = _shared_evict(case, 3, 1, 2, 16, 60, 20, 2, 6, oracle.KEEP_KV_HEAD)
    c, *cc = _shared_evict(case, 3, 1, 2, 16, 60, 20, 2, 6, oracle.KEEP_GLOBAL)
    assert np.array_equal(b["keep_idx"], c["keep_idx"]) and np.array_equal(b["agg"], c["agg"])
    assert all(np.array_equal(x, y) for x, y in zip(cb, cc))
    case = _shared_case(33, 1, 1, 4, 16, 60)
    a, *_ = _shared_evict(case, 1, 1, 4, 16, 60, 20, 2, 6, oracle.KEEP_UNIT)
    c, *_ = _shared_evict(case, 1, 1, 4, 16, 60, 20, 2, 6, oracle.KEEP_GLOBAL)
    assert np.array_equal(a["keep_idx"], c["keep_idx"])


def test_shared_group_score_is_the_max_over_members():
    """A layer whose keys are all equal has sigma = 0, so its z-scores are 0: the group
    score of the two-layer KV head is max(z_layer0, 0), not a mean or a sum (those would
    keep layer 0's order below zero; the max ties every such row at 0, and ties go to
    the lower row).  The budget reaches below zero, where the two readings part."""
    L, Hkv, Hq, hd, n = 2, 1, 2, 16, 80
    case = list(_shared_case(34, L, Hkv, Hq, hd, n))
    case[0][1] = case[0][1][:, :1]  # layer 1: every key row the same
    out, *_ = _shared_evict(case, L, Hkv, Hq, hd, n, 60, 3, 8, oracle.KEEP_KV_HEAD,
                            compact=False)
    unit, *_ = _shared_evict(case, L, Hkv, Hq, hd, n, 60, 3, 8, oracle.KEEP_UNIT, compact=False)
    z0 = unit["agg"][0, 0]
    assert np.all(unit["agg"][1, 0] == 0.0)
    want = np.maximum(z0, 0.0)
    assert np.allclose(out["agg"][0, 0], want, rtol=0, atol=0)
    keep = brute_keep(want, 60, 3, 8)
    assert out["keep_idx"][0, 0].tolist() == keep and out["keep_idx"][1, 0].tolist() == keep
    # a mean over the layers would give another keep set on this input
    assert brute_keep(z0 / 2, 60, 3, 8) != keep


def test_shared_nonfinite_score_evicts_the_row_in_every_layer():
    L, Hkv, Hq, hd, n = 3, 2, 4, 16, 50
    case = list(_shared_case(35, L, Hkv, Hq, hd, n))
    k16 = case[0].view(np.float16).reshape(L, Hkv, n, hd)
    k16[2, 1, 20, 3] = np.float16(np.inf)  # one key element of layer 2, KV head 1, row 20
    for mode, groups in ((oracle.KEEP_KV_HEAD, [(g,) for g in range(Hkv)]),
                         (oracle.KEEP_GLOBAL, [tuple(range(Hkv))])):
        out, *_ = _shared_evict(case, L, Hkv, Hq, hd, n, 40, 2, 4, mode, compact=False)
        for grp in groups:
            hit = 1 in grp
            for l in range(L):
                for g in grp:
                    assert (out["agg"][l, g, 20] == -np.inf) == hit
                    assert (20 in out["keep_idx"][l, g]) == (not hit)


def test_shared_members_share_keep_sets_and_gather_exactly():
    L, Hkv, Hq, hd, n = 3, 2, 4, 16, 70
    case = _shared_case(36, L, Hkv, Hq, hd, n)
    kb0, vb0, p0 = case[0], case[1], case[2]
    for mode in (oracle.KEEP_KV_HEAD, oracle.KEEP_GLOBAL):
        out, kb, vb, pos = _shared_evict(case, L, Hkv, Hq, hd, n, 25, 2, 5, mode)
        K = out["kept"]
        for l in range(L):
            for g in range(Hkv):
                ref = out["keep_idx"][0, g if mode == oracle.KEEP_KV_HEAD else 0]
                keep = out["keep_idx"][l, g]
                assert np.array_equal(keep, ref)
                assert np.array_equal(kb[l, g, :K], kb0[l, g, keep])
                assert np.array_equal(vb[l, g, :K], vb0[l, g, keep])
                assert np.array_equal(pos[l, g, :K], p0[l, g, keep])
                assert keep.tolist() == brute_keep(out["agg"][l, g], 25, 2, 5)


def test_shared_layer_order_does_not_matter():
    L, Hkv, Hq, hd, n = 4, 2, 4, 16, 64
    case = _shared_case(37, L, Hkv, Hq, hd, n)
    perm = [2, 0, 3, 1]
    pcase = [x[perm].copy() for x in case]
    for mode in (oracle.KEEP_KV_HEAD, oracle.KEEP_GLOBAL):
        a, *_ = _shared_evict(case, L, Hkv, Hq, hd, n, 20, 1, 4, mode, compact=False)
        b, *_ = _shared_evict(pcase, L, Hkv, Hq, hd, n, 20, 1, 4, mode, compact=False)
        assert np.array_equal(a["keep_idx"][perm], b["keep_idx"])
        assert np.array_equal(a["agg"][perm], b["agg"])


# ---------------------------------------------------------------------------
# Hole-filling compaction (variant)
# ---------------------------------------------------------------------------

def test_holefill_layout_rules():
    """Rows [0, K) hold exactly the kept rows; kept rows below the trailing run do not
    move; the trailing run of kept rows ends at row K-1 in its order; every moved row
    is a hole below the run or a row of the run."""
    rng = np.random.default_rng(40)
    for trial in range(300):
        n = int(rng.integers(2, 90))
        K = int(rng.integers(1, n + 1))
        keep = np.sort(rng.choice(n, K, replace=False)).astype(np.int32)
        if trial % 3 == 0:  # a protected-window-like run at the end
            run = int(rng.integers(1, K + 1))
            rest = np.sort(rng.choice(n - run, K - run, replace=False))
            keep = np.concatenate([rest, np.arange(n - run, n)]).astype(np.int32)
        rows = np.arange(n, dtype=np.int64) * 7 + 3
        out, moves = oracle.compact_holefill(rows, keep, n)
        if K == n:
            assert moves == 0 and np.array_equal(out, rows)
            continue
        assert sorted(out[:K].tolist()) == sorted(rows[keep].tolist())
        run = 0
        while run < K and keep[K - 1 - run] == n - 1 - run:
            run += 1
        lim = K - run
        assert np.array_equal(out[lim:K], rows[n - run:n])
        kept_low = keep[keep < lim]
        assert np.array_equal(out[kept_low], rows[kept_low])
        holes = sorted(set(range(lim)) - set(kept_low.tolist()))
        tails = [r for r in keep[:K - run] if r >= lim]
        assert len(holes) == len(tails)
        assert [out[h] for h in holes] == [rows[t] for t in tails]
        assert moves == len(tails) + (run if n > K else 0)


def _rounds(mode, rounds, seed, L=2, Hkv=2, Hq=4, hd=32, n0=300, budget=120, sink=4,
            window=40, append=24):
    """Rounds of 'append `append` fresh rows, evict to the budget' on a contiguous cache;
    returns the kept positions (as sets per unit) and the moved rows of every round."""
    rng = np.random.default_rng(seed)
    F = hd // 2
    cap = n0 + rounds * append
    q_re = rng.standard_normal((L, Hq, F)).astype(np.float32)
    q_im = rng.standard_normal((L, Hq, F)).astype(np.float32)
    w = np.abs(rng.standard_normal((L, Hq, F))).astype(np.float32)
    fresh = rng.standard_normal((L, Hkv, cap, hd)).astype(np.float16)
    k = np.zeros((L, Hkv, cap, 2 * hd), np.uint8)
    v = np.zeros((L, Hkv, cap, 2 * hd), np.uint8)
    pos = np.zeros((L, Hkv, cap), np.int32)
    k[:, :, :n0] = fresh[:, :, :n0].view(np.uint8).reshape(L, Hkv, n0, 2 * hd)
    v[:, :, :n0] = k[:, :, :n0] ^ 0x5A
    pos[:, :, :n0] = np.arange(n0)
    n, nxt, out = n0, n0, []
    for r in range(rounds):
        if r > 0:  # append fresh rows at the next positions
            sl = slice(n, n + append)
            k[:, :, sl] = fresh[:, :, nxt:nxt + append].view(np.uint8).reshape(L, Hkv, append, 2 * hd)
            v[:, :, sl] = k[:, :, sl] ^ 0x5A
            pos[:, :, sl] = np.arange(nxt, nxt + append)
            n += append
            nxt += append
        before = pos.copy()
        o = oracle.evict(oracle.KV_F16, oracle.KV_F16, L, Hkv, Hq, hd, 1e6, [1, 8, 64], k, v, pos,
                         n, budget, sink, window, q_re, q_im, w, compact_mode=mode)
        K = o["kept"]
        # every kept row carries its own K and V bytes
        for l in range(L):
            for g in range(Hkv):
                p = pos[l, g, :K]
                assert np.array_equal(k[l, g, :K], fresh[l, g, p].view(np.uint8).reshape(K, 2 * hd))
                assert np.array_equal(v[l, g, :K], k[l, g, :K] ^ 0x5A)
        moved = int((pos[:, :, :K] != before[:, :, :K]).sum())
        out.append(([set(pos[l, g, :K].tolist()) for l in range(L) for g in range(Hkv)], moved))
        n = K
    return out


def test_holefill_rounds_keep_the_same_tokens_as_the_ordered_gather():
    """Sinks stay first and the newest rows stay last, so every round protects the same
    tokens and scores them the same: with continuous scores (no ties at the cutoff) the
    kept positions equal the order-preserving pass's, round after round, while the
    variant moves far fewer rows once the cache is in steady state."""
    a = _rounds(oracle.COMPACT_ORDERED, 8, 41)
    b = _rounds(oracle.COMPACT_HOLEFILL, 8, 41)
    for (sa, ma), (sb, mb) in zip(a, b):
        assert sa == sb
    steady_a = sum(m for _, m in a[2:])
    steady_b = sum(m for _, m in b[2:])
    assert steady_b * 2 < steady_a, (steady_a, steady_b)


# ---------------------------------------------------------------------------
# Calibration statistics
# ---------------------------------------------------------------------------

def test_calib_constant_stream():
    """Every token the same: the mean is that query, q_abs its magnitude, w = 0."""
    rng = np.random.default_rng(50)
    q1 = rng.standard_normal((3, 16))
    q = np.broadcast_to(q1, (37, 3, 16)).copy()
    re, im, ab, w = oracle.calib_stats(q)
    assert np.allclose(re, q1[:, :8], atol=1e-15) and np.allclose(im, q1[:, 8:], atol=1e-15)
    assert np.allclose(ab, np.hypot(q1[:, :8], q1[:, 8:]), rtol=1e-15)
    assert np.allclose(w, 0.0, atol=1e-14)


def test_calib_rotating_pair_cancels():
    """A pair of fixed length A whose phase turns by 2 pi / T per token: the mean is
    0, q_abs = A and w = A (the directions cancel exactly)."""
    T, A = 64, 2.5
    t = np.arange(T)
    q = np.zeros((T, 1, 4))
    q[:, 0, 0] = A * np.cos(2 * np.pi * t / T)
    q[:, 0, 2] = A * np.sin(2 * np.pi * t / T)
    q[:, 0, 1] = 1.0  # second pair: constant (1, 0)
    re, im, ab, w = oracle.calib_stats(q)
    assert abs(re[0, 0]) < 1e-13 and abs(im[0, 0]) < 1e-13
    assert abs(ab[0, 0] - A) < 1e-13 and abs(w[0, 0] - A) < 1e-12
    assert re[0, 1] == 1.0 and im[0, 1] == 0.0 and w[0, 1] == 0.0


def test_calib_opposite_halves_and_scaling():
    """Half the tokens c, half -c: mean 0, w = |c|.  Scaling the stream by s scales
    the mean by s and q_abs and w by |s|; w is never negative (triangle inequality)."""
    c = np.array([[0.3, -1.2, 0.7, 2.0]])
    q = np.concatenate([np.broadcast_to(c, (10, 1, 4)), np.broadcast_to(-c, (10, 1, 4))])
    re, im, ab, w = oracle.calib_stats(q)
    mag = np.hypot(c[0, :2], c[0, 2:])
    assert np.allclose(re, 0, atol=1e-15) and np.allclose(w[0], mag, rtol=1e-14)
    rng = np.random.default_rng(51)
    q = rng.standard_normal((200, 5, 32)) + 0.4
    a = oracle.calib_stats(q)
    b = oracle.calib_stats(-3.0 * q)
    assert np.allclose(b[0], -3.0 * a[0], rtol=1e-12) and np.allclose(b[1], -3.0 * a[1], rtol=1e-12)
    assert np.allclose(b[2], 3.0 * a[2], rtol=1e-12) and np.allclose(b[3], 3.0 * a[3], rtol=1e-11)
    assert np.all(a[3] >= -1e-15)


# ---------------------------------------------------------------------------
# Decode attention
# ---------------------------------------------------------------------------

def _rows_f16(x):
    return np.ascontiguousarray(x.astype(np.float16)).view(np.uint8).reshape(x.shape[0], -1)


def test_attention_equal_keys_average_the_values():
    """Every key the same: uniform weights, the output is the mean of V (any scale)."""
    rng = np.random.default_rng(70)
    hd, n = 32, 37
    k = np.broadcast_to(rng.standard_normal(hd), (n, hd))
    v = rng.standard_normal((n, hd)).astype(np.float16)
    q = rng.standard_normal((3, hd))
    out = oracle.decode_attention_unit(oracle.KV_F16, oracle.KV_F16, _rows_f16(k), _rows_f16(v),
                                       hd, q, 0.7)
    want = v.astype(np.float64).mean(axis=0)
    assert np.allclose(out, np.broadcast_to(want, out.shape), atol=1e-12)


def test_attention_two_rows_closed_form_and_order():
    """Two rows: weights are a logistic function of the score gap; permuting the rows
    (a compaction's order) changes nothing; a dominant key returns its own V."""
    hd = 16
    k = np.zeros((2, hd)); k[0, 0] = 1.0; k[1, 1] = 1.0
    v = np.zeros((2, hd)); v[0, :] = 2.0; v[1, :] = -1.0
    q = np.zeros((1, hd)); q[0, 0] = 3.0; q[0, 1] = 1.0
    sc = 0.5
    out = oracle.decode_attention_unit(oracle.KV_F16, oracle.KV_F16, _rows_f16(k), _rows_f16(v),
                                       hd, q, sc)
    p0 = 1.0 / (1.0 + np.exp(-sc * (3.0 - 1.0)))
    assert np.allclose(out[0], p0 * 2.0 + (1 - p0) * -1.0, atol=1e-14)
    outp = oracle.decode_attention_unit(oracle.KV_F16, oracle.KV_F16, _rows_f16(k[::-1]),
                                        _rows_f16(v[::-1]), hd, q, sc)
    assert np.allclose(out, outp, atol=1e-15)
    big = oracle.decode_attention_unit(oracle.KV_F16, oracle.KV_F16, _rows_f16(k), _rows_f16(v),
                                       hd, q * 200.0, sc)
    assert np.allclose(big[0], 2.0, atol=1e-12)


def test_attention_q8_rows_equal_the_decoded_fp16_rows():
    """q8_0 keys holding values that fp16 also represents exactly give the same output
    as the fp16 rows."""
    rng = np.random.default_rng(71)
    hd, n = 64, 20
    d = np.float16(0.125)
    qv = rng.integers(-100, 101, size=(n, hd)).astype(np.int8)
    blocks = []
    for r in range(n):
        row = b""
        for b_ in range(hd // 32):
            row += np.array([d]).view(np.uint8).tobytes() + qv[r, 32 * b_:32 * b_ + 32].tobytes()
        blocks.append(np.frombuffer(row, np.uint8))
    k8 = np.stack(blocks)
    k16 = _rows_f16(qv.astype(np.float64) * 0.125)
    v = _rows_f16(rng.standard_normal((n, hd)))
    q = rng.standard_normal((2, hd))
    a = oracle.decode_attention_unit(oracle.KV_Q8_0, oracle.KV_F16, k8, v, hd, q, 0.1)
    b = oracle.decode_attention_unit(oracle.KV_F16, oracle.KV_F16, k16, v, hd, q, 0.1)
    assert np.allclose(a, b, atol=1e-13)
