"""The in-place compaction's ordering rule, checked on the CPU, as the GPU kernel
applies it.

The kernel moves destination chunks of CR rows (CR = 256, 128 or 64, the widest
whose pieces fit a workgroup's registers) of every unit as tasks ordered by
chunk, then unit, and numbered densely (only the chunks a unit moves are
tasks).  Workgroups take a few tasks per ticket (2 to 16, chosen by the host) from a
counter and run the tasks of a ticket one after another; a task loads its sources,
publishes, waits for the earlier chunks of its unit that read its destination
rows, and then stores.  The readers of chunk c's rows are found from the
selector's prefix counts P[e] = (kept rows below row 64 e), e = 0 .. nb with
nb = ceil(kept / 64): ranks P[kPerP c] .. P[min(kPerP c + kPerP, nb)] - 1,
kPerP = CR / 64, i.e. chunks lo = P[kPerP c] // CR .. hi = min(c - 1,
(P[...] - 1) // CR).  Here the same rule drives randomised interleavings of
loads, publishes and stores over plain arrays; every interleaving the rule
allows must leave the exact gather in every unit, and a model with the waits
removed must fail on the same inputs (the test is not vacuous).
"""
import os
import re

import numpy as np
import pytest

ROWS64 = 64          # granularity of the prefix counts
TICKET_SIZES = (1, 2, 4, 16)  # tasks taken per ticket, modelled


def prefix_counts(keep):
    """P[e] for e = 0 .. nb: kept rows below row 64 e (nb = 64-row chunks of kept)."""
    nb = (len(keep) + ROWS64 - 1) // ROWS64
    return np.searchsorted(keep, np.arange(nb + 1) * ROWS64, side="left"), nb


def wait_range(P, nb, c, cr):
    """Chunks of cr rows (same unit) that chunk c waits for, as (lo, hi), or None."""
    per = cr // ROWS64
    p0, p1 = P[per * c], P[min(per * c + per, nb)]
    if p1 <= p0:
        return None
    return p0 // cr, min(c - 1, (p1 - 1) // cr)


def simulate(units, cr, n_workers, rng, respect_waits=True, ticket_tasks=2):
    """units: list of (keep, n).  Workers take ticket_tasks consecutive tasks per ticket
    and run them in order; a task's loads complete at any later time, and the steps of
    different workers interleave at random."""
    U = len(units)
    mems, wants, plans = [], [], []
    for u, (keep, n) in enumerate(units):
        rows = np.arange(n) * 7 + 1000 * u + 1  # distinct row contents
        mems.append(rows.copy())
        wants.append(rows[keep])
        P, nb = prefix_counts(keep)
        plans.append((keep, n, P, nb))
    # the kernel's dense numbering (each unit its own sequence here): only the
    # chunks a unit moves are tasks, level by level
    chunks = [(len(k) + cr - 1) // cr if 0 < len(k) < n else 0 for k, n in units]
    n_tasks = sum(chunks)
    order = [decode(t, dense_plan(chunks, 1), 1) for t in range(n_tasks)]
    published = set()
    ticket = 0
    workers = [[] for _ in range(n_workers)]  # pending tasks of a worker's ticket
    state = [None] * n_workers  # (task, stage, loaded values)
    done = 0

    while True:
        choices = []
        for w in range(n_workers):
            if state[w] is None:
                if workers[w]:
                    choices.append((w, "begin"))
                elif ticket < n_tasks:
                    choices.append((w, "ticket"))
            else:
                task, stage, _ = state[w]
                if stage == "issued":
                    choices.append((w, "arrive"))
                else:  # published: store once every reader of its rows has loaded
                    c, u = order[task]
                    keep, n, P, nb = plans[u]
                    rng_ = wait_range(P, nb, c, cr)
                    ready = rng_ is None or all((cc, u) in published
                                                for cc in range(rng_[0], rng_[1] + 1))
                    if ready or not respect_waits:
                        choices.append((w, "store"))
        if not choices:
            break
        w, kind = choices[rng.integers(len(choices))]
        if kind == "ticket":
            workers[w] = list(range(ticket, min(ticket + ticket_tasks, n_tasks)))
            ticket += ticket_tasks
        elif kind == "begin":
            task = workers[w].pop(0)
            state[w] = (task, "issued", None)
        elif kind == "arrive":
            task, _, _ = state[w]
            c, u = order[task]
            keep = plans[u][0]
            d = np.arange(c * cr, min((c + 1) * cr, len(keep)))
            vals = mems[u][keep[d]].copy()
            published.add((c, u))
            state[w] = (task, "published", (d, vals))
        else:
            task, _, (d, vals) = state[w]
            c, u = order[task]
            mems[u][d] = vals
            state[w] = None
            done += 1
    assert done == n_tasks
    return [m[:len(k)] for m, (k, _) in zip(mems, units)], wants


def patterns(rng):
    n = 3000
    yield "quarter", np.sort(rng.choice(n, n // 4, replace=False)), n
    yield "steady", np.sort(np.setdiff1d(np.arange(n), rng.choice(n - 512, 128, replace=False))), n
    yield "tail", np.arange(n - 700, n), n
    yield "alternate", np.arange(1, n, 2), n
    yield "head_run", np.concatenate([np.arange(0, 900), np.arange(1000, n, 3)]), n
    yield "dense_gap", np.concatenate([np.arange(0, 64), np.arange(200, n)]), n
    yield "ragged", np.sort(rng.choice(1777, 1000, replace=False)), 1777
    yield "keep_all", np.arange(500), 500  # kept == n: no task moves anything


def unit_sets(seed):
    """Groups of three units with different patterns (and sizes) in one launch."""
    pats = list(patterns(np.random.default_rng(seed)))
    for i in range(0, len(pats), 2):
        trio = [pats[i], pats[(i + 1) % len(pats)], pats[(i + 5) % len(pats)]]
        yield "+".join(p[0] for p in trio), [(p[1].astype(np.int64), p[2]) for p in trio]


def test_the_kernel_takes_a_modelled_ticket_size():
    """The host picks the tasks per ticket within bounds the model covers."""
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "kv_cache_eviction_tria_amd", "csrc", "tria_compact.hip")).read()
    m = re.search(r"return \(int\)\(tt < (\d+) \? \d+ : \(tt > (\d+) \? \d+ : tt\)\);", src)
    assert m
    lo, hi = int(m.group(1)), int(m.group(2))
    assert lo >= min(TICKET_SIZES) and hi <= max(TICKET_SIZES)


@pytest.mark.parametrize("tt", TICKET_SIZES)
@pytest.mark.parametrize("cr", [64, 128, 256])
@pytest.mark.parametrize("seed", range(3))
def test_rule_gives_the_exact_gather(cr, seed, tt):
    rng = np.random.default_rng(100 + seed + 10 * tt)
    for name, units in unit_sets(seed):
        got, want = simulate(units, cr, 5, rng, ticket_tasks=tt)
        for g, w in zip(got, want):
            assert np.array_equal(g, w), (name, cr, tt)


@pytest.mark.parametrize("tt", TICKET_SIZES)
@pytest.mark.parametrize("cr", [64, 128, 256])
def test_without_waits_it_breaks(cr, tt):
    rng = np.random.default_rng(11)
    broken = 0
    for seed in range(3):
        for name, units in unit_sets(seed):
            got, want = simulate(units, cr, 5, rng, respect_waits=False, ticket_tasks=tt)
            broken += sum(not np.array_equal(g, w) for g, w in zip(got, want))
    assert broken > 0


@pytest.mark.parametrize("cr", [64, 128, 256])
def test_readers_of_a_chunk_are_earlier_or_itself(cr):
    """The moves reading the destination rows of chunk c have ranks inside the range
    the prefix counts give; none of them belongs to a later chunk, since sources lie
    at or above destinations."""
    rng = np.random.default_rng(5)
    for name, keep, n in patterns(rng):
        K = len(keep)
        P, nb = prefix_counts(keep)
        per = cr // ROWS64
        for c in range((K + cr - 1) // cr):
            dst_hi = min((c + 1) * cr, K)
            readers = np.nonzero((keep >= c * cr) & (keep < dst_hi))[0]
            if len(readers):
                assert readers.min() >= P[per * c], name
                assert readers.max() <= P[min(per * c + per, nb)] - 1, name
                assert readers.max() // cr <= c, name


def dense_plan(chunks, per_seq):
    """The kernel's dense task numbering, restated: sequences sorted by chunk count
    (descending, ties by index); segment k covers levels [v[k+1], v[k]) with the
    first k + 1 sorted sequences present and starts at task
    per_seq * ((k + 1) v[k+1] + sum(v[k+1:]))."""
    order = sorted(range(len(chunks)), key=lambda i: (-chunks[i], i))
    v = [chunks[i] for i in order if chunks[i] > 0]
    segs = len(v)
    t0 = [per_seq * ((k + 1) * (v[k + 1] if k + 1 < segs else 0) + sum(v[k + 1:]))
          for k in range(segs)]
    c0 = [v[k + 1] if k + 1 < segs else 0 for k in range(segs)]
    return order, t0, c0, segs


def decode(task, plan, per_seq):
    order, t0, c0, segs = plan
    lo, hi = 0, segs - 1  # smallest k with t0[k] <= task
    while lo < hi:
        mid = (lo + hi) // 2
        if t0[mid] <= task:
            hi = mid
        else:
            lo = mid + 1
    rel = task - t0[lo]
    level = (lo + 1) * per_seq
    c = c0[lo] + rel // level
    r = rel % level
    return c, order[r // per_seq] * per_seq + r % per_seq


@pytest.mark.parametrize("seed", range(40))
def test_dense_task_numbering_is_a_level_ordered_bijection(seed):
    """Every (chunk, unit) a batch moves is exactly one task, tasks run level by
    level (so a chunk's waits are on smaller tasks), and no task is empty."""
    rng = np.random.default_rng(seed)
    n_seq = int(rng.integers(1, 65))
    per_seq = int(rng.integers(1, 9)) * int(rng.integers(1, 5))
    chunks = [int(x) for x in rng.integers(0, 40, size=n_seq)]
    if seed % 5 == 0:
        chunks = [chunks[0]] * n_seq  # all equal
    if seed % 7 == 0:
        chunks[int(rng.integers(0, n_seq))] = 0
    total = per_seq * sum(chunks)
    if total == 0:
        return
    plan = dense_plan(chunks, per_seq)
    seen = set()
    last_level = 0
    for task in range(total):
        c, u = decode(task, plan, per_seq)
        assert 0 <= u < n_seq * per_seq
        assert 0 <= c < chunks[u // per_seq], (task, c, u)
        assert c >= last_level
        last_level = c
        seen.add((c, u))
    assert len(seen) == total
    if n_seq == 1 or len(set(chunks)) == 1:  # one chunk count: task = c * units + u
        units = n_seq * per_seq
        for task in range(total):
            assert decode(task, plan, per_seq) == (task // units, task % units)
