"""The in-place compaction's ordering rule, checked on the CPU.

The GPU kernel moves 64-row destination chunks as independent tasks: a task
loads its sources, publishes, waits for the earlier chunks that read its
destination rows -- the chunks holding ranks P(64c) .. P(64c+64)-1, with P(x)
the number of kept rows below x -- and then stores.  Here the same rule drives
a randomised interleaving of loads and stores over a plain array; every
interleaving the rule allows must leave the exact gather.  A model with the
waits removed must fail on the same inputs (the test is not vacuous).
"""
import numpy as np
import pytest

CHUNK = 64


def prefix_bounds(keep, n_chunks):
    """P(64 e) for e = 0 .. n_chunks (number of kept rows below 64 e)."""
    return np.searchsorted(keep, np.arange(n_chunks + 1) * CHUNK, side="left")


def simulate(keep, n, rng, respect_waits=True):
    """Tasks start in chunk order (a persistent grid takes them in order), but a
    started task's loads complete at any later time, in any order across tasks."""
    K = len(keep)
    rows = np.arange(n) * 7 + 1  # distinct row contents
    mem = rows.copy()
    nch = (K + CHUNK - 1) // CHUNK
    P = prefix_bounds(keep, nch)
    started = 0
    loaded = [None] * nch  # the values a task read, once its loads completed
    stored = [False] * nch
    while not all(stored):
        choices = []
        if started < nch:
            choices.append(("start", started))
        for c in range(started):
            if loaded[c] is None:
                choices.append(("load", c))
            elif not stored[c]:
                lo, hi = P[c] // CHUNK, min(c - 1, (P[c + 1] - 1) // CHUNK)
                ready = P[c + 1] <= P[c] or all(loaded[cc] is not None for cc in range(lo, hi + 1))
                if ready or not respect_waits:
                    choices.append(("store", c))
        kind, c = choices[rng.integers(len(choices))]
        if kind == "start":
            started += 1
        elif kind == "load":
            d = np.arange(c * CHUNK, min((c + 1) * CHUNK, K))
            loaded[c] = (d, mem[keep[d]].copy())  # published once loaded
        else:
            d, vals = loaded[c]
            mem[d] = vals
            stored[c] = True
    return mem[:K], rows[keep]


def patterns(rng):
    n = 3000
    yield "quarter", np.sort(rng.choice(n, n // 4, replace=False)), n
    yield "steady", np.sort(np.setdiff1d(np.arange(n), rng.choice(n - 512, 128, replace=False))), n
    yield "tail", np.arange(n - 700, n), n
    yield "alternate", np.arange(1, n, 2), n
    yield "head_run", np.concatenate([np.arange(0, 900), np.arange(1000, n, 3)]), n
    yield "dense_gap", np.concatenate([np.arange(0, 64), np.arange(200, n)]), n


@pytest.mark.parametrize("seed", range(4))
def test_rule_gives_the_exact_gather(seed):
    rng = np.random.default_rng(seed)
    for name, keep, n in patterns(rng):
        got, want = simulate(keep, n, rng)
        assert np.array_equal(got, want), name


def test_without_waits_it_breaks():
    rng = np.random.default_rng(11)
    broken = 0
    for seed in range(4):
        for name, keep, n in patterns(np.random.default_rng(seed)):
            got, want = simulate(keep, n, rng, respect_waits=False)
            broken += not np.array_equal(got, want)
    assert broken > 0


def test_readers_of_a_chunk_are_earlier_or_itself():
    """The moves reading rows [64c, 64c+64) have ranks in [P(64c), P(64c+64)); none
    of them belongs to a later chunk, since sources lie at or above destinations."""
    rng = np.random.default_rng(5)
    for name, keep, n in patterns(rng):
        nch = (len(keep) + CHUNK - 1) // CHUNK
        P = prefix_bounds(keep, nch)
        for c in range(nch):
            readers = np.nonzero((keep >= c * CHUNK) & (keep < (c + 1) * CHUNK))[0]
            if len(readers):
                assert readers.min() == P[c] and readers.max() == P[c + 1] - 1, name
                assert readers.max() // CHUNK <= c, name
