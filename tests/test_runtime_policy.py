"""The decode-loop policy (host logic in the library, no GPU needed): when an
eviction pass runs and with which arguments, against the schedule the worklog
logs and the rules both pages state."""
import json
import os

import pytest

from kv_cache_eviction_tria_amd import tria

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "schedule_worklog.json")


def policy(**kw):
    d = dict(trigger=tria.TRIA_TRIGGER_THRESHOLD, protect_prefill=1, budget=3072,
             divide_length=128, interval=128, sink=0, window=512)
    d.update(kw)
    return tria.Policy(**d)


def run(p, n_prompt, steps):
    """Decode `steps` tokens after a prompt: one row appended per step; a due pass
    leaves tria_kept_count rows.  Returns [(abs_pos, rows_before, rows_after)]."""
    st = tria.DecodeState(n_rows=n_prompt, n_prompt=n_prompt, steps=0, passes=0)
    out = []
    for t in range(steps):
        st.n_rows += 1
        st.steps += 1
        due = tria.tria_policy_due(p, st)
        if due is not None:
            b, s, w = due
            kept = tria.tria_kept_count(st.n_rows, b, s, w)
            out.append((n_prompt + t + 1, st.n_rows, kept))
            st.n_rows, st.steps, st.passes = kept, 0, st.passes + 1
    return out


def test_threshold_schedule_matches_the_worklog_logs():
    g = json.load(open(GOLD))
    sched = run(policy(), 0, 3700)
    assert [a for a, _, _ in sched[:4]] == [3200] + g["abs_pos_after_first"]
    assert all(rb == g["rows_before_each"] and ra == 3072 for _, rb, ra in sched[:4])
    big = run(policy(budget=6144, divide_length=1024), 0, 7200)
    assert big[0] == (7168, 7168, 6144)


def test_prompt_rows_are_protected_and_not_counted():
    """A 700-row prompt with a 128-row budget: nothing runs until 128 + 64 decode rows
    exist, and each pass keeps the whole prompt plus 128 decode rows."""
    p = policy(budget=128, divide_length=64, window=32)
    sched = run(p, 700, 400)
    assert sched[0] == (700 + 192, 892, 700 + 128)
    st = tria.DecodeState(n_rows=892, n_prompt=700, steps=5, passes=0)
    assert tria.tria_policy_due(p, st) == (828, 700, 32)
    # without protection the prompt counts and a pass runs at the first step
    q = policy(budget=128, divide_length=64, window=32, protect_prefill=0)
    assert run(q, 700, 3)[0] == (701, 701, 128)


def test_interval_trigger():
    """llama.cpp's --tri-interval: a pass every `interval` decode steps once the rows
    exceed the budget; none before that."""
    p = policy(trigger=tria.TRIA_TRIGGER_INTERVAL, budget=1000, interval=128, protect_prefill=0)
    sched = run(p, 900, 600)
    assert [a for a, _, _ in sched] == [900 + 128 * i for i in (1, 2, 3, 4)]
    assert all(ra == 1000 for _, _, ra in sched)
    assert sched[0][1] == 1028 and sched[1][1] == 1128


def test_peak_rows_bound_every_state_seen():
    for p, n_prompt in ((policy(), 0), (policy(budget=128, divide_length=64, window=32), 700),
                        (policy(budget=128, divide_length=64, window=32, protect_prefill=0), 700),
                        (policy(trigger=tria.TRIA_TRIGGER_INTERVAL, budget=1000, interval=128,
                                protect_prefill=0), 900)):
        peak = tria.tria_policy_peak_rows(p, n_prompt)
        sched = run(p, n_prompt, 2000)
        seen = max([n_prompt + 1] + [rb for _, rb, _ in sched])
        assert seen <= peak, (seen, peak)


def test_bad_policies_are_rejected():
    st = tria.DecodeState(n_rows=10, n_prompt=0, steps=0, passes=0)
    for bad in (policy(budget=0), policy(divide_length=0), policy(trigger=7), policy(sink=-1),
                policy(trigger=tria.TRIA_TRIGGER_INTERVAL, interval=0)):
        with pytest.raises(tria.TriaError):
            tria.tria_policy_due(bad, st)
    with pytest.raises(tria.TriaError):
        tria.tria_policy_due(policy(), tria.DecodeState(n_rows=5, n_prompt=6, steps=0, passes=0))
