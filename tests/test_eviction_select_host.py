"""Host transcription of the merge planner's eviction select (CPU only).

The planning kernel finds the cut-off frame of the eviction by walking the
distinct last-update frames of the eligible slots upward (a block-wide minimum
and its count per step, up to eight steps), and falls back to a radix select
(8-bit digits, most significant first, digits above the largest possible value
frame - 1 skipped) when eight values do not cover the need; ties on the cut-off
frame go by slot id.  This file replays those steps in Python as the kernel
takes them, checks them against the eviction rule itself (smallest
(last, slot) among the slots not merged into this frame), and checks that the
kernel's guard fires — fewer slots found than needed — for the states the host
refuses to import (a last-update frame at or after the frame counter).
"""

import numpy as np
import pytest


def _take(last, eligible, n_live, cut, take_eq):
    out, taken = [], 0
    for s in range(n_live):
        if not eligible[s]:
            continue
        lv = int(last[s]) & 0xFFFFFFFF
        if lv < cut:
            out.append(s)
        elif lv == cut and taken < take_eq:
            out.append(s)
            taken += 1
    return out


def kernel_select(last, eligible, n_live, need, f, walk_steps=8):
    """The planner's select; returns the evicted slots in ascending order."""
    keys = [int(last[s]) & 0xFFFFFFFF for s in range(n_live) if eligible[s]]
    krem, lo = need, 0
    for _ in range(walk_steps):
        above = [k for k in keys if k >= lo]
        if not above:
            break
        mv = min(above)
        cv = sum(1 for k in keys if k == mv)
        if cv >= krem:
            return _take(last, eligible, n_live, mv, krem)
        krem -= cv
        lo = mv + 1
    return radix_select(last, eligible, n_live, need, f)


def radix_select(last, eligible, n_live, need, f):
    """The planner's fallback: radix select on 8-bit digits."""
    krem, prefix, maxv = need, 0, (f - 1) & 0xFFFFFFFF
    for shift in (24, 16, 8, 0):
        if shift > 0 and (maxv >> shift) == 0:
            continue
        hist = [0] * 256
        hi_mask = ~((1 << (shift + 8)) - 1) & 0xFFFFFFFFFFFFFFFF
        for s in range(n_live):
            if not eligible[s]:
                continue
            lv = int(last[s]) & 0xFFFFFFFF
            if (lv & hi_mask) != (prefix & hi_mask):
                continue
            hist[(lv >> shift) & 255] += 1
        cum, dg = 0, 0
        while dg < 256:
            if cum + hist[dg] >= krem:
                break
            cum += hist[dg]
            dg += 1
        krem -= cum
        prefix |= dg << shift
    return _take(last, eligible, n_live, prefix, krem)


def rule_select(last, eligible, n_live, need):
    cand = sorted((int(last[s]), s) for s in range(n_live) if eligible[s])
    return sorted(s for _, s in cand[:need])


@pytest.mark.parametrize("seed", range(12))
def test_select_is_the_lru_rule_on_valid_states(seed):
    rng = np.random.default_rng(seed)
    f = int(rng.choice([1, 2, 7, 255, 256, 257, 70000, 2**24 + 5]))
    n_live = int(rng.integers(1, 600))
    spread = int(rng.choice([1, 3, f]))
    last = rng.integers(max(0, f - spread), f, size=n_live)       # every last <= f - 1
    eligible = rng.random(n_live) < 0.8
    n_el = int(eligible.sum())
    if n_el == 0:
        return
    need = int(rng.integers(1, n_el + 1))
    want = rule_select(last, eligible, n_live, need)
    for steps in (8, 0, 2):   # the kernel's walk, the radix path alone, a short walk
        got = kernel_select(last, eligible, n_live, need, f, walk_steps=steps)
        assert got == want and len(got) == need


def test_guard_fires_on_last_update_frames_from_the_future():
    # a state whose live slots were "updated" at frames 600..999 while the
    # frame counter is 1: the select finds fewer slots than it needs, which is
    # exactly when the planner refuses the frame instead of reading entries
    # of its eviction list that were never written
    n_live, f, need = 400, 1, 100
    last = np.arange(600, 1000)
    eligible = np.ones(n_live, dtype=bool)
    for steps in (8, 0):
        assert len(kernel_select(last, eligible, n_live, need, f, walk_steps=steps)) < need


def test_guard_fires_when_too_few_slots_are_eligible():
    last = np.zeros(10, dtype=np.int64)
    eligible = np.zeros(10, dtype=bool)
    eligible[:3] = True
    for steps in (8, 0):
        assert len(kernel_select(last, eligible, 10, 5, 4, walk_steps=steps)) == 3


def test_walk_covers_many_distinct_frames_through_the_fallback():
    # the need spans 20 distinct frames: more than the walk's eight steps
    last = np.repeat(np.arange(20), 5)
    eligible = np.ones(100, dtype=bool)
    got = kernel_select(last, eligible, 100, 97, 21)
    assert got == rule_select(last, eligible, 100, 97)
