"""Pins of the residency-manager reference (oracle/residency.py) against a
hand-worked case and an independent formulation."""
import json
import os

import numpy as np
import pytest

from oracle import PageState, update_residency

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "residency_worked_example.json")


def _state(stamp, host_valid):
    st = PageState(len(stamp))
    st.stamp[:] = stamp
    st.host_valid[:] = np.asarray(host_valid, dtype=bool)
    return st


def test_worked_example():
    g = json.load(open(GOLDEN))
    st = _state(g["stamp"], g["host_valid"])
    gp = np.array(g["gpu_page"], dtype=np.int64)
    out = update_residency(st, gp, g["context_len"], g["page_size"], g["budget"], g["max_copy"],
                           g["max_demote"])
    e = g["expect"]
    assert out["copied"] == e["copied"]
    assert out["demoted"] == e["demoted"]
    assert out["freed"] == e["freed"]
    assert gp.tolist() == e["gpu_page_after"]
    assert st.host_valid.astype(int).tolist() == e["host_valid_after"]


def _one_at_a_time(stamp, host_valid, gpu_page, L, ps, budget, max_copy, max_demote):
    """Independent formulation: walk the pages to copy, then release one
    coldest page at a time until the budget holds or nothing is left."""
    hv = list(host_valid)
    gp = list(gpu_page)
    copied = []
    p = 0
    while p < L // ps and len(copied) < max_copy:
        if gp[p] >= 0 and not hv[p]:
            copied.append(p)
            hv[p] = True
        p += 1
    npg = -(-L // ps)
    demoted = []
    while len(demoted) < max_demote and sum(1 for q in range(npg) if gp[q] >= 0) > budget:
        best = None
        for q in range(L // ps):
            if gp[q] >= 0 and hv[q] and (best is None or (stamp[q], q) < (stamp[best], best)):
                best = q
        if best is None:
            break
        demoted.append(best)
        gp[best] = -1
    return copied, sorted(demoted), gp, hv


@pytest.mark.parametrize("seed", range(40))
def test_matches_one_at_a_time(seed):
    rng = np.random.default_rng(seed)
    ps = int(rng.choice([1, 2, 4, 8]))
    P = int(rng.integers(1, 40))
    L = int(rng.integers(0, P * ps + 1))
    stamp = rng.integers(0, 6, P)          # many ties
    hv = rng.random(P) < 0.5
    gpu = np.where(rng.random(P) < 0.6, rng.permutation(1000)[:P], -1)
    budget = int(rng.integers(0, P + 1))
    mc, md = int(rng.integers(0, 5)), int(rng.integers(0, 8))
    st = _state(stamp, hv)
    gp = gpu.astype(np.int64).copy()
    out = update_residency(st, gp, L, ps, budget, mc, md)
    c2, d2, gp2, hv2 = _one_at_a_time(stamp.tolist(), hv.tolist(), gpu.tolist(), L, ps, budget, mc, md)
    assert out["copied"] == c2
    assert out["demoted"] == d2
    assert gp.tolist() == gp2
    assert st.host_valid.tolist() == hv2
    assert out["freed"] == [int(gpu[p]) for p in d2]


def test_invariants_random():
    rng = np.random.default_rng(7)
    for _ in range(200):
        ps = 4
        P = 30
        L = int(rng.integers(1, P * ps + 1))
        stamp = rng.integers(0, 10, P)
        hv = rng.random(P) < 0.7
        gpu = np.where(rng.random(P) < 0.7, np.arange(100, 100 + P), -1)
        budget = int(rng.integers(0, P))
        st = _state(stamp, hv)
        gp = gpu.astype(np.int64).copy()
        out = update_residency(st, gp, L, ps, budget, 3, 64)
        full = L // ps
        for p in out["demoted"]:
            assert p < full, "an incomplete page was released"
            assert st.host_valid[p], "a page without a host copy was released"
        kept = [p for p in range(full) if gp[p] >= 0 and st.host_valid[p]]
        for p in out["demoted"]:
            for q in kept:  # every released page is at least as cold as every kept candidate
                assert (stamp[p], p) < (stamp[q], q)
        held = int(np.count_nonzero(gp[:-(-L // ps)] >= 0))
        assert held <= budget or not kept, "pressure left while candidates remain"
        assert out["copied"] == sorted(out["copied"])


def test_context_entry_and_touch():
    st = PageState(10)
    st.enter_context(0, 13, 0, 4)       # pages 0..3 enter at step 0
    st.touch(np.array([1, 5, -1]), 1, 4)
    st.enter_context(13, 21, 1, 4)      # pages 4, 5 enter at step 1
    st.touch(np.array([20, -1, -1]), 2, 4)
    assert st.stamp.tolist() == [1, 1, 0, 0, 1, 2, 0, 0, 0, 0]
    st.mark_given(0, np.array([5, -1, 7]), host_copy_valid=False)
    assert st.host_valid[:3].tolist() == [False, True, False]
