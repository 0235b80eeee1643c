"""Pins for the oracle's resolve (classification, LRU victims, plan).

* hand-computed traces in tests/golden (the LRU rule and its tie
  conventions, residency precedence, a stale hot copy, a reset);
* invariants over random histories;
* equality with a second, independent formulation of the same policy (an
  explicit LRU order list updated by compaction, the form a GPU kernel
  uses), written here from the policy's statement, not from the oracle.
"""
import json
import os

import numpy as np
import pytest

from oracle import HOT, MISS, RESIDENT, HotBufferOracle, resolve_step

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lru_worked_examples.json")
KIND = {"R": RESIDENT, "H": HOT, "M": MISS}


@pytest.mark.parametrize("ex", json.load(open(GOLDEN))["examples"], ids=lambda e: e["name"])
def test_worked_examples(ex):
    ps = ex["page_size"]
    hb = HotBufferOracle(ex["slots"], 64)
    hot_pages = np.array(ex["hot_pages"])
    for st in ex["steps"]:
        if st["reset_hot"]:
            hb.reset()
        res = resolve_step(hb, np.array(st["sel"]), np.array(st["gpu_page"]), hot_pages, ps)
        assert res["kind"].tolist() == [KIND[c] for c in st["kind"]]
        assert hb.tag.tolist() == st["tags"]
        assert hb.stamp.tolist() == st["stamps"]
        assert res["counts"].tolist() == st["counts"]
        assert res["plan"].tolist() == st["plan"]


class OrderListLRU:
    """Second formulation: keep all S slots in one list, least recent first.

    A step removes the slots hit this step; the first M remaining slots are
    the victims; the list becomes (remaining minus victims) followed by
    (hit slots and victims) in ascending slot number, since all of them now
    carry the newest stamp and equal stamps order by slot.
    """

    def __init__(self, S, cap):
        self.order = list(range(S))
        self.tag = [-1] * S
        self.where = {}

    def step(self, sel, gpu_page, ps):
        kinds, hit_slots, misses = [], set(), []
        for t in sel:
            if t < 0:
                continue
            if gpu_page[t // ps] >= 0:
                kinds.append(RESIDENT)
            elif t in self.where:
                kinds.append(HOT)
                hit_slots.add(self.where[t])
            else:
                kinds.append(MISS)
                misses.append(t)
        rest = [s for s in self.order if s not in hit_slots]
        victims = rest[:len(misses)]
        for t, s in zip(misses, victims):
            if self.tag[s] >= 0:
                del self.where[self.tag[s]]
            self.tag[s] = t
            self.where[t] = s
        self.order = rest[len(misses):] + sorted(hit_slots | set(victims))
        return kinds


def _random_history(seed, S=16, K=6, L=96, ps=8, steps=60):
    rng = np.random.default_rng(seed)
    P = L // ps
    hot_pages = np.arange(100, 100 + S // ps)
    gpu_page = np.where(rng.random(P) < 0.3, rng.permutation(P), -1)
    for _ in range(steps):
        if rng.random() < 0.2:  # residency changes between steps
            flip = rng.integers(0, P)
            gpu_page[flip] = -1 if gpu_page[flip] >= 0 else 500 + flip
        # a drifting working set so that hits recur
        base = int(rng.integers(0, L - 3 * K))
        pool = np.arange(base, base + 3 * K)
        n = int(rng.integers(1, K + 1))
        sel = np.sort(rng.choice(pool, size=n, replace=False))
        sel = np.concatenate([sel, -np.ones(K - n, dtype=np.int64)])
        yield sel, gpu_page.copy(), hot_pages, ps


@pytest.mark.parametrize("seed", range(12))
def test_order_list_formulation_agrees(seed):
    S, K, L = 16, 6, 96
    hb = HotBufferOracle(S, L)
    ol = OrderListLRU(S, L)
    for sel, gpu_page, hot_pages, ps in _random_history(seed, S, K, L):
        res = resolve_step(hb, sel, gpu_page, hot_pages, ps)
        kinds = ol.step(sel, gpu_page, ps)
        assert res["kind"][res["kind"] >= 0].tolist() == kinds
        assert hb.tag.tolist() == ol.tag


@pytest.mark.parametrize("seed", range(6))
def test_invariants(seed):
    S, K, L = 16, 6, 96
    hb = HotBufferOracle(S, L)
    prev_tags = set()
    for sel, gpu_page, hot_pages, ps in _random_history(seed, S, K, L):
        before = {int(t) for t in hb.tag if t >= 0}
        res = resolve_step(hb, sel, gpu_page, hot_pages, ps)
        n = hb.step
        valid = sel[sel >= 0]
        # counts add up to the number of selected tokens
        assert res["counts"].sum() == valid.size
        # tags and reverse map are mutual inverses
        for s, t in enumerate(hb.tag):
            if t >= 0:
                assert hb.rev[t] == s
        assert (hb.rev >= 0).sum() == (hb.tag >= 0).sum()
        # every selected host-only token is in the hot buffer afterwards
        for t in valid:
            if gpu_page[t // ps] < 0:
                assert hb.rev[t] >= 0
        # a miss was absent before; a hit was present
        for t, k in zip(valid, res["kind"][: valid.size]):
            if k == MISS:
                assert int(t) not in before
            if k == HOT:
                assert int(t) in before
        # slots touched this step carry stamp n; nothing touched was evicted
        touched = hb.rev[valid[res["kind"][: valid.size] != RESIDENT]]
        assert (hb.stamp[touched] == n).all()
        # plan rows of hot/missed tokens are inside the leased hot pages
        hrows = res["plan"][: valid.size][res["kind"][: valid.size] != RESIDENT]
        assert ((hrows // ps >= hot_pages.min()) & (hrows // ps <= hot_pages.max())).all()
        prev_tags = before


def test_fully_resident_request_never_touches_hot_buffer():
    hb = HotBufferOracle(8, 64)
    gpu_page = np.arange(8) + 40
    for step in range(5):
        sel = np.sort(np.random.default_rng(step).choice(64, 4, replace=False))
        res = resolve_step(hb, sel, gpu_page, np.array([0]), 8)
        assert res["counts"].tolist() == [4, 0, 0]
        assert (hb.tag == -1).all() and (hb.stamp == 0).all()
        assert res["plan"].tolist() == [(40 + t // 8) * 8 + t % 8 for t in sel]


def test_resident_takes_precedence_over_stale_hot_copy():
    hb = HotBufferOracle(4, 32)
    hot_pages = np.array([9])
    host = np.full(4, -1)
    resolve_step(hb, np.array([3, 5]), host, hot_pages, 4)     # both missed -> hot
    back = host.copy()
    back[0] = 2                                               # page 0 returns to GPU
    res = resolve_step(hb, np.array([3, 5]), back, hot_pages, 4)
    assert res["kind"].tolist() == [RESIDENT, HOT]
    assert res["plan"][0] == 2 * 4 + 3


def test_empty_slots_fill_before_any_eviction():
    hb = HotBufferOracle(8, 64)
    host = np.full(16, -1)
    hot_pages = np.array([0])
    resolve_step(hb, np.array([1, 2]), host, hot_pages, 8)
    res = resolve_step(hb, np.array([3, 4, 5]), host, hot_pages, 8)
    assert res["miss_slots"].tolist() == [2, 3, 4]
    assert sorted(t for t in hb.tag if t >= 0) == [1, 2, 3, 4, 5]
