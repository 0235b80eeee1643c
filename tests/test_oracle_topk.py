"""Pins for the oracle's top-K: hand cases, brute force, invariants."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import select_topk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "topk_examples.json")


def brute_topk(scores, K):
    """Independent O(L^2) definition: token i is kept iff fewer than K
    tokens beat it, where j beats i when s_j > s_i, or s_j == s_i and j < i."""
    L = len(scores)
    keep = []
    for i in range(L):
        beaten_by = sum(1 for j in range(L)
                        if scores[j] > scores[i] or (scores[j] == scores[i] and j < i))
        if beaten_by < K:
            keep.append(i)
    return keep + [-1] * (K - len(keep))


def test_hand_examples():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        s = np.array(c["scores"], dtype=np.float32)
        got = select_topk(s, len(s), c["k"]).tolist()
        assert got == c["expect"], c


@pytest.mark.parametrize("L", range(0, 9))
def test_brute_force_all_k_small_alphabet(L):
    # every score vector over a 3-symbol alphabet (forces ties and +-0)
    alphabet = [np.float32(-0.0), np.float32(0.0), np.float32(1.5)]
    for combo in itertools.product(range(3), repeat=L) if L <= 6 else []:
        s = np.array([alphabet[c] for c in combo], dtype=np.float32)
        for K in range(1, L + 2):
            assert select_topk(s, L, K).tolist() == brute_topk(list(s), K)


def test_brute_force_random():
    rng = np.random.default_rng(7)
    for _ in range(300):
        L = int(rng.integers(1, 13))
        s = rng.integers(-3, 4, size=L).astype(np.float32) * np.float32(0.5)
        s[rng.random(L) < 0.2] = np.float32(-0.0)
        K = int(rng.integers(1, 14))
        assert select_topk(s, L, K).tolist() == brute_topk(list(s), K)


def test_invariants_large():
    rng = np.random.default_rng(11)
    L, K = 50000, 2048
    s = rng.standard_normal(L).astype(np.float32)
    s[::97] = s[5]  # plant ties
    sel = select_topk(s, L, K)
    assert (sel >= 0).all() and np.all(np.diff(sel) > 0)
    mask = np.zeros(L, bool)
    mask[sel] = True
    smin = s[sel].min()
    assert s[~mask].max() <= smin
    # among boundary ties, selected ones have lower indices than rejected ones
    tie = np.flatnonzero(s == smin)
    chosen = tie[mask[tie]]
    rejected = tie[~mask[tie]]
    if rejected.size:
        assert chosen.max() < rejected.min()


def test_prefix_only_and_k_ge_l():
    s = np.array([1, 9, 2, 8, 100, 100], dtype=np.float32)  # entries past L ignored
    assert select_topk(s, 4, 2).tolist() == [1, 3]
    assert select_topk(s, 4, 10).tolist() == [0, 1, 2, 3] + [-1] * 6
