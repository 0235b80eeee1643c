"""Pins of the indexer score oracle (oracle/indexer.py) against hand-worked
values, closed forms and identities of the positive part; CPU only."""
import json
import os

import numpy as np
import pytest

from oracle import indexer_scores

HERE = os.path.dirname(os.path.abspath(__file__))
D = 128


def _pad(a, n=D):
    a = np.asarray(a, dtype=np.float64)
    out = np.zeros(a.shape[:-1] + (n,))
    out[..., :a.shape[-1]] = a
    return out


def _rand(seed, H=8, L=37):
    g = np.random.default_rng(seed)
    return g.standard_normal((H, D)), g.standard_normal(H), g.standard_normal((L, D))


def test_hand_worked_examples():
    with open(os.path.join(HERE, "golden", "indexer_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        s = indexer_scores(_pad(c["q"]), np.asarray(c["w"]), _pad(c["keys"]), len(c["keys"]))
        np.testing.assert_array_equal(s, np.asarray(c["scores"]), err_msg=c["name"])


def test_one_head_on_a_unit_axis_is_the_positive_part_of_a_coordinate():
    _, _, k = _rand(1)
    for d in (0, 5, 127):
        q = np.zeros((1, D))
        q[0, d] = 1.0
        np.testing.assert_array_equal(indexer_scores(q, np.ones(1), k, k.shape[0]), np.clip(k[:, d], 0, None))


def test_positive_part_identity():
    # max(0, x) - max(0, -x) = x, so score(q) - score(-q) is the plain
    # weighted dot product sum_j w_j <q_j, k_t>
    q, w, k = _rand(2)
    lhs = indexer_scores(q, w, k, k.shape[0]) - indexer_scores(-q, w, k, k.shape[0])
    rhs = np.array([sum(w[j] * float(np.dot(q[j], k[t])) for j in range(q.shape[0])) for t in range(k.shape[0])])
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_positive_part_sum_is_the_absolute_value():
    # max(0, x) + max(0, -x) = |x|
    q, w, k = _rand(3)
    s = indexer_scores(q, w, k, k.shape[0]) + indexer_scores(-q, w, k, k.shape[0])
    ref = np.abs(k @ q.T) @ w
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=1e-12)


def test_homogeneity_and_linearity():
    q, w, k = _rand(4)
    L = k.shape[0]
    base = indexer_scores(q, w, k, L)
    np.testing.assert_allclose(indexer_scores(q, 3.0 * w, k, L), 3.0 * base, rtol=1e-12)
    np.testing.assert_allclose(indexer_scores(2.5 * q, w, k, L), 2.5 * base, rtol=1e-12)   # positive scale
    np.testing.assert_allclose(indexer_scores(q, w, 0.5 * k, L), 0.5 * base, rtol=1e-12)
    w2 = np.random.default_rng(5).standard_normal(w.shape)
    np.testing.assert_allclose(indexer_scores(q, w + w2, k, L), base + indexer_scores(q, w2, k, L),
                               rtol=1e-11, atol=1e-11)


def test_heads_permute_split_and_vanish():
    q, w, k = _rand(6)
    L = k.shape[0]
    base = indexer_scores(q, w, k, L)
    p = np.random.default_rng(7).permutation(q.shape[0])
    np.testing.assert_allclose(indexer_scores(q[p], w[p], k, L), base, rtol=1e-12)
    # a head duplicated with its weight split a / (w - a) is the same head
    q2 = np.vstack([q, q[:1]])
    w2 = np.concatenate([w, [0.25]])
    w2[0] -= 0.25
    np.testing.assert_allclose(indexer_scores(q2, w2, k, L), base, rtol=1e-11, atol=1e-12)
    # a zero-weight head contributes nothing, whatever its query
    q3 = np.vstack([q, 100.0 * np.ones((1, D))])
    np.testing.assert_allclose(indexer_scores(q3, np.concatenate([w, [0.0]]), k, L), base, rtol=1e-12)


def test_tokens_are_independent_and_nonnegative_weights_give_nonnegative_scores():
    q, w, k = _rand(8, L=50)
    full = indexer_scores(q, np.abs(w), k, 50)
    assert np.all(full >= 0)
    for L in (0, 1, 17, 49):
        np.testing.assert_allclose(indexer_scores(q, np.abs(w), k, L), full[:L], rtol=1e-13, atol=1e-13)
    # a token whose key is orthogonal to every head scores 0
    k0 = k.copy()
    k0[3] = 0.0
    assert indexer_scores(q, w, k0, 50)[3] == 0.0


@pytest.mark.parametrize("H", [16, 64])
def test_bf16_inputs_widen_exactly(H):
    # bf16 values are exact in fp64, so scores of bf16-rounded inputs do not
    # depend on how they are widened (torch's bf16 -> fp64 as the library check)
    import torch
    g = torch.Generator().manual_seed(H)
    q = torch.randn(H, D, generator=g).to(torch.bfloat16)
    k = torch.randn(40, D, generator=g).to(torch.bfloat16)
    w = torch.rand(H, generator=g)
    s = indexer_scores(q.double().numpy(), w.double().numpy(), k.double().numpy(), 40)
    ref = (torch.relu(k.double() @ q.double().T) @ w.double()).numpy()
    np.testing.assert_allclose(s, ref, rtol=1e-13, atol=1e-13)
