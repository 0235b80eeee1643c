"""Pins for the oracle's absorbed-MLA attention: closed forms, a library
routine, and the textbook identity behind the absorbed form."""
import math

import numpy as np
import torch

from oracle import mla_attention

D, DV = 576, 512


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_single_row_returns_its_value_exactly():
    rng = np.random.default_rng(0)
    q, rows = _rand(rng, 5, D), _rand(rng, 1, D)
    out, lse = mla_attention(q, rows, 0.3)
    assert np.array_equal(out, np.broadcast_to(rows[0, :DV], out.shape))
    assert np.allclose(lse, 0.3 * q @ rows[0])


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(1)
    rows = _rand(rng, 37, D)
    out, lse = mla_attention(np.zeros((2, D)), rows, 1 / 24)
    assert np.allclose(out, rows[:, :DV].mean(axis=0), rtol=0, atol=1e-13)
    assert np.allclose(lse, math.log(37))


def test_two_row_closed_form():
    rng = np.random.default_rng(2)
    q, rows = _rand(rng, 3, D), _rand(rng, 2, D)
    sc = 1 / 24
    out, lse = mla_attention(q, rows, sc)
    s1, s2 = sc * q @ rows[0], sc * q @ rows[1]
    sig = lambda x: 1 / (1 + np.exp(-x))
    ref = sig(s1 - s2)[:, None] * rows[0, :DV] + sig(s2 - s1)[:, None] * rows[1, :DV]
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-13)
    assert np.allclose(lse, np.logaddexp(s1, s2), rtol=1e-14)


def test_matches_torch_sdpa_float64():
    rng = np.random.default_rng(3)
    q, rows = _rand(rng, 16, D), _rand(rng, 300, D) * 2
    sc = 1 / 24
    out, _ = mla_attention(q, rows, sc)
    tq = torch.from_numpy(q)[None, None]
    tk = torch.from_numpy(rows)[None, None]
    tv = torch.from_numpy(rows[:, :DV].copy())[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=sc)[0, 0].numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_empty_selection():
    out, lse = mla_attention(np.ones((4, D)), np.zeros((0, D)), 0.1)
    assert (out == 0).all() and np.isneginf(lse).all()


def test_absorbed_form_equals_per_head_attention():
    """With a per-head key up-projection W_UK (128 x 512) and value
    up-projection W_UV (128 x 512), attention with keys k = [W_UK c ; k_rope]
    and values v = W_UV c equals attention of the absorbed query
    [W_UK^T q_nope ; q_rope] over the latent rows, followed by W_UV."""
    rng = np.random.default_rng(4)
    n, dn = 50, 128
    c = _rand(rng, n, DV)            # latent (nope) part of each row
    k_rope = _rand(rng, n, 64)
    W_UK, W_UV = _rand(rng, dn, DV) / 20, _rand(rng, dn, DV) / 20
    q_nope, q_rope = _rand(rng, dn), _rand(rng, 64)
    sc = 0.07
    # per-head attention in the up-projected space
    keys = np.concatenate([c @ W_UK.T, k_rope], axis=1)
    vals = c @ W_UV.T
    s = sc * keys @ np.concatenate([q_nope, q_rope])
    p = np.exp(s - s.max())
    p /= p.sum()
    ref = p @ vals
    # absorbed form over the latent rows
    q_abs = np.concatenate([W_UK.T @ q_nope, q_rope])
    rows = np.concatenate([c, k_rope], axis=1)
    out, _ = mla_attention(q_abs[None], rows, sc)
    assert np.allclose(out[0] @ W_UV.T, ref, rtol=1e-12, atol=1e-12)


def test_permutation_invariance():
    rng = np.random.default_rng(5)
    q, rows = _rand(rng, 4, D), _rand(rng, 64, D)
    a, la = mla_attention(q, rows, 0.05)
    b, lb = mla_attention(q, rows[rng.permutation(64)], 0.05)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13) and np.allclose(la, lb)
