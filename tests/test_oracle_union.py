"""Pins for the speculative-step oracle (union_of_selections and
DecodeOracle.step_union): each query token of a request has its own top-K,
the union of the selections is resolved once (one plan, one LRU update, the
query tokens sharing the request's hot state, [P2] "vLLM GLM 5.3 优化：混合
HiSparse 卸载" §"与 vLLM 栈的集成"), and each query token attends over only its
own selected rows ([P3] "vLLM Hybrid HiSparse：稀疏MLA破解长上下文显存瓶颈"
§"稀疏MLA的核心思想").

* the union against an independent formulation (a two-pointer merge of the
  sorted selections, written here);
* identical scores for every query token: the union is that one selection
  and the step equals the plan-replay step (DecodeOracle.step with the same
  queries) in every output and in the hot state;
* brute force on tiny inputs: per-token selection by repeated maximum scan,
  the union as a Python set, the LRU resolve of the union and per-token
  attention in plain loops (the simulator of test_oracle_step), field by
  field every step;
* per-token outputs against torch's scaled_dot_product_attention over that
  token's own rows, and the union invariants, on random histories.
"""
import numpy as np
import pytest

from oracle import DecodeOracle, select_topk, union_of_selections
from test_oracle_step import SM, BruteRequest, brute_attention, brute_step, brute_topk, sdpa_f64, store

D, NOPE = 576, 512


def merge_union(sels):
    """Two-pointer merge of ascending lists into an ascending list without repeats."""
    cur = []
    for sel in sels:
        a, b = cur, [int(x) for x in sel if x >= 0]
        i = j = 0
        out = []
        while i < len(a) or j < len(b):
            if j == len(b) or (i < len(a) and a[i] < b[j]):
                x = a[i]; i += 1
            elif i == len(a) or b[j] < a[i]:
                x = b[j]; j += 1
            else:
                x = a[i]; i += 1; j += 1
            out.append(x)
        cur = out
    return cur


@pytest.mark.parametrize("seed", range(6))
def test_union_against_a_merge(seed):
    rng = np.random.default_rng(seed)
    L, K, Q = int(rng.integers(5, 300)), int(rng.integers(1, 40)), int(rng.integers(1, 5))
    sels = [select_topk(rng.integers(0, 6, size=L).astype(np.float32), L, K) for _ in range(Q)]
    union, upos = union_of_selections(sels, Q * K)
    m = merge_union(sels)
    assert union[:len(m)].tolist() == m and (union[len(m):] == -1).all()
    for t, sel in enumerate(sels):
        ok = sel >= 0
        assert np.array_equal(union[upos[t][ok]], sel[ok]) and (upos[t][~ok] == -1).all()
    assert max(int((s >= 0).sum()) for s in sels) <= len(m) <= sum(int((s >= 0).sum()) for s in sels)


def _oracle(rows, base, gpu, hot, ps, K, S, caps):
    return DecodeOracle(rows=rows, scales=None, kv_dtype="f32", host_base=base,
                        gpu_page=[np.asarray(g) for g in gpu], hot_pages=np.asarray(hot), page_size=ps,
                        top_k=K, hot_rows=S, ctx_capacity=caps, sm_scale=SM)


def test_identical_scores_equal_plan_replay():
    rng = np.random.default_rng(3)
    ps, k, Q, L = 8, 16, 4, 400
    rows = store(rng, 2 * L + 10)
    P = L // ps
    gpu = [np.where(rng.random(P) < 0.3, rng.permutation(P), -1) for _ in range(2)]
    hot = np.array([np.arange(200, 208), np.arange(208, 216)])
    base = [0, L + 10]
    a = _oracle(rows, base, gpu, hot, ps, Q * k, 64, [L, L])   # union capacity Q * k
    b = _oracle(rows, base, gpu, hot, ps, k, 64, [L, L])       # plan replay, top-K k
    for n in range(6):
        sc = rng.standard_normal((2, L)).astype(np.float32)
        q = rng.standard_normal((2, Q, 3, D))
        ua = a.step_union(np.repeat(sc[:, None], Q, axis=1), q, [L, L], k)
        rb = b.step(sc, q, [L, L])
        for r in range(2):
            m = int((rb["idx"][r] >= 0).sum())
            assert np.array_equal(ua["union"][r][:m], rb["idx"][r][:m]) and (ua["union"][r][m:] == -1).all()
            assert np.array_equal(ua["plan"][r][:m], rb["plan"][r][:m])
            assert np.array_equal(ua["counts"][r], rb["counts"][r])
            assert np.array_equal(a.hot[r].tag, b.hot[r].tag) and np.array_equal(a.hot[r].stamp, b.hot[r].stamp)
            assert np.array_equal(ua["out"][r], rb["out"][r]) and np.array_equal(ua["lse"][r], rb["lse"][r])
            assert np.array_equal(a.pages[r].stamp, b.pages[r].stamp)


def test_brute_force_tiny_union_steps():
    rng = np.random.default_rng(99)
    ps, k, Q, S = 4, 3, 3, 12          # union capacity Q * k = 9 <= S
    caps = [12, 10]
    base = [2, 2 + 12 + 1]
    rows = store(rng, base[1] + 10 + 1)
    hot = np.array([[30, 31, 32], [33, 34, 35]])
    gpu0 = [np.array([-1, 5, -1]), np.array([-1, -1, 6])]
    orc = _oracle(rows, base, [g.copy() for g in gpu0], hot, ps, Q * k, S, caps)
    br = [BruteRequest(base[r], S, ps, hot[r], 3) for r in range(2)]
    for r in range(2):
        br[r].give_pages(0, gpu0[r].tolist())
    sched = [[8, 7], [8, 7], [9, 9], [12, 10], [12, 10], [12, 10], [12, 10]]
    seen = set()
    for n, lens in enumerate(sched):
        if n == 3:
            orc.set_pages(0, 0, np.array([7]))
            br[0].give_pages(0, [7])
        sc = rng.standard_normal((2, Q, 12)).astype(np.float32)
        sc[0, 1, :4] = sc[0, 0, :4]        # shared and tied scores across tokens
        sc[1, 2, 5] = sc[1, 2, 6] = 2.0
        q = rng.standard_normal((2, Q, 2, D))
        got = orc.step_union(sc, q, lens, k)
        for r in range(2):
            sels = [brute_topk(sc[r][t], lens[r], k) for t in range(Q)]
            uni = sorted(set(x for s_ in sels for x in s_))
            u_sel, kinds, plan, counts, _, _ = brute_step(br[r], None, lens[r], None, rows, q[r][0], SM, sel=uni)
            tag = f"step {n + 1} req {r}"
            assert got["union"][r][:len(uni)].tolist() == uni and (got["union"][r][len(uni):] == -1).all(), tag
            for t in range(Q):
                assert got["sel"][r][t][:len(sels[t])].tolist() == sels[t], tag
                assert [uni[p] for p in got["upos"][r][t][:len(sels[t])]] == sels[t], tag
            assert got["plan"][r][:len(uni)].tolist() == plan, tag
            assert got["counts"][r].tolist() == counts, tag
            seen |= set(kinds)
            hb = orc.hot[r]
            assert hb.tag.tolist() == [-1 if x is None else x for x in br[r].holder], tag
            assert hb.stamp.tolist() == br[r].used, tag
            assert orc.pages[r].stamp.tolist() == br[r].page_last, tag
            for t in range(Q):
                o, l = brute_attention(q[r][t], [rows[base[r] + x] for x in sels[t]], SM)
                np.testing.assert_allclose(got["out"][r][t], o, rtol=1e-10, atol=1e-12)
                np.testing.assert_allclose(got["lse"][r][t], l, rtol=1e-12)
    assert seen == {"R", "H", "M"}


def test_union_invariants_and_per_token_attention():
    rng = np.random.default_rng(7)
    ps, k, Q, L = 16, 24, 4, 600
    rows = store(rng, L)
    P = -(-L // ps)
    g = np.where(rng.random(P) < 0.25, np.arange(P), -1)
    orc = _oracle(rows, [0], [g], np.arange(100, 106)[None], ps, Q * k, 96, [L])
    base_sc = rng.standard_normal(L).astype(np.float32)
    for n in range(12):
        base_sc = (0.9 * base_sc + rng.standard_normal(L)).astype(np.float32)
        sc = (base_sc[None] + 0.5 * rng.standard_normal((Q, L))).astype(np.float32)[None]
        q = rng.standard_normal((1, Q, 2, D))
        got = orc.step_union(sc, q, [L], k)
        u = got["union"][0]
        m = int((u >= 0).sum())
        assert np.all(np.diff(u[:m]) > 0) and k <= m <= Q * k
        assert got["counts"][0].sum() == m
        for t in range(Q):
            sel = got["sel"][0][t]
            assert np.array_equal(u[got["upos"][0][t]], sel)
            o, l = sdpa_f64(q[0][t], rows[sel].astype(np.float64), SM)
            np.testing.assert_allclose(got["out"][0][t], o, rtol=1e-11, atol=1e-12)
        # every union token is in the hot buffer or on a GPU page afterwards
        host = u[:m][g[u[:m] // ps] < 0]
        assert (orc.hot[0].rev[host] >= 0).all()
