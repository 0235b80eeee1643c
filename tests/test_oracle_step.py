"""Pins for the whole decode step of the oracle (DecodeOracle.step and
logical_rows), against things fixed outside the oracle:

* every page resident: the step never touches the hot buffer, counts are
  (min(K, L), 0, 0), the plan reads each row in place, and the output is
  dense attention over the same selected rows, computed by a library routine
  (torch's scaled_dot_product_attention in float64) straight from the store;
* K >= L: every token is selected and the output equals full dense MLA over
  all L rows, written as a softmax over every row by the same library
  routine, whatever the residency and hot state;
* the three tiers give one value: the same inputs under all-resident,
  all-host and mixed residency give identical outputs;
* brute force on tiny inputs: an independent per-token simulation in plain
  Python loops over dicts (selection by repeated maximum scan, sequential
  LRU scan per miss, float loops for attention) for two requests with
  non-zero host row bases, growth, residency changed mid-run and a hot
  reset, compared field by field with the oracle every step (indices, kinds,
  plan, counts, slot tags, stamps, reverse map, page stamps, host-copy marks,
  outputs and log-sum-exp).

The definition being pinned: only the top-K rows enter attention ([P3]
"vLLM Hybrid HiSparse：稀疏MLA破解长上下文显存瓶颈", §"稀疏MLA的核心思想"),
and a row read in place, from the hot buffer or copied on a miss has the same
value ([P2] "vLLM GLM 5.3 优化：混合 HiSparse 卸载", §"混合 HiSparse 的技术实现").
"""
import math

import numpy as np
import pytest
import torch

from oracle import HOT, MISS, RESIDENT, DecodeOracle

NOPE = 512
D = 576


def sdpa_f64(q: np.ndarray, kv: np.ndarray, sm_scale: float):
    """Library attention: q [n_q, 576] over rows kv [n, 576] (K = rows,
    V = rows[:, :512]) in float64; returns out [n_q, 512] and lse [n_q]."""
    qt = torch.from_numpy(np.asarray(q, dtype=np.float64))[None, None]
    kt = torch.from_numpy(np.asarray(kv, dtype=np.float64))[None, None]
    vt = kt[..., :NOPE].contiguous()
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=sm_scale)[0, 0]
    s = sm_scale * (qt[0, 0] @ kt[0, 0].T)
    lse = torch.logsumexp(s, dim=-1)
    return out.numpy(), lse.numpy()


def make_oracle(rows, host_base, gpu_page, hot_pages, ps, K, S, caps, sm_scale, kv="f32", scales=None):
    return DecodeOracle(rows=rows, scales=scales, kv_dtype=kv, host_base=host_base,
                        gpu_page=[np.asarray(g) for g in gpu_page], hot_pages=np.asarray(hot_pages),
                        page_size=ps, top_k=K, hot_rows=S, ctx_capacity=caps, sm_scale=sm_scale)


def store(rng, n):
    sig = np.exp(0.5 * rng.standard_normal(n)).astype(np.float32)
    return (rng.standard_normal((n, D)).astype(np.float32) * sig[:, None]).astype(np.float32)


SM = float(np.float32(1.0 / 24.0))


# ----------------------------------------------------------------- all resident
def test_all_resident_equals_dense_over_selected_rows():
    rng = np.random.default_rng(11)
    ps, K, S, L = 16, 32, 64, 300
    base = [7, 7 + L + 5]
    rows = store(rng, base[1] + L + 2)
    P = -(-L // ps)
    gpu = [rng.permutation(1000)[:P], 1000 + rng.permutation(1000)[:P]]
    hot = np.array([[2000, 2001, 2002, 2003], [2004, 2005, 2006, 2007]])
    orc = make_oracle(rows, base, gpu, hot, ps, K, S, [L, L], SM)
    for n in range(4):
        sc = rng.standard_normal((2, L)).astype(np.float32)
        q = rng.standard_normal((2, 2, 3, D))
        out = orc.step(sc, q, [L, L])
        for r in range(2):
            sel = out["idx"][r]
            assert (sel >= 0).all() and np.all(np.diff(sel) > 0)
            assert out["counts"][r].tolist() == [K, 0, 0]
            assert (out["kind"][r] == RESIDENT).all()
            assert np.array_equal(out["plan"][r], gpu[r][sel // ps] * ps + sel % ps)
            # the hot buffer is never touched, but the step counter advances
            assert (orc.hot[r].tag == -1).all() and (orc.hot[r].stamp == 0).all()
            assert orc.hot[r].step == n + 1
            kv = rows[base[r] + sel].astype(np.float64)
            o_ref, l_ref = sdpa_f64(q[r].reshape(-1, D), kv, SM)
            np.testing.assert_allclose(out["out"][r].reshape(-1, NOPE), o_ref, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(out["lse"][r].reshape(-1), l_ref, rtol=1e-12, atol=0)


# ----------------------------------------------------------------- K >= L
@pytest.mark.parametrize("L", [1, 5, 40, 64])
def test_k_ge_len_is_full_dense_mla(L):
    rng = np.random.default_rng(100 + L)
    ps, K, S = 8, 64, 128
    base = [3]
    rows = store(rng, 3 + L + 1)
    P = -(-L // ps)
    g = np.where(rng.random(P) < 0.5, rng.permutation(50)[:P], -1)
    orc = make_oracle(rows, base, [g], np.arange(60, 60 + S // ps)[None], ps, K, S, [L], SM)
    full = rows[3:3 + L].astype(np.float64)
    n_host = int(sum(min(ps, L - p * ps) for p in range(P) if g[p] < 0))
    for n in range(3):
        sc = rng.standard_normal((1, L)).astype(np.float32)
        q = rng.standard_normal((1, 1, 4, D))
        out = orc.step(sc, q, [L])
        assert out["idx"][0][:L].tolist() == list(range(L)) and (out["idx"][0][L:] == -1).all()
        c = out["counts"][0].tolist()
        # first step: every host token misses; afterwards all of them are hot
        assert c == ([L - n_host, 0, n_host] if n == 0 else [L - n_host, n_host, 0])
        o_ref, l_ref = sdpa_f64(q[0].reshape(-1, D), full, SM)
        np.testing.assert_allclose(out["out"][0].reshape(-1, NOPE), o_ref, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(out["lse"][0].reshape(-1), l_ref, rtol=1e-12)


# ----------------------------------------------------------------- tiers agree
def test_residency_does_not_change_values():
    rng = np.random.default_rng(5)
    ps, K, S, L = 8, 24, 48, 200
    rows = store(rng, L)
    P = L // ps
    layouts = {
        "resident": np.arange(P),
        "host": np.full(P, -1),
        "mixed": np.where(np.arange(P) % 3 == 0, np.arange(P), -1),
    }
    orcs = {k: make_oracle(rows, [0], [g], np.arange(500, 506)[None], ps, K, S, [L], SM)
            for k, g in layouts.items()}
    kinds_seen = set()
    for n in range(5):
        sc = rng.standard_normal((1, L)).astype(np.float32)
        q = rng.standard_normal((1, 1, 2, D))
        outs = {k: o.step(sc, q, [L]) for k, o in orcs.items()}
        for k, o in outs.items():
            kinds_seen |= set(o["kind"][0].tolist())
            assert np.array_equal(o["idx"][0], outs["resident"]["idx"][0])
            assert np.array_equal(o["out"][0], outs["resident"]["out"][0]), k
            assert np.array_equal(o["lse"][0], outs["resident"]["lse"][0]), k
    assert kinds_seen == {RESIDENT, HOT, MISS}


# ----------------------------------------------------------------- brute force
class BruteRequest:
    """One request's state as plain Python containers."""

    def __init__(self, base, S, ps, hot_pages, pages):
        self.base, self.S, self.ps = base, S, ps
        self.hot_pages = [int(x) for x in hot_pages]
        self.holder = [None] * S       # token held by each slot
        self.used = [0] * S            # step of the slot's last hit or fill
        self.where = {}                # token -> slot
        self.done = 0                  # resolves completed
        self.length = 0
        self.on_gpu = {}               # logical page -> pool page (absent: host only)
        self.page_last = [0] * pages   # page recency stamp
        self.copied = [False] * pages  # host store holds the page

    def give_pages(self, first, ids, host_copy_valid=False):
        for i, g in enumerate(ids):
            p = first + i
            if g >= 0:
                self.on_gpu[p] = int(g)
            else:
                self.on_gpu.pop(p, None)
            self.copied[p] = g < 0 or host_copy_valid

    def reset_hot(self):
        self.holder = [None] * self.S
        self.used = [0] * self.S
        self.where = {}


def brute_topk(scores, L, K):
    chosen = []
    for _ in range(min(K, L)):
        best = None
        for t in range(L):
            if t in chosen:
                continue
            if best is None or float(scores[t]) > float(scores[best]):  # ties keep the lower index
                best = t
        chosen.append(best)
    return sorted(chosen)


def brute_attention(qrows, kv, sm):
    outs, lses = [], []
    for qv in qrows:
        s = []
        for row in kv:
            acc = 0.0
            for d in range(D):
                acc += float(qv[d]) * float(row[d])
            s.append(sm * acc)
        m = max(s)
        w = [math.exp(x - m) for x in s]
        tot = sum(w)
        o = [0.0] * NOPE
        for wj, row in zip(w, kv):
            for d in range(NOPE):
                o[d] += wj * float(row[d])
        outs.append([x / tot for x in o])
        lses.append(m + math.log(tot))
    return np.array(outs), np.array(lses)


def brute_step(rq: BruteRequest, scores, L, K, rows, qrows, sm, sel=None):
    """One step of one request; `sel` (ascending tokens) replaces the top-K
    of `scores` when given (the union of several selections)."""
    ps = rq.ps
    for p in range(-(-rq.length // ps), -(-L // ps)):
        rq.page_last[p] = rq.done          # entering pages take the count so far
    rq.length = L
    if sel is None:
        sel = brute_topk(scores, L, K)
    rq.done += 1
    n = rq.done
    kind = {}
    for t in sel:
        if (t // ps) in rq.on_gpu:
            kind[t] = "R"
        elif t in rq.where:
            kind[t] = "H"
        else:
            kind[t] = "M"
    for t in sel:
        if kind[t] == "H":
            rq.used[rq.where[t]] = n
    for t in sel:                           # ascending token order
        if kind[t] != "M":
            continue
        best = None
        for s in range(rq.S):               # least recent slot not touched at n
            if rq.used[s] >= n:
                continue
            if best is None or rq.used[s] < rq.used[best]:
                best = s
        old = rq.holder[best]
        if old is not None:
            del rq.where[old]
        rq.holder[best] = t
        rq.where[t] = best
        rq.used[best] = n
    plan = []
    for t in sel:
        if kind[t] == "R":
            plan.append(rq.on_gpu[t // ps] * ps + t % ps)
        else:
            s = rq.where[t]
            plan.append(rq.hot_pages[s // ps] * ps + s % ps)
    for t in sel:
        rq.page_last[t // ps] = n
    counts = [sum(1 for t in sel if kind[t] == c) for c in "RHM"]
    kv = [rows[rq.base + t] for t in sel]
    o, l = brute_attention(qrows, kv, sm) if kv else (None, None)
    return sel, [kind[t] for t in sel], plan, counts, o, l


def test_brute_force_tiny_steps():
    rng = np.random.default_rng(2024)
    ps, K, S = 4, 3, 4                      # one hot page: evictions on most steps
    caps = [12, 11]
    base = [5, 5 + 12 + 3]                   # store rows before, between and after the requests
    rows = store(rng, base[1] + 11 + 2)
    pages = [3, 3]
    hot = np.array([[40], [42]])
    gpu0 = [np.array([-1, 7, -1]), np.array([-1, -1, 9])]
    orc = make_oracle(rows, base, [g.copy() for g in gpu0], hot, ps, K, S, caps, SM)
    br = [BruteRequest(base[r], S, ps, hot[r], pages[r]) for r in range(2)]
    for r in range(2):
        br[r].give_pages(0, gpu0[r].tolist())
    sched = [[7, 6], [7, 6], [8, 9], [8, 9], [10, 9], [12, 11], [12, 11], [12, 11], [12, 11], [12, 11]]
    kinds_seen = set()
    evictions = 0
    for n, lens in enumerate(sched):
        if n == 4:                         # page 1 of request 0 leaves the GPU; page 0 of request 1 arrives
            orc.set_pages(0, 1, np.array([-1]))
            br[0].give_pages(1, [-1])
            orc.set_pages(1, 0, np.array([11]), host_copy_valid=True)
            br[1].give_pages(0, [11], host_copy_valid=True)
        if n == 7:                         # request 1 starts again with an empty hot buffer
            orc.hot[1].reset()
            br[1].reset_hot()
        sc = rng.standard_normal((2, 12)).astype(np.float32)
        sc[0, 2] = sc[0, 5] = sc[0, 6] = 1.5          # exact ties
        if n % 3 == 0:
            sc[1, :3] = 0.0
            sc[1, 3] = -0.0
        q = rng.standard_normal((2, 2, 2, D))
        got = orc.step(sc, q, lens)
        for r in range(2):
            evictions += sum(1 for x in br[r].holder if x is not None) == S
            sel, kinds, plan, counts, o, l = brute_step(br[r], sc[r], lens[r], K, rows,
                                                        q[r].reshape(-1, D), SM)
            tag = f"step {n + 1} req {r}"
            m = len(sel)
            assert got["idx"][r][:m].tolist() == sel and (got["idx"][r][m:] == -1).all(), tag
            code = {RESIDENT: "R", HOT: "H", MISS: "M"}
            assert [code[k] for k in got["kind"][r][:m].tolist()] == kinds, tag
            kinds_seen |= set(kinds)
            assert got["plan"][r][:m].tolist() == plan, tag
            assert got["counts"][r].tolist() == counts, tag
            assert sum(counts) == min(K, lens[r])
            hb = orc.hot[r]
            assert hb.tag.tolist() == [-1 if x is None else x for x in br[r].holder], tag
            assert hb.stamp.tolist() == br[r].used, tag
            for t in range(caps[r]):
                assert hb.rev[t] == br[r].where.get(t, -1), tag
            assert hb.step == br[r].done
            assert orc.pages[r].stamp.tolist() == br[r].page_last, tag
            assert orc.pages[r].host_valid.tolist() == br[r].copied, tag
            np.testing.assert_allclose(got["out"][r].reshape(-1, NOPE), o, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(got["lse"][r].reshape(-1), l, rtol=1e-12)
    assert kinds_seen == {"R", "H", "M"}
    assert evictions >= 5


def test_counts_sum_over_a_long_history():
    """resident + hot + miss = min(K, L) on every step of a growing request
    whose residency changes, and every host-only selected token is in the hot
    buffer afterwards."""
    rng = np.random.default_rng(77)
    ps, K, S = 8, 16, 32
    cap = 400
    rows = store(rng, cap)
    P = cap // ps
    g = np.where(rng.random(P) < 0.4, np.arange(P), -1)
    orc = make_oracle(rows, [0], [g], np.arange(100, 104)[None], ps, K, S, [cap], SM)
    L = 10
    for n in range(80):
        L = min(cap, L + int(rng.integers(0, 7)))
        if n % 17 == 16:
            p = int(rng.integers(0, P))
            orc.set_pages(0, p, np.array([-1 if orc.gpu_page[0][p] >= 0 else 300 + p]))
        sc = rng.standard_normal((1, cap)).astype(np.float32)
        out = orc.step(sc, None, [L], with_attention=False)
        assert out["counts"][0].sum() == min(K, L)
        sel = out["idx"][0][out["idx"][0] >= 0]
        host_sel = sel[orc.gpu_page[0][sel // ps] < 0]
        assert (orc.hot[0].rev[host_sel] >= 0).all()
        hb = orc.hot[0]
        held = hb.tag[hb.tag >= 0]
        assert np.array_equal(hb.rev[held], np.flatnonzero(hb.tag >= 0))
        # the reverse map names a slot only for the token that slot holds
        where = np.flatnonzero(hb.rev >= 0)
        assert np.array_equal(hb.tag[hb.rev[where]], where)
