"""Plain fp64 / integer CPU oracle of one sparse-MLA decode step over a
GPU/host-tiered latent KV cache. TEST INFRASTRUCTURE (see package header).

What one step computes, per request r (the pages' order):
  1. the indexer keeps only the top-K tokens for attention
     ([P3] §"稀疏MLA的核心思想"; [P2] §"解决 KV 缓存内存压力", last paragraphs);
  2. one resolve pass classifies each selected token: its page is on GPU
     (read in place), or it sits in the request's hot buffer (read there and
     its LRU entry refreshed), or it is missing (its single row is copied
     from host memory into the LRU slot of the hot buffer)
     ([P2] §"混合 HiSparse 的技术实现", state 2; [P3] §"融合内核与CUDA图兼容");
     the hot buffer is 2x top-K rows by default, made of ordinary pool
     blocks ([P2] §"关键架构细节", first bullet; [P3] §"复用现有内存池");
  3. MLA decode attention over only the K gathered latent rows
     ([P3] §"稀疏MLA的核心思想" and its MLA note: K and V share one
     low-rank latent vector per token).

Speculative steps (DecodeOracle.step_union): each query token of a request
has its own indexer scores and top-K; the union of the selections is
resolved once per step (one plan, one LRU update: the query tokens share the
request's hot state, [P2] §"与 vLLM 栈的集成", speculative decoding), and each
query token attends over its own selected rows only.

Readings where the pages are silent (each listed in the design notes):
  * top-K ties go to the lower token index; the output lists the selected
    tokens in ascending index order, padded with -1 when L < K;
  * within a step all hits refresh first, then misses take, in ascending
    token order, the least-recently-used slots among those not touched this
    step, ordered by (stamp, slot); empty slots carry stamp 0 and tag -1 and
    steps count from 1, so empty slots are used first;
  * precedence resident > hot > miss, so a stale hot copy of a page that is
    back on GPU is never read;
  * K = the full 576-dim row (512 nope + 64 rope), V = its first 512 dims;
    scores are sm_scale * <q, k>; no masking among the selected rows;
  * fp8 rows are OCP e4m3fn codes times one fp32 scale per row.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from .residency import PageState, update_residency

RESIDENT, HOT, MISS = 0, 1, 2
NOPE = 512


# --------------------------------------------------------------- top-K
def select_topk(scores: np.ndarray, L: int, K: int) -> np.ndarray:
    """Indices of the min(K, L) largest scores among scores[:L].

    Larger score first; equal scores keep the lower index (a stable sort of
    the negated scores; -0.0 and +0.0 compare equal). Returned in ascending
    index order, padded with -1 to length K.
    """
    s = np.asarray(scores[:L], dtype=np.float64)
    order = np.argsort(-s, kind="stable")
    sel = np.sort(order[:min(K, L)])
    out = np.full(K, -1, dtype=np.int64)
    out[:sel.size] = sel
    return out


def union_of_selections(sels: Sequence[np.ndarray], capacity: int):
    """Sorted union of several selections and where each selected token sits
    in it (speculative decoding with one resolve per step: the resolve plan
    of a step serves every query token of the request and they share its
    hot state, [P2] "vLLM GLM 5.3 优化：混合 HiSparse 卸载" §"与 vLLM 栈的集成").

    sels: per query token, ascending token ids padded with -1. Returns
    union [capacity] (the distinct tokens, ascending, -1 padded) and upos
    [len(sels), K] (the union position of each selected token, -1 for
    padding)."""
    toks = sorted({int(x) for sel in sels for x in np.asarray(sel) if x >= 0})
    if len(toks) > capacity:
        raise ValueError("union larger than its capacity")
    union = np.full(int(capacity), -1, dtype=np.int64)
    union[:len(toks)] = toks
    where = {x: i for i, x in enumerate(toks)}
    upos = np.array([[where[int(x)] if x >= 0 else -1 for x in np.asarray(sel)] for sel in sels],
                    dtype=np.int64)
    return union, upos


# --------------------------------------------------------------- row decode
def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (a bf16 is the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 ("fn": no infinities) codes -> float64.

    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits. Exponent
    field 0 is subnormal: (m/8) * 2^-6. Exponent 15 with mantissa 7 is NaN;
    the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def decode_rows(rows: np.ndarray, scales: Optional[np.ndarray], kv_dtype: str) -> np.ndarray:
    """Stored latent rows -> exact float64 values.

    f32 rows widen exactly; bf16 bit patterns widen exactly; fp8 rows are
    decode(code) * scale_row, formed in float64 (exact: a 4-bit significand
    times a 24-bit one).
    """
    if kv_dtype == "f32":
        return np.asarray(rows, dtype=np.float32).astype(np.float64)
    if kv_dtype == "bf16":
        return bf16_decode(rows)
    if kv_dtype == "fp8":
        return e4m3fn_decode(rows) * np.asarray(scales, dtype=np.float32).astype(np.float64)[..., None]
    raise ValueError(kv_dtype)


# --------------------------------------------------------------- attention
def mla_attention(q: np.ndarray, rows: np.ndarray, sm_scale: float):
    """Absorbed-MLA decode attention of query rows over latent rows.

    q: [n_q, 576], rows: [n, 576] (float64). Each latent row is both the key
    (all 576 dims) and the value (its first 512 dims). Returns
    out [n_q, 512] = softmax(sm_scale * q @ rows^T) @ rows[:, :512] and
    lse [n_q] = log sum_j exp(sm_scale * <q, row_j>). With n = 0 the output
    is zero and lse is -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64)
    if rows.shape[0] == 0:
        return np.zeros((q.shape[0], NOPE)), np.full(q.shape[0], -np.inf)
    s = float(sm_scale) * (q @ rows.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    out = (e @ rows[:, :NOPE]) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


# --------------------------------------------------------------- resolve
class HotBufferOracle:
    """Per-request hot buffer: S slots of leased pool rows plus LRU state.

    tag[s]   token held by slot s, or -1 when empty
    stamp[s] last step at which slot s was hit or filled (0 = never)
    rev[t]   slot holding token t, or -1
    step     per-request step counter; the n-th resolve uses stamp n
    """

    def __init__(self, slots: int, ctx_capacity: int):
        self.S = int(slots)
        self.tag = np.full(self.S, -1, dtype=np.int64)
        self.stamp = np.zeros(self.S, dtype=np.int64)
        self.rev = np.full(int(ctx_capacity), -1, dtype=np.int64)
        self.step = 0

    def reset(self):
        """Empty the buffer (a request that starts with nothing hot)."""
        held = self.tag[self.tag >= 0]
        self.rev[held] = -1
        self.tag[:] = -1
        self.stamp[:] = 0


def resolve_step(hb: HotBufferOracle, sel: np.ndarray, gpu_page: np.ndarray,
                 hot_pages: np.ndarray, page_size: int) -> Dict[str, np.ndarray]:
    """One resolve of the selected tokens of one request (mutates `hb`).

    sel: [K] ascending token ids, -1 padded. gpu_page[p]: pool page of
    logical page p, or -1 when that page lives only in host memory.
    hot_pages[i]: pool page backing hot slots [i*ps, (i+1)*ps).

    Returns plan [K] (physical pool row, -1 pad), kind [K] (RESIDENT / HOT /
    MISS, -1 pad), counts [3], and the misses as (token, slot) pairs in the
    order they were filled.
    """
    ps = int(page_size)
    hb.step += 1
    n = hb.step
    K = sel.shape[0]
    valid = sel >= 0
    t = sel[valid]
    page = t // ps
    on_gpu = gpu_page[page] >= 0
    slot_of = hb.rev[t]
    kind_v = np.where(on_gpu, RESIDENT, np.where(slot_of >= 0, HOT, MISS))

    # hits refresh their LRU entry first
    hit_slots = slot_of[kind_v == HOT]
    hb.stamp[hit_slots] = n

    # victims: slots not touched this step, oldest (stamp, slot) first
    cand = np.flatnonzero(hb.stamp < n)
    cand = cand[np.lexsort((cand, hb.stamp[cand]))]
    miss_tok = t[kind_v == MISS]           # ascending token order
    victims = cand[:miss_tok.size]
    if victims.size < miss_tok.size:
        raise RuntimeError("hot buffer smaller than the misses of one step")
    old = hb.tag[victims]
    hb.rev[old[old >= 0]] = -1
    hb.tag[victims] = miss_tok
    hb.rev[miss_tok] = victims
    hb.stamp[victims] = n

    # physical rows: a resident token is read in place from its pool page;
    # a hot or just-filled token is read from its hot slot's leased page
    plan_v = np.empty(t.size, dtype=np.int64)
    res = kind_v == RESIDENT
    plan_v[res] = gpu_page[page[res]] * ps + t[res] % ps
    slot_now = hb.rev[t[~res]]
    plan_v[~res] = hot_pages[slot_now // ps] * ps + slot_now % ps
    plan = np.full(K, -1, dtype=np.int64)
    plan[valid] = plan_v
    kind = np.full(K, -1, dtype=np.int64)
    kind[valid] = kind_v
    counts = np.array([(kind_v == RESIDENT).sum(), (kind_v == HOT).sum(),
                       (kind_v == MISS).sum()], dtype=np.int64)
    return {"plan": plan, "kind": kind, "counts": counts,
            "miss_tokens": miss_tok, "miss_slots": victims}


# --------------------------------------------------------------- one step
class DecodeOracle:
    """Runs whole decode steps for a batch of requests on plain arrays.

    rows/scales: the logical store of every token of every request (request
    r's token t is store row host_base[r] + t); it is read by logical
    position only, never through pool, hot-buffer or residency state, so
    "every tier yields the same values" holds by construction.
    """

    def __init__(self, *, rows, scales, kv_dtype: str, host_base: Sequence[int],
                 gpu_page: List[np.ndarray], hot_pages: np.ndarray, page_size: int,
                 top_k: int, hot_rows: int, ctx_capacity: Sequence[int], sm_scale):
        self.rows, self.scales, self.kv_dtype = rows, scales, kv_dtype
        self.host_base = np.asarray(host_base, dtype=np.int64)
        self.gpu_page = [np.asarray(g, dtype=np.int64).copy() for g in gpu_page]
        self.hot_pages = np.asarray(hot_pages, dtype=np.int64)
        self.ps, self.K = int(page_size), int(top_k)
        self.sm_scale = float(np.float32(sm_scale))
        self.hot = [HotBufferOracle(hot_rows, c) for c in ctx_capacity]
        # page recency and host-copy marks for the residency manager
        self.pages = [PageState(len(g)) for g in self.gpu_page]
        for r, g in enumerate(self.gpu_page):
            self.pages[r].mark_given(0, g, host_copy_valid=False)
        self.prev_len = [0] * len(self.gpu_page)

    def set_pages(self, r: int, first_page: int, gpu_ids: np.ndarray, host_copy_valid: bool = False):
        """Residency of pages [first_page, first_page + len) set from outside."""
        g = np.asarray(gpu_ids, dtype=np.int64)
        self.gpu_page[r][first_page:first_page + g.size] = g
        self.pages[r].mark_given(first_page, g, host_copy_valid)

    def update_residency(self, r: int, budget: Optional[int], max_copy: int, max_demote: int):
        return update_residency(self.pages[r], self.gpu_page[r], self.prev_len[r], self.ps,
                                budget, max_copy, max_demote)

    def logical_rows(self, r: int, tokens: np.ndarray) -> np.ndarray:
        idx = self.host_base[r] + tokens
        sc = None if self.scales is None else self.scales[idx]
        return decode_rows(self.rows[idx], sc, self.kv_dtype)

    def step_union(self, scores: np.ndarray, q: Optional[np.ndarray], lens: Sequence[int], k_per_token: int,
                   with_attention: bool = True) -> Dict[str, list]:
        """One speculative step: query token t of request r has its own
        indexer scores scores[r][t] and its own top-k_per_token selection;
        the union of a request's selections is resolved once (one plan, one
        LRU update: the query tokens share the hot state) and each query
        token attends over its own selected rows only. q [R, Q, H, 576]. The
        union capacity is the oracle's top_k."""
        R = len(lens)
        out = {"sel": [], "union": [], "upos": [], "plan": [], "kind": [], "counts": [], "out": [], "lse": []}
        for r in range(R):
            self.pages[r].enter_context(self.prev_len[r], int(lens[r]), self.hot[r].step, self.ps)
            self.prev_len[r] = int(lens[r])
            Qn = scores[r].shape[0]
            sels = [select_topk(scores[r][t], int(lens[r]), int(k_per_token)) for t in range(Qn)]
            union, upos = union_of_selections(sels, self.K)
            res = resolve_step(self.hot[r], union, self.gpu_page[r], self.hot_pages[r], self.ps)
            self.pages[r].touch(union, self.hot[r].step, self.ps)
            out["sel"].append(np.stack(sels))
            out["union"].append(union)
            out["upos"].append(upos)
            for k in ("plan", "kind", "counts"):
                out[k].append(res[k])
            if with_attention:
                qr = np.asarray(q[r], dtype=np.float64)
                os_, ls_ = [], []
                for t in range(Qn):
                    toks = sels[t][sels[t] >= 0]
                    o, lse = mla_attention(qr[t], self.logical_rows(r, toks), self.sm_scale)
                    os_.append(o)
                    ls_.append(lse)
                out["out"].append(np.stack(os_))
                out["lse"].append(np.stack(ls_))
        return out

    def step(self, scores: np.ndarray, q: np.ndarray, lens: Sequence[int],
             with_attention: bool = True) -> Dict[str, np.ndarray]:
        """scores [R, >=L], q [R, Q, H, 576] (decoded to float64 by caller
        or given as float arrays), lens [R]. Returns per-request arrays."""
        R = len(lens)
        out = {"idx": [], "plan": [], "kind": [], "counts": [], "miss_tokens": [],
               "miss_slots": [], "out": [], "lse": []}
        for r in range(R):
            # pages entering the context take the step count before this resolve
            self.pages[r].enter_context(self.prev_len[r], int(lens[r]), self.hot[r].step, self.ps)
            self.prev_len[r] = int(lens[r])
            sel = select_topk(scores[r], int(lens[r]), self.K)
            res = resolve_step(self.hot[r], sel, self.gpu_page[r], self.hot_pages[r], self.ps)
            self.pages[r].touch(sel, self.hot[r].step, self.ps)
            out["idx"].append(sel)
            for k in ("plan", "kind", "counts", "miss_tokens", "miss_slots"):
                out[k].append(res[k])
            if with_attention:
                toks = sel[sel >= 0]
                kv = self.logical_rows(r, toks)
                qr = np.asarray(q[r], dtype=np.float64)
                Qn, H = qr.shape[0], qr.shape[1]
                o, lse = mla_attention(qr.reshape(Qn * H, -1), kv, self.sm_scale)
                out["out"].append(o.reshape(Qn, H, NOPE))
                out["lse"].append(lse.reshape(Qn, H))
        return out
