"""Seeded synthetic workloads for the tiered sparse-MLA decode step.

This module only *generates inputs*: it holds none of the method's
arithmetic (no top-K, no residency classification, no LRU, no attention).
Both the CPU oracle (through the tests) and the HIP path (through the
binding, the tests and the benchmark) consume the exact bytes it produces.

Shapes follow the pages' description of the method:
  * latent MLA rows of 512 "nope" + 64 "rope" dims, one per token
    (page 3, "The core idea of sparse MLA" and the MLA note below it);
  * a paged KV pool with 64-token pages (page 3, the PagedAttention note);
  * a per-request GPU/host residency per page (page 2, "Technical
    implementation of Hybrid HiSparse", the three residency states);
  * a per-request hot buffer of 2x top-K rows leased from the pool
    (page 2, "Key architecture details", first bullet);
  * the agent workload shape: 74,160-token first turn, 753-token later
    turns, 220 output tokens, MTP with 3 drafts (page 2, "Performance
    benchmarking").

Recipe (all draws seeded; every array is produced once on the host):
  * master seed = 20261202 + c for workload c in 1..6;
    ``numpy.random.SeedSequence(seed).spawn(6)`` gives independent streams
    for scores, rows, queries, page placement, context lengths and topic
    shifts; the rows stream is split again per request and per chunk of
    65,536 rows;
  * latent row t: x = sigma_t * z, z ~ N(0,1)^576, sigma_t = exp(0.5*N(0,1))
    (per-row log-normal magnitude so per-row fp8 scales differ); stored as
    fp32, bf16 (round-to-nearest-even) or OCP fp8 e4m3fn codes with one fp32
    scale per row (scale = amax/448, values clamped to +-448, RNE);
  * queries N(0,1), fresh every step, fp32 or bf16;
  * indexer scores fp32: i.i.d. N(0,1), or a per-token AR(1) chain
    s <- rho*s + eps (eps ~ N(0,1)) whose first value is drawn from the
    stationary law N(0, 1/(1-rho^2)); the 1M workload redraws every chain
    from the stationary law on 5% of steps (topic shift);
  * GPU pages sit at pool page ids taken from a seeded permutation, so the
    row gathers are scattered; each request leases hot_rows/page_size pool
    pages for its hot buffer from the same permutation.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import math
import os
from typing import Dict, List, Optional, Tuple

import numpy as np

NOPE_DIM = 512
ROPE_DIM = 64
ROW_DIM = NOPE_DIM + ROPE_DIM
PAGE_SIZE = 64
FP8_MAX = 448.0
MASTER_SEED = 20261202
ROW_CHUNK = 65536  # rows generated per draw call (part of the recipe)

KV_F32, KV_BF16, KV_FP8 = "f32", "bf16", "fp8"


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    """One synthetic workload: shapes, dtypes, residency and score process."""

    name: str
    index: int              # 1..5, selects the master seed
    n_req: int
    kv_dtype: str           # f32 | bf16 | fp8
    q_dtype: str            # f32 | bf16
    heads: int
    q_per_req: int
    top_k: int
    hot_rows: int
    steps: int
    residency: str          # see _gpu_page_mask
    scores: Tuple           # ("iid",) | ("ar1", rho) | ("ar1_shift", rho, p)
    ctx: Optional[int] = None          # fixed context length, or None
    ctx_range: Optional[Tuple[int, int]] = None  # uniform integer range
    host_pages: Optional[int] = None   # oldest pages on host (fixed-ctx specs)
    growth: Optional[Tuple[int, int, int, int]] = None  # first, later, out, turns
    gpu_token_budget: Optional[int] = None  # newest tokens on GPU per request
    page_size: int = PAGE_SIZE
    # Multi-layer step: n_req counts request slots, layer-major (slot =
    # layer * n_req // layers + request); every slot has its own rows, page
    # table, hot buffer, scores and queries, and the slots of one request
    # share its context length.
    layers: int = 1
    # Speculative steps with a selection per query token: each of the
    # q_per_req query tokens selects select_k tokens (top_k is then the
    # union capacity, >= q_per_req * select_k); query token 0 has the
    # request's score chain, token t >= 1 that chain plus N(0, token_noise^2)
    # drawn afresh every step.
    select_k: Optional[int] = None
    token_noise: float = 0.0

    @property
    def seed(self) -> int:
        return MASTER_SEED + self.index


# The five workloads. Sizes in tokens use 1K = 1024.
SPECS: Dict[str, WorkloadSpec] = {
    "tiny": WorkloadSpec(
        name="tiny", index=1, n_req=1, ctx=4096, kv_dtype=KV_F32, q_dtype="f32",
        heads=16, q_per_req=1, top_k=256, hot_rows=512, steps=8,
        residency="oldest_host", host_pages=48, scores=("iid",)),
    "single-128k": WorkloadSpec(
        name="single-128k", index=2, n_req=1, ctx=131072, kv_dtype=KV_BF16,
        q_dtype="bf16", heads=128, q_per_req=1, top_k=2048, hot_rows=4096,
        steps=64, residency="oldest_host", host_pages=1536,
        scores=("ar1", 0.9)),
    "batch32": WorkloadSpec(
        name="batch32", index=3, n_req=32, ctx_range=(16384, 262144),
        kv_dtype=KV_BF16, q_dtype="bf16", heads=128, q_per_req=1, top_k=2048,
        hot_rows=4096, steps=32, residency="mod3", scores=("ar1", 0.9)),
    "single-1m-fp8": WorkloadSpec(
        name="single-1m-fp8", index=4, n_req=1, ctx=1048576, kv_dtype=KV_FP8,
        q_dtype="bf16", heads=128, q_per_req=1, top_k=2048, hot_rows=4096,
        steps=128, residency="oldest_host", host_pages=14745,
        scores=("ar1_shift", 0.95, 0.05)),
    "agent16": WorkloadSpec(
        name="agent16", index=5, n_req=16, kv_dtype=KV_FP8, q_dtype="bf16",
        heads=128, q_per_req=4, top_k=2048, hot_rows=4096, steps=715,
        residency="budget", gpu_token_budget=145408, growth=(74160, 753, 220, 13),
        scores=("ar1", 0.9)),
    # Multi-layer step: the sparse-MLA work of 16 layers of one 128K-token
    # request (fp8 rows, 75% of each layer's pages on the host) in one call
    # of each entry point.
    "layers16-128k-fp8": WorkloadSpec(
        name="layers16-128k-fp8", index=6, n_req=16, layers=16, ctx=131072,
        kv_dtype=KV_FP8, q_dtype="bf16", heads=128, q_per_req=1, top_k=2048,
        hot_rows=4096, steps=32, residency="oldest_host", host_pages=1536,
        scores=("ar1", 0.9)),
    # Aggregate reading of the 142K admission limit: 9,088 newest tokens
    # (142 pages) of each of the 16 requests stay on GPU.
    "agent16-b": WorkloadSpec(
        name="agent16-b", index=5, n_req=16, kv_dtype=KV_FP8, q_dtype="bf16",
        heads=128, q_per_req=4, top_k=2048, hot_rows=4096, steps=715,
        residency="budget", gpu_token_budget=9088, growth=(74160, 753, 220, 13),
        scores=("ar1", 0.9)),
    # Speculative steps with one top-K per query token (1 + 3 drafts, 1,024
    # tokens each) and one resolve of their union (capacity 4,096) per step;
    # the agent shape with the aggregate GPU budget, so that misses occur.
    "agent16-union": WorkloadSpec(
        name="agent16-union", index=7, n_req=16, kv_dtype=KV_FP8, q_dtype="bf16",
        heads=128, q_per_req=4, top_k=4096, hot_rows=4096, steps=715,
        residency="budget", gpu_token_budget=9088, growth=(74160, 753, 220, 13),
        scores=("ar1", 0.9), select_k=1024, token_noise=0.5),
}


def row_bytes(kv_dtype: str) -> int:
    """Bytes of one stored row payload (the fp8 scale is stored apart)."""
    return {KV_F32: 4 * ROW_DIM, KV_BF16: 2 * ROW_DIM, KV_FP8: ROW_DIM}[kv_dtype]


# ---------------------------------------------------------------- encodings
# Pure numpy (no torch), so the row generator's worker threads call no
# library with thread pools or lazy initialisation of its own. Both are
# checked bit for bit against torch's conversions in the CPU tests.
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even) and return the
    raw 16-bit patterns (NaN -> the quiet NaN 0x7FC0 with its sign)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) & np.uint32(0x8000)).astype(np.uint16) | np.uint16(0x7FC0)
    return r


_FP8_MIN_NORMAL = np.float32(2.0 ** -6)


def _e4m3fn_codes(y: np.ndarray) -> np.ndarray:
    """OCP e4m3fn codes of fp32 values with |y| <= 448, round to nearest,
    ties to even. Normal results (|y| >= 2^-6) keep the fp32 exponent and
    the top 3 mantissa bits after rounding the fp32 pattern at bit 20;
    subnormal results are multiples of 2^-9, so their code is rint(|y|*2^9)
    (0..8, where 8 is the smallest normal, code 0x08)."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    a = np.abs(y)
    u = a.view(np.uint32)
    r = (u + (np.uint32(0x7FFFF) + ((u >> np.uint32(20)) & np.uint32(1)))) >> np.uint32(20)
    normal = ((r >> np.uint32(3)) - np.uint32(120)) << np.uint32(3) | (r & np.uint32(7))
    sub = np.rint(a * np.float32(512.0)).astype(np.uint32)
    code = np.where(a < _FP8_MIN_NORMAL, sub, normal).astype(np.uint8)
    return code | ((y.view(np.uint32) >> np.uint32(24)) & np.uint32(0x80)).astype(np.uint8)


def f32_rows_to_fp8(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Encode rows as OCP e4m3fn codes with one fp32 scale per row."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0))
    scale = scale.astype(np.float32)
    y = np.clip(x / scale[:, None], -FP8_MAX, FP8_MAX).astype(np.float32)
    return _e4m3fn_codes(y), scale


# ---------------------------------------------------------------- schedules
def context_schedule(spec: WorkloadSpec, ctx0: np.ndarray, steps: int) -> np.ndarray:
    """Context length of every request at decode steps 1..steps, [steps, R].

    Fixed-length workloads keep ctx0. The agent workload grows: turn 1 is
    the first prompt; each turn emits out/Q steps that commit Q tokens each;
    turns 2.. add a prompt of `later` tokens before their first step.
    """
    R = ctx0.shape[0]
    if spec.growth is None:
        return np.broadcast_to(ctx0, (steps, R)).astype(np.int64).copy()
    first, later, out, turns = spec.growth
    per_turn = out // spec.q_per_req
    lens = []
    cur = first
    for turn in range(turns):
        if turn > 0:
            cur += later
        for _ in range(per_turn):
            lens.append(cur)
            cur += spec.q_per_req
    lens = np.asarray(lens, dtype=np.int64)
    if steps > lens.size:
        raise ValueError(f"{spec.name} defines {lens.size} steps")
    return np.broadcast_to(lens[:steps, None], (steps, R)).copy()


def final_context(spec: WorkloadSpec, ctx0: np.ndarray) -> np.ndarray:
    """Largest context each request reaches over its full schedule."""
    if spec.growth is None:
        return ctx0.copy()
    first, later, out, turns = spec.growth
    total = first + (turns - 1) * later + turns * out
    return np.full_like(ctx0, total)


@dataclasses.dataclass
class Workload:
    """Generated inputs of one workload (host arrays only)."""

    spec: WorkloadSpec
    ctx0: np.ndarray            # [R] context at step 1
    ctx_final: np.ndarray       # [R] largest context over the run
    host_base: np.ndarray       # [R] int64 first row of request r in the store
    rows: np.ndarray            # logical store: f32 [N,576] | u16 [N,576] | u8 [N,576]
    scales: Optional[np.ndarray]  # fp8 only: f32 [N]
    gpu_page: List[np.ndarray]  # per request: int32 [pages(final)], pool page or -1
    hot_pages: np.ndarray       # [R, hot_rows/page_size] int32 pool pages
    num_pool_pages: int
    sm_scale: np.float32
    _streams: Dict[str, np.random.Generator] = dataclasses.field(repr=False, default_factory=dict)

    @property
    def n_req(self) -> int:
        return self.spec.n_req

    @property
    def max_context(self) -> int:
        return int(self.ctx_final.max())

    def row_slice(self, r: int) -> slice:
        b = int(self.host_base[r])
        return slice(b, b + int(self.ctx_final[r]))


def _gpu_page_mask(spec: WorkloadSpec, ctx_final: np.ndarray, r: int) -> np.ndarray:
    """Which logical pages of request r start on GPU (True) vs host."""
    P = -(-int(ctx_final[r]) // spec.page_size)
    mask = np.zeros(P, dtype=bool)
    if spec.residency == "oldest_host":
        mask[spec.host_pages:] = True
    elif spec.residency == "mod3":
        kind = r % 3
        if kind == 0:
            mask[:] = True
        elif kind == 1:
            n_gpu = math.ceil(0.25 * P)
            mask[P - n_gpu:] = True
        # kind 2: none resident
    elif spec.residency == "budget":
        n_gpu = min(P, -(-spec.gpu_token_budget // spec.page_size))
        mask[P - n_gpu:] = True
    else:
        raise ValueError(spec.residency)
    return mask


def generate(spec: WorkloadSpec) -> Workload:
    """Build the host-side inputs of `spec` (rows, residency, placement).

    Scores and queries are drawn step by step with `ScoreStream` and
    `QueryStream`. Reduced variants for quick tests are plain
    ``dataclasses.replace`` copies of a spec.
    """
    ss = np.random.SeedSequence(spec.seed).spawn(6)
    gens = {k: np.random.Generator(np.random.PCG64(s)) for k, s in
            zip(("scores", "rows", "queries", "pages", "contexts", "shifts"), ss)}
    R = spec.n_req
    if spec.n_req % spec.layers:
        raise ValueError("n_req must be a multiple of layers")
    if spec.ctx_range is not None:
        lo, hi = spec.ctx_range
        per = gens["contexts"].integers(lo, hi, endpoint=True, size=R // spec.layers).astype(np.int64)
        ctx0 = np.tile(per, spec.layers)
    elif spec.growth is not None:
        ctx0 = np.full(R, spec.growth[0], dtype=np.int64)
    else:
        ctx0 = np.full(R, spec.ctx, dtype=np.int64)
    ctx_final = final_context(spec, ctx0)
    host_base = np.zeros(R, dtype=np.int64)
    host_base[1:] = np.cumsum(ctx_final)[:-1]
    N = int(ctx_final.sum())

    # latent rows: request r, chunk c (ROW_CHUNK rows) draws from its own
    # stream rows_seq.spawn(R)[r].spawn(n_chunks_r)[c], so chunks can be
    # generated in parallel
    if spec.kv_dtype == KV_F32:
        rows = np.empty((N, ROW_DIM), dtype=np.float32)
    elif spec.kv_dtype == KV_BF16:
        rows = np.empty((N, ROW_DIM), dtype=np.uint16)
    else:
        rows = np.empty((N, ROW_DIM), dtype=np.uint8)
    scales = np.empty(N, dtype=np.float32) if spec.kv_dtype == KV_FP8 else None
    tasks = []
    for r, rss in enumerate(ss[1].spawn(R)):
        n_r = int(ctx_final[r])
        nch = -(-n_r // ROW_CHUNK)
        for c, css in enumerate(rss.spawn(nch)):
            start = int(host_base[r]) + c * ROW_CHUNK
            tasks.append((css, start, min(ROW_CHUNK, n_r - c * ROW_CHUNK)))

    def fill(task):
        css, start, n = task
        g = np.random.Generator(np.random.PCG64(css))
        sigma = np.exp(0.5 * g.standard_normal(n, dtype=np.float32)).astype(np.float32)
        x = g.standard_normal((n, ROW_DIM), dtype=np.float32) * sigma[:, None]
        if spec.kv_dtype == KV_F32:
            rows[start:start + n] = x
        elif spec.kv_dtype == KV_BF16:
            rows[start:start + n] = f32_to_bf16_bits(x)
        else:
            c8, sc = f32_rows_to_fp8(x)
            rows[start:start + n] = c8
            scales[start:start + n] = sc

    with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, tasks))

    # residency and pool placement
    ps = spec.page_size
    masks = [_gpu_page_mask(spec, ctx_final, r) for r in range(R)]
    hot_per_req = spec.hot_rows // ps
    total = int(sum(m.sum() for m in masks)) + R * hot_per_req
    perm = gens["pages"].permutation(total).astype(np.int32)
    cur = 0
    hot_pages = np.empty((R, hot_per_req), dtype=np.int32)
    gpu_page = []
    for r in range(R):
        hot_pages[r] = perm[cur:cur + hot_per_req]
        cur += hot_per_req
        g = np.full(masks[r].size, -1, dtype=np.int32)
        k = int(masks[r].sum())
        g[masks[r]] = perm[cur:cur + k]
        cur += k
        gpu_page.append(g)
    wl = Workload(spec=spec, ctx0=ctx0, ctx_final=ctx_final, host_base=host_base,
                  rows=rows, scales=scales, gpu_page=gpu_page, hot_pages=hot_pages,
                  num_pool_pages=total, sm_scale=np.float32(1.0 / math.sqrt(ROW_DIM)))
    wl._streams = gens
    return wl


class ScoreStream:
    """Per-step indexer scores, [R, max_context] fp32 (zero past each L_r)."""

    def __init__(self, wl: Workload, ctx_sched: Optional[np.ndarray] = None):
        self.wl = wl
        self.g = wl._streams["scores"]
        self.shift_g = wl._streams["shifts"]
        self.proc = wl.spec.scores
        self.state: List[Optional[np.ndarray]] = [None] * wl.n_req
        self.n = 0
        self.shift_steps: List[int] = []

    def planned_shift_steps(self, steps: int) -> List[int]:
        """Steps n <= `steps` (counted from 1) at which the topic-shift draw
        redraws every score, from a copy of the shift stream's state (the
        stream itself is not advanced); [] without topic shifts."""
        if self.proc[0] != "ar1_shift":
            return []
        g = np.random.Generator(np.random.PCG64())
        g.bit_generator.state = self.shift_g.bit_generator.state
        out = []
        for n in range(max(self.n + 1, 2), steps + 1):
            if g.random() < self.proc[2]:
                out.append(n)
        return out

    def next_tokens(self, lens: np.ndarray) -> np.ndarray:
        """Per-query-token scores [R, Q, max_context] of the next
        speculative step (token_scores of the next request scores)."""
        return token_scores(self.wl, self.next(lens), lens, self.g)

    def next(self, lens: np.ndarray) -> np.ndarray:
        """Scores of the next step for context lengths `lens` [R]."""
        self.n += 1
        R = self.wl.n_req
        out = np.zeros((R, self.wl.max_context), dtype=np.float32)
        kind = self.proc[0]
        if kind == "iid":
            for r in range(R):
                out[r, :lens[r]] = self.g.standard_normal(int(lens[r]), dtype=np.float32)
            return out
        rho = np.float32(self.proc[1])
        sd = np.float32(1.0 / math.sqrt(1.0 - float(rho) ** 2))
        shift = False
        if kind == "ar1_shift" and self.n >= 2:
            shift = bool(self.shift_g.random() < self.proc[2])
            if shift:
                self.shift_steps.append(self.n)
        for r in range(R):
            L = int(lens[r])
            prev = self.state[r]
            if prev is None or shift:
                s = self.g.standard_normal(L, dtype=np.float32) * sd
            else:
                k = min(prev.size, L)
                s = np.empty(L, dtype=np.float32)
                s[:k] = rho * prev[:k] + self.g.standard_normal(k, dtype=np.float32)
                if L > k:  # new tokens start from the stationary law
                    s[k:] = self.g.standard_normal(L - k, dtype=np.float32) * sd
            self.state[r] = s
            out[r, :L] = s
        return out


def token_scores(wl: Workload, base: np.ndarray, lens: np.ndarray, g: np.random.Generator) -> np.ndarray:
    """Per-query-token scores [R, Q, max_context] of a speculative step from
    the request scores `base` [R, max_context]: token 0 keeps them, token
    t >= 1 adds N(0, token_noise^2) noise over each request's first lens[r]."""
    s = wl.spec
    R, Q = base.shape[0], s.q_per_req
    out = np.repeat(base[:, None, :], Q, axis=1)
    for r in range(R):
        n = int(lens[r])
        for t in range(1, Q):
            out[r, t, :n] += (np.float32(s.token_noise) *
                              g.standard_normal(n, dtype=np.float32)).astype(np.float32)
    return out


class QueryStream:
    """Per-step absorbed queries [R, Q, H, 576]: fp32 array or bf16 bits."""

    def __init__(self, wl: Workload):
        self.wl = wl
        self.g = wl._streams["queries"]

    def next(self) -> np.ndarray:
        s = self.wl.spec
        q = self.g.standard_normal((s.n_req, s.q_per_req, s.heads, ROW_DIM), dtype=np.float32)
        if s.q_dtype == "bf16":
            return f32_to_bf16_bits(q)
        return q


# ---------------------------------------------------------------- indexer inputs
INDEXER_DIM = 128
INDEXER_HEADS = 64


class IndexerInputs:
    """Synthetic inputs of the indexer score step (no method arithmetic).

    Per request slot r: indexer keys [capacity, 128] as bf16 bits, drawn
    N(0, 1) per element from the request's own stream. Per step: indexer
    queries [R, H, 128] (bf16 bits, N(0, 1)) and head weights [R, H] (fp32,
    N(0, 1) / sqrt(H)). Seeded from the workload's master seed with a stream
    of its own, so the latent-row and score streams are unchanged.
    """

    def __init__(self, seed: int, n_req: int, capacity: np.ndarray, heads: int = INDEXER_HEADS):
        ss = np.random.SeedSequence([seed, 7]).spawn(2)
        self.heads = heads
        self.n_req = n_req
        self.capacity = np.asarray(capacity, dtype=np.int64)
        self.keys = []
        for r, rs in enumerate(ss[0].spawn(n_req)):
            g = np.random.Generator(np.random.PCG64(rs))
            k = g.standard_normal((int(self.capacity[r]), INDEXER_DIM), dtype=np.float32)
            self.keys.append(f32_to_bf16_bits(k))
        self.g = np.random.Generator(np.random.PCG64(ss[1]))

    def next(self) -> Tuple[np.ndarray, np.ndarray]:
        """(queries as bf16 bits [R, H, 128], weights fp32 [R, H]) of the next step."""
        q = self.g.standard_normal((self.n_req, self.heads, INDEXER_DIM), dtype=np.float32)
        w = (self.g.standard_normal((self.n_req, self.heads), dtype=np.float32)
             / np.float32(math.sqrt(self.heads))).astype(np.float32)
        return f32_to_bf16_bits(q), w
