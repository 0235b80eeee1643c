"""Load a synthetic workload into a TieredPool and drive decode steps.

Data movement only (host store fill, resident-page upload, residency
calls, per-step buffers); the decode step itself is the three library
calls select_topk -> resolve_rows -> sparse_mla_decode.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np
import torch

from . import workload as W
from .pool import TieredPool


def make_pool(wl: W.Workload, device: str = "cuda", spare_pages: int = 0) -> TieredPool:
    s = wl.spec
    return TieredPool(page_size=s.page_size, num_pool_pages=wl.num_pool_pages + spare_pages,
                      max_requests=s.n_req, max_context=wl.max_context, kv_dtype=s.kv_dtype,
                      top_k=s.top_k, hot_rows=s.hot_rows, max_batch=s.n_req,
                      max_q_rows=s.q_per_req * s.heads, host_rows=int(wl.rows.shape[0]),
                      select_q=s.q_per_req if s.select_k else 0, device=device)


def store_bytes(wl: W.Workload) -> np.ndarray:
    """The logical store as raw row bytes [N, row_bytes]."""
    return np.ascontiguousarray(wl.rows).view(np.uint8).reshape(wl.rows.shape[0], -1)


def load_workload(pool: TieredPool, wl: W.Workload, poison_hot: bool = True,
                  chunk_rows: int = 1 << 18):
    """Fill the host store with every row, upload resident pages into their
    pool pages, and set each request's residency (hot buffer empty)."""
    s = wl.spec
    ps = s.page_size
    raw = store_bytes(wl)
    pool.host_store[:] = raw
    if pool.host_scales is not None:
        pool.host_scales[:] = wl.scales
    dev = pool.device
    prv = pool.pool_row_view()
    if poison_hot:  # hot slots hold garbage until a miss fills them
        prv.fill_(0xFF)  # bf16/f32 NaN patterns; fp8 0xFF is NaN too
        if pool.pool_scales is not None:
            pool.pool_scales.fill_(float("nan"))
    # resident rows: pool row (page * ps + o) <- store row (base + p * ps + o)
    src, dst = [], []
    for r in range(s.n_req):
        g = wl.gpu_page[r]
        pages = np.flatnonzero(g >= 0)
        if pages.size == 0:
            continue
        o = np.arange(ps)
        tok = (pages[:, None] * ps + o[None, :]).ravel()
        prow = (g[pages][:, None].astype(np.int64) * ps + o[None, :]).ravel()
        keep = tok < wl.ctx_final[r]
        src.append(wl.host_base[r] + tok[keep])
        dst.append(prow[keep])
    if src:
        src = np.concatenate(src)
        dst = np.concatenate(dst)
        for a in range(0, src.size, chunk_rows):
            sl = slice(a, a + chunk_rows)
            rows = torch.from_numpy(raw[src[sl]]).to(dev, non_blocking=False)
            prv.index_copy_(0, torch.from_numpy(dst[sl]).to(dev), rows)
            if pool.pool_scales is not None:
                sc = torch.from_numpy(wl.scales[src[sl]]).to(dev)
                pool.pool_scales.index_copy_(0, torch.from_numpy(dst[sl]).to(dev), sc)
    for r in range(s.n_req):
        set_request(pool, wl, r, int(wl.ctx0[r]), reset_hot=True, with_hot_pages=True)
    torch.cuda.synchronize()


def set_request(pool: TieredPool, wl: W.Workload, r: int, ctx: int, reset_hot: bool = False,
                with_hot_pages: bool = False, gpu_page: Optional[np.ndarray] = None,
                first_page: int = 0, num_pages: Optional[int] = None):
    """Context length of request r, and the residency of pages
    [first_page, first_page + num_pages) (default: every page of the
    workload's table) from `gpu_page` (default: the workload's)."""
    dev = pool.device
    g = wl.gpu_page[r] if gpu_page is None else gpu_page
    n = g.size - first_page if num_pages is None else num_pages
    gp = torch.from_numpy(g[first_page:first_page + n].astype(np.int32)).to(dev) if n > 0 else None
    hp = torch.from_numpy(wl.hot_pages[r].astype(np.int32)).to(dev) if with_hot_pages else None
    pool.set_residency(r, ctx, int(wl.host_base[r]), gp, first_page, hp, reset_hot)


class StepBuffers:
    """Device buffers of one decode step for R requests."""

    def __init__(self, wl: W.Workload, device: str = "cuda", n_steps: int = 1):
        s = wl.spec
        R, K = s.n_req, s.top_k
        dev = torch.device(device)
        qdt = torch.float32 if s.q_dtype == "f32" else torch.bfloat16
        self.req_ids = torch.arange(R, dtype=torch.int32, device=dev)
        stride = -(-wl.max_context // 64) * 64  # 16-byte aligned rows
        # speculative steps with a selection per query token: per-token
        # scores, selections and union positions, and the union
        self.union = s.select_k is not None
        if self.union:
            Q, k = s.q_per_req, s.select_k
            self.scores = torch.zeros(n_steps, R, Q, stride, dtype=torch.float32, device=dev)
            self.sel = torch.full((R, Q, k), -1, dtype=torch.int32, device=dev)
            self.upos = torch.full((R, Q, k), -1, dtype=torch.int32, device=dev)
        else:
            self.scores = torch.zeros(n_steps, R, stride, dtype=torch.float32, device=dev)
        self.q = torch.zeros(n_steps, R, s.q_per_req, s.heads, W.ROW_DIM, dtype=qdt, device=dev)
        self.idx = torch.full((R, K), -1, dtype=torch.int32, device=dev)
        self.plan = torch.full((R, K), -1, dtype=torch.int32, device=dev)
        self.counts = torch.zeros(R, 3, dtype=torch.int32, device=dev)
        self.out = torch.zeros(R, s.q_per_req, s.heads, W.NOPE_DIM, dtype=torch.float32, device=dev)
        self.lse = torch.zeros(R, s.q_per_req, s.heads, dtype=torch.float32, device=dev)
        self.sm_scale = float(wl.sm_scale)

    def upload(self, n: int, scores: np.ndarray, q: np.ndarray):
        self.scores[n, ..., :scores.shape[-1]].copy_(torch.from_numpy(scores))
        if q.dtype == np.uint16:
            self.q[n].copy_(torch.from_numpy(q.view(np.int16)).view(torch.bfloat16))
        else:
            self.q[n].copy_(torch.from_numpy(q))


def decode_step(pool: TieredPool, buf: StepBuffers, n: int = 0, fused: bool = False):
    """One step: top-K -> resolve -> sparse MLA attention (stream-ordered);
    with `fused`, top-K and resolve run as hs_select_resolve (same results).
    A speculative step with a selection per query token selects per token,
    resolves the union (buf.idx) once and attends per token through it."""
    if buf.union:
        pool.select_topk_union(buf.scores[n], buf.req_ids, buf.sel, buf.idx, buf.upos)
        pool.resolve_rows(buf.idx, buf.req_ids, buf.plan, buf.counts)
        pool.sparse_mla_decode_union(buf.q[n], buf.plan, buf.upos, buf.sm_scale, buf.out, buf.lse)
        return
    if fused:
        pool.select_resolve(buf.scores[n], buf.req_ids, buf.idx, buf.plan, buf.counts)
    else:
        pool.select_topk(buf.scores[n], buf.req_ids, buf.idx)
        pool.resolve_rows(buf.idx, buf.req_ids, buf.plan, buf.counts)
    pool.sparse_mla_decode(buf.q[n], buf.plan, buf.sm_scale, buf.out, buf.lse)


def request_groups(n_req: int, group: int) -> List[slice]:
    """Consecutive batch positions in groups of `group` (the last one shorter)."""
    return [slice(a, min(a + group, n_req)) for a in range(0, n_req, group)]


class PipelinedStep:
    """One decode step of a batch as a pipeline over groups of requests.

    The three entry points run per group on three streams: top-K of group
    g, then its resolve (which waits for that top-K), then its attention
    (which waits for that resolve). Each entry point keeps its own stream,
    so its calls stay in order (their scratch memory is indexed by batch
    position), while the attention of group g overlaps the resolve (the
    PCIe transfer of the missed rows) of group g + 1 and the top-K of later
    groups. The step computes what decode_step computes; the calls fork from
    and join back into the caller's current stream, so the whole step can be
    captured in one hipGraph. Streams keep the default priority."""

    def __init__(self, pool: TieredPool, buf: StepBuffers, group: int):
        self.pool, self.buf = pool, buf
        self.groups = request_groups(int(buf.req_ids.numel()), group)
        self.streams = [torch.cuda.Stream(device=buf.req_ids.device) for _ in range(3)]

    def __call__(self, n: int = 0):
        pool, buf = self.pool, self.buf
        s_tk, s_rs, s_at = self.streams
        cur = torch.cuda.current_stream()
        for st in self.streams:
            st.wait_stream(cur)
        for g in self.groups:
            with torch.cuda.stream(s_tk):
                pool.select_topk(buf.scores[n][g], buf.req_ids[g], buf.idx[g])
            s_rs.wait_stream(s_tk)
            with torch.cuda.stream(s_rs):
                pool.resolve_rows(buf.idx[g], buf.req_ids[g], buf.plan[g], buf.counts[g])
            s_at.wait_stream(s_rs)
            with torch.cuda.stream(s_at):
                pool.sparse_mla_decode(buf.q[n][g], buf.plan[g], buf.sm_scale, buf.out[g], buf.lse[g])
        for st in self.streams:
            cur.wait_stream(st)
