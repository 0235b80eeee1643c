"""TieredPool: torch owns the device buffers, libhisparse does the work.

Marshalling only: this class allocates the caller-owned device buffers the
C ABI asks for (pool rows, fp8 scales, state workspace) with torch, exposes
the pinned host store as numpy arrays, and forwards each call to the
library on torch's current HIP stream.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional

import numpy as np
import torch

from . import binding as B

ROW_DIM, NOPE = 576, 512


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


class TieredPool:
    def __init__(self, *, page_size: int, num_pool_pages: int, max_requests: int, max_context: int,
                 kv_dtype: str, top_k: int, hot_rows: int = 0, max_batch: Optional[int] = None,
                 max_q_rows: int = 128, host_rows: int, select_q: int = 0, device: str = "cuda"):
        self.desc = B.HsPoolDesc(page_size=page_size, num_pool_pages=num_pool_pages,
                                 max_requests=max_requests, max_context=max_context, nope_dim=512,
                                 rope_dim=64, kv_dtype=B.DTYPE_CODES[kv_dtype], top_k=top_k,
                                 hot_rows=hot_rows, max_batch=max_batch or max_requests,
                                 max_q_rows=max_q_rows, select_q=select_q, host_rows=host_rows)
        self.kv_dtype = kv_dtype
        self.sizes = B.pool_requirements(self.desc)
        self.device = torch.device(device)
        self.row_bytes = int(self.sizes.row_bytes)
        self.n_pool_rows = num_pool_pages * page_size
        self.pool_rows = torch.empty(int(self.sizes.pool_bytes), dtype=torch.uint8, device=self.device)
        self.pool_scales = (torch.zeros(self.n_pool_rows, dtype=torch.float32, device=self.device)
                            if kv_dtype == "fp8" else None)
        self.state = torch.empty(int(self.sizes.state_bytes), dtype=torch.uint8, device=self.device)
        assert self.state.data_ptr() % 256 == 0
        self.handle = B.init_pool(self.desc, self.pool_rows.data_ptr(), _ptr(self.pool_scales),
                                  self.state.data_ptr(), int(self.sizes.state_bytes), _stream())
        # host store views: row r at byte r * host_row_stride; an fp8 row's
        # fp32 scale follows its 576 code bytes
        rows_p, scales_p = B.host_rows(self.handle)
        stride = int(self.sizes.host_row_stride)
        raw = (ctypes.c_uint8 * (host_rows * stride)).from_address(rows_p)
        self.host_store = np.ndarray((host_rows, self.row_bytes), dtype=np.uint8, buffer=raw,
                                     strides=(stride, 1))
        self.host_scales = (np.ndarray((host_rows,), dtype=np.float32, buffer=raw,
                                       offset=scales_p - rows_p, strides=(stride,))
                            if kv_dtype == "fp8" else None)
        self.layout = B.get_state_layout(self.handle)
        self.hot_rows = int(self.sizes.hot_rows)
        self.pages_per_request = int(self.sizes.pages_per_request)

    # ------------------------------------------------------------ views
    def pool_row_view(self) -> torch.Tensor:
        return self.pool_rows.view(self.n_pool_rows, self.row_bytes)

    def state_views(self) -> Dict[str, torch.Tensor]:
        d, L = self.desc, self.layout
        R, S = d.max_requests, self.hot_rows

        def v(off, dtype, *shape):
            n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
            return self.state[off:off + n].view(dtype).view(*shape)
        return {
            "ctx_len": v(L.ctx_len, torch.int32, R),
            "host_base": v(L.host_base, torch.int64, R),
            "page_table": v(L.page_table, torch.int32, R, self.pages_per_request),
            "hot_pages": v(L.hot_pages, torch.int32, R, S // d.page_size),
            "rev": v(L.rev, torch.int32, R, d.max_context),
            "slot_tag": v(L.slot_tag, torch.int32, R, S),
            "slot_stamp": v(L.slot_stamp, torch.int32, R, S),
            "lru_order": v(L.lru_order, torch.int32, R, S),
            "step": v(L.step, torch.int32, R),
            "counters": v(L.counters, torch.int64, R, 3),
            "error": v(L.error, torch.int32, 4),
            "page_stamp": v(L.page_stamp, torch.int32, R, self.pages_per_request),
            "host_valid": v(L.host_valid, torch.uint8, R, self.pages_per_request),
        }

    # ------------------------------------------------------------ calls
    def set_residency(self, req: int, context_len: int, host_row_base: int,
                      gpu_page_ids: Optional[torch.Tensor], first_page: int = 0,
                      hot_page_ids: Optional[torch.Tensor] = None, reset_hot: bool = False,
                      host_copy_valid: bool = False, reset_pages: bool = False):
        n = 0 if gpu_page_ids is None else int(gpu_page_ids.numel())
        flags = ((B.HS_RESET_HOT if reset_hot else 0) | (B.HS_HOST_COPY_VALID if host_copy_valid else 0) |
                 (B.HS_RESET_PAGES if reset_pages else 0))
        B.set_residency(self.handle, req, context_len, host_row_base, first_page, n,
                        _ptr(gpu_page_ids), _ptr(hot_page_ids), flags, _stream())

    def update_residency(self, req_ids: torch.Tensor, budget_pages: Optional[torch.Tensor],
                         max_copy_pages: int, max_demote_pages: int,
                         freed_out: Optional[torch.Tensor] = None,
                         counts_out: Optional[torch.Tensor] = None):
        B.update_residency(self.handle, req_ids.data_ptr(), int(req_ids.numel()), _ptr(budget_pages),
                           max_copy_pages, max_demote_pages, _ptr(freed_out), _ptr(counts_out), _stream())

    def select_topk(self, scores: torch.Tensor, req_ids: torch.Tensor, idx_out: torch.Tensor):
        B.select_topk(self.handle, scores.data_ptr(), scores.stride(0), req_ids.data_ptr(),
                      int(req_ids.numel()), idx_out.data_ptr(), _stream())

    def select_topk_union(self, scores: torch.Tensor, req_ids: torch.Tensor, idx_out: torch.Tensor,
                          union_out: torch.Tensor, upos_out: torch.Tensor):
        """scores fp32 [n, Q, stride]; idx_out and upos_out int32 [n, Q, k]; union_out int32 [n, top_k]."""
        n, Q, k = idx_out.shape
        B.select_topk_union(self.handle, scores.data_ptr(), scores.stride(1), req_ids.data_ptr(), n, Q, k,
                            idx_out.data_ptr(), union_out.data_ptr(), upos_out.data_ptr(), _stream())

    def sparse_mla_decode_union(self, q: torch.Tensor, plan: torch.Tensor, upos: torch.Tensor, sm_scale: float,
                                out: torch.Tensor, lse: Optional[torch.Tensor] = None):
        """q [n, Q, H, 576]; plan [n, top_k] (of the union); upos [n, Q, k]."""
        n_req, q_per_req, n_heads, _ = q.shape
        qd = B.HS_F32 if q.dtype == torch.float32 else B.HS_BF16
        B.sparse_mla_decode_union(self.handle, q.data_ptr(), qd, n_req, q_per_req, n_heads, plan.data_ptr(),
                                  upos.data_ptr(), int(upos.shape[-1]), sm_scale, out.data_ptr(), _ptr(lse), _stream())

    def indexer_scores(self, iq: torch.Tensor, iw: torch.Tensor, ik: torch.Tensor, req_ids: torch.Tensor,
                       scores: torch.Tensor):
        """iq bf16 [n, H, 128], iw fp32 [n, H], ik bf16 [max_requests, stride, 128] (request slot r's
        indexer keys in ik[r]), scores fp32 [n, stride'] (row i gets tokens 0..L_r-1)."""
        n, H, _ = iq.shape
        B.indexer_scores(self.handle, iq.data_ptr(), iw.data_ptr(), ik.data_ptr(), ik.stride(0) // ik.stride(1),
                         H, req_ids.data_ptr(), n, scores.data_ptr(), scores.stride(0), _stream())

    def resolve_rows(self, idx: torch.Tensor, req_ids: torch.Tensor, plan_out: torch.Tensor,
                     counts_out: Optional[torch.Tensor] = None):
        B.resolve_rows(self.handle, idx.data_ptr(), req_ids.data_ptr(), int(req_ids.numel()),
                       plan_out.data_ptr(), _ptr(counts_out), _stream())

    def select_resolve(self, scores: torch.Tensor, req_ids: torch.Tensor, idx_out: torch.Tensor,
                       plan_out: torch.Tensor, counts_out: Optional[torch.Tensor] = None):
        """select_topk then resolve_rows, fused (same results)."""
        B.select_resolve(self.handle, scores.data_ptr(), scores.stride(0), req_ids.data_ptr(), int(req_ids.numel()),
                         idx_out.data_ptr(), plan_out.data_ptr(), _ptr(counts_out), _stream())

    def sparse_mla_decode(self, q: torch.Tensor, plan: torch.Tensor, sm_scale: float,
                          out: torch.Tensor, lse: Optional[torch.Tensor] = None):
        n_req, q_per_req, n_heads, _ = q.shape
        qd = B.HS_F32 if q.dtype == torch.float32 else B.HS_BF16
        B.sparse_mla_decode(self.handle, q.data_ptr(), qd, n_req, q_per_req, n_heads, plan.data_ptr(),
                            sm_scale, out.data_ptr(), _ptr(lse), _stream())

    def sparse_mla_decode_noalloc(self, q: torch.Tensor, plan: torch.Tensor, sm_scale: float,
                                  out: torch.Tensor, lse: Optional[torch.Tensor] = None):
        """sparse_mla_decode with its split partials in the library's fixed
        per-GPU array instead of the pool workspace (allocates nothing)."""
        n_req, q_per_req, n_heads, _ = q.shape
        qd = B.HS_F32 if q.dtype == torch.float32 else B.HS_BF16
        B.sparse_mla_decode_noalloc(self.handle, q.data_ptr(), qd, n_req, q_per_req, n_heads, plan.data_ptr(),
                                    sm_scale, out.data_ptr(), _ptr(lse), _stream())

    def device_error(self):
        return B.get_device_error(self.handle, _stream())

    def clear_device_error(self):
        B.clear_device_error(self.handle, _stream())

    def close(self):
        if self.handle:
            B.destroy_pool(self.handle)
            self.handle = 0
            self.host_store = self.host_scales = None
