"""ctypes binding of libhisparse.so (argument marshalling only).

The functions below carry the C ABI's names without the ``hs_`` prefix and
take the same arguments: plain integers for device pointers and streams.
Every step of the decode path runs in the library's HIP kernels; nothing
here computes. A missing library raises at load time — there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhisparse.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "hisparse.h")

HS_F32, HS_BF16, HS_FP8_E4M3 = 0, 1, 2
HS_RESET_HOT = 1
HS_HOST_COPY_VALID = 2
HS_RESET_PAGES = 4
DTYPE_CODES = {"f32": HS_F32, "bf16": HS_BF16, "fp8": HS_FP8_E4M3}
STATUS = {0: "HS_OK", 1: "HS_ERR_INVALID_ARGUMENT", 2: "HS_ERR_CAPACITY", 3: "HS_ERR_UNSUPPORTED",
          4: "HS_ERR_HIP", 5: "HS_ERR_OUT_OF_MEMORY", 6: "HS_ERR_DEVICE"}
DEVICE_ERRORS = {0: "ok", 1: "index past context", 2: "page id outside pool",
                 3: "plan row outside pool", 4: "request id out of range", 5: "bounded wait timed out"}


class HsPoolDesc(ctypes.Structure):
    _fields_ = [("page_size", ctypes.c_int32), ("num_pool_pages", ctypes.c_int32),
                ("max_requests", ctypes.c_int32), ("max_context", ctypes.c_int32),
                ("nope_dim", ctypes.c_int32), ("rope_dim", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("hot_rows", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("max_q_rows", ctypes.c_int32), ("select_q", ctypes.c_int32),
                ("host_rows", ctypes.c_int64)]


class HsPoolSizes(ctypes.Structure):
    _fields_ = [("row_bytes", ctypes.c_size_t), ("pool_bytes", ctypes.c_size_t),
                ("pool_scale_bytes", ctypes.c_size_t), ("state_bytes", ctypes.c_size_t),
                ("host_store_bytes", ctypes.c_size_t), ("hot_rows", ctypes.c_int32),
                ("pages_per_request", ctypes.c_int32), ("host_row_stride", ctypes.c_size_t)]


class HsStateLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "ctx_len", "host_base", "page_table", "hot_pages", "rev", "slot_tag", "slot_stamp",
        "lru_order", "step", "counters", "error", "page_stamp", "host_valid", "scratch", "total")]


class HiSparseError(RuntimeError):
    def __init__(self, status: int, call: str, detail: str = ""):
        self.status = status
        super().__init__(f"{call}: {STATUS.get(status, status)} {detail}".strip())


_VP, _I32, _I64, _U32, _F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float
_SIGS = {
    "hs_pool_requirements": [ctypes.POINTER(HsPoolDesc), ctypes.POINTER(HsPoolSizes)],
    "hs_init_pool": [ctypes.POINTER(HsPoolDesc), _VP, _VP, _VP, ctypes.c_size_t, _VP, ctypes.POINTER(_VP)],
    "hs_host_rows": [_VP, ctypes.POINTER(_VP), ctypes.POINTER(_VP)],
    "hs_set_residency": [_VP, _I32, _I32, _I64, _I32, _I32, _VP, _VP, _U32, _VP],
    "hs_select_topk": [_VP, _VP, _I64, _VP, _I32, _VP, _VP],
    "hs_select_topk_union": [_VP, _VP, _I64, _VP, _I32, _I32, _I32, _VP, _VP, _VP, _VP],
    "hs_sparse_mla_decode_union": [_VP, _VP, _I32, _I32, _I32, _I32, _VP, _VP, _I32, _F32, _VP, _VP, _VP],
    "hs_indexer_scores": [_VP, _VP, _VP, _VP, _I64, _I32, _VP, _I32, _VP, _I64, _VP],
    "hs_resolve_rows": [_VP, _VP, _VP, _I32, _VP, _VP, _VP],
    "hs_select_resolve": [_VP, _VP, _I64, _VP, _I32, _VP, _VP, _VP, _VP],
    "hs_update_residency": [_VP, _VP, _I32, _VP, _I32, _I32, _VP, _VP, _VP],
    "hs_sparse_mla_decode": [_VP, _VP, _I32, _I32, _I32, _I32, _VP, _F32, _VP, _VP, _VP],
    "hs_sparse_mla_decode_noalloc": [_VP, _VP, _I32, _I32, _I32, _I32, _VP, _F32, _VP, _VP, _VP],
    "hs_get_state_layout": [_VP, ctypes.POINTER(HsStateLayout)],
    "hs_get_device_error": [_VP, ctypes.POINTER(_U32 * 4), _VP],
    "hs_clear_device_error": [_VP, _VP],
    "hs_last_hip_error": [],
    "hs_status_string": [_I32],
    "hs_destroy_pool": [_VP],
}

_lib: Optional[ctypes.CDLL] = None


def header_functions():
    """Names of the functions include/hisparse.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:hs_status|int32_t|const char\*)\s+(hs_\w+)\(", text, re.M)))


def lib() -> ctypes.CDLL:
    """Load libhisparse.so once; raise if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_mla_decode_indexer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_char_p if name == "hs_status_string" else ctypes.c_int32
        _lib = L
    return _lib


def _check(st: int, call: str):
    if st != 0:
        detail = ""
        if st == 4:
            detail = f"(hipError {lib().hs_last_hip_error()})"
        raise HiSparseError(st, call, detail)


def status_string(st: int) -> str:
    return lib().hs_status_string(st).decode()


def pool_requirements(desc: HsPoolDesc) -> HsPoolSizes:
    out = HsPoolSizes()
    _check(lib().hs_pool_requirements(ctypes.byref(desc), ctypes.byref(out)), "hs_pool_requirements")
    return out


def init_pool(desc: HsPoolDesc, pool_rows: int, pool_scales: int, state: int, state_bytes: int,
              stream: int) -> int:
    h = _VP()
    _check(lib().hs_init_pool(ctypes.byref(desc), pool_rows, pool_scales or None, state, state_bytes,
                              stream or None, ctypes.byref(h)), "hs_init_pool")
    return h.value


def host_rows(pool: int) -> Tuple[int, int]:
    r, s = _VP(), _VP()
    _check(lib().hs_host_rows(pool, ctypes.byref(r), ctypes.byref(s)), "hs_host_rows")
    return r.value, (s.value or 0)


def set_residency(pool: int, req: int, context_len: int, host_row_base: int, first_page: int,
                  num_pages: int, gpu_page_ids: int, hot_page_ids: int, flags: int, stream: int):
    _check(lib().hs_set_residency(pool, req, context_len, host_row_base, first_page, num_pages,
                                  gpu_page_ids or None, hot_page_ids or None, flags, stream or None),
           "hs_set_residency")


def select_topk(pool: int, scores: int, score_stride: int, req_ids: int, n_req: int, idx_out: int,
                stream: int):
    _check(lib().hs_select_topk(pool, scores, score_stride, req_ids, n_req, idx_out, stream or None),
           "hs_select_topk")


def select_topk_union(pool: int, scores: int, score_stride: int, req_ids: int, n_req: int, q_per_req: int,
                      k_per_token: int, idx_out: int, union_out: int, upos_out: int, stream: int):
    _check(lib().hs_select_topk_union(pool, scores, score_stride, req_ids, n_req, q_per_req, k_per_token, idx_out,
                                      union_out, upos_out, stream or None), "hs_select_topk_union")


def sparse_mla_decode_union(pool: int, q: int, q_dtype: int, n_req: int, q_per_req: int, n_heads: int, plan: int,
                            upos: int, k_per_token: int, sm_scale: float, out: int, lse_out: int, stream: int):
    _check(lib().hs_sparse_mla_decode_union(pool, q, q_dtype, n_req, q_per_req, n_heads, plan, upos, k_per_token,
                                            float(sm_scale), out, lse_out or None, stream or None),
           "hs_sparse_mla_decode_union")


def indexer_scores(pool: int, iq: int, iw: int, ik: int, ik_stride: int, n_heads: int, req_ids: int,
                   n_req: int, scores: int, score_stride: int, stream: int):
    _check(lib().hs_indexer_scores(pool, iq, iw, ik, ik_stride, n_heads, req_ids, n_req, scores, score_stride,
                                   stream or None), "hs_indexer_scores")


def resolve_rows(pool: int, idx: int, req_ids: int, n_req: int, plan_out: int, counts_out: int,
                 stream: int):
    _check(lib().hs_resolve_rows(pool, idx, req_ids, n_req, plan_out, counts_out or None, stream or None),
           "hs_resolve_rows")


def select_resolve(pool: int, scores: int, score_stride: int, req_ids: int, n_req: int, idx_out: int,
                   plan_out: int, counts_out: int, stream: int):
    _check(lib().hs_select_resolve(pool, scores, score_stride, req_ids, n_req, idx_out, plan_out,
                                   counts_out or None, stream or None), "hs_select_resolve")


def update_residency(pool: int, req_ids: int, n_req: int, budget_pages: int, max_copy_pages: int,
                     max_demote_pages: int, freed_out: int, counts_out: int, stream: int):
    _check(lib().hs_update_residency(pool, req_ids, n_req, budget_pages or None, max_copy_pages,
                                     max_demote_pages, freed_out or None, counts_out or None,
                                     stream or None), "hs_update_residency")


def sparse_mla_decode(pool: int, q: int, q_dtype: int, n_req: int, q_per_req: int, n_heads: int,
                      plan: int, sm_scale: float, out: int, lse_out: int, stream: int):
    _check(lib().hs_sparse_mla_decode(pool, q, q_dtype, n_req, q_per_req, n_heads, plan,
                                      float(sm_scale), out, lse_out or None, stream or None),
           "hs_sparse_mla_decode")


def sparse_mla_decode_noalloc(pool: int, q: int, q_dtype: int, n_req: int, q_per_req: int, n_heads: int,
                              plan: int, sm_scale: float, out: int, lse_out: int, stream: int):
    _check(lib().hs_sparse_mla_decode_noalloc(pool, q, q_dtype, n_req, q_per_req, n_heads, plan,
                                              float(sm_scale), out, lse_out or None, stream or None),
           "hs_sparse_mla_decode_noalloc")


def get_state_layout(pool: int) -> HsStateLayout:
    out = HsStateLayout()
    _check(lib().hs_get_state_layout(pool, ctypes.byref(out)), "hs_get_state_layout")
    return out


def get_device_error(pool: int, stream: int) -> Tuple[int, int, int]:
    code = (_U32 * 4)()
    st = lib().hs_get_device_error(pool, ctypes.byref(code), stream or None)
    if st not in (0, 6):
        _check(st, "hs_get_device_error")
    return int(code[0]), int(code[1]), int(code[2])


def clear_device_error(pool: int, stream: int):
    _check(lib().hs_clear_device_error(pool, stream or None), "hs_clear_device_error")


def destroy_pool(pool: int):
    _check(lib().hs_destroy_pool(pool), "hs_destroy_pool")
