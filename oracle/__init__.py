"""CPU oracle for the tiered sparse-MLA decode step — TEST INFRASTRUCTURE.

This package is the plain, slow, obviously-correct reference that the HIP
path is checked against. It is test infrastructure only: it may be
imported by ``tests/``, by ``__graft_entry__.smoke()`` and by the
``cpu_baseline`` leg of ``bench.py``, and by nothing else. The product path
never routes through it. It shares no code with the HIP path (no kernels,
headers, helpers, tables or constants): it takes plain numpy arrays and
returns plain numpy arrays.

Pages it follows (cited by title and section):
  [P2] "vLLM GLM 5.3 优化：混合 HiSparse 卸载" (agentlenshq.com)
  [P3] "vLLM Hybrid HiSparse：稀疏MLA破解长上下文显存瓶颈" (kongchang.com)

Every function is pinned by a ``-m "not gpu"`` test against something other
than itself (brute force, closed forms, library routines, a hand-computed
LRU trace, invariants). Conventions the pages leave open — the softmax scale
value, the choice of the first 512 dims as V, the LRU tie rules and the
page-coldness order of the residency manager — are
fixed here and shared with the HIP path; the pages cannot confirm them
("parity unpinned" by the pages; pinned only as conventions).
"""
from .hisparse_oracle import (  # noqa: F401
    HOT, MISS, RESIDENT,
    HotBufferOracle,
    DecodeOracle,
    bf16_decode,
    decode_rows,
    e4m3fn_decode,
    mla_attention,
    resolve_step,
    select_topk,
    union_of_selections,
)
from .indexer import indexer_scores  # noqa: F401
from .residency import PageState, update_residency  # noqa: F401
