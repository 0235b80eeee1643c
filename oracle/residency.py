"""Reference of the residency manager around the decode step.
TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's CPU
baseline may use it; the product path never does.

What the pages describe ([P2] "vLLM GLM 5.3 优化：混合 HiSparse 卸载",
§"混合 HiSparse 的技术实现" and §"关键架构细节"; [P3] "vLLM Hybrid
HiSparse：稀疏MLA破解长上下文显存瓶颈", §"分级内存的运作机制"):
  * residency is tracked per page; while there is room the KV stays on the
    GPU, and only under memory pressure does a request release pages;
  * completed prefix pages are queued for copying to host memory while
    they are still served from the GPU, so that under pressure their GPU
    places can be freed at once, with no copy then;
  * under pressure a request releases its coldest pages to host memory and
    keeps serving the indexer's rows through its hot buffer.

Readings where the pages are silent (each listed in the design notes):
  * a page's stamp is the last step whose top-K selected one of its tokens,
    or the step at which the page entered the context; 0 = neither;
  * "coldest" = ascending (stamp, page);
  * only pages entirely inside the context with a valid host copy can be
    released; pressure = more GPU pages inside the context than the
    request's page budget;
  * the copy queue takes the lowest-numbered pending pages first, a bounded
    number per call, and a bounded number of pages is released per call.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import numpy as np


class PageState:
    """Per-request page recency and host-copy marks."""

    def __init__(self, pages: int):
        self.stamp = np.zeros(int(pages), dtype=np.int64)
        self.host_valid = np.zeros(int(pages), dtype=bool)

    def reset(self):
        self.stamp[:] = 0
        self.host_valid[:] = False

    def enter_context(self, old_len: int, new_len: int, step: int, page_size: int):
        """Pages that become part of the context take the current step."""
        a = -(-int(old_len) // page_size)
        b = -(-int(new_len) // page_size)
        if b > a:
            self.stamp[a:b] = step

    def touch(self, sel: np.ndarray, step: int, page_size: int):
        """The pages of the tokens the top-K selected at `step`."""
        t = sel[sel >= 0]
        self.stamp[t // page_size] = step

    def mark_given(self, first_page: int, gpu_ids: np.ndarray, host_copy_valid: bool):
        """Residency set from outside: host-only pages are in the host store;
        GPU pages are there only when the caller says so."""
        g = np.asarray(gpu_ids)
        self.host_valid[first_page:first_page + g.size] = (g < 0) | bool(host_copy_valid)


def update_residency(st: PageState, gpu_page: np.ndarray, context_len: int, page_size: int,
                     budget: Optional[int], max_copy: int, max_demote: int) -> Dict[str, List[int]]:
    """One call of the manager for one request (mutates `st` and `gpu_page`).

    Returns the pages copied to the host store (ascending), the pages
    released (ascending) and the pool pages they held (same order)."""
    ps = int(page_size)
    L = int(context_len)
    npg = -(-L // ps)
    full = L // ps
    # proactive copy: complete GPU pages without a host copy, lowest first
    pending = [p for p in range(full) if gpu_page[p] >= 0 and not st.host_valid[p]]
    copied = pending[:max_copy]
    st.host_valid[copied] = True
    # pressure: more GPU pages in the context than the budget
    demoted: List[int] = []
    if budget is not None:
        held = int(np.count_nonzero(gpu_page[:npg] >= 0))
        d = min(max(held - int(budget), 0), int(max_demote))
        cand = [p for p in range(full) if gpu_page[p] >= 0 and st.host_valid[p]]
        cand.sort(key=lambda p: (int(st.stamp[p]), p))
        demoted = sorted(cand[:d])
    freed = [int(gpu_page[p]) for p in demoted]
    gpu_page[demoted] = -1
    return {"copied": [int(p) for p in copied], "demoted": demoted, "freed": freed}
