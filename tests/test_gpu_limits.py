"""GPU parity at the library's size limits (through the C ABI).

One request whose context is the longest a pool accepts (4,194,304 tokens:
2,048 filter chunks of 2,048 scores), the largest top-K (4,096) and the
largest hot buffer (8,192 rows), fp8 rows with 90% of the pages on the host
(so the bookkeeper looks the page table up in global memory), and a topic
shift on about every other step so that the hot buffer fills and evicts.
Every step is compared with the oracle as in the reduced workloads: top-K,
plan, counts, the whole LRU state, the bytes behind every plan entry, and
attention on every head. Both step forms run: the two calls (select_topk,
resolve_rows) and select_resolve.
"""
import dataclasses

import pytest

from gpu_helpers import Runner, log
from sparse_mla_decode_indexer_amd import workload as W

pytestmark = pytest.mark.gpu

MAX_CONTEXT = 2048 * 2048
MAX_TOP_K = 4096
MAX_HOT_ROWS = 8192
STEPS = 5


@pytest.fixture(scope="module")
def limits_workload():
    spec = dataclasses.replace(W.SPECS["single-1m-fp8"], name="limits", ctx=MAX_CONTEXT,
                               host_pages=MAX_CONTEXT // 64 * 9 // 10, top_k=MAX_TOP_K,
                               hot_rows=MAX_HOT_ROWS, steps=STEPS, scores=("ar1_shift", 0.95, 0.5))
    log(f"[gpu] limits: generating {MAX_CONTEXT} fp8 rows")
    return W.generate(spec)


@pytest.mark.parametrize("fused", [False, True], ids=["two-calls", "select_resolve"])
def test_maximum_context_top_k_and_hot_buffer(limits_workload, fused):
    wl = limits_workload
    rn = Runner(wl, fused=fused)
    try:
        total_miss = 0
        for n in range(STEPS):
            log(f"[gpu] limits fused={fused}: step {n + 1}")
            ref = rn.step()
            total_miss += int(ref["counts"][0][2])
        # the misses of the first steps outgrow the hot buffer, so later
        # steps evict slots that earlier steps filled
        assert total_miss > MAX_HOT_ROWS
        log(f"[gpu] limits fused={fused}: {total_miss} misses, max attention rel err {rn.max_err:.2e}")
    finally:
        rn.close()
