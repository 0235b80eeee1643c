"""GPU parity of the whole step on shapes at the edges of what a pool
accepts (through the C ABI), each stepped in lockstep with the oracle as the
reduced workloads are (gpu_helpers.Runner: top-K, plan, counts, LRU state,
pool bytes behind the plan, attention on every head):

  page-1      one token per page (the page table as long as the context, one
              pool page per hot slot), bf16 rows
  page-1024   the largest page, a hot buffer of exactly K rows, fp8 rows,
              three requests with every residency kind
  f32-k1000   fp32 rows and queries with a top-K that is not a multiple of
              the 32-row tile, through the split fp32 attention
  page-4-q4   fp8 rows, 4 query tokens sharing one plan, K = 33 over a hot
              buffer of 36 rows, growing contexts under a GPU token budget
  k1-s2       the smallest top-K and hot buffer (K = 1, S = 2, pages of 2)
Each runs as the two calls and as select_resolve.
"""
import pytest

from gpu_helpers import Runner, log, small
from sparse_mla_decode_indexer_amd import workload as W

pytestmark = pytest.mark.gpu

CONFIGS = {
    "page-1": lambda: small("single-128k", ctx=3000, host_pages=2000, page_size=1, top_k=64, hot_rows=128,
                            scores=("ar1_shift", 0.9, 0.5)),
    "page-1024": lambda: small("batch32", n_req=3, ctx_range=(3000, 9000), page_size=1024, top_k=2048,
                               hot_rows=2048, kv_dtype="fp8", scores=("ar1_shift", 0.9, 0.5)),
    "f32-k1000": lambda: small("tiny", ctx=20000, host_pages=200, top_k=1000, hot_rows=1024,
                               scores=("ar1_shift", 0.9, 0.5)),
    "page-4-q4": lambda: small("agent16", n_req=2, growth=(300, 50, 20, 2), gpu_token_budget=64, page_size=4,
                               top_k=33, hot_rows=36, steps=10),
    "k1-s2": lambda: small("single-128k", ctx=500, host_pages=100, page_size=2, top_k=1, hot_rows=2),
}
STEPS = 5


@pytest.mark.parametrize("fused", [False, True], ids=["two-calls", "select_resolve"])
@pytest.mark.parametrize("name", list(CONFIGS))
def test_step_at_shape_edges(name, fused):
    spec = CONFIGS[name]()
    log(f"[gpu] config {name}: page {spec.page_size}, K {spec.top_k}, S {spec.hot_rows}, {spec.kv_dtype}, "
        f"fused={fused}")
    rn = Runner(W.generate(spec), fused=fused)
    rn.incremental = spec.growth is not None
    try:
        for _ in range(STEPS):
            rn.step()
        log(f"[gpu] config {name}: max attention rel err {rn.max_err:.2e}")
    finally:
        rn.close()
