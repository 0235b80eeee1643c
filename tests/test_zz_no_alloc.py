"""hs_sparse_mla_decode_noalloc (split partials in the library's fixed
per-GPU array, no allocation) against hs_sparse_mla_decode on the same
plans, through the C ABI: two calls in a row, the second with a smaller
batch, for bf16 and fp8 pools, both compared to the existing entry point
and to the fp64 oracle within the attention bar (max over query rows of
max_d |o - ref| / max_d |ref| <= 2e-3, lse within 1e-4 relative); and a
batch too large for the array is rejected with HS_ERR_CAPACITY before
anything is enqueued."""
import numpy as np
import pytest
import torch

from gpu_helpers import ATTN_TOL, LSE_TOL, Runner, attn_rel_err, log, q_f64, small
from oracle import mla_attention
from sparse_mla_decode_indexer_amd import binding as B
from sparse_mla_decode_indexer_amd import harness as Hn
from sparse_mla_decode_indexer_amd import workload as W

pytestmark = pytest.mark.gpu


def _compare(rn, q_np, plans_idx, n, out_a, lse_a, out_b, lse_b, tag):
    qd = q_f64(q_np)
    o_a, o_b = out_a[:n].cpu().numpy(), out_b[:n].cpu().numpy()
    l_a, l_b = lse_a[:n].cpu().numpy(), lse_b[:n].cpu().numpy()
    for r in range(n):
        e = attn_rel_err(o_b[r].reshape(-1, 512), o_a[r].reshape(-1, 512))
        assert e <= ATTN_TOL, f"{tag} req {r}: no-alloc vs pool-workspace attention {e:.3e}"
        assert np.allclose(l_b[r], l_a[r], rtol=LSE_TOL, atol=0), f"{tag} req {r}: lse"
        toks = plans_idx[r][plans_idx[r] >= 0]
        rows = rn.oracle.logical_rows(r, toks)
        heads = [0, 63, 127]
        o_ref, l_ref = mla_attention(qd[r][:, heads].reshape(-1, 576), rows, float(rn.wl.sm_scale))
        e2 = attn_rel_err(o_b[r][:, heads].reshape(-1, 512), o_ref)
        assert e2 <= ATTN_TOL, f"{tag} req {r}: no-alloc vs oracle {e2:.3e}"


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_noalloc_matches_pool_workspace_entry_point(kv):
    base = "batch32" if kv == "bf16" else "agent16-b"
    spec = small(base, n_req=3, ctx_range=None, ctx=20000, residency="mod3", growth=None,
                 gpu_token_budget=None, steps=2, q_per_req=1)
    log(f"[gpu] no-alloc attention {kv}: 3 requests then 1")
    wl = W.generate(spec)
    rn = Runner(wl)
    try:
        ref = rn.step()  # a plan for every request (pool workspace entry point inside)
        idx = [np.asarray(x) for x in ref["idx"]]
        buf = rn.buf
        q = buf.q[0]
        # the queries of the step just run, as host bits for the oracle
        q_np = q.view(torch.int16).cpu().numpy().view(np.uint16)
        for n in (3, 1):  # two calls in a row, the second with a smaller batch
            out_a = torch.full_like(buf.out, float("nan"))
            lse_a = torch.full_like(buf.lse, float("nan"))
            out_b = torch.full_like(buf.out, float("nan"))
            lse_b = torch.full_like(buf.lse, float("nan"))
            rn.pool.sparse_mla_decode(q[:n], buf.plan[:n], buf.sm_scale, out_a, lse_a)
            rn.pool.sparse_mla_decode_noalloc(q[:n], buf.plan[:n], buf.sm_scale, out_b, lse_b)
            torch.cuda.synchronize()
            _compare(rn, q_np, idx, n, out_a, lse_a, out_b, lse_b, f"{kv} n={n}")
            assert torch.isnan(out_b[n:]).all(), "rows past the batch were written"
        assert rn.pool.device_error()[0] == 0
    finally:
        rn.close()


def test_noalloc_rejects_a_batch_too_large_for_its_array():
    # top_k 4096 needs two 2,048-row splits: 64 requests x 128 query rows x 2
    # = 16,384 partial rows > 8,176
    from sparse_mla_decode_indexer_amd.pool import TieredPool
    log("[gpu] no-alloc attention capacity check")
    pool = TieredPool(page_size=64, num_pool_pages=4096, max_requests=64, max_context=8192, kv_dtype="bf16",
                      top_k=4096, hot_rows=4096, max_batch=64, max_q_rows=128, host_rows=8192)
    try:
        q = torch.zeros(64, 1, 128, 576, dtype=torch.bfloat16, device="cuda")
        plan = torch.full((64, 4096), -1, dtype=torch.int32, device="cuda")
        out = torch.full((64, 1, 128, 512), 7.0, device="cuda")
        with pytest.raises(B.HiSparseError) as e:
            pool.sparse_mla_decode_noalloc(q, plan, 0.04, out)
        assert e.value.status == 2
        torch.cuda.synchronize()
        assert (out == 7.0).all()  # nothing enqueued
        # 31 requests fit (31 x 128 x 2 = 7,936 rows): all plan rows absent -> zeros, lse -inf
        lse = torch.zeros(31, 1, 128, device="cuda")
        pool.sparse_mla_decode_noalloc(q[:31], plan[:31], 0.04, out[:31], lse)
        torch.cuda.synchronize()
        assert (out[:31] == 0).all() and torch.isneginf(lse).all()
        assert (out[31:] == 7.0).all()
    finally:
        pool.close()
