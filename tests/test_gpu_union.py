"""GPU parity of the speculative step with a selection per query token
(hs_select_topk_union -> hs_resolve_rows of the union ->
hs_sparse_mla_decode_union) against DecodeOracle.step_union, through the C
ABI: per-token top-K, the union and each token's union positions, the plan,
counts, slot tags, stamps, reverse map, LRU order, page stamps and step
counters bit-exact; pool rows behind the plan byte-identical to the logical
rows; each query token's attention over its own rows within 2e-3 of the fp64
oracle.

Cases: the agent shape reduced (4 requests, growing contexts, fp8 rows,
drafts scored near the base token), drafts scored independently (unions up
to the capacity), identical scores for every token (union = selection),
contexts shorter than the per-token K, a bf16 pool, a request id out of
range, and the full-size agent16-union workload over its first two turns.
"""
import dataclasses

import numpy as np
import pytest
import torch

from gpu_helpers import Runner, log, small
from sparse_mla_decode_indexer_amd import workload as W

pytestmark = pytest.mark.gpu


def _union_spec(**kw):
    base = dict(n_req=4, growth=(6000, 300, 40, 3), gpu_token_budget=1024, steps=30)
    base.update(kw)
    return small("agent16-union", **base)


@pytest.mark.parametrize("case", ["drafts-near", "drafts-independent", "identical", "short", "bf16"])
def test_union_step(case):
    kw = {}
    if case == "drafts-independent":
        kw = dict(token_noise=100.0, steps=12)
    elif case == "identical":
        kw = dict(token_noise=0.0, steps=12)
    elif case == "short":
        kw = dict(growth=(900, 200, 40, 2), steps=20)  # L < k in turn 1, L > k in turn 2
    elif case == "bf16":
        kw = dict(kv_dtype="bf16", steps=12)
    spec = _union_spec(**kw)
    log(f"[gpu] union step {case}: {spec.n_req} requests, Q={spec.q_per_req}, k={spec.select_k}, "
        f"capacity {spec.top_k}, {spec.steps} steps")
    wl = W.generate(spec)
    rn = Runner(wl)
    rn.incremental = True
    sizes = []
    try:
        for n in range(spec.steps):
            ref = rn.step(heads=None if n in (0, spec.steps - 1) else [0, 77])
            sizes.append(max(int((u >= 0).sum()) for u in ref["union"]))
        log(f"[gpu]   {case}: union sizes {min(sizes)}..{max(sizes)}, max err {rn.max_err:.2e}")
        if case == "identical":
            assert max(sizes) <= spec.select_k
        if case == "drafts-independent":
            assert max(sizes) > 3 * spec.select_k
    finally:
        rn.close()


def test_union_request_id_out_of_range():
    spec = _union_spec(steps=2)
    wl = W.generate(spec)
    rn = Runner(wl)
    try:
        rn.step()
        buf = rn.buf
        bad = torch.tensor([0, 99, 2, 3], dtype=torch.int32, device="cuda")
        buf.sel.fill_(7)
        buf.idx.fill_(7)
        buf.upos.fill_(7)
        rn.pool.select_topk_union(buf.scores[0], bad, buf.sel, buf.idx, buf.upos)
        torch.cuda.synchronize()
        code = rn.pool.device_error()
        assert code[0] == 4 and code[1] == 1 and code[2] == 99, code
        assert (buf.sel[1] == -1).all() and (buf.idx[1] == -1).all() and (buf.upos[1] == -1).all()
        assert (buf.idx[0] >= 0).any()
    finally:
        rn.close()


def test_union_full_size_first_turns():
    spec = dataclasses.replace(W.SPECS["agent16-union"], steps=110)
    log(f"[gpu] union full size: {spec.n_req} requests, first {spec.steps} steps")
    wl = W.generate(spec)
    rn = Runner(wl, sharded=True)
    rn.incremental = True
    try:
        for n in range(spec.steps):
            ref = rn.step(heads=None if n in (0, 55, 109) else [3, 64])
            if n % 25 == 0 or n == 109:
                log(f"[gpu]   agent16-union step {n + 1}: union sizes "
                    f"{min(int((u >= 0).sum()) for u in ref['union'])}.."
                    f"{max(int((u >= 0).sum()) for u in ref['union'])}, counts "
                    f"{np.asarray(ref['counts']).sum(axis=0).tolist()}, max err {rn.max_err:.2e}")
    finally:
        rn.close()
