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


def _graph_vs_eager(spec, step_fn, replays=4, eager_fn=None):
    """Capture one step in a hipGraph on pool B and replay it `replays`
    times, with new inputs copied in eagerly between the replays; the same
    steps run eagerly on twin pool A (through eager_fn when given). Every
    replay's outputs and the final LRU state must be bit-identical to the
    eager run."""
    eager_fn = eager_fn or step_fn
    from sparse_mla_decode_indexer_amd import harness as Hn
    wl_a, wl_b = W.generate(spec), W.generate(spec)
    pa, pb = Hn.make_pool(wl_a), Hn.make_pool(wl_b)
    try:
        Hn.load_workload(pa, wl_a)
        Hn.load_workload(pb, wl_b)
        ba, bb = Hn.StepBuffers(wl_a), Hn.StepBuffers(wl_b)
        ss, qs = W.ScoreStream(wl_a), W.QueryStream(wl_a)
        nxt = (lambda: ss.next_tokens(wl_a.ctx0)) if spec.select_k else (lambda: ss.next(wl_a.ctx0))
        sc, q = nxt(), qs.next()
        ba.upload(0, sc, q)
        bb.upload(0, sc, q)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step_fn(pb, bb)
        for n in range(replays):
            if n > 0:
                sc, q = nxt(), qs.next()
                ba.upload(0, sc, q)
                bb.upload(0, sc, q)
            torch.cuda.synchronize()
            g.replay()
            eager_fn(pa, ba)
            torch.cuda.synchronize()
            for name in ("idx", "plan", "counts", "out", "lse") + (("sel", "upos") if spec.select_k else ()):
                assert torch.equal(getattr(ba, name), getattr(bb, name)), f"replay {n}: {name}"
        sa, sb = pa.state_views(), pb.state_views()
        for k in ("slot_tag", "slot_stamp", "lru_order", "rev", "step", "page_stamp"):
            assert torch.equal(sa[k], sb[k]), k
        assert pa.device_error()[0] == 0 and pb.device_error()[0] == 0
    finally:
        pa.close()
        pb.close()


def test_union_step_graph_replays_match_eager():
    log("[gpu] union step: hipGraph replays vs eager")
    from sparse_mla_decode_indexer_amd import harness as Hn
    _graph_vs_eager(_union_spec(steps=4), lambda pool, buf: Hn.decode_step(pool, buf, 0))


@pytest.mark.parametrize("case", ["fp8-q1", "fp8-q4", "f32"])
def test_fp8_and_f32_step_graph_replays_match_eager(case):
    """A plain step over fp8 rows (one query token, and four sharing one
    plan; the attention widens the codes in registers) or fp32 rows (split
    vector attention and its merge) captured in a hipGraph and replayed with
    new inputs, bit-identical to eager steps."""
    log(f"[gpu] step ({case}): hipGraph replays vs eager")
    from sparse_mla_decode_indexer_amd import harness as Hn
    if case == "fp8-q1":
        spec = small("single-1m-fp8", ctx=40000, host_pages=563, scores=("ar1_shift", 0.95, 0.5), steps=4)
    elif case == "fp8-q4":
        spec = small("agent16", n_req=3, growth=(5000, 300, 40, 2), gpu_token_budget=2048, steps=20)
    else:
        spec = W.SPECS["tiny"]
    _graph_vs_eager(spec, lambda pool, buf: Hn.decode_step(pool, buf, 0))


def test_noalloc_attention_graph_replays_match_eager():
    """The allocation-free attention entry point (the form for callers under
    graph capture) inside a captured step, replayed with new inputs."""
    log("[gpu] no-alloc attention step: hipGraph replays vs eager")

    def step(pool, buf):
        pool.select_topk(buf.scores[0], buf.req_ids, buf.idx)
        pool.resolve_rows(buf.idx, buf.req_ids, buf.plan, buf.counts)
        pool.sparse_mla_decode_noalloc(buf.q[0], buf.plan, buf.sm_scale, buf.out, buf.lse)
    _graph_vs_eager(small("batch32", n_req=3, ctx_range=(8192, 30000), steps=4), step)


def test_select_resolve_step_graph_replays_match_two_calls():
    """A step with top-K and resolve as one call (hs_select_resolve), captured
    in a hipGraph and replayed with new inputs, against the same steps run
    eagerly as separate top-K and resolve calls."""
    log("[gpu] select_resolve step: hipGraph replays vs eager two-call steps")
    from sparse_mla_decode_indexer_amd import harness as Hn
    _graph_vs_eager(small("batch32", n_req=5, ctx_range=(4096, 40000), steps=4),
                    lambda pool, buf: Hn.decode_step(pool, buf, 0, fused=True),
                    eager_fn=lambda pool, buf: Hn.decode_step(pool, buf, 0))


@pytest.mark.parametrize("Q,cap", [(4, 2048), (8, 4096)], ids=["q4", "q8-limits"])
@pytest.mark.parametrize("max_ctx", [20000, 1 << 20], ids=["bitmap", "search"])
def test_union_kernel_forms(max_ctx, Q, cap):
    """The union of per-token selections is formed from a token bitmap in LDS
    when the pool's max_context fits one, else by binary searches over the
    selections (here: a pool sized for 1M-token contexts). Either way it
    equals the per-token definition: each query token's top-k of its own
    scores, their sorted union and each selected token's union position.
    Also at the limits: 8 query tokens with a selection each (the most)
    and a union capacity of 4,096 (the largest top-K)."""
    from oracle import select_topk, union_of_selections
    from sparse_mla_decode_indexer_amd.pool import TieredPool
    log(f"[gpu] union kernel form for max_context {max_ctx}, Q={Q}, capacity {cap}")
    k, R = 512, 3
    lens = [300, 9000, 20000]  # L < k, L > k, L = the small pool's max_context
    rng = np.random.default_rng(11)
    pool = TieredPool(page_size=64, num_pool_pages=8, max_requests=R, max_context=max_ctx, kv_dtype="bf16",
                      top_k=cap, hot_rows=cap, max_batch=R, max_q_rows=64, host_rows=R * 20000, select_q=Q)
    try:
        stride = max_ctx
        sc = np.zeros((R, Q, stride), dtype=np.float32)
        for r, L in enumerate(lens):
            base = rng.standard_normal(L).astype(np.float32)
            for t in range(Q):  # nearby drafts: overlapping but different selections
                sc[r, t, :L] = base + np.float32(0.3) * rng.standard_normal(L).astype(np.float32)
            sc[r, 2, :L:7] = sc[r, 1, :L:7]  # some equal scores across tokens
            if Q > 4:  # independent drafts: unions near the capacity
                sc[r, 4:, :L] = rng.standard_normal((Q - 4, L)).astype(np.float32)
            pool.set_residency(r, L, r * 20000, None)
        d_sc = torch.from_numpy(sc).cuda()
        req = torch.arange(R, dtype=torch.int32, device="cuda")
        sel = torch.full((R, Q, k), -5, dtype=torch.int32, device="cuda")
        union = torch.full((R, cap), -5, dtype=torch.int32, device="cuda")
        upos = torch.full((R, Q, k), -5, dtype=torch.int32, device="cuda")
        for rep in range(2):  # the scratch must be clean for a second call
            pool.select_topk_union(d_sc, req, sel, union, upos)
            g_sel, g_un, g_up = sel.cpu().numpy(), union.cpu().numpy(), upos.cpu().numpy()
            for r, L in enumerate(lens):
                want = [select_topk(sc[r, t], L, k) for t in range(Q)]
                u_ref, up_ref = union_of_selections(want, cap)
                assert np.array_equal(g_sel[r], np.stack(want)), (rep, r)
                assert np.array_equal(g_un[r], u_ref), (rep, r)
                assert np.array_equal(g_up[r], up_ref), (rep, r)
        assert pool.device_error()[0] == 0
    finally:
        pool.close()
