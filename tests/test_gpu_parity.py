"""GPU parity of the decode step against the CPU oracle (through the C ABI).

Reduced variants of every workload (same dtypes, heads, top-K, hot rows,
residency rule and score process; shorter contexts) step in lockstep with
the oracle; see gpu_helpers.Runner for what is compared.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import Runner, log, small
from oracle import mla_attention, select_topk
from sparse_mla_decode_indexer_amd import harness as Hn
from sparse_mla_decode_indexer_amd import workload as W
from sparse_mla_decode_indexer_amd.pool import TieredPool

pytestmark = pytest.mark.gpu


def run_steps(spec, steps, heads=None):
    log(f"[gpu] {spec.name}: ctx={spec.ctx or spec.ctx_range or spec.growth} steps={steps}")
    wl = W.generate(spec)
    rn = Runner(wl)
    try:
        for _ in range(steps):
            rn.step(heads=heads)
        log(f"[gpu] {spec.name}: max attention rel err {rn.max_err:.2e}")
        return rn.max_err
    finally:
        rn.close()


def test_tiny_fp32_all_steps():
    run_steps(W.SPECS["tiny"], 8)


def test_single_bf16_reduced():
    run_steps(small("single-128k", ctx=16384, host_pages=192), 6)


def test_batch_ragged_bf16_reduced():
    # contexts 1000..20000: several requests have L < K = 2048 (all selected,
    # -1 padding) and one has a partial last page
    run_steps(small("batch32", n_req=6, ctx_range=(1000, 20000)), 5)


def test_single_fp8_reduced_with_topic_shifts():
    run_steps(small("single-1m-fp8", ctx=40000, host_pages=563, scores=("ar1_shift", 0.95, 0.5)), 6)


def test_agent_q4_fp8_growing():
    spec = small("agent16", n_req=3, growth=(5000, 300, 40, 2), gpu_token_budget=1 << 20, steps=20)
    run_steps(spec, 12)


def test_multi_layer_step():
    """Four layers of two requests in one call of each entry point (layer-
    major slots, each with its own rows, scores, queries, page table and hot
    buffer): every slot bit-exact / within the bar, as a batch would be."""
    run_steps(small("layers16-128k-fp8", n_req=8, layers=4, ctx=16384, host_pages=192), 4, heads=[0, 127])


def test_small_page_and_min_hot_buffer():
    # page size 16, S == K: every miss must reuse an untouched slot
    spec = small("single-128k", ctx=6000, host_pages=280, page_size=16, top_k=256, hot_rows=256)
    run_steps(spec, 6)


@pytest.mark.parametrize("base", ["single-128k", "single-1m-fp8"])
@pytest.mark.parametrize("K,S", [(100, 256), (7, 64)])
def test_ragged_top_k_through_the_step(base, K, S):
    # a top-K that is not a multiple of the 32-row attention tile: the last
    # tile of the plan is partly empty (100 = 3 x 32 + 4; 7 < 32), through
    # top-K, resolve (misses, hits, LRU) and attention, bf16 and fp8 rows
    scores = ("ar1", 0.9)
    run_steps(small(base, ctx=6000, host_pages=60, top_k=K, hot_rows=S, scores=scores), 6)


@pytest.mark.parametrize("K", [1, 7, 256, 2048])
def test_topk_ties_and_sizes(K):
    rng = np.random.default_rng(K)
    max_ctx = 70000
    pool = TieredPool(page_size=64, num_pool_pages=8, max_requests=8, max_context=max_ctx,
                      kv_dtype="bf16", top_k=K, hot_rows=max(2 * K, 64), max_batch=8, max_q_rows=16,
                      host_rows=8 * max_ctx)
    try:
        lens = [0, 1, K, K + 1, 5000, 2049, 65537, max_ctx]
        stride = 70016
        sc = np.zeros((8, stride), dtype=np.float32)
        sc[0] = rng.standard_normal(stride)
        sc[1] = -0.0
        sc[2] = rng.integers(-2, 3, stride)
        sc[3] = 1.0                                          # all equal
        sc[4] = rng.integers(-3, 3, stride) * np.float32(0.5)
        sc[4, ::3] = -0.0
        sc[5] = rng.standard_normal(stride) * 1e-30          # tiny magnitudes
        sc[6] = rng.standard_normal(stride).astype(np.float32)
        sc[6, 100:200] = 1e38
        sc[7] = rng.standard_normal(stride)
        sc[7, rng.integers(0, max_ctx, 3000)] = 7.25          # many ties at the top
        for r, L in enumerate(lens):
            pool.set_residency(r, L, r * max_ctx, None)
        d_sc = torch.from_numpy(sc).cuda()
        req = torch.arange(8, dtype=torch.int32, device="cuda")
        idx = torch.full((8, K), -5, dtype=torch.int32, device="cuda")
        for rep in range(2):  # the scratch must be clean for a second call
            pool.select_topk(d_sc, req, idx)
            got = idx.cpu().numpy()
            for r, L in enumerate(lens):
                want = select_topk(sc[r], L, K)
                assert np.array_equal(got[r], want), f"K={K} req {r} L={L} rep {rep}"
        assert pool.device_error()[0] == 0
    finally:
        pool.close()


def test_topk_many_requests():
    """The tie, magnitude and length cases of test_topk_ties_and_sizes
    repeated over 40 requests in one call (360 filter workgroups, 40 select
    workgroups), two calls each."""
    rng = np.random.default_rng(11)
    K, R, max_ctx = 2048, 40, 70000
    pool = TieredPool(page_size=64, num_pool_pages=8, max_requests=R, max_context=max_ctx,
                      kv_dtype="bf16", top_k=K, hot_rows=2 * K, max_batch=R, max_q_rows=16,
                      host_rows=R * max_ctx)
    try:
        lens = [0, 1, K, K + 1, 5000, 2049, 65537, max_ctx] * (R // 8)
        stride = 70016
        sc = rng.standard_normal((R, stride)).astype(np.float32)
        for r in range(0, R, 8):
            sc[r + 1] = -0.0
            sc[r + 2] = rng.integers(-2, 3, stride)
            sc[r + 3] = 1.0
            sc[r + 5] *= 1e-30
            sc[r + 6, 100:200] = 1e38
            sc[r + 7, rng.integers(0, max_ctx, 3000)] = 7.25
        for r, L in enumerate(lens):
            pool.set_residency(r, L, r * max_ctx, None)
        d_sc = torch.from_numpy(sc).cuda()
        req = torch.arange(R, dtype=torch.int32, device="cuda")
        idx = torch.full((R, K), -5, dtype=torch.int32, device="cuda")
        for rep in range(2):
            pool.select_topk(d_sc, req, idx)
            got = idx.cpu().numpy()
            for r, L in enumerate(lens):
                assert np.array_equal(got[r], select_topk(sc[r], L, K)), f"req {r} L={L} rep {rep}"
        assert pool.device_error()[0] == 0
    finally:
        pool.close()


def test_fp8_codes_exhaustive_single_row():
    """With K = 1 the output is the selected row's value part exactly, so
    every finite e4m3 code, widened by the kernel and scaled, must equal the
    OCP decoding times the row scale."""
    from oracle import e4m3fn_decode
    spec = small("single-1m-fp8", ctx=256, host_pages=0, top_k=1, hot_rows=64, heads=16, steps=1)
    wl = W.generate(spec)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    for t in range(wl.rows.shape[0]):
        wl.rows[t] = np.resize(np.roll(codes, t), 576)
    wl.scales[:] = np.float32(0.375)
    rn = Runner(wl)
    try:
        rn.step()
        out = rn.buf.out.cpu().numpy()[0, 0]
        t = int(rn.buf.idx.cpu().numpy()[0, 0])
        want = e4m3fn_decode(wl.rows[t][:512]) * 0.375
        assert np.array_equal(out, np.broadcast_to(want, out.shape).astype(np.float32))
    finally:
        rn.close()


def test_residency_invariance_bitwise():
    """The same logical inputs under all-resident, 75%-host and all-host
    layouts give bit-identical attention outputs (rows from every tier are
    the same bytes)."""
    outs = []
    for hp in (0, 96, 128):
        spec = small("single-128k", ctx=8192, host_pages=hp)
        wl = W.generate(spec)
        rn = Runner(wl)
        try:
            per = []
            for _ in range(3):
                rn.step(heads=range(8))
                per.append((rn.buf.out.cpu().numpy().copy(), rn.buf.lse.cpu().numpy().copy()))
            outs.append(per)
        finally:
            rn.close()
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    for a, b in zip(outs[0], outs[2]):
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_unselected_rows_never_read():
    """Poison every row that no step selects (host store and pool) with NaN
    patterns: outputs stay finite and bit-identical to a clean run."""
    spec = small("single-128k", ctx=8192, host_pages=96)
    steps = 4
    clean = W.generate(spec)
    # selections of the run, from the oracle
    from gpu_helpers import make_oracle
    orc = make_oracle(clean)
    ss = W.ScoreStream(clean)
    used = set()
    for _ in range(steps):
        res = orc.step(ss.next(clean.ctx0), None, clean.ctx0, with_attention=False)
        used.update(int(t) for t in res["idx"][0] if t >= 0)
    runs = []
    for poison in (False, True):
        wl = W.generate(spec)
        if poison:
            mask = np.ones(wl.rows.shape[0], bool)
            mask[list(used)] = False
            wl.rows[mask] = 0xFFFF
        rn = Runner(wl)
        try:
            outs = []
            for _ in range(steps):
                rn.step(heads=range(4))
                o = rn.buf.out.cpu().numpy().copy()
                assert np.isfinite(o).all()
                outs.append(o)
            runs.append(outs)
        finally:
            rn.close()
    for a, b in zip(*runs):
        assert np.array_equal(a, b)


def test_graph_replay_matches_eager():
    """The three calls captured in a hipGraph and replayed give bit-identical
    results to eager launches, step after step (device state advances
    without host input)."""
    from sparse_mla_decode_indexer_amd import harness as Hn
    spec = small("single-128k", ctx=16384, host_pages=192)
    steps = 5
    wl_a, wl_b = W.generate(spec), W.generate(spec)
    pa, pb = Hn.make_pool(wl_a), Hn.make_pool(wl_b)
    try:
        Hn.load_workload(pa, wl_a)
        Hn.load_workload(pb, wl_b)
        ba, bb = Hn.StepBuffers(wl_a, n_steps=steps), Hn.StepBuffers(wl_b, n_steps=steps)
        ss, qs = W.ScoreStream(wl_a), W.QueryStream(wl_a)
        for n in range(steps):
            sc, q = ss.next(wl_a.ctx0), qs.next()
            ba.upload(n, sc, q)
            bb.upload(n, sc, q)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        outs_b = []
        with torch.cuda.graph(g):
            for n in range(steps):
                Hn.decode_step(pb, bb, n)
                outs_b.append((bb.idx.clone(), bb.plan.clone(), bb.out.clone(), bb.lse.clone()))
        g.replay()
        torch.cuda.synchronize()
        for n in range(steps):
            Hn.decode_step(pa, ba, n)
            torch.cuda.synchronize()
            for x, y in zip((ba.idx, ba.plan, ba.out, ba.lse), outs_b[n]):
                assert torch.equal(x, y), f"step {n}"
        sa, sb = pa.state_views(), pb.state_views()
        for k in ("slot_tag", "slot_stamp", "lru_order", "rev", "step"):
            assert torch.equal(sa[k], sb[k]), k
    finally:
        pa.close()
        pb.close()


def test_device_error_on_index_past_context():
    spec = small("single-128k", ctx=4096, host_pages=48, top_k=256, hot_rows=512)
    wl = W.generate(spec)
    rn = Runner(wl)
    try:
        idx = torch.arange(256, dtype=torch.int32, device="cuda")[None].clone()
        idx[0, 5] = 5000  # past L = 4096
        rn.pool.resolve_rows(idx, rn.buf.req_ids, rn.buf.plan, rn.buf.counts)
        code = rn.pool.device_error()
        assert code[0] == 1 and code[2] == 5000
        assert rn.buf.plan[0, 5].item() == -1
        assert rn.buf.counts[0].sum().item() == 255
        rn.pool.clear_device_error()
        assert rn.pool.device_error()[0] == 0
    finally:
        rn.close()


def test_topk_both_paths_in_one_batch():
    """Long contexts (up to 300K tokens) in one call, with ties, -0.0 and an
    empty request. On the first call (no bound yet) every score survives the
    filter: the select narrows them to a cut by histogram passes, except for
    the all-equal request, whose ties at the K-th value exceed what LDS can
    stage and which takes the unstaged path; the second call starts from the
    bound the first one left."""
    rng = np.random.default_rng(5)
    max_ctx, K = 300000, 2048
    lens = [300000, 262145, 262144, 70001, 0, 290000]
    R = len(lens)
    pool = TieredPool(page_size=64, num_pool_pages=8, max_requests=R, max_context=max_ctx,
                      kv_dtype="bf16", top_k=K, hot_rows=4096, max_batch=R, max_q_rows=16,
                      host_rows=R * max_ctx)
    try:
        stride = 300032
        sc = rng.standard_normal((R, stride)).astype(np.float32)
        sc[1, ::7] = np.float32(2.5)          # many ties near the threshold
        sc[2] = np.round(sc[2] * 4) / 4       # coarse values: heavy ties
        sc[3, ::5] = -0.0
        sc[5] = 1.0                            # all equal
        for r, L in enumerate(lens):
            pool.set_residency(r, L, r * max_ctx, None)
        d_sc = torch.from_numpy(sc).cuda()
        req = torch.arange(R, dtype=torch.int32, device="cuda")
        idx = torch.full((R, K), -5, dtype=torch.int32, device="cuda")
        for rep in range(2):
            pool.select_topk(d_sc, req, idx)
            got = idx.cpu().numpy()
            for r, L in enumerate(lens):
                assert np.array_equal(got[r], select_topk(sc[r], L, K)), f"req {r} L={L} rep {rep}"
        assert pool.device_error()[0] == 0
    finally:
        pool.close()


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("shape", ["rising", "jumps", "falling", "one_dominant"])
def test_attention_score_jumps(kv, shape):
    """The kernel's softmax keeps a reference maximum that moves only when a
    score passes it by more than 2^8. Scores that climb slowly (rising: the
    reference moves now and then, weights up to ~2^8 in between, about 8
    rows share the weight), climb by far more than that from tile to tile
    (jumps), start high and decay (falling), or are set by one row in the
    last tile (one_dominant), with absent plan entries mixed in: every head
    within the fp64 bar."""
    from oracle import bf16_decode, e4m3fn_decode
    from gpu_helpers import ATTN_TOL, LSE_TOL, attn_rel_err
    rng = np.random.default_rng({"rising": 1, "jumps": 4, "falling": 2, "one_dominant": 3}[shape])
    K, H, n_rows = 2048, 128, 4096
    pool = TieredPool(page_size=64, num_pool_pages=n_rows // 64, max_requests=1, max_context=n_rows,
                      kv_dtype=kv, top_k=K, hot_rows=4096, max_batch=1, max_q_rows=H, host_rows=64)
    try:
        x = rng.standard_normal((n_rows, W.ROW_DIM)).astype(np.float32)
        plan = rng.permutation(n_rows)[:K].astype(np.int32)
        plan[rng.integers(0, K, 40)] = -1
        plan[-7:] = -1
        tile = np.arange(K) // 32
        if shape == "rising":
            f = 1.0 + 0.05 * tile
        elif shape == "jumps":
            f = 1.0 + 2.0 * tile
        elif shape == "falling":
            f = 1.0 + 2.0 * (tile.max() - tile)
        else:
            f = np.full(K, 0.5)
        q = rng.standard_normal((H, W.ROW_DIM)).astype(np.float32)
        live = plan >= 0
        x[plan[live]] *= f[live, None].astype(np.float32)
        if shape == "one_dominant":
            j = int(np.flatnonzero(live)[-1])
            x[plan[j]] = 3.0 * q[5]          # head 5 puts nearly all weight on it
        sm = 1.0 / np.sqrt(W.ROW_DIM)
        if kv == "bf16":
            bits = W.f32_to_bf16_bits(x)
            pool.pool_row_view().copy_(torch.from_numpy(bits.view(np.uint8).reshape(n_rows, -1)).cuda())
            logical = bf16_decode(bits)
        else:
            codes, sc = W.f32_rows_to_fp8(x)
            pool.pool_row_view().copy_(torch.from_numpy(codes).cuda())
            pool.pool_scales.copy_(torch.from_numpy(sc).cuda())
            logical = e4m3fn_decode(codes) * sc[:, None].astype(np.float64)
        qb = W.f32_to_bf16_bits(q)
        d_q = torch.from_numpy(qb.view(np.int16)).cuda().view(torch.bfloat16).reshape(1, 1, H, W.ROW_DIM)
        d_plan = torch.from_numpy(plan).cuda().reshape(1, K)
        out = torch.full((1, 1, H, W.NOPE_DIM), np.nan, device="cuda")
        lse = torch.full((1, 1, H), np.nan, device="cuda")
        pool.sparse_mla_decode(d_q, d_plan, sm, out, lse)
        o = out.cpu().numpy().reshape(H, -1)
        l = lse.cpu().numpy().reshape(H)
        o_ref, l_ref = mla_attention(bf16_decode(qb), logical[plan[live]], sm)
        e = attn_rel_err(o, o_ref)
        assert e <= ATTN_TOL, f"{kv} {shape}: attention rel err {e:.3e}"
        le = float(np.max(np.abs(l - l_ref) / np.maximum(1.0, np.abs(l_ref))))
        assert le <= LSE_TOL, f"{kv} {shape}: lse err {le:.3e}"
        assert pool.device_error()[0] == 0
    finally:
        pool.close()


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_attention_absent_rows_over_nan_lds(kv):
    """Absent plan entries read zeros, whatever the tile buffers held
    before: a first call gathers NaN rows into every tile buffer, then a
    plan with absent entries (a ragged tail and scattered -1s) over finite
    rows must give finite outputs within the fp64 bar. A gather that left
    stale bytes in place of an absent row would turn its zero weight into
    NaN."""
    from oracle import bf16_decode, e4m3fn_decode
    from gpu_helpers import ATTN_TOL, attn_rel_err
    rng = np.random.default_rng(11)
    K, H, n_rows = 2048, 128, 4096
    pool = TieredPool(page_size=64, num_pool_pages=n_rows // 64, max_requests=1, max_context=n_rows,
                      kv_dtype=kv, top_k=K, hot_rows=4096, max_batch=1, max_q_rows=H, host_rows=64)
    try:
        sm = 1.0 / np.sqrt(W.ROW_DIM)
        q = rng.standard_normal((H, W.ROW_DIM)).astype(np.float32)
        qb = W.f32_to_bf16_bits(q)
        d_q = torch.from_numpy(qb.view(np.int16)).cuda().view(torch.bfloat16).reshape(1, 1, H, W.ROW_DIM)
        out = torch.empty((1, 1, H, W.NOPE_DIM), device="cuda")
        # 1. every row NaN (bf16 0x7FC0; e4m3fn 0x7F), every plan entry present
        if kv == "bf16":
            pool.pool_row_view().view(torch.int16).fill_(0x7FC0)
        else:
            pool.pool_row_view().fill_(0x7F)
            pool.pool_scales.fill_(1.0)
        full = torch.from_numpy(rng.permutation(n_rows)[:K].astype(np.int32)).cuda().reshape(1, K)
        pool.sparse_mla_decode(d_q, full, sm, out, None)
        torch.cuda.synchronize()
        # 2. finite rows, absent entries
        x = rng.standard_normal((n_rows, W.ROW_DIM)).astype(np.float32)
        if kv == "bf16":
            bits = W.f32_to_bf16_bits(x)
            pool.pool_row_view().copy_(torch.from_numpy(bits.view(np.uint8).reshape(n_rows, -1)).cuda())
            logical = bf16_decode(bits)
        else:
            codes, sc = W.f32_rows_to_fp8(x)
            pool.pool_row_view().copy_(torch.from_numpy(codes).cuda())
            pool.pool_scales.copy_(torch.from_numpy(sc).cuda())
            logical = e4m3fn_decode(codes) * sc[:, None].astype(np.float64)
        plan = rng.permutation(n_rows)[:K].astype(np.int32)
        plan[rng.integers(0, K, 300)] = -1
        plan[-100:] = -1
        live = plan >= 0
        d_plan = torch.from_numpy(plan).cuda().reshape(1, K)
        pool.sparse_mla_decode(d_q, d_plan, sm, out, None)
        o = out.cpu().numpy().reshape(H, -1)
        assert np.isfinite(o).all()
        o_ref, _ = mla_attention(bf16_decode(qb), logical[plan[live]], sm)
        e = attn_rel_err(o, o_ref)
        assert e <= ATTN_TOL, f"{kv}: attention rel err {e:.3e}"
        assert pool.device_error()[0] == 0
    finally:
        pool.close()


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_attention_pool_over_4gib(kv):
    """A pool of more than 4 GiB of rows (65,536 bf16 or 131,072 fp8 pages of
    64 rows): the gathers then use 64-bit addresses instead of a 32-bit
    buffer view. The plan's rows are spread over the whole pool, the highest
    ones past the 4 GiB mark, with absent entries; every head within the
    fp64 bar."""
    from oracle import bf16_decode, e4m3fn_decode
    from gpu_helpers import ATTN_TOL, attn_rel_err
    rng = np.random.default_rng(12)
    K, H = 2048, 128
    pages = 65536 if kv == "bf16" else 131072
    n_rows = pages * 64
    pool = TieredPool(page_size=64, num_pool_pages=pages, max_requests=1, max_context=1 << 16,
                      kv_dtype=kv, top_k=K, hot_rows=4096, max_batch=1, max_q_rows=H, host_rows=64)
    try:
        assert n_rows * pool.row_bytes > (1 << 32)
        top = n_rows - 16 + np.arange(16)        # the pool's last 16 rows
        plan = np.concatenate([np.sort(rng.choice(n_rows - 16, K - 16, replace=False)), top]).astype(np.int32)
        assert int(plan.max()) * pool.row_bytes >= (1 << 32)
        x = rng.standard_normal((K, W.ROW_DIM)).astype(np.float32)
        d_idx = torch.from_numpy(plan.astype(np.int64)).cuda()
        if kv == "bf16":
            bits = W.f32_to_bf16_bits(x)
            pool.pool_row_view()[d_idx] = torch.from_numpy(bits.view(np.uint8).reshape(K, -1)).cuda()
            logical = bf16_decode(bits)
        else:
            codes, sc = W.f32_rows_to_fp8(x)
            pool.pool_row_view()[d_idx] = torch.from_numpy(codes).cuda()
            pool.pool_scales[d_idx] = torch.from_numpy(sc).cuda()
            logical = e4m3fn_decode(codes) * sc[:, None].astype(np.float64)
        live = np.ones(K, bool)
        live[rng.integers(0, K, 50)] = False
        q = rng.standard_normal((H, W.ROW_DIM)).astype(np.float32)
        qb = W.f32_to_bf16_bits(q)
        d_q = torch.from_numpy(qb.view(np.int16)).cuda().view(torch.bfloat16).reshape(1, 1, H, W.ROW_DIM)
        d_plan = torch.from_numpy(np.where(live, plan, -1).astype(np.int32)).cuda().reshape(1, K)
        out = torch.empty((1, 1, H, W.NOPE_DIM), device="cuda")
        sm = 1.0 / np.sqrt(W.ROW_DIM)
        pool.sparse_mla_decode(d_q, d_plan, sm, out, None)
        o = out.cpu().numpy().reshape(H, -1)
        o_ref, _ = mla_attention(bf16_decode(qb), logical[live], sm)
        e = attn_rel_err(o, o_ref)
        assert e <= ATTN_TOL, f"{kv}: attention rel err {e:.3e}"
        assert pool.device_error()[0] == 0
    finally:
        pool.close()


def test_imported_prefix_start_shared_host_rows():
    """None-resident start from an imported prefix ([P2] residency state 3,
    and P/D imports landing host-side): request 1 reuses request 0's prefix,
    which exists only in the host store (its page table is all placeholders,
    its hot buffer empty), while request 0 keeps its newest pages on the GPU.
    The prefix rows land in the host store after both requests are set up.
    Both requests read the same host rows; every step is checked as in the
    other parity tests."""
    spec = small("single-128k", n_req=2, ctx=16384, host_pages=160, steps=6)
    wl = W.generate(spec)
    wl.gpu_page[1][:] = -1                  # request 1: placeholders only
    wl.host_base[1] = wl.host_base[0]       # ... over request 0's imported rows
    rn = Runner(wl)
    try:
        a, n = int(wl.host_base[0]), int(wl.ctx0[0])
        rn.pool.host_store[a:a + n] = 0xFF  # the import has not landed yet
        rn.pool.host_store[a:a + n] = rn.raw[a:a + n]  # ... now it has
        for _ in range(spec.steps):
            ref = rn.step(heads=[0, 127])
        assert np.asarray(ref["counts"])[1][0] == 0  # request 1 never reads a resident row
    finally:
        rn.close()


@pytest.mark.parametrize("kv", ["bf16", "fp8", "f32"])
def test_attention_plan_row_outside_pool_is_flagged_and_skipped(kv):
    """A plan entry at or past the pool's row count raises HS_DEV_PLAN_RANGE
    (first such entry: request position and plan index) and is treated as
    absent: the output equals attention over the remaining rows."""
    from oracle import bf16_decode, e4m3fn_decode
    from gpu_helpers import ATTN_TOL, attn_rel_err
    rng = np.random.default_rng(11)
    K, H, n_rows = 256, 16, 1024
    pool = TieredPool(page_size=64, num_pool_pages=n_rows // 64, max_requests=1, max_context=n_rows,
                      kv_dtype=kv, top_k=K, hot_rows=512, max_batch=1, max_q_rows=H, host_rows=64)
    try:
        x = rng.standard_normal((n_rows, W.ROW_DIM)).astype(np.float32)
        plan = rng.permutation(n_rows)[:K].astype(np.int32)
        bad = 37
        plan[bad] = n_rows + 5          # outside the pool
        live = np.ones(K, dtype=bool)
        live[bad] = False
        q = rng.standard_normal((H, W.ROW_DIM)).astype(np.float32)
        sm = 1.0 / np.sqrt(W.ROW_DIM)
        if kv == "f32":
            pool.pool_row_view().copy_(torch.from_numpy(x.view(np.uint8).reshape(n_rows, -1)).cuda())
            logical = x.astype(np.float64)
            qd = q.astype(np.float64)
            d_q = torch.from_numpy(q).cuda().reshape(1, 1, H, W.ROW_DIM)
        else:
            if kv == "bf16":
                bits = W.f32_to_bf16_bits(x)
                pool.pool_row_view().copy_(torch.from_numpy(bits.view(np.uint8).reshape(n_rows, -1)).cuda())
                logical = bf16_decode(bits)
            else:
                codes, sc = W.f32_rows_to_fp8(x)
                pool.pool_row_view().copy_(torch.from_numpy(codes).cuda())
                pool.pool_scales.copy_(torch.from_numpy(sc).cuda())
                logical = e4m3fn_decode(codes) * sc[:, None].astype(np.float64)
            qb = W.f32_to_bf16_bits(q)
            qd = bf16_decode(qb)
            d_q = torch.from_numpy(qb.view(np.int16)).cuda().view(torch.bfloat16).reshape(1, 1, H, W.ROW_DIM)
        d_plan = torch.from_numpy(plan).cuda().reshape(1, K)
        out = torch.full((1, 1, H, W.NOPE_DIM), np.nan, device="cuda")
        log(f"[gpu] plan row outside the pool, {kv}")
        pool.sparse_mla_decode(d_q, d_plan, sm, out, None)
        torch.cuda.synchronize()
        o = out.cpu().numpy().reshape(H, -1)
        o_ref, _ = mla_attention(qd, logical[plan[live]], sm)
        assert attn_rel_err(o, o_ref) <= ATTN_TOL
        err = pool.device_error()
        assert err[0] == 3 and err[1] == 0 and err[2] == bad, err  # HS_DEV_PLAN_RANGE
        pool.clear_device_error()
        assert pool.device_error()[0] == 0
    finally:
        pool.close()


def test_topk_request_id_outside_pool_is_flagged_and_padded():
    """A req_ids entry outside [0, max_requests) raises HS_DEV_REQUEST_RANGE
    and its top-K row is all -1; the other rows are unaffected."""
    K, maxc = 64, 4096
    pool = TieredPool(page_size=64, num_pool_pages=8, max_requests=2, max_context=maxc, kv_dtype="bf16",
                      top_k=K, hot_rows=64, max_batch=2, max_q_rows=16, host_rows=2 * maxc)
    try:
        rng = np.random.default_rng(5)
        sc = rng.standard_normal((2, maxc)).astype(np.float32)
        pool.set_residency(1, 3000, 0, None)
        req = torch.tensor([7, 1], dtype=torch.int32, device="cuda")
        idx = torch.full((2, K), -5, dtype=torch.int32, device="cuda")
        log("[gpu] top-K with a request id outside the pool")
        pool.select_topk(torch.from_numpy(sc).cuda(), req, idx)
        got = idx.cpu().numpy()
        assert np.all(got[0] == -1)
        assert np.array_equal(got[1], select_topk(sc[1], 3000, K))
        err = pool.device_error()
        assert err[0] == 4 and err[1] == 0 and err[2] == 7, err  # HS_DEV_REQUEST_RANGE
    finally:
        pool.close()


def test_set_residency_page_id_outside_pool_becomes_host_only():
    """A GPU page id at or past num_pool_pages given to set_residency raises
    HS_DEV_PAGE_RANGE (request, logical page) and the page is recorded as
    host-only: the following steps read its tokens from the host store and
    match the oracle with that page on the host (state checked too)."""
    spec = small("single-128k", ctx=6000, host_pages=60, top_k=256, hot_rows=512)
    wl = W.generate(spec)
    rn = Runner(wl)
    try:
        p = int(np.flatnonzero(wl.gpu_page[0] >= 0)[0])  # the oldest GPU page
        bad = torch.tensor([rn.pool.desc.num_pool_pages + 3], dtype=torch.int32, device="cuda")
        log(f"[gpu] set_residency with a page id outside the pool (logical page {p})")
        rn.pool.set_residency(0, int(wl.ctx0[0]), int(wl.host_base[0]), bad, first_page=p)
        torch.cuda.synchronize()
        err = rn.pool.device_error()
        assert err[0] == 2 and err[1] == 0 and err[2] == p, err  # HS_DEV_PAGE_RANGE
        rn.pool.clear_device_error()
        rn.oracle.set_pages(0, p, np.array([-1]))
        for _ in range(4):
            rn.step()
    finally:
        rn.close()


@pytest.mark.parametrize("group", [1, 3])
def test_pipelined_step_over_request_groups(group):
    """The step run as a pipeline over request groups on three streams
    (top-K, resolve and attention of group g; attention of g overlapping the
    resolve of g + 1) is bit-exact with the oracle like the sequential step:
    7 requests of mixed residency in groups of 1 and 3 (the last group
    shorter), cold and warm steps."""
    spec = small("batch32", n_req=7, ctx_range=(4096, 40000), steps=4)
    log(f"[gpu] pipelined step, groups of {group}")
    wl = W.generate(spec)
    rn = Runner(wl, group=group)
    try:
        for _ in range(4):
            rn.step(heads=[0, 77])
    finally:
        rn.close()


@pytest.mark.parametrize("fused", [False, True], ids=["two-calls", "select_resolve"])
def test_resolve_wait_that_gives_up_then_hot_reset_is_exact(monkeypatch, fused):
    """A copy wave whose bounded wait gives up raises HS_DEV_TIMEOUT (batch
    and plan position in range) instead of hanging; after clearing the error
    and resetting the hot buffers (the documented recovery) the following
    steps are bit-exact with the oracle, so no destination published late by
    the call that gave up is taken by a later call (each carries its call's
    epoch). The wait is made to give up with HS_RESOLVE_SPIN_LIMIT=0 (one
    poll); whether it does depends on timing, and both outcomes are checked.
    With top-K and resolve as one call the copy waves' first wait is for the
    selection, published by the bookkeeper after its select."""
    spec = small("batch32", n_req=8, ctx_range=(8192, 40000), steps=5)
    log(f"[gpu] resolve wait giving up (spin limit 0), then hot reset; fused {fused}")
    wl = W.generate(spec)
    rn = Runner(wl, fused=fused)
    try:
        rn.step()
        monkeypatch.setenv("HS_RESOLVE_SPIN_LIMIT", "0")
        lens = rn.sched[rn.n]
        sc, q = rn.scores.next(lens), rn.queries.next()
        rn.buf.upload(0, sc, q)
        Hn.decode_step(rn.pool, rn.buf, fused=fused)
        torch.cuda.synchronize()
        rn.oracle.step(sc, None, lens, with_attention=False)
        rn.n += 1
        monkeypatch.delenv("HS_RESOLVE_SPIN_LIMIT")
        code = rn.pool.device_error()
        assert code[0] in (0, 5), code
        if code[0] == 5:
            assert code[1] < spec.n_req and code[2] < spec.top_k and code[2] % 4 == 0, code
        log(f"[gpu]   device error after the spin-limited call: {code}")
        rn.pool.clear_device_error()
        for r in range(spec.n_req):
            Hn.set_request(rn.pool, wl, r, int(lens[r]), reset_hot=True)
            rn.oracle.hot[r].reset()
        for _ in range(3):
            rn.step(heads=[0, 77])
    finally:
        rn.close()


FUSED_CASES = [
    ("single-128k", dict(ctx=20000, host_pages=240, steps=6)),
    ("batch32", dict(n_req=7, ctx_range=(4096, 40000), steps=5)),
    ("single-1m-fp8", dict(ctx=30000, host_pages=400, steps=6)),
    ("tiny", dict(steps=4)),
    ("batch32", dict(n_req=3, ctx_range=(600, 1500), steps=3)),  # L < K for every request
]


@pytest.mark.parametrize("name,kw", FUSED_CASES, ids=[f"{c[0]}-{i}" for i, c in enumerate(FUSED_CASES)])
def test_select_resolve_fused(name, kw):
    """hs_select_resolve (top-K and resolve in one launch after the filter)
    gives the same selection, plan, counts and device state as the two
    calls, bit for bit against the oracle, cold and warm steps; bf16, fp8
    and fp32 pools, mixed residency, contexts shorter than K."""
    spec = small(name, **kw)
    log(f"[gpu] select+resolve fused: {name} {kw}")
    wl = W.generate(spec)
    rn = Runner(wl, fused=True)
    try:
        for _ in range(spec.steps):
            rn.step(heads=[0, 5])
    finally:
        rn.close()


def test_select_resolve_fused_bad_request_id():
    spec = small("batch32", n_req=3, ctx_range=(4096, 9000), steps=2)
    wl = W.generate(spec)
    rn = Runner(wl, fused=True)
    try:
        rn.step()
        buf = rn.buf
        bad = torch.tensor([0, 77, 2], dtype=torch.int32, device="cuda")
        buf.idx.fill_(5)
        buf.plan.fill_(5)
        rn.pool.select_resolve(buf.scores[0], bad, buf.idx, buf.plan, buf.counts)
        torch.cuda.synchronize()
        code = rn.pool.device_error()
        assert code[0] == 4 and code[1] == 1 and code[2] == 77, code
        assert (buf.idx[1] == -1).all() and (buf.plan[1] == -1).all() and (buf.counts[1] == 0).all()
    finally:
        rn.close()
