"""GPU parity of the residency manager (hs_update_residency) against the
oracle's reference, interleaved with decode steps: page tables, released
pool pages, copy and release counts, page stamps and host-copy marks
bit-exact after every call; the rows copied into the host store
byte-identical to the logical rows; and every following decode step (whose
misses now read the copied rows) bit-exact as in test_gpu_parity.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import Runner, log, small
from sparse_mla_decode_indexer_amd import workload as W

pytestmark = pytest.mark.gpu


def _poison_gpu_pages_on_host(rn: Runner):
    """Garbage in the host store for every row of a GPU page: only the
    manager's copies can make those rows readable again."""
    wl, pool = rn.wl, rn.pool
    ps = wl.spec.page_size
    for r in range(wl.spec.n_req):
        pages = np.flatnonzero(wl.gpu_page[r] >= 0)
        tok = (pages[:, None] * ps + np.arange(ps)[None, :]).ravel()
        tok = tok[tok < wl.ctx_final[r]]
        pool.host_store[wl.host_base[r] + tok] = 0xFF
        if pool.host_scales is not None:
            pool.host_scales[wl.host_base[r] + tok] = np.nan


def _update_and_check(rn: Runner, budget, max_copy: int, max_demote: int, tag: str):
    R = rn.spec.n_req
    dev = rn.pool.device
    b = None if budget is None else torch.tensor(budget, dtype=torch.int32, device=dev)
    freed = torch.full((R, max(max_demote, 1)), -7, dtype=torch.int32, device=dev)
    counts = torch.full((R, 2), -7, dtype=torch.int32, device=dev)
    rn.pool.update_residency(rn.buf.req_ids, b, max_copy, max_demote, freed if max_demote else None, counts)
    torch.cuda.synchronize()
    freed, counts = freed.cpu().numpy(), counts.cpu().numpy()
    ps = rn.spec.page_size
    tot = np.zeros(2, dtype=np.int64)
    for r in range(R):
        ref = rn.oracle.update_residency(r, None if budget is None else int(budget[r]), max_copy, max_demote)
        assert counts[r].tolist() == [len(ref["copied"]), len(ref["demoted"])], f"{tag} req {r}: counts"
        if max_demote:
            want = ref["freed"] + [-1] * (max_demote - len(ref["freed"]))
            assert freed[r].tolist() == want, f"{tag} req {r}: released pool pages"
        tot += counts[r]
        # the copied pages' rows (and fp8 scales) now sit in the host store
        for p in ref["copied"]:
            rows = rn.wl.host_base[r] + p * ps + np.arange(ps)
            assert np.array_equal(rn.pool.host_store[rows], rn.raw[rows]), f"{tag} req {r}: host copy of page {p}"
            if rn.pool.host_scales is not None:
                assert np.array_equal(rn.pool.host_scales[rows], rn.wl.scales[rows]), f"{tag}: host scales"
    rn._check_state(tag)
    code = rn.pool.device_error()
    assert code[0] == 0, f"{tag}: device error {code}"
    return tot


def test_manager_under_budget_with_growth_fp8():
    """Agent-like requests (fp8 rows, Q = 4, growing contexts), every page
    resident at the start with no host copy; a 50-page budget forces the
    manager to copy pages to host, then release the coldest ones; later
    misses read those copies."""
    spec = small("agent16", n_req=3, growth=(5000, 300, 40, 2), gpu_token_budget=1 << 20, steps=20)
    wl = W.generate(spec)
    rn = Runner(wl)
    rn.incremental = True
    try:
        _poison_gpu_pages_on_host(rn)
        moved = np.zeros(2, dtype=np.int64)
        for n in range(12):
            rn.step(heads=[0, 77])
            moved += _update_and_check(rn, [50] * spec.n_req, 16, 8, f"step {n + 1}")
            log(f"[gpu] residency step {n + 1}: copied/demoted so far {moved.tolist()}")
        assert moved[0] > 0 and moved[1] > 0
        pt = rn.pool.state_views()["page_table"].cpu().numpy()
        ps = spec.page_size
        for r in range(spec.n_req):
            npg = -(-int(rn.cur_len[r]) // ps)
            assert (pt[r, :npg] >= 0).sum() <= 50, f"req {r} holds more GPU pages than its budget"
    finally:
        rn.close()


@pytest.mark.parametrize("ps,kv,budget", [(4, "fp8", 300), (1024, "bf16", 3)], ids=["page-4-fp8", "page-1024-bf16"])
def test_manager_at_page_size_edges(ps, kv, budget):
    """The manager with pages of 4 tokens (fp8 rows: each copied row carries
    its scale into the host store) and of 1,024 tokens (bf16): every page
    resident at the start without a host copy, a budget below the request's
    pages, so each call copies pages to the host, then releases the coldest
    ones, and later steps miss on them."""
    spec = small("single-128k", ctx=8192, host_pages=0, page_size=ps, kv_dtype=kv, top_k=256,
                 hot_rows=max(512, ps), scores=("ar1_shift", 0.9, 0.5))
    wl = W.generate(spec)
    rn = Runner(wl)
    try:
        _poison_gpu_pages_on_host(rn)
        moved = np.zeros(2, dtype=np.int64)
        for n in range(6):
            rn.step(heads=[0, 77])
            moved += _update_and_check(rn, [budget], 256, 128, f"page {ps} step {n + 1}")
        log(f"[gpu] residency page {ps} {kv}: copied/demoted {moved.tolist()}")
        assert moved[0] > 0 and moved[1] > 0
        rn.step(heads=[0, 77])
    finally:
        rn.close()


def test_manager_shrinking_budget_single_request():
    """One 128k-style request, all pages resident with valid host copies;
    the budget drops in large steps, so one call releases many pages at once
    (the radix threshold over stamps with many ties)."""
    spec = small("single-128k", ctx=16384, host_pages=0)
    wl = W.generate(spec)
    rn = Runner(wl)
    try:
        g = torch.from_numpy(wl.gpu_page[0].astype(np.int32)).to(rn.pool.device)
        rn.pool.set_residency(0, int(wl.ctx0[0]), int(wl.host_base[0]), g, host_copy_valid=True)
        rn.oracle.set_pages(0, 0, wl.gpu_page[0], host_copy_valid=True)
        for n, budget in enumerate([256, 200, 120, 40, 40, 3]):
            rn.step(heads=[0, 64])
            moved = _update_and_check(rn, [budget], 0, 1024, f"budget {budget}")
            log(f"[gpu] budget {budget}: demoted {moved[1]}")
        rn.step(heads=[0, 64])
    finally:
        rn.close()


def test_manager_copy_only_and_no_budget():
    """No budget: the manager only copies (bounded per call), releases
    nothing."""
    spec = small("single-128k", ctx=8192, host_pages=64)
    wl = W.generate(spec)
    rn = Runner(wl)
    try:
        _poison_gpu_pages_on_host(rn)
        for n in range(3):
            rn.step(heads=[3])
            moved = _update_and_check(rn, None, 20, 0, f"copy-only {n + 1}")
            assert moved[1] == 0
    finally:
        rn.close()


def test_manager_call_replayed_from_a_graph():
    """hs_update_residency captured in a hipGraph (a copy-only call of 8
    pages): each replay, between eager decode steps, copies the next pages
    exactly as the oracle's manager does, with every state word and host
    copy checked after it."""
    spec = small("single-128k", ctx=16384, host_pages=192)
    wl = W.generate(spec)
    rn = Runner(wl)
    try:
        _poison_gpu_pages_on_host(rn)
        rn.step(heads=[0, 127])  # (the oracle takes the context length from its steps)
        _update_and_check(rn, None, 8, 0, "eager call")  # loads the kernels outside capture
        dev = rn.pool.device
        counts = torch.zeros((1, 2), dtype=torch.int32, device=dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            rn.pool.update_residency(rn.buf.req_ids, None, 8, 0, None, counts)
        ps = spec.page_size
        for rep in range(3):
            rn.step(heads=[0, 127])
            counts.fill_(-7)
            g.replay()
            torch.cuda.synchronize()
            ref = rn.oracle.update_residency(0, None, 8, 0)
            c = counts.cpu().numpy()[0]
            log(f"[gpu] residency graph replay {rep}: copied {c[0]}")
            assert c.tolist() == [len(ref["copied"]), len(ref["demoted"])], f"replay {rep}: counts"
            for p in ref["copied"]:
                rows = wl.host_base[0] + p * ps + np.arange(ps)
                assert np.array_equal(rn.pool.host_store[rows], rn.raw[rows]), f"replay {rep}: page {p}"
            rn._check_state(f"replay {rep}")
            assert rn.pool.device_error()[0] == 0
        rn.step(heads=[0, 127])  # misses now read the copied rows
    finally:
        rn.close()
