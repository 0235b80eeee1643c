"""GPU parity of the indexer score entry point (hs_indexer_scores, through
the C ABI) against the CPU oracle (oracle/indexer.py), and of the chain
indexer -> top-K.

Scores are fp32 sums of exact bf16 products on the GPU and exact fp64 in the
oracle: each token's score must lie within 2e-5 * B_t of the oracle, where
B_t = sum_j |w_j| sum_d |q_jd k_td| bounds every term (at most ~200 fp32
roundings of partial sums no larger than B_t). Top-K over the GPU's scores
is compared bit-exactly with the oracle's top-K over the same fp32 scores
(the selection is decided in the kernel's precision).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_helpers import log
from oracle import bf16_decode, indexer_scores, select_topk
from sparse_mla_decode_indexer_amd import workload as W
from sparse_mla_decode_indexer_amd.pool import TieredPool

pytestmark = pytest.mark.gpu
TOL = 2e-5
D = W.INDEXER_DIM


def _pool(R, maxc, top_k=256):
    return TieredPool(page_size=64, num_pool_pages=(2 * top_k // 64) * R + 8, max_requests=R,
                      max_context=maxc, kv_dtype="fp8", top_k=top_k, hot_rows=2 * top_k, max_batch=R,
                      host_rows=maxc, device="cuda")


def _bits_to_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def _setup(pool, inp: W.IndexerInputs, ctx):
    R = inp.n_req
    stride = int(pool.desc.max_context)
    keys = np.zeros((R, stride, D), dtype=np.uint16)
    for r in range(R):
        keys[r, :inp.keys[r].shape[0]] = inp.keys[r]
        pool.set_residency(r, int(ctx[r]), 0, None)
    return _bits_to_bf16(keys).cuda()


def _check(scores_gpu, q, w, keys_bits, L, tokens=None):
    """Oracle scores of `tokens` (default: all of 0..L-1) vs the GPU's."""
    if L == 0:
        return 0.0
    tok = np.arange(L) if tokens is None else tokens
    qd, kd = bf16_decode(q), bf16_decode(keys_bits[tok])
    ref = indexer_scores(qd, w.astype(np.float64), kd, tok.size)
    bound = (np.abs(kd) @ np.abs(qd).T) @ np.abs(w.astype(np.float64))
    err = np.abs(scores_gpu[tok].astype(np.float64) - ref)
    assert np.all(err <= TOL * bound + 1e-30), f"max err/bound {np.max(err / np.maximum(bound, 1e-30)):.3e}"
    return float(np.max(err / np.maximum(bound, 1e-30)))


@pytest.mark.parametrize("H", [16, 32, 48, 64])
def test_indexer_scores_parity_ragged(H):
    maxc = 5000
    ctx = np.array([4999, 1, 300, 0])
    inp = W.IndexerInputs(31 + H, 4, np.full(4, maxc), heads=H)
    pool = _pool(4, maxc)
    try:
        ik = _setup(pool, inp, ctx)
        req = torch.tensor([2, 0, 3, 1], dtype=torch.int32, device="cuda")  # slots out of order
        for step in range(2):
            q, w = inp.next()
            iq = _bits_to_bf16(q).cuda()
            iw = torch.from_numpy(w).cuda()
            out = torch.full((4, maxc + 12), float("nan"), dtype=torch.float32, device="cuda")
            log(f"[indexer] H={H} step {step}: contexts {ctx[[2, 0, 3, 1]].tolist()}")
            pool.indexer_scores(iq, iw, ik, req, out)
            torch.cuda.synchronize()
            o = out.cpu().numpy()
            worst = 0.0
            for i, r in enumerate([2, 0, 3, 1]):
                L = int(ctx[r])
                worst = max(worst, _check(o[i], q[i], w[i], inp.keys[r], L))
                assert np.all(np.isnan(o[i, L:])), "entries past the context were written"
            log(f"[indexer]   max err / bound {worst:.2e}")
        assert pool.device_error()[0] == 0
    finally:
        pool.close()


def test_indexer_bad_request_id_sets_device_error_and_skips_row():
    maxc = 1024
    inp = W.IndexerInputs(5, 2, np.full(2, maxc), heads=16)
    pool = _pool(2, maxc)
    try:
        ik = _setup(pool, inp, np.array([1000, 700]))
        q, w = inp.next()
        out = torch.full((2, maxc), -7.0, dtype=torch.float32, device="cuda")
        req = torch.tensor([1, 9], dtype=torch.int32, device="cuda")  # 9 is not a request slot
        pool.indexer_scores(_bits_to_bf16(q).cuda(), torch.from_numpy(w).cuda(), ik, req, out)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        _check(o[0], q[0], w[0], inp.keys[1], 700)
        assert np.all(o[1] == -7.0)
        err = pool.device_error()
        assert err[0] == 4 and err[1] == 1 and err[2] == 9, err  # HS_DEV_REQUEST_RANGE, position, id
    finally:
        pool.close()


def test_indexer_then_topk_chain():
    """Scores from the indexer kernel feed select_topk; the selection equals
    the oracle's top-K over the same fp32 scores, and agrees with the top-K of
    the exact scores except where they differ by less than the score error."""
    maxc, K = 8192, 256
    ctx = np.array([8192, 3000, 200])
    inp = W.IndexerInputs(77, 3, np.full(3, maxc), heads=64)
    pool = _pool(3, maxc, top_k=K)
    try:
        ik = _setup(pool, inp, ctx)
        req = torch.arange(3, dtype=torch.int32, device="cuda")
        scores = torch.zeros((3, maxc), dtype=torch.float32, device="cuda")
        idx = torch.empty((3, K), dtype=torch.int32, device="cuda")
        for step in range(3):
            q, w = inp.next()
            log(f"[indexer->topk] step {step}")
            pool.indexer_scores(_bits_to_bf16(q).cuda(), torch.from_numpy(w).cuda(), ik, req, scores)
            pool.select_topk(scores, req, idx)
            torch.cuda.synchronize()
            s, ix = scores.cpu().numpy(), idx.cpu().numpy()
            for r in range(3):
                L = int(ctx[r])
                _check(s[r], q[r], w[r], inp.keys[r], L)
                assert np.array_equal(ix[r], select_topk(s[r], L, K)), f"request {r}"
                exact = indexer_scores(bf16_decode(q[r]), w[r].astype(np.float64), bf16_decode(inp.keys[r][:L]), L)
                sel_e = set(select_topk(exact, L, K).tolist()) - {-1}
                sel_g = set(ix[r].tolist()) - {-1}
                if sel_e != sel_g:  # only near-ties at the boundary may differ
                    thr = np.sort(exact)[::-1][min(K, L) - 1]
                    diff = np.array(sorted(sel_e ^ sel_g))
                    assert np.all(np.abs(exact[diff] - thr) <= 1e-4 * np.abs(exact).max()), diff
        assert pool.device_error()[0] == 0
    finally:
        pool.close()


@pytest.mark.parametrize("R,maxc", [(1, 131072), (32, 262144)])
def test_indexer_full_size_sampled(R, maxc):
    """The launch shapes bench.py times (one 128K request; 32 requests up to
    256K), 64 heads, checked on sampled tokens of every request."""
    g = np.random.default_rng(R)
    ctx = np.full(R, maxc) if R == 1 else g.integers(16384, maxc, endpoint=True, size=R)
    inp = W.IndexerInputs(1000 + R, R, ctx, heads=64)
    pool = _pool(R, maxc, top_k=2048)
    try:
        ik = _setup(pool, inp, ctx)
        req = torch.arange(R, dtype=torch.int32, device="cuda")
        q, w = inp.next()
        out = torch.zeros((R, maxc), dtype=torch.float32, device="cuda")
        log(f"[indexer full] R={R} max context {maxc}")
        pool.indexer_scores(_bits_to_bf16(q).cuda(), torch.from_numpy(w).cuda(), ik, req, out)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        worst = 0.0
        for r in range(R):
            L = int(ctx[r])
            tok = np.unique(np.concatenate([g.integers(0, L, size=512), np.arange(max(0, L - 300), L),
                                            np.arange(min(L, 300))]))
            worst = max(worst, _check(o[r], q[r], w[r], inp.keys[r], L, tok))
        log(f"[indexer full]   max err / bound {worst:.2e}")
        assert pool.device_error()[0] == 0
    finally:
        pool.close()


def test_indexer_scores_graph_replay_matches_eager():
    """hs_indexer_scores captured in a hipGraph: every replay (with eager work
    and synchronisations between replays) equals the eager result bit for bit."""
    maxc = 4096
    ctx = np.array([4096, 1000])
    inp = W.IndexerInputs(404, 2, np.full(2, maxc), heads=32)
    pool = _pool(2, maxc)
    try:
        ik = _setup(pool, inp, ctx)
        req = torch.arange(2, dtype=torch.int32, device="cuda")
        q, w = inp.next()
        iq, iw = _bits_to_bf16(q).cuda(), torch.from_numpy(w).cuda()
        eager = torch.zeros((2, maxc), dtype=torch.float32, device="cuda")
        pool.indexer_scores(iq, iw, ik, req, eager)
        torch.cuda.synchronize()
        out = torch.zeros_like(eager)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            pool.indexer_scores(iq, iw, ik, req, out)  # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            pool.indexer_scores(iq, iw, ik, req, out)
        for rep in range(3):
            out.fill_(-1.0)
            _ = (eager * 2.0).sum().item()  # eager work between replays
            g.replay()
            torch.cuda.synchronize()
            log(f"[indexer graph] replay {rep}")
            assert torch.equal(out[0], eager[0]) and torch.equal(out[1, :1000], eager[1, :1000]), rep
            assert torch.all(out[1, 1000:] == -1.0)
        _check(eager.cpu().numpy()[1], q[1], w[1], inp.keys[1], 1000)
    finally:
        pool.close()
