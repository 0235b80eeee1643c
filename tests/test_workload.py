"""The seeded input generator: determinism and the stated structure."""
import dataclasses

import numpy as np
import pytest

from sparse_mla_decode_indexer_amd import workload as W


def small(name, **kw):
    return dataclasses.replace(W.SPECS[name], **kw)


def test_deterministic_bytes():
    a = W.generate(small("single-128k", ctx=4096, host_pages=48))
    b = W.generate(small("single-128k", ctx=4096, host_pages=48))
    assert np.array_equal(a.rows, b.rows)
    sa, sb = W.ScoreStream(a), W.ScoreStream(b)
    for _ in range(3):
        assert np.array_equal(sa.next(a.ctx0), sb.next(b.ctx0))
    assert np.array_equal(W.QueryStream(a).next(), W.QueryStream(b).next())


def test_residency_and_placement_tiny():
    wl = W.generate(W.SPECS["tiny"])
    g = wl.gpu_page[0]
    assert (g[:48] == -1).all() and (g[48:] >= 0).all() and g.size == 64
    ids = np.concatenate([g[g >= 0], wl.hot_pages.ravel()])
    assert np.unique(ids).size == ids.size == wl.num_pool_pages
    assert wl.rows.dtype == np.float32 and wl.rows.shape == (4096, 576)


def test_mod3_states_and_ranges():
    spec = small("batch32", ctx_range=(1000, 5000))
    wl = W.generate(spec)
    for r in range(spec.n_req):
        g = wl.gpu_page[r]
        P = g.size
        if r % 3 == 0:
            assert (g >= 0).all()
        elif r % 3 == 1:
            n_gpu = int(np.ceil(0.25 * P))
            assert (g[P - n_gpu:] >= 0).all() and (g[:P - n_gpu] == -1).all()
        else:
            assert (g == -1).all()
    assert wl.ctx0.min() >= 1000 and wl.ctx0.max() <= 5000


def test_fp8_rows_use_full_range_and_decode_close():
    from oracle import decode_rows
    spec = small("single-1m-fp8", ctx=2048, host_pages=29)
    wl = W.generate(spec)
    codes = wl.rows
    # every row reaches |code| = 448 (scale = amax / 448)
    mags = codes & 0x7F
    assert (mags.max(axis=1) == 0x7E).all()
    x = decode_rows(codes[:4], wl.scales[:4], "fp8")
    assert np.isfinite(x).all()


def test_ar1_stationary_variance():
    spec = small("single-128k", ctx=65536, host_pages=768)
    wl = W.generate(spec)
    ss = W.ScoreStream(wl)
    v = [ss.next(wl.ctx0)[0].var() for _ in range(3)]
    assert all(abs(x - 1 / (1 - 0.81)) < 0.2 for x in v)


def test_agent_schedule():
    sched = W.context_schedule(W.SPECS["agent16"], np.full(16, 74160), 715)
    assert sched[0, 0] == 74160 and sched[54, 0] == 74160 + 54 * 4
    assert sched[55, 0] == 74160 + 220 + 753
    assert sched[-1, 0] == 86056 - 4
    assert W.final_context(W.SPECS["agent16"], np.array([74160]))[0] == 86056


def test_multi_layer_slots_share_contexts():
    """Multi-layer specs: slots are layer-major and the slots of one request
    share its context length; each slot still draws its own rows."""
    spec = small("batch32", n_req=6, layers=3, ctx_range=(3000, 9000), steps=1)
    wl = W.generate(spec)
    per = wl.ctx0.reshape(3, 2)
    assert (per == per[0]).all() and per[0, 0] != per[0, 1]
    a, b = wl.host_base[0], wl.host_base[2]  # request 0 in layers 0 and 1
    assert not np.array_equal(wl.rows[a:a + 64], wl.rows[b:b + 64])
    with pytest.raises(ValueError):
        W.generate(small("batch32", n_req=5, layers=3, ctx_range=(3000, 9000), steps=1))


def test_bf16_encoder_matches_torch():
    """The generator's numpy bf16 rounding equals torch's fp32 -> bf16
    conversion (round to nearest, ties to even) bit for bit, ties included."""
    import torch
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(400_000) * np.exp(3 * rng.standard_normal(400_000))).astype(np.float32)
    u = rng.integers(0, 1 << 16, size=20_000, dtype=np.uint32) << np.uint32(16)
    ties = (u | np.uint32(0x8000)).view(np.float32)          # exactly halfway
    near = (u | np.uint32(0x7FFF)).view(np.float32)
    x = np.concatenate([x, ties, near, np.float32([0.0, -0.0, 3.3895314e38, -1e-45])])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.f32_to_bf16_bits(x), ref)


def test_fp8_encoder_matches_torch():
    """The generator's numpy e4m3fn rounding equals torch's fp32 ->
    float8_e4m3fn conversion on every representable value, every midpoint
    between neighbours (ties to even), their float32 neighbours, the
    subnormal range and random values in [-448, 448]."""
    import torch
    codes = np.arange(0x7F, dtype=np.uint8)
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    mids = ((v[:-1].astype(np.float64) + v[1:]) / 2).astype(np.float32)
    c = np.concatenate([v, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e3))])
    rng = np.random.default_rng(10)
    c = np.concatenate([c, -c, np.float32([-0.0]), rng.uniform(-448, 448, 200_000).astype(np.float32),
                        (rng.standard_normal(100_000) * 0.02).astype(np.float32)])
    y = np.clip(c, -448, 448).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(W._e4m3fn_codes(y), ref)
    x = (rng.standard_normal((64, 576)) * np.exp(rng.standard_normal(64))[:, None]).astype(np.float32)
    codes8, scale = W.f32_rows_to_fp8(x)
    dec = torch.from_numpy(codes8).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.abs(dec).max(axis=1).tolist() == [448.0] * 64   # amax maps to the largest code
    assert np.array_equal(scale, (np.abs(x).max(axis=1) / np.float32(448.0)).astype(np.float32))
