"""Benchmark: tiered sparse-MLA decode steps on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload batch32]

The default workload is the largest one that fits one GPU: 32 concurrent
requests with contexts uniform in [16K, 256K] tokens (bf16 latent rows,
128 heads, top-K 2048, hot buffer 4096 rows, a third of the requests fully
resident, a third with the newest quarter of their pages on the GPU, a third
host-only), 28 timed + 4 warm-up steps = its 32 decode steps.

Growing-context workloads (agent16, agent16-b) are timed with every
request at its first step's context length.

A step is the whole hot path for every request of the workload: top-K over
the indexer scores -> fused resolve (resident / hot / miss copy over PCIe)
-> sparse MLA attention over the K resolved rows. Inputs (scores and
queries of every step) are resident in HBM before timing; the K timed
steps are one hipGraph replay, bracketed by HIP events on the replay
stream. Prints one JSON line.

Roofline: the same K steps are replayed again from a snapshot of the
pool state, with HIP events (on the stream the kernels run on) around each
of the three entry points (a spin kernel first lets the host queue run
ahead, so the events see GPU time only). The entry point with the largest
average duration is reported against its bound (PCIe for the miss copy,
HBM for the scans and gathers, MFMA for attention when its FLOP per
algorithmic byte is above the bf16 ridge, as with fp8 rows or four query
tokens per request) with its algorithmic bytes (or FLOPs) per launch;
`traffic` is the HBM bytes per launch its kernels actually moved, from the
committed counter summary profiles/decode_step_<workload>_hbm_traffic.json
(null when absent or taken on other kernel sources).

Measured denominators: before it touches the GPU, bench.py runs the probes
of libhsprobe in a child process (python -m sparse_mla_decode_indexer_amd.probe):
zero-copy coalesced reads of 512 MiB of pinned host memory (the PCIe
host-read rate the miss copy is priced against beside the published link
rate), a device copy and read (HBM), and a bf16 MFMA loop. A failure there
leaves `measured_peaks` null and the published peaks in use.

cpu_baseline: the CPU oracle (tests' reference, fp64 numpy) timed on a
bounded prefix of the same steps on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np
import faulthandler

ROOT = os.path.dirname(os.path.abspath(__file__))
faulthandler.enable(all_threads=True)  # a host crash prints every thread's Python stack
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
PCIE_PEAK_GBS = 64.0         # PCIe 5.0 x16, one direction, published
MFMA_BF16_PEAK_TFS = 2500.0  # dense bf16


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=28)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--workload", default="batch32")
    ap.add_argument("--no-probe", action="store_true", help="skip the measured-denominator probes")
    ap.add_argument("--group", type=int, default=-1,
                    help="requests per group of the pipelined step (harness.PipelinedStep); -1, the "
                         "default: the three entry points in sequence on one stream")
    ap.add_argument("--fused", action="store_true",
                    help="top-K and resolve as one call (hs_select_resolve) in the timed step")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget for the CPU oracle baseline (0 = skip)")
    ap.add_argument("--no-roofline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times (the "
                         "reference kernel that scales the HBM byte counters) and exit")
    return ap.parse_args()


def copy_probe(mib: int):
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 5}))


def run_probes(timeout_s: int = 180):
    """Measured denominators from libhsprobe, run in a child process (see the
    module docstring). Returns the probe's JSON object, or None on failure."""
    cmd = [sys.executable, "-u", "-m", "sparse_mla_decode_indexer_amd.probe"]
    print("[bench] probes: PCIe host read, HBM copy/read, bf16 MFMA", file=sys.stderr, flush=True)
    try:
        r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=timeout_s)
    except subprocess.TimeoutExpired:
        print("[bench] probes timed out; published peaks only", file=sys.stderr, flush=True)
        return None
    if r.returncode != 0:
        print(f"[bench] probes failed (rc {r.returncode}); published peaks only\n{r.stderr[-2000:]}",
              file=sys.stderr, flush=True)
        return None
    for line in reversed(r.stdout.splitlines()):
        if line.startswith("{"):
            return json.loads(line)
    return None


def main():
    args = parse()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); requests are independent "
              "and shard by request with no exchange, so a multi-GPU figure is not measured here.",
              file=sys.stderr)
        sys.exit(2)
    probes = None if args.no_probe else run_probes()
    pcie_meas = probes["pcie_host_read_gbs"] if probes else None
    import torch

    from sparse_mla_decode_indexer_amd import harness as Hn
    from sparse_mla_decode_indexer_amd import workload as W

    spec = W.SPECS[args.workload]
    K, Wm = args.steps, args.warmup
    T = K + Wm
    wl = W.generate(spec)
    if spec.growth is not None and T > spec.steps:
        raise SystemExit(f"{spec.name} defines {spec.steps} steps")
    # Growing (agent) workloads are timed at their first step's context: the
    # growth between steps is the engine writing new rows, outside the step,
    # so every timed step sees the turn-1 length (the parity tests follow
    # the full growing schedule).
    sched = np.broadcast_to(wl.ctx0, (T, spec.n_req))
    dev = "cuda"
    torch.cuda.set_device(0)
    pool = Hn.make_pool(wl, device=dev)
    Hn.load_workload(pool, wl)
    buf = Hn.StepBuffers(wl, device=dev, n_steps=T)
    group = args.group
    fused = args.fused and not spec.select_k
    if group > 0 and group < spec.n_req and not fused:
        step_fn = Hn.PipelinedStep(pool, buf, group)
    else:
        group = -1

        def step_fn(n):
            Hn.decode_step(pool, buf, n, fused=fused)
    ss, qs = W.ScoreStream(wl), W.QueryStream(wl)
    host_scores, host_q = [], []
    for n in range(T):
        sc = ss.next_tokens(sched[n]) if spec.select_k else ss.next(sched[n])
        q = qs.next()
        buf.upload(n, sc, q)
        if n < 64 and sc.nbytes * (n + 1) < (1 << 30):
            host_scores.append(sc)
            host_q.append(q)
    torch.cuda.synchronize()
    print(f"[bench] {spec.name}: inputs resident, {T} steps", file=sys.stderr, flush=True)

    # warmup: W eager steps. The cold step (empty hot buffers, top-K bound not
    # yet set) is step 0 from the freshly loaded state, timed per entry point
    # after every kernel has run once (so that no first-launch code loading
    # is timed): snapshot, warm-up step, restore, timed step, warm-up.
    cold = None
    if not args.no_roofline and Wm > 0:
        s_state, s_rows = pool.state.clone(), pool.pool_rows.clone()
        s_scales = None if pool.pool_scales is None else pool.pool_scales.clone()
        Hn.decode_step(pool, buf, 0)
        torch.cuda.synchronize()
        pool.state.copy_(s_state)
        pool.pool_rows.copy_(s_rows)
        if s_scales is not None:
            pool.pool_scales.copy_(s_scales)
        del s_state, s_rows, s_scales
        cold = timed_entry_points(pool, buf, [0])
        cold["misses"] = int(buf.counts[:, 2].sum().item())
    for n in range(1 if cold is not None else 0, Wm):
        step_fn(n)
    torch.cuda.synchronize()

    # capture the K timed steps
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for n in range(Wm, T):
            step_fn(n)
    torch.cuda.synchronize()
    snap_state = pool.state.clone()
    snap_rows = pool.pool_rows.clone()
    snap_scales = None if pool.pool_scales is None else pool.pool_scales.clone()
    views = pool.state_views()
    c0 = views["counters"].clone()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    ms_per_step = ms / K
    dc = (views["counters"] - c0).cpu().numpy().sum(axis=0)  # resident, hot, miss over K steps
    code = pool.device_error()
    if code[0] != 0:
        raise SystemExit(f"device error {code}")
    print(f"[bench] timed {K} steps: {ms:.3f} ms", file=sys.stderr, flush=True)

    R, Kt, S = spec.n_req, spec.top_k, spec.hot_rows
    rb = W.row_bytes(spec.kv_dtype) + (4 if spec.kv_dtype == "fp8" else 0)
    lens = np.asarray(wl.ctx0, dtype=np.int64)
    misses_per_step = dc[2] / K
    qb = 4 if spec.q_dtype == "f32" else 2
    QH = spec.q_per_req * spec.heads
    # algorithmic bytes of one step (what the method must move)
    if spec.select_k:  # a top-K per query token, one resolve of the union
        Qn, kt = spec.q_per_req, spec.select_k
        rows_per_step = int(dc.sum() / K)  # union rows resolved per step
        b_topk = 4 * Qn * lens.sum() + 4 * R * Qn * kt + 8 * R * Qn * kt + 4 * R * Kt
        b_resolve_hbm = R * 8 * S + 12 * rows_per_step + misses_per_step * rb
        attn_rows = Qn * int(np.minimum(kt, lens).sum())  # each token reads its own rows
        b_attn = attn_rows * rb + R * QH * (576 * qb + 512 * 4 + 4) + 8 * R * Qn * kt
        flops_attn = 2.0 * spec.heads * attn_rows * (576 + 512)
    else:
        rows_per_step = int(np.minimum(Kt, lens).sum())
        b_topk = 4 * lens.sum() + 4 * R * Kt
        b_resolve_hbm = R * (12 * Kt + 8 * S) + misses_per_step * rb
        b_attn = rows_per_step * rb + R * QH * (576 * qb + 512 * 4 + 4) + 4 * R * Kt
        flops_attn = 2.0 * QH * rows_per_step * (576 + 512)
    b_pcie = misses_per_step * rb

    roof = None
    if not args.no_roofline:
        pool.state.copy_(snap_state)
        pool.pool_rows.copy_(snap_rows)
        if snap_scales is not None:
            pool.pool_scales.copy_(snap_scales)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
        torch.cuda._sleep(int(2e8))  # let the host queue run ahead of the GPU
        for j, n in enumerate(range(Wm, T)):
            ev = evs[j]
            for a, call in enumerate(entry_calls(pool, buf, n)):
                ev[a].record(stream)
                call()
            ev[3].record(stream)
        torch.cuda.synchronize()
        dur = np.array([[ev[a].elapsed_time(ev[a + 1]) for a in range(3)] for ev in evs])  # ms
        avg = dur.mean(axis=0) * 1e3  # us
        names = ["select_topk", "resolve_rows", "sparse_mla_decode"]
        # attention is a bf16 MFMA contraction (fp8 rows are widened to
        # bf16): priced against MFMA when its FLOP per algorithmic byte is
        # above the ridge, else against HBM
        attn_mfma = flops_attn / b_attn > MFMA_BF16_PEAK_TFS * 1e3 / HBM_PEAK_GBS
        per = {
            "select_topk": dict(bound="hbm", bytes=b_topk, peak=HBM_PEAK_GBS, unit="GB/s"),
            "resolve_rows": dict(bound="pcie", bytes=b_pcie, peak=PCIE_PEAK_GBS, unit="GB/s"),
            "sparse_mla_decode": dict(bound="mfma", flops=flops_attn, peak=MFMA_BF16_PEAK_TFS,
                                      unit="TFLOP/s", bytes=b_attn) if attn_mfma else
                                 dict(bound="hbm", bytes=b_attn, peak=HBM_PEAK_GBS, unit="GB/s"),
        }
        dom = int(np.argmax(avg))
        name = names[dom]
        d = per[name]
        if d["bound"] == "mfma":
            achieved = d["flops"] / (avg[dom] * 1e-6) / 1e12
        else:
            achieved = d["bytes"] / (avg[dom] * 1e-6) / 1e9
        meas = None
        if probes:
            meas = {"pcie": probes["pcie_host_read_gbs"], "hbm": probes["hbm_read_gbs"],
                    "mfma": probes["mfma_bf16_tflops"]}[d["bound"]]
        roof = {"kernel": name, "kernels": ENTRY_KERNELS[name], "bound": d["bound"],
                "achieved": round(achieved, 2), "peak": d["peak"], "unit": d["unit"],
                "frac": round(achieved / d["peak"], 4),
                "measured_peak": meas,
                "frac_of_measured": round(achieved / meas, 4) if meas else None,
                "traffic": measured_traffic(spec.name, ENTRY_KERNELS[name]),
                "avg_us": {n: round(float(a), 2) for n, a in zip(names, avg)},
                "bytes_per_launch": {n: int(per[n]["bytes"]) for n in names},
                "attention_tflops": round(flops_attn / (avg[2] * 1e-6) / 1e12, 2),
                "attention_mfma_frac": round(flops_attn / (avg[2] * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFS, 4)}

    # hit-only replay: the last step's inputs again, after that step filled the
    # hot buffers, so every selected row is resident or hot (no PCIe)
    hit = None
    if not args.no_roofline:
        hit = timed_entry_points(pool, buf, [T - 1] * 8)
        hit["misses"] = int(buf.counts[:, 2].sum().item())
        step_us = sum(hit["avg_us"].values())
        hit["step_us"] = round(step_us, 2)
        hbm_no_miss = b_topk + R * (12 * Kt + 8 * S) + b_attn
        hit["hbm_bytes_per_step"] = int(hbm_no_miss)
        hit["hbm_frac"] = round(hbm_no_miss / (step_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 5)
    if cold is not None:
        mb = cold["misses"] * rb
        cold["pcie_bytes"] = int(mb)
        cold["resolve_pcie_gbs"] = round(mb / (cold["avg_us"]["resolve_rows"] * 1e-6) / 1e9, 2)
        cold["resolve_pcie_frac"] = round(cold["resolve_pcie_gbs"] / PCIE_PEAK_GBS, 4)
        if pcie_meas:
            cold["resolve_pcie_frac_of_measured"] = round(cold["resolve_pcie_gbs"] / pcie_meas, 4)
    if roof is not None:
        # the HBM target is read on the hit-only replay, the PCIe target on
        # the steps with misses (timed steps and the cold step)
        roof["hit_only_hbm_frac"] = hit["hbm_frac"] if hit else None
        miss_gbs = b_pcie / (avg[1] * 1e-6) / 1e9 if b_pcie > 0 else None
        roof["miss_pcie_gbs"] = round(miss_gbs, 2) if miss_gbs else None
        roof["miss_pcie_frac_of_measured"] = round(miss_gbs / pcie_meas, 4) if (miss_gbs and pcie_meas) else None
        roof["cold_pcie_frac_of_measured"] = cold.get("resolve_pcie_frac_of_measured") if cold else None

    resid = None if args.no_roofline else residency_probe(pool, buf, spec)
    indexer = None if args.no_roofline else indexer_probe(pool, buf, spec, wl)

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(wl, host_scores, host_q, sched, args.cpu_seconds)

    step_hbm = b_topk + b_resolve_hbm + b_attn
    value = 1e3 / ms_per_step
    # roofline of the whole step: the slowest of its three resources at the
    # published HBM and MFMA peaks and the measured PCIe host-read rate
    pcie_den = pcie_meas or PCIE_PEAK_GBS
    t_roof = max(step_hbm / (HBM_PEAK_GBS * 1e9), b_pcie / (pcie_den * 1e9),
                 flops_attn / (MFMA_BF16_PEAK_TFS * 1e12))
    step_roof = {"t_roof_us": round(t_roof * 1e6, 2), "t_step_us": round(ms_per_step * 1e3, 2),
                 "frac": round(t_roof / (ms_per_step * 1e-3), 4),
                 "pcie_denominator": "measured host read" if pcie_meas else "published link rate",
                 "bound": ["hbm", "pcie", "mfma"][int(np.argmax([step_hbm / (HBM_PEAK_GBS * 1e9),
                                                                 b_pcie / (pcie_den * 1e9),
                                                                 flops_attn / (MFMA_BF16_PEAK_TFS * 1e12)]))]}
    line = {
        "metric": "sparse-MLA decode steps/s + top-K rows resolved/s; % of HBM/PCIe roofline",
        "value": round(value, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8e4m3+bf16"}[spec.kv_dtype],
        "data": "synthetic",
        "config": {"workload": spec.name, "requests": R, "context": int(lens.max()),
                   "kv_dtype": spec.kv_dtype, "heads": spec.heads, "q_per_req": spec.q_per_req,
                   "top_k": Kt, "hot_rows": S, "residency": spec.residency,
                   "step": (f"pipelined over groups of {group} requests on three streams"
                            if group > 0 else
                            "select_resolve then sparse_mla_decode on one stream" if fused else
                            "three entry points in sequence on one stream"),
                   **({"growth": "context frozen at the first step's length"}
                      if spec.growth is not None else {}),
                   **({"layers": spec.layers} if spec.layers > 1 else {}),
                   **({"top_k_per_query_token": spec.select_k, "union_capacity": spec.top_k}
                      if spec.select_k else {})},
        **({"layer_steps_per_s": round(value * spec.layers, 1)} if spec.layers > 1 else {}),
        "rows_resolved_per_s": round(rows_per_step * value, 1),
        "misses_per_step": round(float(misses_per_step), 1),
        "hits_per_step": round(float(dc[1] / K), 1),
        "resident_per_step": round(float(dc[0] / K), 1),
        "step_hbm_frac": round(step_hbm / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 5),
        "step_pcie_frac": round(b_pcie / (ms_per_step * 1e-3) / 1e9 / PCIE_PEAK_GBS, 4),
        "step_pcie_frac_of_measured": (round(b_pcie / (ms_per_step * 1e-3) / 1e9 / pcie_meas, 4)
                                       if pcie_meas else None),
        "step_roofline": step_roof,
        "roofline": roof,
        "measured_peaks": probes,
        "cpu_baseline": cpu,
        "cold_step": cold,
        "hit_only_replay": hit,
        "residency_manager": resid,
        "indexer": indexer,
    }
    pool.close()
    print(json.dumps(line))


# HIP kernels behind each entry point (name prefixes as the profiler lists them)
ENTRY_KERNELS = {
    "select_topk": ["k_topk_filter", "k_topk_select", "k_topk_union"],
    "resolve_rows": ["k_resolve"],
    "sparse_mla_decode": ["k_attn_mfma", "k_attn_combine"],
}


# Sources the decode-step kernels (top-K, resolve, attention) are built from:
# the counters recorded for them stay valid while these files are unchanged.
STEP_SOURCES = ["sparse_mla_decode_indexer_amd/csrc/topk.hip", "sparse_mla_decode_indexer_amd/csrc/topk_select.h", "sparse_mla_decode_indexer_amd/csrc/resolve.hip",
                "sparse_mla_decode_indexer_amd/csrc/attention.hip", "sparse_mla_decode_indexer_amd/csrc/hs_internal.h",
                "include/hisparse.h"]


def source_sha256() -> str:
    """Hash of the decode-step kernel sources, as recorded with the HBM byte counters."""
    import hashlib
    src = sorted(os.path.join(ROOT, p) for p in STEP_SOURCES)
    h = hashlib.sha256()
    for p in src:
        h.update(os.path.relpath(p, ROOT).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernels):
    """HBM bytes per launch of an entry point from the committed counter
    summary (FETCH_SIZE / WRITE_SIZE scaled by a plain copy), or None when
    there is none for this workload or the kernel sources have changed since
    the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"decode_step_{workload}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256") != source_sha256():
        return None
    total = 0
    for name, k in t["kernels"].items():
        if any(name.startswith(p) for p in kernels):
            total += int(k["hbm_bytes"])
    return total or None


def entry_calls(pool, buf, n):
    """The step's three entry points as calls for step n (top-K, resolve,
    attention; the union forms for a speculative step with a selection per
    query token)."""
    if buf.union:
        return [lambda: pool.select_topk_union(buf.scores[n], buf.req_ids, buf.sel, buf.idx, buf.upos),
                lambda: pool.resolve_rows(buf.idx, buf.req_ids, buf.plan, buf.counts),
                lambda: pool.sparse_mla_decode_union(buf.q[n], buf.plan, buf.upos, buf.sm_scale, buf.out, buf.lse)]
    return [lambda: pool.select_topk(buf.scores[n], buf.req_ids, buf.idx),
            lambda: pool.resolve_rows(buf.idx, buf.req_ids, buf.plan, buf.counts),
            lambda: pool.sparse_mla_decode(buf.q[n], buf.plan, buf.sm_scale, buf.out, buf.lse)]


def timed_entry_points(pool, buf, steps):
    """Run the given steps eagerly with HIP events around each entry point
    (a spin kernel first lets the host queue run ahead). Returns the average
    duration of each entry point in us."""
    import torch
    stream = torch.cuda.current_stream()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in steps]
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2e8))
    for j, n in enumerate(steps):
        ev = evs[j]
        for a, call in enumerate(entry_calls(pool, buf, n)):
            ev[a].record(stream)
            call()
        ev[3].record(stream)
    torch.cuda.synchronize()
    dur = np.array([[ev[a].elapsed_time(ev[a + 1]) for a in range(3)] for ev in evs]) * 1e3
    names = ["select_topk", "resolve_rows", "sparse_mla_decode"]
    return {"steps": len(steps), "avg_us": {k: round(float(v), 2) for k, v in zip(names, dur.mean(axis=0))}}


def residency_probe(pool, buf, spec, pages_per_call: int = 64, calls: int = 4):
    """Residency manager on the benchmark's pool after the timed steps (not
    part of a decode step): `calls` proactive-copy calls of `pages_per_call`
    complete GPU pages each into the pinned host store (PCIe device-to-host
    writes), enqueued back to back, then one release call under a budget of
    half the GPU pages. HIP events on the stream the kernels run on; a spin
    kernel (~0.1 s) is enqueued first so that the host has queued every
    launch of the calls before the first event is reached and the events
    time GPU work only."""
    import torch
    R = spec.n_req
    dev = buf.req_ids.device
    stream = torch.cuda.current_stream()

    def timed(fn):
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2e8))  # keeps the GPU busy while the host enqueues fn's launches
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    cnts = [torch.zeros(R, 2, dtype=torch.int32, device=dev) for _ in range(calls)]

    def copies():
        for c in cnts:
            pool.update_residency(buf.req_ids, None, pages_per_call, 0, None, c)

    copy_ms = timed(copies)
    copied = int(sum(int(c[:, 0].sum().item()) for c in cnts))
    pt = pool.state_views()["page_table"]
    held = int((pt[:R] >= 0).sum().item())
    budget = torch.full((R,), max(held // (2 * R), 0), dtype=torch.int32, device=dev)
    freed = torch.empty(R, 1024, dtype=torch.int32, device=dev)
    counts = torch.zeros(R, 2, dtype=torch.int32, device=dev)
    rel_ms = timed(lambda: pool.update_residency(buf.req_ids, budget, 0, 1024, freed, counts))
    released = int(counts[:, 1].sum().item())
    row_bytes = pool.row_bytes + (4 if spec.kv_dtype == "fp8" else 0)
    copied_bytes = copied * spec.page_size * row_bytes
    gbs = copied_bytes / (copy_ms * 1e-3) / 1e9 if copied else 0.0
    return {"calls": calls, "copied_pages": copied, "copied_bytes": copied_bytes,
            "copy_call_us": round(copy_ms * 1e3 / calls, 2), "copy_gbs": round(gbs, 2),
            "pcie_peak_gbs": PCIE_PEAK_GBS, "copy_frac": round(gbs / PCIE_PEAK_GBS, 4),
            "release_call_us": round(rel_ms * 1e3, 2), "released_pages": released}


def indexer_probe(pool, buf, spec, wl, heads: int = 64, calls: int = 20):
    """Indexer scores (upstream of the step, which starts from scores) for
    every request of the workload at its context length: 64 heads, bf16
    queries and 128-dim bf16 indexer keys drawn on the device from a seeded
    generator, fp32 head weights. HIP events around `calls` back-to-back
    launches on the stream the kernel runs on (a spin kernel first lets the
    host queue run ahead); priced against HBM by the bytes the formula must
    read and write (keys 256 B per token, queries and weights, fp32 scores)."""
    import torch
    R = spec.n_req
    dev = buf.req_ids.device
    g = torch.Generator(device=dev).manual_seed(spec.seed)
    maxc = int(wl.max_context)
    ik = torch.empty((R, maxc, 128), dtype=torch.bfloat16, device=dev)
    for r in range(R):  # one request at a time (bounded fp32 temporary)
        ik[r] = torch.randn((maxc, 128), generator=g, device=dev).to(torch.bfloat16)
    iq = torch.randn((R, heads, 128), generator=g, device=dev).to(torch.bfloat16)
    iw = torch.randn((R, heads), generator=g, device=dev) / heads ** 0.5
    out = torch.empty((R, buf.scores.shape[-1]), dtype=torch.float32, device=dev)
    for _ in range(2):
        pool.indexer_scores(iq, iw, ik, buf.req_ids, out)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(2e8))
    e0.record(stream)
    for _ in range(calls):
        pool.indexer_scores(iq, iw, ik, buf.req_ids, out)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / calls
    tokens = int(np.asarray(wl.ctx0, dtype=np.int64).sum())
    nbytes = tokens * (128 * 2 + 4) + R * heads * (128 * 2 + 4)
    gbs = nbytes / (us * 1e-6) / 1e9
    del ik
    return {"calls": calls, "heads": heads, "tokens_per_call": tokens, "avg_us": round(us, 2),
            "bytes_per_call": nbytes, "gbs": round(gbs, 1), "hbm_peak_gbs": HBM_PEAK_GBS,
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def cpu_baseline(wl, host_scores, host_q, sched, budget_s):
    """Time the CPU oracle (full step: top-K, LRU, fp64 attention) on the
    first steps of the same inputs until the budget is spent."""
    from oracle import DecodeOracle, bf16_decode

    s = wl.spec
    orc = DecodeOracle(rows=wl.rows, scales=wl.scales, kv_dtype=s.kv_dtype, host_base=wl.host_base,
                       gpu_page=wl.gpu_page, hot_pages=wl.hot_pages, page_size=s.page_size,
                       top_k=s.top_k, hot_rows=s.hot_rows, ctx_capacity=wl.ctx_final,
                       sm_scale=wl.sm_scale)
    t0 = time.perf_counter()
    n = 0
    m = len(host_scores)
    while time.perf_counter() - t0 < budget_s:  # cycles through the stored steps
        j = n % m
        q = host_q[j]
        qd = bf16_decode(q) if q.dtype == np.uint16 else q.astype(np.float64)
        if s.select_k:
            orc.step_union(host_scores[j], qd, sched[j], s.select_k, with_attention=True)
        else:
            orc.step(host_scores[j], qd, sched[j], with_attention=True)
        n += 1
    el = time.perf_counter() - t0
    try:  # the BLAS threads numpy actually runs with
        from threadpoolctl import threadpool_info
        cores = max([int(x["num_threads"]) for x in threadpool_info() if x.get("user_api") == "blas"] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    return {"value": round(n / el, 3), "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} decode steps of {s.name} (its first {min(n, m)} score/query sets, "
                      f"repeated; top-K sort, LRU simulation, fp64 attention over all heads), "
                      f"numpy with {cores} BLAS threads, {el:.1f} s",
            "seconds": round(el, 2)}


if __name__ == "__main__":
    main()
