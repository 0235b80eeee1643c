"""GPU parity at the full sizes of every workload, over each workload's whole
schedule, in the launch configuration that bench.py times (the same three
entry points on the same pool layout; bench.py replays them in a hipGraph,
which test_gpu_parity shows to be bit-identical to eager launches).

Every step of every schedule is compared with the CPU oracle: top-K, plan,
counts, slot tags, stamps, reverse map, LRU order, page stamps, host-copy
marks, page table and step counters bit-exact; the pool row behind every
plan entry byte-identical to its logical row (and its fp8 scale). Attention
is compared within 2e-3 of the fp64 oracle on every head at the first step,
at the turn boundaries named below and at the last step, and on a sample of
heads (every query token of every request) at every other step.

Schedules (single-128k and batch32 also with top-K and resolve as one
call, hs_select_resolve):
  single-128k        64 steps
  batch32            32 steps
  single-1m-fp8      128 steps (every score redrawn at each topic-shift step;
                     every head at the first one)
  agent16, agent16-b 715 steps: 13 turns of 55 steps, the context growing
                     from 74,160 to 86,056 tokens (all heads at the first
                     step of turn 2, step 56, and of turn 13, step 661)
  layers16-128k-fp8  32 steps
The oracle runs one single-request oracle per request on a thread pool.
"""
import time

import numpy as np
import pytest

from gpu_helpers import Runner, log
from sparse_mla_decode_indexer_amd import workload as W

pytestmark = pytest.mark.gpu

# (workload, sampled heads, steps with every head checked besides the first and last)
FULL = [
    ("single-128k", [0, 1, 64, 127], [32]),
    ("batch32", [0, 77], [16]),
    ("single-1m-fp8", [5, 100], []),      # plus the first topic-shift step
    ("agent16", [3, 64], [56, 661]),
    ("agent16-b", [3, 64], [56, 661]),
    ("layers16-128k-fp8", [0, 127], []),
]


@pytest.mark.parametrize("name,heads,full_steps", FULL, ids=[f[0] for f in FULL])
def test_full_size_whole_schedule(name, heads, full_steps):
    _whole_schedule(name, heads, full_steps, fused=False)


# hs_select_resolve (top-K and resolve in one call) on the two workloads
# whose steps it is timed on (bench.py --fused)
FUSED = [f for f in FULL if f[0] in ("single-128k", "batch32")]


@pytest.mark.parametrize("name,heads,full_steps", FUSED, ids=[f[0] for f in FUSED])
def test_full_size_whole_schedule_select_resolve(name, heads, full_steps):
    _whole_schedule(name, heads, full_steps, fused=True)


def _whole_schedule(name, heads, full_steps, fused):
    spec = W.SPECS[name]
    steps = spec.steps
    log(f"[gpu] full size {name}{' (select_resolve)' if fused else ''}: all {steps} steps, sampled heads "
        f"{heads}, every head at 1, {full_steps}, {steps}")
    t0 = time.time()
    wl = W.generate(spec)
    rn = Runner(wl, sharded=True, fused=fused)
    if spec.growth is not None:
        rn.incremental = True          # the engine sets only the pages entering the context
    try:
        shifts = rn.scores.planned_shift_steps(steps)
        every = set(full_steps) | {1, steps} | set(shifts[:1])
        counts = np.zeros(3, dtype=np.int64)
        lens_seen = set()
        for n in range(1, steps + 1):
            all_heads = n in every
            ref = rn.step(heads=None if all_heads else heads)
            if n in shifts:
                log(f"[gpu]   {name} step {n}: topic shift (every score redrawn), counts "
                    f"{np.asarray(ref['counts']).sum(axis=0).tolist()}")
            counts += np.asarray(ref["counts"]).sum(axis=0)
            lens_seen.add(int(rn.cur_len.max()))
            if n % 50 == 0 or all_heads:
                log(f"[gpu]   {name} step {n}/{steps}: context {int(rn.cur_len.max())}, counts so far "
                    f"{counts.tolist()}, max err {rn.max_err:.2e} (element-wise {rn.max_elem_err:.2e}), "
                    f"{time.time() - t0:.0f} s")
        if name == "single-1m-fp8":
            assert shifts and rn.scores.shift_steps == shifts, "planned and drawn topic shifts agree"
        if spec.growth is not None:
            first, later, out, turns = spec.growth
            assert max(lens_seen) == first + (turns - 1) * later + turns * out - spec.q_per_req
            assert len(lens_seen) == steps  # the context grew at every step
        log(f"[gpu] {name}: {steps} steps bit-exact, attention max err {rn.max_err:.2e} "
            f"(element-wise, floor 1e-3 of the row maximum: {rn.max_elem_err:.2e}), {time.time() - t0:.0f} s")
    finally:
        rn.close()
