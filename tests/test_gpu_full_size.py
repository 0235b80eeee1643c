"""GPU parity at the full sizes of every workload, in the launch
configuration that bench.py times (the same three entry points on the same
pool layout; bench.py replays them in a hipGraph, which test_gpu_parity
shows to be bit-identical to eager launches).

Each step is compared with the CPU oracle: top-K, plan, counts, slot tags,
stamps, reverse map, LRU order and step counters bit-exact; the pool row
behind every plan entry byte-identical to its logical row; attention on a
sample of heads (every query token of every request) within 2e-3 of the
fp64 oracle. The step counts cover the cold first step, steady state, and
(for the 1M-token fp8 workload) a topic-shift step, where every score is
redrawn.
"""
import numpy as np
import pytest

from gpu_helpers import Runner, log
from sparse_mla_decode_indexer_amd import workload as W

pytestmark = pytest.mark.gpu

# (workload, steps, sampled heads)
FULL = [
    ("single-128k", 12, [0, 1, 64, 127]),
    ("batch32", 3, [0, 77]),
    ("single-1m-fp8", 8, [5, 100]),  # the score stream redraws every score at step 3
    ("agent16", 6, [3, 64]),
    ("agent16-b", 6, [3, 64]),
    ("layers16-128k-fp8", 3, [0, 127]),
]


@pytest.mark.parametrize("name,steps,heads", FULL, ids=[f[0] for f in FULL])
def test_full_size(name, steps, heads):
    spec = W.SPECS[name]
    log(f"[gpu] full size {name}: {steps} steps, heads {heads}")
    wl = W.generate(spec)
    rn = Runner(wl)
    try:
        for n in range(steps):
            ref = rn.step(heads=heads)
            log(f"[gpu]   {name} step {n + 1}: counts {np.asarray(ref['counts']).sum(axis=0).tolist()} "
                f"max err {rn.max_err:.2e}")
        if name == "single-1m-fp8":
            assert 3 in rn.scores.shift_steps
    finally:
        rn.close()
