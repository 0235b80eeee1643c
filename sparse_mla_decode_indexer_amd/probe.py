"""ctypes binding of libhsprobe.so and the measured roofline denominators.

    python -m sparse_mla_decode_indexer_amd.probe      # prints one JSON object

Measures on the GPU at hand, with HIP events on the stream the probe
kernels run on:
  * PCIe host read: zero-copy coalesced reads of a 512 MiB pinned, mapped
    host buffer (the kind of memory the pool's host store is), best of a
    few grid sizes; and reads of random rows as the miss copy makes them:
    1,152-byte bf16 rows, and the 592 bytes of an fp8 row (576 code bytes
    and the row scale, in 16-byte chunks) at the fp8 host row stride of 640
    bytes (rows on 128-byte boundaries) and, for comparison, packed at a
    592-byte stride;
  * HBM: a plain device copy (bytes read + written) and a plain device read;
  * MFMA: independent chains of the bf16 16x16x32 MFMA the attention kernel
    uses, counted at 16,384 FLOP each.
bench.py runs this as a child process before it touches the GPU itself, so
that a failure here costs only the measured denominators.
"""
from __future__ import annotations

import ctypes
import json
import os
import sys
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libhsprobe.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "hsprobe.h")

_VP, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "hsp_alloc_pinned": [_SZ, ctypes.POINTER(_VP)],
    "hsp_free_pinned": [_VP],
    "hsp_host_read": [_VP, _SZ, _I32, _VP, _VP],
    "hsp_host_gather": [_VP, _I64, _I64, _I64, _VP, _I32, _VP, _VP],
    "hsp_device_copy": [_VP, _VP, _SZ, _I32, _VP],
    "hsp_device_read": [_VP, _SZ, _I32, _VP, _VP],
    "hsp_mfma_bf16": [_I32, _I32, _I32, _I32, _VP, _VP],
}
_lib: Optional[ctypes.CDLL] = None


def header_functions():
    import re
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^int32_t\s+(hsp_\w+)\(", text, re.M)))


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_mla_decode_indexer_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int32
        _lib = L
    return _lib


def _ok(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what}: hipError {rc}")


def measure(host_mib: int = 512, copy_mib: int = 1024, reps: int = 5) -> dict:
    import numpy as np
    import torch

    torch.cuda.set_device(0)
    L = lib()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    sink = torch.zeros(65536, dtype=torch.int32, device="cuda")

    def timed(fn, n=reps):
        fn()
        fn()  # warm-up
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e-3  # s per call

    out = {}
    # ---- PCIe host read
    nbytes = host_mib << 20
    hp = _VP()
    _ok(L.hsp_alloc_pinned(nbytes, ctypes.byref(hp)), "hsp_alloc_pinned")
    try:
        grids = {}
        for blocks in (512, 1024, 2048, 4096):
            t = timed(lambda: _ok(L.hsp_host_read(hp, nbytes, blocks, sink.data_ptr(), sp), "hsp_host_read"))
            grids[blocks] = round(nbytes / t / 1e9, 2)
        best = max(grids.values())
        out["pcie_host_read_gbs"] = best
        out["pcie_host_read"] = {"bytes": nbytes, "gbs_by_grid": grids, "kind": "zero-copy coalesced 16-B loads"}
        rng = np.random.default_rng(1)
        gathers = {}
        for rb, stride, key in ((1152, 1152, "1152"), (592, 640, "592"), (592, 592, "592_packed")):
            n_src = nbytes // stride
            n = 65536
            rows = torch.from_numpy(rng.integers(0, n_src, size=n).astype(np.int64)).cuda()
            dst = torch.empty(n * rb, dtype=torch.uint8, device="cuda")
            t = timed(lambda: _ok(L.hsp_host_gather(hp, n_src, rb, stride, rows.data_ptr(), n, dst.data_ptr(), sp),
                                  "hsp_host_gather"))
            gathers[key] = round(n * rb / t / 1e9, 2)
            del dst
        out["pcie_row_gather_gbs"] = gathers
    finally:
        torch.cuda.synchronize()
        L.hsp_free_pinned(hp)
    # ---- HBM
    cb = copy_mib << 20
    a = torch.empty(cb, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    copy = {}
    for blocks in (2048, 4096, 8192):
        t = timed(lambda: _ok(L.hsp_device_copy(a.data_ptr(), b.data_ptr(), cb, blocks, sp), "hsp_device_copy"))
        copy[blocks] = round(2 * cb / t / 1e9, 1)
    read = {}
    for blocks in (2048, 4096, 8192):
        t = timed(lambda: _ok(L.hsp_device_read(a.data_ptr(), cb, blocks, sink.data_ptr(), sp), "hsp_device_read"))
        read[blocks] = round(cb / t / 1e9, 1)
    del a, b
    out["hbm_copy_gbs"] = max(copy.values())
    out["hbm_read_gbs"] = max(read.values())
    out["hbm"] = {"copy_bytes": cb, "copy_gbs_by_grid": copy, "read_gbs_by_grid": read,
                  "copy_counts": "bytes read + bytes written"}
    # ---- MFMA bf16
    mf = {}
    iters = 2048
    for blocks, waves, chains in ((1024, 4, 8), (1024, 8, 8), (2048, 8, 16), (4096, 4, 16)):
        t = timed(lambda: _ok(L.hsp_mfma_bf16(blocks, waves, iters, chains, sink.data_ptr(), sp), "hsp_mfma_bf16"))
        mf[f"{blocks}x{waves}w x{chains}"] = round(blocks * waves * iters * chains * 16384 / t / 1e12, 1)
    out["mfma_bf16_tflops"] = max(mf.values())
    out["mfma_bf16"] = {"tflops_by_shape": mf, "instruction": "v_mfma_f32_16x16x32_bf16",
                        "flop_per_instruction": 16384, "iters": iters}
    return out


if __name__ == "__main__":
    import faulthandler
    faulthandler.enable(all_threads=True)
    print(json.dumps(measure()), flush=True)
    sys.exit(0)
