"""Build libhisparse.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m sparse_mla_decode_indexer_amd.build

Every .hip file under csrc/ is compiled to an object in _build/, then
linked into sparse_mla_decode_indexer_amd/libhisparse.so (the decode path).
The measurement probes under csrc/probe/ become libhsprobe.so, a library of
their own that the decode path never loads.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libhisparse.so")
PROBE_LIB = os.path.join(PKG, "libhsprobe.so")
PROBE_SRC = os.path.join(CSRC, "probe")
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Wno-unused-command-line-argument",
    # packed fp32 ops are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source extra flags. attention.hip: keep MFMA accumulators in ordinary
# VGPRs. With four waves per workgroup the compiler otherwise places them in
# AGPRs and copies all 64 of them to VGPRs and back every tile around the
# softmax rescale (about 130 extra vector instructions per tile).
EXTRA_FLAGS = {
    "attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources(d: str = CSRC):
    return sorted(os.path.join(d, f) for f in os.listdir(d) if f.endswith(".hip"))


def _compile(src: str) -> str:
    sub = os.path.basename(os.path.dirname(src))
    stem = os.path.basename(src)[:-4]
    obj = os.path.join(BUILD, (stem if sub == "csrc" else f"{sub}_{stem}") + ".o")
    cmd = [HIPCC, *CFLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l).strip()
    if err:
        print(err, file=sys.stderr)
    return obj


def _link(objs, lib: str):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link both shared libraries; returns the
    decode library's path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs, psrcs = sources(), sources(PROBE_SRC)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(psrcs))) as ex:
        objs = list(ex.map(_compile, srcs + psrcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
