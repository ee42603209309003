"""Build libttt_mi355x.so in-tree with hipcc for gfx950.

    python -m chunked_weight_sequence_amd.build [-v]

Every HIP source is compiled to an object under _build/ (in parallel) and linked into
chunked_weight_sequence_amd/libttt_mi355x.so. Only the C ABI symbols are exported.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libttt_mi355x.so")
ARCH = "gfx950"

SOURCES = ["scan_simt.hip", "scan_mfma.hip", "linear.hip", "linear_b32.hip", "linear_chunk.hip",
           "route.hip", "target.hip", "gated_z.hip", "readout.hip", "clip.hip", "noalloc.hip",
           "api.cpp"]
# per-file options: routing decisions must round every operation on its own (no fused
# multiply-add), and its latency-bound kernel schedules better for instruction-level parallelism
PER_FILE = {
    "route.hip": ["-ffp-contract=off", "-mllvm", "-amdgpu-sched-strategy=max-ilp"],  # 18.4 -> 17.4 us
    # the readout's two dependent gathers: its loads grouped into clauses (30.7 -> 30.35 us)
    "readout.hip": ["-mllvm", "-amdgpu-sched-strategy=max-memory-clause"],
    # small 16x16 products whose results feed VALU work at once: keep them in ordinary VGPRs; the
    # latency-bound mini-batch chain schedules better for instruction-level parallelism (b = 16
    # and b = 64 about 5% faster, same results; b = 32 is about 3% slower under it, so its kernels
    # are built in linear_b32.hip with the default scheduler)
    "linear.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "linear_b32.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    # the chunked kernel: same results under both schedulers; scheduled for instruction-level
    # parallelism it runs b = 16 about 3% faster (b = 64 the same)
    "linear_chunk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # keep the compiler from forming packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src: str, verbose: bool) -> str:
    out = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src), "-o", out]
    if verbose and src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if verbose and msg.strip():
        print(msg)
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
