"""Build libwq.so (the HIP library behind include/wq.h) for gfx950, in-tree.

    python -m quantized_gemm_rtn_amd.build [-v]

Each .hip file is compiled separately with hipcc (object files under
_build/, outside version control) and linked into
quantized_gemm_rtn_amd/libwq.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libwq.so")
# the benchmark's streaming-read probe (include/wq_probe.h), a library of its own
PROBE_LIB = os.path.join(HERE, "libwq_probe.so")
PROBE_SOURCES = ["probe.hip"]
ARCH = "gfx950"

SOURCES = ["wq_api.hip", "split.hip", "quant.hip", "gemv.hip", "gemv_fmt.hip", "gemv_dot.hip", "gemm.hip",
           "lowrank.hip", "actorder.hip", "w4a8.hip"]

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no hand-written or compiler-made packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE float32 division, as the quantizer's definition requires
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # the first kernel arguments arrive in scalar registers with the wave, so its
    # first loads need not wait for a load of the argument block (about 0.2 us per
    # decode launch)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]
# The quantizer and split decide integers with float32 arithmetic: no contraction.
PER_FILE = {"quant.hip": ["-ffp-contract=off"], "split.hip": ["-ffp-contract=off"], "w4a8.hip": ["-ffp-contract=off", "-mllvm", "-amdgpu-mfma-vgpr-form"]}
# The product kernels must keep everything in registers and LDS: the compiler
# reports each kernel's per-lane scratch, and any use of it fails the build.
NO_SCRATCH = {"gemv.hip", "gemv_fmt.hip", "gemv_dot.hip", "gemm.hip", "lowrank.hip", "w4a8.hip"}
RESOURCE_REMARK = "-Rpass-analysis=kernel-resource-usage"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    check = src in NO_SCRATCH
    cmd = [hipcc(), *COMMON, *PER_FILE.get(src, []), *([RESOURCE_REMARK] if check else []),
           "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if check:
        bad = scratch_users(r.stderr)
        if bad:
            raise RuntimeError(f"{src}: kernels using scratch memory (bytes per lane): {bad}")
    elif verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def scratch_users(remarks: str) -> dict:
    """Kernels with a nonzero ScratchSize in the compiler's resource-usage remarks."""
    bad, name = {}, None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name is not None and int(m.group(1)) > 0:
            bad[name] = int(m.group(1))
    return bad


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    # no undefined symbols left for the loader to find (a missing object fails here)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source, link libwq.so and the benchmark's probe library;
    returns the path of libwq.so."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    jobs = min(len(srcs), max(1, int(os.environ.get("MAX_JOBS", "8"))))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
