"""Build libkda.so (HIP, gfx950) in-tree with hipcc.

    python gated_delta_rule_74_amd/build.py     (or __graft_entry__.build())

Every call recompiles (the objects are small and the check is cheap to keep
honest).  Packed-fp32 instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkda.so")
# measurement only (bench.py): the state pass's load floor
PROBE_SOURCES = ["probe_read_rate.hip"]
PROBE_LIB = os.path.join(HERE, "libkda_probe.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

SOURCES = ["kda_api.hip", "kda_prep_f32.hip", "kda_prep_bf16_f32.hip",
           "kda_prep_bf16_bf16.hip", "kda_prep_gdn.hip", "kda_prep_d128.hip", "kda_state.hip", "kda_decode.hip",
           "kda_backward.hip",
           "kda_conv.hip"]
ARCH = os.environ.get("KDA_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CXXFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CXXFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    nlib = len(SOURCES)
    for lib, parts in ((LIB, objs[:nlib]), (PROBE_LIB, objs[nlib:])):
        tmp = lib + ".tmp"
        cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *parts,
               "-o", tmp]
        subprocess.run(cmd, check=True, capture_output=not verbose)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
