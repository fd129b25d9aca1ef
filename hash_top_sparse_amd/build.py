"""Build libhata.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Every source is compiled on each call (object files go to _build/, then one
shared library is linked next to this file).  Packed-fp32 instruction
generation is disabled for all device code.

A second library, libhata_trace.so, is linked from the same objects except
the fused decode step, which is compiled with HATA_PHASE_TRACE: its kernel
stores a timestamp per phase and workgroup into the workspace.  It serves
the phase measurement of bench.py (--phase-trace) only.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libhata.so")
TRACE_LIB = os.path.join(HERE, "libhata_trace.so")
TRACED = "decode_step.hip"
ARCH = "gfx950"

HIP_SOURCES = ["encode.hip", "encode_bulk.hip", "score_select.hip", "attention.hip",
               "decode_step.hip", "stream_read.hip", "train.hip", "prefill.hip"]
CPP_SOURCES = ["api.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-Wall", "-Wno-unused-function"]
DEVICE_ONLY = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str, trace: bool = False) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + (".trace.o" if trace else ".o"))
    cmd = ["hipcc", *COMMON, *(["-DHATA_PHASE_TRACE"] if trace else []), "-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = DEVICE_ONLY
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    # -z defs: an unresolved symbol fails the link instead of the first load
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, trace: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in HIP_SOURCES + CPP_SOURCES if os.path.exists(os.path.join(CSRC, s))]
    jobs = [(s, False) for s in srcs] + ([(TRACED, True)] if trace else [])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    plain = objs[:len(srcs)]
    _link(plain, LIB)
    if verbose:
        print("built", LIB)
    if trace:
        traced = [objs[-1] if src == TRACED else o for src, o in zip(srcs, plain)]
        _link(traced, TRACE_LIB)
        if verbose:
            print("built", TRACE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
