"""Build libbwa.so (the C-ABI HIP library) in-tree for gfx950.

Usage: python -m ring_exact_attention_amd.build
Compiles every csrc/*.hip with hipcc into _build/ and links
ring_exact_attention_amd/libbwa.so, then links the diagnostic build
libbwa_slot_timers.so: the same objects except fwd.hip, compiled again with
BWA_SLOT_TIMERS=1 (phase clocks in the forward kernel, include/bwa_diag.h).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbwa.so")
LIB_TIMERS = os.path.join(PKG, "libbwa_slot_timers.so")
TIMED_SRC = "fwd.hip"
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# Packed-fp32 instructions stay disabled: the compiler emits ordinary
# v_fma/v_mul/v_add instead of v_pk_* forms.
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
]


def _compile(src: str, timers: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + (".timers.o" if timers else ".o"))
    extra = ["-DBWA_SLOT_TIMERS=1"] if timers else []
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that noise
    noise = ("packed-fp32-ops", "not a recognized feature", "warning generated")
    msg = "\n".join(l for l in r.stderr.splitlines() if l and not any(n in l for n in noise))
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def _link(objs, lib: str):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.check_call(cmd)
    os.replace(tmp, lib)


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    timed = os.path.join(CSRC, TIMED_SRC)
    jobs = jobs or min(len(srcs) + 1, os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_compile, s) for s in srcs]
        fut_timed = ex.submit(_compile, timed, True)
        objs = [f.result() for f in futs]
        obj_timed = fut_timed.result()
    _link(objs, LIB)
    plain = os.path.join(BUILD, TIMED_SRC + ".o")
    _link([obj_timed if o == plain else o for o in objs], LIB_TIMERS)
    return LIB


if __name__ == "__main__":
    print(build())
