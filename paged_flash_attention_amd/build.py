"""Build libpfa.so (the C-ABI library of include/pfa.h) for gfx950 with hipcc.

    python -m paged_flash_attention_amd.build [--jobs N]

Each .hip source under csrc/ is compiled to an object in _build/, then linked
in-tree as paged_flash_attention_amd/libpfa.so.  A second library,
libpfa_debug.so, is the same code built with
  PFA_PREFILL_AUDIT=1  every prefill ring step waits for all loads and all waves,
  PFA_DECODE_AUDIT=1   and every INT8 decode page at G = 8 for all of its wave's
                       direct loads (GPU tests check that the normal build gives
                       the same bits);
  PFA_BOUNDS_CHECK=1   the kernels report block-table entries and lengths outside
                       the device-side contract in an error word
                       (pfa_bounds_errors).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libpfa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep hipcc from forming packed-fp32 instructions on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division: the INT8 quantiser's scale and codes must be bit-exact
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


DEBUG_LIB = os.path.join(HERE, "libpfa_debug.so")
DEBUG_DEFINES = ("PFA_PREFILL_AUDIT=1", "PFA_DECODE_AUDIT=1", "PFA_BOUNDS_CHECK=1")


def compile_one(src: str, outdir: str = BUILD, defines=()) -> str:
    obj = os.path.join(outdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if l.strip() and noise not in l]
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build(jobs: int = 8) -> str:
    debug_dir = os.path.join(BUILD, "debug")
    os.makedirs(debug_dir, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = ex.map(compile_one, srcs)
        debug_objs = ex.map(lambda f: compile_one(f, debug_dir, DEBUG_DEFINES), srcs)
        objs, debug_objs = list(objs), list(debug_objs)
    link(debug_objs, DEBUG_LIB)
    return link(objs, LIB)


def link(objs, target: str) -> str:
    tmp = target + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    # every kernel launch stub must be defined in the library
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in nm.stdout.splitlines() if "__device_stub__" in l]
    if missing:
        raise RuntimeError("undefined kernel launch stubs in libpfa.so:\n" + "\n".join(missing))
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    print(build(ap.parse_args().jobs))
