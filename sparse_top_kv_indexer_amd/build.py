"""Build libsparsekv.so (all HIP sources, gfx950) in-tree with hipcc, and
its checking variant libsparsekv_debug.so (compiled with SKV_DEBUG: every
entry point first validates the device-resident tables, windows and
selected positions into a flag word the library holds).

Every source is compiled on its own (in parallel) and linked into one shared
library next to this file.  Flags: -O3, C++17, the packed-fp32 target
feature switched off (hand-written kernels never rely on v_pk_* fp32 forms),
and no fp contraction in the retrieval kernels, whose fp32 operation order is
part of their definition.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libsparsekv.so")
LIB_DEBUG = os.path.join(HERE, "libsparsekv_debug.so")
YARDSTICK = os.path.join(HERE, "libskv_yardstick.so")
BUILD = os.path.join(ROOT, "_build")
BUILD_DEBUG = os.path.join(ROOT, "_build_debug")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + os.path.join(ROOT, "include")]
# files whose fp32 arithmetic must follow a prescribed operation order
NO_CONTRACT = {"paris.hip"}


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, debug: bool = False) -> str:
    obj = os.path.join(BUILD_DEBUG if debug else BUILD, src.replace(".hip", ".o"))
    flags = list(COMMON) + (["-DSKV_DEBUG"] if debug else [])
    if src in NO_CONTRACT:
        flags += ["-ffp-contract=off"]
    cmd = [HIPCC] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = True, debug: bool = False) -> str:
    lib = LIB_DEBUG if debug else LIB
    os.makedirs(BUILD_DEBUG if debug else BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, debug), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


def build_yardstick(verbose: bool = True) -> str:
    """libskv_yardstick.so: the streaming-read probe beside the library."""
    src = os.path.join(HERE, "yardstick", "read_probe.hip")
    tmp = YARDSTICK + ".tmp"
    cmd = [HIPCC] + COMMON + ["-shared", src, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for read_probe.hip:\n" + r.stdout + r.stderr)
    os.replace(tmp, YARDSTICK)
    if verbose:
        print("built", YARDSTICK)
    return YARDSTICK


if __name__ == "__main__":
    build()
    build(debug=True)
    build_yardstick()
