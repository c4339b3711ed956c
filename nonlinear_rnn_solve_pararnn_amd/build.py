"""Build libpararnn.so (HIP, gfx950) in-tree with hipcc.

    python -m nonlinear_rnn_solve_pararnn_amd.build

Each .hip translation unit under csrc/ is compiled to an object in parallel
and the objects are linked into nonlinear_rnn_solve_pararnn_amd/libpararnn.so.
All device code is built with packed fp32 instructions disabled
(-target-feature -packed-fp32-ops); the host pass prints a harmless warning
that it does not know that feature.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpararnn.so")
# measurement-only probe (arithmetic issue rates), a library of its own
PROBE_SRC = os.path.join(HERE, "probe", "alu_probe.hip")
PROBE_LIB = os.path.join(HERE, "libpararnn_probe.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")  # the C ABI header
ARCH = os.environ.get("PARARNN_ARCH", "gfx950")

CFLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function", "-I" + INCLUDE,
]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.exists(c) or c == "hipcc":
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    build_probe(verbose)
    return LIB


def build_probe(verbose: bool = False) -> str:
    obj = _compile(PROBE_SRC)
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", obj, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("probe link failed:\n" + r.stderr)
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print("built", PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    build(verbose=True)
