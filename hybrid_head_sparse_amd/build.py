"""Compile the gfx950 library liblychee.so in-tree with hipcc.

    python -m hybrid_head_sparse_amd.build            # liblychee.so
    python -m hybrid_head_sparse_amd.build --trace    # liblychee_trace.so: the same
        library with phase timestamps in the attention kernel (a measuring aid,
        read by hybrid_head_sparse_amd.timeline)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblychee.so")
TRACE_BUILD = os.path.join(HERE, "_build_trace")
TRACE_LIB = os.path.join(HERE, "liblychee_trace.so")
SOURCES = ["attend.hip", "correction.hip", "abi.hip"]
ARCH = os.environ.get("LYCHEE_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 instructions are kept out of all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def _compile(src: str, trace: bool = False) -> str:
    obj = os.path.join(TRACE_BUILD if trace else BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, *(["-DLYCHEE_TRACE"] if trace else []), "-I", os.path.join(ROOT, "include"), "-c",
           os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = True, trace: bool = False) -> str:
    out = TRACE_LIB if trace else LIB
    os.makedirs(TRACE_BUILD if trace else BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, trace), SOURCES))
    tmp = out + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(trace="--trace" in sys.argv[1:])
    sys.exit(0)
