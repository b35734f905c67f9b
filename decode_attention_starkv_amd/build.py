"""Build libstarkv.so in-tree with hipcc for gfx950.

Usage: python -m decode_attention_starkv_amd.build  (or call build()).
Each source compiles to its own object in parallel (under _build/, next to
this file), then the objects are linked into libstarkv.so.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libstarkv.so")
OBJ = os.path.join(HERE, "_build")
SOURCES = ["api.cpp", "append.hip", "decode.hip", "prefill.hip", "stream.hip",
           "noalloc.hip", "oproj.hip", "rope.hip", "decode_rope.hip",
           "decode_u4.hip", "decode_u4_rope.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-result",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libstarkv")
    return path


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    return res.returncode, out


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link libstarkv.so next to this
    file."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = list(SOURCES)
    jobs = []
    for s in srcs:
        obj = os.path.join(OBJ, os.path.splitext(s)[0] + ".o")
        jobs.append((obj, [hipcc(), *HIPCC_FLAGS, "-x", "hip", "-c",
                           os.path.join(CSRC, s), "-o", obj]))
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", "8"))))
    with cf.ThreadPoolExecutor(workers) as pool:
        results = list(pool.map(lambda j: (j[1], *_run(j[1])), jobs))
    for cmd, rc, out in results:
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError(f"hipcc failed ({rc}):\n{out}")
        if verbose and out.strip():
            print(out)
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=HERE)
    os.close(fd)
    link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC",
            *[j[0] for j in jobs], "-o", tmp]
    rc, out = _run(link)
    if verbose:
        print(" ".join(link), flush=True)
    if rc != 0:
        os.unlink(tmp)
        raise RuntimeError(f"link failed ({rc}):\n{out}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
