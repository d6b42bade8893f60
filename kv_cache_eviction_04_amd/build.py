"""Build libconfkv.so (gfx950) in-tree with hipcc.

    python -m kv_cache_eviction_04_amd.build

Each source is compiled to an object in parallel (every call compiles them
all again), then the objects are linked into the shared library.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libconfkv.so")
OBJ_DIR = os.path.join(ROOT, "_build")
SOURCES = [os.path.join(HERE, "csrc", n)
           for n in ("kernels.hip", "split_attend.hip", "sample.hip", "kvpop_prefill.hip", "probe.hip", "api.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # packed fp32 VALU ops stay disabled: the compiler may otherwise fuse
    # scalar float code into v_pk_* instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
]
NOISE = "packed-fp32-ops"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(x for x in res.stderr.splitlines() if NOISE not in x)
    return res.returncode, err


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    objs = [os.path.join(OBJ_DIR, os.path.basename(s) + ".o") for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, *extra_flags, "-c", "-o", o, s] for s, o in zip(SOURCES, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    for (rc, err), s in zip(results, SOURCES):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(s)} ({rc}):\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    rc, err = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
