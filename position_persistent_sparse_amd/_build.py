"""Build of libppsa.so with hipcc for gfx950 (in-tree, next to the binding).

Each HIP source is compiled to its own object in parallel (whole-program
device code is not needed: every kernel lives in one translation unit), then
the objects are linked into the shared library.
"""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libppsa.so")
OBJ_DIR = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # Keep the compiler from forming packed-FP32 (v_pk_*_f32) instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
_NOISE = "is not a recognized feature for this target"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(line for line in (res.stdout + res.stderr).splitlines() if _NOISE not in line)
    return res.returncode, msgs


def build_library(verbose: bool = False, extra_flags=None, out=None, jobs=None) -> str:
    """Compiles every csrc/*.hip and links them into `out` (default: libppsa.so next to this file)."""
    out = out or LIB
    tag = os.path.splitext(os.path.basename(out))[0]
    obj_dir = os.path.join(OBJ_DIR, tag)
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sources()
    flags = [*FLAGS, *(extra_flags or [])]
    cmds = [[HIPCC, *flags, "-c", "-o", os.path.join(obj_dir, os.path.basename(s) + ".o"), s] for s in srcs]
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, msgs) in zip(cmds, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError(f"hipcc failed ({rc}) on {cmd[-1]}:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs, flush=True)
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out + ".tmp", *[c[-2] for c in cmds]]
    rc, msgs = _run(link)
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{msgs}")
    os.replace(out + ".tmp", out)
    return out
