"""Build libttt.so (HIP, gfx950) in-tree: ``python -m chunkwise_weight_recurrence_amd.build``.

Compiles every source under ``csrc/`` with hipcc for gfx950 and links the
shared library next to this file.  Packed-fp32 VALU instructions are switched
off for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libttt.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")

SOURCES = ["ttt_host.cpp", "ttt_timing.cpp", "ttt_generic.hip", "ttt_mfma_fwd.hip", "ttt_mfma_bwd.hip", "ttt_decay_prep.hip", "ttt_linear.hip", "inplace.hip", "ttt_mlp.hip", "ttt_mlp_bwd.hip", "ttt_norm.hip", "ttt_noalloc.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++20", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found")
    return h


def _compile(src, extra):
    out = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", out]
    p = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (p.stdout + p.stderr).splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    return out, msgs


def _stale(src):
    """True when src's object is missing or older than src or any header it may include."""
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    deps = [os.path.join(CSRC, src)] + [os.path.join(CSRC, h) for h in os.listdir(CSRC) if h.endswith(".h")]
    deps.append(os.path.join(INCLUDE, "ttt.h"))
    return any(os.path.getmtime(d) > t for d in deps)


def build(verbose: bool = False, extra_flags=None, incremental: bool = False) -> str:
    """Compile the sources and link libttt.so; returns the library path.

    Every source is compiled unless ``incremental`` is set, which recompiles
    only sources whose object is older than the source or a header."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra_flags or [])
    todo = [s for s in SOURCES if _stale(s)] if incremental else list(SOURCES)
    jobs = min(max(1, len(todo)), max(1, (os.cpu_count() or 4)), 16)
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, extra), todo))
    for _, msgs in results:
        if verbose and msgs.strip():
            print(msgs, file=sys.stderr)
    objs = [os.path.join(BUILD, os.path.basename(src) + ".o") for src in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("link failed:\n" + p.stdout + p.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv[1:])
