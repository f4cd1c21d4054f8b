"""Builds libfa.so (the HIP kernels and the C ABI of include/fa.h) in-tree for gfx950.

Usage: ``python -m exact_tiled_attention_02_amd.build`` (or ``build()`` from Python).
Every call recompiles.  Translation units compile in parallel, then link.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa.so")
ATOMIC_RATE = os.path.join(PKG, "atomic_rate")
LDS_RATE = os.path.join(PKG, "lds_rate")
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_decode.hip", "fa_check.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # Packed fp32 VALU forms stay off: scalar fp32 code only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + "\n".join(msgs))
    return "\n".join(msgs)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link libfa.so; returns its path."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cmds = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append([HIPCC] + FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=jobs or min(len(cmds), os.cpu_count() or 1)) as ex:
        logs = list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    logs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs))
    os.replace(tmp, LIB)
    # the measurement programs of the fp32 atomic rate and the LDS read rate (not part of the library)
    for src, prog in (("atomic_rate.hip", ATOMIC_RATE), ("lds_rate.hip", LDS_RATE)):
        logs.append(_run([HIPCC] + FLAGS + ["-x", "hip", os.path.join(CSRC, src), "-o", prog]))
    if verbose:
        for log in logs:
            if log.strip():
                print(log)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
