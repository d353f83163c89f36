"""Compiles the HIP library libmoe_fp4.so in-tree for gfx950 with hipcc.

Each source is compiled to an object of its own (in parallel, under _build/),
then the objects are linked into the shared library.
"""
from __future__ import annotations

import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmoe_fp4.so")
OBJDIR = os.path.join(ROOT, "_build")
SRC = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip"))) + [os.path.join(PKG, "csrc", "moe_api.cpp")]
HDR = sorted(glob.glob(os.path.join(PKG, "csrc", "*.h"))) + [
    os.path.join(ROOT, "include", "moe_fp4.h")]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU instructions are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    return res.stdout + res.stderr


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, os.path.basename(s) + ".o") for s in SRC]
    jobs = [[hipcc, *FLAGS, "-c", "-o", o, s] for s, o in zip(SRC, objs)]
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        logs = list(ex.map(_run, jobs))
    tmp = LIB + ".tmp"
    logs.append(_run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]))
    if verbose:
        out = "\n".join(l for l in "\n".join(logs).splitlines() if "packed-fp32-ops" not in l)
        if out.strip():
            print(out)
    os.replace(tmp, LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in SRC + HDR)


if __name__ == "__main__":
    print(build(verbose=True))
