"""Build the HIP libraries in-tree for gfx950 with hipcc.

* ``quantized_kv_cache_loopkv_amd/libloopkv.so``: the C-ABI library (include/loopkv.h).
* ``synth/libloopkv_synth.so``: the GPU side of the seeded input generator.

Every object is compiled with packed fp32 instructions disabled. The quantizer
(append.hip) is compiled with -ffp-contract=off so its float64 arithmetic is
exactly the sequence of rounded operations it spells out.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "unknown target feature" not in l
                    and "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed ({r.returncode}):\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build_loopkv(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    units = [("runtime.cpp", []), ("planner.cpp", []), ("append.hip", ["-ffp-contract=off"]), ("decode.hip", [])]
    for src, extra in units:
        obj = os.path.join(BUILD, src.replace(".", "_") + ".o")
        lang = ["-x", "hip"]
        _run([hipcc, *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    out = os.path.join(PKG, "libloopkv.so")
    tmp = out + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)
    return out


def build_synth(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    src = os.path.join(ROOT, "synth", "csrc", "synth_kernel.hip")
    out = os.path.join(ROOT, "synth", "libloopkv_synth.so")
    tmp = out + ".tmp"
    _run([hipcc, *COMMON, "-shared", src, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False):
    return build_loopkv(verbose), build_synth(verbose)


if __name__ == "__main__":
    for p in build_all(verbose="-v" in sys.argv):
        print(p)
