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
    """Compile the units in parallel (decode.hip twice: 32-bit and 64-bit record offsets), link."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    units = [("runtime.cpp", [], "runtime"), ("planner.cpp", [], "planner"),
             ("append.hip", ["-ffp-contract=off"], "append"), ("decode.hip", [], "decode"),
             ("decode.hip", ["-DLKV_DECODE_BIG=1"], "decode_big")]
    cmds, objs = [], []
    for src, extra, name in units:
        obj = os.path.join(BUILD, name + ".o")
        cmds.append([hipcc, *COMMON, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "0")) or (os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    out = os.path.join(PKG, "libloopkv.so")
    tmp = out + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)
    return out


SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that a process loading the sanitized library
    must preload (the Python interpreter itself is not instrumented)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "lib", "llvm", "bin", "clang++")
    for c in (clang, "/opt/rocm/llvm/bin/clang++"):
        if os.path.exists(c):
            r = subprocess.run([c, "--print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE, text=True)
            path = r.stdout.strip()
            if os.path.exists(path):
                return path
    raise RuntimeError("clang's AddressSanitizer runtime not found")


def build_sanitized(verbose: bool = False) -> str:
    """A host-sanitized copy of the library for CPU-only checks of the host code: runtime.cpp
    and planner.cpp built with AddressSanitizer and UndefinedBehaviorSanitizer on the host side
    only (device code unchanged), linked with the regular kernel objects into
    _build/libloopkv_san.so. Load it with LOOPKV_LIB pointing at it and the ASan runtime
    preloaded (asan_runtime())."""
    from concurrent.futures import ThreadPoolExecutor
    build_loopkv(verbose)   # the kernel objects
    hipcc = _hipcc()
    cmds, objs = [], []
    for src, name in (("runtime.cpp", "runtime_san"), ("planner.cpp", "planner_san")):
        obj = os.path.join(BUILD, name + ".o")
        cmds.append([hipcc, *COMMON, *SAN_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(2) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    objs += [os.path.join(BUILD, n + ".o") for n in ("append", "decode", "decode_big")]
    out = os.path.join(BUILD, "libloopkv_san.so")
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", out, *objs], verbose)
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
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
        print(asan_runtime())
    else:
        for p in build_all(verbose="-v" in sys.argv):
            print(p)
