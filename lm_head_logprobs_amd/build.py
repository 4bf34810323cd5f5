"""Compile librlloss.so for gfx950 in-tree (hipcc, one object per source, in parallel)."""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
SOURCES = ("api.hip", "gemm.hip", "head.hip", "sparse.hip", "elementwise.hip", "mis.hip",
           "validate.hip", "calib.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in r.stderr.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    workers = min(len(jobs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        for msg in ex.map(_run, jobs):
            if verbose and msg:
                print(msg)
    out = os.path.join(HERE, "librlloss.so")
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, out)
    return out


# Host-sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer on the
# host half only; device code is built as usual): librlloss_asan.so, loaded by
# the CPU tests of the ABI's host checks under the sanitizer runtime.
ASAN_BUILD = os.path.join(HERE, "_build_asan")
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=undefined",
              "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime that must be preloaded into a
    non-instrumented host process (python) before the library loads."""
    out = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        base = "/opt/rocm/llvm/lib/clang"
        for v in sorted(os.listdir(base)) if os.path.isdir(base) else []:
            cand = os.path.join(base, v, "lib", "linux", "libclang_rt.asan-x86_64.so")
            if os.path.exists(cand):
                return cand
        raise RuntimeError("AddressSanitizer runtime not found")
    return out


def build_asan(verbose: bool = False) -> str:
    os.makedirs(ASAN_BUILD, exist_ok=True)
    objs, jobs = [], []
    for src in SOURCES:
        obj = os.path.join(ASAN_BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([HIPCC, *FLAGS, *ASAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    workers = min(len(jobs), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        for msg in ex.map(_run, jobs):
            if verbose and msg:
                print(msg)
    out = os.path.join(ASAN_BUILD, "librlloss_asan.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *ASAN_FLAGS[:4],
          "-Xarch_host", "-shared-libsan", "-o", out, *objs])
    return out


if __name__ == "__main__":
    print(build(verbose=True))
