"""Build the gfx950 shared library ``libgrouped_linear.so`` in-tree with hipcc.

Usage: ``python -m grouped_gemm_gl_amd.build`` (or ``build()`` from Python).  Each
``csrc/*.hip`` file is compiled to an object in ``_build/`` in parallel and the
objects are linked into ``grouped_gemm_gl_amd/libgrouped_linear.so``.

``python -m grouped_gemm_gl_amd.build --host-sanitize`` (``build(host_sanitize=True)``)
builds a second copy, ``_build/hostsan/libgrouped_linear_hostsan.so``, whose host code
carries AddressSanitizer and UndefinedBehaviorSanitizer (device code is built as
usual, without them).  It is for CPU runs of the argument validation and the
deferred-wgrad queue: load it with the clang ASan runtime preloaded
(``asan_runtime()``) and ``GL_LIBRARY_PATH`` pointing at it.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libgrouped_linear.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SAN_DIR = os.path.join(BUILD_DIR, "hostsan")
SAN_OUT = os.path.join(SAN_DIR, "libgrouped_linear_hostsan.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    "-Wno-unused-function",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]

# host-only sanitizers: each -fsanitize= is bound to the host pass by -Xarch_host
SAN_COMPILE = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-g",
]
SAN_LINK = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-shared-libasan",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    text = "\n".join(l for l in r.stdout.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{text}")
    return text


def asan_runtime() -> str:
    """Path of the clang ASan runtime that a host-sanitized library needs preloaded."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    clang = os.path.join(rocm, "llvm", "bin", "clang")
    return subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE,
                          text=True, check=True).stdout.strip()


def build(verbose: bool = False, host_sanitize: bool = False) -> str:
    out_dir = SAN_DIR if host_sanitize else BUILD_DIR
    out = SAN_OUT if host_sanitize else OUT
    os.makedirs(out_dir, exist_ok=True)
    hipcc = _hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(out_dir, os.path.basename(s) + ".o") for s in srcs]
    flags = HIP_FLAGS
    if host_sanitize:
        flags = [f for f in HIP_FLAGS if f != "-O3"] + ["-O1"] + SAN_COMPILE

    def compile_one(pair):
        src, obj = pair
        return _run([hipcc, *flags, "-c", src, "-o", obj])

    workers = max(1, min(len(srcs), os.cpu_count() or 1, 16))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        logs = list(ex.map(compile_one, zip(srcs, objs)))
    tmp = out + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(SAN_LINK if host_sanitize else []), "-o", tmp,
          *objs])
    os.replace(tmp, out)
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, host_sanitize="--host-sanitize" in sys.argv))
