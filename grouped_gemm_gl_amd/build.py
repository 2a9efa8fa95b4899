"""Build the gfx950 shared library ``libgrouped_linear.so`` in-tree with hipcc.

Usage: ``python -m grouped_gemm_gl_amd.build`` (or ``build()`` from Python).  Each
``csrc/*.hip`` file is compiled to an object in ``_build/`` in parallel and the
objects are linked into ``grouped_gemm_gl_amd/libgrouped_linear.so``.

``build()`` also builds the device-check copy ``grouped_gemm_gl_amd/libgrouped_linear_checked.so``
(the same sources with ``GL_DEVICE_CHECKS=1``): its persistent kernels verify every work
item they decode and flag a failure in the workspace status word
(``GL_STATUS_DEVICE_CHECK``) instead of touching memory.  Select it with
``GL_LIBRARY_PATH``.  ``--product-only`` (``build(device_checks=False)``) skips it.

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
CHECKED_DIR = os.path.join(BUILD_DIR, "checked")
CHECKED_OUT = os.path.join(HERE, "libgrouped_linear_checked.so")
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


def build(verbose: bool = False, host_sanitize: bool = False, device_checks: bool = True) -> str:
    """Compile and link the library (returns its path); with device_checks, also the
    device-check copy, its objects compiled in the same pool."""
    hipcc = _hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    # (output directory, library, compile flags, link flags) of each copy
    if host_sanitize:
        copies = [(SAN_DIR, SAN_OUT, [f for f in HIP_FLAGS if f != "-O3"] + ["-O1"] + SAN_COMPILE, SAN_LINK)]
    else:
        copies = [(BUILD_DIR, OUT, HIP_FLAGS, [])]
        if device_checks:
            copies.append((CHECKED_DIR, CHECKED_OUT, HIP_FLAGS + ["-DGL_DEVICE_CHECKS=1"], []))
    jobs = []
    for out_dir, _, flags, _ in copies:
        os.makedirs(out_dir, exist_ok=True)
        jobs += [(src, os.path.join(out_dir, os.path.basename(src) + ".o"), flags) for src in srcs]

    def compile_one(job):
        src, obj, flags = job
        return _run([hipcc, *flags, "-c", src, "-o", obj])

    workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        logs = list(ex.map(compile_one, jobs))
    for out_dir, out, _, link in copies:
        objs = [os.path.join(out_dir, os.path.basename(s) + ".o") for s in srcs]
        tmp = out + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link, "-o", tmp, *objs])
        os.replace(tmp, out)
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
    return copies[0][1]


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, host_sanitize="--host-sanitize" in sys.argv,
                device_checks="--product-only" not in sys.argv))
