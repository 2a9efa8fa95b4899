"""The host code of the library (argument validation, workspace checks, the
deferred-wgrad queue) under AddressSanitizer and UndefinedBehaviorSanitizer, on the
CPU: builds the host-sanitized copy of the library if it is missing or older than a
source, then runs the ABI and queue tests against it in a child process with the
ASan runtime preloaded.  Device code in that copy is built without sanitizers and
never runs here (every call in those tests fails validation or touches only host
state)."""
import glob
import os
import subprocess
import sys

import pytest

from grouped_gemm_gl_amd import build as gl_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale(lib):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = glob.glob(os.path.join(gl_build.CSRC, "*")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    return any(os.path.getmtime(s) > t for s in srcs)


@pytest.fixture(scope="module")
def sanitized_library():
    try:
        runtime = gl_build.asan_runtime()
    except (OSError, subprocess.CalledProcessError) as e:
        pytest.skip(f"no clang ASan runtime: {e}")
    if not os.path.exists(runtime):
        pytest.skip(f"no clang ASan runtime at {runtime}")
    if _stale(gl_build.SAN_OUT):
        gl_build.build(host_sanitize=True)
    return gl_build.SAN_OUT, runtime


def test_abi_and_queue_tests_clean_under_host_sanitizers(sanitized_library):
    lib, runtime = sanitized_library
    env = dict(os.environ)
    env.update(LD_PRELOAD=runtime, GL_LIBRARY_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87")
    code = ("import sys, pytest, grouped_gemm_gl_amd as gl\n"
            f"assert gl.library_path == {lib!r}, gl.library_path\n"
            "sys.exit(pytest.main(['-q', '-s', '-p', 'no:cacheprovider', 'tests/test_abi.py', "
            "'tests/test_wgrad_queue.py']))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=600)
    tail = "\n".join(r.stdout.splitlines()[-30:])
    assert "ERROR: AddressSanitizer" not in r.stdout and "runtime error:" not in r.stdout, tail
    assert r.returncode == 0, tail
    assert " passed" in r.stdout, tail
