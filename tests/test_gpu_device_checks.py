"""The device-check build of the library on the GPU.

libgrouped_linear_checked.so is the library's sources compiled with
GL_DEVICE_CHECKS=1: its persistent kernels verify each work item they decode (group,
tile row inside the group, tile column, contraction-schedule entry) and flag a
failure in the workspace status word (GL_STATUS_DEVICE_CHECK) instead of touching
memory.  It runs in a child process (one library per process) on the cases of
device_check_cases.py:

- valid launches: the checks stay silent (status 0) and every output is bit-identical
  to the product build's on the same inputs;
- a workspace whose offsets were changed after the offsets call (group 0 ends at row
  200 while the tile table still gives it two 256-row tiles): the forward flags the
  tile past group 0's rows, skips it, and computes every other tile.
"""
import os
import subprocess
import sys

import pytest
import torch

import device_check_cases as cases
import grouped_gemm_gl_amd as gl
import oracle
from gl_testutil import TOL_BF16, assert_bits_equal, assert_close, to64
from grouped_gemm_gl_amd import build as gl_build

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STATUS_DEVICE_CHECK = 8  # GL_STATUS_DEVICE_CHECK


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def checked(tmp_path_factory):
    lib = gl_build.CHECKED_OUT
    assert os.path.exists(lib), f"{lib} is missing: build() makes it beside the library"
    out = str(tmp_path_factory.mktemp("device_checks") / "results.pt")
    say(f"device-check build in a child process: {lib}")
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "tests", "device_check_cases.py"), out],
                       cwd=ROOT, env=dict(os.environ, GL_LIBRARY_PATH=lib), stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=300)
    say(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-4000:]
    res = torch.load(out, weights_only=True)
    assert bytes(res.pop("library").tolist()).decode() == lib
    return res


def test_checked_build_is_silent_and_bit_identical(checked):
    gl.load()
    assert os.path.abspath(gl.library_path) != os.path.abspath(gl_build.CHECKED_OUT)
    mine = cases.run(gl)
    for k, v in mine.items():
        say(f"  {k}")
        if k.endswith("_status"):
            assert int(v) == 0, f"product build: {k} = {int(v)}"
            assert int(checked[k]) == 0, f"device-check build: {k} = {int(checked[k])}"
        else:
            assert_bits_equal(checked[k], v, f"{k}: device-check build vs product build")


def test_checked_forward_flags_and_skips_a_tile_past_its_group(checked):
    r = checked
    assert int(r["tamper_status_ok"]) == 0
    assert int(r["tamper_status"]) == STATUS_DEVICE_CHECK
    y_ok, y = r["tamper_y_ok"], r["tamper_y"]
    # group 0 keeps its first tile (rows 0 .. 199 now); its second tile is skipped
    assert_bits_equal(y[:200], y_ok[:200], "group 0, rows 0..199")
    # group 1's one tile now starts at row 200
    X, W, B = to64(r["tamper_x"]), to64(r["tamper_w"]), to64(r["tamper_b"])
    assert_close(y[200:456], oracle.forward(X[200:456], W[1:2], B[1:2], [256]), TOL_BF16, "group 1 over rows 200..455")
    assert torch.isnan(y[456:500].float()).all(), "rows 456..499 lie in no tile and stay untouched"
    assert_bits_equal(y[500:], y_ok[500:], "group 3")
