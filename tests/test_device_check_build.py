"""The device-check copy of the library (CPU checks; its GPU behaviour is covered by
test_gpu_device_checks.py): build() makes it beside the library, it loads, and it
exports every entry point the header declares, so GL_LIBRARY_PATH can select it
for any caller."""
import ctypes
import os

import pytest

import grouped_gemm_gl_amd as gl
from grouped_gemm_gl_amd import build as gl_build
from test_abi import declared_symbols

pytestmark = pytest.mark.skipif(not os.path.exists(gl.library_path), reason="library not built")


def test_device_check_build_exists_beside_the_library():
    assert os.path.dirname(gl_build.CHECKED_OUT) == os.path.dirname(gl_build.OUT)
    assert os.path.exists(gl_build.CHECKED_OUT), "build() makes the device-check copy with the library"


def test_device_check_build_exports_every_declared_symbol():
    lib = ctypes.CDLL(gl_build.CHECKED_OUT)
    missing = [n for n in declared_symbols() if not hasattr(lib, n)]
    assert not missing


def test_status_bit_is_declared():
    text = open(os.path.join(os.path.dirname(gl_build.HERE), "include", "grouped_linear.h")).read()
    assert "GL_STATUS_DEVICE_CHECK = 8" in text
