"""The C ABI without Python: a plain host program (tests/native/abi_caller.cpp)
allocates device buffers with hipMalloc, calls xsymv_d, xhemv_z and xtrmv_s on
a stream of its own through include/xsymv.h only, and checks every result
against the oracle's C functions (integer inputs: equal value for value)."""
import os
import subprocess
import sys

import pytest

from tests import native

pytestmark = pytest.mark.gpu


def test_native_program_through_the_c_header():
    exe = native.ABI_CALLER
    if not os.path.exists(exe):
        native.build_abi_caller()
    sys.stdout.write("native abi caller\n")
    sys.stdout.flush()
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    sys.stdout.write(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
