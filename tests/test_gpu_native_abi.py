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


LOAD_FIRST = r'''
import sys
sys.path.insert(0, sys.argv[1])
import blas_symmetric_mat_amd as X
X.library()  # the binding's first act, before this program imports torch
import torch
n = 300
g = torch.Generator().manual_seed(5)
A = torch.rand(n * n, dtype=torch.float64, generator=g)
x = torch.rand(n, dtype=torch.float64, generator=g)
y = torch.zeros(n, dtype=torch.float64, device="cuda")
X.xsymv_d("L", n, 1.0, A.cuda(), n, x.cuda(), 1, 0.0, y, 1)
torch.cuda.synchronize()
M = A.view(n, n).T                       # M[i, j] = A(i, j), column-major
S = torch.tril(M) + torch.tril(M, -1).T
ref = S @ x
bound = 4 * n * 2.0 ** -53 * (S.abs() @ x.abs())
assert bool(((y.cpu() - ref).abs() <= bound).all()), "result beyond the bound"
med, best = X.read_bandwidth(256 << 20, reps=2)
assert 0 < med <= best
print("ok")
'''


def test_binding_loaded_before_torch_in_a_fresh_process():
    """A fresh process whose first call loads the library before it imports
    torch itself: the binding brings torch's HIP runtime in first, so the
    library and torch share one runtime and the calls succeed."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.stdout.write("binding loaded before torch\n")
    sys.stdout.flush()
    r = subprocess.run([sys.executable, "-c", LOAD_FIRST, root], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
