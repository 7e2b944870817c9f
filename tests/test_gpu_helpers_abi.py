"""The helper calls of the C ABI on the device: per-call timing records
(xsymv_timing_enable / xsymv_timing_read), the workgroup count a row-strip
configuration is launched with (xsymv_config_workgroups), and the GEMV
workspace size (xgemv_workspace_bytes) being exactly enough for a
caller-installed workspace."""
import numpy as np
import pytest

import oracle
from blas_symmetric_mat_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def test_timing_records_one_entry_per_call():
    import torch
    import blas_symmetric_mat_amd as X
    G.log("timing records")
    p = W.make_problem("d", "L", 2000, 2000, seed=3)
    d = G.DeviceProblem(p)
    y = G.to_device(p.y)
    X.timing_read()  # drop anything recorded before
    X.timing_enable(True)
    try:
        for _ in range(3):
            d.run_device(y)
        torch.cuda.synchronize()
        rec = X.timing_read()
    finally:
        X.timing_enable(False)
    assert len(rec) == 3
    assert all(main > 0 and merge > 0 for main, merge in rec)
    assert X.timing_read() == []  # read once
    d.run_device(y)
    torch.cuda.synchronize()
    assert X.timing_read() == []  # disabled: nothing recorded
    # whole-call mode: (span, 0) per call, the span longer than the main
    # kernel alone takes
    X.timing_enable(2)
    try:
        for _ in range(3):
            d.run_device(y)
        torch.cuda.synchronize()
        whole = X.timing_read()
    finally:
        X.timing_enable(False)
    assert len(whole) == 3
    assert all(span > 0 and merge == 0 for span, merge in whole)
    assert sorted(s for s, _ in whole)[1] > sorted(m for m, _ in rec)[1]
    # one-kernel calls: the rank-2 update records (kernel, 0) in both modes
    A = torch.zeros(500 * 500, dtype=torch.float64, device="cuda")
    v = torch.ones(500, dtype=torch.float64, device="cuda")
    for mode in (1, 2):
        X.timing_enable(mode)
        try:
            X.xsyr2_d("L", 500, 1.0, v, 1, v, 1, A, 500)
            torch.cuda.synchronize()
            one = X.timing_read()
        finally:
            X.timing_enable(False)
        assert len(one) == 1 and one[0][0] > 0 and one[0][1] == 0


def test_strip_configurations_fill_every_cu():
    import torch
    import blas_symmetric_mat_amd as X
    G.log("config workgroups")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for p in "sdczw":
        for i in range(X.num_configs(p)):
            if X.config_info(p, i)["column_runs"] >= 4:
                for u in "LU":
                    g = X.config_workgroups(p, i, u)
                    assert g >= cus and g % cus == 0, (p, i, u, g, cus)


@pytest.mark.parametrize("trans", ["N", "T"])
def test_gemv_workspace_bytes_exactly_enough(trans):
    import torch
    import blas_symmetric_mat_amd as X
    G.log(f"gemv workspace {trans}")
    m, n = 3000, 2000
    p = W.make_gemv_problem("d", trans, m, n, m + 1, seed=5)
    need = X.gemv_workspace_bytes("d", trans, m, n)
    assert 0 < need < 1 << 32
    A, x = G.to_device(p.A), G.to_device(p.x)
    stream = torch.cuda.Stream()
    buf = torch.empty(need, dtype=torch.uint8, device="cuda")
    small = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    try:
        X.set_workspace(buf, stream=stream)
        y = G.to_device(p.y)
        X.xgemv_d(trans, m, n, p.alpha, A, p.lda, x, 1, p.beta, y, 1, stream=stream)
        stream.synchronize()
        G.assert_close_gemv(p, y.cpu().numpy(), oracle.gemv_problem(p), label="installed")
        X.set_workspace(small, stream=stream)
        y2 = G.to_device(p.y)
        with pytest.raises(X.XsymvError) as e:
            X.xgemv_d(trans, m, n, p.alpha, A, p.lda, x, 1, p.beta, y2, 1, stream=stream)
        assert e.value.code == 2000
        stream.synchronize()
        assert np.array_equal(y2.cpu().numpy(), p.y)  # nothing was enqueued
    finally:
        X.set_workspace(None, stream=stream)
