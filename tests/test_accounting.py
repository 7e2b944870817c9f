"""The benchmark's byte/flop accounting against the figures the CUDA-xSYMV
report prints (section 4; fixture tests/golden/report_bytes_per_flop.json)."""
import json
import os

import pytest

from blas_symmetric_mat_amd import roofline as R

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "report_bytes_per_flop.json")))


@pytest.mark.parametrize("prec", ["s", "d", "c", "z", "w"])
def test_bytes_per_flop_matches_report(prec):
    assert R.bytes_per_flop(prec) == GOLD["bytes_per_flop"][prec]


@pytest.mark.parametrize("prec", ["s", "d", "c", "z", "w"])
def test_ceilings_match_report(prec):
    assert R.bandwidth_bound_gflops(prec, GOLD["peak_gbps"]) == GOLD["ceiling_gflops"][prec]


def test_dd_op_count():
    # (3 loads + 1 store) x 16 bytes / 21 flops per double-double operation
    assert round((3 + 1) * (8 * 2) / 21, 1) == GOLD["dd_bytes_per_flop"]


def test_call_bytes():
    n = 1024
    assert R.stored_elements(n) == 524800
    # the small single-precision workload: triangle + x + y read + y write
    assert R.call_bytes("s", n, beta_zero=False) == 2111488
    # the padded double workload with beta = 0 (y not read)
    assert R.call_bytes("d", 8192, beta_zero=True) == 268599296
    assert R.call_bytes("s", 32768, False) == 2147942400
    assert R.call_bytes("d", 32768, False) == 4295884800
    assert R.gflops_2n2(1000, 1e-3) == 2.0
