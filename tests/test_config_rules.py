"""Configuration selection rules and their files (the autotuner's record), on
the CPU: caller rules take precedence over the built-in ones, the latest
matching rule wins, index -1 defers to the built-in choice, rule files round
trip through save/load, malformed or missing files are refused, rules for
shapes that are not compiled are skipped, and argument errors are caught.
The on-device search itself is tested in test_gpu_autotune.py."""
import json

import pytest

import blas_symmetric_mat_amd as X


@pytest.fixture(autouse=True)
def _clean_rules():
    X.clear_config()
    yield
    X.clear_config()


def test_caller_rules_take_precedence_latest_first():
    builtin = X.current_config("d", "L", 5000)
    builtin_6001 = X.current_config("d", "L", 6001)
    builtin_u = X.current_config("d", "U", 5000)
    other = (builtin + 1) % X.num_configs("d")
    X.select_config("d", "L", 4000, 6000, other)
    assert X.current_config("d", "L", 5000) == other
    assert X.current_config("d", "L", 6001) == builtin_6001  # outside the rule's range
    assert X.current_config("d", "U", 5000) == builtin_u     # the other triangle
    third = (other + 1) % X.num_configs("d")
    X.select_config("d", "L", 5000, 5000, third)  # later and narrower
    assert X.current_config("d", "L", 5000) == third
    assert X.current_config("d", "L", 4999) == other
    X.select_config("d", "L", 0, 1 << 30, -1)  # defers to the built-in rules
    assert X.current_config("d", "L", 5000) == builtin
    X.clear_config()
    assert X.current_config("d", "L", 5000) == builtin


def test_rule_file_round_trip(tmp_path):
    picks = {("s", "L", 100, 900): 3, ("z", "U", 2048, 4096): 1, ("w", "L", 7, 7): 0}
    for (p, u, lo, hi), idx in picks.items():
        X.select_config(p, u, lo, hi, idx)
    path = tmp_path / "rules.json"
    X.save_config(str(path))
    doc = json.loads(path.read_text())  # the file is plain JSON
    assert len(doc["rules"]) == len(picks)
    X.clear_config()
    assert X.load_config(str(path)) == len(picks)
    for (p, u, lo, hi), idx in picks.items():
        for n in (lo, (lo + hi) // 2, hi):
            assert X.current_config(p, u, n) == idx, (p, u, n)


def test_rule_files_refused_or_skipped(tmp_path):
    with pytest.raises(OSError):
        X.load_config(str(tmp_path / "missing.json"))
    bad = tmp_path / "bad.json"
    bad.write_text('{"rules": [ {"prec": "s", ')
    with pytest.raises(ValueError):
        X.load_config(str(bad))
    # a shape that no compiled configuration has, an unknown precision and a
    # rule with a missing key are skipped; the good rule is installed
    ci = X.config_info("d", 2)
    good = {"prec": "d", "uplo": "U", "n_lo": 10, "n_hi": 20, "waves": ci["waves"],
            "cols_per_wave": ci["cols_per_wave"], "stripes": ci["stripes"],
            "nontemporal": ci["nontemporal"], "x_in_lds": ci["x_in_lds"],
            "column_runs": ci["column_runs"]}
    rules = [good, {**good, "waves": 3}, {**good, "prec": "q"},
             {k: v for k, v in good.items() if k != "stripes"}]
    f = tmp_path / "mixed.json"
    f.write_text(json.dumps({"library": "x", "rules": rules}))
    assert X.load_config(str(f)) == 1
    # a rule names a shape; it selects the first configuration of that shape
    first = min(i for i in range(X.num_configs("d")) if X.config_info("d", i) == ci)
    assert X.current_config("d", "U", 15) == first


def test_selection_argument_errors():
    lib = X.library()
    k = X.num_configs("s")
    assert lib.xsymv_select_config(0, b"L", 0, 10, k) == -1      # no such configuration
    assert lib.xsymv_select_config(0, b"L", 0, 10, -2) == -1
    assert lib.xsymv_select_config(0, b"X", 0, 10, 0) == -1      # bad uplo
    assert lib.xsymv_select_config(5, b"L", 0, 10, 0) == -1      # bad precision
    assert lib.xsymv_select_config(0, b"L", 10, 9, 0) == -1      # empty range
    assert lib.xsymv_current_config(7, b"L", 10) == -1
    assert lib.xsymv_save_config(None) == -1 and lib.xsymv_load_config(None) == -1
    # the on-device search refuses bad arguments before touching the device
    assert lib.xsymv_autotune(0, b"L", 0, 0, 10, 3, None, None, None, 0) == -1
    assert lib.xsymv_autotune(0, b"Q", 64, 0, 10, 3, None, None, None, 0) == -1
    assert lib.xsymv_autotune(0, b"L", 64, 0, 10, 0, None, None, None, 0) == -1
    assert lib.xsymv_autotune(9, b"L", 64, 0, 10, 3, None, None, None, 0) == -1


def test_stride_class_choice():
    """A leading dimension whose columns are whole 64-byte lines (class 0)
    and one that is not (class 1) may get different built-in choices at
    large orders; below the orders class 1 was measured on, and for
    precisions without class-1 rules there, the class-0 choice applies."""
    lib = X.library()
    assert X.current_config("s", "L", 1000, 1000) == X.current_config("s", "L", 1000, 1001)
    for p, size in (("s", 4), ("d", 8), ("c", 8), ("z", 16), ("w", 16)):
        for n in (5000, 20000, 32768):
            aligned = n + (-n * size % 64) // size
            assert X.current_config(p, "U", n, aligned) == X.current_config(p, "U", n)
            X.current_config(p, "U", n, aligned + 1)  # a valid index either way
    # a caller rule applies to every leading dimension
    X.select_config("s", "U", 30000, 40000, 3)
    assert X.current_config("s", "U", 32768, 32768) == 3
    assert X.current_config("s", "U", 32768, 32769) == 3
    assert lib.xsymv_current_config_lda(0, b"L", 10, 0) == -1
    assert lib.xsymv_current_config_lda(5, b"L", 10, 10) == -1
    assert lib.xsymv_autotune_lda(0, b"L", 64, 63, 0, 10, 3, None, None, None, 0) == -1
