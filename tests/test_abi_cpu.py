"""The C ABI library on the CPU: it loads, exports every function that
include/xsymv.h declares, and its host logic (argument checks, quick
returns, configuration tables, tile plans) behaves -- no device work."""
import ctypes
import os
import re

import numpy as np
import pytest

import blas_symmetric_mat_amd as X

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "xsymv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(x(?:symv|hemv|gemv|syr2|her2|trmv)_\w+)\s*\(", text)))


def test_exports_every_declared_function():
    lib = ctypes.CDLL(X.LIB_PATH)
    names = declared_functions()
    assert {"xsymv_s", "xsymv_d", "xhemv_c", "xhemv_z", "xsymv_w", "xgemv_s", "xgemv_d",
            "xgemv_c", "xgemv_z", "xgemv_w", "xsymv_set_workspace", "xsyr2_s", "xsyr2_d",
            "xher2_c", "xher2_z", "xsyr2_w", "xtrmv_s", "xtrmv_d", "xtrmv_c", "xtrmv_z",
            "xtrmv_w", "xtrmv_workspace_bytes", "xsymv_shard_s", "xhemv_shard_z",
            "xsymv_combine_w", "xhemv_combine_c", "xsymv_shard_columns"} <= set(names)
    for nm in names:
        assert hasattr(lib, nm), nm


def test_exports_nothing_undeclared():
    """Every C function the library exports is declared in include/xsymv.h
    (the dynamic symbol table, read with nm; C++ symbols are mangled and
    start with an underscore)."""
    import shutil
    import subprocess
    if shutil.which("nm") is None:
        pytest.skip("nm not available")
    out = subprocess.run(["nm", "-D", "--defined-only", X.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {f[2] for f in (line.split() for line in out.splitlines())
                if len(f) == 3 and f[1] == "T" and not f[2].startswith("_")}
    assert exported and exported == set(declared_functions()), \
        sorted(exported ^ set(declared_functions()))


@pytest.mark.parametrize("prec", ["s", "d", "c", "z", "w"])
def test_argument_errors_before_device_work(prec):
    f = getattr(X, {"s": "xsymv_s", "d": "xsymv_d", "c": "xhemv_c", "z": "xhemv_z",
                    "w": "xsymv_w"}[prec])
    one = (1.0, 0.0) if prec == "w" else 1.0
    zero = (0.0, 0.0) if prec == "w" else 0.0
    cases = [(("Q", 4, one, 8, 4, 8, 1, zero, 8, 1), -1),
             (("L", -3, one, 8, 4, 8, 1, zero, 8, 1), -2),
             (("U", 4, one, None, 4, 8, 1, zero, 8, 1), -4),
             (("U", 4, one, 8, 2, 8, 1, zero, 8, 1), -5),
             (("l", 4, one, 8, 4, None, 1, zero, 8, 1), -6),
             (("u", 4, one, 8, 4, 8, 0, zero, 8, 1), -7),
             (("L", 4, one, 8, 4, 8, 1, zero, None, 1), -9),
             (("L", 4, one, 8, 4, 8, 1, zero, 8, 0), -10),
             (("L", 0, one, 8, 0, 8, 1, zero, 8, 1), -5)]
    for args, code in cases:
        with pytest.raises(X.XsymvError) as e:
            f(*args, stream=0)
        assert e.value.code == code
    # quick returns: n == 0; alpha == 0 and beta == 1 (pointers never touched)
    f("L", 0, one, None, 1, None, 1, zero, None, 1, stream=0)
    f("L", 5, zero, 8, 5, 8, 1, one, 8, 1, stream=0)


def test_config_tables():
    for p in "sdczw":
        k = X.num_configs(p)
        assert k >= 1
        for i in range(k):
            ci = X.config_info(p, i)
            assert ci["panel"] & (ci["panel"] - 1) == 0
            assert 64 % ci["cols_per_wave"] == 0
        with pytest.raises(IndexError):
            X.config_info(p, k)
    X.clear_config()
    builtin = {u: [X.current_config("d", u, n) for n in (150, 201)] for u in "LU"}
    X.select_config("d", "U", 100, 200, 1)
    assert X.current_config("d", "U", 150) == 1
    assert X.current_config("d", "U", 201) == builtin["U"][1]
    assert X.current_config("d", "L", 150) == builtin["L"][0]
    X.select_config("d", "U", 100, 200, -1)  # back to the built-in choice
    assert X.current_config("d", "U", 150) == builtin["U"][0]
    with pytest.raises(ValueError):
        X.select_config("d", "U", 0, 10, 99)
    X.clear_config()


def test_builtin_rules_match_sweep_record():
    """The rules compiled into the library are the ones the committed sweep
    record yields (csrc/xsymv_tuned.inc regenerated from it), and they cover
    every order."""
    import json
    from blas_symmetric_mat_amd import tune_sweep
    here = os.path.dirname(X.LIB_PATH)
    with open(os.path.join(here, "tuned", "mi355x_sweep.json")) as f:
        record = json.load(f)
    rows = tune_sweep.rules_from_record(record)
    assert rows
    X.clear_config()
    size = {"s": 4, "d": 8, "c": 8, "z": 16, "w": 16}

    def lda_of_class(prec, n, cls):
        lda = max(1, n)
        lda += (-lda * size[prec] % 64) // size[prec]  # whole 64-byte lines
        return lda + cls

    for r in rows:
        for n in {r["n_lo"], r["n_hi"], (r["n_lo"] + r["n_hi"]) // 2}:
            lda = lda_of_class(r["prec"], min(n, 1 << 20), r["cls"])
            assert (lda * size[r["prec"]] % 64 != 0) == bool(r["cls"])
            ci = X.config_info(r["prec"], X.current_config(r["prec"], r["uplo"], n, lda))
            assert all(ci[k] == r[k] for k in tune_sweep.SHAPE_KEYS), (r, n)
    for p in "sdczw":
        for u in "LU":
            for cls in (0, 1):
                spans = sorted((r["n_lo"], r["n_hi"]) for r in rows
                               if r["prec"] == p and r["uplo"] == u and r["cls"] == cls)
                if cls == 1 and not spans:
                    continue
                # class 0 covers every order, class 1 a tail of them
                assert spans[-1][1] == 2**31 - 1 and (cls or spans[0][0] == 0)
                assert all(a[1] + 1 == b[0] for a, b in zip(spans, spans[1:]))


def test_workspace_bytes_grow_with_n():
    # a tile-family configuration: its workspace needs no device query (the
    # strip family's depends on how many workgroups the device holds)
    idx = next(i for i in range(X.num_configs("d")) if X.config_info("d", i)["column_runs"] < 4)
    X.select_config("d", "L", 0, 1 << 30, idx)
    try:
        a = X.workspace_bytes("d", "L", 1000)
        b = X.workspace_bytes("d", "L", 4000)
        assert 0 < a < b
        assert X.workspace_bytes("d", "L", 0) == 0
        ci = X.config_info("d", idx)
        P = (4000 + ci["panel"] - 1) // ci["panel"]
        assert b >= P * 4000 * 8
    finally:
        X.clear_config()


@pytest.mark.parametrize("split", [0, 1, 2])
@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("n,R,G", [(1, 64, 7), (100, 64, 3), (1000, 256, 37), (1031, 128, 200),
                                   (4096, 1024, 1792), (10007, 2048, 1792), (5000, 512, 1)])
def test_strip_plan_covers_triangle_once(uplo, n, R, G, split):
    """Emulate the strip kernel's walk: every stored element (i, j) is visited
    by exactly one workgroup, every (strip, column) sum is written once, and
    the segments of each strip are the slots the merge reads."""
    blocks, sb, segb = X.strip_plan(uplo, n, R, G, split)
    NS = (n + R - 1) // R
    assert sb[0] == 0 and segb[0] == 0
    upper = uplo == "U"
    visits = np.zeros((n, n), dtype=np.int32)
    colsum_writes = {}
    slots_of_strip = {}
    prev_end = 0
    for u0, u1, slot, strip in blocks:
        assert u0 == prev_end and u1 >= u0
        prev_end = u1
        u = u0
        while u < u1:
            assert sb[strip] <= u < sb[strip + 1]
            end = min(u1, sb[strip + 1])
            rs0, rs1 = strip * R, min(n, strip * R + R)
            cfirst = rs0 if upper else 0
            for pos in range(u, end):
                j = cfirst + pos - sb[strip]
                assert 0 <= j < n
                rows = np.arange(rs0, rs1)
                st = rows[rows <= j] if upper else rows[rows >= j]
                visits[st, j] += 1
                key = (strip, j)
                colsum_writes[key] = colsum_writes.get(key, 0) + 1
            slots_of_strip.setdefault(strip, []).append(slot)
            u = end
            slot += 1
            strip += 1
    assert prev_end == sb[NS]
    stored = np.triu(np.ones((n, n), bool)) if upper else np.tril(np.ones((n, n), bool))
    assert np.all(visits[stored] == 1) and np.all(visits[~stored] == 0)
    assert all(v == 1 for v in colsum_writes.values())
    for i in range(NS):
        assert slots_of_strip[i] == list(range(segb[i], segb[i + 1]))
    # every column j is summed in exactly the strips the merge reads
    for j in range(0, n, max(1, n // 50)):
        strips = sorted(i for (i, jj) in colsum_writes if jj == j)
        I = j // R
        assert strips == (list(range(0, I + 1)) if upper else list(range(I, NS)))


def test_bench_labels_every_configuration():
    """bench.py names the kernel of whatever configuration runs."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "bench", os.path.join(os.path.dirname(os.path.dirname(X.LIB_PATH)), "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    for p in "sdczw":
        for i in range(X.num_configs(p)):
            for u in "LU":
                assert bench.kernel_label(X, p, u, i).startswith("symv_")


def test_set_workspace_argument_check():
    # a NULL buffer with a size is refused before any device query
    assert X.library().xsymv_set_workspace(None, 64, None) == -2


def test_gemv_workspace_bytes_without_a_device():
    # empty products need no workspace; an unknown precision is refused
    for p in "sdczw":
        assert X.gemv_workspace_bytes(p, "N", 0, 10) == 0
        assert X.gemv_workspace_bytes(p, "T", 10, 0) == 0
    assert X.library().xgemv_workspace_bytes(9, b"N", 10, 10) == 2 ** 64 - 1


def test_config_workgroups_without_a_device():
    # families other than the row strips launch one workgroup per tile (0);
    # out-of-range indices and precisions are refused (-1)
    lib = X.library()
    for p in "sdczw":
        for i in range(X.num_configs(p)):
            if X.config_info(p, i)["column_runs"] < 4:
                assert X.config_workgroups(p, i, "L") == 0
        assert X.config_workgroups(p, X.num_configs(p), "L") == -1
        assert X.config_workgroups(p, -1, "U") == -1
    assert lib.xsymv_config_workgroups(7, 0, b"L") == -1


def test_read_bandwidth_argument_check():
    # below 64 MiB, or no repetition: refused before any allocation
    lib = X.library()
    assert lib.xsymv_read_bandwidth((64 << 20) - 1, 3, None, None, None) == -1
    assert lib.xsymv_read_bandwidth(64 << 20, 0, None, None, None) == -1


@pytest.mark.parametrize("prec", ["s", "d", "c", "z", "w"])
def test_gemv_argument_errors_before_device_work(prec):
    f = getattr(X, "xgemv_" + prec)
    one = (1.0, 0.0) if prec == "w" else 1.0
    zero = (0.0, 0.0) if prec == "w" else 0.0
    # (trans, m, n, alpha, A, lda, x, incx, beta, y, incy); pointers are never touched
    cases = [(("Q", 4, 3, one, 8, 4, 8, 1, zero, 8, 1), -1),
             (("N", -1, 3, one, 8, 4, 8, 1, zero, 8, 1), -2),
             (("T", 4, -1, one, 8, 4, 8, 1, zero, 8, 1), -3),
             (("C", 4, 3, one, None, 4, 8, 1, zero, 8, 1), -5),
             (("n", 4, 3, one, 8, 3, 8, 1, zero, 8, 1), -6),
             (("t", 4, 3, one, 8, 4, None, 1, zero, 8, 1), -7),
             (("c", 4, 3, one, 8, 4, 8, 0, zero, 8, 1), -8),
             (("N", 4, 3, one, 8, 4, 8, 1, zero, None, 1), -10),
             (("N", 4, 3, one, 8, 4, 8, 1, zero, 8, 0), -11),
             (("N", 0, 3, one, 8, 0, 8, 1, zero, 8, 1), -6)]
    for args, code in cases:
        with pytest.raises(X.XsymvError) as e:
            f(*args, stream=0)
        assert e.value.code == code, (args, e.value.code)
    # quick returns: m == 0 or n == 0 (lda >= 1), alpha == 0 and beta == 1
    f("N", 0, 5, one, None, 1, None, 1, zero, None, 1, stream=0)
    f("T", 5, 0, one, None, 5, None, 1, zero, None, 1, stream=0)
    f("N", 5, 4, zero, 8, 5, 8, 1, one, 8, 1, stream=0)


def test_gemv_config_tables():
    for p in "sdczw":
        k = X.gemv_num_configs(p)
        assert k >= 1
        for i in range(k):
            ci = X.gemv_config_info(p, i)
            assert ci["rows_per_strip"] == ci["waves"] * ci["stripes_per_wave"] * 64 * \
                {"s": 4, "d": 2, "c": 2, "z": 1, "w": 1}[p]
        with pytest.raises(IndexError):
            X.gemv_config_info(p, k)
    X.gemv_select_config("d", 1)
    for trans, m, n in (("N", 8, 8), ("T", 40000, 40000), ("C", 1, 1 << 20)):
        assert X.gemv_current_config("d", trans, m, n) == 1
    X.gemv_select_config("d", -1)
    assert X.gemv_current_config("d", "N", 16384, 16384) == _level2_tables()["gemv"]["d"][0][1]
    with pytest.raises(ValueError):
        X.gemv_select_config("s", 99)


def _level2_tables():
    """The built-in tables of xGEMV, xTRMV and the rank-2 update, as the
    committed measurement record gives them (tune_level2 emit)."""
    import json
    from blas_symmetric_mat_amd import tune_level2
    path = os.path.join(os.path.dirname(X.__file__), "tuned", "mi355x_level2.json")
    return tune_level2.tables_from_record(json.load(open(path)))


# The built-in xGEMV choice [0 'N', 1 'T'/'C'][size class of m*n]
GEMV_BUILTIN = _level2_tables()["gemv"]


def test_gemv_builtin_choice_by_transposition_and_size():
    """Size classes by the element count m*n (below 12288^2, below 20000^2,
    larger) and 'T' and 'C' sharing a column; every entry a valid index;
    a forced index applies to every shape; bad arguments give -1."""
    for p, tab in GEMV_BUILTIN.items():
        k = X.gemv_num_configs(p)
        X.gemv_select_config(p, -1)
        for trans in "NTCntc":
            row = tab[0 if trans in "Nn" else 1]
            # class edges: 12288^2 - 1, 12288^2, 20000^2 - 1, 20000^2
            for m, n, cls in ((0, 0, 0), (8192, 8192, 0), (1, 12288 * 12288 - 1, 0),
                              (12288, 12288, 1), (3, 50331648, 1), (16384, 16384, 1),
                              (19999, 20000, 1), (20000, 20000, 2), (32768, 32768, 2),
                              (1, 1 << 30, 2)):
                got = X.gemv_current_config(p, trans, m, n)
                assert got == row[cls], (p, trans, m, n)
                assert 0 <= got < k
        X.gemv_select_config(p, k - 1)
        assert X.gemv_current_config(p, "N", 8, 8) == k - 1
        assert X.gemv_current_config(p, "T", 32768, 32768) == k - 1
        X.gemv_select_config(p, -1)
    lib = X.library()
    assert lib.xgemv_current_config(0, b"X", 8, 8) == -1
    assert lib.xgemv_current_config(0, b"N", -1, 8) == -1
    assert lib.xgemv_current_config(0, b"N", 8, -1) == -1
    assert lib.xgemv_current_config(7, b"N", 8, 8) == -1


@pytest.mark.parametrize("m,n,R,G", [(1, 1, 64, 5), (100, 7, 64, 3), (1000, 77, 256, 37),
                                     (4096, 4096, 1024, 1024), (10007, 333, 2048, 256),
                                     (300, 5000, 512, 1)])
def test_gemv_plan_covers_every_column_once(m, n, R, G):
    """Every (strip, column) pair is in exactly one workgroup's range, each
    range's pieces get consecutive slots, and seg_base lists each strip's
    slots in order (the order the merge reads)."""
    blocks, segb = X.gemv_plan(m, n, R, G)
    NS = (m + R - 1) // R
    seen = np.zeros(NS * n, dtype=np.int32)
    slots_of_strip = {}
    prev_end = 0
    slot_expect = 0
    for u0, u1, slot, strip in blocks:
        assert u0 == prev_end and u1 >= u0
        prev_end = u1
        assert slot == slot_expect
        u, st = u0, strip
        if u0 < u1:
            assert st == u0 // n
        while u < u1:
            e = min(u1, (st + 1) * n)
            seen[u:e] += 1
            slots_of_strip.setdefault(st, []).append(slot_expect)
            slot_expect += 1
            u = e
            st += 1
    assert prev_end == NS * n
    assert np.all(seen == 1)
    assert segb[NS] == slot_expect
    for st in range(NS):
        assert slots_of_strip[st] == list(range(segb[st], segb[st + 1]))


@pytest.mark.parametrize("prec", ["s", "d", "c", "z", "w"])
def test_syr2_argument_errors_before_device_work(prec):
    f = getattr(X, {"s": "xsyr2_s", "d": "xsyr2_d", "c": "xher2_c", "z": "xher2_z",
                    "w": "xsyr2_w"}[prec])
    one = (1.0, 0.0) if prec == "w" else 1.0
    zero = (0.0, 0.0) if prec == "w" else 0.0
    # (uplo, n, alpha, x, incx, y, incy, A, lda); pointers are never touched
    cases = [(("Q", 4, one, 8, 1, 8, 1, 8, 4), -1), (("L", -1, one, 8, 1, 8, 1, 8, 4), -2),
             (("U", 4, one, None, 1, 8, 1, 8, 4), -4), (("u", 4, one, 8, 0, 8, 1, 8, 4), -5),
             (("l", 4, one, 8, 1, None, 1, 8, 4), -6), (("L", 4, one, 8, 1, 8, 0, 8, 4), -7),
             (("L", 4, one, 8, 1, 8, 1, None, 4), -8), (("L", 4, one, 8, 1, 8, 1, 8, 3), -9)]
    for args, code in cases:
        with pytest.raises(X.XsymvError) as e:
            f(*args, stream=0)
        assert e.value.code == code, (args, e.value.code)
    f("L", 0, one, None, 1, None, 1, None, 1, stream=0)   # n == 0
    f("U", 4, zero, 8, 1, 8, 1, 8, 4, stream=0)           # alpha == 0


def test_syr2_config_tables():
    for p in "sdczw":
        k = X.syr2_num_configs(p)
        assert k >= 1
        for i in range(k):
            ci = X.syr2_config_info(p, i)
            assert ci["split"] in (0, 1, 2)
        for uplo in "LUlu":
            for n in (0, 1000, 16384, 32768):
                assert 0 <= X.syr2_current_config(p, uplo, n) < k
    X.syr2_select_config("s", 1)
    assert all(X.syr2_current_config("s", u, n) == 1 for u in "LU" for n in (8, 40000))
    X.syr2_select_config("s", -1)
    assert X.syr2_current_config("s", "L", 8192) == _level2_tables()["syr2"]["s"][0][0]
    with pytest.raises(ValueError):
        X.syr2_select_config("s", 99)
    with pytest.raises(ValueError):
        X.syr2_current_config("s", "Q", 8)
    with pytest.raises(ValueError):
        X.syr2_current_config("s", "L", -1)


# The built-in rank-2 choice [upper][size class of n]
SYR2_BUILTIN = _level2_tables()["syr2"]


def test_syr2_builtin_choice_by_triangle_and_size():
    """Size classes by n (below 12288, below 20000, larger) and their edges."""
    for p, tab in SYR2_BUILTIN.items():
        X.syr2_select_config(p, -1)
        for ui, uplo in enumerate("LU"):
            for n, cls in ((0, 0), (8192, 0), (12287, 0), (12288, 1), (19999, 1), (20000, 2),
                           (32768, 2)):
                assert X.syr2_current_config(p, uplo, n) == tab[ui][cls], (p, uplo, n)


@pytest.mark.parametrize("prec", ["s", "d", "c", "z", "w"])
def test_trmv_argument_errors_before_device_work(prec):
    f = getattr(X, "xtrmv_" + prec)
    # (uplo, trans, diag, n, A, lda, x, incx); pointers are never touched
    cases = [(("Q", "N", "N", 4, 8, 4, 8, 1), -1), (("L", "Q", "N", 4, 8, 4, 8, 1), -2),
             (("U", "T", "Q", 4, 8, 4, 8, 1), -3), (("u", "c", "n", -1, 8, 4, 8, 1), -4),
             (("l", "N", "U", 4, None, 4, 8, 1), -5), (("L", "N", "u", 4, 8, 3, 8, 1), -6),
             (("L", "t", "N", 4, 8, 4, None, 1), -7), (("U", "C", "N", 4, 8, 4, 8, 0), -8)]
    for args, code in cases:
        with pytest.raises(X.XsymvError) as e:
            f(*args, stream=0)
        assert e.value.code == code, (args, e.value.code)
    f("L", "N", "N", 0, None, 1, None, 1, stream=0)   # n == 0


def test_trmv_config_tables():
    for p in "sdczw":
        k = X.trmv_num_configs(p)
        assert k >= 1
        for i in range(k):
            ci = X.trmv_config_info(p, i)
            assert ci["split"] in (0, 1, 2)
            assert ci["rows_per_strip"] == ci["waves"] * ci["stripes_per_wave"] * 64 * \
                {"s": 4, "d": 2, "c": 2, "z": 1, "w": 1}[p]
        for uplo in "LU":
            for trans in "NTC":
                for n in (0, 1000, 16384, 32768):
                    assert 0 <= X.trmv_current_config(p, uplo, trans, n) < k
            # 'T' and 'C' share the built-in choice
            for n in (1000, 16384, 32768):
                assert X.trmv_current_config(p, uplo, "T", n) == \
                    X.trmv_current_config(p, uplo, "C", n)
    keys = [(u, t, n) for u in "LU" for t in "NT" for n in (8192, 16384, 32768)]
    before = {key: X.trmv_current_config("d", *key) for key in keys}
    X.trmv_select_config("d", 2)
    assert all(X.trmv_current_config("d", *key) == 2 for key in keys)
    X.trmv_select_config("d", -1)
    assert before == {key: X.trmv_current_config("d", *key) for key in keys}
    with pytest.raises(ValueError):
        X.trmv_select_config("d", 99)
    with pytest.raises(IndexError):
        X.trmv_config_info("d", 99)
    with pytest.raises(ValueError):
        X.trmv_current_config("d", "Q", "N", 8)
    with pytest.raises(ValueError):
        X.trmv_current_config("d", "L", "Q", 8)
    with pytest.raises(ValueError):
        X.trmv_current_config("d", "L", "N", -1)


# The built-in xTRMV choice [upper][0 'N', 1 'T'/'C'][size class of n]
TRMV_BUILTIN = _level2_tables()["trmv"]


def test_trmv_builtin_choice_by_triangle_transposition_and_size():
    """Size classes by n (below 12288, below 20000, larger), their edges,
    and 'T' and 'C' sharing a column."""
    for p, tab in TRMV_BUILTIN.items():
        X.trmv_select_config(p, -1)
        for ui, uplo in enumerate("LU"):
            for trans in "NTC":
                row = tab[ui][0 if trans == "N" else 1]
                for n, cls in ((0, 0), (1, 0), (8192, 0), (12287, 0), (12288, 1), (19999, 1),
                               (20000, 2), (32768, 2), (46341, 2)):
                    assert X.trmv_current_config(p, uplo, trans, n) == row[cls], (p, uplo, trans, n)


@pytest.mark.parametrize("n,panel,nshards", [(0, 1, 1), (1, 1, 1), (10, 2, 3), (37, 4, 3),
                                             (1000, 64, 8), (100, 7, 5)])
def test_shard_columns_match_the_oracle(n, panel, nshards):
    """The library's dealing of panels agrees with the oracle's."""
    import oracle
    for g in range(nshards):
        assert X.shard_columns(n, panel, nshards, g) == list(
            oracle.shard_columns(n, panel, nshards, g))
    with pytest.raises(ValueError):
        X.shard_columns(10, 0, 2, 0)


@pytest.mark.parametrize("prec", ["s", "d", "c", "z", "w"])
def test_shard_argument_errors_before_device_work(prec):
    f = getattr(X, {"s": "xsymv_shard_s", "d": "xsymv_shard_d", "c": "xhemv_shard_c",
                    "z": "xhemv_shard_z", "w": "xsymv_shard_w"}[prec])
    # (uplo, n, panel, nshards, shard, Aloc, lda, x, incx, p); pointers never touched
    cases = [(("Q", 8, 2, 2, 0, 8, 8, 8, 1, 8), -1), (("L", -1, 2, 2, 0, 8, 8, 8, 1, 8), -2),
             (("L", 8, 0, 2, 0, 8, 8, 8, 1, 8), -3), (("U", 8, 2, 0, 0, 8, 8, 8, 1, 8), -4),
             (("U", 8, 2, 2, 2, 8, 8, 8, 1, 8), -5), (("U", 8, 2, 2, -1, 8, 8, 8, 1, 8), -5),
             (("l", 8, 2, 2, 1, None, 8, 8, 1, 8), -6), (("L", 8, 2, 2, 0, 8, 7, 8, 1, 8), -7),
             (("L", 8, 2, 2, 0, 8, 8, None, 1, 8), -8), (("L", 8, 2, 2, 0, 8, 8, 8, 0, 8), -9),
             (("u", 8, 2, 2, 0, 8, 8, 8, 1, None), -10)]
    for args, code in cases:
        with pytest.raises(X.XsymvError) as e:
            f(*args, stream=0)
        assert e.value.code == code, (args, e.value.code)
    f("L", 0, 1, 1, 0, None, 1, None, 1, None, stream=0)   # n == 0
    g = getattr(X, {"s": "xsymv_combine_s", "d": "xsymv_combine_d", "c": "xhemv_combine_c",
                    "z": "xhemv_combine_z", "w": "xsymv_combine_w"}[prec])
    one = (1.0, 0.0) if prec == "w" else 1.0
    cases = [((-1, 2, one, 8, 4, one, 8, 1), -1), ((4, 0, one, 8, 4, one, 8, 1), -2),
             ((4, 2, one, None, 4, one, 8, 1), -4), ((4, 2, one, 8, 3, one, 8, 1), -5),
             ((4, 2, one, 8, 4, one, None, 1), -7), ((4, 2, one, 8, 4, one, 8, 0), -8)]
    for args, code in cases:
        with pytest.raises(X.XsymvError) as e:
            g(*args, stream=0)
        assert e.value.code == code, (args, e.value.code)
    zero = (0.0, 0.0) if prec == "w" else 0.0
    g(0, 2, one, None, 1, one, None, 1, stream=0)         # n == 0
    g(4, 2, zero, 8, 4, one, 8, 1, stream=0)              # alpha == 0, beta == 1


@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("n,R,G,panel,nshards", [(1000, 256, 37, 16, 3), (4099, 1024, 64, 128, 8),
                                                 (777, 512, 5, 1, 4)])
def test_shard_plan_covers_the_shards_triangle_once(uplo, n, R, G, panel, nshards):
    """For every shard, the strips' local column ranges hold exactly the
    shard's columns with stored rows in each strip (host plan, no device)."""
    for g in range(nshards):
        cols = X.shard_columns(n, panel, nshards, g)
        NS = (n + R - 1) // R
        for st in range(NS):
            rs0, rs1 = st * R, min(n, st * R + R)
            want = [c for c in cols if (c >= rs0 if uplo == "U" else c < rs1)]
            if uplo == "U":
                assert want == cols[len(cols) - len(want):]
            else:
                assert want == cols[:len(want)]


def _simulate_shard(uplo, n, R, Greq, split, panel, nshards, shard, cpg):
    """Walk a shard's plan as the kernel and the merge do and check every
    index they form: local columns in [0, ncol), segment slots in [0, nseg),
    each (strip, column) of the shard's triangle visited once, the diagonal
    pass of an upper segment only on a real column, and every partial the
    merge reads written by some workgroup."""
    cols = X.shard_columns(n, panel, nshards, shard)
    ncol = len(cols)
    blocks, sb, segb, c0 = X.shard_plan(uplo, n, R, Greq, split, panel, nshards, shard)
    if ncol == 0:
        assert len(blocks) == 0
        return
    NS = (n + R - 1) // R
    nseg = int(segb[NS])
    upper = uplo == "U"
    visited = set()
    slot_strip = {}
    for u0, u1, slot, strip in blocks:
        u = int(u0)
        while u < u1:
            assert 0 <= strip < NS
            sb0, useg = int(sb[strip]), min(int(u1), int(sb[strip + 1]))
            rs0, rs1 = strip * R, min(n, strip * R + R)
            coff = (int(c0[strip]) if upper else 0) - sb0
            assert 0 <= slot < nseg and slot not in slot_strip
            slot_strip[int(slot)] = strip
            for g0 in range(u, useg, cpg):
                jg, ng = g0 + coff, min(cpg, useg - g0)
                assert 0 <= jg and jg + ng - 1 < ncol
                for l in range(jg, jg + ng):
                    c = cols[l]
                    assert (c >= rs0) if upper else (c < rs1)  # stored rows in the strip
                    assert (strip, l) not in visited
                    visited.add((strip, l))
            if upper and useg > u:
                assert 0 <= u + coff < ncol
            u = useg
            slot += 1
            strip += 1
    want = {(s, l) for s in range(NS) for l, c in enumerate(cols)
            if ((c >= s * R) if upper else (c < min(n, s * R + R)))}
    assert visited == want
    gloc = {c: l for l, c in enumerate(cols)}
    for i in range(n):
        I = i // R
        s_lo, nrow = int(segb[I]), int(segb[I + 1] - segb[I])
        assert nrow >= 0 and 0 <= s_lo and s_lo + nrow <= nseg
        assert all(slot_strip.get(s) == I for s in range(s_lo, s_lo + nrow))
        if i in gloc:
            strips = range(0, I + 1) if upper else range(I, NS)
            assert all((s, gloc[i]) in visited for s in strips)


@pytest.mark.parametrize("uplo", ["L", "U"])
@pytest.mark.parametrize("n,R", [(1, 1024), (17, 2048), (2111, 2048), (4099, 1024),
                                 (8549, 4096), (3000, 256)])
@pytest.mark.parametrize("panel,nshards", [(1, 3), (128, 8), (1024, 8), (37, 5), (4096, 2)])
def test_shard_plan_indices_in_bounds(uplo, n, R, panel, nshards):
    """Every shard's plan, including strips that hold none of its columns,
    keeps the kernel's and the merge's indices in bounds (the check that a
    strip without columns needs: no slot -1, no column past the local
    matrix)."""
    for Greq, split, cpg in ((1, 0, 4), (7, 1, 16), (64, 0, 8), (512, 1, 16)):
        for g in range(nshards):
            _simulate_shard(uplo, n, R, Greq, split, panel, nshards, g, cpg)


def test_timing_modes():
    """Modes 0, 1 and 2 are accepted (host state only, nothing launched);
    any other is refused."""
    for m in (1, 2, 0, True, False):
        X.timing_enable(m)
    for bad in (3, -1):
        with pytest.raises(ValueError):
            X.timing_enable(bad)
    assert X.library().xsymv_timing_enable(0) == 0
