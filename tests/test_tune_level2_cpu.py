"""Host logic of the Level-2 tuning tool (tables from a measurement record)."""
import json

from blas_symmetric_mat_amd import tune_level2 as T


def _times(best_by_order, nconf=4, passes=2):
    """A variant's record: configuration `best` fastest at each order."""
    out = {}
    for n, best in best_by_order.items():
        out[str(n)] = [[1.0 + 0.1 * abs(i - best) for i in range(nconf)] for _ in range(passes)]
    return out


def test_variants():
    assert T.variants("gemv", "s") == ["N", "T"]
    assert T.variants("gemv", "z") == ["N", "T", "C"]
    assert T.variants("trmv", "c") == ["LN", "LT", "LC", "UN", "UT", "UC"]
    assert T.variants("syr2", "w") == ["L", "U"]


def test_tables_layout_and_picks():
    o = T.ORDERS["s"]
    rec = {"times": {
        "gemv": {"s": {"N": _times({o[0]: 1, o[1]: 2, o[2]: 3}),
                       "T": _times({o[0]: 0, o[1]: 0, o[2]: 1})}},
        "trmv": {"s": {"LN": _times({o[0]: 3, o[1]: 3, o[2]: 3}),
                       "LT": _times({o[0]: 2, o[1]: 1, o[2]: 0}),
                       "UN": _times({o[0]: 0, o[1]: 1, o[2]: 2}),
                       "UT": _times({o[0]: 1, o[1]: 1, o[2]: 1})}},
        "syr2": {"s": {"L": _times({o[0]: 2, o[1]: 0, o[2]: 1}),
                       "U": _times({o[0]: 3, o[1]: 3, o[2]: 0})}}}}
    tab = T.tables_from_record(rec)
    assert tab["gemv"]["s"] == [[1, 2, 3], [0, 0, 1]]
    assert tab["trmv"]["s"] == [[[3, 3, 3], [2, 1, 0]], [[0, 1, 2], [1, 1, 1]]]
    assert tab["syr2"]["s"] == [[2, 0, 1], [3, 3, 0]]


def test_transposes_scored_together_and_passes_averaged():
    o = T.ORDERS["z"]
    # 'T' alone prefers 0, 'C' alone prefers 2; summed, 1 wins
    t_rec = {str(n): [[1.0, 1.1, 3.0]] for n in o}
    c_rec = {str(n): [[3.0, 1.1, 1.0]] for n in o}
    # 'N': pass 1 prefers 0, pass 2 prefers 1, the mean prefers 1
    n_rec = {str(n): [[1.0, 1.2, 2.0], [2.0, 1.2, 2.0]] for n in o}
    rec = {"times": {"gemv": {"z": {"N": n_rec, "T": t_rec, "C": c_rec}}}}
    assert T.tables_from_record(rec)["gemv"]["z"] == [[1, 1, 1], [1, 1, 1]]


def test_ties_go_to_the_lower_index():
    o = T.ORDERS["d"]
    rec = {"times": {"syr2": {"d": {u: {str(n): [[2.0, 1.0, 1.0]] for n in o} for u in "LU"}}}}
    assert T.tables_from_record(rec)["syr2"]["d"] == [[1, 1, 1], [1, 1, 1]]


def test_emit_prints_initialisers(tmp_path, capsys):
    o = T.ORDERS["w"]
    rec = {"passes": 2, "reps": 20,
           "times": {"syr2": {"w": {"L": _times({o[0]: 0, o[1]: 0, o[2]: 1}, nconf=3),
                                    "U": _times({o[0]: 0, o[1]: 1, o[2]: 1}, nconf=3)}}}}
    p = tmp_path / "rec.json"
    p.write_text(json.dumps(rec))
    T.emit(str(p))
    out = capsys.readouterr().out
    assert "template <> Syr2Defaults syr2_defaults<ddreal>() " \
           "{ return Syr2Defaults{{{0, 0, 1}, {0, 1, 1}}}; }" in out
    assert "orders 8192, 16384, 23170" in out


def test_committed_record_matches_the_compiled_lists():
    """The record behind the built-in tables covers every product, precision,
    variant and order, with one time per compiled configuration of that
    precision, in every pass: a configuration added to or removed from a
    list makes this fail until the record is measured again."""
    import os
    import blas_symmetric_mat_amd as X
    path = os.path.join(os.path.dirname(X.__file__), "tuned", "mi355x_level2.json")
    rec = json.load(open(path))
    count = {"gemv": X.gemv_num_configs, "trmv": X.trmv_num_configs, "syr2": X.syr2_num_configs}
    assert rec["passes"] >= 2 and rec["reps"] >= 10
    for op in T.OPS:
        for prec in "sdczw":
            times = rec["times"][op][prec]
            assert sorted(times) == sorted(T.variants(op, prec)), (op, prec)
            for var, by_order in times.items():
                assert sorted(by_order, key=int) == [str(n) for n in T.ORDERS[prec]]
                for passes in by_order.values():
                    assert len(passes) == rec["passes"]
                    assert all(len(row) == count[op](prec) for row in passes), (op, prec, var)
                    assert all(t > 0 for row in passes for t in row)
