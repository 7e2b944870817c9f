"""Size sweep of the on-device autotuner and the built-in selection rules.

The report tunes its CUDA kernels per GPU and condenses the results into
per-size rules (§3, Table 3).  This is the MI355X counterpart:

  measure:  python -m blas_symmetric_mat_amd.tune_sweep measure OUT.json
            For every precision, triangle and order of a grid, runs
            ``xsymv_autotune_lda`` (every compiled configuration, median of
            ``--reps`` timed calls on device-generated data, caches flushed
            for matrices under 1 GiB) and records each configuration's median
            time and the winner.  ``--stride-class 1`` measures with
            lda = n + 1 (columns that are not whole 64-byte lines; the grid
            orders are multiples of 64, so lda = n is class 0), and adds the
            size sweep's odd orders (10007 and 32767 for s and d) with
            lda = n, ``--n-min``
            skips the smaller orders, ``--uplos`` limits the triangles, and
            ``--append`` adds the results to an existing record (replacing
            those of the same key), ``--passes`` averages each
            configuration's median over several autotuner passes.  Needs a
            GPU.

  emit:     python -m blas_symmetric_mat_amd.tune_sweep emit IN.json OUT.inc
            Turns a measurement record into the rule rows compiled into the
            library (csrc/xsymv_tuned.inc), per stride class: the winner at
            grid order n_k covers the orders between the geometric midpoints
            with its neighbours; adjacent rows with the same kernel are
            merged.  Class 1 rows cover only the orders that class was
            measured on; elsewhere the library falls back to class 0.

Kernels are recorded by shape (waves, columns per wave, stripes,
non-temporal loads, x in LDS, family), as the JSON rule files of
``xsymv_save_config`` are, so a record stays valid when the configuration
lists are reordered.
"""
from __future__ import annotations

import argparse
import json
import math
import sys
import time

GRID = {
    "s": [64, 128, 256, 512, 1024, 2048, 4096, 8192, 12288, 16384, 24576, 32768],
    "d": [64, 128, 256, 512, 1024, 2048, 4096, 8192, 12288, 16384, 24576, 32768],
    "c": [64, 128, 256, 512, 1024, 2048, 4096, 8192, 12288, 16384, 24576, 32768],
    "z": [64, 128, 256, 512, 1024, 2048, 4096, 8192, 12288, 16384, 24576],
    "w": [64, 128, 256, 512, 1024, 2048, 4096, 8192, 12288, 16384, 24576],
}
# orders measured for stride class 1 only, with lda = n: the odd orders of
# the [SD]SYMV size-sweep workload, whose columns are not whole 64-byte lines
EXTRA_CLASS1 = {"s": [10007, 32767], "d": [10007, 32767]}
ELEM_BYTES = {"s": 4, "d": 8, "c": 8, "z": 16, "w": 16}
SHAPE_KEYS = ("waves", "cols_per_wave", "stripes", "nontemporal", "x_in_lds", "column_runs")
INT_MAX = 2**31 - 1


def _shape(X, prec, idx):
    ci = X.config_info(prec, idx)
    return {k: ci[k] for k in SHAPE_KEYS}


def measure(out_path: str, precs: str, reps: int, grid_max: int | None, cls: int = 0,
            n_min: int = 0, append: bool = False, uplos: str = "LU", passes: int = 1) -> None:
    import os
    import torch
    import blas_symmetric_mat_amd as X

    torch.cuda.init()
    record = {"library": X.version(), "device": torch.cuda.get_device_name(0), "reps": reps,
              "passes": passes, "shapes": {}, "results": []}
    if append and os.path.exists(out_path):
        with open(out_path) as f:
            record = json.load(f)
    for prec in precs:
        shapes = [_shape(X, prec, i) for i in range(X.num_configs(prec))]
        old = record["shapes"].get(prec, [])
        # configurations are only ever appended: earlier indices keep their shapes
        assert shapes[:len(old)] == old, f"configuration list of {prec} was reordered"
        record["shapes"][prec] = shapes
        orders = sorted(set(GRID[prec]) | (set(EXTRA_CLASS1.get(prec, [])) if cls else set()))
        for uplo in uplos:
            for n in orders:
                if (grid_max and n > grid_max) or n < n_min:
                    continue
                # class 1: lda = n where its columns are already not whole
                # 64-byte lines (odd orders), else n + 1
                lda = n if cls and (n * ELEM_BYTES[prec]) % 64 else n + cls
                t0 = time.time()
                # each configuration's median averaged over `passes` autotuner
                # passes: shapes within a per cent of one another are common, and
                # one pass names whichever a noisy run flatters
                runs = []
                for _ in range(passes):
                    X.clear_config()
                    runs.append(X.autotune(prec, uplo, n, reps=reps, lda=lda)[1])
                X.clear_config()
                ms = [sum(t) / len(t) for t in zip(*runs)]
                best = min(range(len(ms)), key=lambda i: ms[i])
                record["results"] = [r for r in record["results"] if
                                     (r["prec"], r["uplo"], r["n"], r.get("cls", 0)) !=
                                     (prec, uplo, n, cls)]
                record["results"].append({"prec": prec, "uplo": uplo, "n": n, "cls": cls,
                                          "best": best, "ms": [round(t, 5) for t in ms]})
                print(f"{prec}{uplo} n={n:6d} lda={lda}: best #{best} {ms[best] * 1e3:9.1f} us "
                      f"(#0 {ms[0] * 1e3:9.1f} us)  [{time.time() - t0:.1f} s]", flush=True)
    with open(out_path, "w") as f:
        json.dump(record, f, indent=None, separators=(",", ":"))


def rules_from_record(record: dict) -> list[dict]:
    """Rule rows (prec, uplo, cls, n_lo, n_hi, shape) from a measurement
    record.  Class 0 rows cover every order; class 1 rows start at the
    geometric midpoint below their smallest measured order (the library
    falls back to class 0 below it)."""
    by_key: dict[tuple[str, str, int], list[dict]] = {}
    for r in record["results"]:
        by_key.setdefault((r["prec"], r["uplo"], r.get("cls", 0)), []).append(r)
    rows = []
    for (prec, uplo, cls), rs in sorted(by_key.items(), key=lambda kv: (kv[0][2], kv[0][:2])):
        rs.sort(key=lambda r: r["n"])
        ns0 = sorted(r["n"] for r in record["results"]
                     if (r["prec"], r["uplo"], r.get("cls", 0)) == (prec, uplo, 0))
        for k, r in enumerate(rs):
            if k > 0:
                lo = math.isqrt(rs[k - 1]["n"] * r["n"]) + 1
            elif cls == 0 or not ns0 or r["n"] <= ns0[0]:
                lo = 0
            else:  # below the first class-1 order: the class-0 grid's midpoint
                prev = max(m for m in ns0 if m < r["n"])
                lo = math.isqrt(prev * r["n"]) + 1
            hi = INT_MAX if k == len(rs) - 1 else math.isqrt(r["n"] * rs[k + 1]["n"])
            shape = record["shapes"][prec][r["best"]]
            row = {"prec": prec, "uplo": uplo, "cls": cls, "n_lo": lo, "n_hi": hi, **shape}
            if rows and all(rows[-1][key] == row[key]
                            for key in ("prec", "uplo", "cls", *SHAPE_KEYS)):
                rows[-1]["n_hi"] = hi
            else:
                rows.append(row)
    return rows


def emit(in_path: str, out_path: str) -> None:
    with open(in_path) as f:
        record = json.load(f)
    rows = rules_from_record(record)
    lines = [f"// Generated by blas_symmetric_mat_amd/tune_sweep.py from {in_path.split('/')[-1]}",
             f"// ({record.get('device', '?')}, {record.get('library', '?')}, "
             f"median of {record.get('reps', '?')} timed calls, averaged over "
             f"{record.get('passes', 1)} autotuner pass(es)).",
             "// {prec, uplo, n_lo, n_hi, waves, cols_per_wave, stripes, nontemporal, "
             "x_in_lds, family[, stride class]}"]
    for r in rows:
        cls = f", {r['cls']}" if r["cls"] else ""
        lines.append("{'%s', '%s', %d, %d, %d, %d, %d, %d, %d, %d%s}," % (
            r["prec"], r["uplo"], r["n_lo"], r["n_hi"], *[r[k] for k in SHAPE_KEYS], cls))
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"{len(rows)} rules -> {out_path}")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    m = sub.add_parser("measure")
    m.add_argument("out")
    m.add_argument("--precs", default="sdczw")
    m.add_argument("--reps", type=int, default=20)
    m.add_argument("--grid-max", type=int, default=None)
    m.add_argument("--stride-class", type=int, choices=(0, 1), default=0)
    m.add_argument("--n-min", type=int, default=0)
    m.add_argument("--append", action="store_true")
    m.add_argument("--uplos", default="LU", choices=("L", "U", "LU"))
    m.add_argument("--passes", type=int, default=1)
    e = sub.add_parser("emit")
    e.add_argument("record")
    e.add_argument("out")
    a = ap.parse_args(argv)
    if a.cmd == "measure":
        measure(a.out, a.precs, a.reps, a.grid_max, a.stride_class, a.n_min, a.append, a.uplos,
                a.passes)
    else:
        emit(a.record, a.out)
    return 0


if __name__ == "__main__":
    sys.exit(main())
