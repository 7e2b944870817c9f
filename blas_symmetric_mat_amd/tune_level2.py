"""Built-in configuration tables of the other Level-2 products: xGEMV, xTRMV
and xSYR2 / xHER2 (the report's §5 carries its approach to these).

  measure:  python -m blas_symmetric_mat_amd.tune_level2 measure OUT.json
            For each product, precision, variant and one order per size
            class, times every compiled configuration of that precision:
            ``--passes`` passes, each the median over ``--reps`` calls of
            (cache flush + call) minus the median of the flush alone (the
            flush writes 1 GiB and reads it back).  Variants: the
            transposition for xGEMV ('N', 'T', and 'C' for the complex
            types), triangle and transposition for xTRMV (non-unit
            diagonal), the triangle for xSYR2 / xHER2.  Orders: 8192, 16384
            and 32768 (23170 for the 16-byte types), one in each size class
            of the tables.  ``--ops`` and ``--precs`` limit the work and
            ``--append`` adds to an existing record.  Needs a GPU.

  emit:     python -m blas_symmetric_mat_amd.tune_level2 emit IN.json
            Prints the initialisers of gemv_defaults, trmv_defaults and
            syr2_defaults (csrc/xsymv_prec_*.hip): per cell the
            configuration with the least mean time over the passes, 'T' and
            'C' scored together by their summed time (they share a column).

Inputs are drawn on the device: uniform values, matrices scaled by 1/n for
the triangular product so that repeated in-place calls stay bounded, and a
small alpha for the rank-2 update, so no call meets an overflow.
"""
from __future__ import annotations

import argparse
import json
import statistics
import sys

ORDERS = {"s": (8192, 16384, 32768), "d": (8192, 16384, 32768), "c": (8192, 16384, 32768),
          "z": (8192, 16384, 23170), "w": (8192, 16384, 23170)}
OPS = ("gemv", "trmv", "syr2")


def variants(op: str, prec: str) -> list[str]:
    """The measured variants of a product for one precision."""
    tr = "NTC" if prec in "cz" else "NT"
    if op == "gemv":
        return list(tr)
    if op == "trmv":
        return [u + t for u in "LU" for t in tr]
    return ["L", "U"]


def _least(scores: list[float]) -> int:
    return min(range(len(scores)), key=lambda i: (scores[i], i))


def _score(times: dict, keys: list[str], order: int) -> list[float]:
    """Each configuration's time summed over the variants `keys` at `order`
    (the mean over passes per variant)."""
    per = [[statistics.fmean(p) for p in zip(*times[k][str(order)])] for k in keys]
    return [sum(col) for col in zip(*per)]


def tables_from_record(record: dict) -> dict:
    """{op: {prec: table}} with the tables' index layout: gemv [op][class],
    trmv [upper][op][class], syr2 [upper][class]; op 0 is 'N', 1 'T' and
    'C' together."""
    out: dict = {}
    for op, by_prec in record.get("times", {}).items():
        for prec, times in by_prec.items():
            orders = ORDERS[prec]
            t_keys = [t for t in "TC" if (t if op == "gemv" else "L" + t) in times]
            if op == "gemv":
                tab = [[_least(_score(times, ["N"], n)) for n in orders],
                       [_least(_score(times, t_keys, n)) for n in orders]]
            elif op == "trmv":
                tab = [[[_least(_score(times, [u + "N"], n)) for n in orders],
                        [_least(_score(times, [u + t for t in t_keys], n)) for n in orders]]
                       for u in "LU"]
            else:
                tab = [[_least(_score(times, [u], n)) for n in orders] for u in "LU"]
            out.setdefault(op, {})[prec] = tab
    return out


def _cxx(v) -> str:
    return "{" + ", ".join(_cxx(x) for x in v) + "}" if isinstance(v, list) else str(v)


def emit(in_path: str) -> None:
    rec = json.load(open(in_path))
    name = {"gemv": "GemvDefaults", "trmv": "TrmvDefaults", "syr2": "Syr2Defaults"}
    ctype = {"s": "float", "d": "double", "c": "cf32", "z": "cf64", "w": "ddreal"}
    for op, by_prec in tables_from_record(rec).items():
        for prec, tab in by_prec.items():
            print(f"// {op} {prec} (orders {', '.join(map(str, ORDERS[prec]))}; "
                  f"{rec.get('passes', '?')} passes of {rec.get('reps', '?')} calls)")
            print(f"template <> {name[op]} {op}_defaults<{ctype[prec]}>() "
                  f"{{ return {name[op]}{{{_cxx(tab)}}}; }}")


# ------------------------------------------------------------- measurement

def _rand(torch, k, prec, gen, scale):
    if prec == "w":  # (hi, lo) pairs with lo = 0
        t = torch.zeros(k, 2, device="cuda", dtype=torch.float64)
        t[:, 0] = torch.rand(k, generator=gen, device="cuda", dtype=torch.float64) * scale
        return t
    dt = {"s": torch.float32, "d": torch.float64, "c": torch.complex64,
          "z": torch.complex128}[prec]
    if dt.is_complex:
        re = torch.rand(k, generator=gen, device="cuda", dtype=torch.float64)
        im = torch.rand(k, generator=gen, device="cuda", dtype=torch.float64)
        return (torch.complex(re, im) * scale).to(dt)
    return (torch.rand(k, generator=gen, device="cuda", dtype=torch.float64) * scale).to(dt)


def _call_ms(torch, call, flush, reps: int) -> float:
    """Median (flush + call) minus median (flush alone), interleaved."""
    pairs = []
    for _ in range(reps):
        row = []
        for with_call in (False, True):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            flush()
            if with_call:
                call()
            e1.record()
            row.append((e0, e1))
        pairs.append(row)
    torch.cuda.synchronize()
    f_only = statistics.median(a.elapsed_time(b) for (a, b), _ in pairs)
    f_call = statistics.median(a.elapsed_time(b) for _, (a, b) in pairs)
    return f_call - f_only


def _one(X, torch, op, prec, var, n, flush, reps, passes, log):
    gen = torch.Generator(device="cuda").manual_seed(n)
    scalar1 = (1.0, 0.0) if prec == "w" else 1.0
    scalar0 = (0.0, 0.0) if prec == "w" else 0.0
    if op == "gemv":
        A = _rand(torch, n * n, prec, gen, 1.0)
        x = _rand(torch, n, prec, gen, 1.0)
        y = _rand(torch, n, prec, gen, 0.0)
        f = getattr(X, "xgemv_" + prec)
        call = lambda: f(var, n, n, scalar1, A, n, x, 1, scalar0, y, 1)  # noqa: E731
        select, count = X.gemv_select_config, X.gemv_num_configs(prec)
    elif op == "trmv":
        A = _rand(torch, n * n, prec, gen, 1.0 / n)
        x = _rand(torch, n, prec, gen, 1.0)
        f = getattr(X, "xtrmv_" + prec)
        call = lambda: f(var[0], var[1], "N", n, A, n, x, 1)  # noqa: E731
        select, count = X.trmv_select_config, X.trmv_num_configs(prec)
    else:
        A = _rand(torch, n * n, prec, gen, 1.0)
        x = _rand(torch, n, prec, gen, 1.0)
        y = _rand(torch, n, prec, gen, 1.0)
        f = getattr(X, {"s": "xsyr2_s", "d": "xsyr2_d", "c": "xher2_c", "z": "xher2_z",
                        "w": "xsyr2_w"}[prec])
        alpha = (1e-6, 0.0) if prec == "w" else 1e-6
        call = lambda: f(var, n, alpha, x, 1, y, 1, A, n)  # noqa: E731
        select, count = X.syr2_select_config, X.syr2_num_configs(prec)
    res = []
    try:
        for _ in range(passes):
            row = []
            for idx in range(count):
                select(prec, idx)
                for _ in range(2):
                    call()
                row.append(_call_ms(torch, call, flush, reps))
            res.append(row)
    finally:
        select(prec, -1)
    log(f"{op} {prec} {var} n={n}: " +
        ", ".join(f"#{i} {statistics.fmean(c) * 1e3:.1f}" for i, c in enumerate(zip(*res))) + " us")
    del A
    torch.cuda.empty_cache()
    return res


def measure(out_path: str, ops: list[str], precs: str, passes: int, reps: int,
            append: bool) -> None:
    import torch
    import blas_symmetric_mat_amd as X
    X.library()
    rec = json.load(open(out_path)) if append else {}
    rec.update({"device": torch.cuda.get_device_name(0), "passes": passes, "reps": reps})
    rec.setdefault("times", {})
    buf = torch.empty(1 << 28, dtype=torch.float32, device="cuda")

    def flush():
        buf.fill_(1.0)
        buf.sum()

    def log(msg):
        sys.stderr.write(msg + "\n")
        sys.stderr.flush()

    for op in ops:
        for prec in precs:
            times = rec["times"].setdefault(op, {}).setdefault(prec, {})
            for var in variants(op, prec):
                times[var] = {str(n): _one(X, torch, op, prec, var, n, flush, reps, passes, log)
                              for n in ORDERS[prec]}
            with open(out_path, "w") as fh:  # after every precision: a partial record survives
                json.dump(rec, fh, indent=0)
                fh.write("\n")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    m = sub.add_parser("measure")
    m.add_argument("out")
    m.add_argument("--ops", default=",".join(OPS))
    m.add_argument("--precs", default="sdczw")
    m.add_argument("--passes", type=int, default=2)
    m.add_argument("--reps", type=int, default=20)
    m.add_argument("--append", action="store_true")
    e = sub.add_parser("emit")
    e.add_argument("record")
    a = ap.parse_args(argv)
    if a.cmd == "measure":
        ops = [o for o in a.ops.split(",") if o]
        bad = [o for o in ops if o not in OPS]
        if bad or any(p not in ORDERS for p in a.precs):
            ap.error(f"--ops from {OPS}, --precs from sdczw")
        measure(a.out, ops, a.precs, a.passes, a.reps, a.append)
    else:
        emit(a.record)
    return 0


if __name__ == "__main__":
    sys.exit(main())
