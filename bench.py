#!/usr/bin/env python3
"""Benchmark of the MI355X SYMV/HEMV/WSYMV library (one GPU).

A step is one call y := alpha*S*x + beta*y of the headline workload: SSYMV,
uplo = L, n = lda = 32768, A's lower triangle, x and y uniform[-1, 1],
alpha = beta = 1, seed 32768 (the largest size of the [SD]SYMV sweep).  The
inputs are resident in HBM before timing starts.  `value` is GFLOPS counted
as 2n^2 per call, over K timed steps between two device synchronisations.

Printed as one JSON line (kept short), with:
  roofline      the streaming kernel's algorithmic bytes (stored triangle + x)
                over its average duration, timed with HIP events that the
                library binds to the launch (hipExtLaunchKernel: the kernel's
                own start and end), against the 8 TB/s HBM peak;
                `traffic` and `traffic_ratio` come from the committed
                rocprofv3 counter record when it was taken on the current
                kernel source and configuration, else null;
  stream_read_gbps / copy_gbps  a plain streaming read of 4 GiB, and a plain
                copy of 2 GiB (bytes read plus written), on the same device:
                the measured references beside the specification;
  cpu_baseline  the CPU oracle on the same inputs, on 1 core and on every
                core the process may use (its outputs are independent, so the
                threads change no bit), per workload;
  configs       one row per benchmark workload, [us per call, % of 8 TB/s
                for the call's algorithmic bytes, % for the streaming kernel's
                own bytes over its time, counter traffic / algorithmic bytes or
                null]: C1 SSYMV L n = 1024; C2 DSYMV U n = 8192, lda = 8200,
                beta = 0; C3 the [SD]SYMV sweep, s/d x L/U x n in {2048, 4096,
                8192, 16384, 24576, 32768, 10007, 32767}; C4 CHEMV/ZHEMV L
                n = 16384; C5 WSYMV L n = 8192; CHEMV/ZHEMV/WSYMV L at
                n = 32768 (inputs drawn on the device).  "us per call" is
                what one call adds to a stream, with nothing recorded inside
                the call: the median of (cache flush + call) minus the median
                of (flush alone), 20 of each, interleaved, each between a
                pair of events (the flush: 1 GiB written and read back).  The
                kernel's own time comes from the library's events bound to
                its launch, on flushed calls too; the detail record adds the
                rate of calls back to back;
  rule_check    at the sweep's odd orders (10007, 32767) the built-in
                configuration's time over the on-device autotuner's best;
  other         SGEMV/DGEMV (the report's SYMV-vs-GEMV comparison),
                SSYR2/DSYR2 (against the copy rate), S/D/Z/WTRMV and
                one GPU's share of the product sharded over 8 GPUs.
--detail-json FILE writes every row's full record.

Only one GPU is used: --gpus N with N > 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SYMV GFLOPS (2n^2) and % of peak HBM GB/s at n=32768, fp32/fp64/c/z/DD"
KERNEL_SOURCES = ["blas_symmetric_mat_amd/csrc/xsymv_kernels.hpp",
                  "blas_symmetric_mat_amd/csrc/xsymv_strip.hpp",
                  "blas_symmetric_mat_amd/csrc/xsymv_arith.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
ENTRY = {"s": "xsymv_s", "d": "xsymv_d", "c": "xhemv_c", "z": "xhemv_z", "w": "xsymv_w"}
DTYPE_NAME = {"s": "f32", "d": "f64", "c": "c64", "z": "c128", "w": "dd (f64 pairs)"}


CTYPE = {"s": "float", "d": "double", "c": "cf32", "z": "cf64", "w": "ddreal"}


def kernel_label(X, prec: str, uplo: str, idx: int) -> str:
    """The streaming kernel a configuration launches, with its shape."""
    ci = X.config_info(prec, idx)
    tri = "upper" if uplo == "U" else "lower"
    load = "nt" if ci["nontemporal"] else "cached"
    fam = ci["column_runs"]
    if fam in (4, 5, 6):
        split = {4: "height", 5: "stored+height", 6: "height only"}[fam]
        return (f"symv_strip<{CTYPE[prec]}, {tri}, W={ci['waves']}, "
                f"SW={ci['stripes'] // ci['waves']}, G={ci['cols_per_wave']}, {load}> "
                f"(split: {split})")
    name = {0: "symv_tiles", 1: "symv_runs", 2: "symv_runs", 3: "symv_block"}[fam]
    return (f"{name}<{CTYPE[prec]}, {tri}, W={ci['waves']}, CW={ci['cols_per_wave']}, "
            f"S={ci['stripes']}, {load}>")


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


class Dev:
    """A problem resident on the device."""

    def __init__(self, p):
        import numpy as np
        import torch
        def dev(a):  # host arrays are uploaded; device-drawn tensors are used as they are
            if isinstance(a, torch.Tensor):
                return a
            return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")

        self.p = p
        self.A = dev(p.A)
        self.x = dev(p.x)
        self.y0 = dev(p.y)
        self.y = self.y0.clone()
        import blas_symmetric_mat_amd as X
        self.f = getattr(X, ENTRY[p.prec])

    def call(self):
        p = self.p
        self.f(p.uplo, p.n, p.alpha, self.A, p.lda, self.x, p.incx, p.beta, self.y, p.incy)

    def reset_y(self):
        self.y.copy_(self.y0)


class GemvDev:
    """A general problem resident on the device."""

    def __init__(self, p):
        import numpy as np
        import torch
        import blas_symmetric_mat_amd as X
        self.p = p
        self.A = torch.from_numpy(np.ascontiguousarray(p.A)).to("cuda")
        self.x = torch.from_numpy(np.ascontiguousarray(p.x)).to("cuda")
        self.y = torch.from_numpy(np.ascontiguousarray(p.y)).to("cuda")
        self.f = getattr(X, "xgemv_" + p.prec)

    def call(self):
        p = self.p
        self.f(p.trans, p.m, p.n, p.alpha, self.A, p.lda, self.x, p.incx, p.beta, self.y,
               p.incy)


def measure_gemv_detail(name, p, reps, read_peak=None, flush=None):
    """The general product beside the symmetric one (the report's comparison:
    same streaming machinery, twice the bytes)."""
    from blas_symmetric_mat_amd import roofline as R
    import torch
    import blas_symmetric_mat_amd as X
    log(f"detail: {name}")
    d = GemvDev(p)
    for _ in range(2):
        d.call()
    main = sorted(r[0] for r in time_kernels(d, reps, flush))
    t_main = main[len(main) // 2] * 1e-3
    t_call = call_ms(d, reps, flush)[0] * 1e-3
    bz = beta_is_zero(p)
    call_b = R.gemv_call_bytes(p.prec, p.m, p.n, p.trans, bz)
    ci = X.gemv_config_info(p.prec, X.gemv_current_config(p.prec, p.trans, p.m, p.n))
    out = {"prec": p.prec, "trans": p.trans, "m": p.m, "n": p.n, "lda": p.lda,
           "kernel": (f"gemv_strip<{CTYPE[p.prec]}, {p.trans}, W={ci['waves']}, "
                      f"SW={ci['stripes_per_wave']}, G={ci['cols_per_group']}, "
                      f"{'nt' if ci['nontemporal'] else 'cached'}>"),
           "ms_per_call_median": round(t_call * 1e3, 4),
           "gflops_2mn": round(2.0 * p.m * p.n / t_call / 1e9, 2),
           "hbm_gbps_algorithmic": round(call_b / t_call / 1e9, 1),
           "pct_peak_hbm": round(100 * call_b / t_call / 1e9 / R.HBM_PEAK_GBPS, 1),
           "tile_kernel_gbps": round(R.gemv_kernel_bytes(p.prec, p.m, p.n, p.trans) / t_main
                                     / 1e9, 1),
           "flushed_between_calls": flush is not None, "calls": reps}
    if read_peak:
        out["pct_measured_read_peak"] = round(100 * call_b / t_call / 1e9 / read_peak, 1)
    del d
    torch.cuda.empty_cache()
    return out


def measure_syr2_detail(name, p, reps, read_peak=None, flush=None):
    """The rank-2 update: the stored triangle read and written once."""
    from blas_symmetric_mat_amd import roofline as R
    import numpy as np
    import torch
    import blas_symmetric_mat_amd as X
    log(f"detail: {name}")
    A = torch.from_numpy(np.ascontiguousarray(p.A)).to("cuda")
    x = torch.from_numpy(np.ascontiguousarray(p.x)).to("cuda")
    y = torch.from_numpy(np.ascontiguousarray(p.y)).to("cuda")
    f = getattr(X, {"s": "xsyr2_s", "d": "xsyr2_d", "c": "xher2_c", "z": "xher2_z",
                    "w": "xsyr2_w"}[p.prec])

    class _D:
        def call(self):
            f(p.uplo, p.n, p.alpha, x, p.incx, y, p.incy, A, p.lda)

    d = _D()
    for _ in range(2):
        d.call()
    t_call = call_ms(d, reps, flush)[0] * 1e-3
    b = R.syr2_call_bytes(p.prec, p.n)
    ci = X.syr2_config_info(p.prec, X.syr2_current_config(p.prec, p.uplo, p.n))
    out = {"prec": p.prec, "uplo": p.uplo, "n": p.n, "lda": p.lda,
           "kernel": (f"syr2_strip<{CTYPE[p.prec]}, {'upper' if p.uplo == 'U' else 'lower'}, "
                      f"W={ci['waves']}, SW={ci['stripes_per_wave']}, G={ci['cols_per_group']}, "
                      f"{'nt' if ci['nontemporal'] else 'cached'}>"),
           "ms_per_call_median": round(t_call * 1e3, 4),
           "hbm_gbps_algorithmic": round(b / t_call / 1e9, 1),
           "pct_peak_hbm": round(100 * b / t_call / 1e9 / R.HBM_PEAK_GBPS, 1),
           "bytes": "triangle read + written, x and y", "calls": reps}
    del A
    torch.cuda.empty_cache()
    return out


def measure_trmv_detail(name, p, reps, read_peak=None, flush=None):
    """The triangular product: the stored triangle read once, x read and
    overwritten (a fresh x per call, so every call does the same work)."""
    from blas_symmetric_mat_amd import roofline as R
    import numpy as np
    import torch
    import blas_symmetric_mat_amd as X
    log(f"detail: {name}")
    A = torch.from_numpy(np.ascontiguousarray(p.A)).to("cuda")
    x0 = torch.from_numpy(np.ascontiguousarray(p.x)).to("cuda")
    x = x0.clone()
    f = getattr(X, "xtrmv_" + p.prec)

    class _D:
        def call(self):
            f(p.uplo, p.trans, p.diag, p.n, A, p.lda, x, p.incx)

    def fresh():  # before every call, outside what is timed: x restored
        if flush is not None:
            flush()
        x.copy_(x0)

    d = _D()
    for _ in range(2):
        fresh()
        d.call()
    main = sorted(r[0] for r in time_kernels(d, reps, fresh))
    t_main = main[len(main) // 2] * 1e-3
    t_call = call_ms(d, reps, fresh)[0] * 1e-3
    unit = p.diag in ("U", "u")
    b = R.trmv_call_bytes(p.prec, p.n, unit)
    idx = X.trmv_current_config(p.prec, p.uplo, p.trans, p.n)
    ci = X.trmv_config_info(p.prec, idx)
    out = {"prec": p.prec, "uplo": p.uplo, "trans": p.trans, "diag": p.diag, "n": p.n,
           "lda": p.lda,
           "kernel": (f"trmv_strip<{CTYPE[p.prec]}, {'upper' if p.uplo == 'U' else 'lower'}, "
                      f"{p.trans}, W={ci['waves']}, SW={ci['stripes_per_wave']}, "
                      f"G={ci['cols_per_group']}, {'nt' if ci['nontemporal'] else 'cached'}> "
                      f"(split: {'stored+height' if ci['split'] else 'height'})"),
           "ms_per_call_median": round(t_call * 1e3, 4),
           "hbm_gbps_algorithmic": round(b / t_call / 1e9, 1),
           "pct_peak_hbm": round(100 * b / t_call / 1e9 / R.HBM_PEAK_GBPS, 1),
           "streaming_kernel_gbps": round((b - R.ELEM_BYTES[p.prec] * p.n) / t_main / 1e9, 1),
           "bytes": "stored triangle once, x read and written", "calls": reps}
    if read_peak:
        out["pct_measured_read_peak"] = round(100 * b / t_call / 1e9 / read_peak, 1)
    del A
    torch.cuda.empty_cache()
    return out


def measure_shard_detail(name, p, panel, nshards, reps, read_peak=None, flush=None):
    """One GPU's share of the sharded product at its real shape: every
    shard's call (kernel + ordered merge) on this GPU in turn, its bytes the
    shard's stored elements, x read and the partial written; then the
    rank-ordered combination of the partials.  Each shard's call is timed
    with call_ms, the caches flushed before every call (a shard's share is
    below 1 GiB); the combination's kernel by the events bound to it.  The
    exchange between GPUs is not measured (one GPU)."""
    from blas_symmetric_mat_amd import roofline as R
    import numpy as np
    import torch
    import blas_symmetric_mat_amd as X
    log(f"detail: {name}")
    es = R.ELEM_BYTES[p.prec]
    n = p.n
    x = torch.from_numpy(np.ascontiguousarray(p.x)).to("cuda")
    width = 2 if p.prec == "w" else 1
    P = torch.empty((nshards * n * width,), dtype=x.dtype, device="cuda")
    f = getattr(X, {"s": "xsymv_shard_s", "d": "xsymv_shard_d", "c": "xhemv_shard_c",
                    "z": "xhemv_shard_z", "w": "xsymv_shard_w"}[p.prec])
    shards = []
    for g in range(nshards):
        cols = X.shard_columns(n, panel, nshards, g)
        idx = (np.asarray(cols, dtype=np.int64)[:, None] * p.lda +
               np.arange(p.lda, dtype=np.int64)[None, :]).reshape(-1)
        Aloc = torch.from_numpy(np.ascontiguousarray(p.A[idx])).to("cuda")
        out = P[g * n * width:(g + 1) * n * width]

        class _D:
            def call(self):
                f(p.uplo, n, panel, nshards, g, Aloc, p.lda, x, 1, out)

        d = _D()
        for _ in range(2):
            d.call()
        main = sorted(r[0] for r in time_kernels(d, reps, flush))
        stored = sum((c + 1) if p.uplo in ("U", "u") else (n - c) for c in cols)
        shards.append({"shard": g, "columns": len(cols), "stored_elements": stored,
                       "ms_per_call_median": round(call_ms(d, reps, flush)[0], 4),
                       "kernel_ms_median": round(main[len(main) // 2], 4),
                       "bytes": es * (stored + 2 * n)})
        del Aloc
        torch.cuda.empty_cache()
    slow = max(shards, key=lambda r: r["ms_per_call_median"])
    t = slow["ms_per_call_median"] * 1e-3
    # the rank-ordered combination of the partials
    y = torch.zeros_like(x)
    cb = getattr(X, {"s": "xsymv_combine_s", "d": "xsymv_combine_d", "c": "xhemv_combine_c",
                     "z": "xhemv_combine_z", "w": "xsymv_combine_w"}[p.prec])
    one = (1.0, 0.0) if p.prec == "w" else 1.0
    class _C:
        def call(self):
            cb(n, nshards, one, P, n, one, y, 1)

    for _ in range(2):
        _C().call()
    # the combination's kernel alone (events bound to its launch): timed back
    # to back, a kernel this short measures the host's launch rate instead
    cms = sorted(r[0] for r in time_kernels(_C(), reps))[reps // 2]
    out = {"prec": p.prec, "uplo": p.uplo, "n": n, "panel": panel, "shards": nshards,
           "kernel": (f"symv_strip<{CTYPE[p.prec]}, {'upper' if p.uplo == 'U' else 'lower'}, "
                      f"..., shard> + ordered merge"),
           "slowest_shard": slow["shard"],
           "ms_per_call_median": slow["ms_per_call_median"],
           "hbm_gbps_algorithmic": round(slow["bytes"] / t / 1e9, 1),
           "pct_peak_hbm": round(100 * slow["bytes"] / t / 1e9 / R.HBM_PEAK_GBPS, 1),
           "stored_elements_min_max": [min(r["stored_elements"] for r in shards),
                                       max(r["stored_elements"] for r in shards)],
           "combine_ms_median": round(cms, 4),
           "per_shard_ms": [r["ms_per_call_median"] for r in shards],
           "bytes": "the shard's stored elements, x read, its partial written",
           "exchange": "not measured (one GPU)", "calls": reps}
    if read_peak:
        out["pct_measured_read_peak"] = round(100 * slow["bytes"] / t / 1e9 / read_peak, 1)
    del P, x
    torch.cuda.empty_cache()
    return out


def beta_is_zero(p):
    b = p.beta
    return (b[0] == 0 and b[1] == 0) if isinstance(b, tuple) else complex(b) == 0


def time_kernels(d: Dev, reps: int, flush=None, mode: int = 1):
    """Per-call (main kernel ms, merge ms) from the library's events bound to
    the launches (mode 1), or (call span ms, 0) with no event between the
    call's kernels (mode 2)."""
    import torch
    import blas_symmetric_mat_amd as X
    torch.cuda.synchronize()
    X.timing_read()  # drop stale records
    X.timing_enable(mode)
    try:
        for _ in range(reps):
            if flush is not None:
                flush()
            d.call()
        torch.cuda.synchronize()
        rec = X.timing_read()
    finally:
        X.timing_enable(False)
    return rec


def time_split_and_call(d, reps, flush=None):
    """(sorted main-kernel ms, sorted merge ms, sorted call ms): mode-1 calls
    for the kernels, then as many mode-2 calls for the whole call."""
    rec = time_kernels(d, reps, flush)
    whole = time_kernels(d, reps, flush, mode=2)
    return (sorted(r[0] for r in rec), sorted(r[1] for r in rec), sorted(r[0] for r in whole))


def call_ms(d, reps, flush=None):
    """(ms one call adds to a stream, ms of the flush alone or None), with
    nothing recorded inside the call: events placed in a call put a gap of a
    few microseconds between its kernels.  With a flush: the median of
    (flush + call) minus the median of (flush alone), each between a pair of
    events, the two interleaved, so each call starts on flushed caches right
    after other work.  Without: `reps` calls back to back between one pair of
    events, over `reps`."""
    import statistics
    import torch
    torch.cuda.synchronize()

    def ev():
        return torch.cuda.Event(enable_timing=True)
    if flush is None:
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(reps):
            d.call()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / reps, None
    pairs = []
    for _ in range(reps):
        row = []
        for with_call in (False, True):
            e0, e1 = ev(), ev()
            e0.record()
            flush()
            if with_call:
                d.call()
            e1.record()
            row.append((e0, e1))
        pairs.append(row)
    torch.cuda.synchronize()
    f_only = statistics.median(a.elapsed_time(b) for (a, b), _ in pairs)
    f_call = statistics.median(a.elapsed_time(b) for _, (a, b) in pairs)
    if f_call - f_only <= 0.0:
        # a call lost in the flush's jitter (never seen): more pairs, then,
        # failing that, the call's span from events bound to it (an upper
        # bound: it holds the gap those events put between the kernels)
        if reps < 80:
            return call_ms(d, 4 * reps, flush)
        span = sorted(r[0] for r in time_kernels(d, reps, flush, mode=2))
        return span[len(span) // 2], f_only
    return f_call - f_only, f_only


def host_cores() -> int:
    """Cores this process may run on (at most 16, the share of one GPU)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_time(p, threads: int, min_seconds: float) -> tuple[float, int]:
    """Seconds per oracle call on the problem with ``threads`` threads, over
    as many calls as take ``min_seconds`` (at least one)."""
    import oracle
    lib = oracle.default()
    assert lib.set_threads(threads) == 0
    try:
        reps, total = 0, 0.0
        while total < min_seconds or reps == 0:
            t0 = time.perf_counter()
            lib.symv_problem(p)
            total += time.perf_counter() - t0
            reps += 1
    finally:
        lib.set_threads(1)
    return total / reps, reps


def cpu_baselines(problems: dict, headline: str, min_seconds: float) -> dict:
    """The oracle (plain C) on the same inputs as the GPU rows, on 1 core and
    on every core this process may use, per workload; the headline's 1-core
    figure is `value`."""
    from blas_symmetric_mat_amd import roofline as R
    cores = host_cores()
    per = {}
    for name, p in problems.items():
        t1, r1 = cpu_time(p, 1, min_seconds)
        tn, rn = cpu_time(p, cores, min_seconds)
        per[name] = [round(R.gflops_2n2(p.n, t1), 3), round(R.gflops_2n2(p.n, tn), 3)]
        log(f"cpu {name}: 1 core {t1:.3f} s, {cores} cores {tn:.3f} s")
    h = per[headline]
    return {"value": h[0], "unit": "GFLOPS", "cores": 1, "kind": "oracle",
            "sample": f"full calls on the GPU rows' own inputs, repeated to >= {min_seconds} s; "
                      f"per_config = [GFLOPS on 1 core, on {cores} cores] (OpenMP over rows)",
            "n_cores": {"value": h[1], "cores": cores},
            "per_config": per, "cpu": cpu_model()}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def workload_key(p) -> str:
    """Name of a symmetric problem in the counter record and in
    --profile-workload: <prec>-<uplo>-n<N>[-lda<L>][-beta0]."""
    k = f"{p.prec}-{p.uplo}-n{p.n}"
    if p.lda != p.n:
        k += f"-lda{p.lda}"
    if beta_is_zero(p):
        k += "-beta0"
    return k


def traffic_record(workload: str, kernel: str):
    """The committed counter record of `workload`, if it was taken on the
    current kernel source and the same kernel configuration."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE)).get(workload)
    if not rec or rec.get("kernel_source_digest") != kernel_source_digest():
        return None
    if rec.get("kernel_config") != kernel:
        return None
    return rec


def compact(row: dict) -> list:
    """[us per call, % of 8 TB/s for the call, % for the streaming kernel,
    counter traffic / algorithmic kernel bytes or None]"""
    return [round(row["ms_per_call_median"] * 1e3, 1), row["pct_peak_hbm"],
            row.get("kernel_pct_peak_hbm"), row.get("traffic_ratio")]


def measure_detail(name, p, reps, flush, read_peak=None, quiet=False):
    """One symmetric workload: the call's cost on the stream (call_ms, the
    caches flushed before each call), its streaming kernel and merge from
    the library's events bound to them (median of `reps` flushed calls), and
    the rate of calls back to back without a flush."""
    from blas_symmetric_mat_amd import roofline as R
    import torch
    import blas_symmetric_mat_amd as X
    if not quiet:
        log(f"detail: {name}")
    d = Dev(p)
    for _ in range(2):
        d.call()
    torch.cuda.synchronize()
    small = p.A.nbytes < (1 << 30)
    rec = time_kernels(d, reps, flush)
    main = sorted(r[0] for r in rec)
    merge = sorted(r[1] for r in rec)
    c_ms, f_ms = call_ms(d, reps, flush)
    t_main = main[len(main) // 2] * 1e-3
    t_call = c_ms * 1e-3
    bz = beta_is_zero(p)
    call_b = R.call_bytes(p.prec, p.n, bz)
    kb = R.tile_kernel_bytes(p.prec, p.n)
    label = kernel_label(X, p.prec, p.uplo, X.current_config(p.prec, p.uplo, p.n, p.lda))
    out = {"prec": p.prec, "uplo": p.uplo, "n": p.n, "lda": p.lda,
           "kernel": label,
           "ms_per_call_median": round(t_call * 1e3, 4),
           "flush_ms_median": round(f_ms, 4) if f_ms is not None else None,
           "kernel_ms_median": round(t_main * 1e3, 4),
           "merge_ms_median": round(merge[len(merge) // 2], 4),
           "gflops_2n2": round(R.gflops_2n2(p.n, t_call), 2),
           "hbm_gbps_algorithmic": round(call_b / t_call / 1e9, 1),
           "pct_peak_hbm": round(100 * call_b / t_call / 1e9 / R.HBM_PEAK_GBPS, 1),
           "tile_kernel_gbps": round(kb / t_main / 1e9, 1),
           "kernel_pct_peak_hbm": round(100 * kb / t_main / 1e9 / R.HBM_PEAK_GBPS, 1),
           "flushed_between_calls": True,
           "calls": reps}
    tr = traffic_record(workload_key(p), label)
    out["traffic_bytes"] = tr["bytes_per_launch"] if tr else None
    out["traffic_ratio"] = round(tr["bytes_per_launch"] / kb, 4) if tr else None
    if read_peak:
        out["pct_measured_read_peak"] = round(100 * call_b / t_call / 1e9 / read_peak, 1)
    if p.prec in ("c", "z"):
        out["gflops_8n2_real"] = round(4 * R.gflops_2n2(p.n, t_call), 2)
    # the same call back to back, no flush (100 calls below 1 GiB of matrix,
    # else 20): the rate a loop of calls sustains
    nb = 100 if small else 20
    out["us_per_call_back_to_back"] = round(call_ms(d, nb)[0] * 1e3, 2)
    del d
    torch.cuda.empty_cache()
    return out


def rule_check(cases, reps: int = 20, passes: int = 3) -> dict:
    """For each (prec, uplo, n) with lda = n: the built-in configuration's
    time over the best configuration's, as the on-device autotuner times
    them (flushed caches, events around the call, median of `reps` calls);
    `passes` autotuner passes, each configuration's medians averaged (one
    pass alone favours whichever configuration a noisy run flatters); and
    both indices."""
    import blas_symmetric_mat_amd as X
    out = {}
    for prec, uplo, n in cases:
        X.clear_config()
        builtin = X.current_config(prec, uplo, n, n)
        runs = [X.autotune(prec, uplo, n, reps=reps, lda=n)[1] for _ in range(passes)]
        X.clear_config()
        ms = [sum(v) / len(v) for v in zip(*runs)]
        best = min(range(len(ms)), key=lambda i: ms[i])
        out[f"{prec}-{uplo}-n{n}"] = [round(ms[builtin] / ms[best], 4), builtin, best]
        log(f"rule check {prec}-{uplo}-n{n}: built-in #{builtin}, fastest #{best}")
    return out


def summarize_trace(trace_csv: str, stats_csv: str, command: str,
                    bench_json: str | None = None) -> str:
    """Markdown summary of a rocprofv3 --kernel-trace --stats run: every
    kernel's calls and mean duration from the stats file, and the per-launch
    durations of each (kernel, grid) pair from the trace (a grid size
    identifies the workload a launch belonged to)."""
    import csv
    import statistics
    stats = list(csv.DictReader(open(stats_csv)))
    trace = list(csv.DictReader(open(trace_csv)))
    out = ["# rocprofv3 kernel trace summary", "", "Command (run from the repository root):", "",
           "```", command, "```", "", "## Kernel statistics (rocprofv3 --stats)", "",
           "| kernel | calls | mean us | min us | max us |", "|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        out.append(f"| `{r['Name'][:110]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    # runs: maximal sequences of launches of one (kernel, grid) pair with no
    # launch of another of the library's kernels between them other than
    # merge kernels -- bench.py times its workloads one after another, so a
    # run is one workload's calls even where two workloads share a kernel
    # and a grid
    runs = []
    last = None
    for r in sorted(trace, key=lambda r: int(r["Start_Timestamp"])):
        k = r["Kernel_Name"]
        if "xsymv" not in k:
            continue
        key = (k, int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
        if "merge" in k:
            continue
        if key != last:
            runs.append((key, []))
            last = key
        runs[-1][1].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out += ["", "## Streaming-kernel runs from the trace, in launch order", "",
            "(merge kernels left out; bench.py's workload order: headline, then the "
            "detail rows as listed in its output)", "",
            "| # | kernel | workgroups | threads/wg | launches | mean us | median us |",
            "|---|---|---|---|---|---|---|"]
    for i, ((k, g, wg), d) in enumerate(runs):
        out.append(f"| {i} | `{k[:90]}` | {g // wg} | {wg} | {len(d)} | {statistics.mean(d):.1f} | "
                   f"{statistics.median(d):.1f} |")
    # bench.py runs the headline first among the products (after the read and
    # copy references, whose kernels are not counted here): `warmup` calls,
    # `steps` timed calls, then `steps` calls timed kernel by kernel -- the
    # first warmup + 2*steps launches of the first streaming kernel launched
    # (later workloads may launch the same kernel on the same grid)
    import re
    def flag(name, default):
        m = re.search(r"--%s[ =](\d+)" % name, command)
        return int(m.group(1)) if m else default
    nhead = flag("warmup", 5) + 2 * flag("steps", 50)
    mains = {}
    for r in sorted(trace, key=lambda r: int(r["Start_Timestamp"])):
        k = r["Kernel_Name"]
        if "xsymv::symv_" in k and "merge" not in k:
            mains.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if mains:
        k, d = next(iter(mains.items()))  # insertion order = order of first launch
        head = d[:nhead]
        timed = head[-flag("steps", 50):]
        out += ["", "## Headline workload (SSYMV L n = 32768)", "",
                f"The first {len(head)} launches of `{k[:90]}`: mean "
                f"{statistics.mean(head):.1f} us, median {statistics.median(head):.1f} us, "
                f"min {min(head):.1f} us, max {max(head):.1f} us.  bench.py's "
                "`roofline.launch_ms_mean` is the mean of the last `steps` of these, "
                "timed with HIP events bound to the launches (hipExtLaunchKernel) on the "
                "launch stream; in the trace those "
                f"{len(timed)} launches average {statistics.mean(timed):.1f} us."]
        if bench_json:
            line = open(bench_json).read().strip().splitlines()[-1]
            roof = json.loads(line)["roofline"]
            ev = roof["launch_ms_mean"] * 1e3
            out += ["", f"The bench line of this profiled run: `launch_ms_mean` {ev:.1f} us "
                        f"({100 * (ev / statistics.mean(timed) - 1):+.1f} % against the "
                        "trace), `achieved` "
                        f"{roof['achieved']} GB/s, `frac` {roof['frac']}."]
    return "\n".join(out) + "\n"


# Workloads of the counter runs (--pmc-workloads), in launch order, drawn on
# the device: C1, C2, C3 at n = 32768 (both triangles, fp32 and fp64), C4,
# C5, and CHEMV/ZHEMV/WSYMV at n = 32768.
PMC_WORKLOADS = ["s-L-n32768", "s-L-n1024", "d-U-n8192-lda8200-beta0", "s-U-n32768",
                 "d-L-n32768", "d-U-n32768", "c-L-n16384", "z-L-n16384", "w-L-n8192",
                 "c-L-n32768", "z-L-n32768", "w-L-n32768"]
PMC_CALLS = 3


def run_pmc_workloads(calls: int) -> None:
    """Every PMC workload `calls` times, one after another, then a plain
    1 GiB elementwise kernel of known traffic (1 GiB read, 1 GiB written)
    that scales the counters."""
    import torch
    for name in PMC_WORKLOADS:
        d = Dev(profile_problem(name))
        for _ in range(calls):
            d.call()
        torch.cuda.synchronize()
        del d
        torch.cuda.empty_cache()
        log(f"pmc workload {name}: {calls} calls")
    a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.neg(a, out=b)
    torch.cuda.synchronize()


def summarize_pmc(fetch_csv: str, write_csv: str, command: str, calls: int = PMC_CALLS) -> dict:
    """Per-launch HBM traffic of the streaming kernel of every PMC workload
    from two rocprofv3 --pmc runs of `--pmc-workloads` (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads
    for the plain 1 GiB elementwise kernel at the end of the run.  The
    streaming-kernel dispatches come in PMC_WORKLOADS order, `calls` each."""
    import csv
    import statistics
    import blas_symmetric_mat_amd as X

    def dispatches(path):
        rows = list(csv.DictReader(open(path)))
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        return rows

    f, w = dispatches(fetch_csv), dispatches(write_csv)
    gib = float(1 << 30)
    calf = [float(r["Counter_Value"]) for r in f if "neg_kernel" in r["Kernel_Name"]]
    calw = [float(r["Counter_Value"]) for r in w if "neg_kernel" in r["Kernel_Name"]]
    if len(calf) != 1 or len(calw) != 1:
        raise ValueError("calibration kernel not found exactly once")
    fetch_scale = gib / (calf[0] * 1024)
    write_scale = gib / (calw[0] * 1024)

    def mains(rows):
        return [r for r in rows if "xsymv::symv_strip<" in r["Kernel_Name"]]

    mf, mw = mains(f), mains(w)
    if len(mf) != len(PMC_WORKLOADS) * calls or len(mw) != len(mf):
        raise ValueError(f"expected {len(PMC_WORKLOADS) * calls} streaming launches, "
                         f"got {len(mf)} / {len(mw)}")
    out = {}
    digest = kernel_source_digest()
    for k, name in enumerate(PMC_WORKLOADS):
        fr, wr = mf[k * calls:(k + 1) * calls], mw[k * calls:(k + 1) * calls]
        fb = statistics.mean(float(r["Counter_Value"]) for r in fr) * 1024 * fetch_scale
        wb = statistics.mean(float(r["Counter_Value"]) for r in wr) * 1024 * write_scale
        parts = name.split("-")
        prec, uplo, n = parts[0], parts[1], int(parts[2][1:])
        lda = next((int(x[3:]) for x in parts[3:] if x.startswith("lda")), n)
        kcfg = kernel_label(X, prec, uplo, X.current_config(prec, uplo, n, lda))
        from blas_symmetric_mat_amd import roofline as R
        kb = R.tile_kernel_bytes(prec, n)
        out[name] = {"kernel": fr[0]["Kernel_Name"], "kernel_config": kcfg,
                     "grid_threads": int(fr[0]["Grid_Size"]),
                     "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
                     "bytes_per_launch": round(fb + wb),
                     "algorithmic_bytes_per_launch": kb,
                     "traffic_ratio": round((fb + wb) / kb, 4),
                     "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
                     "launches": calls, "kernel_source_digest": digest, "command": command}
    return out


def summarize_calls(trace_csv: str, name: str, command: str, events_json: str | None = None) -> str:
    """Markdown breakdown of a `--profile-workload NAME --calls N --flush
    [--read-probe]` run under rocprofv3 --kernel-trace.  That run makes 2
    warm-up calls, N flushed calls timed with the library's events in mode 1
    (bound to each kernel), N in mode 2 (bound to the call's first start and
    last end) and N with no library events (bench.py's per-call protocol:
    flush + call against flush alone); per group, the medians of the
    streaming kernel, the gap to its merge, the merge and the span from the
    kernel's start to the merge's end, against the algorithmic bytes; then
    the plain streaming read of the matrix's size (xsymv_read_bandwidth,
    every layout) and, when the run wrote it, what the timings measured."""
    import csv
    import re
    import statistics
    from blas_symmetric_mat_amd import roofline as R
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    lib = [r for r in rows if "xsymv::" in r["Kernel_Name"]]
    first = next(r["Kernel_Name"] for r in lib if "merge" not in r["Kernel_Name"])
    calls = []
    for i, r in enumerate(lib):
        if r["Kernel_Name"] == first and i + 1 < len(lib) and "merge" in lib[i + 1]["Kernel_Name"]:
            m = lib[i + 1]
            s0, e0 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            s1, e1 = int(m["Start_Timestamp"]), int(m["End_Timestamp"])
            calls.append(((e0 - s0) / 1e3, (s1 - e0) / 1e3, (e1 - s1) / 1e3, (e1 - s0) / 1e3,
                          m["Kernel_Name"]))
    if not calls:
        raise ValueError(f"no streaming launch followed by a merge for {first}")
    mc = re.search(r"--calls[ =](\d+)", command)
    nc = int(mc.group(1)) if mc else (len(calls) - 2) // 3
    groups = [("warm-up, no timing, no flush", calls[:2]),
              ("flushed, events bound to each kernel (mode 1)", calls[2:2 + nc]),
              ("flushed, events bound to the call (mode 2)", calls[2 + nc:2 + 2 * nc]),
              ("flushed, no library events (per-call protocol)", calls[2 + 2 * nc:2 + 3 * nc])]
    groups = [(g, c) for g, c in groups if c]
    parts = name.split("-")
    prec, n = parts[0], int(parts[2][1:])
    kb = R.tile_kernel_bytes(prec, n)
    cb = R.call_bytes(prec, n, "beta0" in parts)

    def med(cs, k):
        return statistics.median(c[k] for c in cs)
    out = [f"# Per-call breakdown, {name}", "", "Command (run from the repository root):", "",
           "```", command, "```", "",
           f"Streaming kernel `{first}`, merge `{calls[0][4]}`.  Medians from the kernel trace, "
           "us; the flush writes 1 GiB and reads it back.", "",
           "| calls | n | streaming kernel | gap to the merge | merge | span |",
           "|---|---|---|---|---|---|"]
    for g, cs in groups:
        out.append(f"| {g} | {len(cs)} | {med(cs, 0):.1f} | {med(cs, 1):.1f} | {med(cs, 2):.1f} | "
                   f"{med(cs, 3):.1f} |")
    last = groups[-1][1]
    out += ["", f"Algorithmic bytes: kernel {kb:,} (stored triangle + x), call {cb:,}.  In the "
                f"last group the kernel moves {kb / med(last, 0) / 1e3:.0f} GB/s "
                f"({100 * kb / med(last, 0) / 1e3 / R.HBM_PEAK_GBPS:.1f} % of 8 TB/s) and the "
                f"call span {cb / med(last, 3) / 1e3:.0f} GB/s "
                f"({100 * cb / med(last, 3) / 1e3 / R.HBM_PEAK_GBPS:.1f} %)."]
    probes = {}
    for r in rows:
        k = r["Kernel_Name"]
        if k.startswith("void read_probe"):
            key = (k.split("(")[0][5:], int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]),
                   int(r["Workgroup_Size_X"]))
            probes.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if probes:
        pb = max(kb, 64 << 20)  # the probe reads at least 64 MiB
        where = ("larger than the 256 MB last-level cache" if pb > (256 << 20) else
                 "it fits in the 256 MB last-level cache, so these reads are served from there")
        out += ["", f"Plain streaming read of {pb:,} B (the matrix's bytes, at least 64 MiB), every "
                    "layout of xsymv_read_bandwidth, same process, no flush between launches "
                    f"({where}):", "",
                "| kernel | workgroups | threads/wg | launches | median us |", "|---|---|---|---|---|"]
        best = None
        for (k, g, wg), d in probes.items():
            m = statistics.median(d)
            best = m if best is None or m < best else best
            out.append(f"| `{k}` | {g} | {wg} | {len(d)} | {m:.1f} |")
        if pb == kb:
            out += ["", f"Fastest layout: {best:.1f} us; the streaming kernel (last group) takes "
                        f"{med(last, 0) / best:.3f} x that."]
        else:
            out += ["", f"Fastest layout: {best:.1f} us (more bytes than the call reads: no ratio)."]
    if events_json and os.path.exists(events_json):
        ev = json.load(open(events_json))
        out += ["", "What the timings measured in the same run: mode-1 events, streaming "
                    f"kernel {ev['kernel_us_median']:.1f} us; mode-2 events, whole call "
                    f"{ev['call_us_median']:.1f} us"]
        if "call_us_differential" in ev:
            out[-1] += (f"; flush + call minus flush alone (medians of {ev['calls']}, flush "
                        f"{ev['flush_us_median']:.1f} us), {ev['call_us_differential']:.1f} us")
        out[-1] += "."
    return "\n".join(out) + "\n"


def traffic_markdown(rec: dict) -> str:
    """Markdown table of a counter record (profiles/traffic_counters.json)."""
    any_rec = next(iter(rec.values()))
    out = ["# HBM traffic of the streaming kernel, per workload", "",
           "Commands (repository root; one counter per run, then the summary):", "", "```",
           any_rec["command"].replace("<COUNTER>", "FETCH_SIZE"),
           any_rec["command"].replace("<COUNTER>", "WRITE_SIZE"),
           "python3 bench.py --summarize-pmc gpurun_out/pmc_FETCH_SIZE/run_counter_collection.csv "
           "gpurun_out/pmc_WRITE_SIZE/run_counter_collection.csv \"<command>\"",
           "python3 bench.py --traffic-md > profiles/symv_strip_traffic_by_workload.md", "```", "",
           f"`--pmc-workloads` runs each workload {any_rec['launches']} times (inputs drawn on "
           "the device), then one plain elementwise kernel (torch.neg, float32) that reads "
           "1 GiB and writes 1 GiB.  On this MI355X FETCH_SIZE reads half of the bytes it "
           f"fetches (scale {any_rec['fetch_scale']}) and WRITE_SIZE all of them (scale "
           f"{any_rec['write_scale']}); every reading is scaled so.  Algorithmic bytes: the "
           "stored triangle once plus x.  Kernel source digest when measured: "
           f"{any_rec['kernel_source_digest']} (bench.py reports `traffic` only while the "
           "sources still have it and the same configuration is chosen).", "",
           "| workload | kernel configuration | fetched B | written B | total / algorithmic |",
           "|---|---|---|---|---|"]
    for name, r in rec.items():
        out.append(f"| {name} | `{r['kernel_config']}` | {r['fetch_bytes_per_launch']:,} | "
                   f"{r['write_bytes_per_launch']:,} | {r['traffic_ratio']:.4f} |")
    out += ["", "The writes are the row partials (one slice of a strip per segment) and the "
                "column partials (one per strip and column) that the merge reads back; the "
                "fetches above the algorithmic bytes are x re-read per segment, the row-strip "
                "x slices and lines shared by neighbouring columns or cut by the leading "
                "dimension."]
    return "\n".join(out) + "\n"


def profile_problem(name: str):
    """The problem a profiler run times: <s|d|c|z|w>-<L|U>-n<N>[-lda<L>][-beta0],
    drawn on the device (lda = n and the scalars of
    workloads.metric_order_on_device unless given)."""
    from blas_symmetric_mat_amd import workloads as W
    parts = name.split("-")
    ok = len(parts) >= 3 and parts[0] in W.PRECISIONS and parts[1] in ("L", "U") and \
        parts[2].startswith("n") and parts[2][1:].isdigit()
    lda, beta0 = None, False
    for extra in parts[3:] if ok else []:
        if extra.startswith("lda") and extra[3:].isdigit():
            lda = int(extra[3:])
        elif extra == "beta0":
            beta0 = True
        else:
            ok = False
    if not ok:
        sys.exit(f"--profile-workload: expected <s|d|c|z|w>-<L|U>-n<N>[-lda<L>][-beta0], "
                 f"got {name}")
    prec, uplo, n = parts[0], parts[1], int(parts[2][1:])
    p = W.metric_order_on_device(prec, n, uplo)
    if lda is not None or beta0:
        kw = {"alpha": p.alpha, "beta": p.beta}
        if beta0:
            kw["beta"] = (0.0, 0.0) if prec == "w" else 0.0
        del p
        p = W.draw_on_device(prec, uplo, n, lda, seed=n, name=name, **kw)
    return p


C3_ORDERS = [2048, 4096, 8192, 16384, 24576, 32768, 10007, 32767]


def make_flush():
    """Flush the caches (4 MB L2 per XCD, 256 MB MALL) before a timed call:
    write a 1 GiB buffer, then read it back, so that they hold clean lines
    of the buffer and the call pays no write-back of dirty ones."""
    import torch
    buf = torch.empty(1 << 28, dtype=torch.float32, device="cuda")

    def flush():
        buf.fill_(1.0)
        buf.sum()
    return flush, buf


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-detail", action="store_true", help="headline workload only")
    ap.add_argument("--detail-reps", type=int, default=20)
    ap.add_argument("--detail-json", metavar="FILE",
                    help="also write every workload's full record to FILE")
    ap.add_argument("--cpu-seconds", type=float, default=1.0,
                    help="minimum CPU time per oracle timing (per workload and core count)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-rule-check", action="store_true")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("TRACE_CSV", "STATS_CSV", "COMMAND"),
                    help="print a markdown summary of a rocprofv3 kernel trace and exit")
    ap.add_argument("--bench-json", help="with --summarize-trace: the profiled run's bench "
                    "output, whose launch_ms_mean the summary sets beside the trace's")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COMMAND"),
                    help="write profiles/traffic_counters.json from two rocprofv3 --pmc "
                         "runs of --pmc-workloads and exit")
    ap.add_argument("--traffic-md", action="store_true",
                    help="print profiles/traffic_counters.json as a markdown table and exit")
    ap.add_argument("--pmc-workloads", action="store_true",
                    help="for rocprofv3 --pmc: run every counter workload a few times, "
                         "then the calibration kernel, and exit")
    ap.add_argument("--profile-workload", metavar="NAME",
                    help="for a profiler: run only NAME's call --calls times and exit, "
                         "printing nothing else (NAME = <s|d|c|z|w>-<L|U>-n<N>[-lda<L>]"
                         "[-beta0]: inputs drawn on the device)")
    ap.add_argument("--calls", type=int, default=5)
    ap.add_argument("--flush", action="store_true",
                    help="with --profile-workload: flush the caches before each call and time "
                         "the calls with the library's events (written to --events-json)")
    ap.add_argument("--read-probe", action="store_true",
                    help="with --profile-workload: then a plain streaming read of the "
                         "matrix's algorithmic bytes (every layout)")
    ap.add_argument("--events-json", metavar="FILE")
    ap.add_argument("--summarize-calls", nargs=3, metavar=("TRACE_CSV", "NAME", "COMMAND"),
                    help="per-call breakdown of a --profile-workload run and exit")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(*args.summarize_trace, bench_json=args.bench_json), end="")
        return
    if args.traffic_md:
        print(traffic_markdown(json.load(open(TRAFFIC_FILE))), end="")
        return
    if args.summarize_calls:
        print(summarize_calls(*args.summarize_calls, events_json=args.events_json), end="")
        return
    if args.summarize_pmc:
        rec = summarize_pmc(*args.summarize_pmc)
        with open(TRAFFIC_FILE, "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
        print(json.dumps({k: v["traffic_ratio"] for k, v in rec.items()}, indent=1))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); "
              f"asked for --gpus {args.gpus}, WORLD_SIZE={world}", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import blas_symmetric_mat_amd as X
    from blas_symmetric_mat_amd import roofline as R
    from blas_symmetric_mat_amd import workloads as W

    if args.profile_workload:
        p = profile_problem(args.profile_workload)
        d = Dev(p)
        if args.flush:
            flush, _buf = make_flush()
            for _ in range(2):
                d.call()
            ks, _, cs = time_split_and_call(d, args.calls, flush)
            diff, f_only = call_ms(d, args.calls, flush)
            ev = {"calls": len(cs), "kernel_us_median": ks[len(ks) // 2] * 1e3,
                  "call_us_median": cs[len(cs) // 2] * 1e3,
                  "call_us_differential": diff * 1e3, "flush_us_median": f_only * 1e3}
            log(f"{args.profile_workload}: {args.calls} flushed calls, events {ev}")
            if args.events_json:
                with open(args.events_json, "w") as fh:
                    json.dump(ev, fh)
            del _buf
        else:
            for _ in range(args.calls):
                d.call()
        torch.cuda.synchronize()
        if args.read_probe:
            nb = R.tile_kernel_bytes(p.prec, p.n)
            del d
            torch.cuda.empty_cache()
            log(f"read probe of {nb} B: {X.read_bandwidth(max(nb, 64 << 20), 10)}")
        log(f"{args.profile_workload}: {args.calls} calls done")
        return
    if args.pmc_workloads:
        run_pmc_workloads(PMC_CALLS)
        return

    if not os.path.exists(X.LIB_PATH):
        from blas_symmetric_mat_amd import build as B
        B.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name}, {props.multi_processor_count} CUs, {X.version()}")

    # measured references beside the specification (first: the machine, then
    # the workload)
    rd_med, rd_best = X.read_bandwidth(4 << 30, reps=10)
    cp_med, _ = X.copy_bandwidth(2 << 30, reps=10)

    # ------------------------------------------------------------- headline
    t0 = time.perf_counter()
    p = W.symv_sweep("s", "L", 32768)
    log(f"headline inputs generated in {time.perf_counter() - t0:.1f} s")
    d = Dev(p)
    cfg_idx = X.current_config("s", "L", p.n)
    for _ in range(args.warmup):
        d.call()
    torch.cuda.synchronize()
    # timed region: K steps between two synchronisations
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        d.call()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    value = R.gflops_2n2(p.n, ms_per_step * 1e-3)
    call_b = R.call_bytes("s", p.n, False)
    log(f"headline: {ms_per_step:.4f} ms/step, {value:.1f} GFLOPS, wall {wall:.3f} s")

    # per-kernel durations from the library's events (same stream)
    rec = time_kernels(d, args.steps)
    main_ms = float(np.mean([r[0] for r in rec]))
    merge_ms = float(np.mean([r[1] for r in rec]))
    kb = R.tile_kernel_bytes("s", p.n)
    achieved = kb / (main_ms * 1e-3) / 1e9
    workload = f"ssymv-L-n{p.n}"
    kname = kernel_label(X, "s", "L", cfg_idx)
    tr = traffic_record(workload_key(p), kname)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": R.HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(achieved / R.HBM_PEAK_GBPS, 4),
            "traffic": tr["bytes_per_launch"] if tr else None,
            "traffic_ratio": round(tr["bytes_per_launch"] / kb, 4) if tr else None,
            "kernel": kname, "launch_ms_mean": round(main_ms, 4),
            "merge_ms_mean": round(merge_ms, 4),
            "algorithmic_bytes_per_launch": kb}
    del d
    torch.cuda.empty_cache()

    out = {"metric": METRIC, "value": round(value, 2), "unit": "GFLOPS", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "data": "synthetic",
           "config": {"workload": workload, "n": p.n, "lda": p.lda, "uplo": "L",
                      "alpha": 1.0, "beta": 1.0, "seed": p.n, "distribution": "uniform[-1,1]"},
           "hbm_gbps_algorithmic": round(call_b / (ms_per_step * 1e-3) / 1e9, 1),
           "pct_peak_hbm": round(100 * call_b / (ms_per_step * 1e-3) / 1e9 / R.HBM_PEAK_GBPS, 2),
           "roofline": roof}

    out["stream_read_gbps"] = round(rd_med, 1)
    out["copy_gbps"] = round(cp_med, 1)
    out["pct_measured_read_peak"] = round(100 * out["hbm_gbps_algorithmic"] / rd_med, 2)
    roof["frac_of_measured_read"] = round(achieved / rd_med, 4)
    log(f"references: read {rd_med:.0f} GB/s, copy {cp_med:.0f}")

    cpu_problems = {"C3 s-L-n32768": p}
    detail = {}
    if not args.no_detail:
        flush, flush_buf = make_flush()
        configs = {}

        def sym(key, prob, keep_for_cpu=False):
            row = measure_detail(key, prob, args.detail_reps, flush, rd_med, quiet=True)
            detail[key] = row
            configs[key] = compact(row)
            if keep_for_cpu:
                cpu_problems[key] = prob

        t0 = time.perf_counter()
        sym("C1 s-L-n1024", W.ssymv_lower_n1024(), True)
        sym("C2 d-U-n8192-lda8200-beta0", W.dsymv_upper_n8192_lda8200_beta0(), True)
        for prec in "sd":
            for uplo in "LU":
                for n in C3_ORDERS:
                    key = f"C3 {prec}-{uplo}-n{n}"
                    sym(key, p if key == "C3 s-L-n32768" else W.symv_sweep(prec, uplo, n))
                log(f"C3 {prec}{uplo}: {len(C3_ORDERS)} orders [{time.perf_counter() - t0:.0f} s]")
        del p
        sym("C4 c-L-n16384", W.hemv_lower_n16384("c"), True)
        sym("C4 z-L-n16384", W.hemv_lower_n16384("z"), True)
        sym("C5 w-L-n8192", W.wsymv_lower_n8192(), True)
        for prec in "czw":
            sym(f"{prec}-L-n32768-devdraw", W.metric_order_on_device(prec, 32768))
        log(f"C1-C5: {len(configs)} workloads [{time.perf_counter() - t0:.0f} s]")
        out["configs"] = configs

        other = {}
        for name, make in [("sgemv-N-n32768", lambda: W.gemv_square("s", "N", 32768)),
                           ("sgemv-T-n32768", lambda: W.gemv_square("s", "T", 32768)),
                           ("dgemv-N-n32768", lambda: W.gemv_square("d", "N", 32768))]:
            detail[name] = measure_gemv_detail(name, make(), args.detail_reps, rd_med, flush)
        for name, make in [
                ("ssyr2-L-n32768", lambda: W.make_syr2_problem("s", "L", 32768, seed=32768)),
                ("dsyr2-U-n32768", lambda: W.make_syr2_problem("d", "U", 32768, seed=32768))]:
            row = measure_syr2_detail(name, make(), args.detail_reps, rd_med, flush)
            row["pct_of_copy"] = round(100 * row["hbm_gbps_algorithmic"] / cp_med, 1)
            detail[name] = row
        for name, make in [
                ("strmv-L-N-n32768",
                 lambda: W.make_trmv_problem("s", "L", "N", "N", 32768, seed=32768)),
                ("dtrmv-U-T-n32768",
                 lambda: W.make_trmv_problem("d", "U", "T", "N", 32768, seed=32768)),
                ("ztrmv-L-C-n16384",
                 lambda: W.make_trmv_problem("z", "L", "C", "N", 16384, seed=16384)),
                ("wtrmv-U-N-n16384",
                 lambda: W.make_trmv_problem("w", "U", "N", "N", 16384, seed=16384))]:
            detail[name] = measure_trmv_detail(name, make(), args.detail_reps, rd_med, flush)
        for name, make in [("ssymv-L-n32768-8shards", lambda: W.symv_sweep("s", "L", 32768)),
                           ("dsymv-U-n32768-8shards", lambda: W.symv_sweep("d", "U", 32768))]:
            detail[name] = measure_shard_detail(name, make(), 256, 8, args.detail_reps, rd_med,
                                                flush)
        for name in ("sgemv-N-n32768", "sgemv-T-n32768", "dgemv-N-n32768", "ssyr2-L-n32768",
                     "dsyr2-U-n32768", "strmv-L-N-n32768", "dtrmv-U-T-n32768",
                     "ztrmv-L-C-n16384", "wtrmv-U-N-n16384"):
            r = detail[name]
            other[name] = [round(r["ms_per_call_median"] * 1e3, 1), r["pct_peak_hbm"]]
        for name in ("ssyr2-L-n32768", "dsyr2-U-n32768"):
            other[name].append(detail[name]["pct_of_copy"])
        for name in ("ssymv-L-n32768-8shards", "dsymv-U-n32768-8shards"):
            r = detail[name]
            other[name] = [round(r["ms_per_call_median"] * 1e3, 1), r["pct_peak_hbm"],
                           round(r["combine_ms_median"] * 1e3, 1)]
        # the report's point: SYMV reads half the bytes of GEMV on the same
        # order, so takes about half the time
        other["symv_over_gemv_time"] = {
            "s-L/sgemv-N": round(ms_per_step / detail["sgemv-N-n32768"]["ms_per_call_median"], 3),
            "d-L/dgemv-N": round(detail["C3 d-L-n32768"]["ms_per_call_median"] /
                                 detail["dgemv-N-n32768"]["ms_per_call_median"], 3)}
        out["other"] = other
        del flush_buf
        torch.cuda.empty_cache()
        if not args.no_rule_check:
            t0 = time.perf_counter()
            out["rule_check"] = rule_check([(pr, u, n) for pr in "sd" for u in "LU"
                                            for n in (10007, 32767)])
            log(f"rule check [{time.perf_counter() - t0:.0f} s]")
    else:
        del p

    # -------------------------------------------------------------- CPU leg
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baselines(cpu_problems, "C3 s-L-n32768", args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    out["kernel_source_digest"] = kernel_source_digest()
    if args.detail_json:
        with open(args.detail_json, "w") as fh:
            json.dump({"detail": detail, "line": out}, fh, indent=1)
    print(json.dumps(out, separators=(",", ":")))


if __name__ == "__main__":
    main()
