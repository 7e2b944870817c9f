"""Byte and flop accounting for y := alpha*S*x + beta*y.

Flops follow the CUDA-xSYMV report's convention (§4): 2n^2 per product for
the "GFLOPS (2n^2)" figure, every stored element feeding two multiply-adds.
The report's bytes-per-flop figures (§4) count one stored element against
its four real flops (two multiply-adds) for real types, sixteen real flops
(two complex multiply-adds) for complex types, and four double-double
operations for the double-double type.

Algorithmic bytes of one call: the stored triangle n(n+1)/2 elements, x (n),
y read (n, unless beta == 0) and y written (n); workspace traffic, re-reads
of x, padding rows and the unread half of the diagonal tiles are excluded.
"""
from __future__ import annotations

ELEM_BYTES = {"s": 4, "d": 8, "c": 8, "z": 16, "w": 16}
# per stored element: real flops (or double-double ops for 'w') of its two uses
FLOPS_PER_ELEMENT = {"s": 4, "d": 4, "c": 16, "z": 16, "w": 4}

HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E, published peak
FP64_VECTOR_TFLOPS = 78.6        # MI355X published peak
FP32_VECTOR_TFLOPS = 157.3


def bytes_per_flop(prec: str) -> float:
    """The report's B/F of the product: bytes of one stored element over the
    flops it feeds (§4: W 4, D 2, S 1, Z 1, C 0.5)."""
    return ELEM_BYTES[prec] / FLOPS_PER_ELEMENT[prec]


def bandwidth_bound_gflops(prec: str, gbps: float) -> float:
    """Flop rate a bandwidth of ``gbps`` GB/s allows, in the report's flop
    convention for ``prec`` (§4's per-precision ceilings)."""
    return gbps / bytes_per_flop(prec)


def gflops_2n2(n: int, seconds: float) -> float:
    return 2.0 * n * n / seconds / 1e9


def stored_elements(n: int) -> int:
    return n * (n + 1) // 2


def call_bytes(prec: str, n: int, beta_zero: bool) -> int:
    """Algorithmic bytes of one call."""
    vec = n * (2 if beta_zero else 3)
    return ELEM_BYTES[prec] * (stored_elements(n) + vec)


def tile_kernel_bytes(prec: str, n: int) -> int:
    """Algorithmic bytes of the streaming kernel of one call: the stored
    triangle and x."""
    return ELEM_BYTES[prec] * (stored_elements(n) + n)


# ------------------------------------------------------------------ xGEMV
# A general m x n matrix is read whole and each element feeds one
# multiply-add (2 real flops; 8 for complex): the report's comparison point.

def gemv_call_bytes(prec: str, m: int, n: int, trans: str, beta_zero: bool) -> int:
    """Algorithmic bytes of one GEMV call: A (m*n), x, y read (unless
    beta == 0) and y written."""
    lenx, leny = (n, m) if trans in ("N", "n") else (m, n)
    return ELEM_BYTES[prec] * (m * n + lenx + leny * (1 if beta_zero else 2))


def gemv_kernel_bytes(prec: str, m: int, n: int, trans: str) -> int:
    """Algorithmic bytes of the GEMV streaming kernel: A and x."""
    lenx = n if trans in ("N", "n") else m
    return ELEM_BYTES[prec] * (m * n + lenx)


# ------------------------------------------------------------ xSYR2 / xHER2
def syr2_call_bytes(prec: str, n: int) -> int:
    """Algorithmic bytes of one rank-2 update: the stored triangle read and
    written once, x and y read."""
    return ELEM_BYTES[prec] * (2 * stored_elements(n) + 2 * n)


# ------------------------------------------------------------------ xTRMV
def trmv_call_bytes(prec: str, n: int, unit: bool) -> int:
    """Algorithmic bytes of one triangular product: the stored triangle (its
    diagonal only when it is read) read once, x read and written."""
    return ELEM_BYTES[prec] * (stored_elements(n) - (n if unit else 0) + 2 * n)
