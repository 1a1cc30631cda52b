"""CPU oracle for the five decode projections — TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package. The GPU library never imports, links or calls it; it shares no
code, headers or tables with it.

What the oracle computes (guide ch. 1 "The problem, the judge and the speed of
light"):
* §1.1: out[i, n] = sum_k x[i, k] * W[n, k] (out = x @ W^T), x BF16 (m x K),
  W BF16 (FP32 for the router), N x K row-major; at <= 8 tokens the unpooler
  only computes and returns its first 1024 rows (the notebook's "The exact
  projection workload" note says the same: the 1,024-row output slice).
* §1.5: the reference is FP64.

The arithmetic lives in linear.c (ascending-k FP64 sums). This wrapper picks
the rows to compute and hands over the raw bits.
"""

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))

# The oracle's own copy of the layer table (guide ch. 1 §1.1): name -> (N, K, W dtype).
_LAYERS = {
    "qkv_gate": (2304, 8192, "bf16"),
    "o": (8192, 1024, "bf16"),
    "pooler": (4096, 8192, "bf16"),
    "unpooler": (8192, 4096, "bf16"),
    "router": (256, 8192, "f32"),
}
# Unpooler slice rule, guide ch. 1 §1.1: at <= 8 tokens only rows 0..1023.
_SLICE_LAYER = "unpooler"
_SLICE_MAX_M = 8
_SLICE_ROWS = 1024

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    from . import build as _build

    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    i64 = ctypes.c_int64
    vp = ctypes.c_void_p
    lib.oracle_linear_bf16w.argtypes = [vp, vp, i64, i64, i64, vp]
    lib.oracle_linear_bf16w.restype = None
    lib.oracle_linear_f32w.argtypes = [vp, vp, i64, i64, i64, vp]
    lib.oracle_linear_f32w.restype = None
    lib.oracle_magnitude_bf16w.argtypes = [vp, vp, i64, i64, i64, vp]
    lib.oracle_magnitude_bf16w.restype = None
    lib.oracle_magnitude_f32w.argtypes = [vp, vp, i64, i64, i64, vp]
    lib.oracle_magnitude_f32w.restype = None
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def threads():
    """OpenMP threads the oracle runs on."""
    return _load().oracle_threads()


def set_threads(n):
    _load().oracle_set_threads(int(n))


def out_cols(layer, m):
    """Columns of out for `layer` at `m` tokens (the unpooler slice rule)."""
    n, _, _ = _LAYERS[layer]
    if layer == _SLICE_LAYER and m <= _SLICE_MAX_M:
        return _SLICE_ROWS
    return n


def matmul_bits(x_bits, w, n_rows=None):
    """FP64 x @ W[:n_rows]^T from raw operands.

    x_bits: uint16 (m x K) BF16 bit patterns. w: uint16 (BF16 bits) or float32,
    shape (N x K). Returns float64 (m x n_rows).
    """
    return _run("linear", x_bits, w, n_rows)


def magnitude_bits(x_bits, w, n_rows=None):
    """FP64 |x| @ |W[:n_rows]|^T: per output, the sum of its terms' magnitudes.

    Same operands and shape as matmul_bits. An FP32 accumulation of the
    products in any order differs from the exact sum by at most a small
    multiple of this value, which the acceptance check uses per element.
    """
    return _run("magnitude", x_bits, w, n_rows)


def _run(kind, x_bits, w, n_rows):
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    if x_bits.ndim != 2 or w.ndim != 2 or x_bits.shape[1] != w.shape[1]:
        raise ValueError("shape mismatch: x %s, W %s" % (x_bits.shape, w.shape))
    m, k = x_bits.shape
    n_rows = w.shape[0] if n_rows is None else int(n_rows)
    if not 0 <= n_rows <= w.shape[0]:
        raise ValueError("n_rows out of range")
    out = np.empty((m, n_rows), dtype=np.float64)
    if m == 0 or n_rows == 0:
        return out
    lib = _load()
    if w.dtype == np.uint16:
        wc = np.ascontiguousarray(w)
        fn = lib.oracle_linear_bf16w if kind == "linear" else lib.oracle_magnitude_bf16w
        fn(x_bits.ctypes.data, wc.ctypes.data, m, n_rows, k, out.ctypes.data)
    elif w.dtype == np.float32:
        wc = np.ascontiguousarray(w)
        fn = lib.oracle_linear_f32w if kind == "linear" else lib.oracle_magnitude_f32w
        fn(x_bits.ctypes.data, wc.ctypes.data, m, n_rows, k, out.ctypes.data)
    else:
        raise TypeError("W must be uint16 BF16 bits or float32, got %s" % w.dtype)
    return out


def _check_layer_operands(layer, w):
    n, k, wdt = _LAYERS[layer]
    if w.shape != (n, k):
        raise ValueError("%s expects W %dx%d, got %s" % (layer, n, k, w.shape))
    if (wdt == "f32") != (w.dtype == np.float32):
        raise TypeError("%s expects %s weights" % (layer, wdt))


def reference(layer, x_bits, w):
    """FP64 reference output of `layer` for BF16 activations `x_bits` (m x K)."""
    _check_layer_operands(layer, w)
    m = x_bits.shape[0]
    return matmul_bits(x_bits, w, out_cols(layer, m))


def magnitude(layer, x_bits, w):
    """Per output of `layer`, the FP64 sum of |x| * |w| over its terms (same shape as reference)."""
    _check_layer_operands(layer, w)
    m = x_bits.shape[0]
    return magnitude_bits(x_bits, w, out_cols(layer, m))


def _rows_of(x_bits, rows):
    rows = np.asarray(rows, dtype=np.int64)
    if rows.ndim != 1:
        raise ValueError("rows must be a 1-D index list")
    m = x_bits.shape[0]
    if rows.size and (rows.min() < 0 or rows.max() >= m):
        raise IndexError("row index out of range 0..%d" % (m - 1))
    return np.ascontiguousarray(x_bits[rows])


def reference_rows(layer, x_bits, w, rows):
    """FP64 reference for a subset of the token rows of an m-row call (sampled
    parity at full size): row j of the result is token rows[j] of
    reference(layer, x_bits, w). The column count follows the call's m, not
    the number of sampled rows (the unpooler slice rule depends on m)."""
    _check_layer_operands(layer, w)
    return matmul_bits(_rows_of(x_bits, rows), w, out_cols(layer, x_bits.shape[0]))


def magnitude_rows(layer, x_bits, w, rows):
    """magnitude() for a subset of token rows, as reference_rows()."""
    _check_layer_operands(layer, w)
    return magnitude_bits(_rows_of(x_bits, rows), w, out_cols(layer, x_bits.shape[0]))
