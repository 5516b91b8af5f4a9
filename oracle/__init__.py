"""CPU oracle for the GGUF quantized matmul -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path never does.

Thin ctypes marshalling over ``qmm_oracle.c``; all arithmetic lives there.
Every function takes and returns NumPy arrays on the host.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

Q4_0, Q5_0, Q8_0, Q4_K, Q6_K, Q8_K = 2, 6, 8, 12, 14, 15
BLOCK = {Q8_0: (32, 34), Q4_K: (256, 144), Q8_K: (256, 292),
         Q4_0: (32, 18), Q5_0: (32, 22), Q6_K: (256, 210)}  # (values, bytes)
ACT_FORMAT = {Q8_0: Q8_0, Q4_K: Q8_K, Q4_0: Q8_0, Q5_0: Q8_0, Q6_K: Q8_K}
WEIGHT_FORMATS = (Q8_0, Q4_K, Q4_0, Q5_0, Q6_K)

_HERE = os.path.dirname(os.path.abspath(__file__))
# QMM_ORACLE_LIB names another build of this oracle's C source: the test that
# plants mistakes in a copy of that source loads its builds this way.
_LIB_PATH = os.environ.get("QMM_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b  # build only when nothing is built
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_f32_to_f16.argtypes = [ctypes.c_float]
    lib.orc_f32_to_f16.restype = ctypes.c_uint16
    lib.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.orc_f16_to_f64.restype = ctypes.c_double
    for name in ("orc_quantize_q8_0", "orc_quantize_q8k", "orc_quantize_q4_k", "orc_quantize_q4_0",
                 "orc_quantize_q5_0", "orc_quantize_q6_k", "orc_quantize_q4_k_search"):
        getattr(lib, name).argtypes = [_p, _i64, _i64, _p]
        getattr(lib, name).restype = None
    for name in ("orc_quantize_q8_0_v", "orc_quantize_q8k_v"):
        getattr(lib, name).argtypes = [_p, _i64, _i64, _p, ctypes.c_int]
        getattr(lib, name).restype = None
    lib.orc_dequantize.argtypes = [ctypes.c_int, _p, _i64, _i64, _p]
    lib.orc_dequantize.restype = None
    for name in ("orc_matmul_a", "orc_matmul_b"):
        getattr(lib, name).argtypes = [ctypes.c_int, _p, _i64, _i64, _p, _i64, _p, _p]
        getattr(lib, name).restype = None
    lib.orc_block_sums.argtypes = [ctypes.c_int, _p, _i64, _i64, _p, _i64, _p]
    lib.orc_block_sums.restype = None
    lib.orc_row_bytes.argtypes = [ctypes.c_int, _i64]
    lib.orc_row_bytes.restype = _i64
    lib.orc_sums_per_row.argtypes = [ctypes.c_int, _i64]
    lib.orc_sums_per_row.restype = _i64
    lib.orc_set_threads.argtypes = [ctypes.c_int]
    lib.orc_set_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert x.ndim == 2
    return x


def set_threads(n: int) -> int:
    """Set the OpenMP thread count (n<=0 queries); returns the count in use."""
    return _load().orc_set_threads(int(n))


def row_bytes(fmt: int, k: int) -> int:
    return int(_load().orc_row_bytes(fmt, k))


def f32_to_f16_bits(v: float) -> int:
    return int(_load().orc_f32_to_f16(float(v)))


def f16_bits_to_f64(h: int) -> float:
    return float(_load().orc_f16_to_f64(int(h)))


def _check_k(fmt: int, k: int):
    qk = BLOCK[fmt][0]
    if k % qk:
        raise ValueError(f"last dim {k} not divisible by block size {qk}")


def quantize(fmt: int, x, variant: int = 0) -> np.ndarray:
    """Quantize rows of x (R x K float32) to `fmt` blocks; returns uint8 (R, row_bytes)."""
    x = _f32(x)
    r, k = x.shape
    _check_k(fmt, k)
    out = np.zeros((r, row_bytes(fmt, k)), dtype=np.uint8)
    lib = _load()
    if fmt == Q8_0:
        lib.orc_quantize_q8_0_v(_ptr(x), r, k, _ptr(out), variant)
    elif fmt == Q8_K:
        lib.orc_quantize_q8k_v(_ptr(x), r, k, _ptr(out), variant)
    elif fmt in (Q4_K, Q4_0, Q5_0, Q6_K):
        assert variant == 0
        name = {Q4_K: "orc_quantize_q4_k", Q4_0: "orc_quantize_q4_0", Q5_0: "orc_quantize_q5_0",
                Q6_K: "orc_quantize_q6_k"}[fmt]
        getattr(lib, name)(_ptr(x), r, k, _ptr(out))
    else:
        raise ValueError(fmt)
    return out


def quantize_q4_k_search(x) -> np.ndarray:
    """Q4_K blocks of the rows of x with the least-squares search for each
    sub-block's scale and min (qmm_oracle.c, orc_quantize_q4_k_search)."""
    x = _f32(x)
    r, k = x.shape
    _check_k(Q4_K, k)
    out = np.zeros((r, row_bytes(Q4_K, k)), dtype=np.uint8)
    _load().orc_quantize_q4_k_search(_ptr(x), r, k, _ptr(out))
    return out


def dequantize(fmt: int, blocks: np.ndarray, k: int) -> np.ndarray:
    """Exact dequantization to float64, shape (R, K)."""
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    rb = row_bytes(fmt, k)
    r = blocks.size // rb
    assert r * rb == blocks.size
    out = np.empty((r, k), dtype=np.float64)
    _load().orc_dequantize(fmt, _ptr(blocks), r, k, _ptr(out))
    return out


def _mm(name: str, fmt: int, w: np.ndarray, n: int, k: int, x):
    x = _f32(x)
    m = x.shape[0]
    assert x.shape[1] == k
    _check_k(fmt, k)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    assert w.size == n * row_bytes(fmt, k)
    y = np.empty((m, n), dtype=np.float64)
    a = np.empty((m, n), dtype=np.float64)
    getattr(_load(), name)(fmt, _ptr(w), n, k, _ptr(x), m, _ptr(y), _ptr(a))
    return y, a


def matmul_a(fmt: int, w: np.ndarray, n: int, k: int, x):
    """Mode (a): f32 activations x dequantized weights, f64 accumulation.
    Returns (y, absacc), both float64 (M, N)."""
    return _mm("orc_matmul_a", fmt, w, n, k, x)


def matmul_b(fmt: int, w: np.ndarray, n: int, k: int, x):
    """Mode (b): row-wise Q8_0/Q8K activations, integer block dots, scaled.
    Returns (y, absacc), both float64 (M, N)."""
    return _mm("orc_matmul_b", fmt, w, n, k, x)


def sums_per_row(fmt: int, k: int) -> int:
    return int(_load().orc_sums_per_row(fmt, k))


def block_sums(fmt: int, w: np.ndarray, n: int, k: int, x) -> np.ndarray:
    """Integer block sums, int64 (M, N, sums_per_row).  Q8_0, Q4_0, Q5_0: S per
    32-block (signed weight values).  Q4_K: per super-block S_0..S_7, sumi,
    summins.  Q6_K: per super-block S_0..S_15 (per 16), sumi."""
    x = _f32(x)
    m = x.shape[0]
    w = np.ascontiguousarray(w, dtype=np.uint8)
    spr = sums_per_row(fmt, k)
    out = np.empty((m, n, spr), dtype=np.int64)
    _load().orc_block_sums(fmt, _ptr(w), n, k, _ptr(x), m, _ptr(out))
    return out
