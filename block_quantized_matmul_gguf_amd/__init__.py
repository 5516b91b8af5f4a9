"""GGUF quantized matmul for MI355X (gfx950): thin binding over libqmatmul.so.

y = x . W^T with W stored as GGUF Q8_0, Q4_K, Q4_0, Q5_0 or Q6_K blocks, in the two numerical
forms of the page "同一个 GGUF，CPU 和 Metal 生成的文字不一样" (section 出处):

* ``MODE_F32ACT`` (a): f32 activations, weight blocks dequantized in-kernel;
* ``MODE_QACT`` (b): activation rows quantized to Q8_0 / Q8K first, integer
  block dot products scaled by the block scales;
* ``MODE_DEQUANT``: the same page's third form (section 修法, the
  CANDLE_DEQUANTIZE_ALL switch): weights decoded to f32 once
  (``dequantize_weights``), then a plain f32 matmul (``Plan.run_dequantized``).

This module only marshals arguments: it checks dtypes, devices, contiguity and
sizes of torch tensors, then calls the C ABI (``include/qmatmul.h``) with their
device pointers and the current HIP stream.  Every step of the computation runs
in the library's HIP kernels; there is no other code path, and importing the
module fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

Q4_0, Q5_0, Q8_0, Q4_K, Q6_K, Q8_K = 2, 6, 8, 12, 14, 15
WEIGHT_FORMATS = (Q8_0, Q4_K, Q4_0, Q5_0, Q6_K)
MODE_F32ACT, MODE_QACT, MODE_DEQUANT = 0, 1, 2
OK, EINVAL, EBLOCK, EUNSUPPORTED, ENOMEM, EHIP = 0, 1, 2, 3, 4, 5
BLOCK_VALUES = {Q8_0: 32, Q4_K: 256, Q8_K: 256, Q4_0: 32, Q5_0: 32, Q6_K: 256}
BLOCK_BYTES = {Q8_0: 34, Q4_K: 144, Q8_K: 292, Q4_0: 18, Q5_0: 22, Q6_K: 210}
ACT_FORMAT = {Q8_0: Q8_0, Q4_K: Q8_K, Q4_0: Q8_0, Q5_0: Q8_0, Q6_K: Q8_K}
GEMV_MAX_M = 8

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmatmul.so")

_p, _i64, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int

# name: (restype, argtypes) for every symbol the header declares
SIGNATURES = {
    "qmatmul_create": (_int, [ctypes.POINTER(_p), _int, _i64, _i64, _i64, _int]),
    "qmatmul_run": (_int, [_p, _p, _p, _p, _i64, _p]),
    "qmatmul_destroy": (_int, [_p]),
    "qmatmul_quantize_act": (_int, [_int, _p, _i64, _i64, _p, _p]),
    "qmatmul_quantize_weights": (_int, [_int, _p, _i64, _i64, _p, _p]),
    "qmatmul_run_block_sums": (_int, [_p, _p, _p, _p, _i64, _p]),
    "qmatmul_run_traced": (_int, [_p, _p, _p, _p, _p, _p, _i64, _p]),
    "qmatmul_dequantize_weights": (_int, [_int, _p, _i64, _i64, _p, _p]),
    "qmatmul_run_dequantized": (_int, [_p, _p, _p, _p, _i64, _p]),
    "qmatmul_run_group": (_int, [ctypes.POINTER(_p), _int, ctypes.POINTER(_p), _p, ctypes.POINTER(_p), _i64, _p]),
    "qmatmul_run_noalloc": (_int, [_int, _i64, _i64, _i64, _int, _p, _p, _p, _p]),
    "qmatmul_quantize_q4_k_search": (_int, [_p, _i64, _i64, _p, _p]),
    "qmatmul_check": (_int, [_int, _i64, _i64, _i64, _int]),
    "qmatmul_row_bytes": (_i64, [_int, _i64]),
    "qmatmul_block_sums_per_row": (_i64, [_int, _i64]),
    "qmatmul_workspace_bytes": (_i64, [_int, _i64, _i64, _i64, _int]),
    "qmatmul_status_string": (ctypes.c_char_p, [_int]),
    "qmatmul_last_error": (ctypes.c_char_p, []),
    "qmatmul_version": (_int, []),
}

_lib = None


class QmmError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: status {status} ({status_string(status)}): {message}")
        self.status = status


def lib():
    """The loaded C library (loaded once)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; build it with "
                "`python -c 'import __graft_entry__ as g; g.build()'` from the repository root")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().qmatmul_status_string(status).decode()


def last_error() -> str:
    return lib().qmatmul_last_error().decode()


def _check(status: int, where: str):
    if status != OK:
        raise QmmError(status, where, last_error())


# ------------------------------------------------------------ host-only ----

def check(fmt: int, n: int, k: int, m_max: int, mode: int) -> int:
    """Validate a plan shape without touching the GPU; returns the status code."""
    return int(lib().qmatmul_check(fmt, n, k, m_max, mode))


def row_bytes(fmt: int, k: int) -> int:
    return int(lib().qmatmul_row_bytes(fmt, k))


def block_sums_per_row(fmt: int, k: int) -> int:
    return int(lib().qmatmul_block_sums_per_row(fmt, k))


def workspace_bytes(fmt: int, n: int, k: int, m_max: int, mode: int) -> int:
    return int(lib().qmatmul_workspace_bytes(fmt, n, k, m_max, mode))


# ---------------------------------------------------------- device calls ---

def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtype, shape, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


class Plan:
    """One weight shape and mode: ``Plan(fmt, N, K, M_max, mode)``.

    ``run(w, x)`` computes y = x . W^T.  w: uint8 tensor of N*row_bytes(fmt, K)
    bytes (any shape, contiguous), x: float32 [M, K] with M <= M_max; returns
    (or fills) float32 [M, N].  The plan's workspace is shared by its runs:
    use one plan per stream.
    """

    def __init__(self, fmt: int, n: int, k: int, m_max: int, mode: int):
        self.fmt, self.n, self.k, self.m_max, self.mode = fmt, n, k, m_max, mode
        self._h = ctypes.c_void_p()
        _check(lib().qmatmul_create(ctypes.byref(self._h), fmt, n, k, m_max, mode), "qmatmul_create")

    def _args(self, w, x):
        torch = _torch()
        _need(w, torch.uint8, None, "w")
        if w.numel() != self.n * row_bytes(self.fmt, self.k):
            raise ValueError(f"w has {w.numel()} bytes, expected {self.n * row_bytes(self.fmt, self.k)}")
        _need(x, torch.float32, None, "x")
        if x.dim() != 2 or x.shape[1] != self.k:
            raise ValueError(f"x must be [M, {self.k}], got {tuple(x.shape)}")
        return x.shape[0]

    def run(self, w, x, y=None, stream=None):
        torch = _torch()
        m = self._args(w, x)
        if y is None:
            y = torch.empty((m, self.n), dtype=torch.float32, device=x.device)
        _need(y, torch.float32, (m, self.n), "y")
        _check(lib().qmatmul_run(self._h, _ptr(w), _ptr(x), _ptr(y), m, _stream(stream)), "qmatmul_run")
        return y

    def run_dequantized(self, w_f32, x, y=None, stream=None):
        """Dequantize-all plans: y = x . W^T with W the f32 [N, K] matrix from
        ``dequantize_weights``."""
        torch = _torch()
        _need(w_f32, torch.float32, (self.n, self.k), "w_f32")
        _need(x, torch.float32, None, "x")
        if x.dim() != 2 or x.shape[1] != self.k:
            raise ValueError(f"x must be [M, {self.k}], got {tuple(x.shape)}")
        m = x.shape[0]
        if y is None:
            y = torch.empty((m, self.n), dtype=torch.float32, device=x.device)
        _need(y, torch.float32, (m, self.n), "y")
        _check(lib().qmatmul_run_dequantized(self._h, _ptr(w_f32), _ptr(x), _ptr(y), m, _stream(stream)),
               "qmatmul_run_dequantized")
        return y

    def block_sums(self, w, x, out=None, stream=None):
        torch = _torch()
        m = self._args(w, x)
        spr = block_sums_per_row(self.fmt, self.k)
        if out is None:
            out = torch.empty((m, self.n, spr), dtype=torch.int32, device=x.device)
        _need(out, torch.int32, (m, self.n, spr), "sums")
        _check(lib().qmatmul_run_block_sums(self._h, _ptr(w), _ptr(x), _ptr(out), m, _stream(stream)),
               "qmatmul_run_block_sums")
        return out

    def run_traced(self, w, x, stream=None):
        """Mode (b): the run's own kernels with their integer parts written out.
        Returns (y, sums, act): y float32 [M, N] (bit-equal to ``run``), sums
        int32 [M, N, block_sums_per_row], act uint8 [M, row_bytes of the
        activation format] (canonical Q8_0 or Q8K blocks)."""
        torch = _torch()
        m = self._args(w, x)
        spr = block_sums_per_row(self.fmt, self.k)
        y = torch.empty((m, self.n), dtype=torch.float32, device=x.device)
        sums = torch.empty((m, self.n, spr), dtype=torch.int32, device=x.device)
        act = torch.empty((m, row_bytes(ACT_FORMAT[self.fmt], self.k)), dtype=torch.uint8, device=x.device)
        _check(lib().qmatmul_run_traced(self._h, _ptr(w), _ptr(x), _ptr(y), _ptr(sums), _ptr(act), m,
                                        _stream(stream)), "qmatmul_run_traced")
        return y, sums, act

    def close(self):
        if self._h:
            _check(lib().qmatmul_destroy(self._h), "qmatmul_destroy")
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            if self._h and _lib is not None:
                _lib.qmatmul_destroy(self._h)
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


GROUP_MAX = 8


def run_group(plans, ws, x, ys=None, stream=None):
    """y[i] = x . W[i]^T for plans sharing format, K and mode (one launch per
    four plans at M = 1 where the one-row kernel takes the rows); returns the
    list of outputs."""
    torch = _torch()
    if not 1 <= len(plans) <= GROUP_MAX or len(ws) != len(plans):
        raise ValueError(f"need 1..{GROUP_MAX} plans and as many weight tensors, got {len(plans)} and {len(ws)}")
    m = plans[0]._args(ws[0], x)
    for p, w in zip(plans[1:], ws[1:]):
        p._args(w, x)
    if ys is None:
        ys = [torch.empty((m, p.n), dtype=torch.float32, device=x.device) for p in plans]
    for p, y in zip(plans, ys):
        _need(y, torch.float32, (m, p.n), "y")
    n = len(plans)
    harr = (_p * n)(*[p._h for p in plans])
    warr = (_p * n)(*[_ptr(w) for w in ws])
    yarr = (_p * n)(*[_ptr(y) for y in ys])
    _check(lib().qmatmul_run_group(harr, n, warr, _ptr(x), yarr, m, _stream(stream)), "qmatmul_run_group")
    return ys


NOALLOC_SCRATCH_BYTES = 32 << 20


def run_noalloc(fmt: int, n: int, k: int, mode: int, w, x, y=None, stream=None):
    """y = x . W^T without a plan and without device allocation in the library
    (its workspace is a static device array of NOALLOC_SCRATCH_BYTES per GPU;
    calls that overlap on one GPU race).  Same arguments and values as
    ``Plan(fmt, n, k, M, mode).run(w, x)``; allocates ``y`` here only when it is
    not given."""
    torch = _torch()
    _need(w, torch.uint8, None, "w")
    rb = row_bytes(fmt, k)
    if rb < 0 or w.numel() != n * rb:
        raise ValueError(f"w has {w.numel()} bytes, expected {n} rows of {rb}")
    _need(x, torch.float32, None, "x")
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x must be [M, {k}], got {tuple(x.shape)}")
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=x.device)
    _need(y, torch.float32, (m, n), "y")
    _check(lib().qmatmul_run_noalloc(fmt, n, k, m, mode, _ptr(w), _ptr(x), _ptr(y), _stream(stream)),
           "qmatmul_run_noalloc")
    return y


def quantize_act(act_fmt: int, x, out=None, stream=None):
    """Canonical Q8_0 (34 B / 32) or Q8K (292 B / 256) blocks of the rows of x
    (float32 [M, K] on the GPU); returns uint8 [M, row_bytes]."""
    torch = _torch()
    _need(x, torch.float32, None, "x")
    m, k = x.shape
    rb = row_bytes(act_fmt, k)
    if rb < 0:
        raise ValueError(f"K={k} is not a multiple of the block size of format {act_fmt}")
    if out is None:
        out = torch.empty((m, rb), dtype=torch.uint8, device=x.device)
    _need(out, torch.uint8, (m, rb), "out")
    _check(lib().qmatmul_quantize_act(act_fmt, _ptr(x), m, k, _ptr(out), _stream(stream)), "qmatmul_quantize_act")
    return out


def quantize_weights(fmt: int, w, out=None, stream=None):
    """GGUF blocks of the rows of w (float32 [N, K] on the GPU); returns uint8 [N, row_bytes]."""
    torch = _torch()
    _need(w, torch.float32, None, "w")
    n, k = w.shape
    rb = row_bytes(fmt, k)
    if rb < 0:
        raise ValueError(f"K={k} is not a multiple of the block size of format {fmt}")
    if out is None:
        out = torch.empty((n, rb), dtype=torch.uint8, device=w.device)
    _need(out, torch.uint8, (n, rb), "out")
    _check(lib().qmatmul_quantize_weights(fmt, _ptr(w), n, k, _ptr(out), _stream(stream)), "qmatmul_quantize_weights")
    return out


def quantize_q4_k_search(w, out=None, stream=None):
    """Q4_K blocks of the rows of w (float32 [N, K] on the GPU) with the
    least-squares search for each sub-block's scale and min."""
    torch = _torch()
    _need(w, torch.float32, None, "w")
    n, k = w.shape
    rb = row_bytes(Q4_K, k)
    if rb < 0:
        raise ValueError(f"K={k} is not a multiple of 256")
    if out is None:
        out = torch.empty((n, rb), dtype=torch.uint8, device=w.device)
    _need(out, torch.uint8, (n, rb), "out")
    _check(lib().qmatmul_quantize_q4_k_search(_ptr(w), n, k, _ptr(out), _stream(stream)), "qmatmul_quantize_q4_k_search")
    return out


def dequantize_weights(fmt: int, w, n: int, k: int, out=None, stream=None):
    """f32 [N, K] of GGUF weight blocks w (uint8, N*row_bytes(fmt, K) bytes, on
    the GPU): the exact dequantized values rounded once to f32."""
    torch = _torch()
    _need(w, torch.uint8, None, "w")
    rb = row_bytes(fmt, k)
    if rb < 0:
        raise ValueError(f"K={k} is not a multiple of the block size of format {fmt}")
    if w.numel() != n * rb:
        raise ValueError(f"w has {w.numel()} bytes, expected {n * rb}")
    if out is None:
        out = torch.empty((n, k), dtype=torch.float32, device=w.device)
    _need(out, torch.float32, (n, k), "out")
    _check(lib().qmatmul_dequantize_weights(fmt, _ptr(w), n, k, _ptr(out), _stream(stream)),
           "qmatmul_dequantize_weights")
    return out
