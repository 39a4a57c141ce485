"""Test infrastructure: the CPU oracle for y = FP16(FP16(x @ weight.T) + b).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (``linear_amd``) never does, and this
package imports nothing from ``linear_amd``.

The arithmetic lives in ``oracle.c`` (plain C, built with gcc, no fast-math).
This module only builds it, loads it with ctypes and marshals numpy arrays.
Binary16 values travel as ``numpy.uint16`` words (their IEEE bit patterns).

The definition followed is the numerical contract of "tensor programs, part 1",
section "One Program and One Numerical Contract": FP32 accumulation of exact
products in any order (the oracle takes sequential k), the projection rounded to
FP16 before the bias add, and the Inductor capture's epilogue (widen both to
f32, add, round to f16).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
          "-Wall", "-Wextra", "-shared", "-fPIC"]


def build(src: str = _SRC, out: str = _LIB, extra: list[str] | None = None) -> str:
    """Compile the oracle with gcc into a shared library and return its path."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *(extra or []), src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def _declare(lib: ctypes.CDLL) -> ctypes.CDLL:
    lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_f16.restype = ctypes.c_uint16
    lib.oracle_f16_to_f32_array.argtypes = [_u16p, _f32p, _i64]
    lib.oracle_f16_to_f32_array.restype = None
    lib.oracle_f32_to_f16_array.argtypes = [_f32p, _u16p, _i64]
    lib.oracle_f32_to_f16_array.restype = None
    lib.oracle_bias_epilogue.argtypes = [ctypes.c_uint16, ctypes.c_uint16]
    lib.oracle_bias_epilogue.restype = ctypes.c_uint16
    lib.oracle_bias_epilogue_array.argtypes = [_u16p, _u16p, _u16p, _i64]
    lib.oracle_bias_epilogue_array.restype = None
    lib.oracle_linear_f16.argtypes = [_u16p, _i64, _u16p, _i64, _u16p, _u16p, _u16p, _i64,
                                      _i64, _i64, _i64, ctypes.c_int]
    lib.oracle_linear_f16.restype = ctypes.c_int
    lib.oracle_linear_f16_points.argtypes = [_u16p, _i64, _u16p, _i64, _u16p, _i64, _i64p, _i64p,
                                             _i64, _u16p, _u16p, _f64p, _f64p, ctypes.c_int]
    lib.oracle_linear_f16_points.restype = None
    lib.oracle_linear.argtypes = [ctypes.c_int, _u16p, _i64, _u16p, _i64, _u16p, _u16p, _u16p, _f32p, _i64,
                                  _i64, _i64, _i64, ctypes.c_int]
    lib.oracle_linear.restype = ctypes.c_int
    lib.oracle_linear_points.argtypes = [ctypes.c_int, _u16p, _i64, _u16p, _i64, _u16p, _i64, _i64p, _i64p,
                                         _i64, _u16p, _u16p, _f32p, _f64p, _f64p, ctypes.c_int]
    lib.oracle_linear_points.restype = None
    lib.oracle_band.argtypes = [ctypes.c_int, _u16p, _i64, _u16p, _i64, _i64, _i64, _i64, _f64p, _f64p,
                                ctypes.c_int]
    lib.oracle_band.restype = ctypes.c_int
    lib.oracle_f64_to_elem.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.oracle_f64_to_elem.restype = ctypes.c_uint16
    _i32p = ctypes.POINTER(ctypes.c_int32)
    lib.oracle_epilogue.argtypes = [ctypes.c_int, _i32p, ctypes.c_int, _u16p, _u16p, _u16p, _u16p, _u16p, _i64]
    lib.oracle_epilogue.restype = None
    lib.oracle_unary_array.argtypes = [ctypes.c_int, ctypes.c_int, _u16p, _u16p, _i64]
    lib.oracle_unary_array.restype = None
    lib.oracle_grouped.argtypes = [ctypes.c_int, _u16p, _i64, _i64, _u16p, _i64, _u16p, _u16p, _u16p, _f32p, _i64,
                                   _i64, _i64, _i64, _i64, _i64, ctypes.c_int]
    lib.oracle_grouped.restype = ctypes.c_int
    lib.oracle_indexed.argtypes = [ctypes.c_int, _u16p, _i64, _u16p, _i64, _i64, _i32p, _u16p, _f32p, _i64,
                                   _i64, _i64, _i64, _i64, ctypes.c_int]
    lib.oracle_indexed.restype = None
    lib.oracle_indexed_band.argtypes = [ctypes.c_int, _u16p, _i64, _u16p, _i64, _i64, _i32p, _f64p, _f64p,
                                        _i64, _i64, _i64, _i64]
    lib.oracle_indexed_band.restype = None
    lib.oracle_bf16_to_f32_array.argtypes = [_u16p, _f32p, _i64]
    lib.oracle_bf16_to_f32_array.restype = None
    lib.oracle_f32_to_bf16_array.argtypes = [_f32p, _u16p, _i64]
    lib.oracle_f32_to_bf16_array.restype = None
    lib.oracle_bias_epilogue_elem_array.argtypes = [ctypes.c_int, _u16p, _u16p, _u16p, _i64]
    lib.oracle_bias_epilogue_elem_array.restype = None
    lib.oracle_band_f64.argtypes = [_u16p, _i64, _u16p, _i64, _i64, _i64, _i64, _f64p, _f64p,
                                    ctypes.c_int]
    lib.oracle_band_f64.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


_lib_cache: dict[str, ctypes.CDLL] = {}


def load(path: str = _LIB) -> ctypes.CDLL:
    """Load (building first if absent or older than the source) the oracle library."""
    if path in _lib_cache:
        return _lib_cache[path]
    if path == _LIB and (not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC)):
        build()
    lib = _declare(ctypes.CDLL(path))
    _lib_cache[path] = lib
    return lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


F16 = 0
BF16 = 1

# Epilogue steps ("The Graph IR", op table: ContractionEpilogue)
EPI_BIAS = 1
EPI_RESIDUAL = 2
EPI_MUL = 3
EPI_SILU = 4
EPI_GELU_TANH = 5
EPI_GELU_ERF = 6
UNARY_EXP = 7
UNARY_ERF = 8


def _as_words(a) -> np.ndarray:
    """Accept a numpy float16/uint16 array or a CPU torch float16/bfloat16 tensor; return uint16 words."""
    if hasattr(a, "detach"):  # torch tensor, CPU
        a = a.detach().contiguous().view(dtype=__import__("torch").int16).numpy().view(np.uint16)
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("binary16 data must be float16 or uint16 words, got %s" % a.dtype)
    return np.ascontiguousarray(a)


class Oracle:
    """ctypes facade over one build of oracle.c (the default build, or a variant)."""

    def __init__(self, path: str = _LIB):
        self.lib = load(path)

    # -- conversions -------------------------------------------------------------
    def f16_to_f32(self, h) -> np.ndarray:
        h = _as_words(h)
        out = np.empty(h.shape, np.float32)
        self.lib.oracle_f16_to_f32_array(_ptr(h, ctypes.c_uint16), _ptr(out, ctypes.c_float), h.size)
        return out

    def f32_to_f16(self, f) -> np.ndarray:
        f = np.ascontiguousarray(np.asarray(f, dtype=np.float32))
        out = np.empty(f.shape, np.uint16)
        self.lib.oracle_f32_to_f16_array(_ptr(f, ctypes.c_float), _ptr(out, ctypes.c_uint16), f.size)
        return out

    def bf16_to_f32(self, h) -> np.ndarray:
        h = _as_words(h)
        out = np.empty(h.shape, np.float32)
        self.lib.oracle_bf16_to_f32_array(_ptr(h, ctypes.c_uint16), _ptr(out, ctypes.c_float), h.size)
        return out

    def f32_to_bf16(self, f) -> np.ndarray:
        f = np.ascontiguousarray(np.asarray(f, dtype=np.float32))
        out = np.empty(f.shape, np.uint16)
        self.lib.oracle_f32_to_bf16_array(_ptr(f, ctypes.c_float), _ptr(out, ctypes.c_uint16), f.size)
        return out

    def bias_epilogue(self, proj16, b16, elem: int = F16) -> np.ndarray:
        p = _as_words(proj16)
        b = _as_words(b16)
        assert p.shape == b.shape
        out = np.empty(p.shape, np.uint16)
        if elem == F16:
            self.lib.oracle_bias_epilogue_array(_ptr(p, ctypes.c_uint16), _ptr(b, ctypes.c_uint16),
                                                _ptr(out, ctypes.c_uint16), p.size)
        else:
            self.lib.oracle_bias_epilogue_elem_array(elem, _ptr(p, ctypes.c_uint16), _ptr(b, ctypes.c_uint16),
                                                     _ptr(out, ctypes.c_uint16), p.size)
        return out

    # -- the layer ---------------------------------------------------------------
    def linear(self, x, w, b=None, nthreads: int = 0, elem: int = F16, sums: bool = False):
        """Return (y, proj) as uint16 [M,N] arrays (and the unrounded FP32 sums as a
        third float32 array if sums).  x: [M,K], w: [N,K], b: [N] or None.
        elem: F16 (binary16) or BF16 (bfloat16) operand and output words."""
        x = _as_words(x)
        w = _as_words(w)
        M, K = x.shape
        N, K2 = w.shape
        assert K == K2, (x.shape, w.shape)
        bb = None if b is None else _as_words(b)
        if bb is not None:
            assert bb.shape == (N,)
        y = np.zeros((M, N), np.uint16)
        proj = np.zeros((M, N), np.uint16)
        y32 = np.zeros((M, N), np.float32) if sums else None
        rc = self.lib.oracle_linear(
            int(elem), _ptr(x, ctypes.c_uint16), max(K, 1), _ptr(w, ctypes.c_uint16), max(K, 1),
            None if bb is None else _ptr(bb, ctypes.c_uint16),
            _ptr(y, ctypes.c_uint16), _ptr(proj, ctypes.c_uint16),
            None if y32 is None else _ptr(y32, ctypes.c_float), max(N, 1), M, N, K, nthreads)
        if rc != 0:
            raise MemoryError("oracle_linear failed")
        return (y, proj, y32) if sums else (y, proj)

    def points(self, x, w, b, ms, ns, nthreads: int = 0, elem: int = F16):
        """Evaluate the definition at coordinates (ms[i], ns[i]).

        Returns dict(y, proj, y32, S, A): uint16 y and proj, float32 unrounded sums
        y32, float64 S = sum x*w and A = sum |x*w| (FP64, products exact)."""
        x = _as_words(x)
        w = _as_words(w)
        ms = np.ascontiguousarray(ms, dtype=np.int64)
        ns = np.ascontiguousarray(ns, dtype=np.int64)
        count = ms.size
        K = x.shape[1]
        bb = None if b is None else _as_words(b)
        y = np.zeros(count, np.uint16)
        proj = np.zeros(count, np.uint16)
        y32 = np.zeros(count, np.float32)
        S = np.zeros(count, np.float64)
        A = np.zeros(count, np.float64)
        self.lib.oracle_linear_points(
            int(elem), _ptr(x, ctypes.c_uint16), max(K, 1), _ptr(w, ctypes.c_uint16), max(K, 1),
            None if bb is None else _ptr(bb, ctypes.c_uint16), K,
            _ptr(ms, ctypes.c_int64), _ptr(ns, ctypes.c_int64), count,
            _ptr(y, ctypes.c_uint16), _ptr(proj, ctypes.c_uint16), _ptr(y32, ctypes.c_float),
            _ptr(S, ctypes.c_double), _ptr(A, ctypes.c_double), nthreads)
        return {"y": y, "proj": proj, "y32": y32, "S": S, "A": A}

    def band(self, x, w, nthreads: int = 0, elem: int = F16):
        """FP64 S = x @ w.T and A = |x| @ |w|.T for the whole output (small problems)."""
        x = _as_words(x)
        w = _as_words(w)
        M, K = x.shape
        N = w.shape[0]
        S = np.zeros((M, N), np.float64)
        A = np.zeros((M, N), np.float64)
        rc = self.lib.oracle_band(int(elem), _ptr(x, ctypes.c_uint16), max(K, 1), _ptr(w, ctypes.c_uint16),
                                  max(K, 1), M, N, K, _ptr(S, ctypes.c_double),
                                  _ptr(A, ctypes.c_double), nthreads)
        if rc != 0:
            raise MemoryError("oracle_band_f64 failed")
        return S, A

    # -- grouped and indexed contractions ------------------------------------------
    def grouped(self, x, w, b=None, elem: int = F16, nthreads: int = 0):
        """x: [G, M, K] words, w: [G*N, K], b: [G*N] or None.  Returns (y, proj, y32) as
        [G, M, N] arrays (y = proj when b is None)."""
        x = _as_words(x)
        w = _as_words(w)
        G, M, K = x.shape
        N = w.shape[0] // max(G, 1)
        assert w.shape == (G * N, K), (x.shape, w.shape)
        bb = None if b is None else _as_words(b)
        y = np.zeros((G, M, N), np.uint16)
        proj = np.zeros((G, M, N), np.uint16)
        y32 = np.zeros((G, M, N), np.float32)
        rc = self.lib.oracle_grouped(int(elem), _ptr(x, ctypes.c_uint16), max(K, 1), M * max(K, 1),
                                     _ptr(w, ctypes.c_uint16), max(K, 1),
                                     None if bb is None else _ptr(bb, ctypes.c_uint16), _ptr(y, ctypes.c_uint16),
                                     _ptr(proj, ctypes.c_uint16), _ptr(y32, ctypes.c_float), max(N, 1), M * max(N, 1),
                                     G, M, N, K, nthreads)
        if rc != 0:
            raise MemoryError("oracle_grouped failed")
        return y, proj, y32

    def indexed(self, x, w, idx, elem: int = F16, y_init=None, nthreads: int = 0):
        """x: [M, K] words, w: [E, K, N] words, idx: [M] int32.  Returns (y, y32) [M, N];
        rows whose idx is outside [0, E) keep y_init (zeros by default)."""
        x = _as_words(x)
        w = _as_words(w)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        M, K = x.shape
        E, K2, N = w.shape
        assert K == K2 and idx.shape == (M,)
        y = np.zeros((M, N), np.uint16) if y_init is None else np.array(y_init, np.uint16, copy=True)
        y32 = np.zeros((M, N), np.float32)
        self.lib.oracle_indexed(int(elem), _ptr(x, ctypes.c_uint16), max(K, 1), _ptr(w, ctypes.c_uint16),
                                max(N, 1), max(K, 1) * max(N, 1), idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                _ptr(y, ctypes.c_uint16), _ptr(y32, ctypes.c_float), max(N, 1), E, M, N, K, nthreads)
        return y, y32

    def indexed_band(self, x, w, idx, elem: int = F16):
        x = _as_words(x)
        w = _as_words(w)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        M, K = x.shape
        E, _, N = w.shape
        S = np.zeros((M, N), np.float64)
        A = np.zeros((M, N), np.float64)
        self.lib.oracle_indexed_band(int(elem), _ptr(x, ctypes.c_uint16), max(K, 1), _ptr(w, ctypes.c_uint16),
                                     max(N, 1), max(K, 1) * max(N, 1),
                                     idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                     _ptr(S, ctypes.c_double), _ptr(A, ctypes.c_double), E, M, N, K)
        return S, A

    # -- multi-step epilogue ------------------------------------------------------
    def f64_to_elem(self, v, elem: int = F16) -> np.ndarray:
        v = np.asarray(v, np.float64)
        out = np.empty(v.shape, np.uint16)
        flat = v.ravel()
        o = out.ravel()
        for i in range(flat.size):
            o[i] = self.lib.oracle_f64_to_elem(int(elem), float(flat[i]))
        return out

    def unary(self, op: int, x, elem: int = F16) -> np.ndarray:
        """An activation (EPI_SILU, EPI_GELU_TANH, EPI_GELU_ERF) or a rounded primitive
        (UNARY_EXP, UNARY_ERF) over element-type words."""
        x = _as_words(x)
        out = np.empty(x.shape, np.uint16)
        self.lib.oracle_unary_array(int(elem), int(op), _ptr(x, ctypes.c_uint16), _ptr(out, ctypes.c_uint16), x.size)
        return out

    def epilogue(self, ops, t, bias=None, res=None, mul=None, elem: int = F16) -> np.ndarray:
        """The steps `ops` applied to element-type words t (any shape); bias, res and
        mul are per-element words of t's shape (broadcast by the caller) or None."""
        t = _as_words(t)
        opsa = np.ascontiguousarray(ops, dtype=np.int32)
        def opt(a):
            if a is None:
                return None, None
            a = np.ascontiguousarray(np.broadcast_to(_as_words(a), t.shape))
            return a, _ptr(a, ctypes.c_uint16)
        bk, bp = opt(bias)
        rk, rp = opt(res)
        mk, mp = opt(mul)
        out = np.empty(t.shape, np.uint16)
        self.lib.oracle_epilogue(int(elem), opsa.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(opsa.size),
                                 _ptr(t, ctypes.c_uint16), bp, rp, mp, _ptr(out, ctypes.c_uint16), t.size)
        return out

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def timed_points(self, x, w, b, ms, ns, nthreads: int = 0):
        """points(), with the wall time in seconds (used for the CPU baseline)."""
        t0 = time.perf_counter()
        r = self.points(x, w, b, ms, ns, nthreads)
        return r, time.perf_counter() - t0


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
