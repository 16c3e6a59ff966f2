"""CPU oracle for the narrow-batch q8_0 decode matmul.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path (the HIP library
and its Python binding) never does, and this package never imports the
product.  The arithmetic lives in plain C (``q8_oracle.c``), built with gcc
and loaded with ctypes; this module only marshals numpy arrays.

Functions and the passages they follow are documented in ``q8_oracle.c``.
Every function here is pinned by CPU tests (``tests/test_oracle_pins.py``) to
values fixed by the format definitions and by mathematics, not by itself, and
``tests/test_oracle_mutants.py`` shows that planted mistakes in the C source
fail those pins.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "q8_oracle.c")
LIB_PATH = os.path.join(_HERE, "libq8oracle.so")

BLOCK = 32

CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
          "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC"]


def compile_oracle(src: str, out: str) -> str:
    """gcc ``src`` into the shared library ``out``."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the oracle into ``oracle/libq8oracle.so``."""
    if force or not os.path.exists(LIB_PATH):
        compile_oracle(SOURCE, LIB_PATH)
    return LIB_PATH


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """The oracle's functions, bound to one build of ``q8_oracle.c``."""

    def __init__(self, lib_path: str = LIB_PATH):
        lib = ctypes.CDLL(lib_path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.q8o_f32_to_f16.argtypes = [ctypes.c_float]
        lib.q8o_f32_to_f16.restype = ctypes.c_uint16
        lib.q8o_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.q8o_f16_to_f32.restype = ctypes.c_float
        lib.q8o_f32_to_f16_array.argtypes = [vp, i64, vp]
        lib.q8o_f32_to_f16_array.restype = None
        lib.q8o_f16_to_f32_array.argtypes = [vp, i64, vp]
        lib.q8o_f16_to_f32_array.restype = None
        lib.q8o_quantize_rows.argtypes = [vp, i64, i64, vp, vp, vp]
        lib.q8o_quantize_rows.restype = i32
        lib.q8o_matmul.argtypes = [vp, vp, i64, i64, vp, vp, i32, vp, i32,
                                   vp, i64, vp, vp]
        lib.q8o_matmul.restype = i32
        lib.q8o_block_dots.argtypes = [vp, i64, i64, vp, i32, vp, i32, vp,
                                       i64, vp]
        lib.q8o_block_dots.restype = i32
        lib.q8o_rope.argtypes = [vp, i64, i64, vp, i64, i64, ctypes.c_double, vp, vp]
        lib.q8o_rope.restype = i32
        lib.q8o_num_threads.argtypes = []
        lib.q8o_num_threads.restype = i32
        lib.q8o_set_num_threads.argtypes = [i32]
        lib.q8o_set_num_threads.restype = None
        self._lib = lib
        self.path = lib_path

    # ---------------------------------------------------------------- fp16
    def f32_to_f16_bits(self, x) -> np.ndarray:
        """IEEE binary32 -> binary16 bits, round to nearest even (uint16)."""
        x = _c(x, np.float32)
        out = np.empty(x.shape, dtype=np.uint16)
        self._lib.q8o_f32_to_f16_array(_ptr(x), x.size, _ptr(out))
        return out

    def f16_bits_to_f32(self, h) -> np.ndarray:
        """IEEE binary16 bits -> binary32 (exact)."""
        h = _c(h, np.uint16)
        out = np.empty(h.shape, dtype=np.float32)
        self._lib.q8o_f16_to_f32_array(_ptr(h), h.size, _ptr(out))
        return out

    # ------------------------------------------------------------ quantise
    def quantize_rows(self, X, return_d32: bool = False):
        """Quantise fp32 rows [R][K] into canonical q8_0.

        Returns ``(q int8 [R][K], d16 uint16 [R][K/32])`` and, if asked, the
        fp32 scales before binary16 rounding ``d32 float32 [R][K/32]``.
        """
        X = _c(X, np.float32)
        if X.ndim != 2:
            raise ValueError("X must be 2-D [rows][K]")
        R, K = X.shape
        if K % BLOCK:
            raise ValueError("K must be a multiple of 32")
        q = np.empty((R, K), dtype=np.int8)
        d16 = np.empty((R, K // BLOCK), dtype=np.uint16)
        d32 = np.empty((R, K // BLOCK), dtype=np.float32) if return_d32 else None
        rc = self._lib.q8o_quantize_rows(_ptr(X), R, K, _ptr(q), _ptr(d16),
                                         _ptr(d32))
        if rc:
            raise ValueError("q8o_quantize_rows rejected the shape")
        return (q, d16, d32) if return_d32 else (q, d16)

    # -------------------------------------------------------------- matmul
    def matmul(self, qw, dw, qx, dx, batch_index, rows=None):
        """Oracle narrow matmul.

        qw int8 [N][K], dw uint16 [N][K/32]: canonical q8_0 weights.
        qx int8 [S][K], dx uint16 [S][K/32]: the activation slot buffer.
        batch_index: int32 [n_live]; token t reads slot batch_index[t].
        rows: optional int64 list of output rows to compute (default: all).

        Returns ``(Y, A)``, both float64 [n_live][len(rows)]: Y is the sum of
        the exact block terms in double, A the sum of their magnitudes.
        """
        qw, dw = _c(qw, np.int8), _c(dw, np.uint16)
        qx, dx = _c(qx, np.int8), _c(dx, np.uint16)
        bi = _c(batch_index, np.int32).reshape(-1)
        N, K = qw.shape
        if (dw.shape != (N, K // BLOCK) or qx.shape[1] != K
                or dx.shape != (qx.shape[0], K // BLOCK)):
            raise ValueError("operand shapes disagree")
        rows_arr = None if rows is None else _c(rows, np.int64).reshape(-1)
        n_rows = N if rows_arr is None else rows_arr.size
        Y = np.empty((bi.size, n_rows), dtype=np.float64)
        A = np.empty((bi.size, n_rows), dtype=np.float64)
        rc = self._lib.q8o_matmul(_ptr(qw), _ptr(dw), N, K, _ptr(qx), _ptr(dx),
                                  qx.shape[0], _ptr(bi), bi.size,
                                  _ptr(rows_arr), n_rows, _ptr(Y), _ptr(A))
        if rc:
            raise ValueError("q8o_matmul rejected the shape")
        return Y, A

    def block_dots(self, qw, qx, batch_index, rows=None):
        """Exact per-block int32 dot products S [n_live][len(rows)][K/32]."""
        qw, qx = _c(qw, np.int8), _c(qx, np.int8)
        bi = _c(batch_index, np.int32).reshape(-1)
        N, K = qw.shape
        rows_arr = None if rows is None else _c(rows, np.int64).reshape(-1)
        n_rows = N if rows_arr is None else rows_arr.size
        S = np.empty((bi.size, n_rows, K // BLOCK), dtype=np.int32)
        rc = self._lib.q8o_block_dots(_ptr(qw), N, K, _ptr(qx), qx.shape[0],
                                      _ptr(bi), bi.size, _ptr(rows_arr),
                                      n_rows, _ptr(S))
        if rc:
            raise ValueError("q8o_block_dots rejected the shape")
        return S

    # ------------------------------------------------------------- threads
    def rope(self, Y, pos, n_heads: int, head_dim: int, base: float):
        """Oracle pos-vector RoPE.

        Y float32 [n_rows][row_stride]: heads 0..n_heads-1 in the first
        n_heads*head_dim columns; pos int32 [n_rows], one position per row.
        Returns ``(out, mag)``, float64 [n_rows][n_heads*head_dim]: the
        rotated values and |a| + |b| of each value's pair.
        """
        Y = _c(Y, np.float32)
        pos = _c(pos, np.int32).reshape(-1)
        n_rows, stride = Y.shape
        if pos.size != n_rows:
            raise ValueError("one position per row")
        out = np.empty((n_rows, n_heads * head_dim), dtype=np.float64)
        mag = np.empty_like(out)
        rc = self._lib.q8o_rope(_ptr(Y), n_rows, stride, _ptr(pos), n_heads, head_dim,
                                float(base), _ptr(out), _ptr(mag))
        if rc:
            raise ValueError("invalid rope arguments")
        return out, mag

    def num_threads(self) -> int:
        return int(self._lib.q8o_num_threads())

    def set_num_threads(self, n: int) -> None:
        self._lib.q8o_set_num_threads(int(n))


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from ``q8_oracle.c`` (compiled on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        _default = Oracle(LIB_PATH)
    return _default


def f32_to_f16_bits(x):
    return get().f32_to_f16_bits(x)


def f16_bits_to_f32(h):
    return get().f16_bits_to_f32(h)


def quantize_rows(X, return_d32: bool = False):
    return get().quantize_rows(X, return_d32)


def matmul(qw, dw, qx, dx, batch_index, rows=None):
    return get().matmul(qw, dw, qx, dx, batch_index, rows)


def block_dots(qw, qx, batch_index, rows=None):
    return get().block_dots(qw, qx, batch_index, rows)


def rope(Y, pos, n_heads: int, head_dim: int, base: float):
    return get().rope(Y, pos, n_heads, head_dim, base)


def num_threads() -> int:
    return get().num_threads()


def set_num_threads(n: int) -> None:
    get().set_num_threads(n)
