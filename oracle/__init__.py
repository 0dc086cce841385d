"""CPU oracle for the FP16 all-reduce combine (test infrastructure only).

This package wraps ``hr_oracle.c``, a plain C definition of the combine:
every add in IEEE binary64 (exact for binary16 operands) followed by one
explicit round-to-nearest-even to binary16, folded left in rank order.  The
two-rank case is the single-rounding commutative sum of the 1Cat-vLLM pull
request "[Kernel] Two-rank FP16 all-reduce through pinned host memory for
GPUs without P2P" (section "Purpose"); the left-fold order for more ranks is
the reading taken where the pages are silent (the SGLang pull request
"[SM120] Add optional FlashInfer PCIe-IPC all-reduce for switch-free hosts",
section "Accuracy", shows that order changes bits).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library and its Python binding never do,
and nothing here imports them.

Arrays cross this boundary as numpy ``uint16`` bit patterns (binary16 or
bfloat16 bits), never as numpy float values, so that no numpy arithmetic is
involved.  The ``*_bf16`` functions are the same combine on bfloat16.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hr_oracle.c")
_LIB = os.path.join(_HERE, "libhr_oracle.so")

# Plain host build: no fast-math, no HIP headers.
BUILD_CMD = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
             "-fopenmp", _SRC, "-o", _LIB, "-lm"]


def build() -> str:
    """Compile the oracle into ``libhr_oracle.so`` next to its source."""
    subprocess.run(BUILD_CMD, check=True)
    return _LIB


def _bind(path: str):
    lib = ctypes.CDLL(path)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    lib.hro_decode.argtypes = [ctypes.c_uint16]
    lib.hro_decode.restype = ctypes.c_double
    lib.hro_round.argtypes = [ctypes.c_double]
    lib.hro_round.restype = ctypes.c_uint16
    lib.hro_add.argtypes = [ctypes.c_uint16, ctypes.c_uint16]
    lib.hro_add.restype = ctypes.c_uint16
    lib.hro_add_vec.argtypes = [u16p, u16p, u16p, ctypes.c_size_t]
    lib.hro_add_vec.restype = None
    lib.hro_decode_vec.argtypes = [u16p, f64p, ctypes.c_size_t]
    lib.hro_decode_vec.restype = None
    lib.hro_round_vec.argtypes = [f64p, u16p, ctypes.c_size_t]
    lib.hro_round_vec.restype = None
    lib.hro_fold.argtypes = [ctypes.POINTER(u16p), ctypes.c_int, ctypes.c_size_t, u16p]
    lib.hro_fold.restype = None
    lib.hro_fold_threads.argtypes = [ctypes.POINTER(u16p), ctypes.c_int, ctypes.c_size_t,
                                     u16p, ctypes.c_int]
    lib.hro_fold_threads.restype = ctypes.c_int
    lib.hro_decode_bf16_vec.argtypes = [u16p, f64p, ctypes.c_size_t]
    lib.hro_decode_bf16_vec.restype = None
    lib.hro_round_bf16_vec.argtypes = [f64p, u16p, ctypes.c_size_t]
    lib.hro_round_bf16_vec.restype = None
    lib.hro_add_bf16_vec.argtypes = [u16p, u16p, u16p, ctypes.c_size_t]
    lib.hro_add_bf16_vec.restype = None
    lib.hro_fold_bf16.argtypes = [ctypes.POINTER(u16p), ctypes.c_int, ctypes.c_size_t, u16p]
    lib.hro_fold_bf16.restype = None
    return lib


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected uint16 bit patterns, got {a.dtype}")
    return a


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class Oracle:
    """The oracle's entry points bound to one compiled ``hr_oracle.c``.

    The module-level functions use the library built next to the source; the
    mutation tests bind copies compiled with planted mistakes.
    """

    def __init__(self, path: str):
        self.path = path
        self.lib = _bind(path)

    def decode(self, h) -> np.ndarray:
        """Exact binary64 value of each binary16 bit pattern."""
        h = _u16(h)
        out = np.empty(h.shape, dtype=np.float64)
        self.lib.hro_decode_vec(_ptr(h, ctypes.c_uint16), _ptr(out, ctypes.c_double), h.size)
        return out

    def round_f16(self, v) -> np.ndarray:
        """Round binary64 values to binary16 bit patterns, ties to even."""
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty(v.shape, dtype=np.uint16)
        self.lib.hro_round_vec(_ptr(v, ctypes.c_double), _ptr(out, ctypes.c_uint16), v.size)
        return out

    def add(self, a, b) -> np.ndarray:
        """Elementwise fl16(a + b) with one rounding (the two-rank combine)."""
        a = _u16(a)
        b = _u16(b)
        if a.shape != b.shape:
            raise ValueError("shape mismatch")
        out = np.empty(a.shape, dtype=np.uint16)
        self.lib.hro_add_vec(_ptr(a, ctypes.c_uint16), _ptr(b, ctypes.c_uint16),
                             _ptr(out, ctypes.c_uint16), a.size)
        return out

    def fold(self, xs, threads: int = 1):
        """Left fold of the contributions ``xs[0..G-1]`` in rank order.

        Returns ``(result, threads_used)`` when ``threads > 1`` and ``result``
        otherwise.  ``threads > 1`` splits the element range over OpenMP
        threads; the result is identical.
        """
        xs = [_u16(x) for x in xs]
        if not xs:
            raise ValueError("need at least one contribution")
        n = xs[0].size
        for x in xs:
            if x.size != n:
                raise ValueError("contributions differ in length")
        out = np.empty(xs[0].shape, dtype=np.uint16)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        arr = (u16p * len(xs))(*[_ptr(x, ctypes.c_uint16) for x in xs])
        if threads > 1:
            used = self.lib.hro_fold_threads(arr, len(xs), n, _ptr(out, ctypes.c_uint16),
                                             threads)
            return out, used
        self.lib.hro_fold(arr, len(xs), n, _ptr(out, ctypes.c_uint16))
        return out


    # bfloat16: the same combine with bfloat16 operands and results
    def decode_bf16(self, h) -> np.ndarray:
        """Exact binary64 value of each bfloat16 bit pattern."""
        h = _u16(h)
        out = np.empty(h.shape, dtype=np.float64)
        self.lib.hro_decode_bf16_vec(_ptr(h, ctypes.c_uint16), _ptr(out, ctypes.c_double), h.size)
        return out

    def round_bf16(self, v) -> np.ndarray:
        """Round binary64 values to bfloat16 bit patterns, ties to even."""
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty(v.shape, dtype=np.uint16)
        self.lib.hro_round_bf16_vec(_ptr(v, ctypes.c_double), _ptr(out, ctypes.c_uint16), v.size)
        return out

    def add_bf16(self, a, b) -> np.ndarray:
        """Elementwise bfloat16 fl(a + b) with one rounding."""
        a = _u16(a)
        b = _u16(b)
        if a.shape != b.shape:
            raise ValueError("shape mismatch")
        out = np.empty(a.shape, dtype=np.uint16)
        self.lib.hro_add_bf16_vec(_ptr(a, ctypes.c_uint16), _ptr(b, ctypes.c_uint16),
                                  _ptr(out, ctypes.c_uint16), a.size)
        return out

    def fold_bf16(self, xs) -> np.ndarray:
        """Left fold of bfloat16 contributions in rank order."""
        xs = [_u16(x) for x in xs]
        if not xs:
            raise ValueError("need at least one contribution")
        n = xs[0].size
        for x in xs:
            if x.size != n:
                raise ValueError("contributions differ in length")
        out = np.empty(xs[0].shape, dtype=np.uint16)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        arr = (u16p * len(xs))(*[_ptr(x, ctypes.c_uint16) for x in xs])
        self.lib.hro_fold_bf16(arr, len(xs), n, _ptr(out, ctypes.c_uint16))
        return out


_default = None


def _get() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _default = Oracle(_LIB)
    return _default


def decode(h) -> np.ndarray:
    """Exact binary64 value of each binary16 bit pattern."""
    return _get().decode(h)


def round_f16(v) -> np.ndarray:
    """Round binary64 values to binary16 bit patterns, ties to even."""
    return _get().round_f16(v)


def add(a, b) -> np.ndarray:
    """Elementwise fl16(a + b) with one rounding (the two-rank combine)."""
    return _get().add(a, b)


def fold(xs, threads: int = 1):
    """Left fold of ``xs[0..G-1]`` in rank order; see ``Oracle.fold``."""
    return _get().fold(xs, threads)


def decode_bf16(h) -> np.ndarray:
    """Exact binary64 value of each bfloat16 bit pattern."""
    return _get().decode_bf16(h)


def round_bf16(v) -> np.ndarray:
    """Round binary64 values to bfloat16 bit patterns, ties to even."""
    return _get().round_bf16(v)


def add_bf16(a, b) -> np.ndarray:
    """Elementwise bfloat16 fl(a + b) with one rounding."""
    return _get().add_bf16(a, b)


def fold_bf16(xs) -> np.ndarray:
    """Left fold of bfloat16 contributions in rank order."""
    return _get().fold_bf16(xs)


def same_bits_bf16(a, b) -> np.ndarray:
    """Elementwise equality of bfloat16 patterns with NaN compared by class."""
    a = _u16(a)
    b = _u16(b)
    a_nan = ((a & 0x7F80) == 0x7F80) & ((a & 0x007F) != 0)
    b_nan = ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)
    return np.where(a_nan | b_nan, a_nan & b_nan, a == b)


def same_bits(a, b) -> np.ndarray:
    """Elementwise equality of binary16 patterns with NaN compared by class.

    IEEE 754 leaves the payload of a NaN produced by an add open, so any NaN
    matches any NaN; every other pattern must match bit for bit.
    """
    a = _u16(a)
    b = _u16(b)
    a_nan = ((a & 0x7C00) == 0x7C00) & ((a & 0x03FF) != 0)
    b_nan = ((b & 0x7C00) == 0x7C00) & ((b & 0x03FF) != 0)
    return np.where(a_nan | b_nan, a_nan & b_nan, a == b)
