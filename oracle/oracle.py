"""ctypes marshalling for the C oracle (``w4a16_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Arrays are numpy; 16-bit activations travel as
their raw uint16 bit patterns so the oracle decodes them itself.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

GROUP = 128
F32, BF16, F16 = 0, 1, 2
ACT_SWIGLU, ACT_GELU_TANH = 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4a16_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_w4a16.so")
_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra"]

_lib = None


def library_path() -> str:
    return _LIB


def build(src: str = _SRC, out: str = _LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (always recompiles)."""
    cmd = ["gcc", *_CFLAGS, *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _declare(lib):
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.oracle_quantize.argtypes = [vp, i32, i64, i64, i64, vp, vp]
    lib.oracle_quantize.restype = i32
    lib.oracle_quantize_int8.argtypes = [vp, i32, i64, i64, i64, vp, vp]
    lib.oracle_quantize_int8.restype = i32
    lib.oracle_codes_to_nibbles.argtypes = [vp, i64, i64, vp]
    lib.oracle_codes_to_nibbles.restype = None
    lib.oracle_nibbles_to_codes.argtypes = [vp, i64, i64, vp]
    lib.oracle_nibbles_to_codes.restype = None
    lib.oracle_dequantize.argtypes = [vp, vp, i64, i64, vp]
    lib.oracle_dequantize.restype = None
    lib.oracle_linear.argtypes = [vp, i32, i64, i64, i64, vp, vp, i64, vp, vp]
    lib.oracle_linear.restype = i32
    lib.oracle_linear_entries.argtypes = [vp, i32, i64, i64, i64, vp, vp, i64, vp, vp, vp, i64, vp]
    lib.oracle_linear_entries.restype = i32
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_double.restype = ctypes.c_double
    lib.oracle_round16.argtypes = [ctypes.c_double, i32]
    lib.oracle_round16.restype = ctypes.c_uint16
    lib.oracle_act_value.argtypes = [ctypes.c_double, ctypes.c_double, i32]
    lib.oracle_act_value.restype = ctypes.c_double
    lib.oracle_activate.argtypes = [vp, i32, i32, i64, i64, i64, vp]
    lib.oracle_activate.restype = i32
    lib.oracle_splitmix64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    lib.oracle_splitmix64.restype = ctypes.c_uint64
    lib.oracle_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    lib.oracle_uniform.restype = ctypes.c_float
    lib.oracle_update.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp, i64, i32, ctypes.c_float, ctypes.c_float,
                                  i32, ctypes.c_uint64, i32]
    lib.oracle_update.restype = i32
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i32
    return lib


def load(path: str | None = None):
    """Load a built oracle; ``path`` loads an alternative build (used by tests)."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dtype_tag(a: np.ndarray, tag):
    if a.dtype == np.float32:
        return F32
    if tag is None:
        raise ValueError("16-bit arrays need an explicit dtype tag (BF16 or F16)")
    return tag


def quantize(w: np.ndarray, dtype_tag=None, lib=None):
    """RTN INT4 g128 quantization. ``w`` [n, k] float32, or uint16 bits with a tag.

    Returns (q int8 [n, k], s float32 [n, k/128]).
    """
    lib = lib or load()
    w = np.ascontiguousarray(w)
    n, k = w.shape
    tag = _dtype_tag(w, dtype_tag)
    q = np.empty((n, k), dtype=np.int8)
    s = np.empty((n, max(k // GROUP, 0)), dtype=np.float32)
    rc = lib.oracle_quantize(_p(w), tag, n, k, k, _p(q), _p(s))
    if rc != 0:
        raise ValueError(f"oracle_quantize rejected shape {w.shape}")
    return q, s


def quantize_int8(w: np.ndarray, dtype_tag=None, lib=None):
    """RTN INT8 g128 quantization: (q int8 [n, k] in [-128, 127], s float32 [n, k/128])."""
    lib = lib or load()
    w = np.ascontiguousarray(w)
    n, k = w.shape
    tag = _dtype_tag(w, dtype_tag)
    q = np.empty((n, k), dtype=np.int8)
    s = np.empty((n, max(k // GROUP, 0)), dtype=np.float32)
    rc = lib.oracle_quantize_int8(_p(w), tag, n, k, k, _p(q), _p(s))
    if rc != 0:
        raise ValueError(f"oracle_quantize_int8 rejected shape {w.shape}")
    return q, s


def codes_to_nibbles(q: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.int8)
    n, k = q.shape
    out = np.empty((n, k // 2), dtype=np.uint8)
    lib.oracle_codes_to_nibbles(_p(q), n, k, _p(out))
    return out


def nibbles_to_codes(codes: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load()
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    n, half = codes.shape
    out = np.empty((n, 2 * half), dtype=np.int8)
    lib.oracle_nibbles_to_codes(_p(codes), n, 2 * half, _p(out))
    return out


def dequantize(q: np.ndarray, s: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    n, k = q.shape
    out = np.empty((n, k), dtype=np.float64)
    lib.oracle_dequantize(_p(q), _p(s), n, k, _p(out))
    return out


def linear(x_bits: np.ndarray, x_tag: int, q: np.ndarray, s: np.ndarray,
           bias_bits: np.ndarray | None = None, lib=None) -> np.ndarray:
    """y = x . (q*s)^T + bias in double.  ``x_bits`` [m, k] uint16, ``bias_bits`` [n] uint16."""
    lib = lib or load()
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    m, k = x_bits.shape
    n = q.shape[0]
    y = np.empty((m, n), dtype=np.float64)
    b = None
    if bias_bits is not None:
        b = np.ascontiguousarray(bias_bits, dtype=np.uint16)
    rc = lib.oracle_linear(_p(x_bits), x_tag, m, k, k, _p(q), _p(s), n,
                           _p(b) if b is not None else None, _p(y))
    if rc != 0:
        raise ValueError("oracle_linear rejected its arguments")
    return y


def linear_entries(x_bits, x_tag, q, s, bias_bits, rows, cols, lib=None) -> np.ndarray:
    """The outputs y[rows[e], cols[e]] only (for full-size cases)."""
    lib = lib or load()
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    m, k = x_bits.shape
    n = q.shape[0]
    out = np.empty(rows.shape[0], dtype=np.float64)
    b = None
    if bias_bits is not None:
        b = np.ascontiguousarray(bias_bits, dtype=np.uint16)
    rc = lib.oracle_linear_entries(_p(x_bits), x_tag, m, k, k, _p(q), _p(s), n,
                                   _p(b) if b is not None else None,
                                   _p(rows), _p(cols), rows.shape[0], _p(out))
    if rc != 0:
        raise ValueError("oracle_linear_entries rejected its arguments")
    return out


def activate(x_bits: np.ndarray, x_tag: int, act: int, lib=None) -> np.ndarray:
    """The activated layer input as 16-bit patterns [m, k].  SwiGLU rows of
    ``x_bits`` hold [up | gate] (2k columns); GELU rows hold k columns."""
    lib = lib or load()
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    m, width = x_bits.shape
    k = width // 2 if act == ACT_SWIGLU else width
    out = np.empty((m, k), dtype=np.uint16)
    rc = lib.oracle_activate(_p(x_bits), x_tag, act, m, k, width, _p(out))
    if rc != 0:
        raise ValueError("oracle_activate rejected its arguments")
    return out


def linear_act(x_bits, x_tag, act, q, s, bias_bits=None, lib=None) -> np.ndarray:
    """y = act(x) . (q*s)^T + bias in double, act(x) rounded to x's dtype first."""
    a = activate(x_bits, x_tag, act, lib=lib)
    return linear(a, x_tag, q, s, bias_bits, lib=lib)


def round16(v: float, tag: int, lib=None) -> int:
    return int((lib or load()).oracle_round16(float(v), tag))


def act_value(v: float, up: float, act: int, lib=None) -> float:
    return float((lib or load()).oracle_act_value(float(v), float(up), act))


def _upd_array(a: np.ndarray, tag):
    a = np.ascontiguousarray(a)
    return a, _dtype_tag(a, tag)


def update(q: np.ndarray, s: np.ndarray, upd=None, mat1=None, mat2=None, alpha=1.0, beta=1.0,
           seed=None, dtype_tag=None, lib=None, bits=4):
    """Requantized codes and scales of beta * dequant(q, s) + alpha * U, U a
    dense [n, k] update or mat1 [n, r] @ mat2 [r, k] (float32, or uint16 bits
    with a dtype tag); stochastic rounding when ``seed`` is given; ``bits``
    4 (INT4 codes, amax/7) or 8 (INT8 codes, amax/127).
    Returns new (q, s); the inputs are not modified."""
    lib = lib or load()
    q = np.array(q, dtype=np.int8, order="C", copy=True)
    s = np.array(s, dtype=np.float32, order="C", copy=True)
    n, k = q.shape
    if upd is not None:
        u, tag = _upd_array(upd, dtype_tag)
        args = (_p(u), k, None, None, 0, tag)
    else:
        a, tag = _upd_array(mat1, dtype_tag)
        b, _ = _upd_array(mat2, dtype_tag)
        args = (None, 0, _p(a), _p(b), a.shape[1], tag)
    rc = lib.oracle_update(_p(q), _p(s), n, k, *args, float(alpha), float(beta), int(seed is not None),
                           int(seed or 0), int(bits))
    if rc != 0:
        raise ValueError("oracle_update rejected its arguments")
    return q, s


def splitmix64(seed: int, e: int, lib=None) -> int:
    return int((lib or load()).oracle_splitmix64(seed, e))


def uniform(seed: int, e: int, lib=None) -> float:
    return float((lib or load()).oracle_uniform(seed, e))


def bf16_to_double(bits: int, lib=None) -> float:
    return (lib or load()).oracle_bf16_to_double(bits)


def f16_to_double(bits: int, lib=None) -> float:
    return (lib or load()).oracle_f16_to_double(bits)


def num_threads(lib=None) -> int:
    return (lib or load()).oracle_num_threads()
