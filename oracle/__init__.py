"""ctypes wrapper of the plain C oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by tests/, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py``.  The product path never imports this package.

``build()`` compiles ``liboracle.so`` with gcc (scalar, -O2, no FMA contraction); ``lib()``
loads it, building it first when it is missing.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    src = os.path.join(_HERE, "oracle.c")
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                           "-fPIC", "-shared", "-o", tmp, src, "-lm"])
    os.replace(tmp, _SO)
    return _SO


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        L.oracle_canonical_bytes.restype = i64
        L.oracle_canonical_bytes.argtypes = [ctypes.c_int, i64, i64]
        L.oracle_half_to_double.restype = ctypes.c_double
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_decode_f64.restype = ctypes.c_int
        L.oracle_decode_f64.argtypes = [ctypes.c_int, i64, i64, vp, i64, i64, vp]
        L.oracle_dequant_f32.restype = ctypes.c_int
        L.oracle_dequant_f32.argtypes = [ctypes.c_int, i64, i64, vp, i64, i64, vp]
        L.oracle_gemm_f64.restype = ctypes.c_int
        L.oracle_gemm_f64.argtypes = [ctypes.c_int, i64, i64, vp, vp, i64, i64, vp, i64, vp, vp]
        L.oracle_silu.restype = ctypes.c_double
        L.oracle_silu.argtypes = [ctypes.c_double]
        L.oracle_silu_mul_f64.restype = ctypes.c_int
        L.oracle_silu_mul_f64.argtypes = [vp, vp, i64, vp]
        L.oracle_residual_add_f64.restype = ctypes.c_int
        L.oracle_residual_add_f64.argtypes = [vp, vp, i64, vp]
        L.oracle_quantize_x_i8.restype = ctypes.c_int
        L.oracle_quantize_x_i8.argtypes = [vp, i64, i64, i64, vp, vp, vp]
        L.oracle_tq2_i8_f64.restype = ctypes.c_int
        L.oracle_tq2_i8_f64.argtypes = [i64, i64, vp, vp, vp, i64, vp, i64, vp, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def canonical_bytes(fmt: int, N: int, K: int) -> int:
    return int(lib().oracle_canonical_bytes(fmt, N, K))


def half_to_double(h: int) -> float:
    return float(lib().oracle_half_to_double(h))


def decode_f64(fmt: int, N: int, K: int, canon: np.ndarray, row0: int = 0, nrows: int | None = None) -> np.ndarray:
    nrows = N - row0 if nrows is None else nrows
    canon = np.ascontiguousarray(canon, dtype=np.uint8)
    w = np.empty((nrows, K), dtype=np.float64)
    rc = lib().oracle_decode_f64(fmt, N, K, _ptr(canon), row0, nrows, _ptr(w))
    if rc:
        raise ValueError(f"oracle_decode_f64 failed: {rc}")
    return w


def dequant_f32(fmt: int, N: int, K: int, canon: np.ndarray, row0: int = 0, nrows: int | None = None) -> np.ndarray:
    nrows = N - row0 if nrows is None else nrows
    canon = np.ascontiguousarray(canon, dtype=np.uint8)
    w = np.empty((nrows, K), dtype=np.float32)
    rc = lib().oracle_dequant_f32(fmt, N, K, _ptr(canon), row0, nrows, _ptr(w))
    if rc:
        raise ValueError(f"oracle_dequant_f32 failed: {rc}")
    return w


def gemm_f64(fmt: int, N: int, K: int, canon: np.ndarray, x_bits: np.ndarray, rows=None):
    """Returns (y, a), each of shape (M, nrows): the fp64 product and the sum of |x*w|."""
    canon = np.ascontiguousarray(canon, dtype=np.uint8)
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    if x_bits.ndim == 1:
        x_bits = x_bits[None, :]
    M = x_bits.shape[0]
    if rows is None:
        nrows, rp = N, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nrows, rp = rows.shape[0], _ptr(rows)
    y = np.empty((M, nrows), dtype=np.float64)
    a = np.empty((M, nrows), dtype=np.float64)
    rc = lib().oracle_gemm_f64(fmt, N, K, _ptr(canon), _ptr(x_bits), M, x_bits.shape[1], rp, nrows,
                               _ptr(y), _ptr(a))
    if rc:
        raise ValueError(f"oracle_gemm_f64 failed: {rc}")
    return y, a


def silu(g: float) -> float:
    """SiLU(g) = g / (1 + e^-g) in fp64."""
    return float(lib().oracle_silu(float(g)))


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Elementwise SiLU(g) * u in fp64 (the gate/up epilogue)."""
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    if g.shape != u.shape:
        raise ValueError("gate and up results differ in shape")
    h = np.empty_like(g)
    rc = lib().oracle_silu_mul_f64(_ptr(g), _ptr(u), g.size, _ptr(h))
    if rc:
        raise ValueError(f"oracle_silu_mul_f64 failed: {rc}")
    return h


def residual_add(r: np.ndarray, y: np.ndarray) -> np.ndarray:
    """Elementwise r + y in fp64, r an fp32 residual, y an fp64 projection result."""
    r = np.ascontiguousarray(r, dtype=np.float32)
    y = np.ascontiguousarray(y, dtype=np.float64)
    if r.shape != y.shape:
        raise ValueError("residual and projection result differ in shape")
    out = np.empty_like(y)
    rc = lib().oracle_residual_add_f64(_ptr(r), _ptr(y), y.size, _ptr(out))
    if rc:
        raise ValueError(f"oracle_residual_add_f64 failed: {rc}")
    return out


def silu_pair_f64(fmt: int, N: int, K: int, canon_gate: np.ndarray, canon_up: np.ndarray,
                  x_gate: np.ndarray, x_up: np.ndarray, rows=None):
    """The fused gate/up projection: returns (h, g, u, a_g, a_u), each (M, nrows), with
    h = SiLU(g) * u, g and u the fp64 gate and up products, a_g and a_u their sums of |x*w|."""
    g, ag = gemm_f64(fmt, N, K, canon_gate, x_gate, rows=rows)
    u, au = gemm_f64(fmt, N, K, canon_up, x_up, rows=rows)
    return silu_mul(g, u), g, u, ag, au


def quantize_x_i8(x_bits: np.ndarray):
    """Per-128-group int8 quantization of fp16 activations: returns (q int8 [M,K], a fp32
    [M,K/128], qsum int32 [M,K/128])."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    if x_bits.ndim == 1:
        x_bits = x_bits[None, :]
    M, K = x_bits.shape
    q = np.empty((M, K), dtype=np.int8)
    a = np.empty((M, K // 128), dtype=np.float32)
    qs = np.empty((M, K // 128), dtype=np.int32)
    rc = lib().oracle_quantize_x_i8(_ptr(x_bits), M, K, K, _ptr(q), _ptr(a), _ptr(qs))
    if rc:
        raise ValueError(f"oracle_quantize_x_i8 failed: {rc}")
    return q, a, qs


def tq2_i8_f64(N: int, K: int, canon: np.ndarray, q: np.ndarray, a: np.ndarray, rows=None):
    """TQ2 rows times int8 activations: returns (y, t), each (M, nrows)."""
    canon = np.ascontiguousarray(canon, dtype=np.uint8)
    q = np.ascontiguousarray(q, dtype=np.int8)
    a = np.ascontiguousarray(a, dtype=np.float32)
    M = q.shape[0]
    if rows is None:
        nrows, rp = N, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nrows, rp = rows.shape[0], _ptr(rows)
    y = np.empty((M, nrows), dtype=np.float64)
    t = np.empty((M, nrows), dtype=np.float64)
    rc = lib().oracle_tq2_i8_f64(N, K, _ptr(canon), _ptr(q), _ptr(a), M, rp, nrows, _ptr(y), _ptr(t))
    if rc:
        raise ValueError(f"oracle_tq2_i8_f64 failed: {rc}")
    return y, t
