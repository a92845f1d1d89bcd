"""Thin ctypes binding of libwqd.so (include/wqd.h): argument marshalling only.

Every function keeps the name of the C entry point it wraps.  Device buffers are torch tensors
(used for memory and streams only); host buffers are numpy arrays.  A non-zero status raises
WqdError.  There is no fallback: if libwqd.so is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SO_PATH = os.path.join(_HERE, "libwqd.so")

WQD_Q4_0, WQD_CB4, WQD_CB8, WQD_TQ2, WQD_AQ2X8, WQD_AQ1X16 = 1, 2, 3, 4, 5, 6
WQD_OK, WQD_EINVAL, WQD_ESHAPE, WQD_EALIGN, WQD_ESPACE, WQD_EHIP, WQD_ESTALE = 0, -1, -2, -3, -4, -5, -6
WQD_ORDERED, WQD_PERSISTENT, WQD_FUSED = 0, 1, 2
WQD_BATCH_INVARIANT = 0x10
WQD_INT8_ACTIVATIONS = 0x20
WQD_EPI_NONE, WQD_EPI_ADD, WQD_EPI_SILU_GATE, WQD_EPI_SILU_UP = 0, 1, 2, 3
WQD_MAX_M = 8
WQD_MAX_M_VERIFY = 16
WQD_MAX_N = 1 << 30
WQD_MAX_K = 1 << 30

EXPORTED = [
    "wqd_canonical_bytes", "wqd_prepared_bytes", "wqd_prepare_host", "wqd_bind", "wqd_workspace_bytes",
    "wqd_gemm", "wqd_dequant_f32", "wqd_stack_workspace_bytes", "wqd_stack_setup",
    "wqd_run_projections", "wqd_run_projections_timed", "wqd_stack_launches", "wqd_stream_check",
    "wqd_last_hip_error", "wqd_status_str", "wqd_gemm_i8_workspace_bytes", "wqd_gemm_i8", "wqd_quantize_i8",
    "wqd_gemm_noalloc",
]
WQD_NOALLOC_MAX_BYTES = 16 << 20


class WqdError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().wqd_status_str(status).decode()
        if status == WQD_EHIP:
            msg += f" (hipError_t {lib().wqd_last_hip_error()})"
        super().__init__(f"{fn} failed with status {status}: {msg}")


class wqd_weight(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("N", ctypes.c_int32), ("K", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("codebooks", ctypes.c_void_p),
                ("code_row_bytes", ctypes.c_int64), ("scale_row_elems", ctypes.c_int64)]


class wqd_proj(ctypes.Structure):
    _fields_ = [("w", ctypes.POINTER(wqd_weight)), ("epi", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("x", ctypes.c_void_p), ("ldx", ctypes.c_int64), ("y", ctypes.c_void_p), ("ldy", ctypes.c_int64)]


class Weight:
    """A bound wqd_weight view and the device buffer it points into (kept alive with it)."""

    def __init__(self, view: wqd_weight, buf=None):
        self.view = view
        self.buf = buf

    @property
    def fmt(self) -> int:
        return self.view.fmt

    @property
    def N(self) -> int:
        return self.view.N

    @property
    def K(self) -> int:
        return self.view.K

    def ref(self):
        return ctypes.byref(self.view)


_lib = None


def lib() -> ctypes.CDLL:
    """Load libwqd.so (raises OSError when it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(SO_PATH):
            raise OSError(f"{SO_PATH} is missing: build it with weight_quantized_decode_amd.build.build()")
        L = ctypes.CDLL(SO_PATH)
        i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        sig = {
            "wqd_canonical_bytes": (i64, [ctypes.c_int, i64, i64]),
            "wqd_prepared_bytes": (i64, [ctypes.c_int, i64, i64]),
            "wqd_prepare_host": (ctypes.c_int, [ctypes.c_int, i64, i64, vp, i64, vp, i64]),
            "wqd_bind": (ctypes.c_int, [ctypes.c_int, i64, i64, vp, ctypes.POINTER(wqd_weight)]),
            "wqd_workspace_bytes": (i64, [ctypes.POINTER(wqd_weight), i64]),
            "wqd_gemm": (ctypes.c_int, [ctypes.POINTER(wqd_weight), vp, i64, i64, vp, i64, vp, i64, vp]),
            "wqd_gemm_noalloc": (ctypes.c_int, [ctypes.POINTER(wqd_weight), vp, i64, i64, vp, i64, vp]),
            "wqd_dequant_f32": (ctypes.c_int, [ctypes.POINTER(wqd_weight), vp, vp]),
            "wqd_gemm_i8_workspace_bytes": (i64, [ctypes.POINTER(wqd_weight), i64]),
            "wqd_gemm_i8": (ctypes.c_int, [ctypes.POINTER(wqd_weight), vp, i64, i64, vp, i64, vp, i64, vp]),
            "wqd_quantize_i8": (ctypes.c_int, [vp, i64, i64, i64, vp, vp, vp, vp]),
            "wqd_stack_workspace_bytes": (i64, [ctypes.POINTER(wqd_proj), i32, i64]),
            "wqd_stack_setup": (ctypes.c_int, [ctypes.POINTER(wqd_proj), i32, i64, i32, vp, i64, vp]),
            "wqd_run_projections": (ctypes.c_int, [ctypes.POINTER(wqd_proj), i32, i64, i32, vp, i64, vp]),
            "wqd_run_projections_timed": (ctypes.c_int, [ctypes.POINTER(wqd_proj), i32, i64, i32, vp, i64, vp,
                                                         ctypes.POINTER(ctypes.c_void_p), i32]),
            "wqd_stack_launches": (ctypes.c_int, [ctypes.POINTER(wqd_proj), i32, i64, i32]),
            "wqd_stream_check": (ctypes.c_int, [vp]),
            "wqd_last_hip_error": (ctypes.c_int, []),
            "wqd_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, status: int) -> int:
    if status < 0:
        raise WqdError(fn, status)
    return status


def _dptr(t) -> Optional[int]:
    """Device pointer of a torch tensor (None passes NULL)."""
    if t is None:
        return None
    return t.data_ptr()


def _mat(t, what: str, rows: Optional[int], cols: int, elem: int, float_ok: bool):
    """Checks a 2-D device matrix argument: on the GPU, `elem`-byte elements (fp16 bits as int16 or
    float16, or float32), unit inner stride, the expected shape; returns nothing."""
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what}: a CUDA tensor is required")
    ok = {2: (torch.int16, torch.float16), 4: (torch.float32,)}[elem]
    if t.dtype not in ok:
        raise TypeError(f"{what}: dtype {t.dtype}, expected one of {ok}")
    if t.dim() != 2 or t.stride(1) != 1 or t.shape[1] != cols or (rows is not None and t.shape[0] != rows):
        raise ValueError(f"{what}: shape {tuple(t.shape)} strides {t.stride()}, expected ({rows if rows else 'M'}, {cols}) "
                         f"with unit inner stride")


def _ws(t, what: str = "workspace"):
    import torch
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{what}: a contiguous CUDA tensor is required")


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------------- layout (host only)

def wqd_canonical_bytes(fmt: int, N: int, K: int) -> int:
    return _check("wqd_canonical_bytes", lib().wqd_canonical_bytes(fmt, N, K))


def wqd_prepared_bytes(fmt: int, N: int, K: int) -> int:
    return _check("wqd_prepared_bytes", lib().wqd_prepared_bytes(fmt, N, K))


def wqd_prepare_host(fmt: int, N: int, K: int, canonical: np.ndarray) -> np.ndarray:
    canonical = np.ascontiguousarray(canonical, dtype=np.uint8)
    out = np.empty(wqd_prepared_bytes(fmt, N, K), dtype=np.uint8)
    _check("wqd_prepare_host", lib().wqd_prepare_host(fmt, N, K, canonical.ctypes.data, canonical.nbytes,
                                                      out.ctypes.data, out.nbytes))
    return out


# ------------------------------------------------------------------------- bound weights

def wqd_bind(fmt: int, N: int, K: int, prepared) -> Weight:
    """The plane view of a prepared weight buffer (a device tensor, or a raw address)."""
    view = wqd_weight()
    if not isinstance(prepared, int):
        import torch
        if not isinstance(prepared, torch.Tensor) or not prepared.is_cuda or not prepared.is_contiguous():
            raise TypeError("wqd_bind: a contiguous CUDA tensor (or a raw device address) is required")
        need = wqd_prepared_bytes(fmt, N, K)
        if prepared.numel() * prepared.element_size() < need:
            raise ValueError(f"wqd_bind: buffer of {prepared.numel() * prepared.element_size()} bytes, "
                             f"the prepared layout takes {need}")
    addr = prepared if isinstance(prepared, int) else _dptr(prepared)
    _check("wqd_bind", lib().wqd_bind(fmt, N, K, addr, ctypes.byref(view)))
    return Weight(view, None if isinstance(prepared, int) else prepared)


# ------------------------------------------------------------------------- one projection

def wqd_workspace_bytes(w: Weight, M: int) -> int:
    return _check("wqd_workspace_bytes", lib().wqd_workspace_bytes(w.ref(), M))


def wqd_gemm(w: Weight, x, y, workspace=None, stream=None) -> None:
    """y[M, N] (fp32) = x[M, K] (fp16) times the dequantized W[N, K]; x and y may have row strides."""
    _mat(x, "x", None, w.K, 2, True)
    M = x.shape[0]
    _mat(y, "y", M, w.N, 4, True)
    _ws(workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("wqd_gemm", lib().wqd_gemm(w.ref(), _dptr(x), M, x.stride(0), _dptr(y), y.stride(0), _dptr(workspace),
                                      ws_bytes, _stream(stream)))


def wqd_gemm_noalloc(w: Weight, x, y, stream=None) -> None:
    """wqd_gemm without a workspace: the library's per-GPU scratch array serves as one."""
    _mat(x, "x", None, w.K, 2, True)
    M = x.shape[0]
    _mat(y, "y", M, w.N, 4, True)
    _check("wqd_gemm_noalloc", lib().wqd_gemm_noalloc(w.ref(), _dptr(x), M, x.stride(0), _dptr(y), y.stride(0),
                                                      _stream(stream)))


def wqd_gemm_i8_workspace_bytes(w: Weight, M: int) -> int:
    return _check("wqd_gemm_i8_workspace_bytes", lib().wqd_gemm_i8_workspace_bytes(w.ref(), M))


def wqd_gemm_i8(w: Weight, x, y, workspace, stream=None) -> None:
    """TQ2 times int8-quantized x (quantized inside the call); x and y may have row strides."""
    _mat(x, "x", None, w.K, 2, True)
    M = x.shape[0]
    _mat(y, "y", M, w.N, 4, True)
    _ws(workspace)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("wqd_gemm_i8", lib().wqd_gemm_i8(w.ref(), _dptr(x), M, x.stride(0), _dptr(y), y.stride(0),
                                            _dptr(workspace), ws_bytes, _stream(stream)))


def wqd_quantize_i8(x, q, a, qsum, stream=None) -> None:
    """q (int8 [M, K]), a (fp32 [M, K/128]) and qsum (int32 [M, K/128]) of fp16 x [M, K]."""
    import torch
    M, K = x.shape
    _mat(x, "x", M, K, 2, True)
    for t, name, dt, n in ((q, "q", torch.int8, M * K), (a, "a", torch.float32, M * (K // 128)),
                           (qsum, "qsum", torch.int32, M * (K // 128))):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != dt or not t.is_contiguous() or t.numel() != n:
            raise ValueError(f"{name}: a contiguous CUDA {dt} tensor of {n} elements is required")
    _check("wqd_quantize_i8", lib().wqd_quantize_i8(_dptr(x), M, K, x.stride(0), _dptr(q), _dptr(a), _dptr(qsum),
                                                    _stream(stream)))


def wqd_dequant_f32(w: Weight, out, stream=None) -> None:
    import torch
    if not isinstance(out, torch.Tensor) or not out.is_cuda or out.dtype != torch.float32 or \
            not out.is_contiguous() or out.numel() != w.N * w.K:
        raise ValueError(f"out: a contiguous CUDA float32 tensor of {w.N} x {w.K} elements is required")
    _check("wqd_dequant_f32", lib().wqd_dequant_f32(w.ref(), _dptr(out), _stream(stream)))


# ------------------------------------------------------------------------- layer / stack

def make_proj_array(projs: Sequence[dict]):
    """projs: dicts with w (a Weight, or a prepared device tensor together with fmt, N and K), x, y
    (torch tensors) and optionally epi (a WQD_EPI_* value; y may be None for a WQD_EPI_SILU_UP
    entry); returns a ctypes array of wqd_proj.  The array holds raw device pointers and keeps the
    weight views alive; the caller keeps the tensors alive while it is used."""
    arr = (wqd_proj * len(projs))()
    keep = []
    for i, p in enumerate(projs):
        w = p["w"]
        if not isinstance(w, Weight):
            w = wqd_bind(p["fmt"], p["N"], p["K"], w)
        keep.append(w)
        arr[i].w = ctypes.pointer(w.view)
        arr[i].epi = p.get("epi", WQD_EPI_NONE)
        _mat(p["x"], f"entry {i} x", None, w.K, 2, True)
        arr[i].x = p["x"].data_ptr()
        arr[i].ldx = p["x"].stride(0)
        y = p.get("y")
        if y is not None:
            _mat(y, f"entry {i} y", p["x"].shape[0], w.N, 4, True)
        arr[i].y = None if y is None else y.data_ptr()
        arr[i].ldy = 0 if y is None else y.stride(0)
    arr._keep = keep
    return arr


def wqd_stack_workspace_bytes(arr, M: int) -> int:
    return _check("wqd_stack_workspace_bytes", lib().wqd_stack_workspace_bytes(arr, len(arr), M))


def wqd_stack_setup(arr, M: int, workspace, stream=None, mode: int = WQD_PERSISTENT) -> None:
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("wqd_stack_setup", lib().wqd_stack_setup(arr, len(arr), M, mode, _dptr(workspace), ws_bytes,
                                                    _stream(stream)))


def wqd_run_projections(arr, M: int, mode: int, workspace, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("wqd_run_projections", lib().wqd_run_projections(arr, len(arr), M, mode, _dptr(workspace), ws_bytes,
                                                            _stream(stream)))


def wqd_stack_launches(arr, M: int, mode: int = WQD_PERSISTENT) -> int:
    return _check("wqd_stack_launches", lib().wqd_stack_launches(arr, len(arr), M, mode))


def wqd_run_projections_timed(arr, M: int, mode: int, workspace, events, stream=None) -> None:
    """events: sequence of raw hipEvent_t handles (ints), 2 per kernel launch."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ev = (ctypes.c_void_p * len(events))(*events)
    _check("wqd_run_projections_timed", lib().wqd_run_projections_timed(
        arr, len(arr), M, mode, _dptr(workspace), ws_bytes, _stream(stream), ev, len(events)))


def wqd_stream_check(stream=None) -> None:
    _check("wqd_stream_check", lib().wqd_stream_check(_stream(stream)))


def wqd_status_str(status: int) -> str:
    return lib().wqd_status_str(status).decode()
