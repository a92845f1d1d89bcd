"""Helpers of the GPU tests: seeded weights uploaded in the prepared layout, and the parity bar."""
import sys

import numpy as np

from weight_quantized_decode_amd import _lib as W
from weight_quantized_decode_amd import inputs as I

# |y_gpu - y_ref| <= REL * sum_k |x_k w_nk| + ABS, fp32 accumulation on the GPU.
REL_TOL = 2e-3
ABS_TOL = 1e-6


def note(msg: str) -> None:
    """Name the case about to run on the GPU (flushed, so it survives a crash)."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def upload_weight(fmt, N, K, canon):
    import torch
    prep = W.wqd_prepare_host(fmt, N, K, canon)
    return torch.from_numpy(prep).to("cuda")


def upload_x(x_bits, ldx=None):
    import torch
    M, K = x_bits.shape
    ldx = K + (K & 1) if ldx is None else ldx  # the library needs an even row stride
    buf = np.zeros((M, ldx), dtype=np.uint16)
    buf[:, :K] = x_bits
    t = torch.from_numpy(buf.view(np.int16)).to("cuda")
    return t[:, :K] if ldx == K else t.as_strided((M, K), (ldx, 1))


def new_y(M, N, ldy=None, fill=float("nan")):
    import torch
    ldy = N if ldy is None else ldy
    y = torch.full((M, ldy), fill, dtype=torch.float32, device="cuda")
    return y if ldy == N else y.as_strided((M, N), (ldy, 1))


def workspace(nbytes):
    """Device workspace, zero-filled before first use as the library requires."""
    import torch
    return torch.zeros(max(int(nbytes), 16), dtype=torch.uint8, device="cuda")


def run_gemm(fmt, N, K, w, x_dev, M, y=None, stream=None):
    import torch
    y = new_y(M, N) if y is None else y
    ws = workspace(W.wqd_gemm_workspace_bytes(fmt, N, K, M))
    W.wqd_gemm(fmt, N, K, w, x_dev, y, ws, stream)
    W.wqd_stream_check(stream)
    return y


def check_parity(y_gpu, y_ref, a_ref, what=""):
    y = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y - y_ref)
    bound = REL_TOL * a_ref + ABS_TOL
    bad = ~(err <= bound)  # NaN counts as bad
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} outputs outside the bound; first {idx.tolist()}: "
                             f"gpu {y[tuple(idx[0])]} ref {y_ref[tuple(idx[0])]} bound {bound[tuple(idx[0])]}")
    return float(np.max(err / (a_ref + 1e-30)))
