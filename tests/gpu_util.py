"""Helpers of the GPU tests: seeded weights uploaded in the prepared layout, and the parity bar."""
import concurrent.futures as cf
import os
import sys

import numpy as np

import oracle

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
    """The prepared weights on the device, bound (a Weight view that keeps its buffer alive)."""
    import torch
    prep = W.wqd_prepare_host(fmt, N, K, canon)
    return W.wqd_bind(fmt, N, K, torch.from_numpy(prep).to("cuda"))


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


def run_gemm(w, x_dev, M, y=None, stream=None):
    y = new_y(M, w.N) if y is None else y
    ws = workspace(W.wqd_workspace_bytes(w, M))
    W.wqd_gemm(w, x_dev, y, ws, stream)
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


_POOL = None


def oracle_gemm_all(fmt, N, K, canon, x_bits, rows=None):
    """The oracle's (y, sum |x*w|) on every row (or the given rows), the rows cut into one range per
    host thread (the oracle's C entry point releases the GIL)."""
    global _POOL
    T = max(1, len(os.sched_getaffinity(0)))
    if _POOL is None:
        _POOL = cf.ThreadPoolExecutor(T)
    rows = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    parts = [r for r in np.array_split(rows, T) if r.size]
    res = list(_POOL.map(lambda r: oracle.gemm_f64(fmt, N, K, canon, x_bits, rows=r), parts))
    return np.concatenate([y for y, _ in res], axis=1), np.concatenate([a for _, a in res], axis=1)


def aq2x8_cancelling(canon, N, K, key, rel=1e-3):
    """AQ2x8 canonical bytes whose two codebooks nearly cancel, C1[c] = fp16(-C0[c] * (1 + rel*n)) with
    n ~ N(0,1), and c1 = c0 in every group: each weight is about `rel` times the entries it is the
    sum of.  A path that rounds a per-group sum of products to fp16 before the two codebooks'
    terms meet makes errors of about 2^-12 of the terms, far above 2e-3 * sum |x*w| here."""
    canon = np.array(canon, dtype=np.uint8, copy=True)
    C = canon[:8192].view("<u2").astype(np.uint16).view(np.float16).astype(np.float64).reshape(2, 256, 8)
    g = I.rng(*[int(k) for k in key], 30)
    C1 = -C[0] * (1.0 + rel * g.standard_normal((256, 8)))
    canon[4096:8192] = I.f16_bits(C1).astype("<u2").view(np.uint8).reshape(-1)
    codes = canon[8192 + 2 * N:].reshape(N, K // 8, 2)
    codes[:, :, 1] = codes[:, :, 0]
    return canon
