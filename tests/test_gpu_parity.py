"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

* Decode: wqd_dequant_f32 must equal oracle_dequant_f32 bit for bit.
* Multiply: |y_gpu - y_ref| <= 2e-3 * sum_k |x_k w_nk| + 1e-6 for every output, on shapes that
  span several 64-row tiles with a ragged last tile and, for the byte formats, a partial last
  16-byte chunk; outputs are poisoned with NaN before each call and the padding of y (ldy > N)
  must stay untouched.
* Determinism: two calls give the same bits.
"""
import numpy as np
import pytest

import oracle
from weight_quantized_decode_amd import _lib as W
from weight_quantized_decode_amd import inputs as I

from gpu_util import check_parity, new_y, note, run_gemm, upload_weight, upload_x, workspace

pytestmark = pytest.mark.gpu

SMALL = [
    (I.Q4_0, 200, 1024), (I.Q4_0, 64, 32), (I.Q4_0, 130, 4128),
    (I.CB4, 200, 1000), (I.CB4, 1, 2), (I.CB4, 77, 4098),
    (I.CB8, 200, 1001), (I.CB8, 65, 16), (I.CB8, 3, 1),
    (I.TQ2, 200, 1280), (I.TQ2, 70, 128), (I.TQ2, 130, 17408),
    (I.AQ2X8, 200, 1000), (I.AQ2X8, 64, 8), (I.AQ2X8, 129, 8192),
    (I.AQ1X16, 200, 1024), (I.AQ1X16, 65, 8), (I.AQ1X16, 130, 8200),
]


@pytest.mark.parametrize("fmt,N,K", SMALL)
def test_dequant_bit_exact(fmt, N, K):
    import torch
    note(f"dequant fmt={fmt} N={N} K={K}")
    canon = I.gen_weight(fmt, N, K, (11, fmt, N, K))
    w = upload_weight(fmt, N, K, canon)
    out = torch.full((N, K), float("nan"), dtype=torch.float32, device="cuda")
    W.wqd_dequant_f32(fmt, N, K, w, out)
    W.wqd_stream_check()
    got = out.cpu().numpy()
    ref = oracle.dequant_f32(fmt, N, K, canon)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_dequant_bit_exact_with_subnormal_scales():
    import torch
    # Q4_0 and TQ2 blocks whose scales are fp16 subnormals, and AQ2x8 codebooks with subnormals
    for fmt, N, K in [(I.Q4_0, 64, 256), (I.TQ2, 64, 256)]:
        note(f"dequant subnormal fmt={fmt}")
        canon = I.gen_weight(fmt, N, K, (12, fmt), scale_sigma=2.0 ** -16)
        w = upload_weight(fmt, N, K, canon)
        out = torch.empty((N, K), dtype=torch.float32, device="cuda")
        W.wqd_dequant_f32(fmt, N, K, w, out)
        W.wqd_stream_check()
        ref = oracle.dequant_f32(fmt, N, K, canon)
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    N, K = 64, 64
    canon = I.gen_weight(I.AQ2X8, N, K, (13,))
    C = canon[:8192].view(np.uint16).copy()
    C[::7] = np.arange(1, C[::7].size + 1, dtype=np.uint16) % 1024  # subnormal entries
    canon = np.concatenate([C.view(np.uint8), canon[8192:]])
    w = upload_weight(I.AQ2X8, N, K, canon)
    out = torch.empty((N, K), dtype=torch.float32, device="cuda")
    W.wqd_dequant_f32(I.AQ2X8, N, K, w, out)
    W.wqd_stream_check()
    ref = oracle.dequant_f32(I.AQ2X8, N, K, canon)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("fmt,N,K", SMALL)
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
def test_gemm_parity_small(fmt, N, K, M):
    note(f"gemm fmt={fmt} N={N} K={K} M={M}")
    canon = I.gen_weight(fmt, N, K, (14, fmt, N, K))
    x = I.gen_x(M, K, (14, fmt, N, K, M))
    w = upload_weight(fmt, N, K, canon)
    y = run_gemm(fmt, N, K, w, upload_x(x), M)
    yref, aref = oracle.gemm_f64(fmt, N, K, canon, x)
    check_parity(y.cpu().numpy(), yref, aref, f"fmt={fmt} N={N} K={K} M={M}")


@pytest.mark.parametrize("fmt", [I.Q4_0, I.CB4, I.CB8, I.TQ2, I.AQ2X8, I.AQ1X16])
def test_gemm_strided_x_and_y(fmt):
    N, K, M = 150, 1024, 3
    note(f"gemm strided fmt={fmt}")
    canon = I.gen_weight(fmt, N, K, (15, fmt))
    x = I.gen_x(M, K, (15, fmt))
    w = upload_weight(fmt, N, K, canon)
    xd = upload_x(x, ldx=K + 40)
    y = new_y(M, N, ldy=N + 10, fill=-7.0)
    run_gemm(fmt, N, K, w, xd, M, y=y)
    full = y.as_strided((M, N + 10), (N + 10, 1)).cpu().numpy()
    assert np.all(full[:, N:] == -7.0)  # padding of y untouched
    yref, aref = oracle.gemm_f64(fmt, N, K, canon, x)
    check_parity(full[:, :N], yref, aref, f"strided fmt={fmt}")


@pytest.mark.parametrize("fmt", [I.Q4_0, I.CB4, I.CB8, I.TQ2, I.AQ2X8, I.AQ1X16])
def test_gemm_deterministic(fmt):
    N, K, M = 300, 2048, 2
    note(f"gemm determinism fmt={fmt}")
    canon = I.gen_weight(fmt, N, K, (16, fmt))
    x = upload_x(I.gen_x(M, K, (16, fmt)))
    w = upload_weight(fmt, N, K, canon)
    a = run_gemm(fmt, N, K, w, x, M).cpu().numpy()
    b = run_gemm(fmt, N, K, w, x, M).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("fmt", [I.Q4_0, I.CB4, I.CB8, I.TQ2, I.AQ2X8, I.AQ1X16])
def test_gemm_one_hot_and_zero_activations(fmt):
    # One-hot x returns a column of the dequantized matrix: exactly for the formats whose weights
    # are exact in fp16 arithmetic; for AQ2x8 the kernel adds the two fp16 codebook entries in
    # fp16 (one rounding, relative error <= 2^-11) before the fp32 product.  Zero x returns zero.
    import torch
    N, K = 128, 512
    note(f"gemm one-hot fmt={fmt}")
    canon = I.gen_weight(fmt, N, K, (17, fmt))
    w = upload_weight(fmt, N, K, canon)
    k = 301
    x = np.zeros((2, K), dtype=np.uint16)
    x[0, k] = 0x3C00  # 1.0
    y = run_gemm(fmt, N, K, w, upload_x(x), 2).cpu().numpy()
    W64 = oracle.decode_f64(fmt, N, K, canon)
    assert np.all(y[1] == 0.0)
    rtol = 2.0 ** -11 + 2.0 ** -23 if fmt == I.AQ2X8 else 1e-7
    assert np.all(np.abs(y[0] - W64[:, k]) <= rtol * np.abs(W64[:, k]))


@pytest.mark.parametrize("fmt", [I.Q4_0, I.CB4, I.CB8, I.TQ2, I.AQ2X8, I.AQ1X16])
def test_workspace_reuse_leaves_counters_zero(fmt):
    # The split-K slice counters in the workspace must be back at zero after every call, so one
    # workspace serves many calls (and differently shaped ones) in a row.
    import torch
    note(f"workspace reuse fmt={fmt}")
    shapes = [(300, 2048, 2), (130, 1024, 1), (300, 2048, 3)]
    need = max(W.wqd_gemm_workspace_bytes(fmt, N, K, M) for N, K, M in shapes)
    ws = workspace(need)
    for i, (N, K, M) in enumerate(shapes):
        canon = I.gen_weight(fmt, N, K, (18, fmt, i))
        x = I.gen_x(M, K, (18, fmt, i))
        w = upload_weight(fmt, N, K, canon)
        y = new_y(M, N)
        W.wqd_gemm(fmt, N, K, w, upload_x(x), y, ws)
        W.wqd_stream_check()
        yref, aref = oracle.gemm_f64(fmt, N, K, canon, x)
        check_parity(y.cpu().numpy(), yref, aref, f"reuse fmt={fmt} call {i}")
        rg = (N + 63) // 64
        assert int(ws[: 4 * rg].view(torch.int32).abs().sum().item()) == 0
