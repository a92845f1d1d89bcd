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

from gpu_util import aq2x8_cancelling, check_parity, new_y, note, run_gemm, upload_weight, upload_x, workspace

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
    W.wqd_dequant_f32(w, out)
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
        W.wqd_dequant_f32(w, out)
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
    W.wqd_dequant_f32(w, out)
    W.wqd_stream_check()
    ref = oracle.dequant_f32(I.AQ2X8, N, K, canon)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("fmt,N,K", SMALL)
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_gemm_parity_small(fmt, N, K, M):
    note(f"gemm fmt={fmt} N={N} K={K} M={M}")
    canon = I.gen_weight(fmt, N, K, (14, fmt, N, K))
    x = I.gen_x(M, K, (14, fmt, N, K, M))
    w = upload_weight(fmt, N, K, canon)
    y = run_gemm(w, upload_x(x), M)
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
    run_gemm(w, xd, M, y=y)
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
    a = run_gemm(w, x, M).cpu().numpy()
    b = run_gemm(w, x, M).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("fmt", [I.Q4_0, I.CB4, I.CB8, I.TQ2, I.AQ2X8, I.AQ1X16])
@pytest.mark.parametrize("M", [1, 2, 3])
def test_gemm_one_hot_and_zero_activations(fmt, M):
    # One-hot x returns a column of the dequantized matrix.  The weights of Q4_0, CB4, CB8, TQ2 and
    # AQ1X16 are exact in fp32, so the column is exact.  An AQ2x8 weight is s * (C0 + C1): the
    # kernels form C0 + C1 in fp32 (the one nonzero lookup-table term or product of each codebook,
    # added once) and scale it once, which is exactly the debug dequant's fp32(fp32(C0 + C1) * s):
    # equal bits, and within two fp32 roundings of the exact weight.  Zero x returns zero.
    # (AQ2x8: M = 1 and 2 take the lookup-table kernels, M = 3 the matrix-core one; rows past 0
    # are zero.)
    N, K = 128, 512
    note(f"gemm one-hot fmt={fmt} M={M}")
    canon = I.gen_weight(fmt, N, K, (17, fmt))
    w = upload_weight(fmt, N, K, canon)
    k = 301
    x = np.zeros((M, K), dtype=np.uint16)
    x[0, k] = 0x3C00  # 1.0
    y = run_gemm(w, upload_x(x), M).cpu().numpy()
    W64 = oracle.decode_f64(fmt, N, K, canon)
    if M > 1:
        assert np.all(y[1:] == 0.0)
    rtol = 2.0 ** -23 + 2.0 ** -46 if fmt == I.AQ2X8 else 1e-7
    assert np.all(np.abs(y[0] - W64[:, k]) <= rtol * np.abs(W64[:, k]))
    if fmt == I.AQ2X8:
        dq = oracle.dequant_f32(fmt, N, K, canon)[:, k]
        assert np.array_equal(y[0].view(np.uint32), dq.view(np.uint32))
    yz = run_gemm(w, upload_x(np.zeros((M, K), dtype=np.uint16)), M).cpu().numpy()
    assert np.all(yz == 0.0)


@pytest.mark.parametrize("N,K", [(200, 1000), (129, 8192)])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_aq2x8_cancelling_codebooks(N, K, M):
    # Codebooks with C1 ~ -C0 and c1 = c0 everywhere: every weight is about 1e-3 of the entries
    # it is the sum of, so the bound 2e-3 * sum |x*w| is about 2e-6 of the group sums the kernels
    # form.  fp16 rounding of those sums (about 2^-12 of them) fails it; fp32 sums pass.
    note(f"aq2x8 cancelling N={N} K={K} M={M}")
    canon = aq2x8_cancelling(I.gen_weight(I.AQ2X8, N, K, (19, N, K)), N, K, (19, N, K))
    x = I.gen_x(M, K, (19, N, K, M))
    w = upload_weight(I.AQ2X8, N, K, canon)
    y = run_gemm(w, upload_x(x), M)
    yref, aref = oracle.gemm_f64(I.AQ2X8, N, K, canon, x)
    check_parity(y.cpu().numpy(), yref, aref, f"cancelling N={N} K={K} M={M}")


@pytest.mark.parametrize("M", [1, 4, 8])
def test_aq2x8_cancelling_codebooks_batch_invariant(M):
    # the same inputs through the batch-invariant list path (the matrix-core kernel at every M)
    N, K = 129, 8192
    note(f"aq2x8 cancelling batch-invariant M={M}")
    canon = aq2x8_cancelling(I.gen_weight(I.AQ2X8, N, K, (20,)), N, K, (20,))
    x = I.gen_x(M, K, (20, M))
    y = new_y(M, N)
    dev = [dict(fmt=I.AQ2X8, N=N, K=K, w=upload_weight(I.AQ2X8, N, K, canon), x=upload_x(x), y=y)]
    arr = W.make_proj_array(dev)
    ws = workspace(W.wqd_stack_workspace_bytes(arr, M))
    W.wqd_run_projections(arr, M, W.WQD_ORDERED | W.WQD_BATCH_INVARIANT, ws)
    W.wqd_stream_check()
    yref, aref = oracle.gemm_f64(I.AQ2X8, N, K, canon, x)
    check_parity(y.cpu().numpy(), yref, aref, f"cancelling batch-invariant M={M}")


TQ2_CODE3 = [(130, 1280), (70, 17408)]


@pytest.mark.parametrize("N,K", TQ2_CODE3)
def test_tq2_code3_dequant_bit_exact(N, K):
    # code 3 decodes to +2d ("Anatomy of a PQ2_0 block"); the workloads never draw it
    import torch
    note(f"tq2 code 3 dequant N={N} K={K}")
    canon = I.gen_weight(I.TQ2, N, K, (21, N, K), tq2_code3=0.1)
    w = upload_weight(I.TQ2, N, K, canon)
    out = torch.full((N, K), float("nan"), dtype=torch.float32, device="cuda")
    W.wqd_dequant_f32(w, out)
    W.wqd_stream_check()
    ref = oracle.dequant_f32(I.TQ2, N, K, canon)
    assert (ref > 0).any() and np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("N,K", TQ2_CODE3)
@pytest.mark.parametrize("M", [1, 2, 5, 8])
def test_tq2_code3_gemm_parity(N, K, M):
    # M = 1: the vector-ALU decode (fp16-subnormal fields); M > 1: the exact-fp16 matrix-core decode
    note(f"tq2 code 3 gemm N={N} K={K} M={M}")
    canon = I.gen_weight(I.TQ2, N, K, (22, N, K), tq2_code3=0.1)
    x = I.gen_x(M, K, (22, N, K, M))
    w = upload_weight(I.TQ2, N, K, canon)
    y = run_gemm(w, upload_x(x), M)
    yref, aref = oracle.gemm_f64(I.TQ2, N, K, canon, x)
    check_parity(y.cpu().numpy(), yref, aref, f"tq2 code 3 N={N} K={K} M={M}")


@pytest.mark.parametrize("fmt", [I.Q4_0, I.CB4, I.CB8, I.TQ2, I.AQ2X8, I.AQ1X16])
def test_workspace_reuse_leaves_counters_zero(fmt):
    # The split-K slice counters in the workspace must be back at zero after every call, so one
    # workspace serves many calls (and differently shaped ones) in a row.
    import torch
    note(f"workspace reuse fmt={fmt}")
    shapes = [(300, 2048, 2), (130, 1024, 1), (300, 2048, 3)]
    ws_ = [upload_weight(fmt, N, K, I.gen_weight(fmt, N, K, (18, fmt, i))) for i, (N, K, M) in enumerate(shapes)]
    need = max(W.wqd_workspace_bytes(w, M) for w, (N, K, M) in zip(ws_, shapes))
    ws = workspace(need)
    for i, (N, K, M) in enumerate(shapes):
        canon = I.gen_weight(fmt, N, K, (18, fmt, i))
        x = I.gen_x(M, K, (18, fmt, i))
        w = ws_[i]
        y = new_y(M, N)
        W.wqd_gemm(w, upload_x(x), y, ws)
        W.wqd_stream_check()
        yref, aref = oracle.gemm_f64(fmt, N, K, canon, x)
        check_parity(y.cpu().numpy(), yref, aref, f"reuse fmt={fmt} call {i}")
        rg = (N + 63) // 64
        assert int(ws[: 4 * rg].view(torch.int32).abs().sum().item()) == 0
