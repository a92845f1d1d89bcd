"""TQ2 with int8 activations ("Making a ternary reasoning model fast in vLLM", "Why small integers
are a good fit") against the CPU oracle, through the C ABI.

* The quantizer (wqd_quantize_i8) equals oracle_quantize_x_i8 bit for bit: q, a and the block
  sums of q (both sides take the fp32 absmax scale and the nearest-even rounding in fp32).
* wqd_gemm_i8 equals the oracle's int8 product up to fp32 rounding: the block sums are exact
  integers on both sides, so |y - y_ref| <= (K/128 + 16) * 2^-23 * sum_b |d_b a_b isum_b|.
* Against the exact product it stays within the quantization bound sum_k |w_k| a(k) / 2.
"""
import numpy as np
import pytest

import oracle
from weight_quantized_decode_amd import _lib as W
from weight_quantized_decode_amd import inputs as I

from gpu_util import new_y, note, upload_weight, upload_x, workspace

pytestmark = pytest.mark.gpu

SHAPES = [(200, 1280), (70, 128), (130, 17408), (64, 5120)]


@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("K", [128, 1280, 17408])
def test_quantizer_bit_exact(K, M):
    import torch
    note(f"int8 quantizer K={K} M={M}")
    xb = I.gen_x(M, K, (90, K, M))
    xb[0, :128] = 0  # an all-zero block
    q = torch.zeros((M, K), dtype=torch.int8, device="cuda")
    a = torch.zeros((M, K // 128), dtype=torch.float32, device="cuda")
    s = torch.zeros((M, K // 128), dtype=torch.int32, device="cuda")
    W.wqd_quantize_i8(upload_x(xb), q, a, s)
    W.wqd_stream_check()
    qr, ar, sr = oracle.quantize_x_i8(xb)
    assert np.array_equal(q.cpu().numpy(), qr)
    assert np.array_equal(a.cpu().numpy().view(np.uint32), ar.view(np.uint32))
    assert np.array_equal(s.cpu().numpy(), sr)


@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("N,K", SHAPES)
def test_int8_gemm_parity(N, K, M):
    note(f"tq2 int8 gemm N={N} K={K} M={M}")
    canon = I.gen_weight(I.TQ2, N, K, (91, N, K))
    xb = I.gen_x(M, K, (91, N, K, M))
    w = upload_weight(I.TQ2, N, K, canon)
    y = new_y(M, N, ldy=N + 2)
    ws = workspace(W.wqd_gemm_i8_workspace_bytes(I.TQ2, N, K, M))
    W.wqd_gemm_i8(I.TQ2, N, K, w, upload_x(xb), y, ws)
    W.wqd_stream_check()
    got = y.cpu().numpy().astype(np.float64)
    q, a, _ = oracle.quantize_x_i8(xb)
    yref, t = oracle.tq2_i8_f64(N, K, canon, q, a)
    bound = (K // 128 + 16) * 2.0 ** -23 * t + 1e-30
    err = np.abs(got - yref)
    assert np.all(err <= bound), f"int8 path off by {err.max()} (bound {bound.flatten()[err.argmax()]})"
    full = y.as_strided((M, N + 2), (N + 2, 1)).cpu().numpy()
    assert np.isnan(full[:, N:]).all()
    # lossy against the exact product, within the quantization bound
    yex, _ = oracle.gemm_f64(I.TQ2, N, K, canon, xb)
    wabs = np.abs(oracle.decode_f64(I.TQ2, N, K, canon))
    step = np.repeat(a.astype(np.float64), 128, axis=1)
    qbound = (wabs[None, :, :] * step[:, None, :]).sum(axis=2) * (0.5 + 2.0 ** -20) + bound
    assert np.all(np.abs(got - yex) <= qbound)


def test_int8_gemm_repeats_bits_and_reuses_its_workspace():
    N, K, M = 300, 5120, 2
    note("tq2 int8 gemm twice on one workspace")
    canon = I.gen_weight(I.TQ2, N, K, (92, 0))
    xb = I.gen_x(M, K, (92, 1))
    w, x = upload_weight(I.TQ2, N, K, canon), upload_x(xb)
    ws = workspace(W.wqd_gemm_i8_workspace_bytes(I.TQ2, N, K, M))
    outs = []
    for _ in range(2):
        y = new_y(M, N)
        W.wqd_gemm_i8(I.TQ2, N, K, w, x, y, ws)
        W.wqd_stream_check()
        outs.append(y.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
