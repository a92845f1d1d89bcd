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


@pytest.mark.parametrize("code3", [0.0, 0.1])
@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("N,K", SHAPES)
def test_int8_gemm_parity(N, K, M, code3):
    # code3 > 0: blocks holding code 3 (+2d, "Anatomy of a PQ2_0 block"), which the workloads never draw
    note(f"tq2 int8 gemm N={N} K={K} M={M} code3={code3}")
    canon = I.gen_weight(I.TQ2, N, K, (91, N, K), tq2_code3=code3)
    xb = I.gen_x(M, K, (91, N, K, M))
    w = upload_weight(I.TQ2, N, K, canon)
    y = new_y(M, N, ldy=N + 2)
    ws = workspace(W.wqd_gemm_i8_workspace_bytes(w, M))
    W.wqd_gemm_i8(w, upload_x(xb), y, ws)
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
    ws = workspace(W.wqd_gemm_i8_workspace_bytes(w, M))
    outs = []
    for _ in range(2):
        y = new_y(M, N)
        W.wqd_gemm_i8(w, x, y, ws)
        W.wqd_stream_check()
        outs.append(y.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


MODES = {"ordered": W.WQD_ORDERED, "persistent": W.WQD_PERSISTENT, "fused": W.WQD_FUSED}


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("M", [1, 3])
def test_int8_list_quantizes_each_x_once_and_matches_the_oracle(M, mode):
    """A TQ2 MLP list (gate and up on one x, down on another, plus a CB4 entry that stays fp16)
    with WQD_INT8_ACTIVATIONS, in every mode."""
    import torch
    note(f"int8 list M={M} mode={mode}")
    specs = [("gate", I.TQ2, 700, 1280, 0), ("up", I.TQ2, 700, 1280, 0), ("down", I.TQ2, 300, 2560, 1),
             ("cb4", I.CB4, 200, 1280, 0)]
    xs = {r: I.gen_x(M, K, (93, r, M)) for r, K in ((0, 1280), (1, 2560))}
    xd = {r: upload_x(v) for r, v in xs.items()}
    canon = {n: I.gen_weight(f, N, K, (93, i)) for i, (n, f, N, K, _) in enumerate(specs)}
    ent = [dict(fmt=f, N=N, K=K, w=upload_weight(f, N, K, canon[n]), x=xd[r], y=new_y(M, N))
           for n, f, N, K, r in specs]
    arr = W.make_proj_array(ent)
    ws = workspace(W.wqd_stack_workspace_bytes(arr, M))
    flags = MODES[mode] | W.WQD_INT8_ACTIVATIONS
    if mode == "persistent":
        W.wqd_stack_setup(arr, M, ws, mode=flags)
    W.wqd_run_projections(arr, M, flags, ws)
    W.wqd_stream_check()
    for (n, f, N, K, r), e in zip(specs, ent):
        got = e["y"].cpu().numpy().astype(np.float64)
        if f == I.TQ2:
            q, a, _ = oracle.quantize_x_i8(xs[r])
            yref, t = oracle.tq2_i8_f64(N, K, canon[n], q, a)
            bound = (K // 128 + 16) * 2.0 ** -23 * t + 1e-30
        else:
            yref, aref = oracle.gemm_f64(f, N, K, canon[n], xs[r])
            bound = 2e-3 * aref + 1e-6
        assert np.all(np.abs(got - yref) <= bound), f"{n} outside the bound"


def test_int8_list_with_a_silu_pair():
    import torch
    M, N, K = 2, 400, 2560
    note("int8 list with a gate/up pair")
    cg, cu = I.gen_weight(I.TQ2, N, K, (94, 0)), I.gen_weight(I.TQ2, N, K, (94, 1))
    xb = I.gen_x(M, K, (94, 2))
    x = upload_x(xb)
    h = new_y(M, N)
    ent = [dict(fmt=I.TQ2, N=N, K=K, w=upload_weight(I.TQ2, N, K, cg), x=x, y=h, epi=W.WQD_EPI_SILU_GATE),
           dict(fmt=I.TQ2, N=N, K=K, w=upload_weight(I.TQ2, N, K, cu), x=x, y=None, epi=W.WQD_EPI_SILU_UP)]
    arr = W.make_proj_array(ent)  # (the array holds raw pointers: `ent` keeps the buffers alive)
    ws = workspace(W.wqd_stack_workspace_bytes(arr, M))
    W.wqd_run_projections(arr, M, W.WQD_FUSED | W.WQD_INT8_ACTIVATIONS, ws)
    W.wqd_stream_check()
    q, a, _ = oracle.quantize_x_i8(xb)
    g, tg = oracle.tq2_i8_f64(N, K, cg, q, a)
    u, tu = oracle.tq2_i8_f64(N, K, cu, q, a)
    eg, eu = (K // 128 + 16) * 2.0 ** -23 * tg, (K // 128 + 16) * 2.0 ** -23 * tu
    href = oracle.silu_mul(g, u)
    sg = np.abs(oracle.silu_mul(g, np.ones_like(g)))
    bound = 1.1 * eg * (np.abs(u) + eu) + sg * eu + 1e-6 * np.abs(href) + 1e-6
    assert np.all(np.abs(h.cpu().numpy() - href) <= bound)
