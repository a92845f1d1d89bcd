"""Pins of the CPU oracle against what the pages and the mathematics fix (runs without a GPU).

Each decode rule is checked against hand-decoded blocks stored under tests/golden/ (each file
cites its page and section); the multiply loop is checked against closed forms (one-hot and zero
activations, row permutations) and against numpy's fp64 matmul of the oracle's decoded matrix.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from weight_quantized_decode_amd import inputs as I
from weight_quantized_decode_amd import metrics as MX

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    out = {}
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


def f16(v):
    return int(np.float16(v).view(np.uint16))


def le16(h):
    return [h & 0xFF, h >> 8]


# ----------------------------------------------------------------------------- fp16 decode


def test_half_to_double_matches_ieee_binary16_everywhere():
    # numpy's float16 is an IEEE binary16 implementation: every one of the 65536 bit patterns must
    # decode to the same value (NaNs compared as NaN), subnormals included.
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert oracle.half_to_double(0x0001) == 2.0 ** -24
    assert oracle.half_to_double(0x7BFF) == 65504.0


# ----------------------------------------------------------------------------- byte budgets


def test_q4_0_is_18_bytes_per_32_weights_4_5_bpw():
    # blog.localai.hex7.com, ladder table: Q4_0 = 4 stored bits, 4.5 effective bits per weight,
    # block-32 with one fp16 scale; "Anatomy of a block": 16-bit scale per 32 weights = 0.5 bpw.
    assert oracle.canonical_bytes(1, 1, 32) == 18
    assert MX.bits_per_weight(oracle.canonical_bytes(1, 4096, 4096), 4096 * 4096) == 4.5
    assert MX.bits_per_weight(2, 32) == 0.5
    assert oracle.canonical_bytes(1, 4096, 4096) == 9_437_184


def test_tq2_is_34_bytes_per_128_weights_and_row_shape():
    # vLLM ternary page, "Anatomy of a PQ2_0 block": 34 bytes per 128 weights = 2.125 bpw, and a
    # weight matrix is a uint8 tensor of shape (N, K/128 * 34).
    assert oracle.canonical_bytes(4, 1, 128) == 34
    assert MX.bits_per_weight(34, 128) == 2.125
    N, K = 17408, 5120
    assert oracle.canonical_bytes(4, N, K) == N * (K // 128 * 34) == 23_674_880


def test_aq2x8_code_bytes_at_4096_square():
    # trapetum "Additive vector-quantization GEMV": at 2 bits (M=2, K=256, D=8), 4.2 MB of codes
    # against 33.6 MB of fp16 weight at 4096x4096.
    N = K = 4096
    codes = oracle.canonical_bytes(5, N, K) - 8192 - 2 * N
    assert codes == 4_194_304 and round(codes / 1e6, 1) == 4.2
    assert round(N * K * 2 / 1e6, 1) == 33.6
    assert MX.bits_per_weight(codes, N * K) == 2.0


def test_aq1x16_is_2_bits_per_weight_with_a_1_mib_codebook():
    # trapetum "Benchmarks", the 70B 1x16 model: one codebook of 65,536 entries of 8 fp16 values
    # (1 MiB, too large for shared memory) and one 16-bit code per group of 8 weights, still
    # 2 bits per weight.
    N = K = 4096
    total = oracle.canonical_bytes(6, N, K)
    codebook = 65536 * 8 * 2
    assert codebook == 1 << 20
    codes = total - codebook - 2 * N
    assert codes == N * K // 8 * 2 == 4_194_304
    assert MX.bits_per_weight(codes, N * K) == 2.0
    assert oracle.canonical_bytes(6, 4, 12) == -1  # K not a whole number of groups


def test_byte_counts_of_the_workloads():
    total = sum(oracle.canonical_bytes(p.fmt, p.N, p.K) for p in I.config_projections(3))
    assert total == 3_369_082_368
    assert sum(oracle.canonical_bytes(p.fmt, p.N, p.K) for p in I.config_projections(2)) == 101_187_808
    assert [oracle.canonical_bytes(p.fmt, p.N, p.K) for p in I.config_projections(5)] == [
        58_785_792, 58_785_792, 58_744_832]
    for p in I.config_projections(4):
        assert oracle.canonical_bytes(p.fmt, p.N, p.K) == 23_674_880


def test_bad_shapes_are_rejected():
    assert oracle.canonical_bytes(1, 4, 48) == -1   # K not a multiple of 32
    assert oracle.canonical_bytes(4, 4, 64) == -1   # K not a multiple of 128
    assert oracle.canonical_bytes(5, 4, 12) == -1   # K not a multiple of 8
    assert oracle.canonical_bytes(2, 4, 3) == -1    # odd K
    assert oracle.canonical_bytes(9, 4, 8) == -1


# ----------------------------------------------------------------------------- byte-model formulas


def test_bandwidth_floor_and_ceiling_of_the_ternary_page():
    # "A rough speed limit": 6.80 GB / 1008 GB/s is about 6.75 ms per token, reciprocal 148 tok/s.
    assert round(MX.floor_seconds(6.80e9, 1008) * 1e3, 2) == 6.75
    assert round(MX.ceiling_tok_s(6.80e9, 1008)) == 148
    # 25 tok/s * 6.80 GB/token = about 170 GB/s, 17% of the card.
    assert round(MX.effective_gbps(25, 6.80e9)) == 170
    assert round(MX.fraction_of_peak(MX.effective_gbps(25, 6.80e9), 1008) * 100) == 17


def test_effective_bandwidth_of_the_70b_2x8_decode():
    # trapetum Llama-2-70B 2x8: about 17.4 GB per token at 38.4 tok/s, so about 670 GB/s,
    # two thirds of 1,008 GB/s.
    g = MX.effective_gbps(38.4, 17.4e9)
    assert abs(g - 670) < 5
    assert abs(MX.fraction_of_peak(g, 1008) - 2 / 3) < 0.01


# ----------------------------------------------------------------------------- hand-decoded blocks


def test_tq2_worked_byte_0x64():
    g = read_golden("tq2_byte_0x64.txt")
    d = int(g["scale_f16"][0], 16)
    byte = int(g["byte"][0], 16)
    qs = [byte] + [0x55] * 31  # remaining codes 1 -> weight 0
    canon = np.array(le16(d) + qs, dtype=np.uint8)
    w = oracle.decode_f64(4, 1, 128, canon)[0]
    assert list(w[:4]) == [float(v) for v in g["weights"]]
    assert np.all(w[4:] == 0.0)
    # code 3 would decode to +2 * d
    canon3 = np.array(le16(d) + [0x03] + [0x55] * 31, dtype=np.uint8)
    assert oracle.decode_f64(4, 1, 128, canon3)[0][0] == float(g["code3_weight"][0])


def test_q4_0_hand_block():
    g = read_golden("q4_0_block.txt")
    d = int(g["scale_f16"][0], 16)
    qs = [int(b, 16) for b in g["qs"]]
    canon = np.array(le16(d) + qs, dtype=np.uint8)
    w = oracle.decode_f64(1, 1, 32, canon)[0]
    assert list(w) == [float(v) for v in g["weights"]]


def test_q4_0_scale_belongs_to_its_own_block():
    # two blocks with different scales: the second block's weights use the second scale
    canon = np.array(le16(f16(1.0)) + [0x99] * 16 + le16(f16(-0.5)) + [0x99] * 16, dtype=np.uint8)
    w = oracle.decode_f64(1, 1, 64, canon)[0]
    assert np.all(w[:32] == 1.0) and np.all(w[32:] == -0.5)


def test_cb4_hand_row():
    g = read_golden("cb4_row.txt")
    cb = [f16(float(v)) for v in g["codebook"]]
    codes = [int(b, 16) for b in g["codes"]]
    canon = np.array(sum((le16(h) for h in cb), []) + codes, dtype=np.uint8)
    w = oracle.decode_f64(2, 1, 2 * len(codes), canon)[0]
    assert list(w) == [float(v) for v in g["weights"]]


def test_cb8_hand_row():
    g = read_golden("cb8_row.txt")
    cb = [f16((i - 128) / 4) for i in range(256)]
    codes = [int(b, 16) for b in g["codes"]]
    canon = np.array(sum((le16(h) for h in cb), []) + codes, dtype=np.uint8)
    w = oracle.decode_f64(3, 1, len(codes), canon)[0]
    assert list(w) == [float(v) for v in g["weights"]]


def _aq_canon_from_golden(g):
    C0 = [[f16(8 * c + j) for j in range(8)] for c in range(256)]
    C1 = [[f16(-c) for _ in range(8)] for c in range(256)]
    cbk = sum((le16(h) for row in C0 + C1 for h in row), [])
    sc = sum((le16(f16(float(v))) for v in g["scales"]), [])
    codes = [int(v) for v in g["codes_row0"]] + [int(v) for v in g["codes_row1"]]
    return np.array(cbk + sc + codes, dtype=np.uint8)


def test_aq2x8_hand_rows():
    g = read_golden("aq2x8_rows.txt")
    canon = _aq_canon_from_golden(g)
    w = oracle.decode_f64(5, 2, 8, canon)
    assert list(w[0]) == [float(v) for v in g["weights_row0"]]
    assert list(w[1]) == [float(v) for v in g["weights_row1"]]


def test_aq2x8_fp32_dequant_rounds_sum_then_product():
    # fp32 reading of the decode: round the codebook sum to fp32 (nearest even), then the product.
    # C0 = 1, C1 = 2^-24 (an fp16 subnormal): the fp32 sum 1 + 2^-24 is a tie and rounds to 1.
    C = np.zeros((2, 256, 8), dtype=np.uint16)
    C[0, 0, :] = f16(1.0)
    C[1, 0, :] = 0x0001
    s = f16(0.75)
    canon = np.concatenate([C.astype("<u2").view(np.uint8).reshape(-1),
                            np.array(le16(s), dtype=np.uint8), np.zeros(2, dtype=np.uint8)])
    w64 = oracle.decode_f64(5, 1, 8, canon)[0]
    w32 = oracle.dequant_f32(5, 1, 8, canon)[0]
    assert np.all(w64 == 0.75 * (1 + 2.0 ** -24))
    assert np.all(w32 == np.float32(0.75))


def _aq1x16_canon(g):
    C = np.zeros((65536, 8), dtype=np.float64)
    c = np.arange(65536)
    hi, lo = (c >> 8).astype(np.float64), (c & 0xFF).astype(np.float64)
    C[:, 0], C[:, 1], C[:, 2], C[:, 3], C[:, 4], C[:, 5], C[:, 6] = hi, lo, -hi, -lo, 0.5 * hi, 1, -1
    cbk = C.astype(np.float16).view(np.uint16).astype("<u2").view(np.uint8).reshape(-1)
    sc = np.array(sum((le16(f16(float(v))) for v in g["scales"]), []), dtype=np.uint8)
    codes = np.array([int(v, 16) for v in g["code_bytes_row0"] + g["code_bytes_row1"]], dtype=np.uint8)
    return np.concatenate([cbk, sc, codes])


def test_aq1x16_hand_rows():
    g = read_golden("aq1x16_rows.txt")
    canon = _aq1x16_canon(g)
    w = oracle.decode_f64(6, 2, 16, canon)
    assert list(w[0]) == [float(v) for v in g["weights_row0"]]
    assert list(w[1]) == [float(v) for v in g["weights_row1"]]
    # the fp32 decode is the exact value (an fp16 scale times an fp16 entry fits in fp32)
    assert np.array_equal(oracle.dequant_f32(6, 2, 16, canon), w.astype(np.float32))


def test_subnormal_scales_are_kept():
    # an fp16 subnormal scale (2^-24) is kept, not flushed: Q4_0 code 15 -> 7 * 2^-24
    canon = np.array(le16(0x0001) + [0xFF] * 16, dtype=np.uint8)
    w = oracle.decode_f64(1, 1, 32, canon)[0]
    assert np.all(w == 7 * 2.0 ** -24)
    assert np.all(oracle.dequant_f32(1, 1, 32, canon)[0] == np.float32(7 * 2.0 ** -24))


# ----------------------------------------------------------------------------- the multiply


SHAPES = [(1, 5, 96), (2, 7, 256), (3, 3, 128), (4, 6, 384), (5, 4, 40), (6, 5, 48)]


@pytest.mark.parametrize("fmt,N,K", SHAPES)
def test_one_hot_activation_returns_a_weight_column(fmt, N, K):
    canon = I.gen_weight(fmt, N, K, (77, fmt))
    W = oracle.decode_f64(fmt, N, K, canon)
    for k in (0, K // 3, K - 1):
        x = np.zeros((1, K), dtype=np.uint16)
        x[0, k] = f16(1.0)
        y, a = oracle.gemm_f64(fmt, N, K, canon, x)
        assert np.array_equal(y[0], W[:, k])
        assert np.array_equal(a[0], np.abs(W[:, k]))


@pytest.mark.parametrize("fmt,N,K", SHAPES)
def test_zero_activation_gives_zero(fmt, N, K):
    canon = I.gen_weight(fmt, N, K, (78, fmt))
    y, a = oracle.gemm_f64(fmt, N, K, canon, np.zeros((2, K), dtype=np.uint16))
    assert np.all(y == 0) and np.all(a == 0)


@pytest.mark.parametrize("fmt,N,K", SHAPES)
def test_gemm_matches_numpy_matmul_of_decoded_matrix(fmt, N, K):
    canon = I.gen_weight(fmt, N, K, (79, fmt))
    x = I.gen_x(3, K, (79, fmt))
    W = oracle.decode_f64(fmt, N, K, canon)
    X = x.view(np.float16).astype(np.float64)
    y, a = oracle.gemm_f64(fmt, N, K, canon, x)
    ref = X @ W.T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-15)
    assert np.allclose(a, np.abs(X) @ np.abs(W).T, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("fmt,N,K", SHAPES)
def test_row_subset_equals_full_rows(fmt, N, K):
    canon = I.gen_weight(fmt, N, K, (80, fmt))
    x = I.gen_x(2, K, (80, fmt))
    y, _ = oracle.gemm_f64(fmt, N, K, canon, x)
    rows = np.array([N - 1, 0, N // 2], dtype=np.int64)
    ys, _ = oracle.gemm_f64(fmt, N, K, canon, x, rows=rows)
    assert np.array_equal(ys, y[:, rows])


def test_gemm_exact_on_dyadic_tiny_case():
    # Brute force with exact rationals: a 2x64 Q4_0 matrix with power-of-two scales and
    # integer activations has an exactly representable product.
    qs0 = [0x1F, 0x2E, 0x3D, 0x4C] * 4
    qs1 = [0x80, 0x08, 0xFF, 0x00] * 4
    canon = np.array(le16(f16(0.5)) + qs0 + le16(f16(2.0)) + qs1
                     + le16(f16(0.25)) + qs1 + le16(f16(4.0)) + qs0, dtype=np.uint8)
    xs = [((k * 7) % 11) - 5 for k in range(64)]
    x = np.array([[f16(v) for v in xs]], dtype=np.uint16)
    y, _ = oracle.gemm_f64(1, 2, 64, canon, x)

    def lo(b):
        return b & 15

    def hi(b):
        return b >> 4

    def row_weights(blocks):
        w = []
        for d, qs in blocks:
            w += [Fraction(lo(b) - 8) * d for b in qs] + [Fraction(hi(b) - 8) * d for b in qs]
        return w

    r0 = row_weights([(Fraction(1, 2), qs0), (Fraction(2), qs1)])
    r1 = row_weights([(Fraction(1, 4), qs1), (Fraction(4), qs0)])
    exact = [sum(Fraction(a) * b for a, b in zip(xs, r)) for r in (r0, r1)]
    assert [Fraction(v) for v in y[0]] == exact


def test_dequant_f32_is_the_rounded_exact_value_for_exact_formats():
    for fmt in (1, 2, 3, 4):
        canon = I.gen_weight(fmt, 4, 256, (81, fmt))
        w64 = oracle.decode_f64(fmt, 4, 256, canon)
        w32 = oracle.dequant_f32(fmt, 4, 256, canon)
        assert np.array_equal(w32.astype(np.float64), w64)  # exact in fp32


# ----------------------------------------------------------------------------- epilogues
# The fused gate/up reduce applies SiLU(gate) * up and the o/down reduces add the residual
# (trapetum "Benchmarks", "Short-context decode, step by step").


def test_silu_closed_forms():
    assert oracle.silu(0.0) == 0.0
    # SiLU(2t) = 2t * sigma(2t) = t * (1 + tanh t): checked through libm's tanh, not exp (for
    # t << 0 the tanh form cancels, hence the absolute term of |t| ulps of 1)
    for t in np.linspace(-20.0, 20.0, 161):
        want = t * (1.0 + math.tanh(t))
        assert oracle.silu(2.0 * t) == pytest.approx(want, rel=4e-15, abs=4e-16 * abs(t))
    # the odd part of SiLU is the identity: SiLU(x) - SiLU(-x) = x * (sigma(x) + sigma(-x)) = x
    for x in np.linspace(-30.0, 30.0, 241):
        assert oracle.silu(x) - oracle.silu(-x) == pytest.approx(x, rel=1e-14, abs=1e-14)


def test_silu_minimum_is_minus_lambert_w_of_1_over_e():
    # SiLU'(x) = 0 at x* = -1 - W(1/e), where SiLU(x*) = -W(1/e) (W the Lambert function)
    from scipy.special import lambertw
    w = float(lambertw(1.0 / math.e).real)
    xs = -1.0 - w + np.linspace(-1e-4, 1e-4, 201)
    vals = np.array([oracle.silu(x) for x in xs])
    assert vals.min() == pytest.approx(-w, rel=1e-12)
    assert abs(xs[vals.argmin()] - (-1.0 - w)) < 2e-6


def test_silu_slope_and_limits():
    h = 1e-6
    assert (oracle.silu(h) - oracle.silu(-h)) / (2 * h) == pytest.approx(0.5, rel=1e-9)  # SiLU'(0) = 1/2
    assert oracle.silu(800.0) == 800.0
    assert oracle.silu(40.0) == 40.0
    lo = oracle.silu(-800.0)
    assert lo == 0.0 and not math.isnan(lo)


def _cb8_canon(codes_nk):
    cb = ((np.arange(256) - 128) / 4.0).astype(np.float16)
    return np.concatenate([cb.view(np.uint16).astype("<u2").view(np.uint8),
                           np.asarray(codes_nk, dtype=np.uint8).reshape(-1)])


def test_silu_pair_hand_rows():
    g = read_golden("silu_pair.txt")
    gc = np.array([int(v) for v in g["gate_codes"]])
    uc = np.array([int(v) for v in g["up_codes"]])
    N, K = len(gc), 3
    r = np.random.default_rng(5)
    gate = r.integers(0, 256, size=(N, K))
    up = r.integers(0, 256, size=(N, K))
    gate[:, 1], up[:, 1] = gc, uc
    x = np.zeros((1, K), dtype=np.uint16)
    x[0, 1] = f16(1.0)
    h, gg, uu, ag, au = oracle.silu_pair_f64(I.CB8, N, K, _cb8_canon(gate), _cb8_canon(up), x, x)
    assert np.array_equal(gg[0], np.array([float(v) for v in g["g"]]))
    assert np.array_equal(uu[0], np.array([float(v) for v in g["u"]]))
    want = np.array([float(v) for v in g["h"]])
    np.testing.assert_allclose(h[0], want, rtol=4e-16, atol=0)
    # gate and up are not interchangeable: the swapped pair gives other values
    assert not np.allclose(oracle.silu_mul(uu, gg)[0], want)


def test_silu_pair_of_random_projections_is_silu_of_gate_times_up():
    N, K = 70, 96
    cg = I.gen_weight(I.CB4, N, K, (77, 0))
    cu = I.gen_weight(I.CB4, N, K, (77, 1))
    xg = I.gen_x(2, K, (77, 2))
    xu = I.gen_x(2, K, (77, 3))
    h, g, u, _, _ = oracle.silu_pair_f64(I.CB4, N, K, cg, cu, xg, xu)
    g2, _ = oracle.gemm_f64(I.CB4, N, K, cg, xg)
    u2, _ = oracle.gemm_f64(I.CB4, N, K, cu, xu)
    assert np.array_equal(g, g2) and np.array_equal(u, u2)
    # h / u = sigma(g) * g where u != 0, and sigma(g) lies in (0, 1) with the sign of h = sign(g*u)
    nz = u != 0
    sig = h[nz] / (u[nz] * g[nz])
    assert np.all((sig > 0) & (sig < 1))
    np.testing.assert_allclose(sig, 0.5 * (1 + np.tanh(g[nz] / 2)), rtol=1e-13)


def test_residual_add_is_exact_on_one_hot_activation():
    N, K, k0 = 9, 64, 17
    canon = I.gen_weight(I.CB8, N, K, (78, 0))
    x = np.zeros((1, K), dtype=np.uint16)
    x[0, k0] = f16(1.0)
    res = np.random.default_rng(6).standard_normal((1, N)).astype(np.float32)
    y, _ = oracle.gemm_f64(I.CB8, N, K, canon, x)
    out = oracle.residual_add(res, y)
    col = oracle.decode_f64(I.CB8, N, K, canon)[:, k0]
    for n in range(N):
        assert Fraction(out[0, n]) == Fraction(float(res[0, n])) + Fraction(col[n])
    # zero activation: the residual comes back unchanged
    y0, _ = oracle.gemm_f64(I.CB8, N, K, canon, np.zeros((1, K), dtype=np.uint16))
    assert np.array_equal(oracle.residual_add(res, y0), res.astype(np.float64))


# ----------------------------------------------------------------------------- TQ2, int8 x
# "Making a ternary reasoning model fast in vLLM", "Why small integers are a good fit".


def test_int8_quantization_hand_group():
    g = read_golden("tq2_i8_group.txt")
    x = np.zeros((1, 128), dtype=np.float16)
    vals = [float(v) for v in g["x"]]
    x[0, :len(vals)] = vals
    q, a, qs = oracle.quantize_x_i8(x.view(np.uint16))
    want = [int(v) for v in g["q"]]
    assert list(q[0, :len(want)]) == want and not q[0, len(want):].any()
    assert a[0, 0] == float(g["a"][0]) and qs[0, 0] == int(g["qsum"][0])


def test_int8_quantization_properties():
    x = I.gen_x(3, 1024, (80, 0))
    x[1, 128:256] = 0  # an all-zero group
    q, a, qs = oracle.quantize_x_i8(x)
    xv = x.view(np.float16).astype(np.float64).reshape(3, 8, 128)
    qv = q.astype(np.float64).reshape(3, 8, 128)
    av = a.astype(np.float64)[:, :, None]
    # rounding to nearest: |x - a q| <= a / 2 (plus the fp32 rounding of x / a)
    assert np.all(np.abs(xv - av * qv) <= av * (0.5 + 2.0 ** -20) + 1e-300)
    # the largest |x| of a group maps to +-127; every |q| <= 127
    nz = a[:, :] > 0
    assert np.all(np.abs(q).reshape(3, 8, 128).max(axis=2)[nz] == 127)
    assert a[1, 1] == 0 and not q[1, 128:256].any()
    assert np.array_equal(qs, q.astype(np.int32).reshape(3, 8, 128).sum(axis=2))
    # a = max|x| / 127 in fp32
    amax = np.abs(xv).max(axis=2).astype(np.float32)
    assert np.array_equal(a, (amax / np.float32(127)).astype(np.float32))


def test_int8_path_equals_exact_path_on_grid_activations():
    # x = q * 2^-7 with one |q| = 127 per group is exactly representable, so quantization gives
    # q back and the int8 product is the exact product
    N, K, M = 40, 512, 2
    r = np.random.default_rng(81)
    qi = r.integers(-127, 128, size=(M, K))
    qi[:, ::128] = 127
    x = (qi * 2.0 ** -7).astype(np.float16)
    canon = I.gen_weight(I.TQ2, N, K, (81, 1))
    q, a, _ = oracle.quantize_x_i8(x.view(np.uint16))
    assert np.array_equal(q, qi) and np.all(a == 2.0 ** -7)
    y8, t = oracle.tq2_i8_f64(N, K, canon, q, a)
    y, _ = oracle.gemm_f64(I.TQ2, N, K, canon, x.view(np.uint16))
    np.testing.assert_allclose(y8, y, rtol=1e-12, atol=1e-12)


def test_int8_path_error_within_the_rounding_bound():
    # |y_i8 - y| <= sum_k |w_k| * a_g(k) / 2 (each activation moves by at most half a step)
    N, K, M = 30, 1024, 3
    canon = I.gen_weight(I.TQ2, N, K, (82, 0))
    x = I.gen_x(M, K, (82, 1))
    q, a, _ = oracle.quantize_x_i8(x)
    y8, _ = oracle.tq2_i8_f64(N, K, canon, q, a)
    y, _ = oracle.gemm_f64(I.TQ2, N, K, canon, x)
    w = np.abs(oracle.decode_f64(I.TQ2, N, K, canon))
    step = np.repeat(a.astype(np.float64), 128, axis=1)  # a_g per k
    bound = (w[None, :, :] * step[:, None, :] * (0.5 + 2.0 ** -20)).sum(axis=2)
    assert np.all(np.abs(y8 - y) <= bound)
    assert np.abs(y8 - y).max() > 0  # the path is lossy
