"""Host-side checks of libwqd (no GPU needed): exported symbols, byte counts, the prepared
layout's re-lay of the canonical bytes, and argument validation before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from weight_quantized_decode_amd import _lib as W
from weight_quantized_decode_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FMTS = [I.Q4_0, I.CB4, I.CB8, I.TQ2, I.AQ2X8, I.AQ1X16]


def declared_symbols(header="wqd.h", api="WQD_API"):
    text = open(os.path.join(ROOT, "include", header)).read()
    return sorted(set(re.findall(api + r"\s+[\w\s\*]+?\b(wqd_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    syms = declared_symbols()
    assert len(syms) >= 12
    L = W.lib()
    for s in syms:
        assert hasattr(L, s), s
    assert sorted(W.EXPORTED) == syms


def test_probe_library_exports_every_declared_symbol():
    # the read-only stream probe the bench times beside the kernels (include/wqd_probe.h)
    import ctypes
    syms = declared_symbols("wqd_probe.h", "WQD_PROBE_API")
    assert syms == ["wqd_probe_read"]
    L = ctypes.CDLL(os.path.join(ROOT, "weight_quantized_decode_amd", "libwqd_probe.so"))
    for s in syms:
        assert hasattr(L, s), s
    L.wqd_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    # bad arguments are refused before any HIP call
    assert L.wqd_probe_read(None, 16384, 256, 0, None) == -1
    assert L.wqd_probe_read(256, 1000, 256, 0, None) == -1
    assert L.wqd_probe_read(257, 16384, 256, 0, None) == -1


@pytest.mark.parametrize("fmt", FMTS)
def test_canonical_bytes_agree_with_oracle(fmt):
    for N, K in [(1, 256), (64, 1024), (4096, 4096), (11008, 4096), (5120, 17408), (8192, 28672)]:
        assert W.wqd_canonical_bytes(fmt, N, K) == oracle.canonical_bytes(fmt, N, K)


def test_prepared_sizes_are_canonical_plus_padding_only():
    # at the workload shapes (N multiple of 64, rows a whole number of 16-byte chunks) the
    # prepared planes hold exactly the canonical bytes, plus plane alignment (<= 3 x 255 bytes)
    for cfg in (1, 2, 4, 5, 6):
        for p in I.config_projections(cfg):
            c = W.wqd_canonical_bytes(p.fmt, p.N, p.K)
            q = W.wqd_prepared_bytes(p.fmt, p.N, p.K)
            assert c <= q <= c + 3 * 256, (p, c, q)


def _tile_rows(prep, fmt, N, K):
    """Code plane back to [N][C*16] row order (inverse of the 64-row tiling)."""
    L = W.wqd_prepared_bytes(fmt, N, K)
    row_bytes = {I.Q4_0: K // 2, I.CB4: K // 2, I.CB8: K, I.TQ2: K // 4, I.AQ2X8: K // 4, I.AQ1X16: K // 4}[fmt]
    C = (row_bytes + 15) // 16
    RG = (N + 63) // 64
    codes = prep[:RG * C * 64 * 16].reshape(RG, C, 64, 16).transpose(0, 2, 1, 3).reshape(RG * 64, C * 16)
    return codes[:N], row_bytes, C, RG


@pytest.mark.parametrize("fmt,N,K", [(I.CB4, 70, 1002), (I.CB8, 70, 1001), (I.AQ1X16, 70, 1000)])
def test_prepare_keeps_canonical_byte_order_for_byte_formats(fmt, N, K):
    canon = I.gen_weight(fmt, N, K, (5, fmt))
    prep = W.wqd_prepare_host(fmt, N, K, canon)
    rows, row_bytes, C, RG = _tile_rows(prep, fmt, N, K)
    head = {I.CB4: 32, I.CB8: 512, I.AQ2X8: 8192 + 2 * N, I.AQ1X16: 65536 * 16 + 2 * N}[fmt]
    assert np.array_equal(rows[:, :row_bytes], canon[head:].reshape(N, row_bytes))
    assert np.all(rows[:, row_bytes:] == 0)  # tail padding is zero
    full = prep[:RG * C * 1024].reshape(RG, C, 64, 16)
    assert np.all(full[:, :, (N - (RG - 1) * 64):, :][-1] == 0)  # padded rows are zero
    if fmt == I.AQ1X16:  # scales and the 1 MiB codebook are copied as they are
        L_off = W.wqd_prepared_bytes(fmt, N, K) - ((65536 * 16 + 255) // 256 * 256)
        assert np.array_equal(prep[L_off:L_off + 65536 * 16], canon[:65536 * 16])


@pytest.mark.parametrize("N,K", [(70, 1000), (64, 512), (8, 8), (130, 8 * 200)])
def test_prepare_tiles_aq2x8_codes(N, K):
    # AQ2X8 codes go to tiles of 16 rows x 32 groups, slice-major: the 16 bytes of lane 32h + g in
    # tile (b16, s) are (c0, c1) of rows 16*b16 + 8h .. + 7 for group 32*s + g.  Rebuild the
    # canonical [N][G][2] code array from the tiles, and check the padding (rows >= N, groups >= G)
    # is zero; scales and codebooks are copied verbatim.
    canon = I.gen_weight(I.AQ2X8, N, K, (5, I.AQ2X8))
    prep = W.wqd_prepare_host(I.AQ2X8, N, K, canon)
    G = K // 8
    KS = (G + 31) // 32
    RG = (N + 63) // 64
    Npad = RG * 64
    tiles = prep[:Npad // 16 * KS * 1024].reshape(KS, Npad // 16, 2, 32, 8, 2)  # [s][b16][h][g][row][c]
    codes = tiles.transpose(1, 2, 4, 0, 3, 5).reshape(Npad, KS * 32, 2)        # [n][group][c]
    want = canon[8192 + 2 * N:].reshape(N, G, 2)
    assert np.array_equal(codes[:N, :G], want)
    assert np.all(codes[N:] == 0) and np.all(codes[:, G:] == 0)
    off_s = (Npad // 16 * KS * 1024 + 255) // 256 * 256
    assert np.array_equal(prep[off_s:off_s + 2 * N], canon[8192:8192 + 2 * N])
    off_c = (off_s + 2 * Npad + 255) // 256 * 256
    assert np.array_equal(prep[off_c:off_c + 8192], canon[:8192])
    assert W.wqd_prepared_bytes(I.AQ2X8, N, K) == (off_c + 8192 + 255) // 256 * 256


@pytest.mark.parametrize("fmt,N,K", [(I.Q4_0, 70, 256), (I.TQ2, 70, 512)])
def test_prepare_permutes_codes_within_rows_only(fmt, N, K):
    # the block formats' code bits are permuted inside each row: every row keeps its multiset of
    # codes, and its scales
    canon = I.gen_weight(fmt, N, K, (6, fmt))
    prep = W.wqd_prepare_host(fmt, N, K, canon)
    rows, row_bytes, C, RG = _tile_rows(prep, fmt, N, K)
    bits = 4 if fmt == I.Q4_0 else 2
    bsz = 18 if fmt == I.Q4_0 else 34
    nb = K // (32 if fmt == I.Q4_0 else 128)
    blk = canon.reshape(N, nb, bsz)

    def hist(b):
        vals = np.stack([(b >> s) & ((1 << bits) - 1) for s in range(0, 8, bits)], -1)
        return np.bincount(vals.reshape(-1), minlength=1 << bits)

    for n in range(N):
        assert np.array_equal(hist(rows[n]), hist(blk[n, :, 2:]))
    scales_canon = np.sort(blk[:, :, 0:2].copy().view(np.uint16).reshape(-1))
    off = ((RG * C * 1024 + 255) // 256) * 256
    Q = (nb + 3) // 4
    sc = prep[off:off + RG * Q * 64 * 8].view(np.uint16).reshape(RG, Q, 64, 4)
    sc = sc.transpose(0, 2, 1, 3).reshape(RG * 64, Q * 4)[:N, :nb]
    assert np.array_equal(np.sort(sc.reshape(-1)), scales_canon)
    assert np.array_equal(sc, blk[:, :, 0:2].copy().view(np.uint16).reshape(N, nb))


def test_prepare_rejects_bad_arguments():
    canon = np.zeros(64, dtype=np.uint8)
    out = np.zeros(4096, dtype=np.uint8)
    L = W.lib()
    assert L.wqd_prepare_host(9, 1, 32, canon.ctypes.data, 64, out.ctypes.data, 4096) == W.WQD_EINVAL
    assert L.wqd_prepare_host(1, 1, 48, canon.ctypes.data, 64, out.ctypes.data, 4096) == W.WQD_ESHAPE
    assert L.wqd_prepare_host(1, 2, 32, canon.ctypes.data, 20, out.ctypes.data, 4096) == W.WQD_ESPACE
    assert L.wqd_prepare_host(1, 1, 32, None, 64, out.ctypes.data, 4096) == W.WQD_EINVAL


FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation first


def _view(fmt, N, K, base=FAKE):
    """A bound view of a never-dereferenced prepared buffer at base."""
    return W.wqd_bind(fmt, N, K, base)


def test_bind_sets_the_planes_of_each_format():
    for fmt in (I.Q4_0, I.CB4, I.CB8, I.TQ2, I.AQ2X8, I.AQ1X16):
        N, K = 96, 1024
        v = _view(fmt, N, K).view
        assert (v.fmt, v.N, v.K, v.codes) == (fmt, N, K, FAKE)
        has_scales = fmt in (I.Q4_0, I.TQ2, I.AQ2X8, I.AQ1X16)
        has_cbk = fmt in (I.CB4, I.CB8, I.AQ2X8, I.AQ1X16)
        assert (v.scales is not None) == has_scales and (v.codebooks is not None) == has_cbk
        # every plane lies inside the prepared buffer
        end = FAKE + W.wqd_prepared_bytes(fmt, N, K)
        for p in (v.scales, v.codebooks):
            assert p is None or FAKE < p < end
        assert v.scale_row_elems == {I.Q4_0: K // 32, I.TQ2: K // 128, I.AQ2X8: 1, I.AQ1X16: 1}.get(fmt, 0)
        assert v.code_row_bytes == {I.Q4_0: K // 2, I.CB4: K // 2, I.CB8: K}.get(fmt, K // 4)


def test_bind_errors():
    L, v = W.lib(), W.wqd_weight()
    assert L.wqd_bind(9, 64, 64, FAKE, ctypes.byref(v)) == W.WQD_EINVAL     # unknown format
    assert L.wqd_bind(1, 64, 48, FAKE, ctypes.byref(v)) == W.WQD_ESHAPE     # K not whole blocks
    assert L.wqd_bind(1, 0, 64, FAKE, ctypes.byref(v)) == W.WQD_ESHAPE      # N = 0
    assert L.wqd_bind(1, 64, 64, None, ctypes.byref(v)) == W.WQD_EINVAL     # null buffer
    assert L.wqd_bind(1, 64, 64, FAKE, None) == W.WQD_EINVAL                # null view
    assert L.wqd_bind(1, 64, 64, FAKE + 8, ctypes.byref(v)) == W.WQD_EALIGN  # buffer not 16-byte aligned


def _edited(base_fmt, **fields):
    w = _view(base_fmt, 64, 64)
    for k, val in fields.items():
        setattr(w.view, k, val)
    return w


@pytest.mark.parametrize("spec,x,M,ldx,y,ldy,status", [
    ((1, dict(fmt=9)), FAKE, 1, 64, FAKE, 64, W.WQD_EINVAL),                 # unknown format
    ((1, dict(K=48)), FAKE, 1, 64, FAKE, 64, W.WQD_ESHAPE),                  # K not whole blocks
    ((1, dict(K=128)), FAKE, 1, 128, FAKE, 64, W.WQD_ESHAPE),                # row sizes of another K
    ((1, dict(scale_row_elems=1)), FAKE, 1, 64, FAKE, 64, W.WQD_ESHAPE),     # scale rows disagree
    ((1, {}), FAKE, 0, 64, FAKE, 64, W.WQD_ESHAPE),                  # M = 0
    ((1, {}), FAKE, 9, 64, FAKE, 64, W.WQD_ESHAPE),                  # M = 9
    ((1, {}), FAKE, 1, 32, FAKE, 64, W.WQD_ESHAPE),                  # ldx < K
    ((1, {}), FAKE, 1, 64, FAKE, 10, W.WQD_ESHAPE),                  # ldy < N
    ((1, dict(codes=FAKE + 8)), FAKE, 1, 64, FAKE, 64, W.WQD_EALIGN),        # codes not 16-byte aligned
    ((1, dict(scales=FAKE + 4100)), FAKE, 1, 64, FAKE, 64, W.WQD_EALIGN),    # Q4_0 scales not 8-byte aligned
    ((5, dict(codebooks=FAKE + 8)), FAKE, 1, 64, FAKE, 64, W.WQD_EALIGN),    # AQ2X8 codebooks not 16-byte aligned
    ((1, {}), FAKE + 2, 1, 64, FAKE, 64, W.WQD_EALIGN),              # x not 4-byte aligned
    ((1, {}), FAKE, 1, 65, FAKE, 64, W.WQD_EALIGN),                  # odd ldx
    ((1, dict(codes=None)), FAKE, 1, 64, FAKE, 64, W.WQD_EINVAL),            # null codes
    ((1, dict(scales=None)), FAKE, 1, 64, FAKE, 64, W.WQD_EINVAL),           # Q4_0 without scales
    ((2, dict(codebooks=None)), FAKE, 1, 64, FAKE, 64, W.WQD_EINVAL),        # CB4 without a codebook
    ((1, {}), None, 1, 64, FAKE, 64, W.WQD_EINVAL),                  # null x
])
def test_gemm_argument_errors_before_any_launch(spec, x, M, ldx, y, ldy, status):
    w = _edited(spec[0], **spec[1])
    L = W.lib()
    assert L.wqd_gemm(w.ref(), x, M, ldx, y, ldy, None, 0, None) == status
    assert L.wqd_gemm_noalloc(w.ref(), x, M, ldx, y, ldy, None) == status


def test_gemm_null_view():
    L = W.lib()
    assert L.wqd_gemm(None, FAKE, 1, 64, FAKE, 64, None, 0, None) == W.WQD_EINVAL
    assert L.wqd_workspace_bytes(None, 1) == W.WQD_EINVAL
    assert L.wqd_dequant_f32(None, FAKE, None) == W.WQD_EINVAL


def test_workspace_bytes_rules():
    w = _view(I.Q4_0, 64, 32768)
    assert W.wqd_workspace_bytes(w, 1) > 0                       # long K: split, needs counters
    assert W.lib().wqd_workspace_bytes(w.ref(), 0) == W.WQD_ESHAPE
    assert W.lib().wqd_workspace_bytes(w.ref(), 9) == W.WQD_ESHAPE
    assert W.lib().wqd_workspace_bytes(_edited(1, fmt=9).ref(), 1) == W.WQD_EINVAL


def test_gemm_workspace_too_small_is_reported():
    # one 64-row group with a long K: its K is split, so it needs counters and partials
    w = _view(I.Q4_0, 64, 32768)
    need = W.wqd_workspace_bytes(w, 1)
    assert need > 0
    assert W.lib().wqd_gemm(w.ref(), FAKE, 1, 32768, FAKE, 64, FAKE, need - 4, None) == W.WQD_ESPACE


def _list(entries):
    """wqd_proj array of (fmt, N, K, epi, x) entries on never-dereferenced pointers."""
    arr = (W.wqd_proj * len(entries))()
    keep = []
    for i, (fmt, N, K, epi, x) in enumerate(entries):
        w = _view(fmt, N, K, FAKE + (i << 26))
        keep.append(w)
        arr[i].w = ctypes.pointer(w.view)
        arr[i].epi, arr[i].x, arr[i].ldx = epi, x, K
        arr[i].y, arr[i].ldy = FAKE + (i << 26) + (1 << 25), N
    arr._keep = keep
    return arr


_fake_list = _list


def test_run_projections_rejects_bad_mode_and_lists():
    arr = _list([(I.CB4, 64, 64, W.WQD_EPI_NONE, FAKE)])
    L = W.lib()
    assert L.wqd_run_projections(arr, 1, 1, 7, FAKE, 1 << 20, None) == W.WQD_EINVAL
    assert L.wqd_run_projections(arr, 1, 0, 0, FAKE, 1 << 20, None) == W.WQD_ESHAPE
    arr[0].epi = 7  # no such epilogue
    assert L.wqd_run_projections(arr, 1, 1, 0, FAKE, 1 << 20, None) == W.WQD_EINVAL
    assert L.wqd_stack_workspace_bytes(arr, 1, 1) == W.WQD_EINVAL
    arr[0].epi = W.WQD_EPI_NONE
    arr[0].w = None  # an entry without a weight view
    assert L.wqd_stack_workspace_bytes(arr, 1, 1) == W.WQD_EINVAL
    bad = _edited(I.CB4, codes=FAKE + 4)  # a view that fails its own checks
    arr[0].w = ctypes.pointer(bad.view)
    assert L.wqd_stack_workspace_bytes(arr, 1, 1) == W.WQD_EALIGN


G, U, A, E0 = W.WQD_EPI_SILU_GATE, W.WQD_EPI_SILU_UP, W.WQD_EPI_ADD, W.WQD_EPI_NONE


@pytest.mark.parametrize("entries", [
    [(I.CB4, 64, 64, G, FAKE)],                                   # gate without its up
    [(I.CB4, 64, 64, U, FAKE)],                                   # up without its gate
    [(I.CB4, 64, 64, G, FAKE), (I.CB4, 64, 64, E0, FAKE)],        # gate followed by a plain entry
    [(I.CB4, 64, 64, G, FAKE), (I.CB4, 128, 64, U, FAKE)],        # pair with different N
    [(I.CB4, 64, 64, G, FAKE), (I.CB8, 64, 64, U, FAKE)],         # pair with different formats
    [(I.CB4, 64, 64, E0, FAKE), (I.CB4, 64, 64, U, FAKE)],        # up after a plain entry
    [(I.AQ2X8, 64, 64, A, FAKE)],                                 # no epilogue on AQ2X8
])
def test_epilogue_list_errors(entries):
    arr = _fake_list(entries)
    L = W.lib()
    for mode in (W.WQD_ORDERED, W.WQD_PERSISTENT, W.WQD_FUSED):
        assert L.wqd_run_projections(arr, len(arr), 1, mode, FAKE, 1 << 30, None) == W.WQD_EINVAL
        assert L.wqd_stack_launches(arr, len(arr), 1, mode) == W.WQD_EINVAL
    assert L.wqd_stack_workspace_bytes(arr, len(arr), 1) == W.WQD_EINVAL


def test_up_entry_may_have_no_output():
    arr = _fake_list([(I.CB4, 64, 64, G, FAKE), (I.CB4, 64, 64, U, FAKE)])
    arr[1].y, arr[1].ldy = None, 0
    assert W.lib().wqd_stack_workspace_bytes(arr, 2, 1) > 0
    arr[0].y = None  # but the gate's output is where the pair writes
    assert W.lib().wqd_stack_workspace_bytes(arr, 2, 1) == W.WQD_EINVAL


def _layer(x_in, x_attn, x_mlp):
    # a 7B layer with its epilogues: q, k, v on the layer input; o + residual; gate/up pair;
    # down + residual
    return [(I.CB4, 4096, 4096, E0, x_in), (I.CB4, 4096, 4096, E0, x_in), (I.CB4, 4096, 4096, E0, x_in),
            (I.CB4, 4096, 4096, A, x_attn), (I.CB4, 11008, 4096, G, x_in), (I.CB4, 11008, 4096, U, x_in),
            (I.CB4, 4096, 11008, A, x_mlp)]


def test_launch_counts_per_mode():
    L = W.lib()
    X = [FAKE + (1 << 40) + (j << 20) for j in range(8)]
    arr = _fake_list(_layer(X[0], X[1], X[2]) + _layer(X[3], X[4], X[5]))
    n = len(arr)
    assert L.wqd_stack_launches(arr, n, 1, W.WQD_PERSISTENT) == 1
    assert L.wqd_stack_launches(arr, n, 1, W.WQD_ORDERED) == 12   # the pair is one launch
    assert L.wqd_stack_launches(arr, n, 1, W.WQD_FUSED) == 8      # qkv, o, gate/up, down per layer
    assert L.wqd_stack_launches(arr, n, 1, 3) == W.WQD_EINVAL
    # runs hold at most 4 entries and never split a pair
    same = _fake_list([(I.CB4, 64, 64, E0, X[6])] * 3 + [(I.CB4, 64, 64, G, X[6]), (I.CB4, 64, 64, U, X[6])]
                      + [(I.CB4, 64, 64, E0, X[6])] * 6)
    assert L.wqd_stack_launches(same, len(same), 1, W.WQD_FUSED) == 3  # 3 | pair + 2 | 4
    # a different x or format ends a run; AQ2X8 entries run alone
    mixed = _fake_list([(I.CB4, 64, 64, E0, X[6]), (I.CB4, 64, 64, E0, X[7]), (I.CB8, 64, 64, E0, X[7]),
                        (I.AQ2X8, 64, 64, E0, X[7]), (I.AQ2X8, 64, 64, E0, X[7])])
    assert L.wqd_stack_launches(mixed, len(mixed), 1, W.WQD_FUSED) == 5


def test_pair_needs_a_workspace():
    arr = _fake_list([(I.CB4, 64, 64, G, FAKE), (I.CB4, 64, 64, U, FAKE)])
    L = W.lib()
    for mode in (W.WQD_ORDERED, W.WQD_FUSED):
        assert L.wqd_run_projections(arr, 2, 1, mode, None, 0, None) == W.WQD_ESPACE
    need = L.wqd_stack_workspace_bytes(arr, 2, 1)
    assert L.wqd_run_projections(arr, 2, 1, W.WQD_FUSED, FAKE, need - 256, None) == W.WQD_ESPACE


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert W.wqd_status_str(s)


def test_batch_invariant_flag_rules():
    L = W.lib()
    BI = W.WQD_BATCH_INVARIANT
    aq = _fake_list([(I.CB4, 64, 64, E0, FAKE), (I.AQ2X8, 64, 64, E0, FAKE)])
    for mode in (W.WQD_ORDERED, W.WQD_PERSISTENT, W.WQD_FUSED):
        assert L.wqd_stack_launches(aq, 2, 1, mode | BI) == 2
    assert L.wqd_stack_workspace_bytes(aq, 2, 1) > 0
    X = FAKE + (1 << 40)
    mixed = _fake_list([(I.CB4, 4096, 4096, E0, X), (I.CB8, 4096, 4096, E0, X)])
    assert L.wqd_stack_launches(mixed, 2, 1, W.WQD_PERSISTENT) == 1        # CB4 and CB8 together
    assert L.wqd_stack_launches(mixed, 2, 1, W.WQD_PERSISTENT | BI) == 2   # one instance each
    assert L.wqd_stack_setup(mixed, 2, 1, W.WQD_ORDERED, FAKE, 1 << 30, None) == W.WQD_EINVAL
    assert L.wqd_run_projections(mixed, 2, 1, 3 | BI, FAKE, 1 << 30, None) == W.WQD_EINVAL


def test_int8_entry_point_rules():
    L = W.lib()
    cb, tq = _view(I.CB4, 64, 1024), _view(I.TQ2, 64, 1024)
    assert L.wqd_gemm_i8_workspace_bytes(cb.ref(), 1) == W.WQD_EINVAL  # TQ2 only
    assert L.wqd_gemm_i8_workspace_bytes(tq.ref(), 1) > 0
    assert L.wqd_gemm_i8(tq.ref(), FAKE, 1, 1024, FAKE, 64, None, 0, None) == W.WQD_EINVAL
    need = L.wqd_gemm_i8_workspace_bytes(tq.ref(), 1)
    assert L.wqd_gemm_i8(tq.ref(), FAKE, 1, 1024, FAKE, 64, FAKE, need - 1, None) == W.WQD_ESPACE
    assert L.wqd_gemm_i8(tq.ref(), FAKE, 1, 1000, FAKE, 64, FAKE, need, None) == W.WQD_ESHAPE
    assert L.wqd_quantize_i8(FAKE, 1, 100, 128, FAKE, FAKE, FAKE, None) == W.WQD_ESHAPE
    assert L.wqd_quantize_i8(None, 1, 128, 128, FAKE, FAKE, FAKE, None) == W.WQD_EINVAL


def test_int8_list_launch_counts():
    L = W.lib()
    I8 = W.WQD_INT8_ACTIVATIONS
    X = [FAKE + (1 << 40) + (j << 20) for j in range(3)]
    mlp = _fake_list([(I.TQ2, 17408, 5120, E0, X[0]), (I.TQ2, 17408, 5120, E0, X[0]),
                      (I.TQ2, 5120, 17408, E0, X[1])])
    assert L.wqd_stack_launches(mlp, 3, 1, W.WQD_PERSISTENT | I8) == 2  # 1 quantizer (both x) + 1 product
    assert L.wqd_stack_launches(mlp, 3, 1, W.WQD_FUSED | I8) == 4       # q(x0) [gate, up] q(x1) [down]
    assert L.wqd_stack_launches(mlp, 3, 1, W.WQD_ORDERED | I8) == 5
    assert L.wqd_stack_launches(mlp, 3, 1, W.WQD_PERSISTENT) == 1
    nine = _fake_list([(I.TQ2, 256, 1024, E0, FAKE + (1 << 40) + (j << 20)) for j in range(9)])
    assert L.wqd_stack_launches(nine, 9, 1, W.WQD_PERSISTENT | I8) == 3  # 8 + 1 activations, then the product
    cb = _fake_list([(I.CB4, 64, 64, E0, X[2])])
    assert L.wqd_stack_launches(cb, 1, 1, W.WQD_PERSISTENT | I8) == 1    # no TQ2 entry: no quantizer
    assert L.wqd_stack_workspace_bytes(mlp, 3, 1) > 0


@pytest.mark.parametrize("fmt", [I.Q4_0, I.CB4, I.CB8, I.TQ2, I.AQ2X8, I.AQ1X16])
def test_size_limits(fmt):
    """N and K up to 2^30 are accepted (sizes only; nothing is allocated), one block more is not."""
    kb = {I.Q4_0: 32, I.CB4: 2, I.CB8: 1, I.TQ2: 128, I.AQ2X8: 8, I.AQ1X16: 8}[fmt]
    assert W.wqd_prepared_bytes(fmt, W.WQD_MAX_N, 1024) > 0
    assert W.wqd_prepared_bytes(fmt, 64, W.WQD_MAX_K) > 0
    assert W.wqd_canonical_bytes(fmt, W.WQD_MAX_N, 1024) > 0
    assert W.lib().wqd_prepared_bytes(fmt, W.WQD_MAX_N + 1, 1024) == W.WQD_ESHAPE
    assert W.lib().wqd_prepared_bytes(fmt, 64, W.WQD_MAX_K + kb) == W.WQD_ESHAPE
    assert W.lib().wqd_canonical_bytes(fmt, 64, W.WQD_MAX_K + kb) == W.WQD_ESHAPE
    v = W.wqd_weight()
    assert W.lib().wqd_bind(fmt, W.WQD_MAX_N + 1, 1024, FAKE, ctypes.byref(v)) == W.WQD_ESHAPE
    assert W.lib().wqd_bind(fmt, 64, W.WQD_MAX_K + kb, FAKE, ctypes.byref(v)) == W.WQD_ESHAPE
    big = _view(fmt, W.WQD_MAX_N, 1024)
    big.view.N = W.WQD_MAX_N + 1  # a hand-edited view past the limit
    assert W.lib().wqd_gemm(big.ref(), FAKE, 1, 1024, FAKE, W.WQD_MAX_N + 1, None, 0, None) == W.WQD_ESHAPE


def test_aq2x8_launch_counts():
    """The AQ2X8 entries of a segment share one launch at every M (the lookup-table kernel at
    M = 1, the matrix-core kernel above and in batch-invariant lists)."""
    L = W.lib()
    X = FAKE + (1 << 40)
    arr = _fake_list([(I.CB4, 64, 64, E0, X), (I.AQ2X8, 128, 1024, E0, X), (I.AQ2X8, 64, 512, E0, X)])
    n = len(arr)
    for M in range(1, 9):
        assert L.wqd_stack_launches(arr, n, M, W.WQD_PERSISTENT) == 2, M       # CB4 + AQ2X8
        assert L.wqd_stack_launches(arr, n, M, W.WQD_ORDERED) == 3, M          # one entry each
        assert L.wqd_stack_launches(arr, n, M, W.WQD_PERSISTENT | W.WQD_BATCH_INVARIANT) == 2, M


def test_gemm_noalloc_rejects_shapes_beyond_the_scratch():
    # an 8-row CB8 call over 2^20 rows with split K needs more than the scratch array holds: the
    # call is refused before any HIP call (the pointers are never read)
    N, K, M = 1 << 20, 4096, 8
    w = _view(I.CB8, N, K, 256)
    need = W.wqd_workspace_bytes(w, M)
    assert need > W.WQD_NOALLOC_MAX_BYTES
    assert W.lib().wqd_gemm_noalloc(w.ref(), 256, M, K, 256, N, None) == W.WQD_ESPACE
    # argument errors come first, as for wqd_gemm
    assert W.lib().wqd_gemm_noalloc(w.ref(), None, M, K, 256, N, None) == W.WQD_EINVAL
    assert W.lib().wqd_gemm_noalloc(w.ref(), 256, 9, K, 256, N, None) == W.WQD_ESHAPE


def test_binding_checks_tensors_before_any_call():
    """The Python binding refuses host tensors, wrong dtypes and shapes before it passes a pointer."""
    import torch
    w = _view(I.CB4, 64, 64)
    x_host = torch.zeros((1, 64), dtype=torch.int16)
    y_host = torch.zeros((1, 64), dtype=torch.float32)
    with pytest.raises(TypeError):
        W.wqd_gemm(w, x_host, y_host)
    with pytest.raises(TypeError):
        W.wqd_gemm_noalloc(w, x_host, y_host)
    with pytest.raises(TypeError):
        W.make_proj_array([dict(w=w, x=x_host, y=y_host)])
    with pytest.raises(TypeError):
        W.wqd_bind(I.CB4, 64, 64, torch.zeros(4096, dtype=torch.uint8))  # a host buffer


def test_verify_rows_limits():
    """Up to 16 rows in batch-invariant lists (one pass); otherwise at most 8; the AQ2X8 entries of a
    9..16-row verify run as two launches (rows 0..7, 8..)."""
    L = W.lib()
    BI, I8 = W.WQD_BATCH_INVARIANT, W.WQD_INT8_ACTIVATIONS
    X = FAKE + (1 << 40)
    arr = _list([(I.CB4, 4096, 4096, E0, X), (I.AQ2X8, 1024, 4096, E0, X)])
    assert L.wqd_stack_launches(arr, 2, 16, W.WQD_PERSISTENT | BI) == 3   # CB4, AQ2X8 rows 0..7, 8..15
    assert L.wqd_stack_launches(arr, 2, 8, W.WQD_PERSISTENT | BI) == 2
    assert L.wqd_stack_launches(arr, 2, 12, W.WQD_ORDERED | BI) == 3
    assert L.wqd_stack_launches(arr, 2, 9, W.WQD_PERSISTENT) == W.WQD_ESHAPE     # not batch-invariant
    assert L.wqd_stack_launches(arr, 2, 17, W.WQD_PERSISTENT | BI) == W.WQD_ESHAPE
    tq = _list([(I.TQ2, 256, 1024, E0, X)])
    assert L.wqd_stack_launches(tq, 1, 9, W.WQD_PERSISTENT | BI | I8) == W.WQD_ESHAPE  # int8: 8 rows
    assert L.wqd_stack_workspace_bytes(arr, 2, 16) > L.wqd_stack_workspace_bytes(arr, 2, 8) > 0
    assert L.wqd_stack_workspace_bytes(arr, 2, 17) == W.WQD_ESHAPE
