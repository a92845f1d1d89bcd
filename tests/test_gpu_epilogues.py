"""GPU parity of the fused projection epilogues against the CPU oracle, through the C ABI.

trapetum "Benchmarks", "Short-context decode, step by step": the gate/up projection applies
SiLU(gate) * up in its reduce, and the o and down projections add the residual in theirs.

Bounds (derived from the per-projection bound |s_gpu - s| <= eps = 2e-3 * sum|x w| + 1e-6):
* residual y = r + s:  |y_gpu - y_ref| <= eps + 2^-23 * (|r| + |s|)  (one fp32 rounding of the add);
* pair h = SiLU(g) * u:  |h_gpu - h_ref| <= 1.1 * eps_g * (|u| + eps_u) + |SiLU(g)| * eps_u
  + 1e-6 * |h| + 1e-6, since |SiLU'| <= 1.1 everywhere, and the fp32 evaluation of
  g / (1 + e^-g) * u adds a few ulps (1e-6 relative covers 16 of them).
"""
import numpy as np
import pytest

import oracle
from weight_quantized_decode_amd import _lib as W
from weight_quantized_decode_amd import inputs as I

from gpu_util import ABS_TOL, REL_TOL, new_y, note, upload_weight, upload_x, workspace

pytestmark = pytest.mark.gpu

MODES = {"ordered": W.WQD_ORDERED, "persistent": W.WQD_PERSISTENT, "fused": W.WQD_FUSED}

# several 64-row tiles with a ragged last one; long K splits into K-slices, short K does not
SHAPES = [
    (I.Q4_0, 200, 1024), (I.Q4_0, 130, 4128),
    (I.CB4, 77, 4098), (I.CB4, 1, 2),
    (I.CB8, 200, 1001), (I.CB8, 3, 1),
    (I.TQ2, 70, 128), (I.TQ2, 130, 17408),
    (I.AQ1X16, 100, 4104),
]


def _bad(err, bound, what, got, ref):
    bad = ~(err <= bound)
    if bad.any():
        idx = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} outputs outside the bound; first {list(idx)}: "
                             f"gpu {got[idx]} ref {ref[idx]} bound {bound[idx]}")


def check_pair(h_gpu, h, g, u, ag, au, what):
    got = np.asarray(h_gpu, dtype=np.float64)
    eg, eu = REL_TOL * ag + ABS_TOL, REL_TOL * au + ABS_TOL
    sg = np.abs(oracle.silu_mul(g, np.ones_like(g)))
    bound = 1.1 * eg * (np.abs(u) + eu) + sg * eu + 1e-6 * np.abs(h) + ABS_TOL
    _bad(np.abs(got - h), bound, what, got, h)


def check_residual(y_gpu, r, s, a, what):
    got = np.asarray(y_gpu, dtype=np.float64)
    ref = oracle.residual_add(r, s)
    bound = REL_TOL * a + ABS_TOL + 2.0 ** -23 * (np.abs(r) + np.abs(s))
    _bad(np.abs(got - ref), bound, what, got, ref)


def _run(entries, M, mode, ws=None):
    arr = W.make_proj_array(entries)
    if ws is None:
        ws = workspace(W.wqd_stack_workspace_bytes(arr, M))
    if mode == W.WQD_PERSISTENT:
        W.wqd_stack_setup(arr, M, ws)
    W.wqd_run_projections(arr, M, mode, ws)
    W.wqd_stream_check()
    return ws


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("fmt,N,K", SHAPES)
def test_silu_pair_parity(fmt, N, K, M, mode):
    import torch
    note(f"silu pair fmt={fmt} N={N} K={K} M={M} mode={mode}")
    cg = I.gen_weight(fmt, N, K, (40, fmt, N, K, 0))
    cu = I.gen_weight(fmt, N, K, (40, fmt, N, K, 1))
    xb = I.gen_x(M, K, (40, fmt, N, K, M))
    x = upload_x(xb)
    h = new_y(M, N, ldy=N + 5)       # padding of h must stay NaN
    up_y = new_y(M, N)               # the up entry's y is never written
    _run([dict(fmt=fmt, N=N, K=K, w=upload_weight(fmt, N, K, cg), x=x, y=h, epi=W.WQD_EPI_SILU_GATE),
          dict(fmt=fmt, N=N, K=K, w=upload_weight(fmt, N, K, cu), x=x, y=up_y, epi=W.WQD_EPI_SILU_UP)],
         M, MODES[mode])
    href, g, u, ag, au = oracle.silu_pair_f64(fmt, N, K, cg, cu, xb, xb)
    check_pair(h.cpu().numpy(), href, g, u, ag, au, f"pair fmt={fmt} N={N} K={K} M={M} {mode}")
    full = h.as_strided((M, N + 5), (N + 5, 1)).cpu().numpy()
    assert np.isnan(full[:, N:]).all()
    assert torch.isnan(up_y).all()


@pytest.mark.parametrize("mode", list(MODES))
def test_silu_pair_with_own_x_and_k_for_up(mode):
    # gate and up may read different activations and have different K (same format and N)
    fmt, N = I.CB4, 300
    note(f"silu pair, gate K=1024 and up K=2050 on their own x, mode={mode}")
    M = 4
    cg = I.gen_weight(fmt, N, 1024, (41, 0))
    cu = I.gen_weight(fmt, N, 2050, (41, 1))
    xg, xu = I.gen_x(M, 1024, (41, 2)), I.gen_x(M, 2050, (41, 3))
    h = new_y(M, N)
    _run([dict(fmt=fmt, N=N, K=1024, w=upload_weight(fmt, N, 1024, cg), x=upload_x(xg), y=h,
               epi=W.WQD_EPI_SILU_GATE),
          dict(fmt=fmt, N=N, K=2050, w=upload_weight(fmt, N, 2050, cu), x=upload_x(xu), y=None,
               epi=W.WQD_EPI_SILU_UP)], M, MODES[mode])
    g, ag = oracle.gemm_f64(fmt, N, 1024, cg, xg)
    u, au = oracle.gemm_f64(fmt, N, 2050, cu, xu)
    check_pair(h.cpu().numpy(), oracle.silu_mul(g, u), g, u, ag, au, f"pair own x {mode}")


@pytest.mark.parametrize("mode", list(MODES))
def test_silu_pair_saturating_gate(mode):
    # a wide codebook makes |g| reach ~100: SiLU(g) is g above and -0 below (e^-g overflows fp32)
    fmt, N, K, M = I.CB8, 256, 1001, 2
    note(f"silu pair with |gate| up to ~100, mode={mode}")
    cg = I.gen_weight(fmt, N, K, (42, 0), cb_sigma=3.0)
    cu = I.gen_weight(fmt, N, K, (42, 1))
    xb = I.gen_x(M, K, (42, 2))
    x = upload_x(xb)
    h = new_y(M, N)
    _run([dict(fmt=fmt, N=N, K=K, w=upload_weight(fmt, N, K, cg), x=x, y=h, epi=W.WQD_EPI_SILU_GATE),
          dict(fmt=fmt, N=N, K=K, w=upload_weight(fmt, N, K, cu), x=x, y=None, epi=W.WQD_EPI_SILU_UP)],
         M, MODES[mode])
    href, g, u, ag, au = oracle.silu_pair_f64(fmt, N, K, cg, cu, xb, xb)
    assert g.max() > 40 and g.min() < -40
    check_pair(h.cpu().numpy(), href, g, u, ag, au, f"saturating pair {mode}")


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("fmt,N,K", SHAPES)
def test_residual_add_parity(fmt, N, K, M, mode):
    import torch
    note(f"residual add fmt={fmt} N={N} K={K} M={M} mode={mode}")
    canon = I.gen_weight(fmt, N, K, (43, fmt, N, K))
    xb = I.gen_x(M, K, (43, fmt, N, K, M))
    r = np.random.default_rng(43 + N + K + M).standard_normal((M, N)).astype(np.float32)
    y = new_y(M, N, ldy=N + 3)
    y.copy_(torch.from_numpy(r))
    _run([dict(fmt=fmt, N=N, K=K, w=upload_weight(fmt, N, K, canon), x=upload_x(xb), y=y,
               epi=W.WQD_EPI_ADD)], M, MODES[mode])
    s, a = oracle.gemm_f64(fmt, N, K, canon, xb)
    check_residual(y.cpu().numpy(), r, s, a, f"residual fmt={fmt} N={N} K={K} M={M} {mode}")
    full = y.as_strided((M, N + 3), (N + 3, 1)).cpu().numpy()
    assert np.isnan(full[:, N:]).all()


def _layer_entries(M, key, scale=1):
    """One 7B-shaped CB4 layer with its epilogues (N and K divided by `scale`): q, k, v on the
    layer input; o + residual on the attention output; the gate/up pair on the layer input;
    down + residual on the MLP hidden state."""
    d, f = 4096 // scale, 11008 // scale
    xs = {role: I.gen_x(M, K, (44, key, role)) for role, K in ((0, d), (1, d), (2, f))}
    xd = {role: upload_x(v) for role, v in xs.items()}
    spec = [("q", d, d, 0, W.WQD_EPI_NONE), ("k", d, d, 0, W.WQD_EPI_NONE), ("v", d, d, 0, W.WQD_EPI_NONE),
            ("o", d, d, 1, W.WQD_EPI_ADD), ("gate", f, d, 0, W.WQD_EPI_SILU_GATE),
            ("up", f, d, 0, W.WQD_EPI_SILU_UP), ("down", d, f, 2, W.WQD_EPI_ADD)]
    ent, host = [], []
    for i, (name, N, K, role, epi) in enumerate(spec):
        canon = I.gen_weight(I.CB4, N, K, (44, key, i))
        ent.append(dict(fmt=I.CB4, N=N, K=K, w=upload_weight(I.CB4, N, K, canon), x=xd[role],
                        y=None if epi == W.WQD_EPI_SILU_UP else new_y(M, N), epi=epi))
        host.append((name, N, K, canon, xs[role], epi))
    return ent, host


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("M", [1, 8])
def test_full_size_layer_with_epilogues(M, mode):
    """A 7B-shaped layer at full size in one call, sampled rows checked against the oracle."""
    import torch
    note(f"7B layer with epilogues M={M} mode={mode}")
    ent, host = _layer_entries(M, 1)
    rng = np.random.default_rng(45)
    res = {}
    for e, (name, N, K, canon, xb, epi) in zip(ent, host):
        if epi == W.WQD_EPI_ADD:
            res[name] = rng.standard_normal((M, N)).astype(np.float32)
            e["y"].copy_(torch.from_numpy(res[name]))
    _run(ent, M, MODES[mode])
    for i, (e, (name, N, K, canon, xb, epi)) in enumerate(zip(ent, host)):
        if epi == W.WQD_EPI_SILU_UP:
            continue
        rows = np.unique(np.concatenate([[0, 63, 64, N - 1], rng.integers(0, N, size=40)])).astype(np.int64)
        got = e["y"].cpu().numpy()[:, rows]
        if epi == W.WQD_EPI_SILU_GATE:
            _, _, _, canon_u, xu, _ = host[i + 1]
            h, g, u, ag, au = oracle.silu_pair_f64(I.CB4, N, K, canon, canon_u, xb, xu, rows=rows)
            check_pair(got, h, g, u, ag, au, f"layer {name} M={M} {mode}")
        else:
            s, a = oracle.gemm_f64(I.CB4, N, K, canon, xb, rows=rows)
            if epi == W.WQD_EPI_ADD:
                check_residual(got, res[name][:, rows], s, a, f"layer {name} M={M} {mode}")
            else:
                bound = REL_TOL * a + ABS_TOL
                _bad(np.abs(got - s), bound, f"layer {name} M={M} {mode}", got, s)


def test_fused_runs_are_deterministic_and_leave_counters_zero():
    """Two FUSED calls give the same bits, and the workspace then serves the other modes."""
    import torch
    M = 2
    note("fused layer twice, then ordered and persistent on the same workspace")
    ent, host = _layer_entries(M, 2, scale=4)
    arr = W.make_proj_array(ent)
    ws = workspace(W.wqd_stack_workspace_bytes(arr, M))
    outs = []
    for mode in (W.WQD_FUSED, W.WQD_FUSED, W.WQD_ORDERED, W.WQD_PERSISTENT):
        for e in ent:
            if e["y"] is not None:
                e["y"].fill_(0.25)  # the residual of the ADD entries
        _run(ent, M, mode, ws)
        outs.append([e["y"].cpu().numpy().copy() for e in ent if e["y"] is not None])
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)
    # the other modes, on the same workspace, agree with it up to their summation order
    for o in outs[2:]:
        for a, b in zip(outs[0], o):
            np.testing.assert_allclose(a, b, rtol=1e-3, atol=1e-3)


def test_fused_layer_in_a_graph_replays_like_eager():
    """A FUSED call captured in a HIP graph: every replay (with eager work and synchronization
    in between) gives the eager call's bits."""
    import torch
    M = 1
    note("fused layer captured in a graph, 3 replays")
    ent, host = _layer_entries(M, 3, scale=4)
    arr = W.make_proj_array(ent)
    ws = workspace(W.wqd_stack_workspace_bytes(arr, M))
    outs = [e["y"] for e in ent if e["y"] is not None]

    def reset():
        for y in outs:
            y.fill_(0.5)

    reset()
    W.wqd_run_projections(arr, M, W.WQD_FUSED, ws)
    W.wqd_stream_check()
    eager = [y.cpu().numpy().copy() for y in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        reset()
        W.wqd_run_projections(arr, M, W.WQD_FUSED, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        W.wqd_run_projections(arr, M, W.WQD_FUSED, ws)
    for rep in range(3):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, y in zip(eager, outs):
            assert np.array_equal(a, y.cpu().numpy()), f"replay {rep} differs from the eager call"
    del g
