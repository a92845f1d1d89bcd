"""Batch-invariant calls (WQD_BATCH_INVARIANT): row m of an M-row call carries the bits of the same
call made with row m alone, for M = 2..16 (9..16 rows in one pass over the weights), in every mode,
with epilogues, and whatever else the list holds (trapetum "Benchmarks", November update: a verify pass whose rows equal M decode
steps bit for bit).  Every result is also checked against the oracle's bound."""
import numpy as np
import pytest

import oracle
from weight_quantized_decode_amd import _lib as W
from weight_quantized_decode_amd import inputs as I

from gpu_util import check_parity, new_y, note, upload_weight, upload_x, workspace

pytestmark = pytest.mark.gpu

BI = W.WQD_BATCH_INVARIANT
MODES = {"ordered": W.WQD_ORDERED, "persistent": W.WQD_PERSISTENT, "fused": W.WQD_FUSED}

# ragged tiles; long K (split into slices), short K (workgroup-split), partial last chunks
SHAPES = [
    (I.Q4_0, 200, 1024), (I.Q4_0, 130, 4128),
    (I.CB4, 77, 4098), (I.CB4, 300, 11008),
    (I.CB8, 200, 1001), (I.CB8, 3, 1),
    (I.TQ2, 70, 128), (I.TQ2, 130, 17408),
    (I.AQ1X16, 100, 4104),
    (I.AQ2X8, 200, 1000), (I.AQ2X8, 129, 8192),
]


def _run(entries, M, mode):
    arr = W.make_proj_array(entries)
    ws = workspace(W.wqd_stack_workspace_bytes(arr, M))
    if (mode & ~BI) == W.WQD_PERSISTENT:
        W.wqd_stack_setup(arr, M, ws, mode=mode)
    W.wqd_run_projections(arr, M, mode, ws)
    W.wqd_stream_check()


def _rows_alone(fmt, N, K, w, xb, mode, epi=W.WQD_EPI_NONE, y0=None):
    """The call made with each activation row alone (M = 1)."""
    import torch
    out = []
    for m in range(xb.shape[0]):
        y = new_y(1, N)
        if y0 is not None:
            y.copy_(torch.from_numpy(y0[m:m + 1]))
        _run([dict(fmt=fmt, N=N, K=K, w=w, x=upload_x(xb[m:m + 1]), y=y, epi=epi)], 1, mode)
        out.append(y.cpu().numpy()[0])
    return np.stack(out)


@pytest.mark.parametrize("M", [2, 3, 5, 8, 12, 16])
@pytest.mark.parametrize("fmt,N,K", SHAPES)
def test_rows_equal_single_row_calls(fmt, N, K, M):
    note(f"batch-invariant fmt={fmt} N={N} K={K} M={M}")
    canon = I.gen_weight(fmt, N, K, (60, fmt, N, K))
    xb = I.gen_x(M, K, (60, fmt, N, K, M))
    w = upload_weight(fmt, N, K, canon)
    y = new_y(M, N)
    _run([dict(fmt=fmt, N=N, K=K, w=w, x=upload_x(xb), y=y)], M, W.WQD_ORDERED | BI)
    got = y.cpu().numpy()
    alone = _rows_alone(fmt, N, K, w, xb, W.WQD_ORDERED | BI)
    assert np.array_equal(got.view(np.uint32), alone.view(np.uint32)), \
        f"rows differ from single-row calls at {np.argwhere(got != alone)[:3].tolist()}"
    yref, aref = oracle.gemm_f64(fmt, N, K, canon, xb)
    check_parity(got, yref, aref, f"batch-invariant fmt={fmt} N={N} K={K} M={M}")


@pytest.mark.parametrize("M", [1, 4, 8, 11, 16])
def test_modes_and_list_contents_do_not_change_bits(M):
    """A mixed list (CB4 + CB8 + Q4_0 + TQ2) gives the same bits in every mode, and each entry's
    bits equal the entry run alone."""
    note(f"batch-invariant list in every mode M={M}")
    specs = [(I.CB4, 4096, 4096), (I.CB4, 1100, 4096), (I.CB8, 2000, 4096), (I.Q4_0, 640, 2048),
             (I.TQ2, 512, 5120), (I.AQ2X8, 1024, 4096)]
    xs = {K: I.gen_x(M, K, (61, K, M)) for K in {k for _, _, k in specs}}
    xd = {K: upload_x(v) for K, v in xs.items()}
    ws_ = [upload_weight(f, N, K, I.gen_weight(f, N, K, (61, f, N, K))) for f, N, K in specs]
    res = {}
    for name, mode in MODES.items():
        ent = [dict(fmt=f, N=N, K=K, w=w, x=xd[K], y=new_y(M, N)) for (f, N, K), w in zip(specs, ws_)]
        _run(ent, M, mode | BI)
        res[name] = [e["y"].cpu().numpy() for e in ent]
    for name in ("persistent", "fused"):
        for a, b in zip(res["ordered"], res[name]):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{name} differs from ordered"
    for (f, N, K), w, got in zip(specs, ws_, res["persistent"]):
        y = new_y(M, N)
        _run([dict(fmt=f, N=N, K=K, w=w, x=xd[K], y=y)], M, W.WQD_ORDERED | BI)
        assert np.array_equal(got.view(np.uint32), y.cpu().numpy().view(np.uint32)), f"fmt={f} N={N} alone"


@pytest.mark.parametrize("M", [5, 13])
@pytest.mark.parametrize("mode", list(MODES))
def test_epilogues_keep_rows_invariant(mode, M):
    import torch
    fmt, N, K = I.CB4, 700, 4096
    note(f"batch-invariant epilogues mode={mode}")
    cg = I.gen_weight(fmt, N, K, (62, 0))
    cu = I.gen_weight(fmt, N, K, (62, 1))
    cr = I.gen_weight(fmt, N, K, (62, 2))
    xb = I.gen_x(M, K, (62, 3))
    wg, wu, wr = (upload_weight(fmt, N, K, c) for c in (cg, cu, cr))
    r = np.random.default_rng(62).standard_normal((M, N)).astype(np.float32)

    def call(rows):
        x = upload_x(xb[rows])
        h, yr = new_y(len(rows), N), new_y(len(rows), N)
        yr.copy_(torch.from_numpy(r[rows]))
        _run([dict(fmt=fmt, N=N, K=K, w=wg, x=x, y=h, epi=W.WQD_EPI_SILU_GATE),
              dict(fmt=fmt, N=N, K=K, w=wu, x=x, y=None, epi=W.WQD_EPI_SILU_UP),
              dict(fmt=fmt, N=N, K=K, w=wr, x=x, y=yr, epi=W.WQD_EPI_ADD)], len(rows), MODES[mode] | BI)
        return h.cpu().numpy(), yr.cpu().numpy()

    h, yr = call(list(range(M)))
    for m in range(M):
        h1, yr1 = call([m])
        assert np.array_equal(h[m].view(np.uint32), h1[0].view(np.uint32)), f"pair row {m}"
        assert np.array_equal(yr[m].view(np.uint32), yr1[0].view(np.uint32)), f"residual row {m}"
