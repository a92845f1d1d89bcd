"""Parity at the workloads' full sizes, in the launch configuration the bench times.

The oracle computes sampled output rows one by one (every output of a 64-row tile is still
produced by the GPU; a sample of rows spread over all tiles and splits is compared).  The stack
runs in WQD_PERSISTENT mode (the bench's headline) and in WQD_ORDERED mode.
"""
import numpy as np
import pytest

import oracle
from weight_quantized_decode_amd import _lib as W
from weight_quantized_decode_amd import inputs as I

from gpu_util import check_parity, new_y, note, upload_weight, upload_x, workspace

pytestmark = pytest.mark.gpu


def sample_rows(N, key, n=48):
    r = np.random.default_rng(key)
    rows = np.unique(np.concatenate([[0, 63, 64, N - 1], r.integers(0, N, size=n)]))
    return rows.astype(np.int64)


def run_config(cfg, M, mode, layers=None):
    import torch
    projs = I.config_projections(cfg, layers=layers)
    dev, host = [], []
    xs = {}
    for p in projs:
        canon = I.gen_proj_weight(p)
        if p.xkey not in xs:
            xb = I.gen_proj_x(p, M)
            xs[p.xkey] = (xb, upload_x(xb))
        xb, xd = xs[p.xkey]
        dev.append(dict(fmt=p.fmt, N=p.N, K=p.K, w=upload_weight(p.fmt, p.N, p.K, canon), x=xd,
                        y=new_y(M, p.N)))
        rows = sample_rows(p.N, hash(p.wkey) & 0xFFFF, n=16 if cfg == 3 else 48)
        host.append((p, canon, xb, rows))
    arr = W.make_proj_array(dev)
    ws = workspace(W.wqd_stack_workspace_bytes(arr, M))
    if mode == W.WQD_PERSISTENT:
        W.wqd_stack_setup(arr, M, ws)
    W.wqd_run_projections(arr, M, mode, ws)
    W.wqd_stream_check()
    worst = 0.0
    for (p, canon, xb, rows), d in zip(host, dev):
        yref, aref = oracle.gemm_f64(p.fmt, p.N, p.K, canon, xb, rows=rows)
        got = d["y"].cpu().numpy()[:, rows]
        worst = max(worst, check_parity(got, yref, aref, f"cfg{cfg} {p.name} M={M}"))
        del canon
    return worst


@pytest.mark.parametrize("cfg,M", [(1, 1), (2, 1), (4, 1), (4, 8), (5, 1), (5, 2), (5, 4), (5, 6), (5, 8), (6, 1), (6, 8)])
def test_config_full_size(cfg, M):
    note(f"config {cfg} M={M} persistent")
    run_config(cfg, M, W.WQD_PERSISTENT)


@pytest.mark.parametrize("cfg,M", [(2, 1), (5, 2), (5, 3)])
def test_config_ordered_mode(cfg, M):
    note(f"config {cfg} M={M} ordered")
    run_config(cfg, M, W.WQD_ORDERED)


@pytest.mark.parametrize("M", [1, 8])
def test_config3_full_stack(M):
    note(f"config 3 full stack M={M} persistent")
    run_config(3, M, W.WQD_PERSISTENT)
