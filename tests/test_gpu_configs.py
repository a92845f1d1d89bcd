"""Parity at the workloads' full sizes, in the launch configuration the bench times.

Every output row of every projection is compared with the oracle, which runs on all host threads
(rows cut into one range per thread).  The stack runs in WQD_PERSISTENT mode (the bench's headline)
and in WQD_ORDERED mode.
"""
import numpy as np
import pytest

import oracle
from weight_quantized_decode_amd import _lib as W
from weight_quantized_decode_amd import inputs as I

from gpu_util import check_parity, new_y, note, oracle_gemm_all, upload_weight, upload_x, workspace

pytestmark = pytest.mark.gpu


def run_config(cfg, M, mode, layers=None):
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
        host.append((p, canon, xb))
    arr = W.make_proj_array(dev)
    ws = workspace(W.wqd_stack_workspace_bytes(arr, M))
    if mode & 3 == W.WQD_PERSISTENT:
        W.wqd_stack_setup(arr, M, ws, mode=mode)
    W.wqd_run_projections(arr, M, mode, ws)
    W.wqd_stream_check()
    worst = 0.0
    for (p, canon, xb), d in zip(host, dev):
        yref, aref = oracle_gemm_all(p.fmt, p.N, p.K, canon, xb)
        worst = max(worst, check_parity(d["y"].cpu().numpy(), yref, aref, f"cfg{cfg} {p.name} M={M}"))
    return worst


@pytest.mark.parametrize("cfg,M", [(1, 1), (2, 1), (4, 1), (4, 8)] + [(5, m) for m in range(1, 9)] + [(6, 1), (6, 8)])
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
