"""wqd_stack_setup on the stream, and the check of a stale descriptor table.

* Setup enqueues kernels only: it may be captured in a graph with the calls that use it, and the
  graph's replays give the eager results (replayed several times, with eager work between).
* A WQD_PERSISTENT call on a list that no longer matches the workspace's table (an output pointer
  changed, setup not repeated) writes no output, and wqd_stream_check reports WQD_ESTALE once;
  setup again, and the call is right.
"""
import numpy as np
import pytest

from weight_quantized_decode_amd import _lib as W
from weight_quantized_decode_amd import inputs as I

from gpu_util import check_parity, new_y, note, oracle_gemm_all, upload_weight, upload_x, workspace

pytestmark = pytest.mark.gpu

ENTRIES = [(I.CB4, 512, 1024), (I.CB4, 256, 1024), (I.AQ2X8, 384, 2048), (I.TQ2, 200, 1024)]


def _list(M, key):
    dev, host = [], []
    for i, (fmt, N, K) in enumerate(ENTRIES):
        canon = I.gen_weight(fmt, N, K, (key, i))
        xb = I.gen_x(M, K, (key, i))
        dev.append(dict(w=upload_weight(fmt, N, K, canon), x=upload_x(xb), y=new_y(M, N)))
        host.append((fmt, N, K, canon, xb))
    return dev, host


def _check(dev, host, what):
    for d, (fmt, N, K, canon, xb) in zip(dev, host):
        yref, aref = oracle_gemm_all(fmt, N, K, canon, xb)
        check_parity(d["y"].cpu().numpy(), yref, aref, f"{what} fmt={fmt} N={N} K={K}")


@pytest.mark.parametrize("M", [1, 3])
def test_stale_table_is_reported_and_writes_nothing(M):
    note(f"stale table M={M}")
    dev, host = _list(M, 81)
    arr = W.make_proj_array(dev)
    ws = workspace(W.wqd_stack_workspace_bytes(arr, M))
    W.wqd_stack_setup(arr, M, ws)
    W.wqd_run_projections(arr, M, W.WQD_PERSISTENT, ws)
    W.wqd_stream_check()
    _check(dev, host, "first call")
    # a new output for entry 0 without a new setup: the table still names the old one
    old_y = dev[0]["y"]
    dev[0]["y"] = new_y(M, ENTRIES[0][1])
    for d in dev:
        d["y"].fill_(float("nan"))
    old_y.fill_(float("nan"))
    stale = W.make_proj_array(dev)
    W.wqd_run_projections(stale, M, W.WQD_PERSISTENT, ws)
    with pytest.raises(W.WqdError) as err:
        W.wqd_stream_check()
    assert err.value.status == W.WQD_ESTALE
    W.wqd_stream_check()  # reported once
    for t in [old_y] + [d["y"] for d in dev]:
        assert bool(t.isnan().all()), "a stale call wrote output"
    # set up again: right results in the new output
    W.wqd_stack_setup(stale, M, ws)
    W.wqd_run_projections(stale, M, W.WQD_PERSISTENT, ws)
    W.wqd_stream_check()
    _check(dev, host, "after setup again")
    assert bool(old_y.isnan().all())


def test_mode_change_needs_setup():
    note("stale table: batch-invariant flag added without setup")
    M = 2
    dev, host = _list(M, 82)
    arr = W.make_proj_array(dev)
    ws = workspace(W.wqd_stack_workspace_bytes(arr, M))
    W.wqd_stack_setup(arr, M, ws)
    for d in dev:
        d["y"].fill_(float("nan"))
    W.wqd_run_projections(arr, M, W.WQD_PERSISTENT | W.WQD_BATCH_INVARIANT, ws)
    with pytest.raises(W.WqdError) as err:
        W.wqd_stream_check()
    assert err.value.status == W.WQD_ESTALE
    assert all(bool(d["y"].isnan().all()) for d in dev)
    W.wqd_stack_setup(arr, M, ws, mode=W.WQD_PERSISTENT | W.WQD_BATCH_INVARIANT)
    W.wqd_run_projections(arr, M, W.WQD_PERSISTENT | W.WQD_BATCH_INVARIANT, ws)
    W.wqd_stream_check()
    _check(dev, host, "batch-invariant after setup")


def test_setup_and_run_captured_in_a_graph():
    import torch
    note("setup + run in a graph")
    M = 1
    dev, host = _list(M, 83)
    arr = W.make_proj_array(dev)
    ws = workspace(W.wqd_stack_workspace_bytes(arr, M))
    # eager reference (also looks up the per-device flag before any capture)
    W.wqd_stack_setup(arr, M, ws)
    W.wqd_run_projections(arr, M, W.WQD_PERSISTENT, ws)
    W.wqd_stream_check()
    _check(dev, host, "eager")
    ref = [d["y"].clone() for d in dev]
    ws.zero_()  # the graph's own setup must write the tables and counters again
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            W.wqd_stack_setup(arr, M, ws)
            W.wqd_run_projections(arr, M, W.WQD_PERSISTENT, ws)
    for rep in range(3):
        for d in dev:
            d["y"].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        W.wqd_stream_check()
        for d, r in zip(dev, ref):
            assert torch.equal(d["y"].view(torch.int32), r.view(torch.int32)), f"replay {rep}"
        # eager work between replays on the same workspace
        W.wqd_run_projections(arr, M, W.WQD_PERSISTENT, ws)
        W.wqd_stream_check()
        for d, r in zip(dev, ref):
            assert torch.equal(d["y"].view(torch.int32), r.view(torch.int32)), f"eager after replay {rep}"
    del g
