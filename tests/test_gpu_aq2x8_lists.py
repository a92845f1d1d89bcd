"""AQ2X8 projection lists longer than the kernels keep as per-workgroup records.

A workgroup's pieces are kept as LDS records when their number is small (the 70B MLP: one piece
of each projection per workgroup); a longer list takes the form that walks the descriptors.  Both
must give the oracle's results: here 70 projections in one persistent launch, so every workgroup
serves at least 70 pieces (more than either kernel's records), half of them split along K (so the
split sums walk the list as well, in rounds of 64 pieces), at M = 1 and 2 (the lookup-table
kernels) and M = 3 (the matrix-core kernel), and the same list in ordered mode.
"""
import numpy as np
import pytest

from weight_quantized_decode_amd import _lib as W
from weight_quantized_decode_amd import inputs as I

from gpu_util import check_parity, new_y, note, oracle_gemm_all, upload_weight, upload_x, workspace

pytestmark = pytest.mark.gpu

SHAPES = [(128, 8192), (100, 1000)] * 35  # split along K / ragged N and K, not split


@pytest.mark.parametrize("M,mode", [(1, W.WQD_PERSISTENT), (2, W.WQD_PERSISTENT), (3, W.WQD_PERSISTENT),
                                    (1, W.WQD_ORDERED)])
def test_long_aq2x8_list(M, mode):
    note(f"aq2x8 list of {len(SHAPES)} M={M} mode={mode}")
    xs = {K: I.gen_x(M, K, (71, K)) for K in {k for _, k in SHAPES}}
    xd = {K: upload_x(x) for K, x in xs.items()}
    dev, host = [], []
    for i, (N, K) in enumerate(SHAPES):
        canon = I.gen_weight(I.AQ2X8, N, K, (71, i))
        dev.append(dict(w=upload_weight(I.AQ2X8, N, K, canon), x=xd[K], y=new_y(M, N)))
        host.append((N, K, canon))
    arr = W.make_proj_array(dev)
    ws = workspace(W.wqd_stack_workspace_bytes(arr, M))
    if mode == W.WQD_PERSISTENT:
        W.wqd_stack_setup(arr, M, ws, mode=mode)
        assert W.wqd_stack_launches(arr, M, mode) == 1
    for rep in range(2):  # the counters are left at zero: a second call gives the same bits
        for d in dev:
            d["y"].fill_(float("nan"))
        W.wqd_run_projections(arr, M, mode, ws)
        W.wqd_stream_check()
        ys = [d["y"].cpu().numpy() for d in dev]
        if rep == 0:
            first = ys
            for i, ((N, K, canon), y) in enumerate(zip(host, ys)):
                yref, aref = oracle_gemm_all(I.AQ2X8, N, K, canon, xs[K])
                check_parity(y, yref, aref, f"aq2x8 list entry {i} N={N} K={K} M={M}")
        else:
            for a, b in zip(first, ys):
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
