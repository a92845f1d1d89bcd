"""wqd_gemm_noalloc (no workspace argument: the library's per-GPU scratch array) against wqd_gemm
on a caller workspace, through the C ABI: two calls in a row, the second on a smaller input, for
every format.  The kernels and the K-split plan are the same, so the outputs must be the same bits;
both must also meet the oracle's bound."""
import numpy as np
import pytest

import oracle
from weight_quantized_decode_amd import _lib as W
from weight_quantized_decode_amd import inputs as I

from gpu_util import check_parity, new_y, note, upload_weight, upload_x, workspace

pytestmark = pytest.mark.gpu

FMTS = [I.Q4_0, I.CB4, I.CB8, I.TQ2, I.AQ2X8, I.AQ1X16]
# (N, K, M): both calls split K (both use the scratch); the second is smaller
CALLS = [(4096, 11008, 3), (1000, 11008, 1)]


@pytest.mark.parametrize("fmt", FMTS)
def test_noalloc_matches_gemm_two_calls(fmt):
    for i, (N, K, M) in enumerate(CALLS):
        note(f"noalloc fmt={fmt} call {i} N={N} K={K} M={M}")
        canon = I.gen_weight(fmt, N, K, (40, fmt, i))
        x = I.gen_x(M, K, (40, fmt, i))
        w = upload_weight(fmt, N, K, canon)
        assert 0 < W.wqd_workspace_bytes(w, M) <= W.WQD_NOALLOC_MAX_BYTES
        xd = upload_x(x)
        y_ref = new_y(M, N)
        W.wqd_gemm(w, xd, y_ref, workspace(W.wqd_workspace_bytes(w, M)))
        y = new_y(M, N)
        W.wqd_gemm_noalloc(w, xd, y)
        W.wqd_stream_check()
        a, b = y.cpu().numpy(), y_ref.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"fmt={fmt} call {i}"
        yo, ao = oracle.gemm_f64(fmt, N, K, canon, x)
        check_parity(a, yo, ao, f"noalloc fmt={fmt} call {i}")

