"""kq_matmul_small_m_noalloc (the library-owned scratch instead of a caller
workspace) against kq_matmul_small_m with a workspace, through the C ABI.

Two calls in a row on one stream, the second with a smaller input (and a
third smaller still that needs no split), each compared bit for bit with the
workspace entry point on the same inputs (same kernels, same grid), and on
sampled rows with the CPU oracle at the matvec tolerance.  The first call
splits row groups over workgroups, so it goes through the scratch's counters
and partial tiles; the second reuses them and must find the counters at zero.
"""
import numpy as np
import pytest
import torch

import oracle
import quant_weight_matvec_amd as kq
from quant_weight_matvec_amd import inputs as I
from gpu_util import NTHREADS, assert_matvec_close, dev, nan_like, sample_rows, weights

pytestmark = pytest.mark.gpu
QT = {"q4k": kq.KQ_QTYPE_Q4K, "q6k": kq.KQ_QTYPE_Q6K}

CASES = [("q4k", 19968, 6656, 16), ("q6k", 3000, 4096, 5), ("q4k", 300, 256, 9)]


def _run_both(qt, n, k, m, seed):
    W = weights(qt, n, k, seed)
    X = I.normal_f32((m, k), stream=seed + 1)
    Wd, Xd = dev(W), dev(X)
    need = kq.kq_matmul_small_m_workspace_bytes(QT[qt], n, k, m)
    ws = torch.zeros(max(need, 256) // 4, dtype=torch.int32, device="cuda")
    Ya, Yb = nan_like((m, n)), nan_like((m, n))
    kq.kq_matmul_small_m(QT[qt], Wd, Xd, k, Ya, n, n, k, m, ws, need)
    kq.kq_matmul_small_m_noalloc(QT[qt], Wd, Xd, k, Yb, n, n, k, m)
    torch.cuda.synchronize()
    return W, X, need, Ya.cpu().numpy(), Yb.cpu().numpy()


def test_noalloc_equals_workspace_entry_on_consecutive_calls():
    for i, (qt, n, k, m) in enumerate(CASES):
        print(f"noalloc call {i}: {qt} {n}x{k} m={m}", flush=True)
        W, X, need, ya, yb = _run_both(qt, n, k, m, 9300 + 10 * i)
        assert (need > 0) == (i < 2), "the first two cases split row groups, the last does not"
        assert np.all(np.isfinite(yb)), f"call {i}: non-finite output"
        assert np.array_equal(ya, yb), f"call {i}: differs from the workspace entry point"
        rows = sample_rows(n, 96, seed=i)
        Yr, S = oracle.get().matmul(qt, np.ascontiguousarray(W[rows]), X, len(rows), k,
                                    nthreads=NTHREADS)
        for j in range(m):
            assert_matvec_close(yb[j, rows].astype(np.float64), Yr[j], S[j],
                                what=f"noalloc call {i} row {j}")


def test_noalloc_repeat_is_bitwise_stable():
    """The same split call twice more: the counters the first call left are
    zero, so the results repeat bit for bit."""
    qt, n, k, m = "q6k", 6656, 19968, 8
    W, X = weights(qt, n, k, 9400), I.normal_f32((m, k), stream=9401)
    Wd, Xd = dev(W), dev(X)
    outs = []
    for _ in range(2):
        Y = nan_like((m, n))
        kq.kq_matmul_small_m_noalloc(QT[qt], Wd, Xd, k, Y, n, n, k, m)
        torch.cuda.synchronize()
        outs.append(Y.cpu().numpy())
    assert np.all(np.isfinite(outs[0])) and np.array_equal(outs[0], outs[1])
