"""kq_matmul_small_m (the batched verify matmul) against the CPU oracle.

Contract per output: |Y[m][r] - Y_ref[m][r]| <= 1e-3 * sum_i |w_ri X_mi|, as for
the matvec.  M = 1 runs the matvec and must equal it bitwise.  Small M (by
default M = 2 for Q4_K; up to 4 when tuned, where the staged rows fit the
LDS) runs the matvec's dot path on every row at once; larger M the
matrix-core kernel with its stream-K split (both are forced below); shapes
below cover row counts
that are not multiples of the 16-row tile or the 256-row group, k from one
superblock up, workgroups whose range holds one tile, several row groups, or
parts of two, and the full FFN shapes on sampled rows.  Every output starts
as NaN, with NaN padding past n_rows inside ldy that must stay untouched.
"""
import numpy as np
import pytest
import torch

import oracle
import quant_weight_matvec_amd as kq
from quant_weight_matvec_amd import inputs as I
from gpu_util import NTHREADS, assert_matvec_close, dev, nan_like, sample_rows, weights

pytestmark = pytest.mark.gpu
O = oracle.get()
QT = {"q4k": kq.KQ_QTYPE_Q4K, "q6k": kq.KQ_QTYPE_Q6K}


def workspace(qt, n, k, m):
    nbytes = kq.kq_matmul_small_m_workspace_bytes(QT[qt], n, k, m)
    ws = torch.zeros(max(nbytes, 256) // 4, dtype=torch.int32, device="cuda")
    return ws, nbytes


def run(qt, Wd, Xd, ldx, n, k, m, ldy=None, ws=None):
    ldy = n + 3 if ldy is None else ldy
    Y = nan_like((m, ldy))
    if ws is None:
        ws = workspace(qt, n, k, m)
    kq.kq_matmul_small_m(QT[qt], Wd, Xd, ldx, Y, ldy, n, k, m, ws[0], ws[1])
    torch.cuda.synchronize()
    Yg = Y.cpu().numpy().astype(np.float64)
    assert np.all(np.isnan(Yg[:, n:])), "wrote past n_rows inside the ldy padding"
    return Yg[:, :n]


def check(qt, n, k, m, seed, rows=None, xscale=None, ldx=None):
    W = weights(qt, n, k, seed)
    ldx = k if ldx is None else ldx
    X = np.zeros((m, ldx), np.float32)
    X[:, :k] = I.normal_f32((m, k), stream=seed + 1)
    if xscale is not None:
        X[:, :k] *= np.asarray(xscale, np.float32).reshape(-1, 1)
    Yg = run(qt, dev(W), dev(X), ldx, n, k, m)
    # every output written, also outside the sampled rows (a partial tile of
    # the stream-K split that never arrives would leave its rows NaN)
    assert np.all(np.isfinite(Yg)), f"{qt} {n}x{k} m={m}: non-finite outputs"
    rows = np.arange(n) if rows is None else rows
    Yr, S = O.matmul(qt, np.ascontiguousarray(W[rows]), X[:, :k], len(rows), k, nthreads=NTHREADS)
    worst = 0.0
    for i in range(m):
        worst = max(worst, assert_matvec_close(Yg[i, rows], Yr[i], S[i], what=f"{qt} {n}x{k} m={m} row {i}"))
    return worst


@pytest.mark.parametrize("qt", ["q4k", "q6k"])
@pytest.mark.parametrize("m", [2, 3, 4, 7, 8, 9, 13, 16])
def test_small_shapes_all_rows(qt, m):
    """Several row groups with a ragged last group, k of 11 superblocks."""
    print("worst |dy|/S", check(qt, 300, 2816, m, 7000 + m))


@pytest.mark.parametrize("qt,n,k", [("q4k", 1, 256), ("q6k", 1, 256), ("q4k", 5, 512),
                                    ("q6k", 17, 1280), ("q4k", 129, 768), ("q6k", 255, 2304),
                                    ("q4k", 1000, 6656), ("q6k", 77, 19968), ("q4k", 4100, 1024),
                                    ("q6k", 2049, 4096), ("q4k", 257, 2816), ("q6k", 513, 1536),
                                    ("q4k", 40, kq.KQ_MAX_K), ("q6k", 40, kq.KQ_MAX_K)])
def test_ragged_shapes(qt, n, k):
    print("worst |dy|/S", check(qt, n, k, 5, 7100 + n, rows=sample_rows(n, 160, seed=n)))


@pytest.mark.parametrize("qt,n,k", [("q4k", 19968, 6656), ("q6k", 6656, 19968)])
@pytest.mark.parametrize("m", [2, 4, 8, 16])
def test_full_size_sampled_rows(qt, n, k, m):
    """The verify shapes at M = 2..16 in the benchmark's launch configuration."""
    print("worst |dy|/S", check(qt, n, k, m, 7200 + m, rows=sample_rows(n, 96, seed=m)))


@pytest.mark.parametrize("qt", ["q4k", "q6k"])
def test_m1_is_the_matvec(qt):
    n, k = 1000, 6656
    W, x = weights(qt, n, k, 7300), I.normal_f32(k, stream=7301)
    Wd, xd = dev(W), dev(x)
    Yg = run(qt, Wd, xd, k, n, k, 1)
    y = nan_like(n)
    (kq.kq_matvec_q4k if qt == "q4k" else kq.kq_matvec_q6k)(Wd, xd, y, n, k)
    torch.cuda.synchronize()
    assert np.array_equal(Yg[0], y.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("qt", ["q4k", "q6k"])
def test_rows_are_independent_of_m(qt):
    """Row m of the result does not depend on the other activation rows:
    M = 16 and M = 3 agree bitwise on the first three rows (same launch plan
    up to LDS chunking, same per-row arithmetic)."""
    n, k = 700, 4096
    W, X = weights(qt, n, k, 7400), I.normal_f32((16, k), stream=7401)
    Wd, Xd = dev(W), dev(X)
    a = run(qt, Wd, Xd, k, n, k, 16)
    b = run(qt, Wd, Xd, k, n, k, 3)
    Yr, S = O.matmul(qt, W, X[:3], n, k, nthreads=NTHREADS)
    for i in range(3):
        assert_matvec_close(a[i], Yr[i], S[i], what=f"m=16 row {i}")
        assert_matvec_close(b[i], Yr[i], S[i], what=f"m=3 row {i}")


@pytest.mark.parametrize("qt", ["q4k", "q6k"])
def test_deterministic_and_workspace_reuse(qt):
    n, k, m = 6656, 19968, 8
    if qt == "q4k":
        n, k = 19968, 6656
    W, X = weights(qt, n, k, 7500), I.normal_f32((m, k), stream=7501)
    Wd, Xd = dev(W), dev(X)
    ws = workspace(qt, n, k, m)
    assert ws[1] > 0, "this shape splits row groups between workgroups"
    a = run(qt, Wd, Xd, k, n, k, m, ws=ws)
    assert not np.any(np.isnan(a))
    # Every call pre-fills Y with NaN, so a row group whose arrival counter was
    # left non-zero by the previous call would never be summed and stay NaN.
    for _ in range(2):
        b = run(qt, Wd, Xd, k, n, k, m, ws=ws)
        assert np.array_equal(a, b)


@pytest.mark.parametrize("qt", ["q4k", "q6k"])
def test_dynamic_range_per_row(qt):
    """Activation rows scaled by 1e-30 .. 1e30: each output row stays within
    its own tolerance (the power-of-two prescale is per row and superblock)."""
    n, k, m = 520, 3072, 6
    print("worst |dy|/S", check(qt, n, k, m, 7600, xscale=[1e-30, 1e-12, 1.0, 3e5, 1e18, 1e30]))


@pytest.mark.parametrize("qt", ["q4k", "q6k"])
def test_heavy_tailed_and_mixed_magnitudes(qt):
    """One superblock group spanning 2^-20 .. 2^20 in magnitude."""
    n, k, m = 256, 2048, 4
    W = weights(qt, n, k, 7700)
    rng = np.random.default_rng(7701)
    X = (rng.standard_normal((m, k)) * np.exp2(rng.uniform(-20, 20, (m, k)))).astype(np.float32)
    Yg = run(qt, dev(W), dev(X), k, n, k, m)
    Yr, S = O.matmul(qt, W, X, n, k, nthreads=NTHREADS)
    for i in range(m):
        assert_matvec_close(Yg[i], Yr[i], S[i], what=f"row {i}")


@pytest.mark.parametrize("m", [4, 12])  # the 16-wave and the 8-wave launch shapes
@pytest.mark.parametrize("qt", ["q4k", "q6k"])
def test_nonfinite_activation_poisons_only_its_row(qt, m):
    n, k = 400, 2048
    W = weights(qt, n, k, 7800)
    X = I.normal_f32((m, k), stream=7801)
    X[1, 1500] = np.nan
    X[2, 37] = np.inf
    Yg = run(qt, dev(W), dev(X), k, n, k, m)
    assert np.all(np.isnan(Yg[1])), "NaN input did not propagate"
    assert not np.any(np.isfinite(Yg[2])), "Inf input did not propagate"
    rest = [i for i in range(m) if i not in (1, 2)]
    Yr, S = O.matmul(qt, W, X[rest], n, k, nthreads=NTHREADS)
    for j, i in enumerate(rest):
        assert_matvec_close(Yg[i], Yr[j], S[j], what=f"row {i}")


@pytest.mark.parametrize("qt", ["q4k", "q6k"])
def test_nonfinite_activation_dot_path(qt):
    """The same rule on the dot path (forced; M = 2 of Q4_K takes it by
    default): a NaN or an infinity in an activation row makes that output row
    non-finite (the matvec's staging gives its group a non-finite sum) and
    leaves the other rows as they are."""
    n, k, m = 400, 2048, 4
    W = weights(qt, n, k, 7810)
    X = I.normal_f32((m, k), stream=7811)
    X[1, 1500] = np.nan
    X[2, 37] = -np.inf
    try:
        kq.kq_tune_set_small_m_rows(QT[qt], 4)
        Yg = run(qt, dev(W), dev(X), k, n, k, m)
    finally:
        kq.kq_tune_set_small_m_rows(QT[qt], -1)
    assert np.all(np.isnan(Yg[1])), "NaN input did not propagate"
    assert not np.any(np.isfinite(Yg[2])), "Inf input did not propagate"
    rest = [0, 3]
    Yr, S = O.matmul(qt, W, X[rest], n, k, nthreads=NTHREADS)
    for j, i in enumerate(rest):
        assert_matvec_close(Yg[i], Yr[j], S[j], what=f"row {i}")


@pytest.mark.parametrize("qt", ["q4k", "q6k"])
def test_strided_x_and_y(qt):
    n, k, m = 333, 1536, 7
    print("worst |dy|/S", check(qt, n, k, m, 7900, ldx=k + 260))


def test_zero_activations_give_zero():
    n, k, m = 300, 1024, 5
    for qt in ("q4k", "q6k"):
        W = weights(qt, n, k, 8000)
        Yg = run(qt, dev(W), dev(np.zeros((m, k), np.float32)), k, n, k, m)
        assert np.all(Yg == 0.0)


def test_workspace_errors():
    qt, n, k, m = "q6k", 6656, 19968, 8
    need = kq.kq_matmul_small_m_workspace_bytes(QT[qt], n, k, m)
    assert need > 0
    W, X = dev(weights(qt, n, k, 8100)), dev(I.normal_f32((m, k), stream=8101))
    Y = nan_like((m, n))
    ws = torch.zeros(need // 4, dtype=torch.int32, device="cuda")
    with pytest.raises(kq.KQError):
        kq.kq_matmul_small_m(QT[qt], W, X, k, Y, n, n, k, m, ws, need - 256)
    with pytest.raises(kq.KQError):
        kq.kq_matmul_small_m(QT[qt], W, X, k, Y, n, n, k, m, None, 0)
    with pytest.raises(kq.KQError):  # output inside the workspace
        kq.kq_matmul_small_m(QT[qt], W, X, k, ws, n, n, k, m, ws, need)
    torch.cuda.synchronize()
    assert torch.isnan(Y).all(), "a rejected call wrote its output"


@pytest.mark.parametrize("qt,n,k,ms", [("q4k", 19968, 6656, (2, 3, 4)), ("q6k", 6656, 19968, (2,))])
def test_dot_path_rows_equal_the_matvec(qt, n, k, ms):
    """At the FFN shapes the matvec sums a row over 8 lanes, as the dot path
    does, so each row of the dot path equals the matvec of that activation
    row bit for bit (the same staged encoding and per-row arithmetic).  The
    dot path takes no workspace."""
    W = weights(qt, n, k, 7700)
    X = I.normal_f32((4, k), stream=7701)
    Wd, Xd = dev(W), dev(X)
    mv = kq.kq_matvec_q4k if qt == "q4k" else kq.kq_matvec_q6k
    ref = []
    for i in range(4):
        y = nan_like(n)
        mv(Wd, Xd[i], y, n, k)
        ref.append(y)
    torch.cuda.synchronize()
    ref = [y.cpu().numpy().astype(np.float64) for y in ref]
    try:
        kq.kq_tune_set_small_m_rows(QT[qt], 4)
        assert all(kq.kq_matmul_small_m_workspace_bytes(QT[qt], n, k, m) == 0 for m in ms)
        for m in ms:
            Yg = run(qt, Wd, Xd, k, n, k, m)
            for i in range(m):
                assert np.array_equal(Yg[i], ref[i]), f"{qt} m={m} row {i}"
    finally:
        kq.kq_tune_set_small_m_rows(QT[qt], -1)


@pytest.mark.parametrize("qt", ["q4k", "q6k"])
@pytest.mark.parametrize("m", [2, 3, 4])
def test_both_small_m_paths_forced(qt, m):
    """The dot path and the matrix-core kernel, each forced for the same
    shapes (ragged rows, a k of a few superblocks, the full Q4_K row width,
    a single row of one superblock, 9 rows), meet the oracle's tolerance;
    the noalloc form equals the workspace form on each path."""
    for n, k in ((333, 1280), (4097, 6656), (1, 256), (9, 768)):
        if qt == "q6k" and k == 6656:
            k = 5120
        W, X = weights(qt, n, k, 7800 + m), I.normal_f32((m, k), stream=7810 + m)
        Wd, Xd = dev(W), dev(X)
        Yr, S = O.matmul(qt, W, X, n, k, nthreads=NTHREADS)
        try:
            for max_m in (4, 0):
                kq.kq_tune_set_small_m_rows(QT[qt], max_m)
                Yg = run(qt, Wd, Xd, k, n, k, m)
                for i in range(m):
                    assert_matvec_close(Yg[i], Yr[i], S[i], what=f"{qt} {n}x{k} m={m} path {max_m} row {i}")
                Y2 = nan_like((m, n + 3))
                kq.kq_matmul_small_m_noalloc(QT[qt], Wd, Xd, k, Y2, n + 3, n, k, m)
                torch.cuda.synchronize()
                assert np.array_equal(Y2.cpu().numpy().astype(np.float64)[:, :n], Yg)
        finally:
            kq.kq_tune_set_small_m_rows(QT[qt], -1)
