"""The verify batch through a whole FFN layer (Ch 10 "The forward pass at a
glance", sections 10.2-10.3; Ch 36 "Prefill vs decode", section 36.4: Y = W X
with M activation rows): kq_ffn_gate_up_q4k_small_m (gate, up and the SiLU
product for M rows), kq_matmul_small_m on the product (the Q6_K down
projection) and kq_fused_residual_norm over the M rows, at the full FFN
shapes (hidden 6656, ffn 19968), for M in {1, 2, 3, 4, 8, 16}.

Each row is held to the oracle's FFN layer from the same (x, residual): the
tail's outputs within 2e-3 absolute; mid within the bound derived from the
two matvec tolerances,
  |dmid| <= 1.1 dg (|u| + du) + |silu(g)| du,  dg = 1e-3 S_g, du = 1e-3 S_u
(1.1 bounds the derivative of silu).  M = 1 takes the one-launch gate+up
kernel and must equal kq_ffn_gate_up_q4k bit for bit; so must every row at
the M (2 and 3 by default, up to 4 when tuned) where gate and up run through
the matvec's dot path in one launch.
"""
import numpy as np
import pytest
import torch

import oracle
import quant_weight_matvec_amd as kq
from quant_weight_matvec_amd import inputs as I
from gpu_util import NTHREADS, dev, nan_like

pytestmark = pytest.mark.gpu
O = oracle.get()
HIDDEN, FFN = 6656, 19968
Q4, Q6 = kq.KQ_QTYPE_Q4K, kq.KQ_QTYPE_Q6K


@pytest.fixture(scope="module")
def layer():
    s = lambda role: I.stream_id(3, 0, role)
    host = dict(wg=I.q4k_matrix(FFN, HIDDEN, stream=s(I.ROLE_W_GATE)),
                wu=I.q4k_matrix(FFN, HIDDEN, stream=s(I.ROLE_W_UP)),
                wd=I.q6k_matrix(HIDDEN, FFN, stream=s(I.ROLE_W_DOWN)),
                gp=I.gains_f32(HIDDEN, stream=s(I.ROLE_GPOST)),
                gn=I.gains_f32(HIDDEN, stream=s(I.ROLE_GNEXT)))
    res = I.normal_f32((16, HIDDEN), stream=s(I.ROLE_RESID)).astype(np.float64)
    X = np.stack([O.rms_norm(r, 1e-5) for r in res]).astype(np.float32)
    return dict(host=host, dev={k: dev(v) for k, v in host.items()}, X=X,
                res=res.astype(np.float32))


def workspace(m):
    need = max(kq.kq_matmul_small_m_workspace_bytes(Q4, FFN, HIDDEN, m),
               kq.kq_matmul_small_m_workspace_bytes(Q6, HIDDEN, FFN, m))
    return torch.zeros(max(need, 256) // 4, dtype=torch.int32, device="cuda"), need


@pytest.mark.parametrize("m", [1, 2, 3, 4, 8, 16])
def test_verify_layer_per_row(layer, m):
    d, h = layer["dev"], layer["host"]
    X, res = layer["X"][:m], layer["res"][:m]
    ws, nb = workspace(m)
    Xd = dev(X)
    mid = nan_like((m, FFN))
    p = nan_like((m, HIDDEN))
    r = dev(res)
    nxt = nan_like((m, HIDDEN))
    kq.kq_ffn_gate_up_q4k_small_m(d["wg"], d["wu"], Xd, HIDDEN, mid, FFN, FFN, HIDDEN, m, ws, nb)
    kq.kq_matmul_small_m(Q6, d["wd"], mid, FFN, p, HIDDEN, HIDDEN, FFN, m, ws, nb)
    kq.kq_fused_residual_norm(r, p, nxt, d["gp"], d["gn"], m, HIDDEN)
    torch.cuda.synchronize()
    mid_g = mid.cpu().numpy().astype(np.float64)
    r_g, n_g = r.cpu().numpy().astype(np.float64), nxt.cpu().numpy().astype(np.float64)
    worst = 0.0
    for i in range(m):
        L = O.ffn_layer(h["wg"], h["wu"], h["wd"], HIDDEN, FFN, X[i], res[i], h["gp"], h["gn"],
                        nthreads=NTHREADS)
        dg, du = 1e-3 * L["s_g"], 1e-3 * L["s_u"]
        sil = np.abs(L["g"] / (1.0 + np.exp(-L["g"])))
        bound = 1.1 * dg * (np.abs(L["u"]) + du) + sil * du
        assert np.all(np.abs(mid_g[i] - L["mid"]) <= bound), f"m={m} row {i}: mid"
        dr = np.max(np.abs(r_g[i] - L["residual"]))
        dn = np.max(np.abs(n_g[i] - L["next_in"]))
        worst = max(worst, dr, dn)
        assert dr <= 2e-3 and dn <= 2e-3, f"m={m} row {i}: tail outputs {dr:.2e} {dn:.2e}"
    print(f"m={m}: worst tail difference {worst:.2e}")


def test_verify_gate_up_m1_is_the_one_launch_kernel(layer):
    d = layer["dev"]
    x = dev(layer["X"][0])
    a, b = nan_like(FFN), nan_like(FFN)
    kq.kq_ffn_gate_up_q4k_small_m(d["wg"], d["wu"], x, HIDDEN, a, FFN, FFN, HIDDEN, 1)
    kq.kq_ffn_gate_up_q4k(d["wg"], d["wu"], x, b, FFN, HIDDEN)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_verify_gate_up_rows_independent_of_m(layer):
    """Row 1 of an M = 16 batch equals row 1 of an M = 9 batch bit for bit (the
    grid and split depend on M only through the launch shape class, M <= 8 or
    M > 8, and both of these are M > 8)."""
    d = layer["dev"]
    outs = []
    for m in (16, 9):
        ws, nb = workspace(m)
        mid = nan_like((m, FFN))
        kq.kq_ffn_gate_up_q4k_small_m(d["wg"], d["wu"], dev(layer["X"][:m]), HIDDEN, mid, FFN, FFN,
                                      HIDDEN, m, ws, nb)
        torch.cuda.synchronize()
        outs.append(mid.cpu().numpy())
    assert np.all(np.isfinite(outs[0])) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("m", [2, 3, 4])
def test_verify_gate_up_dot_path_rows_equal_the_one_launch_kernel(layer, m):
    """The fused dot path (forced up to M = 4) gives, row by row, the bits of
    kq_ffn_gate_up_q4k on that activation row, needs no workspace, and
    leaves the padding past n_rows inside ldm untouched."""
    d = layer["dev"]
    ref = []
    for i in range(m):
        y = nan_like(FFN)
        kq.kq_ffn_gate_up_q4k(d["wg"], d["wu"], dev(layer["X"][i]), y, FFN, HIDDEN)
        ref.append(y)
    try:
        kq.kq_tune_set_gate_up_rows(4)
        mid = nan_like((m, FFN + 5))
        kq.kq_ffn_gate_up_q4k_small_m(d["wg"], d["wu"], dev(layer["X"][:m]), HIDDEN, mid, FFN + 5,
                                      FFN, HIDDEN, m)
        torch.cuda.synchronize()
    finally:
        kq.kq_tune_set_gate_up_rows(-1)
    assert torch.isnan(mid[:, FFN:]).all(), "wrote past n_rows inside ldm"
    for i in range(m):
        assert torch.equal(mid[i, :FFN], ref[i]), f"m={m} row {i}"


@pytest.mark.parametrize("n,k", [(333, 1280), (4100, 2816), (8, 256)])
def test_verify_gate_up_dot_path_ragged(n, k):
    """Ragged row counts (not a multiple of the 8-row task or of the grid),
    a k of one superblock, strided X: each row of the fused dot path equals
    the one-launch kernel on that row bit for bit (that kernel is held to
    the oracle in the parity tests)."""
    Wg = I.q4k_matrix(n, k, stream=7900 + n)
    Wu = I.q4k_matrix(n, k, stream=7901 + n)
    ldx = k + 8
    X = np.zeros((4, ldx), np.float32)
    X[:, :k] = I.normal_f32((4, k), stream=7902 + n)
    wg, wu, Xd = dev(Wg), dev(Wu), dev(X)
    ref = []
    for i in range(4):
        y = nan_like(n)
        kq.kq_ffn_gate_up_q4k(wg, wu, dev(np.ascontiguousarray(X[i, :k])), y, n, k)
        ref.append(y)
    try:
        kq.kq_tune_set_gate_up_rows(4)
        for m in (2, 3, 4):
            mid = nan_like((m, n + 3))
            kq.kq_ffn_gate_up_q4k_small_m(wg, wu, Xd, ldx, mid, n + 3, n, k, m)
            torch.cuda.synchronize()
            assert torch.isnan(mid[:, n:]).all()
            for i in range(m):
                assert torch.equal(mid[i, :n], ref[i]), f"{n}x{k} m={m} row {i}"
    finally:
        kq.kq_tune_set_gate_up_rows(-1)
