"""Staged activations: the matvecs, the fused gate+up and the tail on inputs
(or with outputs) in the staged form.

The staged form is the encoding every matvec workgroup otherwise applies to
its f32 input in LDS, so the contract is bitwise: a matvec on a staged vector
equals the same matvec on the f32 vector, a producer's staged output equals
kq_stage_activation of its f32 output, and the staged layer pass equals the
f32 pass.  One oracle comparison per entry point checks the path end to end.
"""
import numpy as np
import pytest
import torch

import oracle
import quant_weight_matvec_amd as kq
from quant_weight_matvec_amd import inputs as I
from gpu_util import NTHREADS, assert_matvec_close, dev, nan_like, oracle_rows, sample_rows

pytestmark = pytest.mark.gpu
QT = {"q4k": kq.KQ_QTYPE_Q4K, "q6k": kq.KQ_QTYPE_Q6K}


def staged(qt, x, k):
    xs = torch.full((kq.kq_staged_bytes(QT[qt], k),), 0xA5, dtype=torch.uint8, device="cuda")
    kq.kq_stage_activation(QT[qt], x, xs, k)
    return xs


def payload(xs, k):
    """The bytes of a staged k-vector that carry data: its three limb planes
    hold 144 bytes per 128 inputs (16 of them padding, never written or read),
    then come the scales and sums."""
    planes = xs[: 3 * (k + k // 8)].reshape(3, k // 128, 144)[:, :, :128]
    return torch.cat([planes.reshape(-1), xs[3 * (k + k // 8):]])


def plain(qt, W, x, n, k, gate=None):
    y = nan_like(n)
    if qt == "q4k":
        kq.kq_matvec_q4k(W, x, y, n, k, gate)
    else:
        kq.kq_matvec_q6k(W, x, y, n, k)
    return y


@pytest.mark.parametrize("qt,n,k", [("q4k", 1, 256), ("q4k", 77, 1024), ("q4k", 1000, 6656),
                                    ("q6k", 3, 256), ("q6k", 129, 2560), ("q6k", 700, 19968),
                                    ("q4k", 6656, 19968), ("q4k", 33, kq.KQ_MAX_K),
                                    ("q6k", 33, kq.KQ_MAX_K)])
def test_staged_matvec_equals_f32(qt, n, k):
    W = dev(I.weight_matrix(qt, n, k, stream=41))
    x = dev(I.normal_f32(k, stream=42))
    xs = staged(qt, x, k)
    y0 = plain(qt, W, x, n, k)
    y1 = nan_like(n)
    kq.kq_matvec_staged(QT[qt], W, xs, y1, n, k)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_staged_matvec_silu_and_oracle():
    n, k = 19968, 6656
    Wh = I.weight_matrix("q4k", n, k, stream=43)
    W, x = dev(Wh), dev(I.normal_f32(k, stream=44))
    g = dev(I.normal_f32(n, stream=45))
    xs = staged("q4k", x, k)
    y0 = plain("q4k", W, x, n, k, g)
    y1 = nan_like(n)
    kq.kq_matvec_staged(QT["q4k"], W, xs, y1, n, k, g)
    yp = nan_like(n)
    kq.kq_matvec_staged(QT["q4k"], W, xs, yp, n, k)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    rows = sample_rows(n, 64)
    yr, S = oracle_rows("q4k", Wh, x.cpu().numpy(), rows, k)
    assert_matvec_close(yp.cpu().numpy()[rows], yr, S, what="staged q4k vs oracle")


@pytest.mark.parametrize("n,k,mq", [(19968, 6656, "q6k"), (512, 1024, "q4k"), (768, 2560, "q6k")])
def test_gate_up_staged(n, k, mq):
    Wg = dev(I.q4k_matrix(n, k, stream=46))
    Wu = dev(I.q4k_matrix(n, k, stream=47))
    x = dev(I.normal_f32(k, stream=48))
    xs = staged("q4k", x, k)
    m0, m1 = nan_like(n), nan_like(n)
    kq.kq_ffn_gate_up_q4k(Wg, Wu, x, m0, n, k)
    ms = torch.full((kq.kq_staged_bytes(QT[mq], n),), 0x5A, dtype=torch.uint8, device="cuda")
    kq.kq_ffn_gate_up_q4k_staged(Wg, Wu, xs, m1, ms, QT[mq], n, k)
    m2 = nan_like(n)
    kq.kq_ffn_gate_up_q4k_staged(Wg, Wu, xs, m2, None, 0, n, k)  # no staged output
    torch.cuda.synchronize()
    assert torch.equal(m0, m1) and torch.equal(m0, m2)
    assert torch.equal(payload(ms, n), payload(staged(mq, m0, n), n))


@pytest.mark.parametrize("rows,n,nq", [(1, 6656, "q4k"), (2, 1024, "q6k"), (1, 16384, "q4k"),
                                       (3, 256, "q4k")])
def test_tail_staged(rows, n, nq):
    res = I.normal_f32(rows * n, stream=49)
    proj = I.normal_f32(rows * n, stream=50)
    gp, gn = dev(I.gains_f32(n, stream=51)), dev(I.gains_f32(n, stream=52))
    r0, r1 = dev(res), dev(res)
    o0, o1 = nan_like(rows * n), nan_like(rows * n)
    p = dev(proj)
    sb = kq.kq_staged_bytes(QT[nq], n)
    xs = torch.full((rows * sb,), 0x3C, dtype=torch.uint8, device="cuda")
    kq.kq_fused_residual_norm(r0, p, o0, gp, gn, rows, n)
    kq.kq_fused_residual_norm_staged(r1, p, o1, xs, QT[nq], gp, gn, rows, n)
    torch.cuda.synchronize()
    assert torch.equal(r0, r1) and torch.equal(o0, o1)
    for r in range(rows):
        assert torch.equal(payload(xs[r * sb:(r + 1) * sb], n),
                           payload(staged(nq, o0[r * n:(r + 1) * n], n), n)), r
    # the f32 outputs against the oracle's tail
    ref_r, ref_o = oracle.get().dual_eps_tail(res.reshape(rows, n), proj.reshape(rows, n),
                                              gp.cpu().numpy(), gn.cpu().numpy())
    assert np.max(np.abs(r1.cpu().numpy() - ref_r.ravel())) <= 2e-3
    assert np.max(np.abs(o1.cpu().numpy() - ref_o.ravel())) <= 2e-3


@pytest.mark.parametrize("n,k,mq,with_x", [(19968, 6656, "q6k", False), (512, 1024, "q4k", True),
                                          (768, 256, "q6k", True), (256, 8192, "q6k", False)])
def test_tail_gate_up_fused(n, k, mq, with_x):
    """kq_ffn_tail_gate_up_q4k equals kq_fused_residual_norm followed by
    kq_ffn_gate_up_q4k, bit for bit (residual, next_in, mid, staged mid)."""
    Wg = dev(I.q4k_matrix(n, k, stream=53))
    Wu = dev(I.q4k_matrix(n, k, stream=54))
    res = dev(I.normal_f32(k, stream=55))
    p = dev(I.normal_f32(k, stream=56) * 3.0)
    gp, gn = dev(I.gains_f32(k, stream=57)), dev(I.gains_f32(k, stream=58))
    # reference: the two separate launches
    r_ref, x_ref, m_ref = res.clone(), nan_like(k), nan_like(n)
    kq.kq_fused_residual_norm(r_ref, p, x_ref, gp, gn, 1, k)
    kq.kq_ffn_gate_up_q4k(Wg, Wu, x_ref, m_ref, n, k)
    ms_ref = staged(mq, m_ref, n)
    # fused
    r_out, m = nan_like(k), nan_like(n)
    x_out = nan_like(k) if with_x else None
    ms = torch.full((kq.kq_staged_bytes(QT[mq], n),), 0x77, dtype=torch.uint8, device="cuda")
    kq.kq_ffn_tail_gate_up_q4k(res, p, gp, gn, r_out, x_out, Wg, Wu, m, ms, QT[mq], n, k)
    torch.cuda.synchronize()
    assert torch.equal(r_out, r_ref) and torch.equal(m, m_ref)
    assert torch.equal(payload(ms, n), payload(ms_ref, n))
    if with_x:
        assert torch.equal(x_out, x_ref)


@pytest.mark.parametrize("qt,k", [("q4k", 256), ("q4k", 6656), ("q6k", 1024), ("q6k", 19968)])
def test_staged_form_decodes_to_x(qt, k):
    """The stored form itself: per scale group a back-scale 2^(e-22) with
    max|x| < 2^e, each input the integer round(x 2^(22-e)) as three balanced
    signed byte limbs in padded planes, and the f32 group sum of x."""
    G = 32 if qt == "q4k" else 16
    x = I.normal_f32(k, stream=59) * np.float32(3.0)
    x[:G] = 0.0                      # an all-zero group
    x[G:2 * G] *= np.float32(1e-30)  # a tiny group
    x[2 * G] = np.float32(2.0 ** 20)  # a group with one large value
    xs = staged(qt, dev(x), k).cpu().numpy()
    P = k + k // 8
    limbs = xs[: 3 * P].reshape(3, k // 128, 144)[:, :, :128].reshape(3, k).view(np.int8)
    q = (limbs[0].astype(np.int64) << 16) + (limbs[1].astype(np.int64) << 8) + limbs[2]
    tables = xs[3 * P:].view(np.float32)
    assert tables.size == 2 * (k // G)
    scale, gsum = tables[: k // G].astype(np.float64), tables[k // G:].astype(np.float64)
    xg = x.astype(np.float64).reshape(-1, G)
    qg = q.reshape(-1, G)
    mx = np.abs(xg).max(axis=1)
    e = np.where(mx > 0, np.floor(np.log2(np.where(mx > 0, mx, 1.0))) + 1, 0)  # max|x| < 2^e
    assert np.array_equal(scale, np.exp2(e - 22))
    assert np.all(np.abs(qg) <= 2 ** 22)
    assert np.all(np.abs(xg - qg * scale[:, None]) <= 0.5 * scale[:, None])
    # an f32 sum of G terms: within G * 2^-24 of sum |x|
    assert np.all(np.abs(gsum - xg.sum(axis=1)) <= G * 2.0 ** -24 * np.abs(xg).sum(axis=1))
