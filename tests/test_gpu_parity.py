"""Parity of the HIP path against the CPU oracle on seeded inputs.

Matvec contract: |y_gpu - y| <= 1e-3 * sum_i |w_i x_i| per row.  Tail
contract: 2e-3 absolute on both outputs.  Sizes span several tiles with
ragged tails; full sizes (the launch configuration the benchmark times) are
checked on sampled rows the oracle computes one by one.  Every output buffer
starts as NaN so an unwritten row fails.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import quant_weight_matvec_amd as kq
from quant_weight_matvec_amd import inputs as I
from gpu_util import (NTHREADS, assert_matvec_close, dev, gpu_matvec, nan_like, oracle_rows,
                      sample_rows, weights)

pytestmark = pytest.mark.gpu
O = oracle.get()
HERE = os.path.dirname(os.path.abspath(__file__))


def _full_check(qt, n, k, stream, xscale=1.0, x=None):
    W = weights(qt, n, k, stream)
    if x is None:
        x = I.normal_f32(k, stream=stream + 1) * np.float32(xscale)
    y = gpu_matvec(qt, dev(W), dev(x), n, k)
    yr, S = O.matvec(qt, W, x, n, k, nthreads=NTHREADS)
    return assert_matvec_close(y, yr, S, what=f"{qt} {n}x{k}")


# ---------------------------------------------------------------- matvec
def test_tiny_q4k_512x1024():
    """The tiny Q4_K workload: 512 x 1024, single seed."""
    print("ratio", _full_check("q4k", 512, 1024, I.stream_id(0, 0, I.ROLE_W)))


@pytest.mark.parametrize("n,k", [(1, 256), (3, 512), (17, 1024), (255, 2304), (1000, 6656),
                                 (4097, 768), (129, 19968), (33, kq.KQ_MAX_K)])
def test_q4k_shapes(n, k):
    print("ratio", _full_check("q4k", n, k, 1000 + n))


@pytest.mark.parametrize("qt", ["q6k", "q5k"])
@pytest.mark.parametrize("n,k", [(1, 256), (3, 512), (17, 1280), (255, 2304), (1000, 6656),
                                 (4097, 768), (129, 19968), (33, kq.KQ_MAX_K)])
def test_q6k_q5k_shapes(qt, n, k):
    print("ratio", _full_check(qt, n, k, 2000 + n))


@pytest.mark.parametrize("qt,n,k", [("q4k", 19968, 6656), ("q4k", 6656, 19968),
                                    ("q6k", 6656, 19968)])
def test_full_size_sampled_rows(qt, n, k):
    """Full FFN shapes in the benchmark's launch configuration; 256 sampled
    rows (and the first and last) against the oracle."""
    W = weights(qt, n, k, 3000 + n)
    x = I.normal_f32(k, stream=3001 + n)
    y = gpu_matvec(qt, dev(W), dev(x), n, k)
    assert np.all(np.isfinite(y)), "unwritten rows"
    rows = sample_rows(n, 256)
    yr, S = oracle_rows(qt, W, x, rows, k)
    print("ratio", assert_matvec_close(y[rows], yr, S, what=f"{qt} {n}x{k} sampled"))


def test_deterministic_bits():
    for qt, n, k in (("q4k", 4096, 6656), ("q6k", 1024, 19968)):
        W, x = dev(weights(qt, n, k, 7)), dev(I.normal_f32(k, stream=8))
        a = gpu_matvec(qt, W, x, n, k)
        b = gpu_matvec(qt, W, x, n, k)
        assert np.array_equal(a, b), f"{qt} not bitwise reproducible"


@pytest.mark.parametrize("scale", [1e-30, 1e-3, 1e4, 1e30])
def test_activation_dynamic_range(scale):
    for qt in ("q4k", "q6k"):
        _full_check(qt, 300, 2048, 4000, xscale=scale)


def test_heavy_tailed_activation():
    """SiLU-times-up style inputs: products of normals, wide dynamic range."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(19968) * rng.standard_normal(19968) * 3e3).astype(np.float32)
    x[::97] *= 50.0
    for qt in ("q4k", "q6k"):
        _full_check(qt, 257, 19968, 4100, x=x)


def test_zero_and_nan_activation():
    n, k = 64, 1024
    for qt in ("q4k", "q6k"):
        Wd = dev(weights(qt, n, k, 9))
        y = gpu_matvec(qt, Wd, dev(np.zeros(k, np.float32)), n, k)
        assert np.array_equal(y, np.zeros(n)), f"{qt}: W*0 != 0"
        x = I.normal_f32(k, stream=10)
        x[517] = np.nan
        y = gpu_matvec(qt, Wd, dev(x), n, k)
        assert np.all(np.isnan(y)), f"{qt}: NaN input did not propagate"
        x[517] = np.inf
        y = gpu_matvec(qt, Wd, dev(x), n, k)
        assert not np.any(np.isfinite(y)), f"{qt}: Inf input did not propagate"


@pytest.mark.parametrize("lanes", [4, 8, 16, 32, 64])
@pytest.mark.parametrize("waves,grid", [(1, 0), (4, 7), (16, 1), (8, 300)])
@pytest.mark.parametrize("depth", [1, 2, 3])
def test_every_launch_shape(lanes, waves, grid, depth):
    n = 301
    try:
        for qt, qti, k in (("q4k", kq.KQ_QTYPE_Q4K, 1792), ("q6k", kq.KQ_QTYPE_Q6K, 2816),
                           ("q5k", kq.KQ_QTYPE_Q5K, 1280)):
            kq.kq_tune_set_shape(qti, lanes, waves, grid, depth)
            _full_check(qt, n, k, 5000 + lanes)
    finally:
        kq.kq_tune_set_shape(kq.KQ_QTYPE_Q4K)
        kq.kq_tune_set_shape(kq.KQ_QTYPE_Q6K)
        kq.kq_tune_set_shape(kq.KQ_QTYPE_Q5K)


def test_failed_call_leaves_output_untouched():
    n, k = 32, 1024
    Wd, xd = dev(weights("q4k", n, k, 11)), dev(I.normal_f32(k, stream=12))
    y = nan_like(n)
    with pytest.raises(kq.KQError):
        kq.kq_matvec_q4k(Wd, xd, y, n, 1000)
    with pytest.raises(kq.KQError):
        kq.kq_matvec_q4k(Wd, xd[1:], y, n, k - 256)  # x not 16-byte aligned
    with pytest.raises(kq.KQError):
        kq.kq_matvec_q4k(Wd, xd, y, n, k, y)  # output on the gate
    torch.cuda.synchronize()
    assert torch.isnan(y).all()


# ---------------------------------------------------------------- SiLU epilogue
def test_silu_epilogue_ffn_entry():
    """Gate and up projections 19968 x 6656 sharing one input; the up matvec
    applies silu(gate) in its epilogue.  Tolerance for ffn_mid derived from the
    two matvec bounds: |dmid| <= 1.1 dg (|u| + du) + |silu(g)| du."""
    n, k = 19968, 6656
    Wg = weights("q4k", n, k, I.stream_id(2, 0, I.ROLE_W_GATE))
    Wu = weights("q4k", n, k, I.stream_id(2, 0, I.ROLE_W_UP))
    x = I.normal_f32(k, stream=I.stream_id(2, 0, I.ROLE_X))
    xd = dev(x)
    g = nan_like(n)
    kq.kq_matvec_q4k(dev(Wg), xd, g, n, k)
    mid = nan_like(n)
    kq.kq_matvec_q4k(dev(Wu), xd, mid, n, k, g)
    torch.cuda.synchronize()
    rows = sample_rows(n, 512, seed=9)
    gr, Sg = oracle_rows("q4k", Wg, x, rows, k)
    ur, Su = oracle_rows("q4k", Wu, x, rows, k)
    mr = O.silu_mul(gr, ur)
    dg, du = 1e-3 * Sg, 1e-3 * Su
    with np.errstate(over="ignore"):  # exp(-g) = inf for g << 0: silu(g) -> 0
        sil = np.abs(gr / (1 + np.exp(-gr)))
    bound = 1.1 * dg * (np.abs(ur) + du) + sil * du
    got = mid.cpu().numpy().astype(np.float64)[rows]
    assert np.all(np.abs(got - mr) <= bound), "ffn_mid outside the derived bound"
    assert_matvec_close(g.cpu().numpy()[rows], gr, Sg, what="gate")


# ---------------------------------------------------------------- dual-eps tail
def _gpu_tail(res, proj, gp, gn, eps_post=1e-8, eps_next=1e-5):
    rows, n = res.shape
    r, p = dev(res.astype(np.float32)), dev(proj.astype(np.float32))
    out = nan_like((rows, n))
    kq.kq_fused_residual_norm(r, p, out, dev(gp.astype(np.float32)), dev(gn.astype(np.float32)),
                              rows, n, eps_post, eps_next)
    torch.cuda.synchronize()
    return r.cpu().numpy().astype(np.float64), out.cpu().numpy().astype(np.float64)


def test_tail_worked_example():
    with open(os.path.join(HERE, "golden", "tail_worked_example.json")) as f:
        gold = json.load(f)
    r, out = _gpu_tail(np.array([gold["residual"]]), np.array([gold["projected"]]),
                       np.array(gold["post_weight"]), np.array(gold["next_weight"]),
                       gold["eps_post"], gold["eps_next"])
    assert np.allclose(r[0], gold["residual_after"], atol=1e-6)
    assert np.all(np.abs(out[0] - gold["next_input"]) <= gold["tolerance"])


@pytest.mark.parametrize("rows,n,pscale", [(1, 6656, 1.0), (3, 6656, 250.0), (2, 4, 1.0),
                                           (5, 1028, 1e-3), (1, 32768, 10.0), (16, 6656, 1.0)])
def test_tail_vs_oracle(rows, n, pscale):
    res = I.normal_f32((rows, n), stream=I.stream_id(1, 0, I.ROLE_RESID) + n).astype(np.float64)
    proj = (I.normal_f32((rows, n), stream=77 + n) * pscale).astype(np.float32).astype(np.float64)
    gp = I.gains_f32(n, stream=I.stream_id(1, 0, I.ROLE_GPOST))
    gn = I.gains_f32(n, stream=I.stream_id(1, 0, I.ROLE_GNEXT))
    r_gpu, o_gpu = _gpu_tail(res, proj, gp, gn)
    r_ref, o_ref = O.dual_eps_tail(res, proj, gp, gn)
    assert np.max(np.abs(r_gpu - r_ref)) <= 2e-3
    assert np.max(np.abs(o_gpu - o_ref)) <= 2e-3


def test_down_projection_then_tail():
    """Q6_K down projection 6656 x 19968 followed by the fused tail, against
    the oracle's f64 matvec and tail (both outputs within 2e-3 absolute)."""
    n, k = 6656, 19968
    W = weights("q6k", n, k, I.stream_id(1, 0, I.ROLE_W_DOWN))
    mid = I.normal_f32(k, stream=I.stream_id(1, 0, I.ROLE_X))
    res = I.normal_f32(n, stream=I.stream_id(1, 0, I.ROLE_RESID))
    gp = I.gains_f32(n, stream=I.stream_id(1, 0, I.ROLE_GPOST))
    gn = I.gains_f32(n, stream=I.stream_id(1, 0, I.ROLE_GNEXT))
    p = nan_like(n)
    kq.kq_matvec_q6k(dev(W), dev(mid), p, n, k)
    r, out = dev(res), nan_like(n)
    kq.kq_fused_residual_norm(r, p, out, dev(gp), dev(gn), 1, n)
    torch.cuda.synchronize()
    p_ref, S = O.matvec("q6k", W, mid, n, k, nthreads=NTHREADS)
    assert_matvec_close(p.cpu().numpy(), p_ref, S, what="down")
    r_ref, o_ref = O.dual_eps_tail(res, p_ref, gp, gn)
    dr = np.max(np.abs(r.cpu().numpy() - r_ref))
    do = np.max(np.abs(out.cpu().numpy() - o_ref))
    print(f"tail max |dr| {dr:.3e} |dout| {do:.3e}")
    assert dr <= 2e-3 and do <= 2e-3


# ---------------------------------------------------------------- graph capture
def test_graph_replay_matches_eager():
    """A captured matvec + tail replayed several times, with eager work and
    synchronisations between replays, matches the eager result every time."""
    n, k = 6656, 19968
    Wd = dev(weights("q6k", n, k, 21))
    xd = dev(I.normal_f32(k, stream=22))
    res0 = I.normal_f32(n, stream=23)
    gp, gn = dev(I.gains_f32(n, stream=24)), dev(I.gains_f32(n, stream=25))
    p, r, out = nan_like(n), dev(res0), nan_like(n)

    def step():
        kq.kq_matvec_q6k(Wd, xd, p, n, k)
        kq.kq_fused_residual_norm(r, p, out, gp, gn, 1, n)

    step()
    torch.cuda.synchronize()
    want_r, want_o = r.clone(), out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        r.copy_(dev(res0))
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            step()
    for _ in range(3):
        r.copy_(dev(res0))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(r, want_r) and torch.equal(out, want_o)
        _ = torch.randn(1000, device="cuda").sum().item()  # eager work between replays


# ---------------------------------------------------------------- gate + up in one launch
def _mid_bound(gr, Sg, ur, Su):
    dg, du = 1e-3 * Sg, 1e-3 * Su
    with np.errstate(over="ignore"):  # exp(-g) = inf for g << 0: silu(g) -> 0
        sil = np.abs(gr / (1 + np.exp(-gr)))
    return 1.1 * dg * (np.abs(ur) + du) + sil * du


@pytest.mark.parametrize("n,k", [(1, 256), (5, 512), (129, 768), (1000, 6656), (4100, 1024),
                                 (19968, 6656), (6656, 19968), (48, kq.KQ_MAX_K)])
def test_ffn_gate_up_one_launch(n, k):
    """mid = silu(W_gate x) * (W_up x) from kq_ffn_gate_up_q4k against the
    oracle's gate and up rows (sampled at the large shapes), within the bound
    derived from the two matvec contracts; and equal to the two-launch path
    within the same bound."""
    Wg = weights("q4k", n, k, 9300 + n)
    Wu = weights("q4k", n, k, 9400 + n)
    x = I.normal_f32(k, stream=9500 + n)
    Wgd, Wud, xd = dev(Wg), dev(Wu), dev(x)
    mid = nan_like(n)
    kq.kq_ffn_gate_up_q4k(Wgd, Wud, xd, mid, n, k)
    g2, mid2 = nan_like(n), nan_like(n)
    kq.kq_matvec_q4k(Wgd, xd, g2, n, k)
    kq.kq_matvec_q4k(Wud, xd, mid2, n, k, g2)
    torch.cuda.synchronize()
    got = mid.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)), "unwritten rows"
    rows = sample_rows(n, 384, seed=n)
    gr, Sg = oracle_rows("q4k", Wg, x, rows, k)
    ur, Su = oracle_rows("q4k", Wu, x, rows, k)
    bound = _mid_bound(gr, Sg, ur, Su)
    err = np.abs(got[rows] - O.silu_mul(gr, ur))
    print(f"worst |dmid|/bound {np.max(err / bound):.2e}")
    assert np.all(err <= bound), "mid outside the derived bound"
    two = mid2.cpu().numpy().astype(np.float64)[rows]
    assert np.all(np.abs(got[rows] - two) <= 2 * bound), "one-launch and two-launch paths disagree"
