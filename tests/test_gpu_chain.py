"""The FFN layer stack against the CPU oracle, run as single-op launches (per
layer kq_ffn_gate_up_q4k, the down matvec, kq_fused_residual_norm), with
staged activations, and as the timed pass (each layer's tail fused into the
next layer's gate+up launch), eagerly and as replayed graphs.

Protocol for the 52-layer stack (a reading: the pages fix no parity protocol
for a layer stack):
  (i)  teacher-forced: each layer is run alone on the GPU from the GPU's own
       (x_l, residual_l) and compared with the oracle's layer from the same
       input, at the tail's 2e-3 absolute tolerance;
  (ii) end to end: all layers in one go against the oracle's binary64
       chain from the same start, at the same 2e-3 absolute tolerance (or, if
       the oracle's own sensitivity shows the stack ill-conditioned at that
       level, at that tolerance scaled by the measured amplification), and
       within a few times the end-to-end difference recorded for this
       workload, so that a regression by an order of magnitude fails.
Small shapes also cover workgroups with no rows (fewer scale groups or down
rows than workgroups).
"""
import numpy as np
import pytest
import torch

import oracle
import quant_weight_matvec_amd as kq
from quant_weight_matvec_amd import inputs as I
from gpu_util import NTHREADS, dev

pytestmark = pytest.mark.gpu
O = oracle.get()
QT = {"q4k": kq.KQ_QTYPE_Q4K, "q6k": kq.KQ_QTYPE_Q6K}


class Stack:
    """Seeded weights of a layer stack, on the GPU (and regenerable on the host)."""

    def __init__(self, layers, hidden, ffn, down="q6k", cfg=9):
        self.layers, self.hidden, self.ffn, self.down, self.cfg = layers, hidden, ffn, down, cfg
        self.dev = [dict((k, dev(v)) for k, v in self.host(l).items()) for l in range(layers)]

    def host(self, l):
        s = lambda role: I.stream_id(self.cfg, l, role)
        return dict(wg=I.q4k_matrix(self.ffn, self.hidden, stream=s(I.ROLE_W_GATE)),
                    wu=I.q4k_matrix(self.ffn, self.hidden, stream=s(I.ROLE_W_UP)),
                    wd=I.weight_matrix(self.down, self.hidden, self.ffn, stream=s(I.ROLE_W_DOWN)),
                    gp=I.gains_f32(self.hidden, stream=s(I.ROLE_GPOST)),
                    gn=I.gains_f32(self.hidden, stream=s(I.ROLE_GNEXT)))

    def ops(self, l, x, xn, r, mid, p):
        """Layer l as the three single-op launches (gate+up+SiLU, down, tail)."""
        d = self.dev[l]
        kq.kq_ffn_gate_up_q4k(d["wg"], d["wu"], x, mid, self.ffn, self.hidden)
        if self.down == "q6k":
            kq.kq_matvec_q6k(d["wd"], mid, p, self.hidden, self.ffn)
        else:
            kq.kq_matvec_q4k(d["wd"], mid, p, self.hidden, self.ffn)
        kq.kq_fused_residual_norm(r, p, xn, d["gp"], d["gn"], 1, self.hidden, 1e-8, 1e-5)

    def ops_staged(self, l, xst, x_next, xst_next, r, mid, mid_s, p):
        """Layer l with staged activations: gate+up reads x staged and writes
        mid staged, the down matvec reads it, the tail writes x staged."""
        d = self.dev[l]
        kq.kq_ffn_gate_up_q4k_staged(d["wg"], d["wu"], xst, mid, mid_s, QT[self.down], self.ffn,
                                     self.hidden)
        kq.kq_matvec_staged(QT[self.down], d["wd"], mid_s, p, self.hidden, self.ffn)
        kq.kq_fused_residual_norm_staged(r, p, x_next, xst_next, kq.KQ_QTYPE_Q4K, d["gp"], d["gn"],
                                         1, self.hidden, 1e-8, 1e-5)

    def run_ops(self, x, res, first=0, count=None, replays=0, staged=False):
        """Layers [first, first+count) through the single-op launches (with
        staged activations if `staged`), eagerly; with replays > 0 also
        captured as one graph and replayed that many times from the same
        start, each replay required to equal the eager result bit for bit.
        Returns (x_out, residual)."""
        count = self.layers - first if count is None else count
        x0, r0 = dev(np.asarray(x, np.float32)), dev(np.asarray(res, np.float32))
        xs = [torch.empty(self.hidden, device="cuda") for _ in range(2)]
        r = torch.empty(self.hidden, device="cuda")
        mid, p = torch.empty(self.ffn, device="cuda"), torch.empty(self.hidden, device="cuda")
        sb = kq.kq_staged_bytes(kq.KQ_QTYPE_Q4K, self.hidden)
        xst = [torch.empty(sb, dtype=torch.uint8, device="cuda") for _ in range(2)]
        mid_s = torch.empty(kq.kq_staged_bytes(QT[self.down], self.ffn), dtype=torch.uint8,
                            device="cuda")

        def body():
            if staged:
                kq.kq_stage_activation(kq.KQ_QTYPE_Q4K, xs[0], xst[0], self.hidden)
            for i in range(count):
                if staged:
                    self.ops_staged(first + i, xst[i % 2], xs[(i + 1) % 2], xst[(i + 1) % 2], r,
                                    mid, mid_s, p)
                else:
                    self.ops(first + i, xs[i % 2], xs[(i + 1) % 2], r, mid, p)

        xs[0].copy_(x0); r.copy_(r0)
        body()
        torch.cuda.synchronize()
        out_x, out_r = xs[count % 2].cpu().numpy(), r.cpu().numpy()
        if replays:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                body()
            torch.cuda.synchronize()
            for k in range(replays):
                xs[0].copy_(x0); r.copy_(r0); xs[1].fill_(float("nan"))
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                assert np.array_equal(xs[count % 2].cpu().numpy(), out_x), f"replay {k}: x differs"
                assert np.array_equal(r.cpu().numpy(), out_r), f"replay {k}: residual differs"
        return out_x.astype(np.float64), out_r.astype(np.float64)

    def run_pass(self, res, mode, replays=0):
        """The whole stack from a residual, on the GPU: x_0 by the GPU's own
        entry norm (the tail with a zero projection and unit gains), then
        every layer.  mode "f32": 3 launches per layer on f32 activations;
        "staged": the same with staged activations; "fusedtail": 2 launches
        per layer (each layer's tail fused into the next layer's gate+up
        launch) and a last tail; "libpass": the same launches enqueued by the
        library's kq_ffn_pass_q4k_q6k (Q6_K down only).  With replays > 0 the pass is also replayed
        as a graph, each replay equal to the eager run bit for bit.
        Returns (x_out, residual)."""
        h, f, L = self.hidden, self.ffn, self.layers
        r0 = dev(np.asarray(res, np.float32))
        zeros, ones = torch.zeros(h, device="cuda"), torch.ones(h, device="cuda")
        R = [torch.empty(h, device="cuda") for _ in range(2)]
        X = [torch.empty(h, device="cuda") for _ in range(2)]
        sb = kq.kq_staged_bytes(kq.KQ_QTYPE_Q4K, h)
        XS = [torch.empty(sb, dtype=torch.uint8, device="cuda") for _ in range(2)]
        mid, p = torch.empty(f, device="cuda"), torch.empty(h, device="cuda")
        mid_s = torch.empty(kq.kq_staged_bytes(QT[self.down], f), dtype=torch.uint8, device="cuda")
        D = self.dev

        def body():
            if mode == "fusedtail":
                for l in range(L):
                    pp, gp, gn = (zeros, ones, ones) if l == 0 else (p, D[l - 1]["gp"], D[l - 1]["gn"])
                    kq.kq_ffn_tail_gate_up_q4k(R[l % 2], pp, gp, gn, R[(l + 1) % 2], None,
                                               D[l]["wg"], D[l]["wu"], mid, mid_s, QT[self.down], f, h)
                    kq.kq_matvec_staged(QT[self.down], D[l]["wd"], mid_s, p, h, f)
                kq.kq_fused_residual_norm(R[L % 2], p, X[0], D[L - 1]["gp"], D[L - 1]["gn"], 1, h)
            elif mode == "staged":
                kq.kq_fused_residual_norm_staged(R[0], zeros, X[0], XS[0], kq.KQ_QTYPE_Q4K, ones,
                                                 ones, 1, h)
                for l in range(L):
                    self.ops_staged(l, XS[l % 2], X[(l + 1) % 2], XS[(l + 1) % 2], R[0], mid, mid_s, p)
            else:
                kq.kq_fused_residual_norm(R[0], zeros, X[0], ones, ones, 1, h)
                for l in range(L):
                    self.ops(l, X[l % 2], X[(l + 1) % 2], R[0], mid, p)

        if mode == "libpass":
            wsb = kq.kq_ffn_pass_workspace_bytes(h, f)
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            table = kq.kq_ffn_layer_table([(d["wg"], d["wu"], d["wd"], d["gp"], d["gn"]) for d in D])

            def body():  # noqa: F811
                kq.kq_ffn_pass_q4k_q6k(table, R[0], X[0], None, ws, wsb, h, f)

        out = lambda: ((X[0], R[L % 2]) if mode == "fusedtail" else
                       (X[0], R[0]) if mode == "libpass" else (X[L % 2], R[0]))
        R[0].copy_(r0)
        body()
        torch.cuda.synchronize()
        xo, ro = (t.cpu().numpy() for t in out())
        if replays:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                body()
            torch.cuda.synchronize()
            for k in range(replays):
                R[0].copy_(r0); R[1].fill_(float("nan")); X[0].fill_(float("nan")); X[1].fill_(float("nan"))
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                xa, ra = (t.cpu().numpy() for t in out())
                assert np.array_equal(xa, xo) and np.array_equal(ra, ro), f"replay {k} differs"
        return xo.astype(np.float64), ro.astype(np.float64)

    def oracle_layer(self, l, x, res):
        h = self.host(l)
        L = O.ffn_layer(h["wg"], h["wu"], h["wd"], self.hidden, self.ffn, x, res, h["gp"],
                        h["gn"], qt_down=self.down, nthreads=NTHREADS)
        return L["next_in"], L["residual"]


def start_state(hidden, cfg=9):
    res = I.normal_f32(hidden, stream=I.stream_id(cfg, 0, I.ROLE_RESID)).astype(np.float64)
    x = O.rms_norm(res, 1e-5)  # weightless entry norm, eps 1e-5
    return x.astype(np.float32), res.astype(np.float32)


@pytest.mark.parametrize("layers,hidden,ffn,down", [(1, 512, 1536, "q6k"), (4, 512, 1536, "q6k"),
                                                    (3, 1024, 4096, "q4k"), (2, 768, 2560, "q6k")])
def test_op_pass_small_end_to_end(layers, hidden, ffn, down):
    """The pass as three launches per layer, eager and as a replayed graph;
    the staged pass equals it bit for bit."""
    st = Stack(layers, hidden, ffn, down)
    x0, r0 = start_state(hidden)
    xg, rg = st.run_ops(x0, r0, replays=2)
    xst, rst = st.run_ops(x0, r0, replays=2, staged=True)
    assert np.array_equal(xg, xst) and np.array_equal(rg, rst)
    x, r = x0.astype(np.float64), r0.astype(np.float64)
    for l in range(layers):
        x, r = st.oracle_layer(l, x, r)
    dx, dr = np.max(np.abs(xg - x)), np.max(np.abs(rg - r))
    print(f"max |dx| {dx:.2e} |dres| {dr:.2e}")
    assert dx <= 2e-3 and dr <= 2e-3


@pytest.mark.parametrize("layers,hidden,ffn,down", [(1, 512, 1536, "q6k"), (3, 1024, 4096, "q4k"),
                                                    (2, 768, 2560, "q6k")])
def test_pass_modes_bitwise(layers, hidden, ffn, down):
    """f32, staged and fused-tail passes from the same residual, and (Q6_K
    down) the library's kq_ffn_pass_q4k_q6k: identical bits, and the oracle's
    stack from the same start within tolerance."""
    st = Stack(layers, hidden, ffn, down, cfg=14)
    _, r0 = start_state(hidden, cfg=14)
    a = st.run_pass(r0, "f32", replays=1)
    b = st.run_pass(r0, "staged", replays=1)
    c = st.run_pass(r0, "fusedtail", replays=2)
    for u, v in ((a, b), (a, c)):
        assert np.array_equal(u[0], v[0]) and np.array_equal(u[1], v[1])
    if down == "q6k":
        d = st.run_pass(r0, "libpass", replays=2)
        assert np.array_equal(c[0], d[0]) and np.array_equal(c[1], d[1])
    x, r = O.rms_norm(r0.astype(np.float64), 1e-5), r0.astype(np.float64)
    for l in range(layers):
        x, r = st.oracle_layer(l, x, r)
    assert np.max(np.abs(c[0] - x)) <= 2e-3 and np.max(np.abs(c[1] - r)) <= 2e-3


FULL = dict(layers=52, hidden=6656, ffn=19968)

# End-to-end GPU-vs-oracle difference of the 52-layer pass measured on MI355X
# (max |dx|, max |dres|), per start: "oracle_x0" starts the GPU from the
# oracle's entry norm (the single-op pass), "gpu_x0" from the GPU's own entry
# norm (every pass mode of run_pass, which give the same bits).  The stack is
# ill-conditioned (the oracle itself moves by 1.6e-2 under a 1e-7 relative
# perturbation of its start), so the two starts end 5x apart.  The end-to-end
# check allows 5x the recorded difference, so a regression by an order of
# magnitude fails even where the amplification bound is loose; a change of the
# kernels' summation order moves these values and they are then re-recorded.
E2E_RECORDED = {"oracle_x0": (1.220e-02, 7.554e-02), "gpu_x0": (2.360e-03, 1.616e-02)}


@pytest.fixture(scope="module")
def full():
    """The 52-layer FFN stream at 6656 / 19968 (Q4_K gate/up, Q6_K down), with
    the oracle's end-to-end result from the seeded start and, beside it, the
    oracle's own result from a start perturbed by 1e-7 (relative)."""
    layers, hidden, ffn = FULL["layers"], FULL["hidden"], FULL["ffn"]
    st = Stack(layers, hidden, ffn, "q6k", cfg=4)
    x0, r0 = start_state(hidden, cfg=4)
    rng = np.random.default_rng(1)
    x, r = x0.astype(np.float64), r0.astype(np.float64)
    xp = x * (1 + 1e-7 * rng.standard_normal(hidden))
    rp = r * (1 + 1e-7 * rng.standard_normal(hidden))
    for l in range(layers):
        x, r = st.oracle_layer(l, x, r)
        xp, rp = st.oracle_layer(l, xp, rp)
    sens = max(np.max(np.abs(xp - x)), np.max(np.abs(rp - r)))
    print(f"oracle end to end from a 1e-7 perturbed start moves by {sens:.2e} "
          f"(|res| max {np.max(np.abs(r)):.1f})", flush=True)
    return dict(st=st, x0=x0, r0=r0, x=x, r=r, sens=sens)


@pytest.fixture(scope="module")
def teacher_forced(full):
    """(i) teacher-forced: every layer through the single-op launches from the
    GPU's own state, against the oracle's layer from that state.  Returns the
    worst per-layer difference (the per-layer error the end-to-end bound
    amplifies)."""
    st = full["st"]
    xg, rg = full["x0"], full["r0"]
    worst = 0.0
    for l in range(st.layers):
        xn, rn = st.run_ops(xg, rg, first=l, count=1)
        xo, ro = st.oracle_layer(l, xg.astype(np.float64), rg.astype(np.float64))
        d = max(np.max(np.abs(xn - xo)), np.max(np.abs(rn - ro)))
        worst = max(worst, d)
        assert d <= 2e-3, f"layer {l}: {d}"
        xg, rg = xn.astype(np.float32), rn.astype(np.float32)
        if l % 13 == 0:
            print(f"teacher-forced layer {l}: max diff {d:.2e}", flush=True)
    print(f"teacher-forced worst {worst:.2e}", flush=True)
    return worst


def check_end_to_end(full, xe, re, worst, start):
    """(ii) end to end.  If the oracle itself moves by more than the 2e-3
    tolerance under a 1e-7 perturbation, the stack is ill-conditioned at that
    tolerance and the end-to-end result is held to the per-layer error
    amplified as that perturbation is (the strict gate is then the
    teacher-forced check) and to a few times the recorded end-to-end
    difference; a gross error (a layer skipped, reordered or mis-wired) still
    fails the sanity bound."""
    x, r, sens = full["x"], full["r"], full["sens"]
    dx, dr = np.max(np.abs(xe - x)), np.max(np.abs(re - r))
    print(f"end to end: GPU vs oracle max |dx| {dx:.3e} |dres| {dr:.3e} "
          f"(teacher-forced worst {worst:.3e})", flush=True)
    assert np.all(np.isfinite(xe)) and np.all(np.isfinite(re))
    if sens * 100 < 2e-3:
        assert dx <= 2e-3 and dr <= 2e-3, "well-conditioned stack: end to end must hold"
    else:
        amp = sens / 1e-7
        assert max(dx, dr) <= 10 * amp * max(worst, 1e-7) + 2e-3, "end-to-end drift too large"
        assert max(dx / 1.0, dr / max(1.0, np.max(np.abs(r)))) < 0.1, "gross end-to-end error"
    rx, rr = E2E_RECORDED[start]
    assert dx <= max(5 * rx, 2e-3) and dr <= max(5 * rr, 2e-3), \
        f"end-to-end difference grew past 5x the recorded ({rx:.2e}, {rr:.2e})"


def test_op_pass_52_layers_full_size(full, teacher_forced):
    """The pass as three launches per layer over the 52 layers, replayed as one
    graph: (i) teacher-forced (the fixture), (ii) end to end, each graph
    replay equal to the eager pass; the staged pass equals it bit for bit."""
    st = full["st"]
    xe, re = st.run_ops(full["x0"], full["r0"], replays=3)
    check_end_to_end(full, xe, re, teacher_forced, "oracle_x0")
    xs_, rs_ = st.run_ops(full["x0"], full["r0"], replays=3, staged=True)
    assert np.array_equal(xe, xs_) and np.array_equal(re, rs_)


def test_pass_modes_52_layers_full_size(full, teacher_forced):
    """The timed decode step (each tail fused into the next layer's gate+up
    launch, staged activations, replayed as a graph; built in Python and by
    the library's kq_ffn_pass_q4k_q6k) against the f32 pass from the same
    residual: identical bits; and end to end against the oracle."""
    st = full["st"]
    a = st.run_pass(full["r0"], "f32")
    c = st.run_pass(full["r0"], "fusedtail", replays=3)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])
    check_end_to_end(full, c[0], c[1], teacher_forced, "gpu_x0")
    d = st.run_pass(full["r0"], "libpass", replays=2)
    assert np.array_equal(a[0], d[0]) and np.array_equal(a[1], d[1])


@pytest.mark.parametrize("layers,hidden,ffn", [(3, 512, 1536), (2, 6656, 19968), (1, 256, 256),
                                               (2, 8192, 4096)])
def test_library_pass_entry_gain_and_reuse(layers, hidden, ffn):
    """kq_ffn_pass_q4k_q6k with an entry gain, twice in a row on one
    workspace whose contents start as garbage: the same bits as the per-layer
    calls with that gain as layer 0's next gain.  Odd and even layer counts
    (the last residual must land in the caller's buffer either way), workgroups
    without gate+up rows (fewer 16-row groups than compute units), one down
    row per workgroup, and the largest hidden size."""
    st = Stack(layers, hidden, ffn, "q6k", cfg=21)
    _, r0 = start_state(hidden, cfg=21)
    h, f, L, D = hidden, ffn, layers, st.dev
    g_entry = dev(I.gains_f32(h, stream=I.stream_id(21, 99, I.ROLE_GNEXT)))
    ones = torch.ones(h, device="cuda")
    zeros = torch.zeros(h, device="cuda")
    R = [dev(r0), torch.empty(h, device="cuda")]
    X0 = torch.empty(h, device="cuda")
    mid, p = torch.empty(f, device="cuda"), torch.empty(h, device="cuda")
    mid_s = torch.empty(kq.kq_staged_bytes(kq.KQ_QTYPE_Q6K, f), dtype=torch.uint8, device="cuda")
    for l in range(L):
        pp, gp, gn = (zeros, ones, g_entry) if l == 0 else (p, D[l - 1]["gp"], D[l - 1]["gn"])
        kq.kq_ffn_tail_gate_up_q4k(R[l % 2], pp, gp, gn, R[(l + 1) % 2], None, D[l]["wg"],
                                   D[l]["wu"], mid, mid_s, kq.KQ_QTYPE_Q6K, f, h)
        kq.kq_matvec_staged(kq.KQ_QTYPE_Q6K, D[l]["wd"], mid_s, p, h, f)
    kq.kq_fused_residual_norm(R[L % 2], p, X0, D[L - 1]["gp"], D[L - 1]["gn"], 1, h)
    torch.cuda.synchronize()
    want_x, want_r = X0.cpu().numpy(), R[L % 2].cpu().numpy()
    assert np.all(np.isfinite(want_x)) and np.all(np.isfinite(want_r))

    table = kq.kq_ffn_layer_table([(d["wg"], d["wu"], d["wd"], d["gp"], d["gn"]) for d in D])
    wsb = kq.kq_ffn_pass_workspace_bytes(h, f)
    ws = torch.full((wsb,), 0xA5, dtype=torch.uint8, device="cuda")
    res, xo = torch.empty(h, device="cuda"), torch.empty(h, device="cuda")
    for rep in range(2):
        res.copy_(dev(r0))
        xo.fill_(float("nan"))
        kq.kq_ffn_pass_q4k_q6k(table, res, xo, g_entry, ws, wsb, h, f)
        torch.cuda.synchronize()
        assert np.array_equal(xo.cpu().numpy(), want_x), f"call {rep}: x differs"
        assert np.array_equal(res.cpu().numpy(), want_r), f"call {rep}: residual differs"
