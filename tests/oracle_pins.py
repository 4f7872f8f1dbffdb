"""Pins for the CPU oracle: checks against facts fixed by the pages or by the
mathematics, not by the oracle itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with the fact.  ``tests/test_oracle_pins.py`` runs every pin
against the real oracle, and runs them against builds with one planted mistake
each to show that every mistake is caught by at least one pin.
"""
from __future__ import annotations

import json
import os

import numpy as np

import kq_encode as E

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------
# binary16 decode: exhaustive against numpy's float16 (a library routine)
def pin_f16_exhaustive(o):
    bits = np.arange(65536, dtype=np.uint32).astype("<u2")
    ref = bits.view("<f2").astype(np.float64)
    got = np.array([o.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "NaN patterns differ"
    assert np.array_equal(got[~nan], ref[~nan]), "f16 values differ"


# --------------------------------------------------------------------------
# Q4_K field mapping by one-hot brute force
def _q4k_onehot_matrix(k: int):
    """Row p has one non-zero quant, at input position p; d = 1, sc = 1, m = 0."""
    nsb = k // 256
    rows, vals = [], []
    for p in range(k):
        blocks = []
        v = 1 + (p % 15)
        for b in range(nsb):
            q = np.zeros(256, np.int64)
            if b == p // 256:
                q[p % 256] = v
            blocks.append(E.encode_q4k(1.0, 0.0, [1] * 8, [0] * 8, q))
        rows.append(np.concatenate(blocks))
        vals.append(v)
    return np.stack(rows), np.array(vals, np.float64)


def pin_q4k_onehot(o):
    for k in (256, 1024):
        W, vals = _q4k_onehot_matrix(k)
        x = np.arange(1, k + 1, dtype=np.float64)
        y, _ = o.matvec("q4k", W, x, k, k)
        assert np.array_equal(y, vals * x), f"Q4_K one-hot positions wrong at k={k}"


def pin_q4k_scale_and_min_fields(o):
    """Each 6-bit scale and each 6-bit min alone, at every value 0..63."""
    x = np.arange(1, 257, dtype=np.float64)
    sub_sum = np.array([x[32 * s:32 * s + 32].sum() for s in range(8)])
    rows, want = [], []
    for s in range(8):
        for v in range(64):
            sc = [0] * 8
            sc[s] = v
            rows.append(E.encode_q4k(1.0, 0.0, sc, [0] * 8, np.ones(256)))
            want.append(v * sub_sum[s])
            m = [0] * 8
            m[s] = v
            rows.append(E.encode_q4k(0.0, 1.0, [0] * 8, m, np.zeros(256)))
            want.append(-v * sub_sum[s])
    y, _ = o.matvec("q4k", np.stack(rows), x, len(rows), 256)
    assert np.array_equal(y, np.array(want)), "Q4_K scale/min fields decode wrong"


# --------------------------------------------------------------------------
# Q6_K field mapping by one-hot brute force
def pin_q6k_onehot(o):
    k = 512
    nsb = k // 256
    rows, vals = [], []
    for p in range(k):
        v = (7 * p + 1) % 64
        v = 63 if v == 32 else v
        blocks = []
        for b in range(nsb):
            q = np.full(256, 32, np.int64)
            if b == p // 256:
                q[p % 256] = v
            blocks.append(E.encode_q6k(1.0, [1] * 16, q))
        rows.append(np.concatenate(blocks))
        vals.append(v - 32)
    x = np.arange(1, k + 1, dtype=np.float64)
    y, _ = o.matvec("q6k", np.stack(rows), x, k, k)
    assert np.array_equal(y, np.array(vals, np.float64) * x), "Q6_K one-hot positions wrong"


def pin_q6k_qh_lanes(o):
    """Raw bytes: ql = 0 and one 2-bit lane of one qh byte set; only the weight
    that lane feeds may move off -32*d*sc (d = 1, sc = 1)."""
    for h in range(2):
        for j in (0, 5, 31):
            for g in range(4):
                for hi in (1, 2, 3):
                    blk = np.zeros(210, np.uint8)
                    blk[128 + 32 * h + j] = hi << (2 * g)
                    blk[192:208] = 1
                    blk[208], blk[209] = 0x00, 0x3C  # d = 1.0
                    w = o.dequant("q6k", blk, 1, 256)[0]
                    want = np.full(256, -32.0)
                    want[128 * h + 32 * g + j] = 16 * hi - 32
                    assert np.array_equal(w, want), f"qh lane h={h} j={j} g={g}"


def pin_q6k_scale_fields(o):
    x = np.arange(1, 257, dtype=np.float64)
    sub_sum = np.array([x[16 * s:16 * s + 16].sum() for s in range(16)])
    rows, want = [], []
    for s in range(16):
        for v in range(-128, 128):
            sc = [0] * 16
            sc[s] = v
            rows.append(E.encode_q6k(1.0, sc, np.full(256, 33)))
            want.append(v * sub_sum[s])
    y, _ = o.matvec("q6k", np.stack(rows), x, len(rows), 256)
    assert np.array_equal(y, np.array(want)), "Q6_K int8 scales decode wrong"


# --------------------------------------------------------------------------
# closed forms
def pin_closed_forms(o):
    rng = np.random.default_rng(7)
    k = 512
    # (a) all quants equal, one scale and one min everywhere, x = 1
    for _ in range(20):
        d, dmin = E.f16_value(rng.uniform(1e-3, 1e-2)), E.f16_value(rng.uniform(1e-3, 1e-2))
        a, b, c = int(rng.integers(0, 64)), int(rng.integers(0, 64)), int(rng.integers(0, 16))
        blk = E.encode_q4k(d, dmin, [a] * 8, [b] * 8, np.full(256, c))
        y, _ = o.matvec("q4k", np.concatenate([blk, blk]), np.ones(k), 1, k)
        want = k * (d * a * c - dmin * b)
        assert abs(y[0] - want) <= 1e-12 * max(1.0, abs(want)), "closed form (a) Q4_K"
        a6, c6 = int(rng.integers(-128, 128)), int(rng.integers(0, 64))
        blk6 = E.encode_q6k(d, [a6] * 16, np.full(256, c6))
        y6, _ = o.matvec("q6k", np.concatenate([blk6, blk6]), np.ones(k), 1, k)
        want6 = k * d * a6 * (c6 - 32)
        assert abs(y6[0] - want6) <= 1e-12 * max(1.0, abs(want6)), "closed form (a) Q6_K"
    # (b) a single non-zero sub-block with zero mins
    x = rng.standard_normal(256)
    for s in range(8):
        q = np.zeros(256, np.int64)
        q[32 * s:32 * s + 32] = rng.integers(0, 16, 32)
        a = int(rng.integers(1, 64))
        sc = [0] * 8
        sc[s] = a
        d = E.f16_value(0.0078125)
        blk = E.encode_q4k(d, 0.5, sc, [0] * 8, q)
        y, _ = o.matvec("q4k", blk, x, 1, 256)
        want = d * a * float(np.dot(q[32 * s:32 * s + 32], x[32 * s:32 * s + 32]))
        assert abs(y[0] - want) <= 1e-12 * (1 + abs(want)), "closed form (b)"
    # (c) zero mins: y = d * sum_s sc_s * sum_{i in s} q_i x_i
    sc = rng.integers(0, 64, 8)
    q = rng.integers(0, 16, 256)
    blk = E.encode_q4k(0.25, 0.0, sc, rng.integers(0, 64, 8), q)
    y, _ = o.matvec("q4k", blk, x, 1, 256)
    want = 0.25 * sum(sc[s] * np.dot(q[32 * s:32 * s + 32], x[32 * s:32 * s + 32]) for s in range(8))
    assert abs(y[0] - want) <= 1e-12 * (1 + abs(want)), "closed form (c)"
    # (d) Q6_K raw bytes: ql = qh = 0 gives q = 0; ql = qh = 0xFF gives q = 63
    for fill, qv in ((0x00, 0), (0xFF, 63)):
        blk = np.zeros(210, np.uint8)
        blk[0:192] = fill
        blk[192:208] = np.arange(1, 17, dtype=np.int8).view(np.uint8)
        blk[208], blk[209] = 0x00, 0x38  # d = 0.5
        w = o.dequant("q6k", blk, 1, 256)[0]
        want = 0.5 * np.repeat(np.arange(1, 17), 16) * (qv - 32)
        assert np.array_equal(w, want), f"closed form (d) fill {fill:#x}"


# --------------------------------------------------------------------------
# Q5_K field mapping: one-hot brute force, each high-bit lane alone from raw
# bytes, each 6-bit field alone, closed forms
def pin_q5k_onehot(o):
    for k in (256, 1024):
        nsb = k // 256
        rows, vals = [], []
        for p in range(k):
            v = 1 + (p % 31)  # 1..31: half the positions carry the high bit
            blocks = []
            for b in range(nsb):
                q = np.zeros(256, np.int64)
                if b == p // 256:
                    q[p % 256] = v
                blocks.append(E.encode_q5k(1.0, 0.0, [1] * 8, [0] * 8, q))
            rows.append(np.concatenate(blocks))
            vals.append(v)
        x = np.arange(1, k + 1, dtype=np.float64)
        y, _ = o.matvec("q5k", np.stack(rows), x, k, k)
        assert np.array_equal(y, np.array(vals, np.float64) * x), f"Q5_K one-hot positions wrong at k={k}"


def pin_q5k_high_bit_lanes(o):
    """Raw bytes: only bit b of high-bit byte j set (d = 1, every scale 1, no
    mins, all nibbles 0): exactly one weight, 16, at input 64 (b // 2) +
    32 (b % 2) + j."""
    base = E.encode_q5k(1.0, 0.0, [1] * 8, [0] * 8, np.zeros(256))
    rows, pos = [], []
    for j in range(32):
        for b in range(8):
            blk = base.copy()
            blk[16 + j] = 1 << b
            rows.append(blk)
            pos.append(64 * (b // 2) + 32 * (b % 2) + j)
    x = np.arange(1, 257, dtype=np.float64)
    y, _ = o.matvec("q5k", np.stack(rows), x, len(rows), 256)
    assert np.array_equal(y, 16.0 * x[np.array(pos)]), "Q5_K high-bit lanes decode wrong"


def pin_q5k_scale_and_min_fields(o):
    x = np.arange(1, 257, dtype=np.float64)
    sub_sum = np.array([x[32 * s:32 * s + 32].sum() for s in range(8)])
    rows, want = [], []
    for s in range(8):
        for v in range(64):
            sc = [0] * 8
            sc[s] = v
            rows.append(E.encode_q5k(1.0, 0.0, sc, [0] * 8, np.full(256, 17)))
            want.append(17 * v * sub_sum[s])
            m = [0] * 8
            m[s] = v
            rows.append(E.encode_q5k(0.0, 1.0, [0] * 8, m, np.zeros(256)))
            want.append(-v * sub_sum[s])
    y, _ = o.matvec("q5k", np.stack(rows), x, len(rows), 256)
    assert np.array_equal(y, np.array(want)), "Q5_K scale/min fields decode wrong"


def pin_q5k_closed_forms(o):
    # all-equal fields with x = 1: y = k (d a c - dmin b), at the largest quant
    d, dmin = E.f16_value(0.0078125), E.f16_value(0.001953125)
    for c in (0, 16, 31):
        blk = E.encode_q5k(d, dmin, [5] * 8, [3] * 8, np.full(256, c))
        y, _ = o.matvec("q5k", np.stack([np.concatenate([blk] * 4)]), np.ones(1024), 1, 1024)
        assert y[0] == 1024 * (d * 5 * c - dmin * 3), f"Q5_K all-equal closed form at q={c}"


# --------------------------------------------------------------------------
# exactness on integer activations: with x in {-3..3} every product is a
# multiple of 2^-24 and the f64 sums are exact, so y * 2^24 must equal an
# int64 sum computed from the encoded field values.
def pin_exact_integer_inputs(o):
    rng = np.random.default_rng(11)
    n, k = 8, 1024
    nsb = k // 256
    x = rng.integers(-3, 4, k)
    for qt in ("q4k", "q6k", "q5k"):
        W, want = [], []
        for _ in range(n):
            row, acc = [], 0
            for b in range(nsb):
                xs = x[256 * b:256 * b + 256]
                if qt in ("q4k", "q5k"):
                    f = E.random_q4k_fields(rng) if qt == "q4k" else E.random_q5k_fields(rng)
                    row.append(E.encode_q4k(**f) if qt == "q4k" else E.encode_q5k(**f))
                    D = int(round(E.f16_value(f["d"]) * 2**24))
                    Dm = int(round(E.f16_value(f["dmin"]) * 2**24))
                    s = np.arange(256) // 32
                    wi = D * f["sc"][s].astype(np.int64) * f["q"] - Dm * f["m"][s].astype(np.int64)
                else:
                    f = E.random_q6k_fields(rng)
                    row.append(E.encode_q6k(**f))
                    D = int(round(E.f16_value(f["d"]) * 2**24))
                    s = np.arange(256) // 16
                    wi = D * f["sc"][s].astype(np.int64) * (f["q"] - 32)
                acc += int(np.dot(wi.astype(np.int64), xs.astype(np.int64)))
            W.append(np.concatenate(row))
            want.append(acc)
        y, _ = o.matvec(qt, np.stack(W), x.astype(np.float64), n, k)
        got = y * 2.0**24
        assert np.array_equal(got, np.array(want, np.float64)), f"{qt} exact integer sum"


# --------------------------------------------------------------------------
# the matvec against numpy's float64 matmul of the field-defined weights
def _random_encoded(qt, rng, n, k):
    nsb = k // 256
    W, dense = [], []
    for _ in range(n):
        row, drow = [], []
        for _ in range(nsb):
            if qt == "q4k":
                f = E.random_q4k_fields(rng)
                row.append(E.encode_q4k(**f))
                drow.append(E.dense_q4k(**f))
            elif qt == "q5k":
                f = E.random_q5k_fields(rng)
                row.append(E.encode_q5k(**f))
                drow.append(E.dense_q5k(**f))
            else:
                f = E.random_q6k_fields(rng)
                row.append(E.encode_q6k(**f))
                drow.append(E.dense_q6k(**f))
        W.append(np.concatenate(row))
        dense.append(np.concatenate(drow))
    return np.stack(W), np.stack(dense)


def pin_matvec_vs_numpy(o):
    rng = np.random.default_rng(3)
    n, k, m = 24, 1024, 5
    for qt in ("q4k", "q6k", "q5k"):
        W, D = _random_encoded(qt, rng, n, k)
        X = rng.standard_normal((m, k))
        Y, S = o.matmul(qt, W, X, n, k)
        Yref = X @ D.T
        Sref = np.abs(X[:, None, :] * D[None, :, :]).sum(-1)
        assert np.all(np.abs(Y - Yref) <= 1e-12 * Sref), f"{qt} matmul vs numpy"
        assert np.allclose(S, Sref, rtol=1e-12, atol=0), f"{qt} S vs numpy"
        y0, s0 = o.matvec(qt, W, X[2], n, k)
        assert np.array_equal(y0, Y[2]) and np.array_equal(s0, S[2]), "small-M row != matvec"


def pin_threaded_matmul_equals_single_thread(o):
    """The row split over threads changes nothing: every row is computed by one
    job in the same order, so Y and S are bitwise those of one thread, for
    thread counts that do and do not divide the row count (37 rows)."""
    rng = np.random.default_rng(17)
    n, k, m = 37, 512, 3
    for qt in ("q4k", "q6k", "q5k"):
        W, D = _random_encoded(qt, rng, n, k)
        X = rng.standard_normal((m, k))
        Y1, S1 = o.matmul(qt, W, X, n, k, nthreads=1)
        Yref = X @ D.T
        assert np.all(np.abs(Y1 - Yref) <= 1e-12 * S1), f"{qt} single-thread vs numpy"
        for t in (2, 3, 16, 64):
            Yt, St = o.matmul(qt, W, X, n, k, nthreads=t)
            assert np.array_equal(Yt, Y1) and np.array_equal(St, S1), \
                f"{qt} matmul with {t} threads differs from one thread"


# --------------------------------------------------------------------------
# embedding lookup: rows of the table dequantized, out-of-range tokens NaN
def pin_embedding_gather(o):
    rng = np.random.default_rng(21)
    vocab, hidden = 40, 512
    for qt in ("q4k", "q5k"):
        W, D = _random_encoded(qt, rng, vocab, hidden)
        tokens = np.array([0, 39, 7, 7, 12, -1, 40, 3])
        got = o.embedding(qt, W, tokens, vocab, hidden)
        for t, row in zip(tokens, got):
            if 0 <= t < vocab:
                assert np.array_equal(row, D[t]), f"{qt} embedding row {t}"
            else:
                assert np.all(np.isnan(row)), f"{qt} out-of-range token {t} not NaN"


# --------------------------------------------------------------------------
# SiLU-gated product
def pin_silu(o):
    import torch
    rng = np.random.default_rng(5)
    g = np.concatenate([rng.standard_normal(1000) * 5, [0.0, 30.0, -30.0, 700.0, -700.0, -800.0]])
    u = rng.standard_normal(g.size)
    got = o.silu_mul(g, u)
    ref = (torch.nn.functional.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-300), "silu vs torch float64"
    one = o.silu_mul(np.array([0.0, 50.0, -800.0]), np.ones(3))
    assert one[0] == 0.0 and abs(one[1] - 50.0) < 1e-15 * 50 and one[2] == 0.0, "silu limits"


# --------------------------------------------------------------------------
# RMSNorm and the dual-eps tail
def pin_rms_norm_invariants(o):
    rng = np.random.default_rng(9)
    for scale in (1.0, 1e-3, 1e3):
        x = rng.standard_normal(6656) * scale
        g = 1 + 0.1 * rng.standard_normal(6656)
        for eps in (1e-5, 1e-8):
            out = o.rms_norm(x, eps, g)
            ms = np.mean(x * x)
            lhs = np.mean((out / g) ** 2)
            assert abs(lhs - ms / (ms + eps)) <= 1e-12, "mean((out/g)^2) = ms/(ms+eps)"
            out2 = o.rms_norm(7.0 * x, eps * 49.0, g)
            assert np.allclose(out, out2, rtol=1e-12, atol=1e-14), "scale invariance"
    c = o.rms_norm(np.full(64, -3.0), 1e-8, np.full(64, 2.0))
    assert np.allclose(c, -2.0, rtol=1e-8), "constant vector"


def pin_tail_worked_example(o):
    with open(os.path.join(GOLDEN, "tail_worked_example.json")) as f:
        gold = json.load(f)
    r, nxt = o.dual_eps_tail(gold["residual"], gold["projected"], gold["post_weight"],
                             gold["next_weight"], gold["eps_post"], gold["eps_next"])
    assert np.allclose(r, gold["residual_after"], atol=1e-7), "residual after the add"
    assert np.all(np.abs(nxt - np.array(gold["next_input"])) <= gold["tolerance"]), "next_input"


def pin_tail_rows_and_invariants(o):
    rng = np.random.default_rng(13)
    rows, n = 3, 6656
    res = rng.standard_normal((rows, n))
    proj = rng.standard_normal((rows, n)) * np.array([[1.0], [1e-3], [1e4]])
    gp, gn = 1 + 0.1 * rng.standard_normal(n), 1 + 0.1 * rng.standard_normal(n)
    r_all, o_all = o.dual_eps_tail(res, proj, gp, gn)
    for i in range(rows):
        r1, o1 = o.dual_eps_tail(res[i], proj[i], gp, gn)
        assert np.array_equal(r1, r_all[i]) and np.array_equal(o1, o_all[i]), "rows independent"
        ms = np.mean(r_all[i] ** 2)
        assert abs(np.mean((o_all[i] / gn) ** 2) - ms / (ms + 1e-5)) <= 1e-12, "next norm invariant"
        a = r_all[i] - res[i]
        msp = np.mean(proj[i] ** 2)
        assert abs(np.mean((a / gp) ** 2) - msp / (msp + 1e-8)) <= 1e-10, "post norm invariant"
    # constant projection c*1 gives a = c/sqrt(c^2 + eps) * g_post
    res0 = np.zeros(n)
    r, _ = o.dual_eps_tail(res0, np.full(n, -2.5), gp, gn)
    assert np.allclose(r, -gp, rtol=1e-8), "constant projection"


# --------------------------------------------------------------------------
# the FFN layer is the composition of the steps above
def pin_ffn_layer_composition(o):
    from quant_weight_matvec_amd import inputs as I
    hidden, ffn = 512, 1536
    Wg = I.q4k_matrix(ffn, hidden, stream=101)
    Wu = I.q4k_matrix(ffn, hidden, stream=102)
    Wd = I.q6k_matrix(hidden, ffn, stream=103)
    x = I.normal_f32(hidden, stream=104).astype(np.float64)
    res = I.normal_f32(hidden, stream=105).astype(np.float64)
    gp, gn = I.gains_f32(hidden, stream=106), I.gains_f32(hidden, stream=107)
    L = o.ffn_layer(Wg, Wu, Wd, hidden, ffn, x, res, gp, gn)
    g, _ = o.matvec("q4k", Wg, x, ffn, hidden)
    u, _ = o.matvec("q4k", Wu, x, ffn, hidden)
    mid = o.silu_mul(g, u)
    p, _ = o.matvec("q6k", Wd, mid, hidden, ffn)
    r, nxt = o.dual_eps_tail(res, p, gp, gn)
    for a, b in ((L["g"], g), (L["u"], u), (L["mid"], mid), (L["p"], p),
                 (L["residual"], r), (L["next_in"], nxt)):
        assert np.array_equal(a, b), "ffn layer != composition of its steps"


ALL_PINS = [
    pin_f16_exhaustive, pin_q4k_onehot, pin_q4k_scale_and_min_fields, pin_q6k_onehot,
    pin_q6k_qh_lanes, pin_q6k_scale_fields, pin_closed_forms, pin_q5k_onehot,
    pin_q5k_high_bit_lanes, pin_q5k_scale_and_min_fields, pin_q5k_closed_forms,
    pin_exact_integer_inputs, pin_matvec_vs_numpy, pin_threaded_matmul_equals_single_thread,
    pin_embedding_gather, pin_silu, pin_rms_norm_invariants, pin_tail_worked_example,
    pin_tail_rows_and_invariants, pin_ffn_layer_composition,
]
