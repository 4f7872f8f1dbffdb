"""The C-ABI library on the CPU: it loads, exports every symbol the public
headers declare, and rejects bad arguments on the host before any device call.

Runs without a GPU: every call here fails validation (or is the n_rows == 0
no-op), and validation happens before the library touches the HIP runtime.
Pointers are fake addresses that are never dereferenced.
"""
import ctypes as C
import glob
import os
import re

import pytest

import code_object as CO
import quant_weight_matvec_amd as kq
from quant_weight_matvec_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(kq_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = kq.lib()
    names = _declared_symbols()
    assert "kq_matvec_q4k" in names and "kq_fused_residual_norm" in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


def test_status_strings_and_build_info():
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        s = kq.kq_status_string(code)
        assert s.startswith("KQ_")
    assert kq.kq_status_string(-99) == "KQ_ERR_UNKNOWN"
    info = kq.kq_build_info()
    assert "gfx950" in info and "q5k_matvec" in info and "q6k_matvec" in info


W, X, Y, G = 0x100000, 0x200000, 0x300000, 0x400000  # fake, aligned, never dereferenced


def _q4(W=W, x=X, y=Y, n=8, k=1024, gate=None):
    return kq.lib().kq_matvec_q4k(W, x, y, n, k, gate, None)


def _q6(W=W, x=X, y=Y, n=8, k=1024):
    return kq.lib().kq_matvec_q6k(W, x, y, n, k, None)


def test_matvec_validation():
    assert _q4(W=None) == B.KQ_ERR_NULL
    assert _q4(x=None) == B.KQ_ERR_NULL
    assert _q4(y=None) == B.KQ_ERR_NULL
    assert _q4(k=300) == B.KQ_ERR_SHAPE
    assert _q4(k=0) == B.KQ_ERR_SHAPE
    assert _q4(k=128) == B.KQ_ERR_SHAPE
    assert _q4(k=B.KQ_MAX_K + 256) == B.KQ_ERR_UNSUPPORTED
    assert _q4(n=-1) == B.KQ_ERR_SHAPE
    assert _q4(n=2**31) == B.KQ_ERR_SHAPE
    assert _q4(W=W + 4) == B.KQ_ERR_ALIGN          # Q4_K needs 16-byte weights
    assert _q4(x=X + 4) == B.KQ_ERR_ALIGN
    assert _q4(y=Y + 2) == B.KQ_ERR_ALIGN
    assert _q4(gate=G + 1) == B.KQ_ERR_ALIGN
    assert _q6(W=W + 2) == B.KQ_ERR_ALIGN            # Q6_K needs 4-byte weights
    assert _q4(y=W + 64) == B.KQ_ERR_ALIAS           # output inside the weights
    assert _q4(y=X + 16) == B.KQ_ERR_ALIAS           # output inside x
    assert _q4(y=G, gate=G) == B.KQ_ERR_ALIAS        # output on the gate
    assert _q6(y=W + 8 * 4 * 210 - 4) == B.KQ_ERR_ALIAS
    assert _q4(n=0) == B.KQ_OK                       # empty: nothing enqueued
    assert _q6(n=0) == B.KQ_OK


def test_gate_up_validation():
    f = kq.lib().kq_ffn_gate_up_q4k
    U, M = 0x500000, 0x300000
    assert f(None, U, X, M, 8, 1024, None) == B.KQ_ERR_NULL
    assert f(W, U, X, None, 8, 1024, None) == B.KQ_ERR_NULL
    assert f(W, U, X, M, 8, 1000, None) == B.KQ_ERR_SHAPE
    assert f(W, U, X, M, -1, 1024, None) == B.KQ_ERR_SHAPE
    assert f(W, U, X, M, 8, B.KQ_MAX_K + 256, None) == B.KQ_ERR_UNSUPPORTED
    assert f(W, U + 8, X, M, 8, 1024, None) == B.KQ_ERR_ALIGN   # Q4_K weights 16-byte aligned
    assert f(W, U, X + 4, M, 8, 1024, None) == B.KQ_ERR_ALIGN
    assert f(W, U, X, M + 2, 8, 1024, None) == B.KQ_ERR_ALIGN
    assert f(W, U, X, U + 64, 8, 1024, None) == B.KQ_ERR_ALIAS  # mid inside W_up
    assert f(W, U, X, X + 16, 8, 1024, None) == B.KQ_ERR_ALIAS  # mid inside x
    assert f(W, U, X, M, 0, 1024, None) == B.KQ_OK


def test_group_validation():
    f = kq.lib().kq_matvec_group
    arr = lambda t, v: (t * len(v))(*v)
    P, I64 = C.c_void_p, C.c_int64
    W0, W1, Y0, Y1 = 1 << 40, 2 << 40, 3 << 40, 4 << 40
    X0 = 5 << 40

    def call(qt=1, count=2, W=(W0, W1), y=(Y0, Y1), n=(256, 4096), x=X0, k=6656):
        return f(qt, count, arr(P, W), arr(P, y), arr(I64, n), x, k, None)

    assert call() == B.KQ_ERR_DEVICE or call() == B.KQ_OK or call() < 0  # reaches the device check
    assert call(qt=4) == B.KQ_ERR_SHAPE                                # qtype 3 is Q5_K
    assert call(count=0) == B.KQ_ERR_SHAPE
    assert call(count=5, W=(W0,) * 5, y=(Y0,) * 5, n=(1,) * 5) == B.KQ_ERR_SHAPE
    assert call(W=(W0, None)) == B.KQ_ERR_NULL
    assert call(y=(None, Y1)) == B.KQ_ERR_NULL
    assert call(x=None) == B.KQ_ERR_NULL
    assert call(n=(-1, 4)) == B.KQ_ERR_SHAPE
    assert call(n=(2**31 - 1, 4)) == B.KQ_ERR_SHAPE                 # total past 2^31
    assert call(k=1000) == B.KQ_ERR_SHAPE
    assert call(k=B.KQ_MAX_K + 256) == B.KQ_ERR_UNSUPPORTED
    assert call(W=(W0 + 8, W1)) == B.KQ_ERR_ALIGN                   # Q4_K weights 16-byte aligned
    assert call(qt=2, W=(W0 + 4, W1)) == B.KQ_OK or call(qt=2, W=(W0 + 4, W1)) == B.KQ_ERR_DEVICE
    assert call(qt=2, W=(W0 + 2, W1)) == B.KQ_ERR_ALIGN             # Q6_K weights 4-byte aligned
    assert call(y=(Y0 + 2, Y1)) == B.KQ_ERR_ALIGN
    assert call(x=X0 + 4) == B.KQ_ERR_ALIGN
    assert call(y=(Y0, Y0 + 512)) == B.KQ_ERR_ALIAS                 # outputs overlap
    assert call(y=(W1 + 64, Y1)) == B.KQ_ERR_ALIAS                  # output inside a matrix
    assert call(y=(X0 + 16, Y1)) == B.KQ_ERR_ALIAS                  # output inside x
    assert call(n=(0, 0)) == B.KQ_OK                                 # nothing to do
    assert call(W=(None, None), y=(None, None), n=(0, 0)) == B.KQ_OK  # empty members: no pointers
    g = kq.lib().kq_matvec_group_staged
    assert g(1, 1, arr(P, (W0,)), arr(P, (Y0,)), arr(I64, (8,)), X0 + 8, 1024, None) == B.KQ_ERR_ALIGN
    assert g(1, 1, arr(P, (W0,)), arr(P, (Y0,)), arr(I64, (8,)), Y0 - 1024, 1024, None) == B.KQ_ERR_ALIAS


def test_small_m_validation():
    f = kq.lib().kq_matmul_small_m
    WS = 0x600000
    a = lambda *v, ws=WS, wsb=1 << 20: f(*v, ws, wsb, None)
    assert a(4, W, X, 1024, Y, 8, 8, 1024, 4) == B.KQ_ERR_SHAPE      # qtype
    assert a(3, W, X, 1024, Y, 8, 8, 1024, 4) == B.KQ_ERR_UNSUPPORTED  # Q5_K: no matrix-core path
    assert a(1, W, X, 1024, Y, 8, 8, 1024, 0) == B.KQ_ERR_SHAPE      # m = 0
    assert a(1, W, X, 1024, Y, 8, 8, 1024, 17) == B.KQ_ERR_UNSUPPORTED
    assert a(1, W, X, 1000, Y, 8, 8, 1024, 4) == B.KQ_ERR_SHAPE      # ldx < k
    assert a(1, W, X, 1026, Y, 8, 8, 1024, 4) == B.KQ_ERR_SHAPE      # ldx % 4
    assert a(1, W, X, 1024, Y, 7, 8, 1024, 4) == B.KQ_ERR_SHAPE      # ldy < n_rows
    assert a(1, W, X, 1024, Y, 8, 8, 1024, 4, wsb=-1) == B.KQ_ERR_SHAPE
    assert a(1, None, X, 1024, Y, 8, 8, 1024, 4) == B.KQ_ERR_NULL
    assert a(2, W + 2, X, 1024, Y, 8, 8, 1024, 4) == B.KQ_ERR_ALIGN
    assert a(1, W, X, 1024, Y, 8, 8, 1024, 4, ws=WS + 16) == B.KQ_ERR_ALIGN
    assert a(1, W, X, 1024, X + 4 * 1024, 8, 8, 1024, 4) == B.KQ_ERR_ALIAS
    assert a(1, W, X, 1024, Y, 8, 0, 1024, 4) == B.KQ_OK             # empty
    q = kq.lib().kq_matmul_small_m_workspace_bytes
    assert q(1, 8, 1024, 17) == B.KQ_ERR_UNSUPPORTED
    assert q(4, 8, 1024, 4) == B.KQ_ERR_SHAPE
    assert q(3, 8, 1024, 4) == B.KQ_ERR_UNSUPPORTED
    assert q(1, 8, 300, 4) == B.KQ_ERR_SHAPE
    assert q(1, 0, 1024, 4) == 0 and q(2, 8, 1024, 1) == 0        # empty, or m = 1 (matvec)


def test_small_m_noalloc_validation():
    """The no-allocation small-M entry: the workspace version's checks, and a
    shape whose split needs more than the library's scratch array is refused
    on the host (KQ_ERR_UNSUPPORTED) before any device call."""
    f = kq.lib().kq_matmul_small_m_noalloc
    a = lambda *v: f(*v, None)
    assert a(4, W, X, 1024, Y, 8, 8, 1024, 4) == B.KQ_ERR_SHAPE      # qtype
    assert a(3, W, X, 1024, Y, 8, 8, 1024, 4) == B.KQ_ERR_UNSUPPORTED  # Q5_K: no matrix-core path
    assert a(1, W, X, 1024, Y, 8, 8, 1024, 0) == B.KQ_ERR_SHAPE      # m = 0
    assert a(1, W, X, 1024, Y, 8, 8, 1024, 17) == B.KQ_ERR_UNSUPPORTED
    assert a(1, W, X, 1000, Y, 8, 8, 1024, 4) == B.KQ_ERR_SHAPE      # ldx < k
    assert a(1, W, X, 1024, Y, 7, 8, 1024, 4) == B.KQ_ERR_SHAPE      # ldy < n_rows
    assert a(1, None, X, 1024, Y, 8, 8, 1024, 4) == B.KQ_ERR_NULL
    assert a(2, W + 2, X, 1024, Y, 8, 8, 1024, 4) == B.KQ_ERR_ALIGN
    assert a(1, W, X, 1024, X + 4 * 1024, 8, 8, 1024, 4) == B.KQ_ERR_ALIAS
    assert a(1, W, X, 1024, Y, 8, 0, 1024, 4) == B.KQ_OK             # empty
    # far-apart fake addresses so that only the size decides
    Wb, Xb, Yb = 1 << 40, 2 << 40, 3 << 40
    n, k, m = 19968, 40960, 16
    plan = kq.kq_tune_small_m_plan(B.KQ_QTYPE_Q4K, n, k, m, 256)
    assert plan["workspace"] > 0 and plan["grid"] * 2 * 16 * 256 * 4 > 16 << 20
    assert a(1, Wb, Xb, k, Yb, n, n, k, m) == B.KQ_ERR_UNSUPPORTED
    assert B.KQ_SMALL_M_SCRATCH_BYTES == 16 * 1024 + 16 * 1024 * 1024


def test_probe_validation():
    f = kq.lib().kq_probe_read_bw
    P, O = 0x100000, 0x900000
    assert f(None, 1 << 20, O, 256, 256, 8, 1, None) == B.KQ_ERR_NULL
    assert f(P, 1000, O, 256, 256, 8, 1, None) == B.KQ_ERR_SHAPE         # not whole 16 B
    assert f(P, 1 << 20, O, 256, 100, 8, 1, None) == B.KQ_ERR_SHAPE      # block % 64
    assert f(P, 1 << 20, O, 256, 2048, 8, 1, None) == B.KQ_ERR_SHAPE     # block > 1024
    assert f(P, 1 << 20, O, 256, 256, 3, 1, None) == B.KQ_ERR_SHAPE      # unroll
    assert f(P, 1 << 20, O, 256, 256, 8, 4, None) == B.KQ_ERR_SHAPE      # flags
    assert f(P + 4, 1 << 20, O, 256, 256, 8, 1, None) == B.KQ_ERR_ALIGN
    assert f(P, 1 << 20, P + 64, 256, 256, 8, 1, None) == B.KQ_ERR_ALIAS


def test_tail_validation():
    f = kq.lib().kq_fused_residual_norm
    R, P, O, GP, GN = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000
    ok = (R, P, O, GP, GN, 2, 6656, C.c_float(1e-8), C.c_float(1e-5), None)
    assert f(*ok[:5], 2, 6, *ok[7:]) == B.KQ_ERR_SHAPE
    assert f(*ok[:5], 2, 0, *ok[7:]) == B.KQ_ERR_SHAPE
    assert f(*ok[:5], 2, B.KQ_MAX_TAIL_N + 4, *ok[7:]) == B.KQ_ERR_UNSUPPORTED
    assert f(*ok[:5], -1, 6656, *ok[7:]) == B.KQ_ERR_SHAPE
    assert f(*ok[:7], C.c_float(float("nan")), ok[8], None) == B.KQ_ERR_SHAPE
    assert f(*ok[:7], ok[7], C.c_float(-1.0), None) == B.KQ_ERR_SHAPE
    assert f(None, *ok[1:]) == B.KQ_ERR_NULL
    assert f(R + 4, *ok[1:]) == B.KQ_ERR_ALIGN
    assert f(R, P, R + 16, *ok[3:]) == B.KQ_ERR_ALIAS                      # next_in on residual
    assert f(R, R + 64, O, *ok[3:]) == B.KQ_ERR_ALIAS                      # projected on residual
    assert f(*ok[:5], 0, 6656, *ok[7:]) == B.KQ_OK                          # empty


def test_staged_validation():
    L = kq.lib()
    # sizes: 3 byte-limb planes of k + k/8 bytes (16 bytes of padding per 128
    # inputs), then a scale and a sum per group (32 for Q4_K, 16 for Q6_K)
    assert kq.kq_staged_bytes(B.KQ_QTYPE_Q4K, 6656) == 3 * (6656 + 832) + 8 * 6656 // 32
    assert kq.kq_staged_bytes(B.KQ_QTYPE_Q6K, 19968) == 3 * (19968 + 2496) + 8 * 19968 // 16
    assert L.kq_staged_bytes(4, 1024) == B.KQ_ERR_SHAPE
    assert L.kq_staged_bytes(3, 1024) == L.kq_staged_bytes(1, 1024)  # Q5_K: groups of 32
    assert L.kq_staged_bytes(1, 1000) == B.KQ_ERR_SHAPE
    assert L.kq_staged_bytes(1, B.KQ_MAX_K + 256) == B.KQ_ERR_UNSUPPORTED
    XS = 0x600000
    st = L.kq_stage_activation
    assert st(4, X, XS, 1024, None) == B.KQ_ERR_SHAPE
    assert st(1, None, XS, 1024, None) == B.KQ_ERR_NULL
    assert st(1, X, XS, 1000, None) == B.KQ_ERR_SHAPE
    assert st(1, X, XS + 8, 1024, None) == B.KQ_ERR_ALIGN
    assert st(1, X, X + 1024, 1024, None) == B.KQ_ERR_ALIAS
    mv = L.kq_matvec_staged
    assert mv(4, W, XS, Y, 8, 1024, None, None) == B.KQ_ERR_SHAPE
    assert mv(3, W + 8, XS, Y, 8, 1024, None, None) == B.KQ_ERR_ALIGN   # Q5_K weights 16-byte aligned
    assert mv(1, W, None, Y, 8, 1024, None, None) == B.KQ_ERR_NULL
    assert mv(2, W, XS, Y, 8, 1024, G, None) == B.KQ_ERR_UNSUPPORTED    # no SiLU epilogue for Q6_K
    assert mv(1, W + 4, XS, Y, 8, 1024, None, None) == B.KQ_ERR_ALIGN
    assert mv(2, W + 2, XS, Y, 8, 1024, None, None) == B.KQ_ERR_ALIGN
    assert mv(1, W, XS + 4, Y, 8, 1024, None, None) == B.KQ_ERR_ALIGN
    assert mv(1, W, XS, XS + 64, 8, 1024, None, None) == B.KQ_ERR_ALIAS  # y inside xs
    assert mv(1, W, XS, Y, 0, 1024, None, None) == B.KQ_OK
    gu = L.kq_ffn_gate_up_q4k_staged
    U, M, MS = 0x500000, 0x700000, 0x800000
    assert gu(W, U, None, M, MS, 2, 512, 1024, None) == B.KQ_ERR_NULL
    assert gu(W, U, XS, M, MS, 4, 512, 1024, None) == B.KQ_ERR_SHAPE     # mid_qtype
    assert gu(W, U, XS, M, MS, 2, 500, 1024, None) == B.KQ_ERR_SHAPE     # staged mid: n_rows % 256
    assert gu(W, U, XS, M, MS + 8, 2, 512, 1024, None) == B.KQ_ERR_ALIGN
    assert gu(W, U, XS, M, M + 16, 2, 512, 1024, None) == B.KQ_ERR_ALIAS  # mid_s on mid
    assert gu(W, U, XS, XS + 16, None, 0, 8, 1024, None) == B.KQ_ERR_ALIAS  # mid inside xs
    assert gu(W, U, XS, M, None, 0, 0, 1024, None) == B.KQ_OK
    tl = L.kq_fused_residual_norm_staged
    R, P, O, GP, GN, OS = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x900000
    e = (C.c_float(1e-8), C.c_float(1e-5), None)
    assert tl(R, P, O, None, 1, GP, GN, 1, 6656, *e) == B.KQ_ERR_NULL
    assert tl(R, P, O, OS, 4, GP, GN, 1, 6656, *e) == B.KQ_ERR_SHAPE
    assert tl(R, P, O, OS, 1, GP, GN, 1, 6660, *e) == B.KQ_ERR_SHAPE      # n % 256
    assert tl(R, P, O, OS + 4, 1, GP, GN, 1, 6656, *e) == B.KQ_ERR_ALIGN
    assert tl(R, P, O, O + 64, 1, GP, GN, 1, 6656, *e) == B.KQ_ERR_ALIAS  # staged on next_in
    assert tl(R, P, O, OS, 1, GP, GN, 0, 6656, *e) == B.KQ_OK


def test_tail_gate_up_validation():
    f = kq.lib().kq_ffn_tail_gate_up_q4k
    R, P, GP, GN, RO, XO = 0x100000, 0x110000, 0x120000, 0x130000, 0x140000, 0x150000
    WG, WU, M, MS = 0x1000000, 0x2000000, 0x3000000, 0x3100000
    e = (C.c_float(1e-8), C.c_float(1e-5), None)
    ok = (R, P, GP, GN, RO, XO, WG, WU, M, MS, 2, 512, 1024)
    a = lambda *v: f(*v, *e)
    assert a(None, *ok[1:]) == B.KQ_ERR_NULL
    assert a(*ok[:4], None, *ok[5:]) == B.KQ_ERR_NULL                  # residual_out
    assert a(*ok[:11], 0, 1024) == B.KQ_ERR_SHAPE                      # n_rows 0
    assert a(*ok[:11], 500, 1024) == B.KQ_ERR_SHAPE                    # staged mid: n_rows % 256
    assert a(*ok[:10], 4, 512, 1024) == B.KQ_ERR_SHAPE                 # mid_qtype
    assert a(*ok[:12], 1000) == B.KQ_ERR_SHAPE
    assert a(*ok[:12], 8448) == B.KQ_ERR_UNSUPPORTED                   # k > KQ_MAX_FUSED_TAIL_K
    assert f(*ok, C.c_float(-1.0), C.c_float(1e-5), None) == B.KQ_ERR_SHAPE
    assert a(R + 4, *ok[1:]) == B.KQ_ERR_ALIGN
    assert a(*ok[:5], XO + 8, *ok[6:]) == B.KQ_ERR_ALIGN               # next_in
    assert a(*ok[:4], R, *ok[5:]) == B.KQ_ERR_ALIAS                    # residual_out on residual_in
    assert a(*ok[:5], RO + 16, *ok[6:]) == B.KQ_ERR_ALIAS              # next_in on residual_out
    assert a(*ok[:8], WG + 64, *ok[9:]) == B.KQ_ERR_ALIAS              # mid inside W_gate
    assert a(*ok[:9], M + 16, *ok[10:]) == B.KQ_ERR_ALIAS              # mid_s on mid


def test_q5k_and_embedding_validation():
    q5 = kq.lib().kq_matvec_q5k
    assert q5(None, X, Y, 8, 1024, None, None) == B.KQ_ERR_NULL
    assert q5(W + 8, X, Y, 8, 1024, None, None) == B.KQ_ERR_ALIGN
    assert q5(W, X, Y, 8, 1000, None, None) == B.KQ_ERR_SHAPE
    assert q5(W, X, W + 64, 8, 1024, None, None) == B.KQ_ERR_ALIAS
    assert q5(W, X, Y, 0, 1024, None, None) == B.KQ_OK
    e = kq.lib().kq_embedding
    E0, T0, O0 = 1 << 40, 2 << 40, 3 << 40
    assert e(2, E0, 100, 1024, T0, 4, O0, None) == B.KQ_ERR_SHAPE        # Q6_K tables: not supported
    assert e(1, None, 100, 1024, T0, 4, O0, None) == B.KQ_ERR_NULL
    assert e(1, E0, 0, 1024, T0, 4, O0, None) == B.KQ_ERR_SHAPE
    assert e(1, E0, 100, 1000, T0, 4, O0, None) == B.KQ_ERR_SHAPE
    assert e(1, E0, 100, 1024, T0, -1, O0, None) == B.KQ_ERR_SHAPE
    assert e(1, E0 + 8, 100, 1024, T0, 4, O0, None) == B.KQ_ERR_ALIGN
    assert e(3, E0, 100, 1024, T0 + 2, 4, O0, None) == B.KQ_ERR_ALIGN
    assert e(1, E0, 100, 1024, T0, 4, O0 + 4, None) == B.KQ_ERR_ALIGN
    assert e(1, E0, 100, 1024, T0, 4, E0 + 1024, None) == B.KQ_ERR_ALIAS  # output inside the table
    assert e(1, E0, 100, 1024, T0, 4, T0, None) == B.KQ_ERR_ALIAS         # output on the tokens
    assert e(3, E0, 100, 1024, T0, 0, O0, None) == B.KQ_OK


def test_verify_gate_up_validation():
    f = kq.lib().kq_ffn_gate_up_q4k_small_m
    U, M_, WS = 1 << 40, 2 << 40, 3 << 40
    a = lambda *v, ws=WS, wsb=1 << 20: f(*v, ws, wsb, None)
    assert a(None, U, X, 1024, M_, 8, 8, 1024, 4) == B.KQ_ERR_NULL
    assert a(W, U, X, 1024, M_, 8, 8, 1024, 0) == B.KQ_ERR_SHAPE
    assert a(W, U, X, 1024, M_, 8, 8, 1024, 17) == B.KQ_ERR_UNSUPPORTED
    assert a(W, U, X, 1000, M_, 8, 8, 1024, 4) == B.KQ_ERR_SHAPE     # ldx < k
    assert a(W, U, X, 1024, M_, 7, 8, 1024, 4) == B.KQ_ERR_SHAPE     # ldm < n_rows
    assert a(W, U + 4, X, 1024, M_, 8, 8, 1024, 4) == B.KQ_ERR_ALIGN
    assert a(W, U, X, 1024, M_, 8, 8, 1024, 4, ws=WS + 16) == B.KQ_ERR_ALIGN
    assert a(W, U, X, 1024, U + 128, 8, 8, 1024, 4) == B.KQ_ERR_ALIAS  # Mid inside W_up
    assert a(W, U, X, 1024, M_, 8, 0, 1024, 4) == B.KQ_OK


def test_tune_validation():
    with pytest.raises(kq.KQError):
        kq.kq_tune_set_shape(1, lanes=12)
    with pytest.raises(kq.KQError):
        kq.kq_tune_set_shape(4, lanes=8)
    with pytest.raises(kq.KQError):
        kq.kq_tune_set_shape(1, waves=17)


def test_binding_raises_on_error_status():
    with pytest.raises(kq.KQError) as e:
        kq.kq_matvec_q4k(W, X, Y, 8, 300, stream=0)
    assert e.value.status == B.KQ_ERR_SHAPE


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(kq.KQLibraryMissing):
        kq.kq_matvec_q4k(W, X, Y, 8, 1024, stream=0)


def test_small_m_plans_fit_and_cover():
    """Host-side launch plans of the verify matmul over a sweep of shapes and
    device sizes: the staged window fits LDS, every workgroup's range is at
    most one row of superblocks (so it touches at most two 256-row groups,
    which the kernel's two register segments assume), and the workspace is
    requested exactly when a row group is split between workgroups."""
    for qt in (B.KQ_QTYPE_Q4K, B.KQ_QTYPE_Q6K):
        for m in (2, 3, 5, 8, 9, 12, 16):
            for k in (256, 512, 1280, 6656, 19968, B.KQ_MAX_K):
                for n in (1, 17, 256, 300, 4097, 19968):
                    for cus in (80, 256, 304):
                        p = kq.kq_tune_small_m_plan(qt, n, k, m, cus)
                        nb, rgs = k // 256, (n + 255) // 256
                        T, G = p["tiles"], p["grid"]
                        assert T == rgs * nb
                        assert min(T, cus) <= G <= T
                        if m <= 8 or qt == B.KQ_QTYPE_Q4K:
                            assert p["threads"] == 1024
                        else:  # Q6_K: 16 waves when their tiles leave room for a one-round window
                            assert p["threads"] in (512, 1024)
                            if p["threads"] == 1024:
                                assert G == min(T, cus), (qt, m, k, n, cus, p)
                        assert p["lds"] <= 160 * 1024, (qt, m, k, n, p)
                        assert p["window"] == -(-T // G) and p["window"] <= nb
                        split = False
                        for g in range(G):
                            t0, t1 = g * T // G, (g + 1) * T // G
                            assert t1 > t0
                            assert (t1 - 1) // nb - t0 // nb <= 1  # at most two row groups
                            split |= t0 % nb != 0 or (t1 % nb != 0 and t1 < T)
                        if split:
                            assert p["workspace"] >= G * 2 * 16 * 256 * 4
                        else:
                            assert p["workspace"] == 0
    assert kq.kq_tune_small_m_plan(1, 8, 1024, 4, 256)["workspace"] >= 0
    with pytest.raises(kq.KQError):
        kq.kq_tune_small_m_plan(1, 8, 1024, 1, 256)


def test_matvec_plans_fit():
    """Automatic M = 1 launch shapes over a sweep of shapes and device sizes:
    a workgroup's activation staging fits LDS, and so do the stagings of all
    workgroups a CU is meant to hold at once; the shape is one the kernels
    are built for."""
    for qt in (B.KQ_QTYPE_Q4K, B.KQ_QTYPE_Q6K):
        for staged in (False, True):
            for k in (256, 1024, 6656, 8192, 8448, 19968, B.KQ_MAX_K):
                for n in (1, 7, 300, 6656, 19968, 100000):
                    for cus in (80, 256, 304):
                        p = kq.kq_tune_matvec_plan(qt, n, k, staged, cus)
                        assert p["lanes"] in (4, 8, 16, 32, 64) and 1 <= p["waves"] <= 16
                        assert p["depth"] in (1, 2, 3)
                        assert 1 <= p["grid"] <= p["per_cu"] * cus
                        # the staged activation as the layout defines it: three byte
                        # planes of k inputs with 16 bytes of padding per 128, then a
                        # f32 scale and a f32 sum per scale group
                        group = 32 if qt == B.KQ_QTYPE_Q4K else 16
                        staged = 3 * (k + 16 * (k // 128)) + 8 * (k // group)
                        assert p["lds"] >= staged, (qt, k, p)
                        # dynamic LDS of the plan plus the largest static LDS of any
                        # matvec kernel in the built library, per CU
                        static = CO.max_static_lds(r"q[46]k_matvec_kernel")
                        assert p["per_cu"] * (p["lds"] + static) <= 160 * 1024, \
                            (qt, k, n, cus, p, static)
    with pytest.raises(kq.KQError):
        kq.kq_tune_matvec_plan(1, 0, 1024, False, 256)


def test_kernel_code_hash_reads_the_built_code_object():
    """bench.py keys its committed HBM counter summaries to a hash of the
    kernel's machine code, read with its own ELF/offload-bundle reader; the
    kernels it finds must be the ones the LLVM tools list from the same code
    object, and the hash must separate kernel families."""
    import sys
    sys.path.insert(0, ROOT)
    import bench
    meta = CO.kernels()
    assert sorted(n for n, _ in bench.kernel_code("")) == sorted(meta)
    for part in bench.PMC_KERNELS.values():
        code = bench.kernel_code(part)
        assert len(code) == 1, (part, code)  # exactly the timed instantiation
        assert [n for n, _ in code] == sorted(n for n in meta if part in n)
        assert all(len(body) >= 4 and len(body) % 4 == 0 for _, body in code)
        assert bench.kernel_code_hash(part) == bench.kernel_code_hash(part)
    hashes = {bench.kernel_code_hash(p) for p in bench.PMC_KERNELS.values()}
    assert None not in hashes and len(hashes) == len(bench.PMC_KERNELS)
    assert bench.kernel_code_hash("no_such_kernel_name") is None


def test_ffn_pass_validation():
    """kq_ffn_pass_q4k_q6k checks its arguments and every layer record of its
    host table before anything is enqueued."""
    R, XO, GE, WS = 0x100000, 0x200000, 0x300000, 0x1000000
    h, f = 6656, 19968
    q4b, q6b = f * (h // 256) * 144, h * (f // 256) * 210
    need = kq.kq_ffn_pass_workspace_bytes(h, f)
    # the residual's second buffer, the down output, staged mid for Q6_K, mid
    up = lambda b: (b + 255) // 256 * 256
    assert need == 2 * up(4 * h) + up(kq.kq_staged_bytes(kq.KQ_QTYPE_Q6K, f)) + up(4 * f)
    base = 0x10000000

    def layer(l, **kw):
        o = base + l * 0x10000000
        d = dict(W_gate=o, W_up=o + 0x4800000, W_down=o + 0x9000000, g_post=o + 0xF000000,
                 g_next=o + 0xF100000)
        d.update(kw)
        return B.KqFfnLayer(**d)

    def call(layers=None, n=2, r=R, xo=XO, ge=None, ws=WS, wsb=need, hidden=h, ffn=f,
             ep=1e-8, en=1e-5):
        layers = layers if layers is not None else [layer(i) for i in range(n)]
        table = (B.KqFfnLayer * max(1, len(layers)))(*layers)
        return kq.lib().kq_ffn_pass_q4k_q6k(table, n, r, xo, ge, ws, wsb, hidden, ffn, ep, en,
                                            None)

    assert kq.lib().kq_ffn_pass_q4k_q6k(None, 1, R, XO, None, WS, need, h, f, 1e-8, 1e-5,
                                        None) == B.KQ_ERR_NULL
    assert call(r=None) == B.KQ_ERR_NULL
    assert call(xo=None) == B.KQ_ERR_NULL
    assert call(ws=None) == B.KQ_ERR_NULL
    assert call(layers=[layer(0), layer(1, W_down=None)]) == B.KQ_ERR_NULL
    assert call(layers=[layer(0, g_next=None), layer(1)]) == B.KQ_ERR_NULL
    assert call(n=0, layers=[layer(0)]) == B.KQ_ERR_SHAPE
    assert call(hidden=300) == B.KQ_ERR_SHAPE
    assert call(ffn=1000) == B.KQ_ERR_SHAPE
    assert call(hidden=B.KQ_MAX_FUSED_TAIL_K + 256) == B.KQ_ERR_UNSUPPORTED
    assert call(ffn=B.KQ_MAX_K + 256) == B.KQ_ERR_UNSUPPORTED
    assert call(wsb=need - 1) == B.KQ_ERR_SHAPE
    assert call(ep=-1.0) == B.KQ_ERR_SHAPE
    assert call(en=float("inf")) == B.KQ_ERR_SHAPE
    assert call(r=R + 4) == B.KQ_ERR_ALIGN
    assert call(xo=XO + 8) == B.KQ_ERR_ALIGN
    assert call(ge=GE + 4) == B.KQ_ERR_ALIGN
    assert call(ws=WS + 128) == B.KQ_ERR_ALIGN
    assert call(layers=[layer(0, W_gate=base + 8), layer(1)]) == B.KQ_ERR_ALIGN
    assert call(layers=[layer(0), layer(1, W_down=base + 0x10000000 + 0x9000002)]) == B.KQ_ERR_ALIGN
    assert call(layers=[layer(0, g_post=base + 0xF000004), layer(1)]) == B.KQ_ERR_ALIGN
    assert call(xo=R + 16) == B.KQ_ERR_ALIAS                      # x_out inside residual
    assert call(ge=XO) == B.KQ_ERR_ALIAS                          # g_entry is x_out
    assert call(ws=R - 256) == B.KQ_ERR_ALIAS                     # workspace covers residual
    assert call(r=base + q4b - 64) == B.KQ_ERR_ALIAS              # residual inside W_gate
    assert call(ws=base + 0x10000000 + 0x9000000 + q6b - 256) == B.KQ_ERR_ALIAS  # in W_down
    assert call(xo=base + 0xF100000 + 16) == B.KQ_ERR_ALIAS       # x_out inside g_next
    # every check passed: only the device is missing here
    assert call(ge=GE) in (B.KQ_ERR_DEVICE, B.KQ_ERR_LAUNCH, B.KQ_OK)
    assert call(n=1, layers=[layer(0)]) in (B.KQ_ERR_DEVICE, B.KQ_ERR_LAUNCH, B.KQ_OK)
    with pytest.raises(kq.KQError):
        kq.kq_ffn_pass_workspace_bytes(100, f)
    with pytest.raises(kq.KQError):
        kq.kq_ffn_pass_workspace_bytes(B.KQ_MAX_FUSED_TAIL_K + 256, f)
    t = kq.kq_ffn_layer_table([(1 << 20, 2 << 20, 3 << 20, 4 << 20, 5 << 20)])
    assert len(t) == 1 and t[0].W_down == 3 << 20 and t[0].g_next == 5 << 20


def test_small_m_path_switch_validation():
    assert kq.lib().kq_tune_set_small_m_rows(B.KQ_QTYPE_Q5K, 2) == B.KQ_ERR_SHAPE
    assert kq.lib().kq_tune_set_small_m_rows(B.KQ_QTYPE_Q4K, 5) == B.KQ_ERR_SHAPE
    assert kq.lib().kq_tune_set_small_m_rows(B.KQ_QTYPE_Q4K, -2) == B.KQ_ERR_SHAPE
    for qt in (B.KQ_QTYPE_Q4K, B.KQ_QTYPE_Q6K):
        for v in (0, 4, -1):
            assert kq.lib().kq_tune_set_small_m_rows(qt, v) == B.KQ_OK
    f = kq.lib().kq_tune_set_gate_up_rows
    assert f(-2) == B.KQ_ERR_SHAPE and f(5) == B.KQ_ERR_SHAPE
    for v in (0, 4, -1):
        assert f(v) == B.KQ_OK


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus 2 exits with status 2 and a message,
    before importing torch or touching a device, and prints no JSON line."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def test_profile_commands_run_committed_sections():
    """Every rocprofv3 command recorded under profiles/ runs bench.py with a
    section and flags bench.py accepts, and stays within one counter pass's
    limits (at most 8 SQ counters and 2 GRBM counters, no trace option with
    --pmc)."""
    import glob
    import re
    import shlex
    src = open(os.path.join(ROOT, "bench.py")).read()
    only = re.search(r'"--only", choices=\(([^)]*)\)', src, re.S).group(1)
    sections = set(re.findall(r'"([a-z_]+)"', only))
    cmds = []
    for path in glob.glob(os.path.join(ROOT, "profiles", "*")):
        for line in open(path):
            m = re.search(r"(rocprofv3 [^\"]*)", line)
            if m and "-- python3 bench.py" in m.group(1):
                cmds.append((os.path.basename(path), m.group(1).strip().rstrip('",')))
    assert cmds, "no recorded commands"
    for name, cmd in cmds:
        argv = shlex.split(cmd)
        prof, prog = argv[:argv.index("--")], argv[argv.index("--") + 1:]
        assert prog[:2] == ["python3", "bench.py"], (name, cmd)
        rest = prog[2:]
        assert rest[rest.index("--only") + 1] in sections, (name, cmd)
        allowed = {"--only", "--steps", "--warmup", "--calibration-copy"}
        assert {a for a in rest if a.startswith("--")} <= allowed, (name, cmd)
        if "--pmc" in prof:
            assert not {"-s", "--sys-trace", "-r", "--runtime-trace", "--kernel-trace"} & set(prof)
            counters = prof[prof.index("--pmc") + 1:]
            counters = counters[:next((i for i, c in enumerate(counters) if c.startswith("-")),
                                      len(counters))]
            assert sum(c.startswith("SQ_") for c in counters) <= 8, (name, cmd)
            assert sum(c.startswith("GRBM_") for c in counters) <= 2, (name, cmd)


def test_timed_kernels_use_no_private_memory():
    """The kernels of the timed pass keep every per-lane value in registers:
    their descriptors give no private (scratch) bytes, while a 16-wave,
    look-ahead-2 Q6_K form, which cannot fit its registers, does (so the
    descriptor reading is shown to see spills)."""
    import bench
    for part in bench.PMC_KERNELS.values():
        d = bench.kernel_descriptors(part)
        assert len(d) == 1, part
        (lds, private), = d.values()
        assert private == 0, f"{part}: {private} private bytes per lane"
    spilled = bench.kernel_descriptors("q6k_matvec_kernelILi8ELi3ELi2ELi16EE")
    assert len(spilled) == 1 and list(spilled.values())[0][1] > 0
