"""CPU oracle for the k-quant decode matvec path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It wraps ``kq_oracle.c`` (plain C,
IEEE binary64, written from "How to Write an Inference Engine -- the Muser
book"; each C function names the passage it follows) through ctypes.  It
shares no code with the HIP library in ``quant_weight_matvec_amd``.

Every function takes and returns numpy arrays.  Activations are accepted in
any float dtype and widened to float64 exactly; results are float64.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

QTYPE_Q4K = 1
QTYPE_Q6K = 2
QTYPE_Q5K = 3
_QT = {"q4k": QTYPE_Q4K, "q6k": QTYPE_Q6K, "q5k": QTYPE_Q5K, QTYPE_Q4K: QTYPE_Q4K,
       QTYPE_Q6K: QTYPE_Q6K, QTYPE_Q5K: QTYPE_Q5K}
BLOCK_BYTES = {QTYPE_Q4K: 144, QTYPE_Q6K: 210, QTYPE_Q5K: 176}

_LIBS: dict[int, C.CDLL] = {}
_dp = C.POINTER(C.c_double)
_u8p = C.POINTER(C.c_uint8)


def _load(plant: int = 0) -> C.CDLL:
    if plant in _LIBS:
        return _LIBS[plant]
    path = _build.lib_path(plant)
    if plant != 0 or not os.path.exists(path) or \
            os.path.getmtime(path) < os.path.getmtime(_build.SRC):
        _build.build(plant)
    lib = C.CDLL(path)
    lib.orc_f16_to_f64.restype = C.c_double
    lib.orc_f16_to_f64.argtypes = [C.c_uint16]
    lib.orc_dequant_rows.argtypes = [C.c_int, _u8p, C.c_int64, C.c_int64, _dp]
    lib.orc_matmul.argtypes = [C.c_int, _u8p, _dp, C.c_int64, C.c_int64, C.c_int64,
                               C.c_int64, _dp, _dp, C.c_int]
    lib.orc_silu_mul.argtypes = [_dp, _dp, C.c_int64, _dp]
    lib.orc_rms_norm.argtypes = [_dp, C.c_int64, C.c_double, _dp, _dp]
    lib.orc_dual_eps_tail.argtypes = [_dp, _dp, _dp, _dp, C.c_int64, C.c_int64,
                                      C.c_double, C.c_double, _dp]
    lib.orc_ffn_layer.argtypes = [C.c_int, _u8p, C.c_int, _u8p, C.c_int, _u8p,
                                  C.c_int64, C.c_int64, _dp, _dp, _dp, _dp,
                                  C.c_double, C.c_double, _dp,
                                  _dp, _dp, _dp, _dp, _dp, _dp, _dp, C.c_int]
    lib.orc_plant.restype = C.c_int
    _LIBS[plant] = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _u8(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.uint8))


def _p(a: np.ndarray, t=_dp):
    return a.ctypes.data_as(t)


class Oracle:
    """Bound to one build of the oracle library (plant 0 = the real oracle)."""

    def __init__(self, plant: int = 0):
        self.lib = _load(plant)
        self.plant = plant

    def f16_to_f64(self, bits: int) -> float:
        return self.lib.orc_f16_to_f64(int(bits) & 0xFFFF)

    def dequant(self, qtype, W, n_rows: int, k: int) -> np.ndarray:
        qt = _QT[qtype]
        W = _u8(W)
        if W.size != n_rows * (k // 256) * BLOCK_BYTES[qt] or k % 256:
            raise ValueError("weight byte count does not match the shape")
        out = np.empty((n_rows, k), np.float64)
        rc = self.lib.orc_dequant_rows(qt, _p(W, _u8p), n_rows, k, _p(out))
        if rc:
            raise ValueError(f"orc_dequant_rows rc={rc}")
        return out

    def embedding(self, qtype, E, tokens, vocab: int, hidden: int) -> np.ndarray:
        """Rows tokens[t] of the embedding table E (vocab rows of `hidden`
        weights, one token per row; the lookup of Ch 10 "The forward pass at a
        glance", section 10.3, box 1), dequantized: [len(tokens)][hidden].
        Tokens outside [0, vocab) give rows of NaN."""
        qt = _QT[qtype]
        E = _u8(E).reshape(vocab, -1)
        tok = np.asarray(tokens, np.int64).reshape(-1)
        out = np.full((tok.size, hidden), np.nan)
        ok = (tok >= 0) & (tok < vocab)
        if ok.any():
            out[ok] = self.dequant(qt, E[tok[ok]], int(ok.sum()), hidden)
        return out

    def matmul(self, qtype, W, X, n_rows: int, k: int, nthreads: int = 1):
        """Y[m][r] = sum_i w[r,i] X[m,i] and S[m][r] = sum_i |w[r,i] X[m,i]|."""
        qt = _QT[qtype]
        W = _u8(W)
        X = _f64(X)
        if X.ndim == 1:
            X = X.reshape(1, -1)
        m = X.shape[0]
        if X.shape[1] != k or W.size != n_rows * (k // 256) * BLOCK_BYTES[qt]:
            raise ValueError("shape mismatch")
        # NaN-filled, so a row the library failed to write cannot pass for a value
        Y = np.full((m, n_rows), np.nan)
        S = np.full((m, n_rows), np.nan)
        rc = self.lib.orc_matmul(qt, _p(W, _u8p), _p(X), k, n_rows, k, m, _p(Y), _p(S),
                                 int(nthreads))
        if rc:
            raise ValueError(f"orc_matmul rc={rc}")
        return Y, S

    def matvec(self, qtype, W, x, n_rows: int, k: int, nthreads: int = 1):
        Y, S = self.matmul(qtype, W, np.asarray(x).reshape(1, -1), n_rows, k, nthreads)
        return Y[0], S[0]

    def silu_mul(self, gate, up) -> np.ndarray:
        g, u = _f64(gate), _f64(up)
        out = np.empty_like(g)
        self.lib.orc_silu_mul(_p(g), _p(u), g.size, _p(out))
        return out

    def rms_norm(self, x, eps: float, gain=None) -> np.ndarray:
        x = _f64(x)
        out = np.empty_like(x)
        g = _f64(gain) if gain is not None else None
        self.lib.orc_rms_norm(_p(x), x.size, eps, _p(g) if g is not None else None, _p(out))
        return out

    def dual_eps_tail(self, residual, projected, g_post, g_next, eps_post: float = 1e-8,
                      eps_next: float = 1e-5):
        """Returns (residual_after_add, next_in); inputs are [rows][n] or [n]."""
        r = _f64(residual).copy()
        p = _f64(projected)
        shape = r.shape
        n = shape[-1]
        rows = r.size // n
        gp, gn = _f64(g_post), _f64(g_next)
        out = np.empty_like(r)
        self.lib.orc_dual_eps_tail(_p(r), _p(p), _p(gp), _p(gn), rows, n, eps_post,
                                   eps_next, _p(out))
        return r.reshape(shape), out.reshape(shape)

    def ffn_layer(self, Wg, Wu, Wd, hidden: int, ffn: int, x, residual, g_post, g_next,
                  qt_gate="q4k", qt_up="q4k", qt_down="q6k", eps_post: float = 1e-8,
                  eps_next: float = 1e-5, nthreads: int = 1) -> dict:
        Wg, Wu, Wd = _u8(Wg), _u8(Wu), _u8(Wd)
        x = _f64(x)
        r = _f64(residual).copy()
        gp, gn = _f64(g_post), _f64(g_next)
        out = {k: np.empty(ffn) for k in ("g", "u", "mid", "s_g", "s_u")}
        out.update({k: np.empty(hidden) for k in ("p", "s_p", "next_in")})
        rc = self.lib.orc_ffn_layer(_QT[qt_gate], _p(Wg, _u8p), _QT[qt_up], _p(Wu, _u8p),
                                    _QT[qt_down], _p(Wd, _u8p), hidden, ffn, _p(x), _p(r),
                                    _p(gp), _p(gn), eps_post, eps_next, _p(out["next_in"]),
                                    _p(out["g"]), _p(out["u"]), _p(out["mid"]), _p(out["p"]),
                                    _p(out["s_g"]), _p(out["s_u"]), _p(out["s_p"]),
                                    int(nthreads))
        if rc:
            raise ValueError(f"orc_ffn_layer rc={rc}")
        out["residual"] = r
        return out


_DEFAULT: Oracle | None = None


def get(plant: int = 0) -> Oracle:
    global _DEFAULT
    if plant:
        return Oracle(plant)
    if _DEFAULT is None:
        _DEFAULT = Oracle(0)
    return _DEFAULT
