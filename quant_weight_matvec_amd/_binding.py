"""ctypes binding of libkq (include/kq.h): argument marshalling only.

Every computation runs in the HIP kernels of ``libkq.so``; this module only
turns tensors into device pointers and streams into handles, and turns a
non-zero status into an exception.  There is no fallback: if the built
library is missing, importing the functions raises ``KQLibraryMissing``.

Pointer arguments accept a ``torch.Tensor`` (its ``data_ptr()``), a plain
integer address, or ``None`` (NULL).  ``stream`` accepts a
``torch.cuda.Stream``, a raw handle, or ``None`` for torch's current stream.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkq.so")

KQ_OK = 0
KQ_ERR_NULL = -1
KQ_ERR_SHAPE = -2
KQ_ERR_ALIGN = -3
KQ_ERR_ALIAS = -4
KQ_ERR_UNSUPPORTED = -5
KQ_ERR_LAUNCH = -6
KQ_ERR_DEVICE = -7
KQ_QTYPE_Q4K = 1
KQ_QTYPE_Q6K = 2
KQ_QTYPE_Q5K = 3
KQ_MAX_K = 40960
KQ_MAX_M = 16
KQ_MAX_TAIL_N = 32768
KQ_MAX_GROUP = 4
KQ_SMALL_M_SCRATCH_BYTES = 16 * 1024 + 16 * 1024 * 1024
KQ_MAX_FUSED_TAIL_K = 8192


class KQLibraryMissing(RuntimeError):
    pass


class KQError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class KqFfnLayer(C.Structure):
    """kq_ffn_layer: device pointers of one layer's matrices and tail gains."""
    _fields_ = [("W_gate", C.c_void_p), ("W_up", C.c_void_p), ("W_down", C.c_void_p),
                ("g_post", C.c_void_p), ("g_next", C.c_void_p)]


_lib: C.CDLL | None = None
_vp = C.c_void_p
_i64 = C.c_int64


def lib() -> C.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise KQLibraryMissing(
            f"{LIB_PATH} is not built; run `python -m quant_weight_matvec_amd.build` "
            "(there is no CPU fallback)")
    L = C.CDLL(LIB_PATH)
    L.kq_matvec_q4k.argtypes = [_vp, _vp, _vp, _i64, _i64, _vp, _vp]
    L.kq_matvec_q6k.argtypes = [_vp, _vp, _vp, _i64, _i64, _vp]
    L.kq_matvec_q5k.argtypes = [_vp, _vp, _vp, _i64, _i64, _vp, _vp]
    L.kq_embedding.argtypes = [C.c_int, _vp, _i64, _i64, _vp, _i64, _vp, _vp]
    L.kq_matvec_group.argtypes = [C.c_int, C.c_int, _vp, _vp, _vp, _vp, _i64, _vp]
    L.kq_matvec_group_staged.argtypes = [C.c_int, C.c_int, _vp, _vp, _vp, _vp, _i64, _vp]
    L.kq_ffn_gate_up_q4k.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _vp]
    L.kq_matmul_small_m.argtypes = [C.c_int, _vp, _vp, _i64, _vp, _i64, _i64, _i64, C.c_int, _vp,
                                    _i64, _vp]
    L.kq_ffn_gate_up_q4k_small_m.argtypes = [_vp, _vp, _vp, _i64, _vp, _i64, _i64, _i64, C.c_int,
                                             _vp, _i64, _vp]
    L.kq_matmul_small_m_noalloc.argtypes = [C.c_int, _vp, _vp, _i64, _vp, _i64, _i64, _i64,
                                            C.c_int, _vp]
    L.kq_matmul_small_m_workspace_bytes.argtypes = [C.c_int, _i64, _i64, C.c_int]
    L.kq_matmul_small_m_workspace_bytes.restype = _i64
    L.kq_fused_residual_norm.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, C.c_float,
                                         C.c_float, _vp]
    L.kq_status_string.argtypes = [C.c_int]
    L.kq_status_string.restype = C.c_char_p
    L.kq_build_info.argtypes = []
    L.kq_build_info.restype = C.c_char_p
    L.kq_last_hip_error.argtypes = []
    L.kq_last_hip_error.restype = C.c_char_p
    L.kq_tune_set_shape.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int, C.c_int]
    L.kq_tune_get_shape.argtypes = [C.c_int, _i64, _i64, C.POINTER(C.c_int),
                                    C.POINTER(C.c_int), C.POINTER(C.c_int), C.POINTER(C.c_int)]
    L.kq_probe_read_bw.argtypes = [_vp, _i64, _vp, C.c_int, C.c_int, C.c_int, C.c_int, _vp]
    L.kq_tune_small_m_plan.argtypes = [C.c_int, _i64, _i64, C.c_int, C.c_int, _vp]
    L.kq_tune_matvec_plan.argtypes = [C.c_int, _i64, _i64, C.c_int, C.c_int, _vp]
    L.kq_staged_bytes.argtypes = [C.c_int, _i64]
    L.kq_staged_bytes.restype = _i64
    L.kq_stage_activation.argtypes = [C.c_int, _vp, _vp, _i64, _vp]
    L.kq_matvec_staged.argtypes = [C.c_int, _vp, _vp, _vp, _i64, _i64, _vp, _vp]
    L.kq_ffn_gate_up_q4k_staged.argtypes = [_vp, _vp, _vp, _vp, _vp, C.c_int, _i64, _i64, _vp]
    L.kq_fused_residual_norm_staged.argtypes = [_vp, _vp, _vp, _vp, C.c_int, _vp, _vp, _i64, _i64,
                                                C.c_float, C.c_float, _vp]
    L.kq_ffn_tail_gate_up_q4k.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                          C.c_int, _i64, _i64, C.c_float, C.c_float, _vp]
    L.kq_ffn_pass_q4k_q6k.argtypes = [C.POINTER(KqFfnLayer), C.c_int, _vp, _vp, _vp, _vp, _i64,
                                      _i64, _i64, C.c_float, C.c_float, _vp]
    L.kq_ffn_pass_workspace_bytes.argtypes = [_i64, _i64]
    L.kq_ffn_pass_workspace_bytes.restype = _i64
    L.kq_tune_set_small_m_rows.argtypes = [C.c_int, C.c_int]
    L.kq_tune_set_gate_up_rows.argtypes = [C.c_int]
    for fn in ("kq_ffn_pass_q4k_q6k", "kq_tune_set_small_m_rows", "kq_tune_set_gate_up_rows", "kq_stage_activation", "kq_matvec_staged", "kq_ffn_gate_up_q4k_staged",
               "kq_ffn_tail_gate_up_q4k",
               "kq_fused_residual_norm_staged",
               "kq_tune_small_m_plan", "kq_tune_matvec_plan",
               "kq_probe_read_bw", "kq_matvec_q4k", "kq_matvec_q6k", "kq_matvec_group",
               "kq_matvec_q5k", "kq_embedding",
               "kq_matvec_group_staged", "kq_ffn_gate_up_q4k", "kq_matmul_small_m", "kq_matmul_small_m_noalloc", "kq_ffn_gate_up_q4k_small_m", "kq_fused_residual_norm",
               "kq_tune_set_shape", "kq_tune_get_shape"):
        getattr(L, fn).restype = C.c_int
    _lib = L
    return L


def _ptr(a) -> int | None:
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(s) -> int | None:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(rc: int, what: str) -> None:
    if rc != KQ_OK:
        detail = f" ({lib().kq_last_hip_error().decode()})" if rc == KQ_ERR_LAUNCH else ""
        raise KQError(rc, f"{what}: {kq_status_string(rc)}{detail}")


def kq_status_string(status: int) -> str:
    return lib().kq_status_string(int(status)).decode()


def kq_build_info() -> str:
    return lib().kq_build_info().decode()


def kq_matvec_q4k(W, x, y, n_rows: int, k: int, silu_gate=None, stream=None) -> None:
    rc = lib().kq_matvec_q4k(_ptr(W), _ptr(x), _ptr(y), int(n_rows), int(k), _ptr(silu_gate),
                             _stream(stream))
    _check(rc, "kq_matvec_q4k")


def kq_matvec_q5k(W, x, y, n_rows: int, k: int, silu_gate=None, stream=None) -> None:
    rc = lib().kq_matvec_q5k(_ptr(W), _ptr(x), _ptr(y), int(n_rows), int(k), _ptr(silu_gate),
                             _stream(stream))
    _check(rc, "kq_matvec_q5k")


def kq_embedding(qtype: int, E, vocab: int, hidden: int, tokens, n_tokens: int, out,
                 stream=None) -> None:
    rc = lib().kq_embedding(int(qtype), _ptr(E), int(vocab), int(hidden), _ptr(tokens),
                            int(n_tokens), _ptr(out), _stream(stream))
    _check(rc, "kq_embedding")


def kq_ffn_gate_up_q4k(W_gate, W_up, x, mid, n_rows: int, k: int, stream=None) -> None:
    rc = lib().kq_ffn_gate_up_q4k(_ptr(W_gate), _ptr(W_up), _ptr(x), _ptr(mid), int(n_rows),
                                  int(k), _stream(stream))
    _check(rc, "kq_ffn_gate_up_q4k")


def kq_matvec_q6k(W, x, y, n_rows: int, k: int, stream=None) -> None:
    rc = lib().kq_matvec_q6k(_ptr(W), _ptr(x), _ptr(y), int(n_rows), int(k), _stream(stream))
    _check(rc, "kq_matvec_q6k")


def _group_args(W, y, n_rows):
    n = len(W)
    if len(y) != n or len(n_rows) != n:
        raise ValueError("W, y and n_rows need one entry per matrix")
    Wa = (C.c_void_p * max(n, 1))(*[_ptr(w) for w in W])
    ya = (C.c_void_p * max(n, 1))(*[_ptr(v) for v in y])
    na = (C.c_int64 * max(n, 1))(*[int(r) for r in n_rows])
    return n, Wa, ya, na


def kq_matvec_group(qtype: int, W, y, n_rows, x, k: int, stream=None) -> None:
    """W, y, n_rows: sequences (one entry per matrix) of weights, outputs and row counts."""
    n, Wa, ya, na = _group_args(W, y, n_rows)
    rc = lib().kq_matvec_group(int(qtype), n, C.cast(Wa, C.c_void_p), C.cast(ya, C.c_void_p),
                               C.cast(na, C.c_void_p), _ptr(x), int(k), _stream(stream))
    _check(rc, "kq_matvec_group")


def kq_matvec_group_staged(qtype: int, W, y, n_rows, xs, k: int, stream=None) -> None:
    n, Wa, ya, na = _group_args(W, y, n_rows)
    rc = lib().kq_matvec_group_staged(int(qtype), n, C.cast(Wa, C.c_void_p),
                                      C.cast(ya, C.c_void_p), C.cast(na, C.c_void_p), _ptr(xs),
                                      int(k), _stream(stream))
    _check(rc, "kq_matvec_group_staged")


def kq_matmul_small_m(qtype: int, W, X, ldx: int, Y, ldy: int, n_rows: int, k: int, m: int,
                      workspace=None, workspace_bytes: int = 0, stream=None) -> None:
    rc = lib().kq_matmul_small_m(int(qtype), _ptr(W), _ptr(X), int(ldx), _ptr(Y), int(ldy),
                                 int(n_rows), int(k), int(m), _ptr(workspace),
                                 int(workspace_bytes), _stream(stream))
    _check(rc, "kq_matmul_small_m")


def kq_ffn_gate_up_q4k_small_m(W_gate, W_up, X, ldx: int, Mid, ldm: int, n_rows: int, k: int,
                               m: int, workspace=None, workspace_bytes: int = 0,
                               stream=None) -> None:
    rc = lib().kq_ffn_gate_up_q4k_small_m(_ptr(W_gate), _ptr(W_up), _ptr(X), int(ldx), _ptr(Mid),
                                          int(ldm), int(n_rows), int(k), int(m), _ptr(workspace),
                                          int(workspace_bytes), _stream(stream))
    _check(rc, "kq_ffn_gate_up_q4k_small_m")


def kq_matmul_small_m_noalloc(qtype: int, W, X, ldx: int, Y, ldy: int, n_rows: int, k: int,
                              m: int, stream=None) -> None:
    rc = lib().kq_matmul_small_m_noalloc(int(qtype), _ptr(W), _ptr(X), int(ldx), _ptr(Y),
                                         int(ldy), int(n_rows), int(k), int(m), _stream(stream))
    _check(rc, "kq_matmul_small_m_noalloc")


def kq_matmul_small_m_workspace_bytes(qtype: int, n_rows: int, k: int, m: int) -> int:
    """Bytes of workspace kq_matmul_small_m needs (0 = none); raises KQError
    for arguments the call would reject."""
    n = int(lib().kq_matmul_small_m_workspace_bytes(int(qtype), int(n_rows), int(k), int(m)))
    if n < 0:
        _check(n, "kq_matmul_small_m_workspace_bytes")
    return n


def kq_fused_residual_norm(residual, projected, next_in, g_post, g_next, rows: int, n: int,
                           eps_post: float = 1e-8, eps_next: float = 1e-5, stream=None) -> None:
    rc = lib().kq_fused_residual_norm(_ptr(residual), _ptr(projected), _ptr(next_in),
                                      _ptr(g_post), _ptr(g_next), int(rows), int(n),
                                      float(eps_post), float(eps_next), _stream(stream))
    _check(rc, "kq_fused_residual_norm")


def kq_staged_bytes(qtype: int, k: int) -> int:
    n = int(lib().kq_staged_bytes(int(qtype), int(k)))
    if n < 0:
        _check(n, "kq_staged_bytes")
    return n


def kq_stage_activation(qtype: int, x, xs, k: int, stream=None) -> None:
    rc = lib().kq_stage_activation(int(qtype), _ptr(x), _ptr(xs), int(k), _stream(stream))
    _check(rc, "kq_stage_activation")


def kq_matvec_staged(qtype: int, W, xs, y, n_rows: int, k: int, silu_gate=None,
                     stream=None) -> None:
    rc = lib().kq_matvec_staged(int(qtype), _ptr(W), _ptr(xs), _ptr(y), int(n_rows), int(k),
                                _ptr(silu_gate), _stream(stream))
    _check(rc, "kq_matvec_staged")


def kq_ffn_gate_up_q4k_staged(W_gate, W_up, xs, mid, mid_s, mid_qtype: int, n_rows: int, k: int,
                              stream=None) -> None:
    rc = lib().kq_ffn_gate_up_q4k_staged(_ptr(W_gate), _ptr(W_up), _ptr(xs), _ptr(mid),
                                         _ptr(mid_s), int(mid_qtype), int(n_rows), int(k),
                                         _stream(stream))
    _check(rc, "kq_ffn_gate_up_q4k_staged")


def kq_fused_residual_norm_staged(residual, projected, next_in, next_in_s, next_qtype: int,
                                  g_post, g_next, rows: int, n: int, eps_post: float = 1e-8,
                                  eps_next: float = 1e-5, stream=None) -> None:
    rc = lib().kq_fused_residual_norm_staged(_ptr(residual), _ptr(projected), _ptr(next_in),
                                             _ptr(next_in_s), int(next_qtype), _ptr(g_post),
                                             _ptr(g_next), int(rows), int(n), float(eps_post),
                                             float(eps_next), _stream(stream))
    _check(rc, "kq_fused_residual_norm_staged")


def kq_ffn_tail_gate_up_q4k(residual_in, projected, g_post, g_next, residual_out, next_in,
                            W_gate, W_up, mid, mid_s, mid_qtype: int, n_rows: int, k: int,
                            eps_post: float = 1e-8, eps_next: float = 1e-5, stream=None) -> None:
    rc = lib().kq_ffn_tail_gate_up_q4k(_ptr(residual_in), _ptr(projected), _ptr(g_post),
                                       _ptr(g_next), _ptr(residual_out), _ptr(next_in),
                                       _ptr(W_gate), _ptr(W_up), _ptr(mid), _ptr(mid_s),
                                       int(mid_qtype), int(n_rows), int(k), float(eps_post),
                                       float(eps_next), _stream(stream))
    _check(rc, "kq_ffn_tail_gate_up_q4k")


def kq_ffn_layer_table(layers):
    """The host array of kq_ffn_layer records kq_ffn_pass_q4k_q6k reads:
    `layers` is a sequence of (W_gate, W_up, W_down, g_post, g_next) tensors
    or addresses, in layer order."""
    recs = []
    for rec in layers:
        if len(rec) != 5:
            raise ValueError("each layer is (W_gate, W_up, W_down, g_post, g_next)")
        recs.append(KqFfnLayer(*[_ptr(t) for t in rec]))
    return (KqFfnLayer * len(recs))(*recs)


def kq_ffn_pass_workspace_bytes(hidden: int, ffn: int) -> int:
    """Bytes of workspace kq_ffn_pass_q4k_q6k needs; raises KQError for
    shapes it would reject."""
    n = lib().kq_ffn_pass_workspace_bytes(int(hidden), int(ffn))
    if n < 0:
        _check(int(n), "kq_ffn_pass_workspace_bytes")
    return int(n)


def kq_ffn_pass_q4k_q6k(layers, residual, x_out, g_entry, workspace, workspace_bytes: int,
                        hidden: int, ffn: int, eps_post: float = 1e-8, eps_next: float = 1e-5,
                        stream=None) -> None:
    """`layers`: a kq_ffn_layer_table array, or a sequence of
    (W_gate, W_up, W_down, g_post, g_next) per layer."""
    table = layers if isinstance(layers, C.Array) else kq_ffn_layer_table(layers)
    rc = lib().kq_ffn_pass_q4k_q6k(table, len(table), _ptr(residual), _ptr(x_out), _ptr(g_entry),
                                   _ptr(workspace), int(workspace_bytes), int(hidden), int(ffn),
                                   float(eps_post), float(eps_next), _stream(stream))
    _check(rc, "kq_ffn_pass_q4k_q6k")


def kq_tune_set_small_m_rows(qtype: int, max_m: int = -1) -> None:
    _check(lib().kq_tune_set_small_m_rows(int(qtype), int(max_m)), "kq_tune_set_small_m_rows")


def kq_tune_set_gate_up_rows(max_m: int = -1) -> None:
    _check(lib().kq_tune_set_gate_up_rows(int(max_m)), "kq_tune_set_gate_up_rows")


def kq_tune_set_shape(qtype: int, lanes: int = 0, waves: int = 0, grid: int = 0,
                      depth: int = 0) -> None:
    _check(lib().kq_tune_set_shape(int(qtype), int(lanes), int(waves), int(grid), int(depth)),
           "kq_tune_set_shape")


def kq_tune_get_shape(qtype: int, n_rows: int, k: int) -> tuple[int, int, int, int]:
    a, b, c, d = C.c_int(), C.c_int(), C.c_int(), C.c_int()
    _check(lib().kq_tune_get_shape(int(qtype), int(n_rows), int(k), C.byref(a), C.byref(b),
                                   C.byref(c), C.byref(d)), "kq_tune_get_shape")
    return a.value, b.value, c.value, d.value


def kq_probe_read_bw(buf, nbytes: int, out, grid: int, block: int = 256, unroll: int = 8,
                     flags: int = 1, stream=None) -> None:
    _check(lib().kq_probe_read_bw(_ptr(buf), int(nbytes), _ptr(out), int(grid), int(block),
                                  int(unroll), int(flags), _stream(stream)), "kq_probe_read_bw")


def kq_tune_matvec_plan(qtype: int, n_rows: int, k: int, staged: bool, cus: int) -> dict:
    """The automatic M = 1 matvec launch shape on a device of `cus` CUs (host arithmetic)."""
    out = (C.c_int64 * 6)()
    _check(lib().kq_tune_matvec_plan(int(qtype), int(n_rows), int(k), int(bool(staged)), int(cus),
                                     C.cast(out, C.c_void_p)), "kq_tune_matvec_plan")
    return dict(zip(("lanes", "waves", "grid", "depth", "lds", "per_cu"), out))


def kq_tune_small_m_plan(qtype: int, n_rows: int, k: int, m: int, cus: int) -> dict:
    """The small-M launch plan on a device of `cus` CUs (host arithmetic)."""
    out = (C.c_int64 * 6)()
    _check(lib().kq_tune_small_m_plan(int(qtype), int(n_rows), int(k), int(m), int(cus),
                                      C.cast(out, C.c_void_p)), "kq_tune_small_m_plan")
    return dict(zip(("grid", "window", "lds", "workspace", "threads", "tiles"), out))
