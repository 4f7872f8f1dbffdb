"""Helpers shared by the GPU tests: device buffers, the HIP calls through the
C ABI, and the tolerance checks.  The expected values always come from the
CPU oracle on the same seeded inputs."""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle
import quant_weight_matvec_amd as kq
from quant_weight_matvec_amd import inputs as I

NTHREADS = max(1, min(16, os.cpu_count() or 1))


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def nan_like(n, dtype=torch.float32) -> torch.Tensor:
    return torch.full((n,) if isinstance(n, int) else n, float("nan"), dtype=dtype, device="cuda")


def gpu_matvec(qt: str, Wd: torch.Tensor, xd: torch.Tensor, n: int, k: int,
               gate: torch.Tensor | None = None) -> np.ndarray:
    y = nan_like(n)
    if qt == "q4k":
        kq.kq_matvec_q4k(Wd, xd, y, n, k, gate)
    elif qt == "q5k":
        kq.kq_matvec_q5k(Wd, xd, y, n, k, gate)
    else:
        assert gate is None
        kq.kq_matvec_q6k(Wd, xd, y, n, k)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def assert_matvec_close(y_gpu, y_ref, S, tol=1e-3, what=""):
    """|y_gpu - y_ref| <= tol * S for every row (the matvec contract)."""
    y_gpu, y_ref, S = (np.asarray(a, np.float64) for a in (y_gpu, y_ref, S))
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output (unwritten row?)"
    err = np.abs(y_gpu - y_ref)
    bad = err > tol * S
    ratio = float(np.max(err / np.maximum(S, 1e-300))) if err.size else 0.0
    assert not bad.any(), (f"{what}: {int(bad.sum())} rows out of tolerance; "
                           f"worst |dy|/S = {ratio:.3e}")
    return ratio


def sample_rows(n: int, count: int, seed: int = 1234) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(n, size=min(count, n), replace=False).tolist())
    rows.update({0, n - 1})
    return np.array(sorted(rows))


def oracle_rows(qt: str, W: np.ndarray, x, rows: np.ndarray, k: int):
    """Oracle y and S for the selected rows only (W is the full [n, row_bytes])."""
    sub = np.ascontiguousarray(W[rows])
    return oracle.get().matvec(qt, sub, np.asarray(x, np.float64), len(rows), k,
                               nthreads=NTHREADS)


def weights(qt: str, n: int, k: int, stream: int) -> np.ndarray:
    return I.weight_matrix(qt, n, k, stream=stream)
