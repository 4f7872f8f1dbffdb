"""The other decode matvec shapes of a layer and the LM head against the CPU
oracle (Ch 10 "The forward pass at a glance", section 10.3, master diagram):
the attention projections Q [6656->4096], K and V [6656->256] and the output
gate [6656->4096] (one group on one input, box 4), o_proj [4096->6656] (box 9)
and the LM head [6656->202048] (box 14), in Q4_K and in Q6_K (the pages do not
give the weight types of these matrices).  Full-size outputs are all checked
for being written; rows are compared with the oracle in full where the oracle
is quick and on samples (first, last and random rows) for the LM head.
"""
import numpy as np
import pytest
import torch

import quant_weight_matvec_amd as kq
from quant_weight_matvec_amd import inputs as I
from gpu_util import (assert_matvec_close, dev, gpu_matvec, nan_like, oracle_rows, sample_rows,
                      weights)

pytestmark = pytest.mark.gpu
QT = {"q4k": kq.KQ_QTYPE_Q4K, "q6k": kq.KQ_QTYPE_Q6K}
HIDDEN, QDIM, KVDIM, VOCAB = 6656, 4096, 256, 202048


def group(qt, mats, x, k, staged=False):
    """kq_matvec_group over [(W device tensor, rows)]; returns the outputs."""
    ys = [nan_like(n) for _, n in mats]
    if staged:
        xs = torch.empty(kq.kq_staged_bytes(QT[qt], k), dtype=torch.uint8, device="cuda")
        kq.kq_stage_activation(QT[qt], x, xs, k)
        kq.kq_matvec_group_staged(QT[qt], [w for w, _ in mats], ys, [n for _, n in mats], xs, k)
    else:
        kq.kq_matvec_group(QT[qt], [w for w, _ in mats], ys, [n for _, n in mats], x, k)
    torch.cuda.synchronize()
    return [y.cpu().numpy().astype(np.float64) for y in ys]


@pytest.mark.parametrize("qt", ["q4k", "q6k"])
def test_qkvg_group_full_size(qt):
    """Q, K, V and gate in one launch on one input: every row of K and V and
    sampled rows of Q and gate against the oracle; the staged input gives the
    same bits."""
    k = HIDDEN
    shapes = [("q", QDIM), ("k", KVDIM), ("v", KVDIM), ("g", QDIM)]
    Ws = [weights(qt, n, k, 9500 + i) for i, (_, n) in enumerate(shapes)]
    x = I.normal_f32(k, stream=9510)
    xd = dev(x)
    mats = [(dev(W), n) for W, (_, n) in zip(Ws, shapes)]
    ys = group(qt, mats, xd, k)
    ys_st = group(qt, mats, xd, k, staged=True)
    for (name, n), W, y, yst in zip(shapes, Ws, ys, ys_st):
        assert np.all(np.isfinite(y)), f"{name}: unwritten rows"
        assert np.array_equal(y, yst), f"{name}: staged input differs"
        rows = np.arange(n) if n <= KVDIM else sample_rows(n, 256, seed=n)
        yr, S = oracle_rows(qt, W, x, rows, k)
        assert_matvec_close(y[rows], yr, S, what=f"{qt} {name} [{k}->{n}] in the group")


@pytest.mark.parametrize("qt", ["q4k", "q6k"])
@pytest.mark.parametrize("n,k", [(KVDIM, HIDDEN), (QDIM, HIDDEN), (HIDDEN, QDIM)])
def test_single_decode_shapes_all_rows(qt, n, k):
    """K or V alone [6656->256], Q alone [6656->4096], o_proj [4096->6656]:
    every row against the oracle."""
    W = weights(qt, n, k, 9600 + n + k)
    x = I.normal_f32(k, stream=9601 + n)
    y = gpu_matvec(qt, dev(W), dev(x), n, k)
    yr, S = oracle_rows(qt, W, x, np.arange(n), k)
    print("worst |dy|/S", assert_matvec_close(y, yr, S, what=f"{qt} {n}x{k}"))


@pytest.mark.parametrize("qt", ["q4k", "q6k"])
def test_lm_head_full_size_sampled_rows(qt):
    """The LM head [6656->202048] (756 MB of Q4_K, 1.1 GB of Q6_K): all rows
    written, sampled rows against the oracle."""
    n, k = VOCAB, HIDDEN
    W = weights(qt, n, k, 9700)
    x = I.normal_f32(k, stream=9701)
    y = gpu_matvec(qt, dev(W), dev(x), n, k)
    assert np.all(np.isfinite(y))
    rows = sample_rows(n, 400, seed=9702)
    yr, S = oracle_rows(qt, W, x, rows, k)
    print("worst |dy|/S", assert_matvec_close(y[rows], yr, S, what=f"{qt} LM head"))
    del W


@pytest.mark.parametrize("qt", ["q4k", "q6k"])
def test_group_ragged_and_empty_members(qt):
    """Row counts that straddle tiles and workgroups, an empty member, and a
    one-member group equal to the plain matvec bit for bit."""
    k = 1280
    counts = [37, 0, 300, 5]
    Ws = [weights(qt, n, k, 9800 + i) for i, n in enumerate(counts)]
    x = I.normal_f32(k, stream=9810)
    xd = dev(x)
    mats = [(dev(W) if n else torch.empty(16, dtype=torch.uint8, device="cuda"), n)
            for W, n in zip(Ws, counts)]
    ys = group(qt, mats, xd, k)
    for W, n, y in zip(Ws, counts, ys):
        if n == 0:
            continue
        yr, S = oracle_rows(qt, W, x, np.arange(n), k)
        assert_matvec_close(y, yr, S, what=f"{qt} group member of {n} rows")
    one = group(qt, mats[2:3], xd, k)[0]
    assert np.array_equal(one, gpu_matvec(qt, mats[2][0], xd, 300, k))


def test_group_rejects_overlapping_outputs():
    k, n = 512, 64
    W = dev(weights("q4k", n, k, 9900))
    x = dev(I.normal_f32(k, stream=9901))
    y = nan_like(2 * n)
    with pytest.raises(kq.KQError):
        kq.kq_matvec_group(QT["q4k"], [W, W], [y, y[8:]], [n, n], x, k)
