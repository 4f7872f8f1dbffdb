"""Q5_K matvec and the embedding row lookup against the CPU oracle.

Q5_K (the pages name it among the pinned decode kernels, Ch 4 "Pipeline state
objects and the three kernel sources", section 4.4): the matvec contract
|dy| <= 1e-3 * sum |w x| per row at the FFN shapes (sampled rows), with the
SiLU epilogue, on a staged input (bit for bit the f32 result), and inside a
projection group.  The embedding lookup (Ch 10 "The forward pass at a
glance", section 10.3, box 1) is exact up to one f32 rounding per value, so
it must equal the oracle's binary64 rows rounded to f32 bit for bit, at the
full table size [202048 x 6656] and on ragged ones; tokens outside the
vocabulary give NaN rows.
"""
import numpy as np
import pytest
import torch

import oracle
import quant_weight_matvec_amd as kq
from quant_weight_matvec_amd import inputs as I
from gpu_util import assert_matvec_close, dev, gpu_matvec, nan_like, oracle_rows, sample_rows, weights

pytestmark = pytest.mark.gpu
O = oracle.get()
QT = {"q4k": kq.KQ_QTYPE_Q4K, "q5k": kq.KQ_QTYPE_Q5K, "q6k": kq.KQ_QTYPE_Q6K}


@pytest.mark.parametrize("n,k", [(19968, 6656), (6656, 19968), (202048, 6656)])
def test_q5k_full_size_sampled_rows(n, k):
    W = weights("q5k", n, k, 9100 + n)
    x = I.normal_f32(k, stream=9101)
    y = gpu_matvec("q5k", dev(W), dev(x), n, k)
    assert np.all(np.isfinite(y)), "unwritten rows"
    rows = sample_rows(n, 256, seed=n)
    yr, S = oracle_rows("q5k", W, x, rows, k)
    print("ratio", assert_matvec_close(y[rows], yr, S, what=f"q5k {n}x{k}"))


def test_q5k_silu_staged_and_group():
    n, k = 4097, 2816
    W = weights("q5k", n, k, 9200)
    x = I.normal_f32(k, stream=9201)
    g = I.normal_f32(n, stream=9202)
    Wd, xd, gd = dev(W), dev(x), dev(g)
    y = gpu_matvec("q5k", Wd, xd, n, k)
    ys = gpu_matvec("q5k", Wd, xd, n, k, gd)
    yr, S = oracle_rows("q5k", W, x, np.arange(n), k)
    assert_matvec_close(y, yr, S, what="q5k 4097x2816")
    gg = g.astype(np.float64)
    assert np.allclose(ys, gg / (1.0 + np.exp(-gg)) * y, rtol=1e-6, atol=1e-30), "SiLU epilogue"
    xs = torch.empty(kq.kq_staged_bytes(QT["q5k"], k), dtype=torch.uint8, device="cuda")
    kq.kq_stage_activation(QT["q5k"], xd, xs, k)
    yst = nan_like(n)
    kq.kq_matvec_staged(QT["q5k"], Wd, xs, yst, n, k)
    torch.cuda.synchronize()
    assert np.array_equal(yst.cpu().numpy().astype(np.float64), y), "staged input differs"
    # the same matrix split in two members of a group, and a third matrix
    W2 = weights("q5k", 300, k, 9203)
    ya, yb, yc = nan_like(1000), nan_like(n - 1000), nan_like(300)
    kq.kq_matvec_group(QT["q5k"], [Wd, Wd[1000:], dev(W2)], [ya, yb, yc], [1000, n - 1000, 300], xd, k)
    torch.cuda.synchronize()
    yg = np.concatenate([ya.cpu().numpy(), yb.cpu().numpy()]).astype(np.float64)
    assert_matvec_close(yg, yr, S, what="q5k group")
    y2r, S2 = oracle_rows("q5k", W2, x, np.arange(300), k)
    assert_matvec_close(yc.cpu().numpy().astype(np.float64), y2r, S2, what="q5k group member 3")


@pytest.mark.parametrize("qt", ["q4k", "q5k"])
@pytest.mark.parametrize("vocab,hidden,ntok", [(202048, 6656, 16), (37, 256, 40), (1000, 1280, 3)])
def test_embedding_rows_exact(qt, vocab, hidden, ntok):
    E = weights(qt, vocab, hidden, 9300 + vocab)
    tok = I.token_ids(ntok, vocab, stream=9301)
    tok[0], tok[-1] = 0, vocab - 1
    if ntok > 4:
        tok[1], tok[2] = -1, vocab  # outside the vocabulary: NaN rows
    out = nan_like((ntok, hidden))
    out.fill_(7.0)
    kq.kq_embedding(QT[qt], dev(E), vocab, hidden, dev(tok), ntok, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = O.embedding(qt, E, tok, vocab, hidden).astype(np.float32)
    assert np.array_equal(np.isnan(got), np.isnan(want)), "NaN rows differ"
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok]), "embedding values differ from the rounded oracle"


def test_small_m_rejects_q5k():
    with pytest.raises(kq.KQError):
        kq.kq_matmul_small_m_workspace_bytes(QT["q5k"], 64, 1024, 4)
