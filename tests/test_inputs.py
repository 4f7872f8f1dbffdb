"""The seeded input generator: determinism, random access, distributions.

CPU only.  The generator holds no arithmetic of the method; these checks make
sure both sides of every parity test see the same bytes and that the fields
follow the workload recipe.
"""
import numpy as np

from quant_weight_matvec_amd import inputs as I


def test_deterministic_and_stream_separated():
    a = I.q4k_matrix(300, 1024, stream=5)
    b = I.q4k_matrix(300, 1024, stream=5)
    c = I.q4k_matrix(300, 1024, stream=6)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)
    assert a.shape == (300, 4 * 144)


def test_row_range_regenerates_the_same_rows():
    full = I.q6k_matrix(700, 512, stream=9)
    part = I.q6k_matrix(700, 512, stream=9, row_lo=250, row_hi=613)
    assert np.array_equal(full[250:613], part)
    full4 = I.q4k_matrix(513, 256, stream=2)
    assert np.array_equal(full4[512:], I.q4k_matrix(513, 256, stream=2, row_lo=512))


def test_q4k_field_distributions():
    W = I.q4k_matrix(256, 4096, stream=1).reshape(-1, 144)
    d = W[:, 0:2].copy().view("<f2").astype(np.float64).ravel()
    dmin = W[:, 2:4].copy().view("<f2").astype(np.float64).ravel()
    for v in (d, dmin):
        assert v.min() >= 1e-3 - 1e-6 and v.max() <= 1e-2 + 1e-5
        assert abs(v.mean() - 5.5e-3) < 1e-4
    nib = np.concatenate([W[:, 16:] & 15, W[:, 16:] >> 4]).ravel()
    assert nib.max() == 15 and abs(nib.mean() - 7.5) < 0.05


def test_q6k_field_distributions():
    W = I.q6k_matrix(256, 4096, stream=1).reshape(-1, 210)
    sc = W[:, 192:208].copy().view(np.int8).ravel()
    assert sc.min() == -32 and sc.max() == 31
    d = W[:, 208:210].copy().view("<f2").astype(np.float64).ravel()
    assert d.min() >= 1e-3 - 1e-6 and d.max() <= 1e-2 + 1e-5


def test_vectors():
    x = I.normal_f32(100000, stream=3)
    assert x.dtype == np.float32 and abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02
    g = I.gains_f32(100000, stream=4)
    assert abs(g.mean() - 1) < 0.002 and abs(g.std() - 0.1) < 0.002
    assert np.array_equal(I.normal_f32((4, 8), stream=3).ravel(), I.normal_f32(32, stream=3))


def test_q5k_field_distributions():
    W = I.q5k_matrix(256, 4096, stream=1).reshape(-1, 176)
    assert np.array_equal(W.reshape(256, -1), I.q5k_matrix(256, 4096, stream=1))
    d = W[:, 0:2].copy().view("<f2").astype(np.float64).ravel()
    assert d.min() >= 1e-3 - 1e-6 and d.max() <= 1e-2 + 1e-5
    bits = np.unpackbits(W[:, 16:48].ravel())
    assert abs(bits.mean() - 0.5) < 0.01  # every high bit uniform
    nib = np.concatenate([W[:, 48:] & 15, W[:, 48:] >> 4]).ravel()
    assert nib.max() == 15 and abs(nib.mean() - 7.5) < 0.05


def test_token_ids():
    t = I.token_ids(100000, 202048, stream=7)
    assert t.dtype == np.int32 and t.min() >= 0 and t.max() < 202048
    assert np.array_equal(t, I.token_ids(100000, 202048, stream=7))
    assert abs(t.mean() / 202048 - 0.5) < 0.01
