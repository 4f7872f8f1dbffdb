"""Superblock encoder for the oracle's pins (tests only).

Packs explicit field values into superblock bytes, written in the encode
direction from the adopted layout reading (the pages give only the sizes,
Ch 19 "The down projection + residual", section 19.3, and the block idea,
Ch 5 "Quantization from scratch", section 5.5).  It is independent of the
oracle's decoder: a pin compares what the oracle decodes from these bytes with
what the test put into the fields.

Q4_K (144 B): d f16 @0, dmin f16 @2, 12 packed bytes @4 holding 6-bit scales
sc[0..7] and mins m[0..7], nibbles @16.  For s < 4: byte s bits 0-5 = sc[s],
byte s+4 bits 0-5 = m[s].  For s >= 4: byte s+4 low nibble = sc[s] bits 0-3,
high nibble = m[s] bits 0-3; byte s-4 bits 6-7 = sc[s] bits 4-5; byte s bits
6-7 = m[s] bits 4-5.  Nibble byte 16 + 32c + j: low nibble = weight 64c + j,
high nibble = weight 64c + 32 + j.

Q5_K (176 B): d f16 @0, dmin f16 @2, the 12 packed bytes of Q4_K @4, 32 bytes
of high bits @16, nibbles @48 laid out as Q4_K's @16.  Weight 64c + j (j < 32)
takes bit 2c of high-bit byte j, weight 64c + 32 + j bit 2c + 1.

Q6_K (210 B): ql @0 (128 B), qh @128 (64 B), int8 scales @192 (16), d f16 @208.
For half h and j < 32: weight 128h + j uses the low nibble of ql[64h + j] and
bits 0-1 of qh[32h + j]; weight 128h+32+j the low nibble of ql[64h+32+j] and
bits 2-3; weight 128h+64+j the high nibble of ql[64h+j] and bits 4-5; weight
128h+96+j the high nibble of ql[64h+32+j] and bits 6-7.
"""
from __future__ import annotations

import numpy as np


def f16_bits(v: float) -> int:
    return int(np.array([v], dtype="<f2").view("<u2")[0])


def f16_value(v: float) -> float:
    """The f16 rounding of v, as float64."""
    return float(np.float16(v))


def encode_q4k(d: float, dmin: float, sc, m, q) -> np.ndarray:
    sc = [int(v) for v in sc]
    m = [int(v) for v in m]
    q = np.asarray(q, dtype=np.int64).reshape(256)
    assert len(sc) == 8 and len(m) == 8
    assert all(0 <= v < 64 for v in sc + m) and q.min() >= 0 and q.max() < 16
    out = np.zeros(144, np.uint8)
    db, mb = f16_bits(d), f16_bits(dmin)
    out[0], out[1], out[2], out[3] = db & 255, db >> 8, mb & 255, mb >> 8
    P = [0] * 12
    for s in range(8):
        if s < 4:
            P[s] |= sc[s] & 63
            P[s + 4] |= m[s] & 63
        else:
            P[s + 4] |= (sc[s] & 15) | ((m[s] & 15) << 4)
            P[s - 4] |= (sc[s] >> 4) << 6
            P[s] |= (m[s] >> 4) << 6
    out[4:16] = P
    for c in range(4):
        for j in range(32):
            lo = q[64 * c + j]
            hi = q[64 * c + 32 + j]
            out[16 + 32 * c + j] = lo | (hi << 4)
    return out


def encode_q5k(d: float, dmin: float, sc, m, q) -> np.ndarray:
    q = np.asarray(q, dtype=np.int64).reshape(256)
    assert q.min() >= 0 and q.max() < 32
    q4 = encode_q4k(d, dmin, sc, m, q & 15)  # header and nibbles as in Q4_K
    out = np.zeros(176, np.uint8)
    out[0:16] = q4[0:16]
    out[48:176] = q4[16:144]
    for c in range(4):
        for j in range(32):
            out[16 + j] |= (q[64 * c + j] >> 4) << (2 * c)
            out[16 + j] |= (q[64 * c + 32 + j] >> 4) << (2 * c + 1)
    return out


def encode_q6k(d: float, sc, q) -> np.ndarray:
    sc = [int(v) for v in sc]
    q = np.asarray(q, dtype=np.int64).reshape(256)
    assert len(sc) == 16 and all(-128 <= v < 128 for v in sc)
    assert q.min() >= 0 and q.max() < 64
    out = np.zeros(210, np.uint8)
    for h in range(2):
        for j in range(32):
            q0 = q[128 * h + j]
            q1 = q[128 * h + 32 + j]
            q2 = q[128 * h + 64 + j]
            q3 = q[128 * h + 96 + j]
            out[64 * h + j] = (q0 & 15) | ((q2 & 15) << 4)
            out[64 * h + 32 + j] = (q1 & 15) | ((q3 & 15) << 4)
            out[128 + 32 * h + j] = (q0 >> 4) | ((q1 >> 4) << 2) | ((q2 >> 4) << 4) | ((q3 >> 4) << 6)
    out[192:208] = np.array(sc, dtype=np.int8).view(np.uint8)
    db = f16_bits(d)
    out[208], out[209] = db & 255, db >> 8
    return out


def dense_q4k(d: float, dmin: float, sc, m, q) -> np.ndarray:
    """Weight values of one Q4_K superblock straight from its fields."""
    d, dmin = f16_value(d), f16_value(dmin)
    q = np.asarray(q, np.float64).reshape(256)
    s = np.arange(256) // 32
    return d * np.asarray(sc, np.float64)[s] * q - dmin * np.asarray(m, np.float64)[s]


def dense_q5k(d: float, dmin: float, sc, m, q) -> np.ndarray:
    """Weight values of one Q5_K superblock straight from its fields (the same
    formula as Q4_K with 5-bit quants)."""
    return dense_q4k(d, dmin, sc, m, q)


def dense_q6k(d: float, sc, q) -> np.ndarray:
    d = f16_value(d)
    q = np.asarray(q, np.float64).reshape(256)
    s = np.arange(256) // 16
    return d * np.asarray(sc, np.float64)[s] * (q - 32.0)


def random_q4k_fields(rng: np.random.Generator):
    return dict(d=float(rng.uniform(1e-3, 1e-2)), dmin=float(rng.uniform(1e-3, 1e-2)),
                sc=rng.integers(0, 64, 8), m=rng.integers(0, 64, 8), q=rng.integers(0, 16, 256))


def random_q6k_fields(rng: np.random.Generator):
    return dict(d=float(rng.uniform(1e-3, 1e-2)), sc=rng.integers(-32, 32, 16),
                q=rng.integers(0, 64, 256))


def random_q5k_fields(rng: np.random.Generator):
    return dict(d=float(rng.uniform(1e-3, 1e-2)), dmin=float(rng.uniform(1e-3, 1e-2)),
                sc=rng.integers(0, 64, 8), m=rng.integers(0, 64, 8), q=rng.integers(0, 32, 256))
