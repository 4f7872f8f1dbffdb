"""Seeded synthetic inputs for the k-quant decode matvec path.

This module is the only code shared by the CPU oracle's tests and the GPU
path.  It draws random bytes and random floats and writes them into the
superblock field positions; it holds none of the method's arithmetic (no
dequantization, no dot products, no norms).

Workload recipe (distributions follow the pages' ffn shapes, Ch 19 "The down
projection + residual", section 19.3, and Ch 5 "Quantization from scratch",
section 5.5 for the block idea):

* Q4_K superblock, 144 bytes: bytes 0-1 ``d`` and 2-3 ``dmin`` are f16 drawn
  from U[1e-3, 1e-2] (rounded to nearest-even f16); bytes 4-15 (the packed
  6-bit scales and mins) and 16-143 (the 4-bit quants) are uniform random
  bytes, which makes every 6-bit field uniform on 0..63 and every nibble
  uniform on 0..15.
* Q5_K superblock, 176 bytes: bytes 0-3 ``d`` and ``dmin`` as for Q4_K; bytes
  4-175 (packed 6-bit scales and mins, the high bits, the low nibbles) are
  uniform random bytes, which makes every 5-bit quant uniform on 0..31.
* Q6_K superblock, 210 bytes: bytes 0-191 (low 4 bits and high 2 bits of the
  quants) are uniform random bytes; bytes 192-207 are int8 scales uniform on
  -32..31; bytes 208-209 ``d`` is f16 from U[1e-3, 1e-2].
* Activations are f32 N(0, 1); norm gains are f32 N(1, 0.1).

Generators: numpy ``SFC64`` (Doty-Humphrey's small fast chaotic generator),
one instance per (seed, stream, block of 256 rows) seeded through numpy's
``SeedSequence``.  Any 256-row block can be regenerated alone, which lets a
test rebuild sampled rows of a full-size matrix without holding the rest, and
lets the blocks be drawn in parallel threads with identical results.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BASE_SEED = 0x4B514D56  # "KQMV"
QK = 256
Q4K_BLOCK_BYTES = 144
Q6K_BLOCK_BYTES = 210
Q5K_BLOCK_BYTES = 176
ROW_BLOCK = 256  # rows per independently seeded generator

# roles inside one configuration (stream = cfg << 24 | layer << 8 | role)
ROLE_W_GATE, ROLE_W_UP, ROLE_W_DOWN, ROLE_X, ROLE_RESID, ROLE_GPOST, ROLE_GNEXT, ROLE_W = range(8)


def stream_id(cfg: int, layer: int, role: int) -> int:
    return (cfg << 24) | (layer << 8) | role


def _rng(seed: int, stream: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.SFC64(np.random.SeedSequence([seed, stream, block])))


def _random_bytes(rng: np.random.Generator, n: int) -> np.ndarray:
    words = rng.integers(0, 2**64 - 1, size=(n + 7) // 8, dtype=np.uint64, endpoint=True)
    return words.view(np.uint8)[:n]


def _f16_uniform_bytes(rng: np.random.Generator, count: int, lo: float, hi: float) -> np.ndarray:
    vals = rng.uniform(lo, hi, size=count).astype("<f2")
    return vals.view(np.uint8).reshape(count, 2)


def _q4k_rows(seed: int, stream: int, block: int, rows: int, nsb: int) -> np.ndarray:
    rng = _rng(seed, stream, block)
    nblk = rows * nsb
    raw = _random_bytes(rng, nblk * Q4K_BLOCK_BYTES).reshape(nblk, Q4K_BLOCK_BYTES)
    dd = _f16_uniform_bytes(rng, 2 * nblk, 1e-3, 1e-2).reshape(nblk, 4)
    raw[:, 0:4] = dd
    return raw.reshape(rows, nsb * Q4K_BLOCK_BYTES)


def _q5k_rows(seed: int, stream: int, block: int, rows: int, nsb: int) -> np.ndarray:
    rng = _rng(seed, stream, block)
    nblk = rows * nsb
    raw = _random_bytes(rng, nblk * Q5K_BLOCK_BYTES).reshape(nblk, Q5K_BLOCK_BYTES)
    raw[:, 0:4] = _f16_uniform_bytes(rng, 2 * nblk, 1e-3, 1e-2).reshape(nblk, 4)
    return raw.reshape(rows, nsb * Q5K_BLOCK_BYTES)


def _q6k_rows(seed: int, stream: int, block: int, rows: int, nsb: int) -> np.ndarray:
    rng = _rng(seed, stream, block)
    nblk = rows * nsb
    raw = _random_bytes(rng, nblk * Q6K_BLOCK_BYTES).reshape(nblk, Q6K_BLOCK_BYTES)
    scales = rng.integers(-32, 32, size=(nblk, 16), dtype=np.int8)
    raw[:, 192:208] = scales.view(np.uint8)
    raw[:, 208:210] = _f16_uniform_bytes(rng, nblk, 1e-3, 1e-2)
    return raw.reshape(rows, nsb * Q6K_BLOCK_BYTES)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _gen_matrix(fn, seed: int, stream: int, n_rows: int, k: int, row_bytes: int,
                row_lo: int = 0, row_hi: int | None = None) -> np.ndarray:
    if k % QK:
        raise ValueError(f"k={k} is not a multiple of {QK}")
    nsb = k // QK
    row_hi = n_rows if row_hi is None else row_hi
    if not (0 <= row_lo <= row_hi <= n_rows):
        raise ValueError("bad row range")
    out = np.empty((row_hi - row_lo, nsb * row_bytes), np.uint8)
    first, last = row_lo // ROW_BLOCK, (row_hi + ROW_BLOCK - 1) // ROW_BLOCK

    def one(b: int) -> None:
        r0 = b * ROW_BLOCK
        rows = min(ROW_BLOCK, n_rows - r0)
        blk = fn(seed, stream, b, rows, nsb)
        lo, hi = max(r0, row_lo), min(r0 + rows, row_hi)
        out[lo - row_lo:hi - row_lo] = blk[lo - r0:hi - r0]

    blocks = range(first, last)
    if len(blocks) > 4:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, blocks))
    else:
        for b in blocks:
            one(b)
    return out


def q4k_matrix(n_rows: int, k: int, seed: int = BASE_SEED, stream: int = 0,
               row_lo: int = 0, row_hi: int | None = None) -> np.ndarray:
    """Q4_K weight bytes, shape [rows, (k/256)*144] uint8, rows row_lo..row_hi-1."""
    return _gen_matrix(_q4k_rows, seed, stream, n_rows, k, Q4K_BLOCK_BYTES, row_lo, row_hi)


def q6k_matrix(n_rows: int, k: int, seed: int = BASE_SEED, stream: int = 0,
               row_lo: int = 0, row_hi: int | None = None) -> np.ndarray:
    """Q6_K weight bytes, shape [rows, (k/256)*210] uint8, rows row_lo..row_hi-1."""
    return _gen_matrix(_q6k_rows, seed, stream, n_rows, k, Q6K_BLOCK_BYTES, row_lo, row_hi)


def normal_f32(n, seed: int = BASE_SEED, stream: int = 0, mean: float = 0.0,
               std: float = 1.0) -> np.ndarray:
    """f32 array of shape ``n`` (int or tuple) drawn from N(mean, std^2)."""
    rng = _rng(seed, stream, 0x7FFFFFFF)
    return (mean + std * rng.standard_normal(size=n)).astype(np.float32)


def gains_f32(n: int, seed: int = BASE_SEED, stream: int = 0) -> np.ndarray:
    """RMSNorm gain vector ~ N(1, 0.1)."""
    return normal_f32(n, seed, stream, 1.0, 0.1)


def q5k_matrix(n_rows: int, k: int, seed: int = BASE_SEED, stream: int = 0,
               row_lo: int = 0, row_hi: int | None = None) -> np.ndarray:
    """Q5_K weight bytes, shape [rows, (k/256)*176] uint8, rows row_lo..row_hi-1."""
    return _gen_matrix(_q5k_rows, seed, stream, n_rows, k, Q5K_BLOCK_BYTES, row_lo, row_hi)


def token_ids(n: int, vocab: int, seed: int = BASE_SEED, stream: int = 0) -> np.ndarray:
    """int32 token ids, uniform on 0..vocab-1."""
    return _rng(seed, stream, 0x7FFFFFFE).integers(0, vocab, size=n).astype(np.int32)


def weight_matrix(qtype: str, n_rows: int, k: int, seed: int = BASE_SEED, stream: int = 0,
                  row_lo: int = 0, row_hi: int | None = None) -> np.ndarray:
    if qtype == "q4k":
        return q4k_matrix(n_rows, k, seed, stream, row_lo, row_hi)
    if qtype == "q5k":
        return q5k_matrix(n_rows, k, seed, stream, row_lo, row_hi)
    if qtype == "q6k":
        return q6k_matrix(n_rows, k, seed, stream, row_lo, row_hi)
    raise ValueError(qtype)
