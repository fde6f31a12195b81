"""Seeded synthetic inputs for the k-quant decode matvec.

Shared by the tests, the benchmark and the oracle checks.  This module only
draws random numbers and places bytes at the field offsets of the block
layouts (muser-book Ch 6, Figures 6.2, 6.4 and 6.5); it holds none of the
method's arithmetic (no decoding, no dequantization, no dot products).

Distributions (the synthetic stand-in for a trained GGUF artifact):
  * d, dmin: binary16 of |N(0,1)| * 0.01 (about 0.5% land on binary16
    subnormals and are kept);
  * Q4_K / Q5_K: the 12-byte scale strip, qh and qs are uniform random bytes;
  * Q6_K: ql and qh uniform random bytes, the 16 int8 scales uniform in
    [-32, 31];
  * x: float32 N(0,1).
Every stream comes from numpy PCG64 seeded with
SeedSequence([20261202, *key]) so that any tensor can be regenerated alone.
"""
from __future__ import annotations

import numpy as np

Q4_K, Q5_K, Q6_K = 12, 13, 14
FORMATS = (Q4_K, Q5_K, Q6_K)
FORMAT_NAMES = {Q4_K: "Q4_K", Q5_K: "Q5_K", Q6_K: "Q6_K"}
BLOCK_BYTES = {Q4_K: 144, Q5_K: 176, Q6_K: 210}
BASE_SEED = 20261202


def rng_for(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, *key])))


def row_bytes(fmt: int, cols: int) -> int:
    return cols // 256 * BLOCK_BYTES[fmt]


def _f16_bytes(rng: np.random.Generator, n: int) -> np.ndarray:
    v = (np.abs(rng.standard_normal(n)) * 0.01).astype(np.float16)
    return v.view(np.uint8).reshape(n, 2)


def random_blocks(fmt: int, nblocks: int, rng: np.random.Generator) -> np.ndarray:
    """uint8 [nblocks, block_bytes] with the distributions above."""
    bb = BLOCK_BYTES[fmt]
    raw = np.frombuffer(bytearray(rng.bytes(nblocks * bb)), dtype=np.uint8).reshape(nblocks, bb)
    if fmt in (Q4_K, Q5_K):
        raw[:, 0:2] = _f16_bytes(rng, nblocks)       # d
        raw[:, 2:4] = _f16_bytes(rng, nblocks)       # dmin
    elif fmt == Q6_K:
        raw[:, 192:208] = rng.integers(-32, 32, size=(nblocks, 16), dtype=np.int8).view(np.uint8)
        raw[:, 208:210] = _f16_bytes(rng, nblocks)   # d (last field)
    else:
        raise ValueError("unknown format %r" % fmt)
    return raw


def weights(fmt: int, rows: int, cols: int, *key: int) -> np.ndarray:
    """Row-major weight bytes uint8 [rows, row_bytes] (one contiguous run of
    cols/256 super-blocks per row)."""
    if cols % 256:
        raise ValueError("cols must be a multiple of 256")
    blocks = random_blocks(fmt, rows * (cols // 256), rng_for(*key))
    return blocks.reshape(rows, row_bytes(fmt, cols))


def activations(ntok: int, cols: int, *key: int) -> np.ndarray:
    """float32 [ntok, cols], N(0,1)."""
    return rng_for(*key).standard_normal((ntok, cols), dtype=np.float32)
