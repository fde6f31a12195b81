"""Adversarial weight rows whose terms cancel: test inputs only.

Rows built here have dequantized weights that are exactly zero, or zero
except for a small fraction of elements, while every block's two terms
(d*sc*q and dmin*m for Q4_K/Q5_K, d*sc*q and the -32 offset for Q6_K) stay
large.  A product that forms sum(d*sc*q*x) and sum(dmin*m*x) apart and
subtracts afterwards leaves a residual of the size of those terms' rounding
on such rows, while the per-row bound 1e-4 * sum_j|W_ij x_j| + 1e-6 shrinks
with the surviving weights, so these rows catch that mistake.

Construction (muser-book Ch 6: W = d*sc*q - dmin*m for Q4_K/Q5_K, sections
6.2 and 6.4; W = d*sc*(q - 32) for Q6_K, section 6.4):
  * Q4_K/Q5_K: d = dmin (a random binary16 of the synthetic distribution),
    sc_j = m_j (random in 1..63) for every sub-block, every code q = 1, so
    W = d*sc_j*1 - d*sc_j = 0 exactly.  A nonzero element gets q = 0 or 2
    (W = -+d*sc_j); in Q5_K the fifth bit plane stays zero.
  * Q6_K: every stored code 32 (ql nibble 0, qh field 2), random int8 scales
    in [-32, 31] and d, so W = 0 exactly.  A nonzero element gets a code of
    32 +- 1..8.
This module only places bytes (the packing is the inverse of the decoders,
with the field offsets of Figures 6.2, 6.4 and 6.5 and the element readings
stated in the oracle header); it computes no product.
"""
from __future__ import annotations

import numpy as np

import kqgen
from kqgen import Q4_K, Q5_K, Q6_K


def _f16(rng, n):
    return (np.abs(rng.standard_normal(n)) * 0.01).astype(np.float16).view(np.uint16)


def _strip(sc, m):
    """[n, 8] 6-bit sc and m -> [n, 12] strip bytes (the section 6.3 packing)."""
    s = np.zeros((sc.shape[0], 12), np.uint8)
    for j in range(4):
        s[:, j] = sc[:, j] | ((sc[:, j + 4] >> 4) << 6)
        s[:, 4 + j] = m[:, j] | ((m[:, j + 4] >> 4) << 6)
        s[:, 8 + j] = (sc[:, j + 4] & 15) | ((m[:, j + 4] & 15) << 4)
    return s


def _qs(q):
    """[n, 256] codes -> [n, 128] qs bytes (low nibble element 64g+l, high
    nibble element 64g+32+l of byte 32g+l)."""
    qs = np.zeros((q.shape[0], 128), np.uint8)
    for g in range(4):
        qs[:, 32 * g:32 * g + 32] = (q[:, 64 * g:64 * g + 32] & 15) | ((q[:, 64 * g + 32:64 * g + 64] & 15) << 4)
    return qs


def _q6(q_unsigned):
    """[n, 256] stored 6-bit codes -> ([n, 128] ql, [n, 64] qh)."""
    n = q_unsigned.shape[0]
    ql = np.zeros((n, 128), np.uint8)
    qh = np.zeros((n, 64), np.uint8)
    for e in range(256):
        h, k, l = e // 128, (e % 128) // 32, e % 32
        u = q_unsigned[:, e]
        ql[:, 64 * h + 32 * (k % 2) + l] |= ((u & 15) << (0 if k < 2 else 4)).astype(np.uint8)
        qh[:, 32 * h + l] |= ((u >> 4) << (2 * k)).astype(np.uint8)
    return ql, qh


def cancel_weights(fmt: int, rows: int, cols: int, frac_nonzero: float, *key: int) -> np.ndarray:
    """uint8 [rows, row_bytes]: weights exactly zero except a fraction
    `frac_nonzero` of elements (chosen at random per element)."""
    rng = kqgen.rng_for(990, fmt, *key)
    nb = rows * (cols // 256)
    bb = kqgen.BLOCK_BYTES[fmt]
    nz = rng.random((nb, 256)) < frac_nonzero
    out = np.zeros((nb, bb), np.uint8)
    if fmt in (Q4_K, Q5_K):
        d = _f16(rng, nb)
        sc = rng.integers(1, 64, size=(nb, 8)).astype(np.uint8)
        q = np.ones((nb, 256), np.uint8)
        q[nz] = rng.choice([0, 2], size=int(nz.sum())).astype(np.uint8)
        out[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
        out[:, 2:4] = d.view(np.uint8).reshape(nb, 2)
        out[:, 4:16] = _strip(sc, sc)
        qs0 = 16 if fmt == Q4_K else 48       # Q5_K: qh[32] (all zero) sits at 16..47
        out[:, qs0:qs0 + 128] = _qs(q)
    elif fmt == Q6_K:
        q = np.full((nb, 256), 32, np.int16)
        k = int(nz.sum())
        q[nz] = 32 + rng.choice([-1, 1], size=k) * rng.integers(1, 9, size=k)
        ql, qh = _q6(q.astype(np.uint16))
        out[:, 0:128] = ql
        out[:, 128:192] = qh
        out[:, 192:208] = rng.integers(-32, 32, size=(nb, 16), dtype=np.int8).view(np.uint8)
        out[:, 208:210] = _f16(rng, nb).view(np.uint8).reshape(nb, 2)
    else:
        raise ValueError(fmt)
    return out.reshape(rows, -1)
