"""Exact-rational re-statement of the k-quant matvec -- TEST INFRASTRUCTURE ONLY.

A second, independent transcription of the decoders of muser-book Ch 6
(section 6.2 for Q4_K, section 6.4 / Figures 6.4-6.5 for Q5_K and Q6_K) and
of the matvec of muser-book Ch 13 section 13.1, in pure Python with
``fractions.Fraction``: no rounding anywhere.  It is slow (tiny inputs only)
and is used to pin the binary64 C oracle, not the HIP path.
"""
from __future__ import annotations

from fractions import Fraction

Q4_K, Q5_K, Q6_K = 12, 13, 14
BLOCK_BYTES = {Q4_K: 144, Q5_K: 176, Q6_K: 210}


def f16(lo: int, hi: int) -> Fraction:
    """Little-endian IEEE binary16 as an exact Fraction (finite values only)."""
    h = lo | (hi << 8)
    sign = -1 if h & 0x8000 else 1
    e = (h >> 10) & 31
    f = h & 1023
    if e == 31:
        raise ValueError("inf/nan header")
    if e == 0:
        return sign * Fraction(f, 1 << 24)
    return sign * Fraction(1024 + f, 1) * Fraction(2) ** (e - 25)


def _k4_scale_min(s, j):
    # six-bit fields of the 12-byte strip (get_scale_min, section 6.2)
    if j < 4:
        return s[j] % 64, s[j + 4] % 64
    return (s[j + 4] % 16) + 16 * (s[j - 4] // 64), (s[j + 4] // 16) + 16 * (s[j] // 64)


def dequant_block(fmt: int, blk) -> list:
    """Exact weights of one super-block, element order 0..255."""
    blk = list(bytes(blk))
    if len(blk) != BLOCK_BYTES[fmt]:
        raise ValueError("wrong block size")
    out = [None] * 256
    if fmt in (Q4_K, Q5_K):
        d, dmin = f16(blk[0], blk[1]), f16(blk[2], blk[3])
        strip = blk[4:16]
        qs = blk[16:144] if fmt == Q4_K else blk[48:176]
        qh = blk[16:48]
        for g in range(4):                 # group of 64 = sub-blocks 2g, 2g+1
            for half in range(2):
                j = 2 * g + half
                sc, m = _k4_scale_min(strip, j)
                for l in range(32):
                    byte = qs[32 * g + l]
                    q = byte % 16 if half == 0 else byte // 16
                    if fmt == Q5_K:
                        q += 16 * ((qh[l] >> j) & 1)
                    out[64 * g + 32 * half + l] = d * sc * q - dmin * m
        return out
    if fmt == Q6_K:
        ql, qh = blk[0:128], blk[128:192]
        scales = [v - 256 if v > 127 else v for v in blk[192:208]]
        d = f16(blk[208], blk[209])
        for n in range(2):
            for k in range(4):
                for l in range(32):
                    byte = ql[64 * n + 32 * (k % 2) + l]
                    nib = byte % 16 if k < 2 else byte // 16
                    two = (qh[32 * n + l] >> (2 * k)) % 4
                    e = 128 * n + 32 * k + l
                    out[e] = d * scales[e // 16] * (nib + 16 * two - 32)
        return out
    raise ValueError("unknown format")


def matvec(fmt: int, w_rows, x_rows):
    """Exact y[t][i] = sum_j W[i,j] x[t][j]; w_rows is a list of row byte
    strings, x_rows a list of float sequences (each value exact as a
    Fraction)."""
    bb = BLOCK_BYTES[fmt]
    result = []
    for x in x_rows:
        xf = [Fraction(float(v)) for v in x]
        ys = []
        for row in w_rows:
            row = bytes(row)
            acc = Fraction(0)
            for b in range(len(row) // bb):
                wb = dequant_block(fmt, row[b * bb:(b + 1) * bb])
                for e in range(256):
                    acc += wb[e] * xf[256 * b + e]
            ys.append(acc)
        result.append(ys)
    return result
