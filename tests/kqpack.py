"""Test-side block encoders (the inverse direction of a decoder).

They build hand-packed super-blocks from chosen fields so that a test can
check the decoder against values it picked.  They follow the packing the
pages print: the Q4_K strip is packed the way muser-book Ch 6 section 6.3
packs it by hand (scales[j] = sc_j | top-2-of-sc_{j+4} << 6, scales[4+j] =
m_j | top-2-of-m_{j+4} << 6, scales[8+j] = low nibble of sc_{j+4} | low
nibble of m_{j+4} << 4), with the field offsets of Figures 6.2, 6.4 and 6.5.
The Q5_K high-bit plane and the Q6_K element order follow the readings
stated in the oracle header.
"""
from __future__ import annotations

import numpy as np

Q4_K, Q5_K, Q6_K = 12, 13, 14


def f16_bits(v: float) -> int:
    return int(np.array([v], np.float16).view(np.uint16)[0])


def _le16(bits: int):
    return [bits & 0xFF, (bits >> 8) & 0xFF]


def pack_strip(sc, m):
    assert all(0 <= v < 64 for v in list(sc) + list(m))
    s = [0] * 12
    for j in range(4):
        s[j] = sc[j] | ((sc[j + 4] >> 4) << 6)
        s[4 + j] = m[j] | ((m[j + 4] >> 4) << 6)
        s[8 + j] = (sc[j + 4] & 0x0F) | ((m[j + 4] & 0x0F) << 4)
    return s


def pack_k4_codes(q):
    """256 low-4-bit codes -> 128 qs bytes (group g, byte l: element 64g+l
    in the low nibble, element 64g+32+l in the high nibble)."""
    qs = [0] * 128
    for g in range(4):
        for l in range(32):
            qs[32 * g + l] = (q[64 * g + l] & 15) | ((q[64 * g + 32 + l] & 15) << 4)
    return qs


def pack_q4k(d_bits, dmin_bits, sc, m, q) -> bytes:
    assert all(0 <= v < 16 for v in q)
    return bytes(_le16(d_bits) + _le16(dmin_bits) + pack_strip(sc, m) + pack_k4_codes(q))


def pack_q5k(d_bits, dmin_bits, sc, m, q) -> bytes:
    assert all(0 <= v < 32 for v in q)
    qh = [0] * 32
    for e in range(256):
        j, l = e // 32, e % 32
        qh[l] |= ((q[e] >> 4) & 1) << j
    return bytes(_le16(d_bits) + _le16(dmin_bits) + pack_strip(sc, m) + qh + pack_k4_codes(q))


def pack_q6k(d_bits, sc, q) -> bytes:
    """q: 256 signed codes in [-32, 31]; sc: 16 int8 scales."""
    assert all(-32 <= v < 32 for v in q) and all(-128 <= v < 128 for v in sc)
    ql = [0] * 128
    qh = [0] * 64
    for e in range(256):
        u = q[e] + 32
        n, k, l = e // 128, (e % 128) // 32, e % 32
        li = 64 * n + 32 * (k % 2) + l
        ql[li] |= (u & 15) << (0 if k < 2 else 4)
        qh[32 * n + l] |= (u >> 4) << (2 * k)
    return bytes(ql + qh + [v & 0xFF for v in sc] + _le16(d_bits))


def pack(fmt, d_bits, dmin_bits, sc, m, q) -> bytes:
    if fmt == Q4_K:
        return pack_q4k(d_bits, dmin_bits, sc, m, q)
    if fmt == Q5_K:
        return pack_q5k(d_bits, dmin_bits, sc, m, q)
    if fmt == Q6_K:
        return pack_q6k(d_bits, sc, q)
    raise ValueError(fmt)
