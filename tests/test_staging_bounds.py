"""Byte ranges the kernels' weight staging reads, on the CPU.

A host-side model of every staging path's address arithmetic (the offsets,
clamps and buffer bounds written in quant_matvec_amd/csrc/kq_kernels.hip),
evaluated for every lane, tile and block column of small tensors with
ragged row counts and both block-count parities.  Each path must read only
bytes of the tensor (W may be a view into a mapped model file, so a byte
past its end may be unmapped), and the matrix-core block loads only bytes
of the block they decode (a Q6_K block that starts 2 bytes into a word may
read the 2 bytes before it, which belong to the previous block).  Block
layouts: Q4_K 144 B, Q5_K 176 B, Q6_K 210 B (muser-book Ch 6 sections
6.2-6.4; Q6_K's d is its last two bytes, Figure 6.5).
"""
import numpy as np
import pytest

BB = {12: 144, 13: 176, 14: 210}
ROWS = [1, 2, 3, 31, 32, 33, 63, 64, 65, 95, 129]
NBS = [1, 2, 3, 4, 5, 26, 27]
LANES = np.arange(64, dtype=np.int64)


def check(reads, total, what):
    """reads: list of (start, length) arrays; every byte in [0, total)."""
    for start, length in reads:
        start = np.asarray(start, dtype=np.int64)
        assert start.min() >= 0, (what, int(start.min()))
        end = start + length
        assert end.max() <= total, (what, int(end.max()), total)


def k45_column(fmt, rows, nb):
    """64-row Q4_K/Q5_K column (K45Column::stage), lane-per-row tiles."""
    bb, rb = BB[fmt], nb * BB[fmt]
    C = bb // 16
    total = rows * rb
    q = 64 * np.arange(C)[:, None] + LANES[None, :]
    off = (q // C) * rb + 16 * (q % C)
    for tile in range((rows + 63) // 64):
        rows_here = min(64, rows - tile * 64)
        for b in range(nb):
            for valid in (True, False):
                max_off = (rows_here - 1) * rb + 16 * (C - 1) if valid else 0
                col = tile * 64 * rb + b * bb if valid else 0
                check([(col + np.minimum(off, max_off), 16)], total, ("K45Column", fmt, rows, nb, tile, b))


def k45_pair(fmt, rows, nb):
    """32-row pair tiles: the one-wave kernel's loads (K45Pair::stage) and
    the pipelined kernel's buffer loads (K45Pair::dma_w)."""
    bb, rb = BB[fmt], nb * BB[fmt]
    C = bb // 16
    C2 = 2 * C
    total = rows * rb
    q = 64 * np.arange(C)[:, None] + LANES[None, :]
    off = (q // C2) * rb + 16 * (q % C2)
    for tile in range((rows + 31) // 32):
        rows_here = min(32, rows - tile * 32)
        for b in range(0, nb - 1, 2):
            for valid in (True, False):
                max_off = (rows_here - 1) * rb + 16 * (C2 - 1) if valid else 0
                col = tile * 32 * rb + b * bb if valid else 0
                check([(col + np.minimum(off, max_off), 16)], total, ("K45Pair", fmt, rows, nb, tile, b))
            base = tile * 32 * rb + b * bb
            size = rows_here * rb - b * bb
            inside = off + 16 <= size
            # a piece either lies wholly inside the buffer or wholly past it
            assert np.all(inside | (off >= size)), ("K45Pair dma straddles", fmt, rows, nb, tile, b)
            check([(base + off[inside], 16)], total, ("K45Pair dma", fmt, rows, nb, tile, b))
            assert base + size <= total


def q6_column(rows, nb):
    """64-row Q6_K column (Q6Offsets + Q6Column::stage): aligned words of
    each row's block, odd rows moved by corr when the block count is odd,
    the tensor's last block read without its word 52."""
    rb = nb * 210
    alt = nb % 2 == 1
    total = rows * rb
    q = 64 * np.arange(13)[:, None] + LANES[None, :]
    r = q // 13
    off = r * rb + 16 * (q % 13)
    odd = r & 1
    off52 = LANES * rb + 208
    odd52 = LANES & 1
    for tile in range((rows + 63) // 64):
        r0 = tile * 64
        last_row = min(64, rows - r0) - 1
        for b in range(nb):
            for valid in (True, False):
                start = r0 * rb + 210 * b
                last = start + last_row * rb
                tail = valid and (r0 + last_row + 1 == rows) and (b == nb - 1) and (last & 3) == 0
                corr = 2 * (start & 3) - 2 if alt else 0
                dl = corr if (last_row & 1) else 0
                max_off = last_row * rb + 16 * 12 + dl if valid else 0
                max52 = last_row * rb + (204 if tail else 208) + dl if valid else 0
                col = (start & ~3) if valid else 0
                at = off + (odd * corr if alt else 0)
                at52 = off52 + (odd52 * corr if alt else 0)
                reads = [(col + np.minimum(at, max_off), 16), (col + np.minimum(at52, max52), 4),
                         (np.array([last + 208 if tail else 0]), 2)]
                check(reads, total, ("Q6Column", rows, nb, tile, b, valid))


def q6_pair(rows, nb):
    """32-row Q6_K pair tiles: Q6Pair::stage and Q6Pair::dma_w."""
    rb = nb * 210
    total = rows * rb
    q = 64 * np.arange(13)[:, None] + LANES[None, :]
    off = (q // 26) * rb + 16 * (q % 26)
    off104 = (LANES & 31) * rb + 416
    for tile in range((rows + 31) // 32):
        rows_here = min(32, rows - tile * 32)
        for b in range(0, nb - 1, 2):
            for valid in (True, False):
                max_off = (rows_here - 1) * rb + 16 * 25 if valid else 0
                max104 = (rows_here - 1) * rb + 416 if valid else 0
                col = tile * 32 * rb + 210 * b if valid else 0
                check([(col + np.minimum(off, max_off), 16), (col + np.minimum(off104, max104), 4)], total,
                      ("Q6Pair", rows, nb, tile, b, valid))
            base = tile * 32 * rb + 210 * b
            assert base % 4 == 0
            size = rows_here * rb - 210 * b
            for o, n in ((off, 16), (off104, 4)):
                inside = o + n <= size
                assert np.all(inside | (o >= size)), ("Q6Pair dma straddles", rows, nb, tile, b)
                check([(base + o[inside], n)], total, ("Q6Pair dma", rows, nb, tile, b))


def mmb6_q6_block(o, total):
    """kq_mmb6_kernel's loads of the Q6_K block at byte o, every lane group
    h: returns the lowest and highest byte read."""
    a = o & ~3
    sh = 16 if (o & 2) else 0
    lo, hi = 1 << 62, -1
    for h in range(4):
        words = []
        for n in range(2):
            for t in range(2):
                for u in range(2):
                    words += [16 * n + 8 * t + 4 * u + h, 16 * n + 8 * t + 4 * u + h + 1]   # ql
            for u in range(2):
                words += [32 + 8 * n + 4 * u + h, 32 + 8 * n + 4 * u + h + 1]               # qh
        words += [48, 49, 50, 51, 51 + (sh >> 4)]                                           # scales
        lo = min(lo, a + 4 * min(words))
        hi = max(hi, a + 4 * max(words) + 3)
    # d: the two bytes at 208
    hi = max(hi, o + 209)
    return lo, hi


@pytest.mark.parametrize("fmt", [12, 13])
@pytest.mark.parametrize("rows", ROWS)
def test_k45_staging_reads_inside_the_tensor(fmt, rows):
    for nb in NBS:
        k45_column(fmt, rows, nb)
        k45_pair(fmt, rows, nb)


@pytest.mark.parametrize("rows", ROWS)
def test_q6_staging_reads_inside_the_tensor(rows):
    for nb in NBS:
        q6_column(rows, nb)
        q6_pair(rows, nb)


def test_q6_matrix_core_loads_stay_in_the_block():
    """Every block of tensors of either block-count parity: nothing past the
    block's last byte (209), at most the 2 bytes before it (in the same
    aligned word as the block's first byte)."""
    for rows, nb in ((1, 1), (3, 3), (37, 3), (5, 26), (7, 27)):
        total = rows * nb * 210
        for blk in range(rows * nb):
            o = blk * 210
            lo, hi = mmb6_q6_block(o, total)
            assert hi <= o + 209, (rows, nb, blk, hi - o)
            assert lo >= o - 2 and lo >= 0, (rows, nb, blk, lo - o)
            assert hi < total


def test_k45_matrix_core_loads_stay_in_the_block():
    """kq_mmb_kernel's loads of a Q4_K/Q5_K block, every lane group h: the
    header, two qs words of each group and (Q5_K) two qh words."""
    for fmt in (12, 13):
        bb = BB[fmt]
        qs = 16 if fmt == 12 else 48
        for h in range(4):
            pieces = [(0, 16)] + [(qs + 32 * g + 8 * h, 8) for g in range(4)]
            if fmt == 13:
                pieces += [(16 + 8 * h, 8)]
            for st, n in pieces:
                assert 0 <= st and st + n <= bb, (fmt, h, st)


def test_the_model_catches_a_read_past_the_end():
    """A planted error in the model (the tensor's last Q6_K block read with
    its word 52) must be reported: the check is not vacuous."""
    rows, nb = 1, 1                         # one block at offset 0: 4-byte aligned, ends 2 bytes into word 52
    with pytest.raises(AssertionError):
        check([(np.array([208]), 4)], rows * nb * 210, "planted")
