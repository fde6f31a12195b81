"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test ties the oracle to something other than itself: values the pages
print (tests/golden, each file cites its page and section), closed forms,
exact rational arithmetic, and brute force over single bits of hand-packed
blocks.  CPU only.
"""
from fractions import Fraction

import numpy as np
import pytest

import kqgen
from kqgen import Q4_K, Q5_K, Q6_K, FORMATS
from conftest import read_golden
import kqpack

NAMES = {"Q4_K": Q4_K, "Q5_K": Q5_K, "Q6_K": Q6_K}


def test_block_geometry_fig6_1(oracle_lib):
    # Figure 6.1: bits/element = block_bytes * 8 / 256
    rows = []
    with open(__import__("conftest").golden("fig6_1_geometry.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if line:
                rows.append(line)
    assert len(rows) == 3
    for name, bb, elems, bits in rows:
        fmt = NAMES[name]
        assert oracle_lib.block_bytes(fmt) == int(bb)
        assert int(elems) == 256
        assert int(bb) * 8 / 256 == float(bits)
    assert oracle_lib.block_bytes(99) == -1


def _twobytwo_rows(fmt):
    """Figure 13.1 packed into two rows of one super-block each; every other
    code is zero and x is zero beyond column 1."""
    g = read_golden("fig13_1_worked_2x2.txt")
    W = [[int(v) for v in r.split()] for r in g["W"].split(";")]
    one = kqpack.f16_bits(1.0)
    rows = []
    for wr in W:
        if fmt == Q6_K:
            q = [0] * 256
            q[0], q[1] = wr
            sc = [1] + [0] * 15
            rows.append(kqpack.pack_q6k(one, sc, q))
        else:
            q = [0] * 256
            q[0], q[1] = wr
            rows.append(kqpack.pack(fmt, one, 0, [1] + [0] * 7, [0] * 8, q))
    x = np.zeros(256, np.float32)
    x[:2] = [float(v) for v in g["x"].split()]
    y = [float(v) for v in g["y"].split()]
    return rows, x, y


@pytest.mark.parametrize("fmt", FORMATS)
def test_worked_2x2_fig13_1(oracle_lib, fmt):
    rows, x, y_expected = _twobytwo_rows(fmt)
    w = np.frombuffer(b"".join(rows), np.uint8)
    y, s = oracle_lib.matvec(fmt, w, 2, 256, x)
    assert y[0].tolist() == y_expected
    assert s[0].tolist() == y_expected       # all products positive here
    from oracle import exact
    ex = exact.matvec(fmt, rows, [x])
    assert [float(v) for v in ex[0]] == y_expected


def test_q4k_worked_block_sec6_3(oracle_lib):
    g = read_golden("sec6_3_q4k_worked_block.txt")
    blk = bytearray(144)
    blk[0:4] = bytes.fromhex(g["header"].replace(" ", ""))
    blk[4:16] = bytes.fromhex(g["scales"].replace(" ", ""))
    blk[16 + 0] = int(g["qs.0"], 16)
    blk[16 + 32] = int(g["qs.32"], 16)
    dec = oracle_lib.decode_block(Q4_K, bytes(blk))
    assert dec["d"] == float(g["d"]) and dec["dmin"] == float(g["dmin"])
    assert dec["scale"][:8].tolist() == [int(v) for v in g["sc"].split()]
    assert dec["min"][:8].tolist() == [int(v) for v in g["m"].split()]
    assert dec["scale"][5] == int(g["sc.5"]) and dec["min"][5] == int(g["m.5"])
    w = oracle_lib.dequant(Q4_K, np.frombuffer(bytes(blk), np.uint8), 1, 256)[0]
    for key in ("w.0", "w.32", "w.64"):
        assert w[int(key.split(".")[1])] == float(g[key])
    # closed form for the untouched elements (zero code): W = -dmin * m_j
    m = [int(v) for v in g["m"].split()]
    for e in range(256):
        if e not in (0, 32, 64, 96):
            assert w[e] == -float(g["dmin"]) * m[e // 32]
    # the page's packing (section 6.3) is the encoder the tests use
    sc = [int(v) for v in g["sc"].split()]
    assert bytes(kqpack.pack_strip(sc, m)) == bytes(blk[4:16])


def _rand_f16_bits(rng, n):
    """Finite binary16 bit patterns, normals and subnormals, both signs."""
    bits = rng.integers(0, 1 << 16, size=n, dtype=np.uint32)
    bits = np.where(((bits >> 10) & 31) == 31, bits & np.uint32(0xBFFF), bits)   # no inf/nan
    return [int(b) for b in bits]


@pytest.mark.parametrize("fmt", FORMATS)
def test_dequant_form_bruteforce(oracle_lib, fmt):
    """Random fields -> hand-packed block -> the oracle decodes the same fields
    and W = d*sc_j*q - dmin*m_j (Q6_K: d*sc_j*q) exactly (section 6.2 form,
    section 6.4 for the siblings)."""
    rng = np.random.default_rng(1234 + fmt)
    for trial in range(60):
        d_bits, dmin_bits = _rand_f16_bits(rng, 2)
        if fmt == Q6_K:
            sc = [int(v) for v in rng.integers(-128, 128, 16)]
            m = [0] * 16
            q = [int(v) for v in rng.integers(-32, 32, 256)]
            blk = kqpack.pack_q6k(d_bits, sc, q)
            sub = 16
            dmin_bits = 0
        else:
            sc = [int(v) for v in rng.integers(0, 64, 8)]
            m = [int(v) for v in rng.integers(0, 64, 8)]
            q = [int(v) for v in rng.integers(0, 16 if fmt == Q4_K else 32, 256)]
            blk = kqpack.pack(fmt, d_bits, dmin_bits, sc, m, q)
            sub = 32
        dec = oracle_lib.decode_block(fmt, blk)
        assert dec["codes"].tolist() == q
        assert dec["scale"][:len(sc)].tolist() == sc
        assert dec["min"][:len(m)].tolist() == m
        from oracle.exact import f16
        d = f16(d_bits & 255, d_bits >> 8)
        dmin = f16(dmin_bits & 255, dmin_bits >> 8)
        assert dec["d"] == float(d) and dec["dmin"] == float(dmin)
        w = oracle_lib.dequant(fmt, np.frombuffer(blk, np.uint8), 1, 256)[0]
        for e in range(256):
            j = e // sub
            exact_w = d * sc[j] * q[e] - dmin * m[j]
            assert Fraction(w[e]) == exact_w, (trial, e)


def _zero_block(fmt):
    return bytearray(kqgen.BLOCK_BYTES[fmt])


CODE_BYTES = {Q4_K: range(16, 144), Q5_K: range(16, 176), Q6_K: range(0, 192)}
CODE_BITS = {Q4_K: 4, Q5_K: 5, Q6_K: 6}


@pytest.mark.parametrize("fmt", FORMATS)
def test_code_bits_are_a_bijection(oracle_lib, fmt):
    """Every code bit of the block reaches exactly one element with one power
    of two, and every element gets exactly 4/5/6 such bits (1024/1280/1536
    code bits per block: Figure 6.1's 4.5/5.5/6.5625 bits less the header)."""
    base = oracle_lib.decode_block(fmt, bytes(_zero_block(fmt)))["codes"]
    seen = {e: [] for e in range(256)}
    for byte in CODE_BYTES[fmt]:
        for bit in range(8):
            blk = _zero_block(fmt)
            blk[byte] = 1 << bit
            delta = oracle_lib.decode_block(fmt, bytes(blk))["codes"] - base
            nz = np.nonzero(delta)[0]
            assert len(nz) == 1, (byte, bit)
            v = int(delta[nz[0]])
            assert v > 0 and (v & (v - 1)) == 0
            seen[int(nz[0])].append(v)
    want = [1 << k for k in range(CODE_BITS[fmt])]
    for e in range(256):
        assert sorted(seen[e]) == want, e
    assert len(CODE_BYTES[fmt]) * 8 == 256 * CODE_BITS[fmt]


@pytest.mark.parametrize("fmt", (Q4_K, Q5_K))
def test_scale_strip_bits_are_a_bijection(oracle_lib, fmt):
    """The 96-bit strip holds 16 six-bit fields (8 sc, 8 m), section 6.2."""
    seen = {}
    for byte in range(4, 16):
        for bit in range(8):
            blk = _zero_block(fmt)
            blk[byte] = 1 << bit
            dec = oracle_lib.decode_block(fmt, bytes(blk))
            fields = np.concatenate([dec["scale"][:8], dec["min"][:8]])
            nz = np.nonzero(fields)[0]
            assert len(nz) == 1, (byte, bit)
            v = int(fields[nz[0]])
            assert v & (v - 1) == 0
            seen.setdefault(int(nz[0]), []).append(v)
    assert sorted(seen) == list(range(16))
    for f, vals in seen.items():
        assert sorted(vals) == [1, 2, 4, 8, 16, 32], f


def test_q6k_scale_and_header_offsets(oracle_lib):
    """Figure 6.5: 16 int8 scales at 192..207, f16 d at 208..209 (last)."""
    for j in range(16):
        blk = _zero_block(Q6_K)
        blk[192 + j] = 0xFF
        dec = oracle_lib.decode_block(Q6_K, bytes(blk))
        assert dec["scale"].tolist() == [-1 if i == j else 0 for i in range(16)]
    blk = _zero_block(Q6_K)
    blk[208:210] = bytes([0x00, 0x40])          # 2.0
    assert oracle_lib.decode_block(Q6_K, bytes(blk))["d"] == 2.0
    assert oracle_lib.decode_block(Q6_K, bytes(blk))["codes"].tolist() == [-32] * 256
    blk[0:192] = bytes([0xFF]) * 192
    assert oracle_lib.decode_block(Q6_K, bytes(blk))["codes"].tolist() == [31] * 256


@pytest.mark.parametrize("fmt", (Q4_K, Q5_K))
def test_k4_header_offsets(oracle_lib, fmt):
    """Figures 6.2 / 6.4: d at 0..1, dmin at 2..3 (little-endian f16)."""
    blk = _zero_block(fmt)
    blk[0:4] = bytes([0x00, 0x3C, 0x00, 0xC0])  # d = 1.0, dmin = -2.0
    dec = oracle_lib.decode_block(fmt, bytes(blk))
    assert dec["d"] == 1.0 and dec["dmin"] == -2.0
    if fmt == Q5_K:
        blk[16:48] = bytes([0xFF]) * 32          # qh plane all ones: +16 on every code
        assert oracle_lib.decode_block(fmt, bytes(blk))["codes"].tolist() == [16] * 256


def test_f16_conversion_exhaustive(oracle_lib):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle_lib.f16_to_f64(int(b)) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])
    # subnormals are kept
    assert oracle_lib.f16_to_f64(1) == 2.0 ** -24


@pytest.mark.parametrize("fmt", FORMATS)
def test_special_cases(oracle_lib, fmt):
    rows, cols = 5, 512
    w = kqgen.weights(fmt, rows, cols, 77, fmt)
    W = oracle_lib.dequant(fmt, w, rows, cols)
    # one-hot x picks a column of W
    for j in (0, 1, 255, 256, 511):
        x = np.zeros(cols, np.float32)
        x[j] = 1.0
        y, _ = oracle_lib.matvec(fmt, w, rows, cols, x)
        assert np.array_equal(y[0], W[:, j])
    # x = 1 gives the row sums, accumulated in column order
    y, _ = oracle_lib.matvec(fmt, w, rows, cols, np.ones(cols, np.float32))
    ref = np.zeros(rows)
    for j in range(cols):
        ref += W[:, j]
    assert np.array_equal(y[0], ref)
    # zero headers give zero weights
    wz = w.copy().reshape(-1, kqgen.BLOCK_BYTES[fmt])
    if fmt == Q6_K:
        wz[:, 208:210] = 0
    else:
        wz[:, 0:4] = 0
    y, s = oracle_lib.matvec(fmt, wz, rows, cols, kqgen.activations(1, cols, 5))
    assert not y.any() and not s.any()
    # zero codes: Q4_K/Q5_K W = -dmin*m_j, Q6_K W = -32*d*sc_j
    blk = kqgen.random_blocks(fmt, 1, kqgen.rng_for(9, fmt))[0].copy()
    for b in CODE_BYTES[fmt]:
        blk[b] = 0
    dec = oracle_lib.decode_block(fmt, blk.tobytes())
    wv = oracle_lib.dequant(fmt, blk, 1, 256)[0]
    for e in range(256):
        if fmt == Q6_K:
            assert wv[e] == -32 * dec["d"] * dec["scale"][e // 16]
        else:
            assert wv[e] == -dec["dmin"] * dec["min"][e // 32]


@pytest.mark.parametrize("fmt", FORMATS)
def test_against_exact_rational(oracle_lib, fmt):
    """Tiny random cases: the binary64 oracle is within its rounding bound of
    the exact rational result, and its dequantized weights are exact."""
    from oracle import exact
    rows, cols, ntok = 3, 512, 2
    w = kqgen.weights(fmt, rows, cols, 31, fmt)
    x = kqgen.activations(ntok, cols, 32, fmt)
    y, s = oracle_lib.matvec(fmt, w, rows, cols, x)
    ex = exact.matvec(fmt, [w[i].tobytes() for i in range(rows)], list(x))
    W = oracle_lib.dequant(fmt, w, rows, cols)
    for i in range(rows):
        blocks = [exact.dequant_block(fmt, w[i, b * kqgen.BLOCK_BYTES[fmt]:(b + 1) * kqgen.BLOCK_BYTES[fmt]].tobytes())
                  for b in range(cols // 256)]
        flat = [v for blk in blocks for v in blk]
        assert all(Fraction(W[i, j]) == flat[j] for j in range(cols))
        for t in range(ntok):
            exact_s = sum(abs(flat[j] * Fraction(float(x[t, j]))) for j in range(cols))
            bound = cols * 2.0 ** -52 * float(exact_s)
            assert abs(Fraction(y[t, i]) - ex[t][i]) <= Fraction(bound)
            assert abs(Fraction(s[t, i]) - exact_s) <= Fraction(bound)


def test_byte_totals(oracle_lib):
    g = read_golden("sec6_6_byte_totals.txt")
    assert kqgen.row_bytes(Q4_K, 6656) == int(g["q4k_row_bytes 6656"])
    assert 4096 * kqgen.row_bytes(Q4_K, 6656) == int(g["q4k_matrix_bytes 4096x6656"])
    assert 202048 * kqgen.row_bytes(Q5_K, 6656) == int(g["q5k_lm_head_bytes 202048x6656"])
    assert 202048 * kqgen.row_bytes(Q4_K, 6656) == int(g["q4k_lm_head_bytes 202048x6656"])
    assert 6656 * 4096 == int(g["params q 6656x4096"])
    assert 6656 * 256 == int(g["params k 6656x256"])
    assert 2 * 6656 * 4096 + 2 * 6656 * 256 == int(g["params set"])
    for fmt in FORMATS:
        assert kqgen.row_bytes(fmt, 6656) == 26 * oracle_lib.block_bytes(fmt)


@pytest.mark.parametrize("fmt", FORMATS)
def test_row_selection_and_threads(oracle_lib, fmt):
    rows, cols = 37, 768
    w = kqgen.weights(fmt, rows, cols, 41, fmt)
    x = kqgen.activations(3, cols, 42, fmt)
    y, s = oracle_lib.matvec(fmt, w, rows, cols, x)
    y4, s4 = oracle_lib.matvec(fmt, w, rows, cols, x, nthreads=4)
    assert np.array_equal(y, y4) and np.array_equal(s, s4)
    idx = [36, 0, 17, 17]
    ys, ss = oracle_lib.matvec(fmt, w, rows, cols, x, row_idx=idx)
    assert np.array_equal(ys, y[:, idx]) and np.array_equal(ss, s[:, idx])
    # s bounds |y|, and the rows really differ
    assert np.all(np.abs(y) <= s)
    assert len(set(y[0].tolist())) > 30


def test_embedding_rows_handpacked(oracle_lib):
    """The embedding lookup (Ch 6 section 6.7) on a table of hand-packed
    Q4_K rows: a 6,656-wide row is 26 blocks, 3,744 bytes (Ch 6 section
    6.6), and the row looked up for each id is d*sc_j*q - dmin*m_j of that
    row's own blocks, exactly.  Ids repeat, come in any order, and ids
    outside [0, rows) give rows of NaN."""
    from oracle.exact import f16
    rng = np.random.default_rng(77)
    rows, cols, nb = 5, 6656, 26
    table = bytearray()
    fields = {}
    for r in range(rows):
        for b in range(nb):
            d_bits, dmin_bits = _rand_f16_bits(rng, 2)
            sc = [int(v) for v in rng.integers(0, 64, 8)]
            m = [int(v) for v in rng.integers(0, 64, 8)]
            q = [int(v) for v in rng.integers(0, 16, 256)]
            table += kqpack.pack_q4k(d_bits, dmin_bits, sc, m, q)
            fields[r, b] = (f16(d_bits & 255, d_bits >> 8), f16(dmin_bits & 255, dmin_bits >> 8), sc, m, q)
    assert len(table) == rows * 3744
    ids = [4, 0, 2, 2, -1, 5, 1, 1 << 30]
    out = oracle_lib.embed(Q4_K, np.frombuffer(bytes(table), np.uint8), rows, cols, ids)
    assert out.shape == (len(ids), cols)
    for t, r in enumerate(ids):
        if not 0 <= r < rows:
            assert np.isnan(out[t]).all()
            continue
        for b in range(nb):
            d, dmin, sc, m, q = fields[r, b]
            for e in range(256):
                assert Fraction(out[t, 256 * b + e]) == d * sc[e // 32] * q[e] - dmin * m[e // 32], (t, b, e)


@pytest.mark.parametrize("fmt", FORMATS)
def test_embedding_is_the_dequantized_row(oracle_lib, fmt):
    """Element-by-element lookup against the block-by-block dequantization
    of the whole table (another code path of the oracle), at widths of 1 and
    26 blocks; a swapped pair of rows swaps the looked-up rows."""
    for rows, cols in ((9, 256), (7, 6656)):
        w = kqgen.weights(fmt, rows, cols, 88, fmt, cols)
        ids = [rows - 1, 0, 3, 3, rows, -5]
        out = oracle_lib.embed(fmt, w, rows, cols, ids)
        full = oracle_lib.dequant(fmt, w, rows, cols)
        assert np.array_equal(out[:4], full[ids[:4]])
        assert np.isnan(out[4:]).all()
        sw = w.copy()
        sw[[0, 3]] = sw[[3, 0]]
        out2 = oracle_lib.embed(fmt, sw, rows, cols, [0, 3, 1])
        assert np.array_equal(out2, full[[3, 0, 1]])
