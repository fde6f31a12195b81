"""The kernel's float32 operation order, emulated on the CPU, against the
per-row bound |y - y_ref| <= 1e-4 * S_i + 1e-6 (S_i = sum_j |W_ij x_j|).

This checks the arithmetic design of kq_matvec, not the kernel itself (the
GPU tests compare the kernel with the oracle on the same inputs).  Two
orders are emulated, step by step, with numpy float32 values:

* the kernel's: Q4_K/Q5_K weights formed with one rounding as
  fma(d*sc, q, -dmin*m) (the pages' single-rounding form, muser-book Ch 13
  section 13.4.2) and multiplied into each sub-block's sum; Q6_K codes with
  their -32 offset taken off before the products, each sub-block of 16
  summed and scaled once by sc and then d (Ch 6 section 6.4);
* a deferred order, planted here as the mistake the tests must catch:
  sum(q*x) and sum(x) per sub-block apart, then d*sc*sum(q*x) -
  dmin*m*sum(x) (or, for Q6_K, 32*sum(x) subtracted after the sum).

On rows whose weights cancel (tests/cancel_blocks.py) the deferred order
leaves a residual of the size of the cancelled terms' rounding, far above
the bound, while the kernel's order stays within a small multiple of
2^-24 * S_i.  The emulated fused multiply-add rounds the exact product plus
addend to binary64 and then to float32; that double rounding differs from
one rounding in rare ties only, which does not matter for the magnitudes
checked here.
"""
import numpy as np
import pytest

import kqgen
import oracle
from cancel_blocks import cancel_weights
from kqgen import FORMATS, Q4_K, Q5_K, Q6_K

U = 2.0 ** -24
F32 = np.float32


def fma32(a, b, c):
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64) + np.asarray(c, np.float64)).astype(F32)


def add32(a, b):
    return (np.asarray(a, F32) + np.asarray(b, F32)).astype(F32)


def _decode(fmt, w, rows, cols):
    """Per-block integers from the oracle's decoder: codes [rows, nb, 256],
    scales and mins [rows, nb, 16], d and dmin [rows, nb] (binary64)."""
    nb = cols // 256
    bb = kqgen.BLOCK_BYTES[fmt]
    blocks = w.reshape(rows * nb, bb)
    q = np.empty((rows * nb, 256), np.int64)
    sc = np.empty((rows * nb, 16), np.int64)
    mn = np.empty((rows * nb, 16), np.int64)
    d = np.empty(rows * nb)
    dm = np.empty(rows * nb)
    for i in range(rows * nb):
        r = oracle.decode_block(fmt, blocks[i].tobytes())
        q[i], sc[i], mn[i], d[i], dm[i] = r["codes"], r["scale"], r["min"], r["d"], r["dmin"]
    return (q.reshape(rows, nb, 256), sc.reshape(rows, nb, 16), mn.reshape(rows, nb, 16),
            d.reshape(rows, nb), dm.reshape(rows, nb))


def kernel_order(fmt, w, rows, cols, x):
    """y [rows] in the kernel's order (one token plane, one-block segments
    summed in block order, as a matrix of at most 1024 rows runs)."""
    nb = cols // 256
    W32 = oracle.dequant(fmt, w, rows, cols).astype(F32).reshape(rows, nb, 256)   # one rounding
    y = np.zeros(rows, F32)
    if fmt in (Q4_K, Q5_K):
        for b in range(nb):
            xb = x[256 * b:256 * b + 256]
            c = np.zeros(rows, F32)
            for g in range(4):
                al = np.zeros(rows, F32)
                ah = np.zeros(rows, F32)
                for k in range(8):
                    for i in range(4):
                        e = 64 * g + 4 * k + i
                        al = fma32(W32[:, b, e], xb[e], al)
                        ah = fma32(W32[:, b, e + 32], xb[e + 32], ah)
                c = add32(add32(c, al), ah)
            y = add32(y, c)
        return y
    q, sc, _, d, _ = _decode(fmt, w, rows, cols)
    for b in range(nb):
        xb = x[256 * b:256 * b + 256]
        tl = np.zeros(rows, F32)
        th = np.zeros(rows, F32)
        for n in range(2):
            for kh in range(2):
                for c in range(4):
                    j = 8 * n + 2 * c + kh                       # sub-block of 16
                    a = np.zeros(rows, F32)
                    for k in range(4 * kh, 4 * kh + 4):
                        for i in range(4):
                            e = 128 * n + 32 * c + 4 * k + i
                            a = fma32(q[:, b, e].astype(F32), xb[e], a)   # signed code (q - 32)
                    if c < 2:
                        tl = fma32(sc[:, b, j].astype(F32), a, tl)
                    else:
                        th = fma32(sc[:, b, j].astype(F32), a, th)
        v = add32(th, tl)
        y = add32(y, (d[:, b].astype(F32) * v).astype(F32))
    return y


def _tree_sum(v):
    """Sum of 32 (or 16) values as the wave reduced them: fours added in
    pairs, then the fours' sums by a butterfly."""
    p = [add32(add32(v[i], v[i + 1]), add32(v[i + 2], v[i + 3])) for i in range(0, len(v), 4)]
    while len(p) > 1:
        p = [add32(p[i], p[i + 1]) for i in range(0, len(p), 2)]
    return p[0]


def deferred_order(fmt, w, rows, cols, x):
    """y [rows] with the scale and the min (or the -32 offset) applied after
    each sub-block's sum of q*x: the planted mistake."""
    nb = cols // 256
    q, sc, mn, d, dm = _decode(fmt, w, rows, cols)
    y = np.zeros(rows, F32)
    for b in range(nb):
        xb = x[256 * b:256 * b + 256].astype(F32)
        if fmt in (Q4_K, Q5_K):
            ts = np.zeros(rows, F32)
            tm = np.zeros(rows, F32)
            for j in range(8):
                a = np.zeros(rows, F32)
                for e in range(32 * j, 32 * j + 32):
                    a = fma32(q[:, b, e].astype(F32), xb[e], a)
                ts = fma32(sc[:, b, j].astype(F32), a, ts)
                tm = fma32(mn[:, b, j].astype(F32), _tree_sum([xb[e] for e in range(32 * j, 32 * j + 32)]), tm)
            y = fma32(d[:, b].astype(F32), ts, y)
            y = fma32(-dm[:, b].astype(F32), tm, y)
        else:
            t = np.zeros(rows, F32)
            for j in range(16):
                a = np.zeros(rows, F32)
                for e in range(16 * j, 16 * j + 16):
                    a = fma32((q[:, b, e] + 32).astype(F32), xb[e], a)       # stored code
                u = fma32(F32(-32.0), _tree_sum([xb[e] for e in range(16 * j, 16 * j + 16)]), a)
                t = fma32(sc[:, b, j].astype(F32), u, t)
            y = fma32(d[:, b].astype(F32), t, y)
    return y


def _ratio(y, y_ref, s):
    err = np.abs(y.astype(np.float64) - y_ref)
    return err / (1e-4 * s + 1e-6)


ROWS, COLS = 48, 2560


@pytest.mark.parametrize("fmt", FORMATS)
def test_all_zero_rows_exact_in_kernel_order(fmt):
    """Weights that are exactly zero give exactly zero: every weight is
    formed exactly (or the code carries its offset) before any product."""
    w = cancel_weights(fmt, ROWS, COLS, 0.0, 1)
    x = kqgen.activations(1, COLS, 991, fmt)[0]
    assert not oracle.dequant(fmt, w, ROWS, COLS).any()
    y = kernel_order(fmt, w, ROWS, COLS, x)
    assert not y.any()


@pytest.mark.parametrize("fmt", FORMATS)
def test_deferred_order_fails_on_all_zero_rows(fmt):
    """The planted mistake: subtracting the min (or the offset) after the
    sum breaks the bound on these rows, so they can see it."""
    w = cancel_weights(fmt, ROWS, COLS, 0.0, 2)
    x = kqgen.activations(1, COLS, 992, fmt)[0]
    y_ref, s = oracle.matvec(fmt, w, ROWS, COLS, x)
    r = _ratio(deferred_order(fmt, w, ROWS, COLS, x), y_ref[0], s[0])
    assert (r > 1).mean() > 0.5, r


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("frac", [0.01, 0.05])
def test_sparse_rows_within_derived_bound(fmt, frac):
    """Rows with 1-5% nonzero weights: the kernel's order stays within the
    bound derived for it, (41 + nb + 2) * 2^-24 * S_i for Q4_K/Q5_K and
    (27 + nb + 2) * 2^-24 * S_i for Q6_K (one-block segments), far inside
    1e-4 * S_i.  (At these fractions S_i is large enough that the deferred
    order's residual also fits 1e-4 * S_i; it fails on rows whose S_i is
    near zero, the all-zero rows above.)"""
    nb = COLS // 256
    w = cancel_weights(fmt, ROWS, COLS, frac, 3, int(frac * 100))
    x = kqgen.activations(1, COLS, 993, fmt, int(frac * 100))[0]
    y_ref, s = oracle.matvec(fmt, w, ROWS, COLS, x)
    y_ref, s = y_ref[0], s[0]
    assert (s > 0).all()
    y = kernel_order(fmt, w, ROWS, COLS, x)
    const = (41 if fmt != Q6_K else 27) + nb + 2
    err = np.abs(y.astype(np.float64) - y_ref)
    assert (err <= const * U * s * (1 + 1e-6)).all(), (err / (U * s)).max()
    assert _ratio(y, y_ref, s).max() < 0.2


@pytest.mark.parametrize("fmt", FORMATS)
def test_random_blocks_within_derived_bound(fmt):
    """The synthetic workload's blocks: both orders meet the tolerance; the
    kernel's within its derived bound."""
    nb = COLS // 256
    w = kqgen.weights(fmt, ROWS, COLS, 994, fmt)
    x = kqgen.activations(1, COLS, 995, fmt)[0]
    y_ref, s = oracle.matvec(fmt, w, ROWS, COLS, x)
    y_ref, s = y_ref[0], s[0]
    y = kernel_order(fmt, w, ROWS, COLS, x)
    const = (41 if fmt != Q6_K else 27) + nb + 2
    assert (np.abs(y.astype(np.float64) - y_ref) <= const * U * s).all()
    assert _ratio(deferred_order(fmt, w, ROWS, COLS, x), y_ref, s).max() < 1
