"""GPU parity, second part: rows whose weights cancel, the ntok 1..8 matrix
on every tile height and segment length, sets up to 16 members, the
invariants of the product, the workspace, and the two large workloads
(the 202,048-row Q6_K matvec and the 52-layer Q/K/V/gate stream) checked
row by row at full size.

Every case runs through the C ABI and is compared with the binary64 oracle
per row, |y_gpu - y_ref| <= 1e-4 * sum_j|W_ij x_j| + 1e-6; where the
library promises equal bits (a set and its single calls, a token plane and
the call with fewer planes of the same plan, scaled inputs, permuted rows)
the bits are compared.
"""
import os

import numpy as np
import pytest

import kqgen
import oracle
import quant_matvec_amd as kq
from cancel_blocks import cancel_weights
from gpu_util import check_tol, dev, gpu_matvec, host, note, torch
from kqgen import FORMATS, Q4_K, Q5_K, Q6_K
from kqgen import workloads as wl

pytestmark = pytest.mark.gpu

NTHREADS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    kq.load()
    oracle.lib()


def _bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def _mm(entry, fmt, w, rows, cols, x):
    """kq_matvec16 / kq_matmul on host arrays; y [ntok, rows]."""
    t = torch()
    x = np.atleast_2d(x).astype(np.float32)
    y = t.full((x.shape[0], rows), float("nan"), dtype=t.float32, device="cuda")
    getattr(kq, entry)(fmt, dev(w.reshape(-1)), rows, cols, dev(x), y, ntok=x.shape[0])
    return host(y)


def _run(entry, fmt, w, rows, cols, x):
    if entry == "kq_matvec":
        return gpu_matvec(fmt, w, rows, cols, x)
    return _mm(entry, fmt, w, rows, cols, x)


# ---- rows whose weights cancel (Ch 13 section 13.4.2: the single-rounding
# form; the weights are exactly zero except a fraction of elements)

CANCEL_CASES = [("kq_matvec", 1, 200), ("kq_matvec", 8, 200), ("kq_matvec", 1, 1100), ("kq_matvec", 2, 1100),
                ("kq_matvec16", 16, 200), ("kq_matmul", 64, 200)]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("frac", [0.0, 0.01, 0.05])
@pytest.mark.parametrize("entry,ntok,rows", CANCEL_CASES)
def test_cancelling_rows(fmt, frac, entry, ntok, rows):
    cols = 6656
    w = cancel_weights(fmt, rows, cols, frac, 11, rows)
    x = kqgen.activations(ntok, cols, 996, fmt, ntok)
    note("cancelling rows %s fmt=%d frac=%g %dx%d ntok=%d" % (entry, fmt, frac, rows, cols, ntok))
    y = _run(entry, fmt, w, rows, cols, x)
    y_ref, s = oracle.matvec(fmt, w, rows, cols, x, nthreads=NTHREADS)
    check_tol(y, y_ref, s, "cancelling %s fmt %d frac %g" % (entry, fmt, frac))
    if frac == 0.0:
        assert not y.any()                       # every weight is exactly zero


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("frac", [0.0, 0.02])
def test_cancelling_rows_in_a_set(fmt, frac):
    """A Q/K/V/gate-shaped set whose members cancel, through kq_matvec_set:
    within tolerance and bitwise equal to the single calls."""
    cols = 6656
    specs = [(Q4_K, 4096), (Q6_K, 256), (fmt, 256), (Q5_K, 1100)]
    ws = [cancel_weights(f, r, cols, frac, 12, i) for i, (f, r) in enumerate(specs)]
    x = kqgen.activations(1, cols, 997, fmt)
    note("cancelling set fmt=%d frac=%g" % (fmt, frac))
    t = torch()
    dx = dev(x)
    ys = [t.full((1, r), float("nan"), dtype=t.float32, device="cuda") for (_, r) in specs]
    kq.kq_matvec_set([dict(fmt=f, w=dev(w.reshape(-1)), x=dx, y=y, rows=r, cols=cols)
                      for (f, r), w, y in zip(specs, ws, ys)])
    for (f, r), w, y in zip(specs, ws, ys):
        yh = host(y)
        y_ref, s = oracle.matvec(f, w, r, cols, x, nthreads=NTHREADS)
        check_tol(yh, y_ref, s, "cancelling set member fmt %d rows %d" % (f, r))
        assert np.array_equal(_bits(yh), _bits(gpu_matvec(f, w, r, cols, x)))


# ---- ntok 1..8 on every plan: 64-row tiles with one- and two-block
# segments, 32-row tiles with two- and four-block segments.  Planes of
# calls that plan the tensor alike are bitwise equal.

# (rows, cols) -> groups of ntok that share one plan for every format
NTOK_SHAPES = {
    (131, 6656): [[1, 2], list(range(3, 9))],  # 32-row two-block at ntok 1-2; 64-row one-block at 3-8
    (1100, 2304): [list(range(1, 9))],         # odd blocks a row: 64-row tiles, two-block (Q6_K one-block)
    (1100, 2560): [list(range(1, 9))],         # 32-row tiles at ntok 1-2, 64-row at 3-8, two-block segments
    (1100, 6656): [list(range(1, 9))],         # 32-row tiles at ntok 1-2, 64-row at 3-8, two-block segments
}


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("shape", list(NTOK_SHAPES))
def test_ntok_1_to_8_every_plan(fmt, shape):
    rows, cols = shape
    w = kqgen.weights(fmt, rows, cols, 640, fmt, rows, cols)
    x = kqgen.activations(8, cols, 641, rows, cols)
    y_ref, s = oracle.matvec(fmt, w, rows, cols, x, nthreads=NTHREADS)
    ys = {}
    for ntok in range(1, 9):
        note("ntok matrix fmt=%d %dx%d ntok=%d" % (fmt, rows, cols, ntok))
        ys[ntok] = gpu_matvec(fmt, w, rows, cols, x[:ntok], ldx=cols + 4, ldy=rows + 1)
        check_tol(ys[ntok], y_ref[:ntok], s[:ntok], "fmt %d %dx%d ntok %d" % (fmt, rows, cols, ntok))
    for group in NTOK_SHAPES[shape]:
        top = max(group)
        for ntok in group:
            assert np.array_equal(_bits(ys[ntok]), _bits(ys[top][:ntok])), (ntok, top)


@pytest.mark.parametrize("swapped", [False, True])
def test_kv_pair_every_ntok_set_equals_singles(swapped):
    """The mixed Q6_K/Q5_K K/V pair (separate x planes) at ntok 1..8: the set
    launch bitwise equal to each tensor's own call, within tolerance."""
    tensors = wl.kv_pair(swapped=swapped)[0]
    t = torch()
    ws = {T.name: kqgen.weights(T.fmt, T.rows, T.cols, *T.wkey) for T in tensors}
    for ntok in range(1, 9):
        xs = {T.xkey: kqgen.activations(ntok, T.cols, *T.xkey) for T in tensors}
        note("kv pair every ntok swapped=%s ntok=%d" % (swapped, ntok))
        ys = {T.name: t.full((ntok, T.rows), float("nan"), dtype=t.float32, device="cuda") for T in tensors}
        kq.kq_matvec_set([dict(fmt=T.fmt, w=dev(ws[T.name].reshape(-1)), x=dev(xs[T.xkey]), y=ys[T.name],
                               rows=T.rows, cols=T.cols) for T in tensors], ntok=ntok)
        for T in tensors:
            y = host(ys[T.name])
            y_ref, s = oracle.matvec(T.fmt, ws[T.name], T.rows, T.cols, xs[T.xkey])
            check_tol(y, y_ref, s, "pair %s ntok %d" % (T.name, ntok))
            single = gpu_matvec(T.fmt, ws[T.name], T.rows, T.cols, xs[T.xkey])
            assert np.array_equal(_bits(single), _bits(y)), (T.name, ntok)


# (fmt, rows, cols, x index): every plan, shared and separate x planes
SET16 = [(Q4_K, 4096, 6656, 0), (Q4_K, 4096, 6656, 0), (Q6_K, 256, 6656, 0), (Q6_K, 256, 6656, 0),
         (Q5_K, 1100, 2560, 1), (Q6_K, 1100, 2304, 1), (Q4_K, 300, 768, 2), (Q5_K, 64, 256, 2),
         (Q6_K, 2000, 6656, 3), (Q4_K, 130, 19968, 4), (Q5_K, 17, 1024, 5), (Q6_K, 16448, 512, 6),
         (Q4_K, 1, 256, 7), (Q5_K, 4100, 6656, 0), (Q6_K, 513, 2560, 1), (Q4_K, 2050, 5120, 8)]


@pytest.mark.parametrize("ntok", [1, 2, 5])
def test_sixteen_member_set(ntok):
    t = torch()
    xcols = {}
    for f, r, c, xi in SET16:
        xcols[xi] = max(c, xcols.get(xi, 0))      # a shared plane is as wide as its widest reader
    xs = {xi: kqgen.activations(ntok, c, 650, xi, ntok) for xi, c in xcols.items()}
    dxs = {xi: dev(v) for xi, v in xs.items()}
    ws = [kqgen.weights(f, r, c, 651, i) for i, (f, r, c, _) in enumerate(SET16)]
    ys = [t.full((ntok, r), float("nan"), dtype=t.float32, device="cuda") for (_, r, _, _) in SET16]
    note("sixteen-member set ntok=%d" % ntok)
    kq.kq_matvec_set([dict(fmt=f, w=dev(w.reshape(-1)), x=dxs[xi], y=y, rows=r, cols=c, ldx=xcols[xi])
                      for (f, r, c, xi), w, y in zip(SET16, ws, ys)], ntok=ntok)
    for i, ((f, r, c, xi), w, y) in enumerate(zip(SET16, ws, ys)):
        yh = host(y)
        x = np.ascontiguousarray(xs[xi][:, :c])
        y_ref, s = oracle.matvec(f, w, r, c, x, nthreads=NTHREADS)
        check_tol(yh, y_ref, s, "set16 member %d fmt %d %dx%d" % (i, f, r, c))
        assert np.array_equal(_bits(yh), _bits(gpu_matvec(f, w, r, c, x, ldx=xcols[xi]))), i


# ---- invariants: y(2^k x) = 2^k y bitwise (every rounding scales with x);
# permuting the rows of W permutes y bitwise (a row's result does not
# depend on where the row sits)

@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("entry,ntok", [("kq_matvec", 1), ("kq_matvec", 4), ("kq_matvec16", 16), ("kq_matmul", 40)])
def test_power_of_two_scaling_bitwise(fmt, entry, ntok):
    rows, cols = 1100, 6656
    w = kqgen.weights(fmt, rows, cols, 660, fmt)
    x = kqgen.activations(ntok, cols, 661, fmt, ntok)
    note("scaling %s fmt=%d ntok=%d" % (entry, fmt, ntok))
    y = _run(entry, fmt, w, rows, cols, x)
    for k in (5, -7):
        yk = _run(entry, fmt, w, rows, cols, (x * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(_bits(yk), _bits((y * np.float32(2.0 ** k)).astype(np.float32))), k


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("entry,ntok", [("kq_matvec", 1), ("kq_matvec", 3), ("kq_matvec16", 16), ("kq_matmul", 40)])
def test_row_permutation_bitwise(fmt, entry, ntok):
    rows, cols = 1100, 6656
    w = kqgen.weights(fmt, rows, cols, 662, fmt)
    x = kqgen.activations(ntok, cols, 663, fmt, ntok)
    perm = np.random.default_rng(664).permutation(rows)
    note("row permutation %s fmt=%d ntok=%d" % (entry, fmt, ntok))
    y = _run(entry, fmt, w, rows, cols, x)
    yp = _run(entry, fmt, np.ascontiguousarray(w[perm]), rows, cols, x)
    assert np.array_equal(_bits(yp), _bits(y[:, perm]))


# ---- the workspace: freed and taken afresh, and grown past its first size
# without a synchronizing call in between

def test_workspace_release_and_regrow():
    fmt, rows, cols = Q4_K, 4100, 6656
    w = kqgen.weights(fmt, rows, cols, 670)
    x = kqgen.activations(2, cols, 671)
    note("workspace release")
    y1 = gpu_matvec(fmt, w, rows, cols, x)
    torch().cuda.synchronize()
    kq.kq_release_workspace()
    y2 = gpu_matvec(fmt, w, rows, cols, x)
    assert np.array_equal(_bits(y1), _bits(y2))
    # 8 token planes of a 19,200 x 65,536 Q4_K matrix take about 79 MB of
    # shared-tile sums, more than the first workspace holds
    rows, cols, ntok = 19200, 65536, 8
    w = kqgen.weights(fmt, rows, cols, 672)
    x = kqgen.activations(ntok, cols, 673)
    note("workspace growth: Q4_K %dx%d ntok=%d" % (rows, cols, ntok))
    ya = gpu_matvec(fmt, w, rows, cols, x)
    yb = gpu_matvec(fmt, w, rows, cols, x)
    assert np.array_equal(_bits(ya), _bits(yb))
    idx = np.unique(np.concatenate([np.arange(0, 70), np.arange(rows - 70, rows),
                                    np.random.default_rng(674).integers(0, rows, 300)]))
    y_ref, s = oracle.matvec(fmt, w, rows, cols, x, row_idx=idx, nthreads=NTHREADS)
    check_tol(ya[:, idx], y_ref, s, "workspace growth")


# ---- the large workloads at full size, every row

def test_lm_head_scale_q6k_all_rows():
    """All 202,048 rows of the 202,048 x 6656 Q6_K matvec, in the launch the
    benchmark times, against the multithreaded oracle."""
    [[T]] = wl.lm_head()
    w = kqgen.weights(T.fmt, T.rows, T.cols, *T.wkey)
    x = kqgen.activations(1, T.cols, *T.xkey)
    note("lm_head Q6_K 202048x6656 all rows")
    y = gpu_matvec(T.fmt, w, T.rows, T.cols, x)
    y_ref, s = oracle.matvec(T.fmt, w, T.rows, T.cols, x, nthreads=NTHREADS)
    check_tol(y, y_ref, s, "lm_head all rows")


def test_stream52_all_layers_all_rows():
    """All 52 layers of the Q/K/V/gate stream (one set launch per layer, as
    the benchmark runs them), every row of every tensor."""
    t = torch()
    for li, tensors in enumerate(wl.qkvg_stream()):
        ws = {T.name: kqgen.weights(T.fmt, T.rows, T.cols, *T.wkey) for T in tensors}
        xs = {T.xkey: kqgen.activations(1, T.cols, *T.xkey) for T in tensors}
        dx = {k: dev(v) for k, v in xs.items()}
        ys = {T.name: t.full((1, T.rows), float("nan"), dtype=t.float32, device="cuda") for T in tensors}
        note("stream layer %d" % li)
        kq.kq_matvec_set([dict(fmt=T.fmt, w=dev(ws[T.name].reshape(-1)), x=dx[T.xkey], y=ys[T.name],
                               rows=T.rows, cols=T.cols) for T in tensors])
        for T in tensors:
            y_ref, s = oracle.matvec(T.fmt, ws[T.name], T.rows, T.cols, xs[T.xkey], nthreads=NTHREADS)
            check_tol(host(ys[T.name]), y_ref, s, "stream layer %d %s" % (li, T.name))


# ---- the pipelined producer/consumer kernel against the one-wave kernel:
# launches whose tensors all run in 32-row tiles at ntok <= 2 may take the
# pipelined kernel (by default only with at least four segment steps a
# compute unit; debug mode 2 at any size); forbidding it makes the same
# launch run in the one-wave kernel, and both must give the same bits (same
# plan, same sums in the same order).

PIPE_CASES = [
    ("qkvg set", [(Q4_K, 4096, 6656, 0), (Q6_K, 256, 6656, 0), (Q6_K, 256, 6656, 0), (Q4_K, 4096, 6656, 0)], 1),
    ("q5 set ntok2", [(Q5_K, 4096, 6656, 0), (Q4_K, 256, 6656, 0)], 2),
    ("kv pair small", [(Q6_K, 256, 6656, 0), (Q5_K, 256, 6656, 1)], 1),
    ("ragged large", [(Q6_K, 20037, 6656, 0)], 1),
    ("short rows", [(Q4_K, 3000, 512, 0), (Q5_K, 77, 1024, 1), (Q6_K, 1, 256, 2)], 2),
    ("one-block segments", [(Q6_K, 16448, 512, 0), (Q4_K, 37, 512, 1)], 1),
    # one-wave kernel: odd blocks; x beside a ring does not fit (long rows,
    # Q6_K at two token planes)
    ("mixed plans", [(Q4_K, 4096, 6656, 0), (Q6_K, 300, 2304, 1)], 1),
    ("long rows", [(Q4_K, 2050, 19968, 0)], 1),
    ("q6 ntok2", [(Q6_K, 4096, 6656, 0)], 2),
]
ONE_WAVE_CASES = ("mixed plans", "long rows", "q6 ntok2")
PC_CASES = ("qkvg set", "q5 set ntok2", "kv pair small", "ragged large", "one-block segments")
# of PC_CASES, those with enough steps to take the pipelined kernel by
# default on a 256-compute-unit GPU (1,768 to 8,151 steps; the others 208
# and 516)
DEFAULT_PC_CASES = ("qkvg set", "q5 set ntok2", "ragged large")


@pytest.mark.parametrize("name,specs,ntok", PIPE_CASES, ids=[c[0] for c in PIPE_CASES])
def test_pipelined_kernel_bitwise_equals_one_wave_kernel(name, specs, ntok):
    t = torch()
    xcols = {}
    for f, r, c, xi in specs:
        xcols[xi] = max(c, xcols.get(xi, 0))
    xs = {xi: kqgen.activations(ntok, c, 680, xi, ntok) for xi, c in xcols.items()}
    dxs = {xi: dev(v) for xi, v in xs.items()}
    ws = [kqgen.weights(f, r, c, 681, i, r) for i, (f, r, c, _) in enumerate(specs)]
    dws = [dev(w.reshape(-1)) for w in ws]
    outs = {}
    for mode in (2, 0):
        kq.kq_debug_set_pipeline(mode)
        try:
            ys = [t.full((ntok, r), float("nan"), dtype=t.float32, device="cuda") for (_, r, _, _) in specs]
            note("pipelined vs one-wave: %s ntok=%d pipeline mode=%d" % (name, ntok, mode))
            members = kq.make_set([dict(fmt=f, w=dw, x=dxs[xi], y=y, rows=r, cols=c, ldx=xcols[xi])
                                   for (f, r, c, xi), dw, y in zip(specs, dws, ys)])
            kernel = kq.kq_debug_plan_kernel(members, ntok=ntok)
            if mode == 0 or name in ONE_WAVE_CASES:
                assert kernel == "kq_matvec_kernel<%d>" % ntok, kernel
            elif name in PC_CASES:
                assert kernel == "kq_pc_kernel<%d>" % ntok, kernel
            kq.kq_matvec_set(members, ntok=ntok)
            outs[mode] = [host(y) for y in ys]
        finally:
            kq.kq_debug_set_pipeline(1)
    if t.cuda.get_device_properties(0).multi_processor_count == 256 and name in PC_CASES + ONE_WAVE_CASES:
        kernel = kq.kq_debug_plan_kernel(members, ntok=ntok)
        want = "kq_pc_kernel<%d>" if name in DEFAULT_PC_CASES else "kq_matvec_kernel<%d>"
        assert kernel == want % ntok, (name, kernel)
    for i, ((f, r, c, xi), w) in enumerate(zip(specs, ws)):
        assert np.array_equal(_bits(outs[2][i]), _bits(outs[0][i])), i
        x = np.ascontiguousarray(xs[xi][:, :c])
        idx = np.unique(np.concatenate([np.arange(min(r, 70)), np.arange(max(0, r - 70), r),
                                        np.random.default_rng(682).integers(0, r, 300)]))
        y_ref, s = oracle.matvec(f, w, r, c, x, row_idx=idx, nthreads=NTHREADS)
        check_tol(outs[2][i][:, idx], y_ref, s, "%s member %d" % (name, i))


# ---- the pipelined kernel on small shapes (debug mode 2: it takes any
# launch that fits, not only those with enough steps): ragged tiles, runs
# shorter than a tile row, a single step; bitwise against the one-wave
# kernel and within the bound of the oracle; zero x gives exact zeros and a
# one-hot x the column of W.
# (A Q6_K matrix of 6656 columns at two token planes is left out: its x
# and a full ring do not fit one workgroup's LDS, so it always takes the
# one-wave kernel.)
PC_SMALL_SHAPES = [(1, 512), (3, 512), (31, 2560), (33, 6656), (64, 6656), (130, 2560), (257, 6656)]
PC_SMALL_CASES = [(f, r, c, n) for n in (1, 2) for (r, c) in PC_SMALL_SHAPES for f in FORMATS
                  if not (f == Q6_K and n == 2 and c == 6656)]


@pytest.mark.parametrize("fmt,rows,cols,ntok", PC_SMALL_CASES)
def test_pipelined_kernel_small_shapes(fmt, rows, cols, ntok):
    t = torch()
    w = kqgen.weights(fmt, rows, cols, 690, fmt, rows, cols)
    dw = dev(w.reshape(-1))
    W = oracle.dequant(fmt, w, rows, cols)
    xs = [kqgen.activations(ntok, cols, 691, rows, cols), np.zeros((ntok, cols), np.float32)]
    # one-hot: token 0 picks the last column (the last block of every row),
    # token 1 the first
    hot = [cols - 1, 0][:ntok]
    onehot = np.zeros((ntok, cols), np.float32)
    for tk, j in enumerate(hot):
        onehot[tk, j] = 1.0
    xs.append(onehot)
    for k, x in enumerate(xs):
        dx = dev(x)
        outs = {}
        for mode in (2, 0):
            kq.kq_debug_set_pipeline(mode)
            try:
                y = t.full((ntok, rows), float("nan"), dtype=t.float32, device="cuda")
                note("pipelined small shape fmt=%d %dx%d ntok=%d input %d mode %d" % (fmt, rows, cols, ntok, k, mode))
                members = kq.make_set([dict(fmt=fmt, w=dw, x=dx, y=y, rows=rows, cols=cols)])
                want = "kq_pc_kernel<%d>" if mode == 2 else "kq_matvec_kernel<%d>"
                assert kq.kq_debug_plan_kernel(members, ntok=ntok) == want % ntok
                kq.kq_matvec_set(members, ntok=ntok)
                outs[mode] = host(y)
            finally:
                kq.kq_debug_set_pipeline(1)
        assert np.array_equal(_bits(outs[2]), _bits(outs[0])), k
        if k == 0:
            y_ref, s = oracle.matvec(fmt, w, rows, cols, x, nthreads=NTHREADS)
            check_tol(outs[2], y_ref, s, "pipelined small shape")
        elif k == 1:
            assert not outs[2].any()
        else:
            for tk, j in enumerate(hot):
                assert np.array_equal(outs[2][tk], W[:, j].astype(np.float32)), tk


# ---- token-plane groups: at ntok >= 3 a launch may run each tensor's planes
# as G groups (members of one launch, planned as at the full ntok); every G
# must give the bits of G = 1.  The automatic choice: the smallest divisor
# of ntok with at most 2 planes a group whose segments fit one round of
# resident workgroups, else the largest divisor that fits, else 2 at ntok 8.
PLANE_CASES = [
    ("kv pair", [(Q6_K, 256, 6656, 0), (Q5_K, 256, 6656, 1)]),
    ("ragged odd blocks", [(Q4_K, 300, 2304, 0), (Q6_K, 77, 768, 1), (Q5_K, 65, 256, 0)]),
    ("attention output", [(Q4_K, 6656, 4096, 0)]),
]
# automatic G on a 256-compute-unit GPU (one-wave capacity 2,048 workgroups):
# the K/V pair has 208 segments at any ntok, the attention output 832
AUTO_GROUPS = {("kv pair", 3): 3, ("kv pair", 4): 2, ("kv pair", 6): 3, ("kv pair", 8): 4,
               ("attention output", 3): 1, ("attention output", 4): 2, ("attention output", 6): 2,
               ("attention output", 8): 2}


@pytest.mark.parametrize("name,specs", PLANE_CASES, ids=[c[0] for c in PLANE_CASES])
@pytest.mark.parametrize("ntok", [3, 4, 6, 8])
def test_plane_groups_bitwise(name, specs, ntok):
    t = torch()
    xcols = {}
    for f, r, c, xi in specs:
        xcols[xi] = max(c, xcols.get(xi, 0))
    xs = {xi: kqgen.activations(ntok, c, 700, xi, ntok) for xi, c in xcols.items()}
    dxs = {xi: dev(v) for xi, v in xs.items()}
    ws = [kqgen.weights(f, r, c, 701, i, r) for i, (f, r, c, _) in enumerate(specs)]
    dws = [dev(w.reshape(-1)) for w in ws]
    groups = [g for g in range(1, ntok + 1) if ntok % g == 0 and len(specs) * g <= 16]

    def run(g, noalloc=False):
        kq.kq_debug_set_plane_groups(g)
        try:
            ys = [t.full((ntok, r), float("nan"), dtype=t.float32, device="cuda") for (_, r, _, _) in specs]
            members = kq.make_set([dict(fmt=f, w=dw, x=dxs[xi], y=y, rows=r, cols=c, ldx=xcols[xi])
                                   for (f, r, c, xi), dw, y in zip(specs, dws, ys)])
            want = g if g > 0 else AUTO_GROUPS.get((name, ntok))
            got = kq.kq_debug_plan_plane_groups(members, ntok=ntok)
            if want is not None and (g > 0 or t.cuda.get_device_properties(0).multi_processor_count == 256):
                assert got == want, (g, got, want)
            note("plane groups: %s ntok=%d G=%d (planned %d)%s" % (name, ntok, g, got, " noalloc" if noalloc else ""))
            if noalloc:
                kq.kq_matvec_set_noalloc(members, ntok=ntok)
            else:
                kq.kq_matvec_set(members, ntok=ntok)
            return [host(y) for y in ys]
        finally:
            kq.kq_debug_set_plane_groups(0)

    ref = run(1)
    for g in groups[1:] + [0]:
        out = run(g)
        for i in range(len(specs)):
            assert np.array_equal(_bits(out[i]), _bits(ref[i])), (g, i)
    out = run(0, noalloc=True)
    for i in range(len(specs)):
        assert np.array_equal(_bits(out[i]), _bits(ref[i])), ("noalloc", i)
    for i, ((f, r, c, xi), w) in enumerate(zip(specs, ws)):
        x = np.ascontiguousarray(xs[xi][:, :c])
        idx = np.unique(np.concatenate([np.arange(min(r, 70)), np.arange(max(0, r - 70), r),
                                        np.random.default_rng(702).integers(0, r, 200)]))
        y_ref, s = oracle.matvec(f, w, r, c, x, row_idx=idx, nthreads=NTHREADS)
        check_tol(ref[i][:, idx], y_ref, s, "%s member %d" % (name, i))
