"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer decode (codes, scales, mins, headers), the dequantized float32
weights and the embedding rows are compared bit for bit; matvec outputs
(kq_matvec, kq_matvec_set, kq_matvec16, kq_matmul) per row against the
binary64 oracle with |y_gpu - y_ref| <= 1e-4 * sum_j|W_ij x_j| + 1e-6.
Inputs are the seeded synthetic blocks of kqgen.
"""
import numpy as np
import pytest

import kqgen
import oracle
import quant_matvec_amd as kq
from gpu_util import check_tol, dev, gpu_matvec, host, note, torch
from kqgen import FORMATS, Q4_K, Q5_K, Q6_K
from kqgen import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    kq.load()
    oracle.lib()


def special_blocks(fmt):
    """Blocks with subnormal / zero / negative headers and extreme codes."""
    bb = kqgen.BLOCK_BYTES[fmt]
    out = []
    for hdr in (0x0001, 0x03FF, 0x0000, 0x8400, 0x7BFF):   # subnormals, zero, -2^-14, max
        b = np.zeros(bb, np.uint8)
        b[:] = 0xFF
        if fmt == Q6_K:
            b[208:210] = [hdr & 0xFF, hdr >> 8]
        else:
            b[0:2] = [hdr & 0xFF, hdr >> 8]
            b[2:4] = [0x01, 0x00]
        out.append(b)
    out.append(np.zeros(bb, np.uint8))
    return np.stack(out)


@pytest.mark.parametrize("fmt", FORMATS)
def test_unpack_bit_exact(fmt):
    nblocks = 1001          # odd count: Q6_K blocks alternate 4-byte and 2-byte alignment
    blocks = np.concatenate([kqgen.random_blocks(fmt, nblocks - 6, kqgen.rng_for(500, fmt)), special_blocks(fmt)])
    note("unpack fmt=%d nblocks=%d" % (fmt, nblocks))
    t = torch()
    w = dev(blocks.reshape(-1))
    codes = t.empty((nblocks, 256), dtype=t.int32, device="cuda")
    scales = t.empty((nblocks, 16), dtype=t.int32, device="cuda")
    mins = t.empty((nblocks, 16), dtype=t.int32, device="cuda")
    d = t.empty(nblocks, dtype=t.float32, device="cuda")
    dmin = t.empty(nblocks, dtype=t.float32, device="cuda")
    kq.kq_unpack_blocks(fmt, w, nblocks, codes, scales, mins, d, dmin)
    codes, scales, mins, d, dmin = (host(v) for v in (codes, scales, mins, d, dmin))
    for i in range(nblocks):
        ref = oracle.decode_block(fmt, blocks[i].tobytes())
        assert np.array_equal(codes[i], ref["codes"]), i
        assert np.array_equal(scales[i], ref["scale"]), i
        assert np.array_equal(mins[i], ref["min"]), i
        assert np.float32(ref["d"]).tobytes() == d[i].tobytes(), i
        assert np.float32(ref["dmin"]).tobytes() == dmin[i].tobytes(), i


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("rows,cols", [(37, 768), (5, 6656), (2, 256)])
def test_dequant_bit_exact(fmt, rows, cols):
    w = kqgen.weights(fmt, rows, cols, 501, fmt, rows, cols)
    note("dequant fmt=%d rows=%d cols=%d" % (fmt, rows, cols))
    t = torch()
    out = t.empty((rows, cols + 8), dtype=t.float32, device="cuda")
    kq.kq_dequant(fmt, dev(w.reshape(-1)), rows, cols, out, ldw=cols + 8)
    got = host(out)[:, :cols]
    ref = oracle.dequant(fmt, w, rows, cols).astype(np.float32)   # exact weight, rounded once
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


SHAPES = [(1, 256), (3, 512), (64, 6656), (65, 768), (130, 2560), (257, 6656), (200, 19968)]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_matvec_parity(fmt, rows, cols):
    w = kqgen.weights(fmt, rows, cols, 502, fmt, rows, cols)
    x = kqgen.activations(1, cols, 503, cols)
    note("matvec fmt=%d rows=%d cols=%d" % (fmt, rows, cols))
    y = gpu_matvec(fmt, w, rows, cols, x)
    y_ref, s = oracle.matvec(fmt, w, rows, cols, x)
    check_tol(y, y_ref, s, "fmt %d %dx%d" % (fmt, rows, cols))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("ntok", [2, 3, 8])
def test_matvec_ntok(fmt, ntok):
    rows, cols = 131, 6656
    w = kqgen.weights(fmt, rows, cols, 504, fmt)
    x = kqgen.activations(ntok, cols, 505, ntok)
    note("matvec ntok fmt=%d ntok=%d" % (fmt, ntok))
    y = gpu_matvec(fmt, w, rows, cols, x, ldx=cols + 4, ldy=rows + 3)
    y_ref, s = oracle.matvec(fmt, w, rows, cols, x)
    check_tol(y, y_ref, s, "fmt %d ntok %d" % (fmt, ntok))
    # every column is bitwise the call with fewer planes of the same plan on
    # it: ntok 1 and 2 share 32-row tiles of two-block segments, ntok 3 and
    # more 64-row tiles of one-block segments (at most 1024 rows)
    ref = 1 if ntok <= 2 else 3
    for t in range(ntok):
        xr = np.repeat(x[t:t + 1], ref, axis=0)
        y1 = gpu_matvec(fmt, w, rows, cols, xr)
        assert np.array_equal(y1[0].view(np.uint32), y[t].view(np.uint32)), t


def test_config1_single_q4k():
    [[T]] = wl.single_q4k()
    w = kqgen.weights(T.fmt, T.rows, T.cols, *T.wkey)
    x = kqgen.activations(1, T.cols, *T.xkey)
    note("config single Q4_K 256x6656")
    y = gpu_matvec(T.fmt, w, T.rows, T.cols, x)
    y_ref, s = oracle.matvec(T.fmt, w, T.rows, T.cols, x)
    check_tol(y, y_ref, s, "single Q4_K")
    # run to run: bitwise identical
    y2 = gpu_matvec(T.fmt, w, T.rows, T.cols, x)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


def _set_inputs(tensors, ntok):
    ws, xs = {}, {}
    for T in tensors:
        ws[T.name] = kqgen.weights(T.fmt, T.rows, T.cols, *T.wkey)
        if T.xkey not in xs:
            xs[T.xkey] = kqgen.activations(ntok, T.cols, *T.xkey)
    return ws, xs


def _run_set(tensors, ws, xs, ntok):
    t = torch()
    dw = {k: dev(v.reshape(-1)) for k, v in ws.items()}
    dx = {k: dev(v) for k, v in xs.items()}
    ys = {T.name: t.full((ntok, T.rows), float("nan"), dtype=t.float32, device="cuda") for T in tensors}
    kq.kq_matvec_set([dict(fmt=T.fmt, w=dw[T.name], x=dx[T.xkey], y=ys[T.name], rows=T.rows, cols=T.cols)
                      for T in tensors], ntok=ntok)
    return {k: host(v) for k, v in ys.items()}


def test_qkvg_set_matches_oracle_and_singles():
    tensors = wl.qkvg_set()[0]
    ws, xs = _set_inputs(tensors, 1)
    note("qkvg set (4096/256/256/4096 x 6656)")
    ys = _run_set(tensors, ws, xs, 1)
    for T in tensors:
        x = xs[T.xkey]
        y_ref, s = oracle.matvec(T.fmt, ws[T.name], T.rows, T.cols, x)
        check_tol(ys[T.name], y_ref, s, "set " + T.name)
        single = gpu_matvec(T.fmt, ws[T.name], T.rows, T.cols, x)
        assert np.array_equal(single.view(np.uint32), ys[T.name].view(np.uint32)), T.name


@pytest.mark.parametrize("swapped", [False, True])
@pytest.mark.parametrize("ntok", [1, 2, 4, 8])
def test_kv_pair_separate_planes(swapped, ntok):
    tensors = wl.kv_pair(swapped=swapped)[0]
    ws, xs = _set_inputs(tensors, ntok)
    note("kv pair swapped=%s ntok=%d" % (swapped, ntok))
    ys = _run_set(tensors, ws, xs, ntok)
    for T, other in ((tensors[0], tensors[1]), (tensors[1], tensors[0])):
        y_ref, s = oracle.matvec(T.fmt, ws[T.name], T.rows, T.cols, xs[T.xkey])
        check_tol(ys[T.name], y_ref, s, "pair " + T.name)
        single = gpu_matvec(T.fmt, ws[T.name], T.rows, T.cols, xs[T.xkey])
        assert np.array_equal(single.view(np.uint32), ys[T.name].view(np.uint32))
        # the check can see a tensor that reads the other tensor's x plane:
        # an oracle fed the wrong plane does not pass it
        y_wrong, _ = oracle.matvec(T.fmt, ws[T.name], T.rows, T.cols, xs[other.xkey])
        with pytest.raises(AssertionError):
            check_tol(ys[T.name], y_wrong, s, "wrong plane")


@pytest.mark.parametrize("fmt", FORMATS)
def test_edge_cases(fmt):
    rows, cols = 70, 512
    w = kqgen.weights(fmt, rows, cols, 506, fmt)
    note("edge cases fmt=%d" % fmt)
    # zero x gives exactly zero
    y = gpu_matvec(fmt, w, rows, cols, np.zeros((1, cols), np.float32))
    assert not y.any()
    # one-hot x gives a column of W (exactly: one product, one rounding)
    W = oracle.dequant(fmt, w, rows, cols)
    for j in (0, 31, 32, 255, 256, 511):
        x = np.zeros((1, cols), np.float32)
        x[0, j] = 1.0
        y = gpu_matvec(fmt, w, rows, cols, x)
        assert np.array_equal(y[0], W[:, j].astype(np.float32)), j
    # zero headers give zero rows
    wz = w.copy().reshape(-1, kqgen.BLOCK_BYTES[fmt])
    if fmt == Q6_K:
        wz[:, 208:210] = 0
    else:
        wz[:, 0:4] = 0
    y = gpu_matvec(fmt, wz, rows, cols, kqgen.activations(1, cols, 507))
    assert not y.any()


@pytest.mark.parametrize("fmt", (Q4_K, Q5_K))
def test_near_cancelling_blocks(fmt):
    """Deferred scaling rounds d*sc*sum(q x) and dmin*m*sum(x) separately;
    on blocks where d*sc*q nearly cancels dmin*m the result must still meet
    the per-row bound."""
    rows, cols = 64, 2560
    rng = kqgen.rng_for(508, fmt)
    w = kqgen.weights(fmt, rows, cols, 509, fmt).reshape(-1, kqgen.BLOCK_BYTES[fmt]).copy()
    # d = dmin, sc_j = m_j = 8 for all sub-blocks, codes 0..2: W = 8*d*(q-1)
    w[:, 0:2] = w[:, 2:4]
    w[:, 4:16] = [8, 8, 8, 8, 8, 8, 8, 8, 0x88, 0x88, 0x88, 0x88]
    qs0 = 16 if fmt == Q4_K else 48
    q = rng.choice(3, size=(w.shape[0], 256), p=[0.05, 0.9, 0.05])   # mostly W = 0
    lo, hi = q[:, :128].reshape(-1, 4, 32), q[:, 128:].reshape(-1, 4, 32)
    codes = np.concatenate([lo, hi], axis=2)    # per group: 32 low + 32 high elements
    packed = (codes[:, :, :32] | (codes[:, :, 32:] << 4)).reshape(-1, 128)
    w[:, qs0:qs0 + 128] = packed.astype(np.uint8)
    if fmt == Q5_K:
        w[:, 16:48] = 0
    x = kqgen.activations(1, cols, 510)
    note("near-cancelling fmt=%d" % fmt)
    y = gpu_matvec(fmt, w, rows, cols, x)
    y_ref, s = oracle.matvec(fmt, w, rows, cols, x)
    check_tol(y, y_ref, s, "near-cancelling")


def test_lm_head_scale_q6k_sampled():
    """The 202,048 x 6656 Q6_K matvec at full size, in the launch the
    benchmark times; the oracle checks a sample of rows (every row tile's
    first and last row, the tail tile, and random rows)."""
    [[T]] = wl.lm_head()
    note("lm_head Q6_K 202048x6656 (full size)")
    w = kqgen.weights(T.fmt, T.rows, T.cols, *T.wkey)
    x = kqgen.activations(1, T.cols, *T.xkey)
    y = gpu_matvec(T.fmt, w, T.rows, T.cols, x)
    assert np.isfinite(y).all()
    rng = np.random.default_rng(7)
    idx = np.unique(np.concatenate([np.arange(0, T.rows, 64), np.arange(63, T.rows, 64),
                                    np.arange(T.rows - 100, T.rows), rng.integers(0, T.rows, 2000)]))
    y_ref, s = oracle.matvec(T.fmt, w, T.rows, T.cols, x, row_idx=idx, nthreads=8)
    check_tol(y[:, idx], y_ref, s, "lm_head sampled")


def test_stream_layers_sampled():
    """Two layers of the 52-layer stream (a Q4_K and a Q5_K layer) at full
    size, one set launch each, rows sampled against the oracle."""
    layers = wl.qkvg_stream(layers=2)
    for tensors in layers:
        ws, xs = _set_inputs(tensors, 1)
        note("stream layer fmt q/gate=%d" % tensors[0].fmt)
        ys = _run_set(tensors, ws, xs, 1)
        for T in tensors:
            idx = np.arange(0, T.rows, 7)
            y_ref, s = oracle.matvec(T.fmt, ws[T.name], T.rows, T.cols, xs[T.xkey], row_idx=idx, nthreads=8)
            check_tol(ys[T.name][:, idx], y_ref, s, "layer " + T.name)


def test_read_probe_runs():
    """The streaming-read calibration launches and leaves its buffer alone."""
    t = torch()
    note("read probe over 64 MiB")
    buf = t.arange(1 << 24, dtype=t.int32, device="cuda")
    sink = t.zeros(1, dtype=t.int32, device="cuda")
    kq.kq_debug_read_probe(buf, sink)
    t.cuda.synchronize()
    assert int(buf[12345]) == 12345 and int(buf[-1]) == (1 << 24) - 1


# Matrices of more than 1024 rows with an even number of blocks a row run
# in 32-row tiles (two lanes a row, a segment a step) at one token plane,
# and at two up to 16384 rows; otherwise, and with an odd number of blocks,
# in 64-row tiles.  Rows 16461 leave a ragged last tile of 13 rows.
@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("rows,cols", [(16461, 6656), (16448, 512), (16449, 768)])
def test_large_matrix_tiles_sampled(fmt, rows, cols):
    w = kqgen.weights(fmt, rows, cols, 621, fmt, rows, cols)
    x = kqgen.activations(1, cols, 622, cols)
    note("large matrix fmt=%d %dx%d" % (fmt, rows, cols))
    y = gpu_matvec(fmt, w, rows, cols, x, ldy=rows + 3)
    assert np.isfinite(y).all()
    rng = np.random.default_rng(11)
    idx = np.unique(np.concatenate([np.arange(0, 96), np.arange(rows - 45, rows),
                                    np.arange(31, rows, 32), rng.integers(0, rows, 600)]))
    y_ref, s = oracle.matvec(fmt, w, rows, cols, x, row_idx=idx, nthreads=8)
    check_tol(y[:, idx], y_ref, s, "large fmt %d %dx%d" % (fmt, rows, cols))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("ntok", [2, 3, 8])
def test_large_matrix_ntok_columns_bitwise(fmt, ntok):
    """In 32-row tiles too, each column of an ntok call is bitwise the
    ntok=1 call on that column."""
    rows, cols = 16416, 2560
    w = kqgen.weights(fmt, rows, cols, 623, fmt, ntok)
    x = kqgen.activations(ntok, cols, 624, ntok)
    note("large matrix ntok fmt=%d ntok=%d" % (fmt, ntok))
    y = gpu_matvec(fmt, w, rows, cols, x)
    for t in range(ntok):
        y1 = gpu_matvec(fmt, w, rows, cols, x[t:t + 1])
        assert np.array_equal(y1[0].view(np.uint32), y[t].view(np.uint32)), t
    idx = np.arange(0, rows, 61)
    y_ref, s = oracle.matvec(fmt, w, rows, cols, x, row_idx=idx, nthreads=8)
    check_tol(y[:, idx], y_ref, s, "large ntok fmt %d" % fmt)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("ntok", [2, 3, 8])
def test_mid_matrix_ntok_columns_bitwise(fmt, ntok):
    """A 4100-row matrix runs in 32-row tiles at one token plane and at two,
    in 64-row tiles at three and eight: every column is still bitwise the
    one-plane call on it (the same two-block segments, summed alike)."""
    rows, cols = 4100, 2560
    w = kqgen.weights(fmt, rows, cols, 625, fmt, ntok)
    x = kqgen.activations(ntok, cols, 626, ntok)
    note("mid matrix ntok fmt=%d ntok=%d" % (fmt, ntok))
    y = gpu_matvec(fmt, w, rows, cols, x)
    for t in range(ntok):
        y1 = gpu_matvec(fmt, w, rows, cols, x[t:t + 1])
        assert np.array_equal(y1[0].view(np.uint32), y[t].view(np.uint32)), t
    y_ref, s = oracle.matvec(fmt, w, rows, cols, x)
    check_tol(y, y_ref, s, "mid ntok fmt %d" % fmt)


@pytest.mark.parametrize("fmt", FORMATS)
def test_long_row_plans_across_ntok(fmt):
    """Rows of 26 blocks run in 32-row tiles at ntok 1 and 2 and in 64-row
    tiles at ntok 3 and more, with two-block segments in both: planes match
    bitwise between calls of the same plan (and across the two heights),
    and every call meets the tolerance."""
    rows, cols = 4100, 6656
    w = kqgen.weights(fmt, rows, cols, 627, fmt)
    x = kqgen.activations(8, cols, 628, fmt)
    note("long-row plans fmt=%d" % fmt)
    y1 = np.concatenate([gpu_matvec(fmt, w, rows, cols, x[t:t + 1]) for t in range(2)])
    y2 = gpu_matvec(fmt, w, rows, cols, x[:2])
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    y3 = gpu_matvec(fmt, w, rows, cols, x[:3])
    y8 = gpu_matvec(fmt, w, rows, cols, x)
    assert np.array_equal(y3.view(np.uint32), y8[:3].view(np.uint32))
    y_ref, s = oracle.matvec(fmt, w, rows, cols, x, nthreads=8)
    check_tol(y2, y_ref[:2], s[:2], "long rows ntok 2")
    check_tol(y8, y_ref, s, "long rows ntok 8")


@pytest.mark.parametrize("fmt", FORMATS)
def test_long_rows_between_small_and_tall_keep_two_block_segments(fmt):
    """Rows of 20 blocks on a matrix of 16448 rows (between 16384 and
    65536 rows, where four-block segments measured slower): two-block
    segments in 32-row tiles at ntok 1 and in 64-row tiles at ntok 2 and 3,
    so every plane is bitwise the one-plane call on it."""
    rows, cols = 16448, 5120
    w = kqgen.weights(fmt, rows, cols, 629, fmt)
    x = kqgen.activations(3, cols, 630, fmt)
    note("long rows mid band fmt=%d" % fmt)
    y1 = np.concatenate([gpu_matvec(fmt, w, rows, cols, x[t:t + 1]) for t in range(3)])
    for ntok in (2, 3):
        y = gpu_matvec(fmt, w, rows, cols, x[:ntok])
        assert np.array_equal(y1[:ntok].view(np.uint32), y.view(np.uint32)), ntok
    y_ref, s = oracle.matvec(fmt, w, rows, cols, x, nthreads=8)
    check_tol(y1, y_ref, s, "long rows mid band")


def test_mixed_tile_set_matches_singles():
    """A set of a 32-row-tile matrix and 64-row-tile ones: every member
    bitwise equal to its own kq_matvec call."""
    t = torch()
    specs = [(Q6_K, 16448, 2560), (Q4_K, 4096, 2560), (Q5_K, 300, 2560)]
    ws = [kqgen.weights(f, r, c, 625, i) for i, (f, r, c) in enumerate(specs)]
    x = kqgen.activations(1, 2560, 626)
    note("mixed tile set")
    dx = dev(x)
    dws = [dev(w.reshape(-1)) for w in ws]
    ys = [t.full((1, r), float("nan"), dtype=t.float32, device="cuda") for (_, r, _) in specs]
    kq.kq_matvec_set([dict(fmt=f, w=dw, x=dx, y=y, rows=r, cols=c)
                      for (f, r, c), dw, y in zip(specs, dws, ys)], ntok=1)
    for (f, r, c), w, y in zip(specs, ws, ys):
        single = gpu_matvec(f, w, r, c, x)
        assert np.array_equal(single.view(np.uint32), host(y).view(np.uint32)), (f, r)


# ---- the rest of a layer's matvecs and the other release shapes (Ch 6
# Figure 6.6), at full size, each launch as the library runs it: attention
# output (16 blocks a row), the FFN gate/up pair as one set, the FFN down
# (78 blocks a row; Q4_K on even layers, Q6_K on odd), the Q5_K LM head and
# the draft projections (130 blocks a row for the fc).

def _sample_rows(rows, seed, tile=64):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([np.arange(0, rows, tile), np.arange(tile - 1, rows, tile),
                                     np.arange(max(0, rows - 70), rows), rng.integers(0, rows, 1500)]))


def _check_launch(launch, seed):
    ws, xs = _set_inputs(launch, 1)
    ys = _run_set(launch, ws, xs, 1)
    for T in launch:
        y = ys[T.name]
        assert np.isfinite(y).all(), T.name
        idx = _sample_rows(T.rows, seed)
        y_ref, s = oracle.matvec(T.fmt, ws[T.name], T.rows, T.cols, xs[T.xkey], row_idx=idx, nthreads=8)
        check_tol(y[:, idx], y_ref, s, "%s %dx%d" % (T.name, T.rows, T.cols))
        if len(launch) > 1:
            single = gpu_matvec(T.fmt, ws[T.name], T.rows, T.cols, xs[T.xkey])
            assert np.array_equal(single.view(np.uint32), y.view(np.uint32)), T.name


@pytest.mark.parametrize("layer", [0, 1])
def test_layer_rest_sampled(layer):
    for k, launch in enumerate(wl.layer_rest(layer=layer)):
        note("layer rest %d: %s" % (layer, ", ".join("%s fmt=%d %dx%d" % (T.name, T.fmt, T.rows, T.cols)
                                                     for T in launch)))
        _check_launch(launch, 40 + 3 * layer + k)


def test_lm_head_q5k_sampled():
    [launch] = wl.lm_head_q5k()
    note("lm_head Q5_K 202048x6656 (full size)")
    _check_launch(launch, 47)


def test_draft_projections():
    for k, launch in enumerate(wl.draft_projections()):
        note("draft: " + ", ".join("%s fmt=%d %dx%d" % (T.name, T.fmt, T.rows, T.cols) for T in launch))
        _check_launch(launch, 50 + k)


# ---- the embedding lookup (Ch 6 section 6.7): rows of a Q4_K table,
# dequantized, bit for bit against the oracle's element-by-element lookup.

def _gpu_embed(w, rows, cols, ids, ldo=None):
    t = torch()
    ldo = ldo or cols
    table = dev(w.reshape(-1))
    dids = dev(np.asarray(ids, np.int32))
    out = t.full((len(ids), ldo), -7.0, dtype=t.float32, device="cuda")
    kq.kq_embed_rows(Q4_K, table, rows, cols, dids, out, ldo=ldo)
    o = host(out)
    if ldo > cols:
        assert (o[:, cols:] == -7.0).all(), "kernel wrote past cols"
    return o[:, :cols]


def _check_embed(o, ref, ids, rows):
    for k, r in enumerate(ids):
        if 0 <= r < rows:
            assert np.array_equal(o[k].view(np.uint32), ref[k].astype(np.float32).view(np.uint32)), (k, r)
        else:
            assert np.isnan(o[k]).all() and np.isnan(ref[k]).all(), (k, r)


@pytest.mark.parametrize("rows,cols", [(37, 768), (5, 256), (300, 6656)])
def test_embed_rows_bit_exact(rows, cols):
    w = kqgen.weights(Q4_K, rows, cols, 700, rows, cols)
    ids = [0, rows - 1, 3 % rows, 3 % rows, -1, rows, 1 << 30] + list(range(1, rows, 7))
    note("embed rows=%d cols=%d n=%d" % (rows, cols, len(ids)))
    o = _gpu_embed(w, rows, cols, ids, ldo=cols + 4)
    _check_embed(o, oracle.embed(Q4_K, w, rows, cols, ids), ids, rows)
    # the same bits as the dequantization export on those rows
    t = torch()
    full = t.empty((rows, cols), dtype=t.float32, device="cuda")
    kq.kq_dequant(Q4_K, dev(w.reshape(-1)), rows, cols, full)
    fh = host(full)
    for k, r in enumerate(ids):
        if 0 <= r < rows:
            assert np.array_equal(o[k].view(np.uint32), fh[r].view(np.uint32))


def test_embed_rows_full_table_sampled():
    """The 202,048 x 6656 Q4_K table at full size: a decode step's single
    id, then a batch of ids with repeats and both ends of the table."""
    T = wl.embedding_table()
    w = kqgen.weights(T.fmt, T.rows, T.cols, *T.wkey)
    note("embed full table 202048x6656")
    rng = np.random.default_rng(5)
    for ids in ([int(rng.integers(0, T.rows))],
                [0, T.rows - 1, T.rows - 1] + [int(v) for v in rng.integers(0, T.rows, 40)]):
        o = _gpu_embed(w, T.rows, T.cols, ids)
        _check_embed(o, oracle.embed(T.fmt, w, T.rows, T.cols, ids), ids, T.rows)


# ---- up to 16 token planes on the matrix cores (kq_matvec16): the verify
# width of Ch 6 section 6.8.

def _gpu_matvec16(fmt, w_np, rows, cols, x_np, ldy=None):
    t = torch()
    x_np = np.atleast_2d(x_np).astype(np.float32)
    ntok = x_np.shape[0]
    ldy = ldy or rows
    y = t.full((ntok, ldy), float("nan"), dtype=t.float32, device="cuda")
    kq.kq_matvec16(fmt, dev(w_np.reshape(-1)), rows, cols, dev(x_np), y, ntok=ntok, ldy=ldy)
    out = host(y)
    if ldy > rows:
        assert np.isnan(out[:, rows:]).all(), "kernel wrote past rows"
    return out[:, :rows]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("rows,cols,ntok", [(37, 768, 16), (300, 6656, 16), (4100, 2560, 9), (16, 256, 1),
                                            (1, 512, 16), (16400, 768, 16), (16420, 512, 3), (8300, 512, 16),
                                            (40000, 768, 7)])
def test_matvec16_parity(fmt, rows, cols, ntok):
    w = kqgen.weights(fmt, rows, cols, 800, fmt, rows, cols)
    x = kqgen.activations(ntok, cols, 801, ntok, cols)
    note("matvec16 fmt=%d %dx%d ntok=%d" % (fmt, rows, cols, ntok))
    y = _gpu_matvec16(fmt, w, rows, cols, x, ldy=rows + 5)
    y_ref, s = oracle.matvec(fmt, w, rows, cols, x, nthreads=8)
    check_tol(y, y_ref, s, "matvec16 fmt %d %dx%d ntok %d" % (fmt, rows, cols, ntok))
    y2 = _gpu_matvec16(fmt, w, rows, cols, x, ldy=rows + 5)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("fmt", FORMATS)
def test_matvec16_plane_independent_of_ntok(fmt):
    """A token plane's result is bitwise the same whatever ntok is."""
    for rows, cols in ((200, 1536), (8300, 512), (16420, 512), (40000, 768)):   # 4, 2, 2, 1 waves a tile
        w = kqgen.weights(fmt, rows, cols, 802, fmt)
        x = kqgen.activations(16, cols, 803, fmt)
        note("matvec16 planes fmt=%d rows=%d" % (fmt, rows))
        y16 = _gpu_matvec16(fmt, w, rows, cols, x)
        for n in (1, 5, 11):
            yn = _gpu_matvec16(fmt, w, rows, cols, x[:n])
            assert np.array_equal(yn.view(np.uint32), y16[:n].view(np.uint32)), n


def test_matvec16_release_shapes_sampled():
    """Full-size release shapes at the 16-token verify width: the attention
    output (Q4_K) and the Q6_K FFN down (78 blocks a row), rows sampled."""
    for launch in (wl.attn_output(layer=0), wl.ffn_down(layer=1)):
        [T] = launch[0]
        w = kqgen.weights(T.fmt, T.rows, T.cols, *T.wkey)
        x = kqgen.activations(16, T.cols, *T.xkey)
        note("matvec16 %s fmt=%d %dx%d" % (T.name, T.fmt, T.rows, T.cols))
        y = _gpu_matvec16(T.fmt, w, T.rows, T.cols, x)
        idx = _sample_rows(T.rows, 60, tile=16)[:700]
        y_ref, s = oracle.matvec(T.fmt, w, T.rows, T.cols, x, row_idx=idx, nthreads=8)
        check_tol(y[:, idx], y_ref, s, "matvec16 " + T.name)


# ---- a prefill batch (kq_matmul): any number of token planes, each block
# decoded once for 32 tokens (the mul_mm rung of Ch 6 Figure 6.7).

def _gpu_matmul(fmt, w_np, rows, cols, x_np, ldy=None):
    t = torch()
    x_np = np.atleast_2d(x_np).astype(np.float32)
    ntok = x_np.shape[0]
    ldy = ldy or rows
    y = t.full((ntok, ldy), float("nan"), dtype=t.float32, device="cuda")
    kq.kq_matmul(fmt, dev(w_np.reshape(-1)), rows, cols, dev(x_np), y, ntok=ntok, ldy=ldy)
    out = host(y)
    if ldy > rows:
        assert np.isnan(out[:, rows:]).all(), "kernel wrote past rows"
    return out[:, :rows]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("rows,cols,ntok", [(37, 768, 17), (300, 2560, 64), (100, 6656, 130), (16, 256, 1),
                                            (1, 256, 40), (5, 512, 33)])
def test_matmul_parity(fmt, rows, cols, ntok):
    w = kqgen.weights(fmt, rows, cols, 810, fmt, rows, cols)
    x = kqgen.activations(ntok, cols, 811, ntok, cols)
    note("matmul fmt=%d %dx%d ntok=%d" % (fmt, rows, cols, ntok))
    y = _gpu_matmul(fmt, w, rows, cols, x, ldy=rows + 3)
    y_ref, s = oracle.matvec(fmt, w, rows, cols, x, nthreads=8)
    check_tol(y, y_ref, s, "matmul fmt %d %dx%d ntok %d" % (fmt, rows, cols, ntok))


@pytest.mark.parametrize("fmt", FORMATS)
def test_matmul_plane_independent_of_ntok(fmt):
    rows, cols = 70, 1024
    w = kqgen.weights(fmt, rows, cols, 812, fmt)
    x = kqgen.activations(130, cols, 813, fmt)
    note("matmul planes fmt=%d" % fmt)
    y = _gpu_matmul(fmt, w, rows, cols, x)
    for n in (1, 64, 65):
        yn = _gpu_matmul(fmt, w, rows, cols, x[:n])
        assert np.array_equal(yn.view(np.uint32), y[:n].view(np.uint32)), n


def test_matmul_prefill_sampled():
    """A 512-token prefill batch through the FFN gate (19968 x 6656 Q4_K)
    and the Q6_K FFN down (6656 x 19968), rows sampled."""
    for launch in (wl.ffn_gate_up(layer=0), wl.ffn_down(layer=1)):
        T = launch[0][0]
        w = kqgen.weights(T.fmt, T.rows, T.cols, *T.wkey)
        x = kqgen.activations(512, T.cols, 814, T.cols)
        note("matmul prefill %s fmt=%d %dx%d ntok=512" % (T.name, T.fmt, T.rows, T.cols))
        y = _gpu_matmul(T.fmt, w, T.rows, T.cols, x)
        idx = _sample_rows(T.rows, 61, tile=16)[:300]
        y_ref, s = oracle.matvec(T.fmt, w, T.rows, T.cols, x, row_idx=idx, nthreads=8)
        check_tol(y[:, idx], y_ref, s, "matmul prefill " + T.name)


@pytest.mark.parametrize("entry", ["kq_matvec16", "kq_matmul"])
def test_matrix_core_paths_strided_planes(entry):
    """Padded x and y planes (ldx > cols, ldy > rows) through the
    matrix-core entry points: the padding is neither read into the result
    nor written."""
    t = torch()
    fmt, rows, cols, ntok = Q4_K, 70, 1024, 12
    ldx, ldy = cols + 20, rows + 9
    w = kqgen.weights(fmt, rows, cols, 820, ntok)
    x = kqgen.activations(ntok, cols, 821, ntok)
    xp = np.full((ntok, ldx), np.nan, np.float32)
    xp[:, :cols] = x
    y = t.full((ntok, ldy), -3.0, dtype=t.float32, device="cuda")
    note("%s strided planes" % entry)
    getattr(kq, entry)(fmt, dev(w.reshape(-1)), rows, cols, dev(xp), y, ntok=ntok, ldx=ldx, ldy=ldy)
    yh = host(y)
    assert (yh[:, rows:] == -3.0).all()
    y_ref, s = oracle.matvec(fmt, w, rows, cols, x)
    check_tol(yh[:, :rows], y_ref, s, entry + " strided")


def test_random_shapes_every_entry_point():
    """Seeded random shapes (ragged rows, odd and even block counts, any
    plane count) through kq_matvec, kq_matvec16 and kq_matmul against the
    oracle."""
    rng = np.random.default_rng(2026)
    for case in range(18):
        fmt = int(rng.choice(FORMATS))
        rows = int(rng.integers(1, 2200))
        cols = 256 * int(rng.integers(1, 14))
        entry = ("kq_matvec", "kq_matvec16", "kq_matmul")[case % 3]
        ntok = int(rng.integers(1, {"kq_matvec": 9, "kq_matvec16": 17, "kq_matmul": 100}[entry]))
        w = kqgen.weights(fmt, rows, cols, 830, case)
        x = kqgen.activations(ntok, cols, 831, case)
        note("random case %d: %s fmt=%d %dx%d ntok=%d" % (case, entry, fmt, rows, cols, ntok))
        if entry == "kq_matvec":
            y = gpu_matvec(fmt, w, rows, cols, x)
        elif entry == "kq_matvec16":
            y = _gpu_matvec16(fmt, w, rows, cols, x)
        else:
            y = _gpu_matmul(fmt, w, rows, cols, x)
        y_ref, s = oracle.matvec(fmt, w, rows, cols, x, nthreads=8)
        check_tol(y, y_ref, s, "random case %d %s" % (case, entry))
