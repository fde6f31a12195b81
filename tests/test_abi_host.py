"""Host-side checks of the C ABI: the library loads, exports every function
include/kqmv.h declares, and rejects bad arguments before any HIP call
(the fail-closed admission of muser-book Ch 6 section 6.1).  CPU only: only
calls that fail validation are made, so no HIP work is ever issued."""
import ctypes
import os
import re

import pytest

import quant_matvec_amd as kq
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "kqmv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kq.LIB_PATH):
        from quant_matvec_amd import build
        build.build()
    return kq.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(kq.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_geometry(lib):
    assert kq.kq_version() == 1
    assert [kq.kq_block_bytes(f) for f in (12, 13, 14)] == [144, 176, 210]
    assert kq.kq_row_bytes(12, 6656) == 3744
    assert kq.kq_row_bytes(13, 6656) == 4576
    assert kq.kq_row_bytes(14, 6656) == 5460
    assert lib.kq_block_bytes(2) == -1
    assert lib.kq_row_bytes(12, 300) == -2
    assert lib.kq_row_bytes(99, 256) == -1
    for code in range(-12, 1):
        assert kq.kq_strerror(code)


BASE = 0x7F0000000000   # fake, never dereferenced: every case below fails validation


def one(**kw):
    d = dict(fmt=12, w=BASE, x=BASE + (1 << 30), y=BASE + (2 << 30), rows=256, cols=6656)
    d.update(kw)
    return d


def status(tensors, ntok=1, n=None):
    return kq.kq_validate_set(kq.make_set(tensors), ntok, n=n)


def test_validation_accepts_a_good_set(lib):
    assert status([one()]) == 0
    assert status([one(), one(fmt=14, w=BASE + (3 << 30), y=BASE + (4 << 30))], ntok=8) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(fmt=2), -1), (dict(fmt=15), -1), (dict(reserved=1), -1),
    (dict(cols=0), -2), (dict(cols=300), -2), (dict(cols=-256), -2),
    (dict(rows=0), -3), (dict(rows=-5), -3),
    (dict(w=0), -5), (dict(x=0), -5), (dict(y=0), -5),
    (dict(w=BASE + 8), -6), (dict(x=BASE + (1 << 30) + 4), -6), (dict(y=BASE + (2 << 30) + 2), -6),
    (dict(ldx=6000), -7), (dict(ldx=6658), -7), (dict(ldy=100), -7),
    (dict(y=BASE + 64), -8), (dict(y=BASE + (1 << 30) + 4096), -8),
    (dict(rows=1 << 32), -11),
])
def test_validation_rejects(lib, kw, code):
    assert status([one(**kw)]) == code


def test_validation_set_rules(lib):
    assert status([one()], ntok=0) == -4
    assert status([one()], ntok=9) == -4
    assert status([one()], n=0) == -9
    assert status([one()] * 17, n=17) == -9
    # two outputs overlap
    assert status([one(), one(w=BASE + (3 << 30))]) == -8
    # outputs of plane t reach y + t*ldy: ntok=2 with ldy=rows overlaps a y placed right after
    a = one(rows=256)
    b = one(w=BASE + (3 << 30), y=BASE + (2 << 30) + 256 * 4)
    assert status([a, b], ntok=1) == 0
    assert status([a, b], ntok=2) == -8
    # shared x is fine; y inside another tensor's x is not
    assert status([one(), one(w=BASE + (3 << 30), y=BASE + (4 << 30))]) == 0
    assert status([one(), one(w=BASE + (3 << 30), x=BASE + (2 << 30), y=BASE + (4 << 30))]) == -8


def test_invalid_calls_fail_before_hip(lib):
    # these return the validation code without touching the GPU (there is none here)
    assert lib.kq_matvec(12, BASE, 256, 300, BASE + (1 << 30), 300, BASE + (2 << 30), 256, 1, None) == -2
    assert lib.kq_matvec(12, BASE, 256, 6656, BASE + (1 << 30), 6656, BASE + (2 << 30), 256, 0, None) == -4
    assert lib.kq_matvec(13, BASE + 1, 256, 6656, BASE + (1 << 30), 6656, BASE + (2 << 30), 256, 1, None) == -6
    arr = kq.make_set([one()])
    assert lib.kq_matvec_set(arr, 0, 1, None) == -9
    assert lib.kq_matvec_set_noalloc(arr, 0, 1, None) == -9
    assert lib.kq_matvec_set_noalloc(arr, 1, 9, None) == -4
    assert lib.kq_matvec_set_noalloc(kq.make_set([one(y=BASE + 64)]), 1, 1, None) == -8
    assert lib.kq_unpack_blocks(7, BASE, 1, None, None, None, None, None, None) == -1
    assert lib.kq_unpack_blocks(12, BASE, 0, None, None, None, None, None, None) == -3
    assert lib.kq_unpack_blocks(12, BASE + 4, 1, None, None, None, None, None, None) == -6
    assert lib.kq_dequant(14, BASE, 4, 512, BASE + (1 << 30), 256, None) == -7
    assert lib.kq_dequant(14, BASE, 4, 500, BASE + (1 << 30), 512, None) == -2
    assert lib.kq_debug_read_probe(None, 256, BASE, None) == -5
    assert lib.kq_debug_read_probe(BASE, 250, BASE + (1 << 30), None) == -3
    assert lib.kq_debug_read_probe(BASE + 4, 256, BASE + (1 << 30), None) == -6
    with pytest.raises(kq.KqError):
        kq.kq_matvec(12, BASE, 256, 300, BASE + (1 << 30), BASE + (2 << 30), stream=0)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(kq, "_lib", None)
    monkeypatch.setattr(kq, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        kq.kq_version()


def test_release_shapes_match_the_pages():
    """The rest-of-layer workloads against the figures the pages print:
    the Q5_K LM head's bytes (Ch 6 section 6.5: 26 blocks x 176 B x 202,048
    rows = 924,571,648 B) and the parameter counts of o_proj (27.3 M) and of
    each FFN matrix (132.9 M) in Ch 13 section 13.6."""
    from kqgen import workloads as wl
    assert wl.total_weight_bytes(wl.lm_head_q5k()) == 924_571_648
    [[o]] = wl.attn_output()
    assert round(o.rows * o.cols / 1e6, 1) == 27.3
    [[g, u]] = wl.ffn_gate_up()
    [[d]] = wl.ffn_down()
    for T in (g, u, d):
        assert round(T.rows * T.cols / 1e6, 1) == 132.9
    assert g.xkey == u.xkey and (g.rows, g.cols) == (d.cols, d.rows)
    assert [T.fmt for layer in (0, 1) for [T] in wl.ffn_down(layer=layer)] == [12, 14]


def test_embed_rows_admission(lib):
    """kq_embed_rows admits a Q4_K table only (the embedding fence of Ch 6
    section 6.1) and checks sizes, alignment, strides and overlap on the
    host; every call here fails before any HIP call."""
    T, I, O = BASE, BASE + (1 << 30), BASE + (2 << 30)
    good = dict(fmt=12, table=T, rows=202048, cols=6656, ids=I, n=4, out=O, ldo=6656)

    def call(**kw):
        a = dict(good, **kw)
        return lib.kq_embed_rows(a["fmt"], a["table"], a["rows"], a["cols"], a["ids"], a["n"], a["out"],
                                 a["ldo"], None)

    for fmt in (13, 14, 0, 7):
        assert call(fmt=fmt) == -1
    assert call(cols=6600) == -2 and call(cols=0) == -2
    assert call(rows=0) == -3 and call(n=0) == -3 and call(n=(1 << 24) + 1) == -3
    assert call(table=None) == -5 and call(ids=None) == -5 and call(out=None) == -5
    assert call(table=T + 8) == -6 and call(ids=I + 2) == -6 and call(out=O + 4) == -6
    assert call(ldo=6652) == -7 and call(ldo=6658) == -7
    # out over the table, or over the ids
    assert call(out=T + 16) == -8
    assert call(out=I - 64, n=1) == -8


def test_matvec16_admission(lib):
    """kq_matvec16 takes 1..16 token planes and otherwise the checks of
    kq_matvec, all on the host."""
    W, X, Y = BASE, BASE + (1 << 30), BASE + (2 << 30)
    assert lib.kq_matvec16(12, W, 256, 6656, X, 6656, Y, 256, 0, None) == -4
    assert lib.kq_matvec16(12, W, 256, 6656, X, 6656, Y, 256, 17, None) == -4
    assert lib.kq_matvec16(7, W, 256, 6656, X, 6656, Y, 256, 16, None) == -1
    assert lib.kq_matvec16(12, W, 256, 6600, X, 6656, Y, 256, 16, None) == -2
    assert lib.kq_matvec16(12, W, 0, 6656, X, 6656, Y, 256, 16, None) == -3
    assert lib.kq_matvec16(12, None, 256, 6656, X, 6656, Y, 256, 16, None) == -5
    assert lib.kq_matvec16(12, W + 4, 256, 6656, X, 6656, Y, 256, 16, None) == -6
    assert lib.kq_matvec16(12, W, 256, 6656, X, 6654, Y, 256, 16, None) == -7
    # y planes reaching into x
    assert lib.kq_matvec16(12, W, 256, 6656, X, 6656, X - 4096, 256, 16, None) == -8


def test_matmul_admission(lib):
    """kq_matmul takes 1..2^20 token planes and otherwise the checks of
    kq_matvec, all on the host."""
    W, X, Y = BASE, BASE + (1 << 36), BASE + (2 << 36)
    assert lib.kq_matmul(12, W, 256, 6656, X, 6656, Y, 256, 0, None) == -4
    assert lib.kq_matmul(12, W, 256, 6656, X, 6656, Y, 256, (1 << 20) + 1, None) == -4
    assert lib.kq_matmul(9, W, 256, 6656, X, 6656, Y, 256, 512, None) == -1
    assert lib.kq_matmul(12, W, 256, 6656, X + 8, 6656, Y, 256, 512, None) == -6
    assert lib.kq_matmul(12, W, 256, 6656, X, 6656, Y, 255, 512, None) == -7
    # 512 planes of y reaching into x
    assert lib.kq_matmul(12, W, 256, 6656, X, 6656, X - 512 * 256 * 4 + 1024, 256, 512, None) == -8


# ---- the workspace slots of shared tiles.  The rule (restated here from
# the plan's description) numbers a shared tile by itself while runs are
# shorter than a tile, else by the first run boundary inside it; every
# contributor of a tile must find the same slot, distinct tiles distinct
# slots, and every slot must lie below the count the host allocates.

def _runs(segs, P):
    q, r = divmod(segs, P)
    starts = [u * q + min(u, r) for u in range(P)] + [segs]
    return q, r, starts


def _slot(tile, nseg, q, r):
    if q < nseg:
        return tile
    t0 = tile * nseg
    return t0 // (q + 1) if t0 < r * (q + 1) else (t0 - r) // q


@pytest.mark.parametrize("tiles,nseg,P", [(272, 7, 2000), (6314, 7, 2048), (4, 26, 104), (3157, 13, 2048),
                                          (104, 39, 2048), (1, 26, 13), (5, 3, 7), (7, 5, 6), (100, 1, 37),
                                          (64, 13, 832), (13, 7, 45), (9, 11, 10)])
def test_shared_tile_slots_unique_and_bounded(tiles, nseg, P):
    segs = tiles * nseg
    P = min(P, segs)
    q, r, starts = _runs(segs, P)
    nslots = 0 if P <= 1 else (tiles if q < nseg else P - 1)
    owner = {}
    for u in range(P):
        j0, j1 = starts[u], starts[u + 1]
        for tile in range(j0 // nseg, (j1 - 1) // nseg + 1):
            t0, t1 = tile * nseg, tile * nseg + nseg
            if j0 <= t0 and t1 <= j1:
                continue                              # owned: summed in registers
            s = _slot(tile, nseg, q, r)
            assert 0 <= s < nslots, (u, tile, s, nslots)
            assert owner.setdefault(s, tile) == tile, (s, owner[s], tile)
