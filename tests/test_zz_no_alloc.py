"""kq_matvec_set_noalloc, the set call for callers that cannot allocate:
through the C ABI, bitwise equal to kq_matvec_set on the same inputs, on
two calls in a row (the second with a smaller input), and a plan larger
than its fixed scratch refused with KQ_ERR_SCRATCH before any launch."""
import numpy as np
import pytest

import kqgen
import quant_matvec_amd as kq
from gpu_util import dev, host, note, torch
from kqgen import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    kq.load()


def _members(tensors, ntok, key):
    t = torch()
    xs, out = {}, []
    for T in tensors:
        w = dev(kqgen.weights(T.fmt, T.rows, T.cols, *T.wkey).reshape(-1))
        if T.xkey not in xs:
            xs[T.xkey] = dev(kqgen.activations(ntok, T.cols, key, *T.xkey))
        out.append(dict(fmt=T.fmt, w=w, x=xs[T.xkey], rows=T.rows, cols=T.cols))
    return out


def _run(entry, members, ntok):
    t = torch()
    ys = [t.full((ntok, m["rows"]), float("nan"), dtype=t.float32, device="cuda") for m in members]
    getattr(kq, entry)([dict(m, y=y) for m, y in zip(members, ys)], ntok=ntok)
    return [host(y) for y in ys]


def _bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def test_noalloc_matches_set_on_two_calls():
    # a Q/K/V/gate set (shared tiles in every tensor), then a smaller K/V pair at two planes
    for tensors, ntok in ((wl.qkvg_layer(2, 0), 1), (wl.kv_pair()[0], 2)):
        members = _members(tensors, ntok, 960)
        note("noalloc %s ntok=%d" % ("+".join(T.name for T in tensors), ntok))
        a = _run("kq_matvec_set_noalloc", members, ntok)
        b = _run("kq_matvec_set", members, ntok)
        for T, ya, yb in zip(tensors, a, b):
            assert np.isfinite(ya).all(), T.name
            assert np.array_equal(_bits(ya), _bits(yb)), T.name


def test_noalloc_refuses_a_plan_beyond_its_scratch():
    """The 202,048-row Q6_K matvec at 8 planes needs about 54 MB of
    shared-tile sums: refused with KQ_ERR_SCRATCH (the buffers are real and
    zeroed, so nothing could fault even if a launch happened)."""
    t = torch()
    [[T]] = wl.lm_head()
    w = t.zeros(T.weight_bytes, dtype=t.uint8, device="cuda")
    x = t.zeros((8, T.cols), dtype=t.float32, device="cuda")
    y = t.full((8, T.rows), -5.0, dtype=t.float32, device="cuda")
    note("noalloc refuses lm_head ntok=8")
    with pytest.raises(kq.KqError) as e:
        kq.kq_matvec_set_noalloc([dict(fmt=T.fmt, w=w, x=x, y=y, rows=T.rows, cols=T.cols)], ntok=8)
    assert e.value.code == -12
    t.cuda.synchronize()
    assert bool((y == -5.0).all())
