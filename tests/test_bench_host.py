"""Host-side logic of bench.py: the code-only digest that ties a committed
counter measurement to the kernel sources, the lookup of that measurement,
and the one-GPU refusal.  No GPU and no kernel call."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_code_only_drops_comments_keeps_literals():
    b = load_bench()
    src = ('int a = 1; // one\n/* block\n comment */ int b=2;\n'
           'const char* s = "a // not a comment /* nor this */";\n'
           "char c = '/'; char q = '\\''; const char* e = \"x\\\"// y\";\n")
    out = b.code_only(src)
    assert "one" not in out and "block" not in out
    assert '"a // not a comment /* nor this */"' in out
    assert "'/'" in out and "'\\''" in out and '"x\\"// y"' in out
    assert "int b=2;" in out


def test_code_only_ignores_comment_and_layout_edits():
    b = load_bench()
    a = "__global__ void k(float* y) {\n    y[0] = 1.0f;   // store\n}\n"
    c = "// a kernel\n__global__ void k(float* y) {\n  /* the store */ y[0] = 1.0f;\n}\n"
    d = "__global__ void k(float* y) {\n    y[0] = 2.0f;\n}\n"
    assert b.code_only(a) == b.code_only(c)
    assert b.code_only(a) != b.code_only(d)


def test_digest_covers_every_kernel_source():
    b = load_bench()
    for f in b.KERNEL_SOURCES:
        assert os.path.isfile(os.path.join(ROOT, f)), f
    dg = b.kernel_sources_digest()
    assert len(dg) == 16 and int(dg, 16) >= 0


def test_measured_traffic_matches_digest_or_none():
    """A committed traffic record is used only under the digest it was taken
    at; either way the value is a positive byte count or None."""
    b = load_bench()
    for w in ("qkvg_stream_52_layers", "lm_head_q6k_202048x6656", "no_such_workload"):
        t = b.measured_traffic(w)
        assert t is None or t > 0
    assert b.measured_traffic("no_such_workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""
