#!/usr/bin/env python3
"""Benchmark of the k-quant decode matvec on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload (one "step"): the 52-layer decode stream -- 52 independent
Q/K/V/gate sets (hidden 6,656 -> 4096/256/256/4096; Q and gate Q4_K on even
layers and Q5_K on odd layers, K and V Q6_K), one grid-split kq_matvec_set
launch per layer, each layer with its own weights and its own x, ntok = 1,
1,917,460,480 weight bytes per step.  Weights and activations are seeded
synthetic data (kqgen) resident in HBM before the timed region.

Prints ONE JSON line: effective weight GB/s over the whole step (launch gaps
included), the roofline of the set kernel (bytes per launch / the average
launch duration from HIP events recorded on the launch stream), the CPU
oracle's rate on a bounded sample on this host, and (default workload) the
other configurations' figures with a streaming-read calibration.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# Sources whose hash ties a committed counter measurement to the kernel it measured.
KERNEL_SOURCES = ["quant_matvec_amd/csrc/kq_kernels.hip", "quant_matvec_amd/csrc/kq_abi.cpp",
                  "quant_matvec_amd/csrc/kq_plan.h", "quant_matvec_amd/csrc/kq_decode.h", "include/kqmv.h"]


def code_only(text):
    """C/C++ source with its comments removed and its whitespace runs
    collapsed: what the compiler sees, so that a comment edit does not
    unlink a counter measurement from the kernel it measured."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":                                 # string or char literal, kept whole
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_sources_digest():
    """16 hex digits of sha256 over the kernel sources' code (comments and
    whitespace runs excluded), in KERNEL_SOURCES order."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(wname):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary of this workload, or None when there is none or the kernel
    sources' code has changed since it was taken."""
    import glob
    digest = kernel_sources_digest()
    for path in glob.glob(os.path.join(ROOT, "profiles", "*_hbm_traffic.md")):
        with open(path) as fh:
            for line in fh:
                line = line.strip()
                if line.startswith("{") and '"traffic_bytes_per_launch"' in line:
                    rec = json.loads(line)
                    if rec.get("workload") == wname and rec.get("src_sha256_16") == digest:
                        return int(rec["traffic_bytes_per_launch"])
    return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default="stream52",
                   choices=["stream52", "qkvg_set", "lm_head", "lm_head_q5k", "lm_head_q4k", "single_q4k",
                            "kv_pair"])
    p.add_argument("--ntok", type=int, default=1, help="kv_pair only")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-other-configs", action="store_true",
                   help="skip the per-configuration figures and the read calibration")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="only run a plain device-to-device copy of BYTES bytes (counter calibration) and exit")
    return p.parse_args()


def build_workload(name, ntok):
    from kqgen import workloads as wl
    if name == "stream52":
        return wl.qkvg_stream(), "qkvg_stream_52_layers", 1
    if name == "qkvg_set":
        # one layer's set, rotated over 16 distinct seeded copies so that the
        # weights come from HBM rather than the 256 MB last-level cache
        return [wl.qkvg_layer(2, i) for i in range(16)], "qkvg_set_x16_rotating", 1
    if name == "lm_head":
        return wl.lm_head(), "lm_head_q6k_202048x6656", 1
    if name == "lm_head_q5k":
        return wl.lm_head_q5k(), "lm_head_q5k_202048x6656", 1
    if name == "lm_head_q4k":
        return wl.lm_head_q4k(), "lm_head_q4k_202048x6656", 1
    if name == "single_q4k":
        return wl.single_q4k(), "single_q4k_256x6656", 1
    return wl.kv_pair() + wl.kv_pair(swapped=True), "kv_pair_q6k_q5k_ntok%d" % ntok, ntok


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import quant_matvec_amd as kq

    if not os.path.exists(kq.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    kq.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, dev)
        return

    launches, wname, ntok = build_workload(args.workload, args.ntok)
    r = run_workload(launches, wname, ntok, args.steps, args.warmup, dev, keep_host=not args.no_cpu_baseline)
    n_launch = r["launches"]
    bytes_per_launch = r["algo_bytes"] / n_launch
    achieved_gbs = bytes_per_launch / (r["us_per_launch_events"] * 1e-6) / 1e9
    value = r["weight_bytes"] * args.steps / r["elapsed"] / 1e9
    ms_per_step = r["elapsed"] / args.steps * 1e3
    weight_bytes = r["weight_bytes"]
    avg_launch_us = r["us_per_launch_events"]

    others = None
    if args.workload == "stream52" and not args.no_other_configs:
        others = other_configs(dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(r["host"], ntok, args.cpu_seconds)

    out = {
        "metric": "effective weight GB/s (and % of HBM peak) + us per QKV+gate set, ntok=1",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded k-quant blocks and N(0,1) activations)",
        "config": {"workload": wname, "launches_per_step": n_launch, "weight_bytes_per_step": weight_bytes,
                   "ntok": ntok, "hbm_peak_frac": round(value / HBM_PEAK_GBS, 4),
                   "us_per_launch_end_to_end": round(ms_per_step * 1e3 / n_launch, 3),
                   "us_per_launch_events": round(avg_launch_us, 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wname),
                     "kernel": r["kernel"], "bytes_per_launch": int(bytes_per_launch)},
        "cpu_baseline": cpu,
    }
    if others is not None:
        out["other_configs"] = others
    print(json.dumps(out), flush=True)


def run_workload(launches, wname, ntok, steps, warmup, dev, keep_host=False):
    """Upload the seeded inputs of `launches` (one kq_matvec_set call each),
    warm up, then time `steps` passes over them back to back.  Returns the
    wall-clock time of the timed region and the launches' average duration
    from two HIP events recorded on the launch stream around it."""
    import torch

    import kqgen
    import quant_matvec_amd as kq

    print("[bench] generating %s (%d launches)" % (wname, len(launches)), file=sys.stderr, flush=True)
    sets = []
    weight_bytes = 0
    algo_bytes = 0
    keep = []
    host = []      # the same seeded inputs, kept for the CPU baseline
    for launch in launches:
        xs = {}
        members = []
        for T in launch:
            w = kqgen.weights(T.fmt, T.rows, T.cols, *T.wkey)
            x = kqgen.activations(ntok, T.cols, *T.xkey)
            if keep_host:
                host.append((T, w, x))
            dw = torch.from_numpy(w.reshape(-1)).to(dev)
            if T.xkey not in xs:
                xs[T.xkey] = torch.from_numpy(x).to(dev)
                algo_bytes += ntok * T.cols * 4
            dy = torch.empty((ntok, T.rows), dtype=torch.float32, device=dev)
            keep += [dw, dy]
            members.append(dict(fmt=T.fmt, w=dw, x=xs[T.xkey], y=dy, rows=T.rows, cols=T.cols))
            weight_bytes += T.weight_bytes
            algo_bytes += T.weight_bytes + ntok * T.rows * 4
        keep += list(xs.values())
        sets.append(kq.make_set(members))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    n_launch = len(sets)
    kernels = sorted({kq.kq_debug_plan_kernel(s, ntok=ntok) for s in sets})

    def step():
        for s in sets:
            kq.kq_matvec_set(s, ntok=ntok, stream=sptr)

    # ---- warmup (also allocates the per-stream workspace outside the timed region)
    for _ in range(max(1, warmup)):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K steps, synchronized on both sides. HIP events on the
    # launch stream bracket the same region; with the launches back to back,
    # their span over all launches is the kernel's average launch duration
    # (per-launch event pairs would add their own queue time to a ~20 us kernel).
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    return {"launches": n_launch, "weight_bytes": weight_bytes, "algo_bytes": algo_bytes, "elapsed": elapsed,
            "us_per_launch_events": ev0.elapsed_time(ev1) * 1e3 / (steps * n_launch), "host": host,
            "kernel": "+".join(kernels)}


def other_configs(dev):
    """The remaining configurations, each timed like the main one (warm GPU,
    launches back to back, HIP events around the timed region), and a plain
    streaming read as the calibration of what HBM delivers to a trivial
    kernel.  C2 rotates over 16 seeded copies of the layer so that its
    weights come from HBM; C1 and C5 are small enough to stay in the caches
    (reported hot).  The F1 lines are the rest of a layer's matvecs and the
    Q5_K LM head, with their release formats (Ch 6 Figure 6.6)."""
    import torch
    from kqgen import workloads as wl

    res = {}

    def one(key, launches, name, ntok, steps, warmup):
        r = run_workload(launches, name, ntok, steps, warmup, dev)
        us = r["us_per_launch_events"]
        res[key] = {"workload": name, "us_per_launch": round(us, 3),
                    "weight_GBs": round(r["weight_bytes"] / r["launches"] / (us * 1e-6) / 1e9, 1)}

    one("C1_single_q4k_hot", wl.single_q4k(), "single_q4k_256x6656", 1, 2000, 500)
    one("C2_qkvg_set_x16_rotating", [wl.qkvg_layer(2, i) for i in range(16)], "qkvg_set_x16_rotating", 1, 100, 50)
    one("C4_lm_head_q6k", wl.lm_head(), "lm_head_q6k_202048x6656", 1, 200, 100)
    for ntok in (1, 2, 4, 8):
        one("C5_kv_pair_ntok%d_hot" % ntok, wl.kv_pair() + wl.kv_pair(swapped=True),
            "kv_pair_q6k_q5k_ntok%d" % ntok, ntok, 1000, 300)
    torch.cuda.empty_cache()
    # the rest of a layer's matvecs (enough rotating copies that the weights
    # come from HBM, not the 256 MB last-level cache), the Q5_K LM head, and
    # whole layers in decode order (four launches a layer)
    one("F1_attn_output_q4k_x24_rotating", [wl.attn_output(layer=i)[0] for i in range(24)],
        "attn_output_q4k_6656x4096_x24", 1, 100, 50)
    one("F1_ffn_gate_up_set_x4_rotating", [wl.ffn_gate_up(layer=i)[0] for i in range(4)],
        "ffn_gate_up_q4k_2x19968x6656_x4", 1, 100, 50)
    one("F1_ffn_down_q4k_x4_rotating", [wl.ffn_down(layer=2 * i)[0] for i in range(4)],
        "ffn_down_q4k_6656x19968_x4", 1, 100, 50)
    one("F1_ffn_down_q6k_x4_rotating", [wl.ffn_down(layer=2 * i + 1)[0] for i in range(4)],
        "ffn_down_q6k_6656x19968_x4", 1, 100, 50)
    one("F1_lm_head_q5k", wl.lm_head_q5k(), "lm_head_q5k_202048x6656", 1, 200, 100)
    torch.cuda.empty_cache()
    layers = [launch for i in range(4) for launch in wl.full_layer(layer=i)]
    one("F1_full_layer_x4_rotating", layers, "full_layer_qkvg_o_gateup_down_x4", 1, 50, 20)
    res["F1_full_layer_x4_rotating"]["us_per_layer"] = round(res["F1_full_layer_x4_rotating"]["us_per_launch"] * 4, 3)
    torch.cuda.empty_cache()
    res.update(embedding_configs(dev))
    torch.cuda.empty_cache()
    res.update(matvec16_configs(dev))
    torch.cuda.empty_cache()
    res.update(matmul_configs(dev))
    torch.cuda.empty_cache()
    # calibration: the library's trivial 16-byte streaming-read probe over 2 GiB
    import quant_matvec_amd as kq
    buf = torch.ones(1 << 29, dtype=torch.float32, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(20):
        kq.kq_debug_read_probe(buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        kq.kq_debug_read_probe(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    gbs = buf.numel() * 4 * 20 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    res["calibration_streaming_read"] = {"what": "kq_debug_read_probe: 16-byte nontemporal loads over 2 GiB, nothing else",
                                         "GBs": round(gbs, 1), "hbm_peak_frac": round(gbs / HBM_PEAK_GBS, 4)}
    del buf
    torch.cuda.empty_cache()
    return res


def matvec16_configs(dev):
    """16 token planes (the verify width) with kq_matvec16 on release shapes,
    rotating copies so the weights come from HBM; each call reads the
    weights once.  For context, the same weights through kq_matvec as two
    8-plane calls."""
    import torch

    import kqgen
    import quant_matvec_amd as kq
    from kqgen import workloads as wl

    out_res = {}
    stream = torch.cuda.current_stream()
    cases = [("attn_output_q4k_x24", [wl.attn_output(layer=i)[0][0] for i in range(24)], 200),
             ("ffn_gate_q4k_x4", [wl.ffn_gate_up(layer=i)[0][0] for i in range(4)], 50),
             ("lm_head_q5k", [wl.lm_head_q5k()[0][0]], 10),
             ("ffn_down_q6k_x2", [wl.ffn_down(layer=i)[0][0] for i in (1, 3)], 50)]
    for name, tensors, reps in cases:
        print("[bench] generating %s for 16 planes" % name, file=sys.stderr, flush=True)
        mem = []
        for T in tensors:
            w = torch.from_numpy(kqgen.weights(T.fmt, T.rows, T.cols, *T.wkey).reshape(-1)).to(dev)
            x = torch.from_numpy(kqgen.activations(16, T.cols, *T.xkey)).to(dev)
            y = torch.empty((16, T.rows), dtype=torch.float32, device=dev)
            mem.append((T, w, x, y))
        wbytes = sum(T.weight_bytes for T, _, _, _ in mem)
        weights = sum(T.rows * T.cols for T, _, _, _ in mem)

        def run16():
            for T, w, x, y in mem:
                kq.kq_matvec16(T.fmt, w, T.rows, T.cols, x, y, ntok=16, stream=stream.cuda_stream)

        def run8x2():
            for T, w, x, y in mem:
                for h in (0, 8):
                    kq.kq_matvec(T.fmt, w, T.rows, T.cols, x[h:h + 8], y[h:h + 8], ntok=8, stream=stream.cuda_stream)

        for key, fn in (("kq_matvec16", run16), ("kq_matvec_2x8", run8x2)):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (reps * len(mem))
            out_res["F2_%s_ntok16_%s" % (name, key)] = {
                "workload": "%s_ntok16" % name, "entry": key, "us_per_tensor": round(us, 3),
                "weight_GBs": round(wbytes / len(mem) / (us * 1e-6) / 1e9, 1),
                "hbm_frac": round(wbytes / len(mem) / (us * 1e-6) / 8e12, 4),
                "TFLOPs": round(2 * 16 * weights / len(mem) / (us * 1e-6) / 1e12, 2)}
        del mem
        torch.cuda.empty_cache()
    return out_res


def matmul_configs(dev):
    """A 512-token prefill batch (kq_matmul) through release shapes: flops
    (2 a weight a token) per second, against the bf16 matrix peak halved
    (two products a weight and token, one for each of x's two parts)."""
    import torch

    import kqgen
    import quant_matvec_amd as kq
    from kqgen import workloads as wl

    out_res = {}
    stream = torch.cuda.current_stream()
    ntok = 512
    for name, T, reps in (("attn_output_q4k", wl.attn_output()[0][0], 20),
                          ("ffn_gate_q4k", wl.ffn_gate_up()[0][0], 5),
                          ("ffn_down_q6k", wl.ffn_down(layer=1)[0][0], 5)):
        print("[bench] generating %s for a prefill batch" % name, file=sys.stderr, flush=True)
        w = torch.from_numpy(kqgen.weights(T.fmt, T.rows, T.cols, *T.wkey).reshape(-1)).to(dev)
        x = torch.from_numpy(kqgen.activations(ntok, T.cols, *T.xkey)).to(dev)
        y = torch.empty((ntok, T.rows), dtype=torch.float32, device=dev)
        for _ in range(2):
            kq.kq_matmul(T.fmt, w, T.rows, T.cols, x, y, ntok=ntok, stream=stream.cuda_stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            kq.kq_matmul(T.fmt, w, T.rows, T.cols, x, y, ntok=ntok, stream=stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        tf = 2 * ntok * T.rows * T.cols / (us * 1e-6) / 1e12
        matrix, peak = "bf16", 2500.0 / 2
        out_res["F4_prefill512_%s" % name] = {"workload": "%s_%dx%d_ntok%d" % (name, T.rows, T.cols, ntok),
                                              "us_per_call": round(us, 1), "TFLOPs": round(tf, 2),
                                              "matrix": matrix, "matrix_peak_frac": round(tf / peak, 4)}
        del w, x, y
        torch.cuda.empty_cache()
    return out_res


def embedding_configs(dev):
    """The embedding lookup (Ch 6 section 6.7) on the 202,048 x 6656 Q4_K
    table: one id a call (a decode step) and 512 ids a call, each call with
    fresh seeded ids.  Bytes moved = the rows read plus the float32 rows
    written."""
    import numpy as np
    import torch

    import kqgen
    import quant_matvec_amd as kq
    from kqgen import workloads as wl

    T = wl.embedding_table()
    print("[bench] generating the embedding table", file=sys.stderr, flush=True)
    table = torch.from_numpy(kqgen.weights(T.fmt, T.rows, T.cols, *T.wkey).reshape(-1)).to(dev)
    row_bytes = T.weight_bytes // T.rows
    out_res = {}
    stream = torch.cuda.current_stream()
    for n, calls in ((1, 2000), (512, 200)):
        gen = np.random.default_rng(900 + n)
        ids = torch.from_numpy(gen.integers(0, T.rows, size=n * calls, dtype=np.int32)).to(dev)
        out = torch.empty((n, T.cols), dtype=torch.float32, device=dev)
        for k in range(min(calls, 100)):
            kq.kq_embed_rows(T.fmt, table, T.rows, T.cols, ids[k * n:(k + 1) * n], out, stream=stream.cuda_stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(calls):
            kq.kq_embed_rows(T.fmt, table, T.rows, T.cols, ids[k * n:(k + 1) * n], out, stream=stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / calls
        moved = n * (row_bytes + T.cols * 4)
        out_res["F3_embedding_q4k_%d_ids" % n] = {"workload": "embedding_q4k_202048x6656_%d_ids" % n,
                                                 "us_per_call": round(us, 3),
                                                 "GBs_moved": round(moved / (us * 1e-6) / 1e9, 1)}
    del table
    return out_res


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(host, ntok, budget_s):
    """The CPU oracle (as it stands, untuned) on a bounded sample of the same
    workload: whole tensors in launch order, wrapping around, timed twice --
    on one thread for about a third of budget_s, then split over rows on
    every CPU this process may run on for the rest.  `value` is the all-core
    rate; the one-thread rate, nproc and the CPU model ride along."""
    import oracle

    def run(threads, seconds):
        done_bytes, spent, tensors = 0, 0.0, 0
        while spent < seconds:
            for T, w, x in host:
                t0 = time.perf_counter()
                oracle.matvec(T.fmt, w, T.rows, T.cols, x, nthreads=threads)
                spent += time.perf_counter() - t0
                done_bytes += T.weight_bytes
                tensors += 1
                if spent >= seconds:
                    break
        return done_bytes, spent, tensors

    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    b1, s1, n1 = run(1, budget_s / 3.0)
    bn, sn, nn = run(ncpu, budget_s * 2.0 / 3.0)
    return {"value": round(bn / sn / 1e9, 4), "unit": "GB/s", "cores": ncpu, "kind": "oracle",
            "sample": "%d whole tensors (%d weight bytes) of the same workload in launch order, ntok=%d, %.1f s "
                      "on %d threads; one thread: %d tensors (%d bytes) in %.1f s" % (nn, bn, ntok, sn, ncpu, n1, b1, s1),
            "single_thread_value": round(b1 / s1 / 1e9, 4), "nproc": os.cpu_count(), "cpu_model": _cpu_model()}


def copy_calibration(nbytes, dev):
    """A plain device-to-device copy of nbytes (torch's copy kernel), run a
    few times: reading its FETCH_SIZE / WRITE_SIZE counters gives the
    factor between those counters and bytes actually moved."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 5}), flush=True)


if __name__ == "__main__":
    main()
