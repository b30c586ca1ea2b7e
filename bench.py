"""Benchmark of the weight-only quantized matmul on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--quick]
    python bench.py --probe WORKLOAD[@ENTRY]  (three calls, for rocprofv3 --pmc)
    python bench.py --phases              (per-wave phase stamps of the headline GEMV)
    python bench.py --trace-summary DB    (per-workload rows of a rocprofv3 trace
                                           taken with --kernel-trace --marker-trace)

A step is one call of the hot path on one batch of synthetic input already
resident in HBM.  The headline workload is the int4 group-128 asymmetric
decode GEMV (M=1, K=N=4096, fp16 x, fp32 accumulation), through qmm_gemm on
weights repacked once by qmm_pack (offline, not timed); `value` is its
effective weight bandwidth (packed weights + scales + zeros per call / time).
The same product through qmm_gemv on the canonical layout is a workload line.
Every other workload is timed the same way and reported under "workloads";
the prefill GEMM (M=4096) is reported in TFLOP/s under "prefill".

Memory-bound calls rotate over a pool of weight copies (> 2 x the 256 MB
Infinity Cache), and before every timed replay an untimed pass over a 1 GiB
buffer evicts the cache, so every call streams its weights from HBM whatever
the number of steps.  The timed calls are captured once in a HIP graph and
replayed five times, each replay bracketed by HIP events on the launch
stream; the median replay gives the time per call.  "calibration" holds what this GPU reaches on plain work of
the same kind (a device-to-device copy, the vendor BLAS's dense bf16 GEMM
of the prefill shape), labelled as such; the roofline peaks stay the
published ones.  The CPU baseline times the oracle on the host's cores, on
the headline product and on bounded row x column samples of every other
workload, with one thread and with all of them ("cpu_baseline").  Prints
one JSON line.
"""
import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = 2500.0       # MI355X dense fp16/bf16 matrix peak
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 matrix peak
POOL_BYTES = 512 << 20          # weight pool for memory-bound workloads

HEADLINE = "int4_g128_asym_gemv_m1_k4096_n4096"
HEADLINE_PATH = "gemm"  # qmm_gemm on the tile layout (qmm_pack, offline): the decode GEMV
OTHERS = [  # (workload, entry)
    (HEADLINE, "gemv"),  # the same product on the canonical layout (qmm_gemv)
    ("int8_gemv_m1_k1024_n1024", "gemv"),
    ("int4_pc_sym_gemv_m1_k4096_n4096", "gemv"),  # per-column scales
    ("int8_skinny_m16_k4096_n14336", "gemm"),
    ("int8_skinny_m32_k4096_n14336", "gemm"),
    ("int8_skinny_m64_k4096_n14336", "gemm"),
    ("int4_g128_sym_m16_k8192_n8192", "gemm"),
    ("int4_g128_asym_smalln_m16_k14336_n1024", "gemm"),  # 64 tiles: 8 waves each
]
PREFILL = [  # (workload, output dtype)
    ("int4_g128_asym_prefill_m4096_k4096_n11008", "f32"),
    ("int2_g64_asym_prefill_m4096_k4096_n11008", "f32"),
    ("int4_g128_asym_prefill_m4096_k4096_n11008", "bf16"),  # qmm_gemm_ex, bf16 y
]
TERNARY = ["i8t2_m16_k4096_n4096", "i8t2_m4096_k4096_n11008"]  # int8 x ternary (qmm_i8t2_gemm)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")
CSRC = os.path.join(ROOT, "gemv_only_quant_amd", "csrc")


def bytes_of(case, y_bytes=4):
    """Algorithmic bytes per call: packed Q, scales, zeros, x and y, each once."""
    w = case.Q.numel() * case.Q.element_size()
    w += case.scales.numel() * case.scales.element_size()
    if case.zeros is not None:
        w += case.zeros.numel() * case.zeros.element_size()
    io = case.x.numel() * case.x.element_size() + case.M * case.N * y_bytes
    return w, w + io


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class _Marks:
    """roctx ranges around the timed replays (no-ops unless a tracer such as
    rocprofv3 --marker-trace is attached), so a kernel trace can be split by
    workload and restricted to the timed, graph-replayed dispatches."""
    lib = False

    @classmethod
    def _get(cls):
        if cls.lib is False:
            import ctypes
            path = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib",
                                "librocprofiler-sdk-roctx.so")
            try:
                cls.lib = ctypes.CDLL(path)
                cls.lib.roctxRangePushA.argtypes = [ctypes.c_char_p]
            except OSError:
                cls.lib = None
        return cls.lib

    @classmethod
    def push(cls, label):
        if cls._get() is not None:
            cls.lib.roctxRangePushA(label.encode())

    @classmethod
    def pop(cls):
        if cls._get() is not None:
            cls.lib.roctxRangePop()


_EVICT = []


def evict_cache():
    """Untimed: read and write a 1 GiB buffer (4x the 256 MB Infinity Cache),
    so no weight copy of the next timed replay is still cached."""
    import torch
    if not _EVICT:
        _EVICT.append(torch.zeros(1 << 30, dtype=torch.uint8, device="cuda"))
    _EVICT[0].add_(1)


def replay_us(graph, steps, label, reps=5):
    """Median µs per call over `reps` timed replays of a `steps`-call graph,
    each after a cache eviction, bracketed by events on the launch stream and
    by a roctx range named `timed <label>`."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = []
    for _ in range(reps):
        evict_cache()
        torch.cuda.synchronize()
        _Marks.push(f"timed {label}")
        start.record()
        graph.replay()
        end.record()
        torch.cuda.synchronize()
        _Marks.pop()
        out.append(start.elapsed_time(end) * 1e3 / steps)
    return statistics.median(out)


def time_workload(name, steps, warmup, path, out="f32"):
    """Average µs per call of `steps` graph-replayed calls (plus eager µs)."""
    import torch
    import gemv_only_quant_amd as qmm
    import synth_inputs as si

    ydt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[out]
    case = si.workload(name)
    wbytes, tbytes = bytes_of(case, torch.tensor([], dtype=ydt).element_size())
    d = case.to("cuda")
    Q0 = d.Q if path == "gemv" else qmm.pack(d.Q, case.N, case.K, case.w_bit)
    copies = 1 if case.M >= 1024 else max(1, -(-POOL_BYTES // wbytes))
    pool = [(Q0, d.scales, d.zeros)]
    for _ in range(copies - 1):
        pool.append((Q0.clone(), d.scales.clone(), None if d.zeros is None else d.zeros.clone()))
    y = torch.empty((case.M, case.N), dtype=ydt, device="cuda")
    ws = qmm.workspace_for(case.M, case.N, case.K, case.w_bit, case.group_size, "cuda")
    if out == "f32":
        fn = qmm.qmm_gemv if path == "gemv" else qmm.qmm_gemm
    else:
        fn = qmm.qmm_gemv_ex if path == "gemv" else qmm.qmm_gemm_ex

    def call(i):
        Q, s, z = pool[i % copies]
        fn(d.x, Q, s, z, y, case.M, case.N, case.K, case.w_bit, case.group_size, workspace=ws)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_eager = min(steps, 200)
    start.record()
    for i in range(n_eager):
        call(i)
    end.record()
    torch.cuda.synchronize()
    eager_us = start.elapsed_time(end) * 1e3 / n_eager

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for i in range(steps):
            call(i)
    graph.replay()
    torch.cuda.synchronize()
    y_graph = y.clone()
    call(steps - 1)  # eager result of the same last call
    torch.cuda.synchronize()
    assert torch.equal(y_graph, y), f"{name}: graph replay differs from eager call"

    us = replay_us(graph, steps, f"{name} {out}")
    del graph, pool
    progress(f"{name} ({out} y): {us:.3f} us per call")
    return dict(case=case, us=us, eager_us=eager_us, wbytes=wbytes, tbytes=tbytes,
                flops=2.0 * case.M * case.N * case.K, copies=copies,
                rotated=min(steps, copies), rotated_bytes=min(steps, copies) * wbytes)


def calibration():
    """What this GPU reaches on plain work: a 1 GiB device-to-device copy
    (read + write bytes / time) and torch's dense bf16 GEMM (vendor BLAS) at
    M=4096, K=4096, N=11008 with fp32 output."""
    import torch
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / n

    src = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    copy_us = timed(lambda: dst.copy_(src), 20)
    del src, dst
    g = torch.Generator(device="cuda").manual_seed(0)
    M, K, N = 4096, 4096, 11008
    a = torch.randn((M, K), device="cuda", dtype=torch.bfloat16, generator=g)
    w = torch.randn((K, N), device="cuda", dtype=torch.bfloat16, generator=g)
    try:
        out_dt = "f32"
        gemm_us = timed(lambda: torch.mm(a, w, out_dtype=torch.float32), 20)
    except (RuntimeError, TypeError):
        out_dt = "bf16"
        gemm_us = timed(lambda: torch.mm(a, w), 20)
    return {"hbm_copy_GBps": round(2 * (1 << 30) / copy_us / 1e3, 1),
            "dense_bf16_gemm_m4096_k4096_n11008_us": round(gemm_us, 1),
            "dense_bf16_gemm_tflops": round(2 * M * N * K / gemm_us / 1e6, 1),
            "dense_gemm_out_dtype": out_dt,
            "note": "measured here on plain work, for context; roofline peaks are the published ones"}


def time_ternary(name, steps, warmup):
    """The int8 x ternary product, timed like time_workload (weights packed
    to the tile layout once, outside the timed region)."""
    import torch
    import gemv_only_quant_amd as qmm
    import synth_inputs as si

    case = si.workload(name)
    d = case.to("cuda")
    Wt0 = qmm.t2_pack(d.Wp, case.N, case.K)
    wbytes = Wt0.numel()
    tbytes = wbytes + case.M * case.K + case.M * case.N * 4
    copies = 1 if case.M >= 1024 else max(1, -(-POOL_BYTES // wbytes))
    pool = [Wt0] + [Wt0.clone() for _ in range(copies - 1)]
    y = torch.empty((case.M, case.N), dtype=torch.int32, device="cuda")

    def call(i):
        qmm.qmm_i8t2_gemm(d.A, pool[i % copies], y, case.M, case.N, case.K)

    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            call(i)
    graph.replay()
    torch.cuda.synchronize()
    us = replay_us(graph, steps, name)
    del graph, pool
    progress(f"{name}: {us:.3f} us per call")
    tops = 2.0 * case.M * case.N * case.K / us / 1e6
    return {"workload": name, "entry": "qmm_i8t2_gemm", "us_per_call": round(us, 3),
            "tops": round(tops, 2), "peak_tops": INT8_PEAK_TOPS,
            "frac": round(tops / INT8_PEAK_TOPS, 4),
            "weight_GBps": round(wbytes / us / 1e3, 1),
            "hbm_frac": round(tbytes / us / 1e3 / HBM_PEAK_GBS, 4)}


def time_quantize(K, N, w_bit, group_size, steps=20):
    """qmm_quantize of a (K, N) fp16 weight (0.02 N(0,1)), graph-replayed.
    Bytes: the fp16 input (read once; the kernel's second pass hits cache)
    plus the packed outputs."""
    import torch
    import gemv_only_quant_amd as qmm

    g = torch.Generator().manual_seed(9000)
    W = (0.02 * torch.randn((K, N), generator=g)).half().cuda()
    pack = 32 // w_bit
    G = K // group_size
    qw = torch.empty((K // pack, N), dtype=torch.int32, device="cuda")
    sc = torch.empty((G, N), dtype=torch.float16, device="cuda")
    qz = torch.empty(((G + pack - 1) // pack, N), dtype=torch.int32, device="cuda")
    call = lambda: qmm.qmm_quantize(W, qmm.QMM_F16, qw, sc, qz, N, K, w_bit, group_size, False)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(steps):
            call()
    graph.replay()
    torch.cuda.synchronize()
    us = replay_us(graph, steps, f"rtn_int{w_bit}_g{group_size}_fp16_k{K}_n{N}")
    progress(f"quantize K={K} N={N}: {us:.3f} us per call")
    nbytes = W.numel() * 2 + qw.numel() * 4 + sc.numel() * 2 + qz.numel() * 4
    return {"workload": f"rtn_int{w_bit}_g{group_size}_fp16_k{K}_n{N}", "entry": "qmm_quantize",
            "us_per_call": round(us, 2), "GBps": round(nbytes / us / 1e3, 1),
            "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}


def traffic_for(name, path):
    """HBM bytes per launch of workload `name` through qmm_<path> from the
    committed counter summary, if the kernel source it was taken with is
    unchanged; else None."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    for m in re.finditer(r"^traffic_bytes_per_launch:\s+(\S+)\s+(\d+)\s+(\S+)\s+([0-9a-f]+)\s*$",
                         text, re.M):
        if m.group(1) != f"{name}@qmm_{path}":
            continue
        src = os.path.join(CSRC, m.group(3))
        try:
            h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        except OSError:
            return None
        return int(m.group(2)) if h == m.group(4) else None
    return None


def host_info():
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model}


def _timed(fn, budget_s):
    """(seconds per run, runs): fn repeated until budget_s has passed."""
    t0 = time.perf_counter()
    runs = 0
    while True:
        fn()
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return el / runs, runs


def _sample_args(case, m_s, n_s):
    """Oracle arguments of rows [0, m_s) and columns [0, n_s) of a workload."""
    x, xdt, Q, S, Z, M, N, K, wb, gs = case.oracle_args()
    x = x[:m_s]
    if wb == 8:
        Q, S = Q[:n_s], S[:n_s]
    else:
        Q, S = Q[:, :n_s], S[:, :n_s]
        Z = None if Z is None else Z[:, :n_s]
    return (x, xdt, Q, S, Z, m_s, n_s, K, wb, gs)


def cpu_baseline(budget_s=4.0):
    """The oracle on the host's cores.  value: the headline product (every
    output, full size) on all threads; then, per workload, a bounded sample
    (at most 256 rows x 1024 columns, full K) on one thread and on all of them,
    scaled to the whole workload's outputs."""
    import oracle
    import synth_inputs as si
    threads = oracle.host_threads()
    progress(f"cpu baseline on {threads} threads")
    case = si.workload(HEADLINE)
    args = case.oracle_args()
    wbytes, _ = bytes_of(case)
    t_all, runs_all = _timed(lambda: oracle.qmm_mt(*args, threads=threads), budget_s)
    t_one, runs_one = _timed(lambda: oracle.qmm(*args), budget_s)
    per = []
    for name, _ in OTHERS + [(n, None) for n, _ in PREFILL[:2]]:
        c = si.workload(name)
        m_s, n_s = min(c.M, 256), min(c.N, 1024)
        sargs = _sample_args(c, m_s, n_s)
        s1, _ = _timed(lambda: oracle.qmm(*sargs), 0.5)
        sa, _ = _timed(lambda: oracle.qmm_mt(*sargs, threads=threads), 0.5)
        scale = (c.M * c.N) / (m_s * n_s)
        per.append({"workload": name, "sample": f"{m_s} rows x {n_s} columns, K={c.K}",
                    "s_per_call_1_thread": round(s1 * scale, 4),
                    "s_per_call_all_threads": round(sa * scale, 4)})
    t2 = si.workload(TERNARY[1])
    m_s, n_s = 256, 1024
    A = t2.A.numpy()[:m_s]
    Wp = np.ascontiguousarray(t2.Wp.numpy()[:, :n_s])
    s1, _ = _timed(lambda: oracle.i8t2_mm(A, Wp, m_s, n_s, t2.K), 0.5)
    sa, _ = _timed(lambda: oracle.i8t2_mm_mt(A, Wp, m_s, n_s, t2.K, threads=threads), 0.5)
    scale = (t2.M * t2.N) / (m_s * n_s)
    per.append({"workload": TERNARY[1], "sample": f"{m_s} rows x {n_s} columns, K={t2.K}",
                "s_per_call_1_thread": round(s1 * scale, 4),
                "s_per_call_all_threads": round(sa * scale, 4)})
    return {"value": round(wbytes / t_all / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{runs_all} full {HEADLINE} products on {threads} threads "
                      f"({t_all:.4f} s each; fp64 oracle, columns divided over threads)",
            "single_thread": {"value": round(wbytes / t_one / 1e9, 4), "unit": "GB/s",
                              "s_per_call": round(t_one, 4), "runs": runs_one},
            "host": host_info(), "per_workload": per}


def line(r, path):
    case, us = r["case"], r["us"]
    out = {"workload": case.name, "entry": f"qmm_{path}", "us_per_call": round(us, 3),
           "weight_copies_rotated": r["rotated"], "rotated_MB": round(r["rotated_bytes"] / 1e6, 1),
           "weight_GBps": round(r["wbytes"] / us / 1e3, 1),
           "hbm_frac": round(r["tbytes"] / us / 1e3 / HBM_PEAK_GBS, 4),
           "tflops": round(r["flops"] / us / 1e6, 2),
           "mfma_frac": round(r["flops"] / us / 1e6 / MFMA_PEAK_TFLOPS, 4)}
    t = traffic_for(case.name, path)
    if t is not None:
        out["traffic_bytes"] = t
    return out


def probe(spec):
    """Counter probe for rocprofv3 --pmc: three calls of one workload's entry
    point, each on its own copy of the weights (a pool of >= 512 MB, so no
    call finds its weights in cache), then three copies of a 256 MiB device
    buffer (kernel __amd_rocclr_copyBuffer), whose counter readings give the
    scale of known byte counts (256 MiB read, 256 MiB written)."""
    import torch
    import gemv_only_quant_amd as qmm
    import synth_inputs as si

    name, _, entry = spec.partition("@")  # WORKLOAD[@qmm_gemv|@qmm_gemm]
    if name in TERNARY:
        case = si.workload(name)
        d = case.to("cuda")
        Wt = qmm.t2_pack(d.Wp, case.N, case.K)
        copies = max(3, -(-POOL_BYTES // Wt.numel())) if case.M < 1024 else 3
        pool = [Wt.clone() for _ in range(copies)]
        y = torch.empty((case.M, case.N), dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        for i in range(3):
            qmm.qmm_i8t2_gemm(d.A, pool[(i * copies) // 3], y, case.M, case.N, case.K)
        path = "i8t2_gemm"
    else:
        if entry:
            path = entry.replace("qmm_", "")
        else:
            path = HEADLINE_PATH if name == HEADLINE else dict(OTHERS).get(name, "gemm")
        case = si.workload(name)
        wbytes, _ = bytes_of(case)
        d = case.to("cuda")
        Q0 = d.Q if path == "gemv" else qmm.pack(d.Q, case.N, case.K, case.w_bit)
        copies = max(3, -(-POOL_BYTES // wbytes)) if case.M < 1024 else 3
        pool = [(Q0.clone(), d.scales.clone(), None if d.zeros is None else d.zeros.clone())
                for _ in range(copies)]
        y = torch.empty((case.M, case.N), dtype=torch.float32, device="cuda")
        ws = qmm.workspace_for(case.M, case.N, case.K, case.w_bit, case.group_size, "cuda")
        fn = qmm.qmm_gemv if path == "gemv" else qmm.qmm_gemm
        torch.cuda.synchronize()
        for i in range(3):
            Q, s, z = pool[(i * copies) // 3]
            fn(d.x, Q, s, z, y, case.M, case.N, case.K, case.w_bit, case.group_size, workspace=ws)
    torch.cuda.synchronize()
    src = torch.ones(1 << 27, dtype=torch.int16, device="cuda")  # 256 MiB
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"probe {name}: 3 x qmm_{path} ({copies} weight copies), 3 x 256 MiB copy", flush=True)


def trace_summary(db_path):
    """Per-workload kernel durations from a rocprofv3 trace of this script run
    with --kernel-trace --marker-trace: only the dispatches inside a `timed
    <workload>` range (the graph replays that give each time per call) count.
    Prints a Markdown table: dispatches, mean, median, p90, min, max (µs)."""
    import sqlite3
    c = sqlite3.connect(db_path)
    regions = []
    for name, extdata, r0, r1 in c.execute("select name, extdata, start, end from regions "
                                           "order by start"):
        try:  # the range's message is the name, or (rocprofv3) extdata's "message"
            msg = json.loads(extdata or "{}").get("message", name)
        except ValueError:
            msg = name
        if msg and msg.startswith("timed "):
            regions.append((msg, r0, r1))
    kern = c.execute("select name, start, end from kernels order by start").fetchall()
    by = {}
    j = 0
    for label, r0, r1 in regions:
        while j < len(kern) and kern[j][1] < r0:
            j += 1
        k = j
        while k < len(kern) and kern[k][1] <= r1:
            name = re.sub(r"\(.*", "", kern[k][0])
            by.setdefault((label[6:], name), []).append((kern[k][2] - kern[k][1]) / 1e3)
            k += 1
    print("| workload (timed replays) | kernel | dispatches | mean µs | median µs | p90 µs | "
          "min µs | max µs |")
    print("|---|---|---|---|---|---|---|---|")
    for (label, name), d in by.items():
        d = sorted(d)
        p90 = d[min(len(d) - 1, int(0.9 * len(d)))]
        print(f"| {label} | `{name}` | {len(d)} | {statistics.mean(d):.3f} | "
              f"{statistics.median(d):.3f} | {p90:.3f} | {d[0]:.3f} | {d[-1]:.3f} |")


def phases(launches=200):
    """Where the headline tile GEMV's time goes: per-wave real-time stamps
    (100 MHz) from the stamp build of the library (gemv_only_quant_amd/
    build.py --phases), beside the same stamps on a read-only kernel with
    the same grid reading the same bytes per workgroup.  Each launch runs on
    its own weight copy (a pool of >= 512 MB) after the previous one has
    finished, and its stamps are read back before the next.  Then both
    kernels graph-replayed back to back over the pool (the read-only one
    gives the best this launch shape does with no arithmetic), the read-only
    kernel with the GEMV's steps added one at a time, and the matrix cores'
    sustained bf16 and int8 rates on register operands."""
    import ctypes
    import torch
    import gemv_only_quant_amd as qmm
    import synth_inputs as si

    path = os.path.join(ROOT, "gemv_only_quant_amd", "libqmm_phases.so")
    if not os.path.exists(path):
        raise SystemExit(f"{path} is not built; run python gemv_only_quant_amd/build.py --phases")
    lib = ctypes.CDLL(path)
    vp, ci, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.qmm_gemm.argtypes = [vp] * 5 + [ci] * 6 + [vp, sz, vp]
    lib.qmm_gemm.restype = ci
    lib.qmm_phase_stamps_read.argtypes = [vp, sz]
    lib.qmm_phase_stamps_read.restype = ci
    lib.qmm_phase_readonly.argtypes = [vp, vp, ci, ci, vp]
    lib.qmm_phase_readonly.restype = ci

    case = si.workload(HEADLINE)
    d = case.to("cuda")
    Q0 = qmm.pack(d.Q, case.N, case.K, case.w_bit)
    wbytes = Q0.numel() * Q0.element_size()
    copies = max(2, -(-POOL_BYTES // wbytes))
    pool = [Q0] + [Q0.clone() for _ in range(copies - 1)]
    y = torch.empty((case.M, case.N), dtype=torch.float32, device="cuda")
    sink = torch.empty((case.N // 16) * 256, dtype=torch.int32, device="cuda")
    waves = (case.N // 16) * 4
    nblk = case.K // 128
    stream = torch.cuda.current_stream().cuda_stream
    buf = np.zeros(waves * 8, dtype=np.uint64)
    x_dt = qmm.QMM_F16 if case.x_dtype == si.F16 else qmm.QMM_BF16

    def gemv(i):
        st = lib.qmm_gemm(d.x.data_ptr(), pool[i % copies].data_ptr(), d.scales.data_ptr(),
                          d.zeros.data_ptr(), y.data_ptr(), case.M, case.N, case.K, case.w_bit,
                          case.group_size, x_dt, None, 0, stream)
        assert st == 0, st

    def readonly(i):
        assert lib.qmm_phase_readonly(pool[i % copies].data_ptr(), sink.data_ptr(),
                                      case.N // 16, nblk, stream) == 0

    def run(fn, slots):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        per_launch = []
        for i in range(launches + 10):
            ev0.record()
            fn(i)
            ev1.record()
            torch.cuda.synchronize()
            assert lib.qmm_phase_stamps_read(buf.ctypes.data, buf.size) == 0
            if i < 10:
                continue  # warm-up
            t = buf.reshape(waves, 8).astype(np.int64)
            t0 = t[:, 0]
            row = {"event_us": ev0.elapsed_time(ev1) * 1e3,
                   "span_us": (t[:, 5].max() - t0.min()) / 100.0,
                   "entry_spread_us": (t0.max() - t0.min()) / 100.0,
                   "wave_total_us": float(np.median(t[:, 5] - t0)) / 100.0}
            for k, name in slots.items():
                row[name] = float(np.median(t[:, k] - t0)) / 100.0
            per_launch.append(row)
        keys = per_launch[0].keys()
        return {k: round(float(np.median([r[k] for r in per_launch])), 3) for k in keys}

    g = run(gemv, {1: "x_slice_ready_us", 2: "group_table_ready_us", 6: "first_block_done_us",
                   7: "half_blocks_done_us", 3: "weights_consumed_us", 4: "scales_in_lds_us"})
    r = run(readonly, {3: "last_load_returned_us"})

    # graph-replayed back to back over the pool (the bench's own timing), the
    # GEMV and the read-only kernel of the same grid: the read rate this
    # launch shape reaches at best, with no arithmetic at all
    def replayed(fn, label, steps=200):
        for i in range(10):
            fn(i)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                fn(i)
        graph.replay()
        torch.cuda.synchronize()
        us = replay_us(graph, steps, label)
        del graph
        return {"us_per_call": round(us, 3), "read_TBps": round(wbytes / us / 1e6, 3)}

    cur = lambda: torch.cuda.current_stream().cuda_stream  # noqa: E731 (the capture stream)

    def gemv_cur(i):
        assert lib.qmm_gemm(d.x.data_ptr(), pool[i % copies].data_ptr(), d.scales.data_ptr(),
                            d.zeros.data_ptr(), y.data_ptr(), case.M, case.N, case.K, case.w_bit,
                            case.group_size, x_dt, None, 0, cur()) == 0

    def readonly_cur(i):
        assert lib.qmm_phase_readonly(pool[i % copies].data_ptr(), sink.data_ptr(),
                                      case.N // 16, nblk, cur()) == 0

    rep = {"tile_gemv_stamp_build": replayed(gemv_cur, "phases gemv"),
           "read_only_same_grid": replayed(readonly_cur, "phases read-only")}

    # the read-only kernel with the GEMV's steps added one at a time
    # (calibrate.hip, readonly_probe_kernel): which of them costs time
    lib.qmm_calib_readonly.argtypes = [ci, vp, vp, vp, ci, vp]
    lib.qmm_calib_readonly.restype = ci
    assert nblk == 32 and d.x.numel() * d.x.element_size() >= 8192
    probes = {}
    for v, label in ((0, "loads_only"), (1, "x_slice"), (2, "per_block_dot_work"),
                     (4, "closing_exchange"), (3, "x_slice+dot_work"), (7, "all_three")):
        def probe_v(i, v=v):
            assert lib.qmm_calib_readonly(v, pool[i % copies].data_ptr(), d.x.data_ptr(),
                                          sink.data_ptr(), case.N // 16, cur()) == 0
        probes[label] = replayed(probe_v, f"phases probe {label}")["us_per_call"]
    rep["read_only_probes_us_per_call"] = probes

    # the matrix cores' sustained rate: 8 independent MFMAs per round on
    # register operands, 4 workgroups per CU, zero and random operands
    lib.qmm_calib_mfma.argtypes = [vp, vp, ci, ci, ci, vp]
    lib.qmm_calib_mfma.restype = ci
    blocks, iters = 1024, 20000
    sink2 = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    gen = torch.Generator().manual_seed(5)
    loops = {}
    for kind, int8, peak in (("bf16_16x16x32", 0, MFMA_PEAK_TFLOPS),
                             ("int8_16x16x64", 1, INT8_PEAK_TOPS)):
        rnd = (torch.randint(-128, 128, (2048,), generator=gen, dtype=torch.int8) if int8 else
               torch.randn(128 * 8, generator=gen).to(torch.bfloat16))
        res = {}
        for label, seed in (("zero_operands", torch.zeros_like(rnd)), ("random_operands", rnd)):
            sd = seed.to("cuda")
            assert lib.qmm_calib_mfma(sd.data_ptr(), sink2.data_ptr(), blocks, 100, int8,
                                      stream) == 0
            torch.cuda.synchronize()
            ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev0.record()
            assert lib.qmm_calib_mfma(sd.data_ptr(), sink2.data_ptr(), blocks, iters, int8,
                                      stream) == 0
            ev1.record()
            torch.cuda.synchronize()
            secs = ev0.elapsed_time(ev1) * 1e-3
            ops = blocks * 4 * iters * 8 * 2.0 * 16 * 16 * (64 if int8 else 32)
            res[label] = {"ms": round(secs * 1e3, 3), "tops": round(ops / secs / 1e12, 1),
                          "frac_of_peak": round(ops / secs / 1e12 / peak, 4)}
        loops["mfma_loop_" + kind] = dict(res, peak=peak)
    out = {"workload": HEADLINE, "launches": launches, "stamp_clock": "s_memrealtime, 100 MHz",
           "tile_gemv": g, "read_only_same_grid": r, "graph_replayed": rep,
           "mfma_loops": dict(loops, blocks=blocks, waves_per_block=4, rounds=iters,
                              mfma_per_round=8)}
    print(json.dumps(out), flush=True)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--quick", action="store_true", help="headline only")
    ap.add_argument("--probe", metavar="WORKLOAD",
                    help="three calls of one workload and a 256 MiB copy, for counter runs")
    ap.add_argument("--trace-summary", metavar="DB",
                    help="per-workload kernel durations from a rocprofv3 trace database")
    ap.add_argument("--phases", action="store_true",
                    help="phase stamps of the headline GEMV (needs build.py --phases)")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the kernels run on a single device; the design notes describe sharding)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth_inputs as si
    torch.cuda.set_device(0)
    if args.probe:
        probe(args.probe)
        return
    if args.phases:
        phases()
        return
    r = time_workload(HEADLINE, args.steps, args.warmup, HEADLINE_PATH)
    case, us = r["case"], r["us"]
    achieved = r["tbytes"] / (us * 1e-6) / 1e9
    out = {
        "metric": "effective weight GB/s @M=1 and TFLOP/s @M=4096, int4-g128 and int8 W-only",
        "value": round(r["wbytes"] / (us * 1e-6) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if case.x_dtype == si.F16 else "bf16",
        "data": "synthetic",
        "config": {"workload": HEADLINE, "M": case.M, "N": case.N, "K": case.K,
                   "w_bit": case.w_bit, "group_size": case.group_size,
                   "zeros": case.zeros is not None, "accumulate": "f32",
                   "entry": f"qmm_{HEADLINE_PATH}",
                   "layout": "tile layout written once by qmm_pack from the canonical qw "
                             "(offline, not timed)" if HEADLINE_PATH == "gemm" else "canonical",
                   "weight_pool_copies": r["copies"], "weight_copies_rotated": r["rotated"],
                   "rotated_MB": round(r["rotated_bytes"] / 1e6, 1),
                   "timing": "hip graph replay, 1 GiB cache eviction before each timed replay",
                   "eager_us_per_call": round(r["eager_us"], 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for(HEADLINE, HEADLINE_PATH)},
    }
    if not args.quick:
        out["workloads"] = [line(time_workload(n, 200, 20, p), p) for n, p in OTHERS]
        pre = []
        for n, out_dt in PREFILL:
            # 50 calls (about 20 ms) per replay: 10-call replays (4 ms) measured 416 us per
            # call against 363 at 50 and 362 at 200 -- too short to reach steady clocks
            p = time_workload(n, 50, 10, "gemm", out_dt)
            tf = p["flops"] / (p["us"] * 1e-6) / 1e12
            pre.append({"workload": n, "entry": "qmm_gemm" if out_dt == "f32" else "qmm_gemm_ex",
                        "y_dtype": out_dt, "us_per_call": round(p["us"], 2),
                        "tflops": round(tf, 2), "peak_tflops": MFMA_PEAK_TFLOPS,
                        "frac": round(tf / MFMA_PEAK_TFLOPS, 4)})
            t = traffic_for(n, "gemm") if out_dt == "f32" else None
            if t is not None:
                pre[-1]["traffic_bytes"] = t
        out["prefill"] = pre
        out["ternary"] = [time_ternary(n, 200 if n.startswith("i8t2_m16") else 50, 10)
                          for n in TERNARY]
        out["quantize"] = [time_quantize(4096, 4096, 4, 128)]
        out["calibration"] = calibration()
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
