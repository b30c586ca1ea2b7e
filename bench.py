"""Benchmark of the weight-only quantized matmul on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--workload NAME]

A step is one call of the hot path on one batch of synthetic input already
resident in HBM.  The headline workload is the int4 group-128 asymmetric
decode GEMV (M=1, K=N=4096, fp16 x, fp32 accumulation) and `value` is its
effective weight bandwidth (packed weights + scales + zeros per call / time).

Memory-bound calls rotate over a pool of weight copies (> 2 x the 256 MB
Infinity Cache), so every call streams its weights from HBM.  The K timed
calls are captured once in a HIP graph and replayed; HIP events on the
launch stream bracket the replay.  The prefill MFMA workload (M=4096) is
timed the same way and reported under "prefill".  The CPU baseline times the
plain single-threaded oracle on the host (see "cpu_baseline.sample").
Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix peak
POOL_BYTES = 512 << 20          # weight pool for memory-bound workloads

HEADLINE = "int4_g128_asym_gemv_m1_k4096_n4096"
PREFILL = "int4_g128_asym_prefill_m4096_k4096_n11008"


def bytes_of(case):
    """Algorithmic bytes per call: packed Q, scales, zeros, x and y, each once."""
    w = case.Q.numel() * case.Q.element_size()
    w += case.scales.numel() * case.scales.element_size()
    if case.zeros is not None:
        w += case.zeros.numel() * case.zeros.element_size()
    io = case.x.numel() * case.x.element_size() + case.M * case.N * 4
    return w, w + io


def make_call(qmm, d, y, ws, path, Q):
    c = d
    fn = qmm.qmm_gemv if path == "gemv" else qmm.qmm_gemm

    def call():
        fn(c.x, Q, c.scales, c.zeros, y, c.M, c.N, c.K, c.w_bit, c.group_size, workspace=ws)
    return call


def time_workload(name, steps, warmup, path):
    import torch
    import gemv_only_quant_amd as qmm
    import synth_inputs as si

    case = si.workload(name)
    wbytes, tbytes = bytes_of(case)
    d = case.to("cuda")
    Q = d.Q if path == "gemv" else qmm.pack(d.Q, case.N, case.K, case.w_bit)
    copies = 1 if path == "gemm" and case.M >= 1024 else max(1, -(-POOL_BYTES // wbytes))
    pool = []
    for i in range(copies):
        if i == 0:
            pool.append((d, Q))
        else:
            di = si.Case(d.name, d.M, d.N, d.K, d.w_bit, d.group_size, d.x_dtype, d.x.clone(),
                         d.Q, d.scales.clone(),
                         None if d.zeros is None else d.zeros.clone())
            pool.append((di, Q.clone()))
    y = torch.empty((case.M, case.N), dtype=torch.float32, device="cuda")
    ws = qmm.workspace_for(case.M, case.N, case.K, case.w_bit, case.group_size, "cuda")
    calls = [make_call(qmm, di, y, ws, path, Qi) for di, Qi in pool]

    for i in range(warmup):
        calls[i % copies]()
    torch.cuda.synchronize()

    # eager timing (host launch per call)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_eager = min(steps, 200)
    start.record()
    for i in range(n_eager):
        calls[i % copies]()
    end.record()
    torch.cuda.synchronize()
    eager_us = start.elapsed_time(end) * 1e3 / n_eager

    # graph of exactly `steps` calls, replayed once untimed, then timed
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls[0]()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for i in range(steps):
            calls[i % copies]()
    graph.replay()
    torch.cuda.synchronize()
    y_graph = y.clone()
    calls[(steps - 1) % copies]()     # eager result of the same last call
    torch.cuda.synchronize()
    assert torch.equal(y_graph, y), "graph replay differs from eager call"

    torch.cuda.synchronize()
    start.record()
    graph.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    us = ms * 1e3 / steps
    flops = 2.0 * case.M * case.N * case.K
    return dict(case=case, us=us, ms_total=ms, eager_us=eager_us, wbytes=wbytes,
                tbytes=tbytes, flops=flops, copies=copies)


def cpu_baseline(name, budget_s=10.0):
    import oracle
    import synth_inputs as si
    case = si.workload(name)
    args = case.oracle_args()
    wbytes, _ = bytes_of(case)
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.qmm(*args)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    t = el / reps
    return {"value": round(wbytes / t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} full {name} products (fp64 oracle, 1 thread), "
                      f"{t:.3f} s each"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--workload", default=HEADLINE)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the kernels run on a single device; see the design notes on sharding)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth_inputs as si
    torch.cuda.set_device(0)
    path = "gemv" if si.workload(args.workload).M <= 16 and args.workload.find("prefill") < 0 \
        else "gemm"
    r = time_workload(args.workload, args.steps, args.warmup, path)
    case = r["case"]
    us = r["us"]
    value = r["wbytes"] / (us * 1e-6) / 1e9
    achieved = r["tbytes"] / (us * 1e-6) / 1e9
    out = {
        "metric": "effective weight GB/s @M=1 and TFLOP/s @M=4096, int4-g128 and int8 W-only",
        "value": round(value, 2),
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
        "config": {"workload": args.workload, "M": case.M, "N": case.N, "K": case.K,
                   "w_bit": case.w_bit, "group_size": case.group_size,
                   "zeros": case.zeros is not None, "accumulate": "f32", "entry": f"qmm_{path}",
                   "weight_pool_copies": r["copies"], "timing": "hip graph replay",
                   "eager_us_per_call": round(r["eager_us"], 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None},
    }
    if not args.no_prefill:
        try:
            p = time_workload(PREFILL, 20, 3, "gemm")
            tf = p["flops"] / (p["us"] * 1e-6) / 1e12
            out["prefill"] = {"workload": PREFILL, "us_per_call": round(p["us"], 2),
                              "tflops": round(tf, 2), "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                              "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
        except Exception as e:  # the MFMA path may not support this shape yet
            out["prefill"] = {"workload": PREFILL, "error": str(e)[:200]}
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
