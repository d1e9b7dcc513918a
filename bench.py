"""Benchmark: fp16 8192^3 GEMM (headline) and the fused SwiGLU-GEMM at M = 2048.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one sg_gemm call C = alpha*A@B + beta*C (NN, fp16 in, fp32 accumulate,
fp16 out, M = N = K = 8192, alpha = 1, beta = 0) on inputs already resident in
HBM: host validation, tile loads, MFMA main loop and epilogue.  Timing uses HIP
events recorded on the stream the library launches on (torch's current stream),
W untimed warm-up steps, then exactly K timed steps between two synchronisations.
Three input sets are rotated so the 256 MB last-level cache cannot keep one set
resident across steps.

Also reported (same run): the fused SwiGLU-GEMM, bf16, A[2048 x 896] x
W_fused[896 x 9728] -> Y[2048 x 4864], against this library's unfused path
(two sg_gemm calls writing Gate and Up, then sg_silu_mul) and torch eager as
context; and the fp64 CPU oracle timed on a bounded sample of the GEMM rows.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TFLOPS & % of MFMA peak: fp16 8192³ GEMM; fused SwiGLU-GEMM at M=2048"
PEAK_F16_TFLOPS = 2500.0        # MI355X dense fp16/bf16 MFMA peak
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm16_f16_nn_8192.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "swiglu_gemm_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_src_sha") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def time_steps(fn, steps, warmup, torch):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        fn(i)
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps          # ms per step


def to_dev(bits, dtype, torch):
    t = torch.from_numpy(np.ascontiguousarray(bits))
    t = t.view(torch.int16).view(torch.float16 if dtype == "f16" else torch.bfloat16)
    return t.to("cuda:0")


def cpu_baseline(p, M, N, K, budget_s=12.0):
    """The fp64 oracle on a bounded sample of the same GEMM: R full rows of C (all
    N columns, full K), R chosen to take about budget_s seconds."""
    import oracle
    threads = oracle.max_threads()
    rows_per_batch = threads
    done = 0
    t_total = 0.0
    while t_total < budget_s and done < M:
        rows = np.arange(done, min(done + rows_per_batch, M))
        sub = dict(A=np.ascontiguousarray(p["A"][rows, :]), C=np.ascontiguousarray(p["C"][rows, :]))
        t0 = time.perf_counter()
        oracle.gemm("N", "N", len(rows), N, K, 1.0, sub["A"], p["lda"], p["B"], p["ldb"], 0.0,
                    sub["C"], p["ldc"], "f16", nthreads=threads)
        t_total += time.perf_counter() - t0
        done += len(rows)
    flops = 2.0 * done * N * K
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d rows of the fp16 %dx%dx%d GEMM (full N and K), fp64 i-p-j "
                      "oracle incl. decode, %.1f s" % (done, M, M, N, K, t_total)}


def bench_swiglu(torch, sg, inputs, steps, warmup):
    M, N, K = 2048, 4864, 896
    sets = []
    for r in range(4):
        pb = inputs.swiglu_problem(4, M + r, N, K, "bf16")      # distinct seeds per set
        A = to_dev(pb["A"][:M], "bf16", torch)
        W1 = to_dev(pb["W1"], "bf16", torch)
        W2 = to_dev(pb["W2"], "bf16", torch)
        Wf = sg.interleave_gate_up(W1, W2)
        sets.append((A, W1, W2, Wf))
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    G = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    U = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")

    def fused(i):
        A, _, _, Wf = sets[i % 4]
        sg.swiglu_gemm(A, Wf, Y)

    def unfused(i):
        A, W1, W2, _ = sets[i % 4]
        sg.gemm(A, W1, G)
        sg.gemm(A, W2, U)
        sg.silu_mul(G, U, Y)

    def eager(i):
        A, W1, W2, _ = sets[i % 4]
        torch.nn.functional.silu(A @ W1) * (A @ W2)

    t_fused = time_steps(fused, steps, warmup, torch)
    cfg = sg.last_config()
    t_unfused = time_steps(unfused, steps, warmup, torch)
    t_eager = time_steps(eager, steps, warmup, torch)
    flops = 4.0 * M * N * K
    tf = flops / (t_fused * 1e-3) / 1e12
    return {"workload": "fused SwiGLU-GEMM bf16 A[2048x896] W_fused[896x9728] -> Y[2048x4864]",
            "ms": round(t_fused, 5), "tflops": round(tf, 2),
            "frac_of_peak": round(tf / PEAK_F16_TFLOPS, 4),
            "unfused_ms": round(t_unfused, 5), "speedup_vs_unfused": round(t_unfused / t_fused, 3),
            "torch_eager_ms": round(t_eager, 5),
            "speedup_vs_torch_eager": round(t_eager / t_fused, 3), "kernel_config": cfg}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-swiglu", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only (the library is single-GPU); --gpus %d is not "
              "supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import swiglu_gemm_amd as sg
    from swiglu_gemm_amd import inputs
    sg.lib()                      # raises if the HIP library is not built
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    M = N = K = 8192
    print("bench: generating inputs", file=sys.stderr, flush=True)
    host = inputs.gemm_problem(2, "N", "N", M, N, K, "f16", "normal", scale=1.0 / np.sqrt(K),
                               beta_zero=True)
    sets = []
    for r in range(3):
        if r == 0:
            A, B = to_dev(host["A"], "f16", torch), to_dev(host["B"], "f16", torch)
        else:   # further sets: same distribution, other seeds
            p2 = inputs.gemm_problem(200 + r, "N", "N", M, N, K, "f16", "normal",
                                     scale=1.0 / np.sqrt(K), beta_zero=True)
            A, B = to_dev(p2["A"], "f16", torch), to_dev(p2["B"], "f16", torch)
        C = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
        sets.append((A, B, C))

    def step(i):
        A, B, C = sets[i % 3]
        sg.gemm(A, B, C, alpha=1.0, beta=0.0)

    print("bench: timing fp16 8192^3 GEMM", file=sys.stderr, flush=True)
    ms = time_steps(step, args.steps, args.warmup, torch)
    cfg = sg.last_config()
    flops = 2.0 * M * N * K
    tflops = flops / (ms * 1e-3) / 1e12
    traffic = measured_traffic()
    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "fp16 GEMM NN M=N=K=8192 alpha=1 beta=0, fp32 accumulate, fp16 out; "
                               "A,B ~ N(0,1)/sqrt(K)", "M": M, "N": N, "K": K,
                   "kernel_config": cfg, "input_sets_rotated": 3},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_F16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_F16_TFLOPS, 4),
                     "traffic": traffic, "kernel": "gemm16_kernel (one launch per step)",
                     "algorithmic_flops_per_launch": flops},
    }
    if not args.no_swiglu:
        print("bench: timing SwiGLU M=2048", file=sys.stderr, flush=True)
        out["swiglu_m2048"] = bench_swiglu(torch, sg, inputs, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(host, M, N, K, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
