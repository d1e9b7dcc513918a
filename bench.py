"""Benchmark: fp16 8192^3 GEMM (headline) and the fused SwiGLU-GEMM (M = 2048 and
the other workload sizes), on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--quick]

A step is one sg_gemm call C = alpha*A@B + beta*C (NN, fp16 in, fp32 accumulate,
fp16 out, M = N = K = 8192, alpha = 1, beta = 0) on inputs already resident in
HBM: host validation, tile loads, MFMA main loop and epilogue (one kernel
launch).  Timing uses HIP events recorded on the stream the library launches on
(torch's current stream): ~0.4 s of untimed spin-up work so the clocks have
ramped, W untimed warm-up steps, then exactly K timed steps between two
synchronisations.  Three input sets are rotated so the 256 MB
last-level cache cannot keep one set resident across steps.

Also reported, same run: per-step median / min / p90 of the headline; the same
GEMM in bf16; the ragged bf16 GEMMs (1000^3 and 4097x3001x2049, every transpose
pair); the fused SwiGLU-GEMM (bf16: A[M x 896], W_fused[896 x 9728], M in {128,
512, 2048, 8192}; e4m3 with per-tensor scales: A[M x 4096], W_fused[4096 x 22016],
M in {1, 16, 256, 4096}) with cold weights (copies rotated past the last-level
cache) and hot, against this library's unfused path (two sg_gemm calls writing
Gate and Up, then sg_silu_mul), the split-weight entry point (separate W1, W2:
w12_ms), Kernel-1's Gate-then-Up schedule on the same split weights (seq_ms), HIP
graph replays of the fused and unfused steps, and torch eager as context; the fused
bias + GELU GEMM epilogue; the fp32 GEMM (256^3 and 4096^3); the clock before,
after and under load and the board's read / copy bandwidth; and the fp64 CPU oracle
timed on a bounded sample of the GEMM rows, whose outputs double as an every-element
check of those rows (numerics).

Prints ONE JSON line.

Counter helpers (used to produce the committed HBM-traffic figure):
    python bench.py --pmc-probe            # copy of a known size, then 3 GEMM launches
    python bench.py --pmc-probe-nt         # bf16 GEMM, B stored N x K, beside hipBLASLt
    python bench.py --pmc-summarize FETCH.csv WRITE.csv   # -> profiles/traffic_*.json

Power-limited MFMA ceiling (context for roofline.frac, a separate run):
    python bench.py --mfma-ceiling         # pure MFMA loop on zero / constant / random data
Pipeline-depth / tile study of the headline GEMM, with hipBLASLt beside it:
    python bench.py --stage-sweep          # one JSON line per configuration
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TFLOPS & % of MFMA peak: fp16 8192³ GEMM; fused SwiGLU-GEMM at M=2048"
PEAK = {"f16": 2500.0, "bf16": 2500.0, "e4m3": 5000.0, "f32": 157.3}   # MI355X dense MFMA TFLOP/s
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm16_f16_nn_8192.json")
COPY_BYTES = 512 * 1024 * 1024          # calibration copy: reads and writes this many bytes


def kernel_source_hash() -> str:
    """The library's source hash (the one built into it, see sg_build_info)."""
    from swiglu_gemm_amd import build
    return build.source_hash()


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


def spin_up(fn, torch, seconds=0.4):
    """Untimed work before the warm-up steps so the GPU clocks have ramped up."""
    t_end = time.perf_counter() + seconds
    i = 0
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def time_steps(fn, steps, warmup, torch):
    spin_up(fn, torch)
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


def time_graph(fn, nsteps, replays, torch, check=None):
    """GPU time per step of `fn`, captured into a HIP graph (nsteps steps per graph)
    and replayed: the per-call host cost of an eager loop is gone, as in a serving
    loop that replays a graph.  `check`, if given, is called after an eager step and
    after each of three replays (with eager work and synchronisations between them)
    and must return the same value each time."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(nsteps):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = check() if check else None
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(nsteps):
            fn(i)
    if check:
        for _ in range(3):
            fn(0)                      # eager work between the replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            if not check() == ref:
                raise RuntimeError("graph replay result differs from the eager one")
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / (replays * nsteps)
    del g
    return ms


def to_dev(bits, dtype, torch):
    t = torch.from_numpy(np.ascontiguousarray(bits))
    if dtype == "e4m3":
        return t.view(torch.float8_e4m3fn).to("cuda:0")
    if dtype == "f32":
        return t.view(torch.float32).to("cuda:0")
    t = t.view(torch.int16).view(torch.float16 if dtype == "f16" else torch.bfloat16)
    return t.to("cuda:0")


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(p, M, N, K, budget_s=12.0):
    """The fp64 oracle on a bounded sample of the same GEMM: R full rows of C (all N
    columns, full K) on every host core, R chosen to take about budget_s seconds.  The
    operands are decoded to fp64 once, before the clock starts, so only the oracle's
    i-p-j loop is timed.  Returns the record and the computed rows (for the error
    report beside it)."""
    import oracle
    threads = oracle.max_threads()
    B = oracle.decode(p["B"], "f16").ravel()
    batch = 2 * threads
    done, t_total = 0, 0.0
    rows_out = []
    while t_total < budget_s and done < M:
        r1 = min(done + batch, M)
        a = oracle.decode(np.ascontiguousarray(p["A"][done:r1, :]), "f16").ravel()
        c = np.zeros((r1 - done) * N)
        t0 = time.perf_counter()
        oracle.gemm_f64("N", "N", r1 - done, N, K, 1.0, a, p["lda"], B, p["ldb"], 0.0, c, N,
                        nthreads=threads)
        t_total += time.perf_counter() - t0
        rows_out.append(c.reshape(r1 - done, N))
        done = r1
    flops = 2.0 * done * N * K
    rec = {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": "rows 0..%d of the %d-row fp16 %dx%dx%d GEMM (full N and K): the fp64 "
                     "i-p-j oracle loop on %d threads, operands decoded before timing, %.1f s"
                     % (done - 1, M, M, N, K, threads, t_total)}
    return rec, np.concatenate(rows_out, axis=0)


def error_report(y, yhat, atol, rtol):
    """Error of GPU values y against oracle values yhat: largest absolute and relative
    error, the largest error over max|yhat|, the share of elements more than 1 % off,
    and the worst error as a fraction of the tolerance atol + rtol*|yhat|."""
    d = np.abs(y - yhat)
    a = np.abs(yhat)
    nz = a > 0
    return {"elements": int(d.size), "max_abs": float(d.max()),
            "max_rel": float((d[nz] / a[nz]).max()) if nz.any() else 0.0,
            "max_abs_over_max_ref": float(d.max() / a.max()) if a.max() > 0 else 0.0,
            "share_rel_gt_1pct": float(np.count_nonzero(d > 0.01 * a)) / d.size,
            "worst_over_tolerance": float(np.max(d / (atol + rtol * a)))}


def f16_bits_to_f64(bits):
    return bits.view(np.float16).astype(np.float64)


def bf16_bits_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


COLD_BYTES = 512 * 1024 * 1024     # rotate operand copies past the 256 MB last-level cache


def bench_swiglu(torch, sg, inputs, dtype, M, N, K, steps, warmup, eager=True, keep=None):
    """Fused vs this library's unfused path (vs torch eager) for one SwiGLU size.
    Cold: the weights rotate through enough device copies (> 512 MB in all) that
    W_fused comes from HBM each step; hot: two copies, which the last-level cache
    keeps.  Two seeded problems; the further copies are device clones.  With a dict
    `keep`, the first problem's inputs and its fused and unfused outputs are stored
    there (host copies) for the error report."""
    workload = 4 if dtype == "bf16" else 5
    base = []
    for r in range(2):
        pb = inputs.swiglu_problem(workload, M, N, K, dtype) if r == 0 else \
            inputs.swiglu_problem(100 + workload, M, N, K, dtype)
        A = to_dev(pb["A"], dtype, torch)
        W1 = to_dev(pb["W1"], dtype, torch)
        W2 = to_dev(pb["W2"], dtype, torch)
        Wf = sg.interleave_gate_up(W1, W2)
        base.append((A, W1, W2, Wf, pb["scale_a"], pb["scale_w"]))
    esz = 1 if dtype == "e4m3" else 2
    per_set = (M * K + 2 * K * 2 * N) * esz           # A, W1 + W2, W_fused
    ncold = max(4, -(-COLD_BYTES // per_set))
    sets = [base[r % 2] if r < 2 else tuple(x.clone() if torch.is_tensor(x) else x
                                            for x in base[r % 2]) for r in range(ncold)]
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    G = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    U = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")

    def fused_over(pool):
        def fn(i):
            A, _, _, Wf, sa, sw = pool[i % len(pool)]
            sg.swiglu_gemm(A, Wf, Y, sa, sw)
        return fn

    def unfused(i):
        A, W1, W2, _, sa, sw = sets[i % ncold]
        sg.gemm(A, W1, G, alpha=sa * sw)
        sg.gemm(A, W2, U, alpha=sa * sw)
        sg.silu_mul(G, U, Y)

    def w12(i):
        A, W1, W2, _, sa, sw = sets[i % ncold]
        sg.swiglu_gemm_w12(A, W1, W2, Y, sa, sw)

    t_fused_eager = time_steps(fused_over(sets), steps, warmup, torch)
    cfg = sg.last_config()
    # the same steps replayed from a HIP graph: kernel time without the per-call host
    # cost (the last step of each replay writes Y from the same copy of the weights)
    nsteps = 2 * ncold
    def y_bits():
        v = Y.view(torch.int16).to(torch.int64)
        return (v.sum().item(), (v * v).sum().item(), (v * torch.arange(
            v.numel(), device=v.device, dtype=torch.int64).view_as(v)).sum().item())
    replays = max(4, steps // nsteps + 1)
    t_fused = time_graph(fused_over(sets), nsteps, replays, torch, check=y_bits)
    t_hot = time_steps(fused_over(base), steps, warmup, torch)
    t_w12 = time_steps(w12, steps, warmup, torch)
    cfg_w12 = sg.last_config()
    # Gate then Up (Kernel-1 of the SwiGLU page) on the same split weights, its tile
    # chosen as the library does (256-row tiles once they fill the CUs, else 128-row
    # tiles with the loads in producer waves)
    big = -(-M // 256) * -(-2 * N // 256) >= 256
    seq_cfg = (51 if big else 54) if dtype == "e4m3" else (49 if big else 53)
    os.environ["SG_FORCE_CONFIG"] = "%d,1" % seq_cfg
    try:
        t_seq = time_steps(w12, steps, warmup, torch)
        cfg_seq = sg.last_config()
    finally:
        os.environ.pop("SG_FORCE_CONFIG", None)
    t_unfused_eager = time_steps(unfused, steps, warmup, torch)
    t_unfused = time_graph(unfused, nsteps, replays, torch, check=y_bits)
    if keep is not None:
        A, W1, W2, Wf, sa, sw = base[0]
        sg.swiglu_gemm(A, Wf, Y, sa, sw)
        keep["fused"] = Y.view(torch.int16).cpu().numpy().view(np.uint16)
        unfused(0)
        keep["unfused"] = Y.view(torch.int16).cpu().numpy().view(np.uint16)
        keep["problem"] = inputs.swiglu_problem(workload, M, N, K, dtype)
    flops = 4.0 * M * N * K
    nbytes = M * K * esz + K * 2 * N * esz + M * N * 2
    tf = flops / (t_fused_eager * 1e-3) / 1e12
    gbs = nbytes / (t_fused_eager * 1e-3) / 1e9
    out = {"dtype": dtype, "M": M, "N": N, "K": K, "ms": round(t_fused_eager, 5),
           "ms_graph": round(t_fused, 5),
           "timing": "eager loop of library calls (ms); the same steps replayed from a HIP graph "
                     "(ms_graph, replays checked against the eager result)",
           "tflops": round(tf, 2), "frac_of_mfma_peak": round(tf / PEAK[dtype], 4),
           "hbm_gbs_algorithmic": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
           "weights": "cold: %d rotated copies, %.0f MB" % (ncold, ncold * per_set / 1e6),
           "ms_hot": round(t_hot, 5),
           "unfused_ms": round(t_unfused_eager, 5), "unfused_ms_graph": round(t_unfused, 5),
           "speedup_vs_unfused": round(t_unfused_eager / t_fused_eager, 3),
           "speedup_vs_unfused_graph": round(t_unfused / t_fused, 3),
           "kernel_config": cfg,
           "w12_ms": round(t_w12, 5), "w12_kernel_config": cfg_w12,
           "seq_ms": round(t_seq, 5), "seq_kernel_config": cfg_seq}
    if eager and dtype == "bf16":
        def eager_fn(i):
            A, W1, W2, _, _, _ = sets[i % ncold]
            torch.nn.functional.silu(A @ W1) * (A @ W2)
        t_eager = time_steps(eager_fn, steps, warmup, torch)
        out["torch_eager_ms"] = round(t_eager, 5)
        out["speedup_vs_torch_eager"] = round(t_eager / t_fused_eager, 3)
    return out


def step_stats(fn, steps, torch):
    """Per-step times (HIP events around each step) after the timed region: the
    median, min and 90th percentile beside the contract's mean."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i, (a, b) in enumerate(ev):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    return {"median_ms": round(float(np.median(t)), 5), "min_ms": round(float(t.min()), 5),
            "p90_ms": round(float(np.percentile(t, 90)), 5), "steps": steps}


def bench_gemm_bf16_8192(torch, sg, steps, warmup):
    """The headline shape in bf16 (same distribution, three rotated sets)."""
    M = N = K = 8192
    sets = []
    for r in range(3):
        g = torch.Generator(device="cuda:0").manual_seed(300 + r)
        A = (torch.randn(M, K, device="cuda:0", generator=g) / np.sqrt(K)).bfloat16()
        B = (torch.randn(K, N, device="cuda:0", generator=g) / np.sqrt(K)).bfloat16()
        sets.append((A, B, torch.empty(M, N, dtype=torch.bfloat16, device="cuda:0")))

    def step(i):
        A, B, C = sets[i % 3]
        sg.gemm(A, B, C)
    ms = time_steps(step, steps, warmup, torch)
    tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 5), "tflops": round(tf, 2), "frac_of_mfma_peak": round(tf / PEAK["bf16"], 4),
            "kernel_config": sg.last_config()}


def bench_gemm_f32(torch, sg, inputs, steps, warmup):
    """fp32 GEMM: the 256^3 parity workload (alpha 1.5, beta 0.5, U[-1,1]; a latency
    figure) and 4096^3 NN (alpha 1, beta 0) against the fp32 MFMA peak."""
    out = []
    for (M, alpha, beta) in ((256, 1.5, 0.5), (4096, 1.0, 0.0)):
        p = inputs.gemm_problem(1, "N", "N", M, M, M, "f32", "uniform")
        A, B, C = (to_dev(p["A"], "f32", torch), to_dev(p["B"], "f32", torch),
                   to_dev(p["C"], "f32", torch))

        def step(i):
            sg.gemm(A, B, C, alpha=alpha, beta=beta, M=M, N=M, K=M, lda=p["lda"], ldb=p["ldb"],
                    ldc=p["ldc"], dtype=0)
        ms = time_steps(step, steps, warmup, torch)
        tf = 2.0 * M ** 3 / (ms * 1e-3) / 1e12
        out.append({"M": M, "N": M, "K": M, "alpha": alpha, "beta": beta, "us": round(ms * 1e3, 2),
                    "tflops": round(tf, 2), "frac_of_fp32_mfma_peak": round(tf / PEAK["f32"], 4),
                    "kernel_config": sg.last_config()})
    return out


def bench_gemm_ragged(torch, sg, inputs, steps, warmup):
    """bf16 GEMMs of the ragged parity shapes (alpha 0.7, beta 0.3, padded ld), every
    transpose pair: TFLOP/s per variant.  With beta = 0.3 each step reads the C the
    previous step wrote (a bounded recurrence); values do not change the time."""
    out = []
    for (M, N, K) in ((1000, 1000, 1000), (4097, 3001, 2049)):
        for tr in ("NN", "NT", "TN", "TT"):
            p = inputs.gemm_problem(3, tr[0], tr[1], M, N, K, "bf16", "normal", ld_mode="padded")
            A, B, C = (to_dev(p["A"], "bf16", torch), to_dev(p["B"], "bf16", torch),
                       to_dev(p["C"], "bf16", torch))

            def step(i):
                sg.gemm(A, B, C, alpha=0.7, beta=0.3, transA=tr[0], transB=tr[1], M=M, N=N, K=K,
                        lda=p["lda"], ldb=p["ldb"], ldc=p["ldc"], dtype=2)
            ms = time_steps(step, steps, warmup, torch)
            tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            out.append({"M": M, "N": N, "K": K, "trans": tr, "ms": round(ms, 5),
                        "tflops": round(tf, 2), "kernel_config": sg.last_config()})
    return out


def bench_epilogue(torch, sg, steps, warmup):
    """Fused GEMM epilogue (sg_gemm_ex) on a 2048 x 896 x 4864 bf16 projection (the
    MLP shape of the SwiGLU rows, here as a plain Linear): the GEMM alone, with bias
    + GELU fused (bf16 out), with bias + GELU + e4m3 output quantisation fused, and
    the unfused sequences: this library's GEMM followed by torch's bias add, GELU
    (and float8 cast) as separate kernels."""
    M, N, K = 2048, 4864, 896
    A = torch.randn((M, K), device="cuda:0").to(torch.bfloat16)
    W = (torch.randn((K, N), device="cuda:0") * 0.03).to(torch.bfloat16)
    bias = torch.randn((N,), device="cuda:0").to(torch.bfloat16)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    C8 = torch.empty((M, N), dtype=torch.uint8, device="cuda:0")
    s8 = 0.05
    F = torch.nn.functional

    def plain(i):
        sg.gemm(A, W, C)

    def fused(i):
        sg.gemm_ex(A, W, C, bias=bias, activation="gelu")

    def fused8(i):
        sg.gemm_ex(A, W, C8, bias=bias, activation="gelu", out_scale=s8)

    def unfused(i):
        sg.gemm(A, W, C)
        F.gelu(C + bias)

    def unfused8(i):
        sg.gemm(A, W, C)
        (F.gelu(C + bias) / s8).to(torch.float8_e4m3fn)

    out = {"shape": "bf16 M=%d K=%d N=%d, bias + GELU" % (M, K, N)}
    for name, fn in (("gemm_ms", plain), ("fused_bias_gelu_ms", fused),
                     ("fused_bias_gelu_e4m3_out_ms", fused8), ("unfused_bias_gelu_ms", unfused),
                     ("unfused_bias_gelu_e4m3_out_ms", unfused8)):
        out[name] = round(time_steps(fn, steps, warmup, torch), 5)
        if name.startswith("fused"):
            out[name.replace("_ms", "_config")] = sg.last_config()
    out["fused_vs_unfused"] = round(out["unfused_bias_gelu_ms"] / out["fused_bias_gelu_ms"], 3)
    out["fused_vs_unfused_e4m3_out"] = round(out["unfused_bias_gelu_e4m3_out_ms"] /
                                             out["fused_bias_gelu_e4m3_out_ms"], 3)
    return out


def env_info(torch):
    props = torch.cuda.get_device_properties(0)
    info = {"device": props.name, "compute_units": props.multi_processor_count,
            "torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
            "cpu_model": cpu_model(), "host_threads": os.cpu_count()}
    for key in ("gcnArchName", "clock_rate"):
        if hasattr(props, key):
            info[key] = getattr(props, key)
    try:
        import subprocess
        r = subprocess.run(["hipcc", "--version"], capture_output=True, text=True, timeout=20)
        info["hipcc"] = " ".join(r.stdout.split()[:6])
    except Exception:
        pass
    return info


def sclk_mhz():
    """The GPU's current shader clock in MHz (rocm-smi), or None."""
    import re
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True,
                           timeout=20)
    except Exception:
        return None
    for line in r.stdout.splitlines():
        if "sclk" in line.lower():
            m = re.search(r"(\d+)\s*Mhz", line, re.I)
            if m:
                return int(m.group(1))
    return None


def sclk_under_load(fn, torch, launches=1500):
    """Shader clock sampled while `launches` queued steps keep the GPU busy (the
    samples are taken after the queue is filled, before it drains)."""
    for i in range(launches):
        fn(i)
    samples = [sclk_mhz() for _ in range(3)]
    torch.cuda.synchronize()
    samples = [x for x in samples if x is not None]
    return samples or None


def read_bandwidth(torch, nbytes=COPY_BYTES, reps=20):
    """Streaming rate of a read-only kernel (the diagnostic library's stream_read:
    16-byte loads, four in flight per thread) over two 512 MiB buffers in turn, so
    the last-level cache holds neither: the practical HBM read ceiling, the yardstick
    of the weight-streaming (skinny) shapes.  Best of three grid sizes; None if the
    diagnostic library is not built."""
    import ctypes
    from swiglu_gemm_amd import build as b
    if not os.path.exists(b.DIAG_LIB):
        return None
    lib = ctypes.CDLL(b.DIAG_LIB)
    lib.sg_diag_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_void_p]
    lib.sg_diag_stream_read.restype = ctypes.c_int
    bufs = [torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0") for _ in range(2)]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = 0.0
    for blocks in (1024, 2048, 4096):
        out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda:0")

        def run(i):
            rc = lib.sg_diag_stream_read(ctypes.c_void_p(bufs[i % 2].data_ptr()), nbytes,
                                         ctypes.c_void_p(out.data_ptr()), blocks, st)
            assert rc == 0, rc
        for i in range(4):
            run(i)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(reps):
            run(i)
        stop.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / reps
        best = max(best, nbytes / (ms * 1e-3) / 1e9)
    del bufs
    torch.cuda.empty_cache()
    return round(best, 1)


def read_same_bytes_ms(torch, nbytes, reps=40):
    """Time of the diagnostic library's plain read kernel over nbytes (rounded down to
    16) with the data cold in HBM (buffers of that size rotated through > 512 MiB, as
    the SwiGLU weights are), an eager loop of launches as in the SwiGLU timing; best of
    four grid sizes.  The floor for a kernel that must stream the same bytes once,
    launch and ramp included.  None if the diagnostic library is not built."""
    import ctypes
    from swiglu_gemm_amd import build as b
    if not os.path.exists(b.DIAG_LIB):
        return None
    lib = ctypes.CDLL(b.DIAG_LIB)
    lib.sg_diag_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_void_p]
    lib.sg_diag_stream_read.restype = ctypes.c_int
    nbytes -= nbytes % 16
    nbuf = max(4, -(-COLD_BYTES // nbytes))
    bufs = [torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0") for _ in range(nbuf)]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    best = None
    for blocks in (256, 512, 1024, 2048):
        out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda:0")

        def run(i):
            rc = lib.sg_diag_stream_read(ctypes.c_void_p(bufs[i % nbuf].data_ptr()), nbytes,
                                         ctypes.c_void_p(out.data_ptr()), blocks, st)
            assert rc == 0, rc
        for i in range(2 * nbuf):
            run(i)
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(reps):
            run(i)
        stop.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop) / reps
        best = ms if best is None else min(best, ms)
    del bufs
    torch.cuda.empty_cache()
    return round(best, 5)


def copy_bandwidth(torch, nbytes=COPY_BYTES, reps=20):
    """Streaming rate of a plain device-to-device copy (read + write bytes per
    second) over two buffer pairs, 2 GiB in all, so the last-level cache holds
    neither: the practical HBM ceiling on this board."""
    bufs = [torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0") for _ in range(4)]
    for b in bufs:
        b.fill_(1.0)
    for i in range(4):
        bufs[2 * (i % 2) + 1].copy_(bufs[2 * (i % 2)])
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(reps):
        bufs[2 * (i % 2) + 1].copy_(bufs[2 * (i % 2)])
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / reps
    del bufs
    torch.cuda.empty_cache()
    return round(2.0 * nbytes / (ms * 1e-3) / 1e9, 1)


def gemm_inputs(inputs, torch, M, N, K, nsets):
    host = inputs.gemm_problem(2, "N", "N", M, N, K, "f16", "normal", scale=1.0 / np.sqrt(K),
                               beta_zero=True)
    sets = []
    for r in range(nsets):
        if r == 0:
            A, B = to_dev(host["A"], "f16", torch), to_dev(host["B"], "f16", torch)
        else:   # further sets: same distribution, other seeds
            p2 = inputs.gemm_problem(200 + r, "N", "N", M, N, K, "f16", "normal",
                                     scale=1.0 / np.sqrt(K), beta_zero=True)
            A, B = to_dev(p2["A"], "f16", torch), to_dev(p2["B"], "f16", torch)
        C = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
        sets.append((A, B, C))
    return host, sets


def pmc_probe():
    """Run under rocprofv3 --pmc: one device copy of COPY_BYTES (the calibration
    kernel), then three launches of the headline GEMM."""
    import torch
    import swiglu_gemm_amd as sg
    from swiglu_gemm_amd import inputs
    sg.lib()
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    _, sets = gemm_inputs(inputs, torch, 8192, 8192, 8192, 1)
    A, B, C = sets[0]
    for _ in range(3):
        sg.gemm(A, B, C)
    torch.cuda.synchronize()
    for _ in range(3):                 # hipBLASLt on the same tensors: the yardstick
        torch.mm(A, B, out=C)
    torch.cuda.synchronize()
    print("pmc probe done: %s" % sg.last_config(), flush=True)


def pmc_probe_nt():
    """Run under rocprofv3 --pmc: the bf16 8192 x 4096 x 4096 GEMM with B stored N x K
    (both operands k-contiguous), three launches of hipBLASLt (torch.mm) before and
    after three of this library, on the same seeded tensors."""
    import torch
    import swiglu_gemm_amd as sg
    from swiglu_gemm_amd import inputs
    sg.lib()
    gen = torch.Generator(device="cpu").manual_seed(7)
    A = torch.randn(8192, 4096, generator=gen).bfloat16().to("cuda:0")
    B = torch.randn(4096, 4096, generator=gen).bfloat16().to("cuda:0")   # N x K
    C = torch.empty(8192, 4096, dtype=torch.bfloat16, device="cuda:0")
    for _ in range(3):
        torch.mm(A, B.t())
    torch.cuda.synchronize()
    for _ in range(3):
        sg.gemm(A, B, C, transB="T")
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mm(A, B.t())
    torch.cuda.synchronize()
    print("pmc probe nt done: %s" % sg.last_config(), flush=True)


def pmc_summarize(fetch_csv, write_csv):
    """Turn the two counter runs into HBM bytes per GEMM launch (calibrated by the
    copy kernel) and write TRAFFIC_FILE."""
    def per_dispatch(path, counter):
        rows = list(csv.DictReader(open(path)))
        agg = {}
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            key = int(r["Dispatch_Id"])
            name = r["Kernel_Name"]
            agg.setdefault(key, [name, 0.0])
            agg[key][1] += float(r["Counter_Value"])
        return [agg[k] for k in sorted(agg)]

    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        d = per_dispatch(path, counter)
        copy = [v for n, v in d if "copy" in n.lower() or "elementwise" in n.lower()]
        gemm = [v for n, v in d if "gemm" in n and "dma" in n]
        if not copy or not gemm:
            raise SystemExit("counter file %s lacks the copy or GEMM dispatches" % path)
        copy_kib = max(copy)                     # the 512 MiB copy dominates
        factor = COPY_BYTES / (copy_kib * 1024.0)
        blas = [v for n, v in d if n.startswith("Cijk") or "gemm" in n.lower() and "dma" not in n]
        out[counter] = {"gemm_kib_per_launch": sum(gemm) / len(gemm),
                        "copy_kib": copy_kib, "scale_factor": factor,
                        "gemm_bytes_per_launch": sum(gemm) / len(gemm) * 1024.0 * factor}
        if blas:
            out[counter]["hipblaslt_bytes_per_launch"] = sum(blas) / len(blas) * 1024.0 * factor
    total = out["FETCH_SIZE"]["gemm_bytes_per_launch"] + out["WRITE_SIZE"]["gemm_bytes_per_launch"]
    res = {"kernel_src_sha": kernel_source_hash(), "workload": "fp16 GEMM NN 8192^3",
           "algorithmic_bytes_per_launch": 3 * 8192 * 8192 * 2,
           "hbm_bytes_per_launch": total, "counters": out}
    if all("hipblaslt_bytes_per_launch" in out[c] for c in out):
        res["hipblaslt_hbm_bytes_per_launch"] = sum(out[c]["hipblaslt_bytes_per_launch"]
                                                    for c in out)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


SWIGLU_COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_swiglu_kernels.md")
# (label, dtype, M, N, K) of the SwiGLU workloads the counter probe runs
SWIGLU_PROBES = [("e4m3 SwiGLU M=1", "e4m3", 1, 11008, 4096),
                 ("e4m3 SwiGLU M=16", "e4m3", 16, 11008, 4096),
                 ("e4m3 SwiGLU M=256", "e4m3", 256, 11008, 4096),
                 ("bf16 SwiGLU M=128", "bf16", 128, 4864, 896),
                 ("bf16 SwiGLU M=512", "bf16", 512, 4864, 896),
                 ("bf16 SwiGLU M=2048", "bf16", 2048, 4864, 896)]


def pmc_probe_swiglu():
    """Run under rocprofv3 --pmc: the calibration copy of pmc_probe, then each SwiGLU
    workload of SWIGLU_PROBES three times, every launch on a fresh copy of W_fused
    (weights in HBM, as in the cold timing), torch's sleep kernel between workloads."""
    import torch
    import swiglu_gemm_amd as sg
    from swiglu_gemm_amd import inputs
    sg.lib()
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1.0)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    for label, dt, M, N, K in SWIGLU_PROBES:
        pb = inputs.swiglu_problem(4 if dt == "bf16" else 5, M, N, K, dt)
        A = to_dev(pb["A"], dt, torch)
        W0 = sg.interleave_gate_up(to_dev(pb["W1"], dt, torch), to_dev(pb["W2"], dt, torch))
        Ws = [W0.clone() for _ in range(3)]
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
        flush = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
        for W in Ws:
            flush.fill_(0.0)                     # evicts W from the last-level cache
            torch.cuda.synchronize()
            sg.swiglu_gemm(A, W, Y, pb["scale_a"], pb["scale_w"])
            torch.cuda.synchronize()
        torch.cuda._sleep(2000000)
        torch.cuda.synchronize()
        del Ws, W0, flush


def pmc_swiglu_summarize(fetch_csv, write_csv, sq_csv):
    """Per-launch HBM bytes (FETCH_SIZE / WRITE_SIZE, calibrated by the copy as in
    pmc_summarize) and SQ counters of the SwiGLU kernels of a --pmc-probe-swiglu run
    set; writes SWIGLU_COUNTERS_FILE."""
    def dispatches(path):
        rows = list(csv.DictReader(open(path)))
        agg = {}
        for r in rows:
            key = int(r["Dispatch_Id"])
            d = agg.setdefault(key, {"name": r["Kernel_Name"], "t0": int(r["Start_Timestamp"]),
                                     "t1": int(r["End_Timestamp"]),
                                     "grid": int(r["Grid_Size"]) // max(int(r["Workgroup_Size"]), 1)})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        return [agg[k] for k in sorted(agg)]

    def swiglu_launches(ds):
        # the SwiGLU kernels in launch order, three per workload
        ks = [d for d in ds if "sg::gemm_dma_kernel" in d["name"] or "sg::decode" in d["name"]]
        if len(ks) != 3 * len(SWIGLU_PROBES):
            raise SystemExit("expected %d SwiGLU launches, found %d" % (3 * len(SWIGLU_PROBES),
                                                                       len(ks)))
        return [ks[3 * i:3 * i + 3] for i in range(len(SWIGLU_PROBES))]

    fd, wd, sd = dispatches(fetch_csv), dispatches(write_csv), dispatches(sq_csv)
    scale = {}
    for counter, ds in (("FETCH_SIZE", fd), ("WRITE_SIZE", wd)):
        copy = [d[counter] for d in ds if "copybuffer" in d["name"].lower()]
        scale[counter] = COPY_BYTES / (max(copy) * 1024.0)
    lines = ["# Counters of the fused SwiGLU kernels (HBM bytes, MFMA busy, LDS), one MI355X", "",
             "Commands (repository root on the MI355X machine, after `cd /tmp && export TMPDIR=/tmp`),",
             "one counter set per run:", "", "```",
             "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/f -o f -- "
             "python <repo>/bench.py --pmc-probe-swiglu",
             "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/w -o w -- "
             "python <repo>/bench.py --pmc-probe-swiglu",
             "rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES "
             "SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT --output-format csv -d <out>/s -o s -- "
             "python <repo>/bench.py --pmc-probe-swiglu",
             "python bench.py --pmc-swiglu-summarize <out>/f/f_counter_collection.csv "
             "<out>/w/w_counter_collection.csv <out>/s/s_counter_collection.csv", "```", "",
             "Each launch reads a fresh copy of W_fused after a 512 MiB fill (weights in HBM). HBM "
             "bytes = counter KiB x the factor that maps the counter of a 512 MiB device copy in the "
             "same run onto its bytes (FETCH_SIZE x%.2f, WRITE_SIZE x%.2f). Algorithmic bytes = A + "
             "W_fused + Y. MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 256 CUs "
             "x 4 SIMDs). Means of the three launches."
             % (scale["FETCH_SIZE"], scale["WRITE_SIZE"]), "",
             "Durations under counter collection are longer than in normal runs (the unprofiled "
             "kernel times are in the bench line and bench_default_kernel_stats.md), so rates are "
             "not derived from them; the clock is not given for these short launches (the "
             "GRBM-based estimate is not meaningful below ~100 us); MFMA busy shares that "
             "denominator and so understates them. Where the launch adds L2 warm-up work-groups "
             "(one per idle CU; bf16 M=128 and 512), the HBM bytes include their loads and the "
             "per-work-group LDS figure counts them among the work-groups.", "",
             "| workload | kernel | HBM read MB | HBM write MB | algorithmic MB | read / algorithmic | "
             "MFMA busy | LDS bank-conflict cycles per work-group |",
             "|---|---|---|---|---|---|---|---|"]
    for (label, dt, M, N, K), f3, w3, s3 in zip(SWIGLU_PROBES, swiglu_launches(fd),
                                               swiglu_launches(wd), swiglu_launches(sd)):
        esz = 1 if dt == "e4m3" else 2
        alg = (M * K + K * 2 * N) * esz + M * N * 2
        rd = sum(d["FETCH_SIZE"] for d in f3) / 3 * 1024 * scale["FETCH_SIZE"]
        wr = sum(d["WRITE_SIZE"] for d in w3) / 3 * 1024 * scale["WRITE_SIZE"]
        grbm = sum(d["GRBM_GUI_ACTIVE"] for d in s3) / 3
        busy = sum(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in s3) / 3 / (grbm / 8 * 256 * 4)
        conf = sum(d["SQ_LDS_BANK_CONFLICT"] for d in s3) / 3
        name = f3[0]["name"].split("(")[0].replace("void ", "").replace("sg::", "")
        wgs = int(s3[0].get("grid", 0)) or None
        lines.append("| %s | `%s` | %.1f | %.2f | %.1f | %.3f | %.3f | %s |" % (
            label, name, rd / 1e6, wr / 1e6, alg / 1e6, rd / alg, busy,
            "%.0f" % (conf / wgs) if wgs else "%.0f (total)" % conf))
    with open(SWIGLU_COUNTERS_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


SWEEP_CFGS = (10, 8, 34, 35, 9, 27, 5, 41, 3, 40, 13, 36, 37, 30, 38, 39, 6, 31)


def stage_sweep(steps):
    """Pipeline-depth / tile study on the headline fp16 8192^3 NN GEMM: every listed
    configuration forced in turn (SG_FORCE_CONFIG), three rotated input sets, HIP
    events; then torch.mm (hipBLASLt) on the same inputs in fp16 and bf16.  One
    JSON line per case.  Run under rocprofv3 --kernel-trace so the per-kernel
    register and LDS use can be joined in (--stage-sweep-summarize)."""
    import torch
    import swiglu_gemm_amd as sg
    from swiglu_gemm_amd import inputs
    sg.lib()
    M = N = K = 8192
    _, sets = gemm_inputs(inputs, torch, M, N, K, 3)
    flops = 2.0 * M * N * K
    for cfg in SWEEP_CFGS:
        os.environ["SG_FORCE_CONFIG"] = "%d,1" % cfg

        def step(i):
            A, B, C = sets[i % 3]
            sg.gemm(A, B, C)
        try:
            ms = time_steps(step, steps, 3, torch)
        finally:
            os.environ.pop("SG_FORCE_CONFIG", None)
        print(json.dumps({"stage_sweep": cfg, "kernel_config": sg.last_config(), "ms": round(ms, 5),
                          "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}), flush=True)
    for dt in (torch.float16, torch.bfloat16):
        mats = [(A.to(dt), B.to(dt)) for A, B, _ in sets]

        def lib_step(i):
            A, B = mats[i % 3]
            torch.mm(A, B)
        ms = time_steps(lib_step, steps, 3, torch)
        print(json.dumps({"stage_sweep": "torch.mm (hipBLASLt)", "dtype": str(dt).split(".")[-1],
                          "ms": round(ms, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}),
              flush=True)
        del mats


STAGE_SWEEP_FILE = os.path.join(ROOT, "profiles", "stage_sweep_gemm16_f16_nn_8192.md")


def stage_sweep_summarize(trace_csv, sweep_jsonl):
    """Join the stage sweep's timings with the per-kernel VGPR / LDS use of the same
    run (rocprofv3 --kernel-trace), compute occupancy, and fit the pipeline model
    of the Ada Lovelace page (throughput proportional to S/(S+kappa)) alone and with
    an occupancy factor W/(W+omega) (W = resident waves per SIMD), one tile
    efficiency A per tile family.  Writes STAGE_SWEEP_FILE."""
    import re
    from scipy.optimize import least_squares
    res = {}
    for r in csv.DictReader(open(trace_csv)):
        m = re.search(r"gemm_(dma|pp)_kernel<1, false, false, 0, (\d+), (\d+), (\d+), (\d+), (\d+), "
                      r"(\d+)>", r["Kernel_Name"])
        if not m:
            continue
        key = (m.group(1),) + tuple(int(x) for x in m.group(2, 3, 4, 5, 6, 7))
        res[key] = (int(r["VGPR_Count"]) + int(r["Accum_VGPR_Count"]), int(r["LDS_Block_Size"]))
    pts, lib = [], []
    for line in open(sweep_jsonl):
        if not line.startswith("{"):
            continue
        d = json.loads(line)
        if not isinstance(d["stage_sweep"], int):
            lib.append(d)
            continue
        m = re.search(r"(dma|pp) (\d+)x(\d+)x(\d+) s(\d+) (\d+)x(\d+)w", d["kernel_config"])
        kind, BM, BN, BK, S, WM, WN = (m.group(1),) + tuple(int(x) for x in m.group(2, 3, 4, 5, 6, 7))
        vgpr, lds = res[(kind, BM, BN, BK, S, WM, WN)]
        waves = WM * WN
        per_simd = -(-waves // 4)
        alloc = -(-max(vgpr, 1) // 8) * 8
        by_lds = (160 * 1024) // lds
        by_regs = (512 // alloc) // per_simd
        ctas = max(1, min(by_lds, by_regs, 8 // per_simd))
        pts.append(dict(cfg=d["stage_sweep"], kind=kind, BM=BM, BN=BN, BK=BK, S=S, waves=waves,
                        vgpr=vgpr, lds=lds, ctas=ctas, W=ctas * per_simd, tf=d["tflops"],
                        fam="%s %dx%dx%d %dw" % (kind, BM, BN, BK, waves)))
    fams = sorted(set(p_["fam"] for p_ in pts))
    S = np.array([p_["S"] for p_ in pts], float)
    W = np.array([p_["W"] for p_ in pts], float)
    T = np.array([p_["tf"] for p_ in pts], float)
    F = np.array([fams.index(p_["fam"]) for p_ in pts])

    def model(x, occ):
        A = x[:len(fams)][F]
        kap = x[len(fams)]
        om = x[len(fams) + 1] if occ else 0.0
        return A * S / (S + kap) * (W / (W + om) if occ else 1.0)

    fits = {}
    for occ in (False, True):
        x0 = [1300.0] * len(fams) + [0.5] + ([0.5] if occ else [])
        lb = [0.0] * len(fams) + [0.0] + ([0.0] if occ else [])
        r = least_squares(lambda x: (model(x, occ) - T) / T, x0, bounds=(lb, np.inf))
        fits[occ] = r.x
    lines = ["# Pipeline depth and tile study: fp16 8192^3 NN GEMM on one MI355X", "",
             "Commands (repository root on the MI355X machine, after `cd /tmp && export TMPDIR=/tmp`):", "",
             "```", "rocprofv3 --kernel-trace --output-format csv -d <out> -o sw -- "
             "python <repo>/bench.py --stage-sweep > sweep.jsonl",
             "python bench.py --stage-sweep-summarize <out>/sw_kernel_trace.csv sweep.jsonl", "```", "",
             "Every configuration forced in turn, three rotated input sets, HIP events; VGPR "
             "(arch + accumulation) and LDS per work-group from the kernel trace of the same run. "
             "Work-groups per CU = min(160 KiB / LDS, 512 registers / VGPRs per wave / waves per "
             "SIMD, 8 wave slots); W = resident waves per SIMD.", "",
             "Model of the Ada Lovelace page: throughput = A * S/(S + kappa) (pipeline efficiency; "
             "one A per tile family); extended with occupancy: * W/(W + omega). Fitted "
             "(relative least squares) over all rows:", "",
             "* S/(S+kappa): kappa = %.3f" % fits[False][len(fams)],
             "* S/(S+kappa) * W/(W+omega): kappa = %.3f, omega = %.3f" % (fits[True][len(fams)],
                                                                          fits[True][len(fams) + 1]),
             "", "| family | S | LDS KiB | VGPR | WG/CU | W | TFLOP/s | S/(S+k) model | with occupancy |",
             "|---|---|---|---|---|---|---|---|---|"]
    m0, m1 = model(fits[False], False), model(fits[True], True)
    for i, p_ in enumerate(pts):
        lines.append("| %s | %d | %d | %d | %d | %d | %.1f | %.1f (%+.1f%%) | %.1f (%+.1f%%) |" % (
            p_["fam"], p_["S"], p_["lds"] // 1024, p_["vgpr"], p_["ctas"], p_["W"], p_["tf"],
            m0[i], 100 * (m0[i] / p_["tf"] - 1), m1[i], 100 * (m1[i] / p_["tf"] - 1)))
    err0 = np.abs(m0 / T - 1).mean() * 100
    err1 = np.abs(m1 / T - 1).mean() * 100
    lines += ["", "Mean absolute model error: %.1f %% (pipeline term only), %.1f %% (with occupancy)."
              % (err0, err1), ""]
    for d in lib:
        lines.append("hipBLASLt (torch.mm, same inputs, same run), %s: %.1f TFLOP/s." %
                     (d["dtype"], d["tflops"]))
    with open(STAGE_SWEEP_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


DECODE_FILE = os.path.join(ROOT, "profiles", "decode_gemv_cold.md")
# decode-shaped problems: (label, kind, dtype, M, N, K, weight layout)
DECODE_CASES = [("bf16 GEMM 1x4096x4096 NT", "gemm", "bf16", 1, 4096, 4096, "T"),
                ("bf16 GEMM 16x4096x4096 NT", "gemm", "bf16", 16, 4096, 4096, "T"),
                ("bf16 GEMM 8x14336x4096 NT", "gemm", "bf16", 8, 14336, 4096, "T"),
                ("bf16 GEMM 16x8192x8192 NN", "gemm", "bf16", 16, 8192, 8192, "N"),
                ("bf16 GEMM 32x14336x4096 NN", "gemm", "bf16", 32, 14336, 4096, "N"),
                ("bf16 SwiGLU 16x896x2*4864", "swiglu", "bf16", 16, 4864, 896, "N"),
                ("e4m3 SwiGLU 1x4096x2*11008", "swiglu", "e4m3", 1, 11008, 4096, "N"),
                ("e4m3 SwiGLU 16x4096x2*11008", "swiglu", "e4m3", 16, 11008, 4096, "N")]
DECODE_PATHS = [("default", {}), ("large-tile", {"SG_FORCE_CONFIG": "-1"}),
                ("decode", {"SG_FORCE_DECODE": "5"})]


def decode_study(steps):
    """Decode-shaped problems (1..32 rows) with the weights cold in HBM: the
    library's default choice, the large-tile path and the stream-K decode path
    forced in turn, and torch.mm (hipBLASLt) for the GEMMs.  Each (case, path) is
    fenced in the kernel trace by torch's sleep kernel; one JSON line each with the
    wall time per call (HIP events; includes launch gaps).  Run under rocprofv3
    --kernel-trace and pass the trace to --decode-summarize for kernel times."""
    import torch
    import swiglu_gemm_amd as sg
    from swiglu_gemm_amd import inputs
    sg.lib()
    dev = "cuda:0"

    def timed(fn):
        for i in range(5):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / steps * 1e3
        torch.cuda._sleep(2000000)          # marks the end of this case in the trace
        torch.cuda.synchronize()
        return us

    for label, kind, dt, M, N, K, tb in DECODE_CASES:
        esz = 1 if dt == "e4m3" else 2
        wbytes = K * N * esz * (2 if kind == "swiglu" else 1)
        ncold = max(4, -(-COLD_BYTES // wbytes))
        if kind == "swiglu":
            pb = inputs.swiglu_problem(4 if dt == "bf16" else 5, M, N, K, dt)
            A = to_dev(pb["A"], dt, torch)
            W0 = sg.interleave_gate_up(to_dev(pb["W1"], dt, torch), to_dev(pb["W2"], dt, torch))
            Ws = [W0] + [W0.clone() for _ in range(ncold - 1)]
            Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            sa, sw = pb["scale_a"], pb["scale_w"]

            def fn(i):
                sg.swiglu_gemm(A, Ws[i % ncold], Y, sa, sw)
            out_bytes = M * N * 2
        else:
            A = torch.randn((M, K), device=dev).to(torch.bfloat16)
            W0 = (torch.randn((N, K) if tb == "T" else (K, N), device=dev) * 0.02).to(torch.bfloat16)
            Ws = [W0] + [W0.clone() for _ in range(ncold - 1)]
            C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

            def fn(i):
                sg.gemm(A, Ws[i % ncold], C, transB=tb)
            out_bytes = M * N * 2
        nbytes = wbytes + M * K * esz + out_bytes
        for path, env in DECODE_PATHS:
            os.environ.update(env)
            try:
                us = timed(fn)
                desc = sg.last_config()
            finally:
                for k in env:
                    os.environ.pop(k, None)
            print(json.dumps({"decode_case": label, "path": path, "wall_us": round(us, 2),
                              "bytes": nbytes, "kernel_config": desc}), flush=True)
        if kind == "gemm":
            def lib_fn(i):
                W = Ws[i % ncold]
                torch.mm(A, W.t() if tb == "T" else W)
            us = timed(lib_fn)
            print(json.dumps({"decode_case": label, "path": "torch.mm (hipBLASLt)",
                              "wall_us": round(us, 2), "bytes": nbytes, "kernel_config": "-"}),
                  flush=True)
        del Ws, W0


def decode_summarize(trace_csv, jsonl):
    """Kernel durations per (case, path) of a --decode run: the trace is cut at
    torch's sleep kernels; the first 5 launches of each segment are warm-up.
    Writes DECODE_FILE."""
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    segs, cur = [], []
    for r in rows:
        name = r["Kernel_Name"]
        if "sleep" in name.lower() or "spin" in name.lower():
            if cur:
                segs.append(cur)
            cur = []
            continue
        cur.append(r)
    # kernels of the problem itself: the library's, or hipBLASLt's for torch.mm
    # (the one-time W_fused interleave before a SwiGLU case's first path is set-up)
    def ours(name):
        return ("sg::" in name and "interleave" not in name) or "Cijk" in name or \
            "gemv" in name.lower()
    segs = [[r for r in sg_ if ours(r["Kernel_Name"])] for sg_ in segs]
    segs = [sg_ for sg_ in segs if sg_]
    cases = [json.loads(l) for l in open(jsonl) if l.startswith('{"decode_case"')]
    assert len(segs) == len(cases), (len(segs), len(cases))
    lines = ["# Decode-shaped GEMM / SwiGLU (1..32 rows), weights cold in HBM, one MI355X", "",
             "Commands (repository root on the MI355X machine, after `cd /tmp && export TMPDIR=/tmp`):", "",
             "```", "rocprofv3 --kernel-trace --output-format csv -d <out> -o dec -- "
             "python <repo>/bench.py --decode > decode.jsonl",
             "python bench.py --decode-summarize <out>/dec_kernel_trace.csv decode.jsonl", "```", "",
             "Weights rotate through > 512 MB of device copies so each call reads them from HBM. "
             "Kernel time = mean duration per call of every kernel the call launches (the "
             "stream-K kernel plus its fix-up kernel, or the large-tile kernel plus its split-K "
             "reduction); GB/s = weight + token + output bytes / kernel time. Wall = HIP events "
             "around back-to-back calls from Python without a clock spin-up: at these sizes it "
             "is bound by the host-side cost of a call (about 30 us here), not by the GPU, so "
             "such calls belong in a captured graph or a native caller.", "",
             "| problem | path | kernels (mean us each) | kernel us | GB/s | wall us | configuration |",
             "|---|---|---|---|---|---|---|"]
    for c, seg in zip(cases, segs):
        by = {}
        for r in seg:
            by.setdefault(r["Kernel_Name"], []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        parts, tot = [], 0.0
        for k, v in by.items():
            v = v[5:] if len(v) > 5 else v
            mean = sum(v) / len(v)
            tot += mean
            short = k.split("(")[0].replace("void ", "")
            if short.startswith("Cijk"):
                short = "hipBLASLt " + short.split("_MT")[1].split("_")[0] if "_MT" in short else short[:30]
            parts.append("%s %.1f" % (short.replace("sg::", ""), mean))
        lines.append("| %s | %s | %s | %.1f | %.0f | %.1f | %s |" % (
            c["decode_case"], c["path"], "; ".join(parts), tot, c["bytes"] / (tot * 1e-6) / 1e9,
            c["wall_us"], c["kernel_config"]))
    with open(DECODE_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def mfma_ceiling():
    """Sustained rate of a pure MFMA loop (no memory traffic) on zero, constant and
    random operand data, per dtype.  The matrix cores' power grows with the
    operands' bit activity; under the board power limit the clock drops, so random
    data sets a lower ceiling than the published peak.  One JSON line per case."""
    import ctypes
    import torch
    from swiglu_gemm_amd import build
    if not os.path.exists(build.DIAG_LIB):
        raise SystemExit("diagnostic library missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(build.DIAG_LIB)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    blocks, iters = 1024, 20000
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    nsrc = 8192                                     # 16-byte operand chunks
    gen = torch.Generator(device="cuda:0").manual_seed(7)
    for kind, dt, shape in ((0, "f16", "32x32x16"), (1, "bf16", "32x32x16"), (2, "e4m3", "32x32x64"),
                            (3, "f16", "16x16x32"), (4, "bf16", "16x16x32")):
        tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn}[dt]
        per = 16 // torch.empty(0, dtype=tdt).element_size()
        datas = {
            "zero": torch.zeros(nsrc * per, device="cuda:0"),
            "constant_1.0": torch.ones(nsrc * per, device="cuda:0"),
            "random_normal": torch.randn(nsrc * per, device="cuda:0", generator=gen) *
            (1.0 if dt == "e4m3" else 1.0 / 90.5),
        }
        for name, v in datas.items():
            src = v.to(tdt).contiguous()
            f = lambda: lib.sg_diag_mfma_loop(kind, blocks, ctypes.c_void_p(src.data_ptr()), nsrc,
                                              iters, ctypes.c_void_p(out.data_ptr()), st)
            assert f() == 0
            torch.cuda.synchronize()
            t_end = time.perf_counter() + 0.3
            while time.perf_counter() < t_end:
                f()
                torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(5):
                f()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 5
            flops = blocks * 4 * iters * 8 * 2 * 32 * 32 * (64 if kind == 2 else 16)
            tf = flops / (ms * 1e-3) / 1e12
            print(json.dumps({"mfma_ceiling": dt, "mfma": shape, "operands": name, "ms": round(ms, 4),
                              "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK[dt], 4)}),
                  flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="headline GEMM and SwiGLU M=2048 only")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--pmc-probe", action="store_true")
    ap.add_argument("--pmc-summarize", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--pmc-probe-swiglu", action="store_true")
    ap.add_argument("--pmc-probe-nt", action="store_true",
                    help="bf16 GEMM with B stored N x K: this library beside hipBLASLt")
    ap.add_argument("--pmc-swiglu-summarize", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "SQ_CSV"))
    ap.add_argument("--mfma-ceiling", action="store_true")
    ap.add_argument("--stage-sweep", action="store_true")
    ap.add_argument("--stage-sweep-summarize", nargs=2, metavar=("TRACE_CSV", "SWEEP_JSONL"))
    ap.add_argument("--decode", action="store_true",
                    help="decode-shaped problems: default vs large-tile vs decode path")
    ap.add_argument("--decode-summarize", nargs=2, metavar=("TRACE_CSV", "DECODE_JSONL"))
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only (the library is single-GPU); --gpus %d is not "
              "supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.pmc_summarize:
        pmc_summarize(*args.pmc_summarize)
        return
    if args.stage_sweep_summarize:
        stage_sweep_summarize(*args.stage_sweep_summarize)
        return
    if args.decode_summarize:
        decode_summarize(*args.decode_summarize)
        return
    if args.decode:
        decode_study(40)
        return
    if args.pmc_probe:
        pmc_probe()
        return
    if args.pmc_probe_swiglu:
        pmc_probe_swiglu()
        return
    if args.pmc_probe_nt:
        pmc_probe_nt()
        return
    if args.pmc_swiglu_summarize:
        pmc_swiglu_summarize(*args.pmc_swiglu_summarize)
        return
    if args.mfma_ceiling:
        mfma_ceiling()
        return
    if args.stage_sweep:
        stage_sweep(max(10, args.steps // 2))
        return

    import torch
    import swiglu_gemm_amd as sg
    from swiglu_gemm_amd import inputs
    sg.lib()                      # raises if the HIP library is not built
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    M = N = K = 8192
    print("bench: generating inputs", file=sys.stderr, flush=True)
    host, sets = gemm_inputs(inputs, torch, M, N, K, 3)

    def step(i):
        A, B, C = sets[i % 3]
        sg.gemm(A, B, C, alpha=1.0, beta=0.0)

    print("bench: timing fp16 8192^3 GEMM", file=sys.stderr, flush=True)
    sclk_before = sclk_mhz()
    ms = time_steps(step, args.steps, args.warmup, torch)
    sclk_after = sclk_mhz()
    cfg = sg.last_config()
    stats = step_stats(step, args.steps, torch)
    sclk_load = sclk_under_load(step, torch)
    flops = 2.0 * M * N * K
    tflops = flops / (ms * 1e-3) / 1e12
    traffic = measured_traffic()
    step(0)                                  # set 0 holds the seeded problem of the oracle
    torch.cuda.synchronize()
    c_gpu = sets[0][2].view(torch.int16).cpu().numpy().view(np.uint16)
    del sets
    torch.cuda.empty_cache()
    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "fp16 GEMM NN M=N=K=8192 alpha=1 beta=0, fp32 accumulate, fp16 out; "
                               "A,B ~ N(0,1)/sqrt(K)", "M": M, "N": N, "K": K,
                   "kernel_config": cfg, "input_sets_rotated": 3},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK["f16"],
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK["f16"], 4),
                     "traffic": traffic, "kernel": "gemm_dma_kernel (one launch per step)",
                     "algorithmic_flops_per_launch": flops},
        "step_stats": stats,
        "env": env_info(torch),
    }
    out["env"].update({"sclk_mhz_before": sclk_before, "sclk_mhz_after": sclk_after,
                       "sclk_mhz_under_load": sclk_load})
    print("bench: device copy bandwidth", file=sys.stderr, flush=True)
    out["env"]["copy_gbs"] = copy_bandwidth(torch)
    out["env"]["read_gbs"] = read_bandwidth(torch)
    if not args.quick:
        print("bench: bf16 8192^3 GEMM and the ragged bf16 GEMMs", file=sys.stderr, flush=True)
        out["gemm_bf16_8192"] = bench_gemm_bf16_8192(torch, sg, max(10, args.steps // 2),
                                                     args.warmup)
        torch.cuda.empty_cache()
        out["gemm_ragged_bf16"] = bench_gemm_ragged(torch, sg, inputs, 20, 3)
        torch.cuda.empty_cache()
        print("bench: fused GEMM epilogue", file=sys.stderr, flush=True)
        out["gemm_epilogue"] = bench_epilogue(torch, sg, max(10, args.steps // 2), args.warmup)
        torch.cuda.empty_cache()
        print("bench: fp32 GEMM", file=sys.stderr, flush=True)
        out["gemm_f32"] = bench_gemm_f32(torch, sg, inputs, 20, 3)
        torch.cuda.empty_cache()
    sizes = [("bf16", 2048, 4864, 896)]
    if not args.quick:
        sizes = [("bf16", m, 4864, 896) for m in (128, 512, 2048, 8192)] + \
                [("e4m3", m, 11008, 4096) for m in (1, 16, 256, 4096)]
    sw = []
    kept = {}
    for dt, m, n, k in sizes:
        print("bench: SwiGLU %s M=%d" % (dt, m), file=sys.stderr, flush=True)
        sw.append(bench_swiglu(torch, sg, inputs, dt, m, n, k, max(10, args.steps // 2),
                               args.warmup, keep=kept if (dt, m) == ("bf16", 2048) else None))
        torch.cuda.empty_cache()
    rb = out["env"].get("read_gbs")
    for s in sw:                  # against what this board's HBM delivers to a plain read
        if rb:
            s["frac_of_read_bw"] = round(s["hbm_gbs_algorithmic"] / rb, 4)
        if (s["dtype"], s["M"]) in (("e4m3", 1), ("e4m3", 16), ("bf16", 128)):
            # the weight-streaming rows: a plain read of the same bytes, cold, same timing
            esz = 1 if s["dtype"] == "e4m3" else 2
            nb = (s["M"] * s["K"] + 2 * s["K"] * s["N"]) * esz + s["M"] * s["N"] * 2
            t = read_same_bytes_ms(torch, nb)
            if t:
                s["plain_read_same_bytes_ms"] = t
                s["frac_of_plain_read_same_bytes"] = round(t / s["ms"], 4)
    out["swiglu_m2048"] = [s for s in sw if s["dtype"] == "bf16" and s["M"] == 2048][0]
    if len(sw) > 1:
        out["swiglu_all"] = sw
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"], ref_rows = cpu_baseline(host, M, N, K, args.cpu_budget)
        out["numerics"] = oracle_checks(c_gpu, ref_rows, kept)
    print(json.dumps(out), flush=True)


def oracle_checks(c_gpu, ref_rows, kept, swiglu_rows=256):
    """The error report of the CPU-baseline leg: the headline GEMM's output on the rows
    the oracle just computed, and the bf16 SwiGLU at M = 2048 (fused kernel and the
    unfused two-GEMM path) on its first swiglu_rows rows against the fp64 oracle."""
    import oracle
    R = ref_rows.shape[0]
    out = {"gemm_f16_8192": dict(error_report(f16_bits_to_f64(c_gpu[:R]), ref_rows, 1e-3, 1e-2),
                                 rows="0..%d" % (R - 1))}
    if kept:
        pb = kept["problem"]
        M, K = pb["A"].shape
        N = pb["W1"].shape[1]
        R2 = min(swiglu_rows, M)
        Wf = oracle.interleave(pb["W1"], pb["W2"])
        ref = oracle.swiglu(R2, N, K, pb["A"][:R2], Wf, "bf16")
        out["swiglu_bf16_m2048"] = {
            "rows": "0..%d" % (R2 - 1),
            "fused": error_report(bf16_bits_to_f64(kept["fused"][:R2]), ref, 1e-2, 2e-2),
            "unfused": error_report(bf16_bits_to_f64(kept["unfused"][:R2]), ref, 1e-2, 2e-2)}
    return out


if __name__ == "__main__":
    main()
