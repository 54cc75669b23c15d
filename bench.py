"""Benchmark of the fused SwiGLU gated-MLP product on one MI355X.

One step = one call of the whole hot path (swiglu_fused_packed: the fused
Gate/Up MFMA GEMM with the SiLU * Up epilogue) over one batch of synthetic,
seeded input already resident in HBM.  The weights are packed once before the
timed region, as a model-load step.

Prints ONE JSON line (metric, value, ..., roofline, cpu_baseline).

    python bench.py [--steps K] [--warmup W] [--prewarm SECONDS] [--workload NAME] [--m M]
                    [--variant auto|data_parallel|split_k|sequential] [--dtype bf16|fp8]
                    [--layout per-tile|interleaved] [--no-cpu] [--all [--repeats R] [--mlp]]

The timed region is exactly K steps after W warm-up steps; before those, the
same calls run untimed for --prewarm seconds so the GPU has left its idle
clock (a 75 us step would otherwise be timed partly at the idle clock).

--all also reports every workload point on stderr (POINT lines): the median of
R timed repeats with its min/max, the unfused pipeline's time, and for the
decode-sized points (M <= 64) the per-call time of a graph-captured loop,
which leaves out the host's launch cost; a CONTEXT line first records the
device, its CUs, the HIP version and rocm-smi's clocks and power limit.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 (256 CU x 4096 flop/clk x 2.4 GHz)
MFMA_FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 (published)
HBM_PEAK_GBS = 8000.0               # MI355X HBM3E
MALL_BYTES = 256 << 20
# the largest single-GPU workload point: 72B MLP width, 4096 tokens
DEFAULT_WORKLOAD = "qwen2.5-72B"
DEFAULT_M = 4096


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def flops(M, K, N):
    return 4.0 * M * K * N


def fused_bytes(M, K, N):
    """Algorithmic HBM bytes of the fused product: read A and both weights once,
    write Y once (bf16)."""
    return 2.0 * (M * K + 2 * K * N + M * N)


def unfused_extra_bytes(M, K, N):
    """Extra bytes of the unfused pipeline: write+read Gate and Up, re-read A."""
    return 8.0 * M * N + 2.0 * M * K


def fused_bytes_fp8(M, K, N):
    """Algorithmic HBM bytes of the FP8 product: A and both weights as one
    byte per element, Y as bf16."""
    return 1.0 * (M * K + 2 * K * N) + 2.0 * M * N


def bound_of(M, K, N, dtype="bf16"):
    if dtype == "fp8":
        ai = flops(M, K, N) / fused_bytes_fp8(M, K, N)
        return "mfma" if ai >= MFMA_FP8_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9) else "hbm"
    ai = flops(M, K, N) / fused_bytes(M, K, N)
    return "mfma" if ai >= MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9) else "hbm"


def rotation_count(M, K, N):
    """Rotated input/output sets so consecutive launches never hit in the
    256 MiB last-level cache: twice its size in total."""
    return max(1, math.ceil(2 * MALL_BYTES / fused_bytes(M, K, N)))


def time_gpu(fn_list, steps, warmup, stream, prewarm_s=0.0):
    """Run fn_list[i % R]() for warmup + steps; time the steps with HIP events
    recorded on the launch stream.  Returns total seconds for `steps`.
    Before the warm-up steps the calls run untimed for prewarm_s seconds of
    wall time: a GPU coming out of idle needs tens of milliseconds to reach
    its sustained clock, longer than a few dozen short steps take."""
    import torch
    R = len(fn_list)
    t_end = time.perf_counter() + prewarm_s
    i = 0
    while time.perf_counter() < t_end:
        for _ in range(16):
            fn_list[i % R]()
            i += 1
        torch.cuda.synchronize()
    for i in range(warmup):
        fn_list[i % R]()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        fn_list[i % R]()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / 1e3


def time_gpu_graph(fn_list, calls, replays, stream):
    """Per-call seconds of `calls` calls captured in one HIP graph and replayed
    `replays` times (after one untimed replay), timed with HIP events on the
    stream; what is left of a call's time is its device time plus the gap the
    device leaves between two graph nodes, with no host launch cost."""
    import torch
    R = len(fn_list)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            fn_list[i % R]()
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(replays):
        g.replay()
    stop.record(stream)
    torch.cuda.synchronize()
    del g
    return start.elapsed_time(stop) / 1e3 / (calls * replays)


def run_context():
    """Device facts for the --all report: name, CUs, HIP and torch versions,
    and what rocm-smi says of clocks and power (when it runs)."""
    import subprocess
    import torch
    prop = torch.cuda.get_device_properties(0)
    ctx = {"device": prop.name, "gcn_arch": getattr(prop, "gcnArchName", None),
           "cus": prop.multi_processor_count, "hbm_gib": round(prop.total_memory / 2 ** 30, 1),
           "hip": torch.version.hip, "torch": torch.__version__,
           "host_cpus": len(os.sched_getaffinity(0))}
    try:
        r = subprocess.run(["rocm-smi", "--showmaxpower", "--showclocks", "--showdriverversion", "--json"],
                           capture_output=True, text=True, timeout=30)
        if r.returncode == 0:
            ctx["rocm_smi"] = json.loads(r.stdout)
    except (OSError, ValueError, subprocess.SubprocessError):
        pass
    return ctx


def kernel_source_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in ("swiglu_gated_mlp_amd/csrc/fused_kernels.hpp", "swiglu_gated_mlp_amd/csrc/swiglu_api.hip"):
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload_label):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    runs (profiles/traffic.json, copy-calibrated), or None when they were taken
    on another workload or on kernel sources that have changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload_label or t.get("source_sha256") != kernel_source_sha256():
        return None
    return t.get("traffic_bytes_per_dispatch")


def cpu_model():
    """The host CPU's model name (lscpu's "Model name", else /proc/cpuinfo)."""
    import subprocess
    try:
        r = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10)
        for line in r.stdout.splitlines():
            if line.strip().lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, M, target_s=12.0):
    """Time the CPU oracle (as it stands) on the first rows of the same workload:
    a few rows first to estimate the rate, then enough rows for ~target_s (the
    whole workload, repeated, when it takes less)."""
    import oracle
    from swiglu_gated_mlp_amd import inputs
    threads = min(len(os.sched_getaffinity(0)), 16)
    oracle.set_threads(threads)
    A, W1, W2 = inputs.workload_tensors(w, M)
    Ab, W1b, W2b = inputs.as_bits(A), inputs.as_bits(W1), inputs.as_bits(W2)
    m0 = min(M, max(1, threads))
    t0 = time.perf_counter()
    oracle.swiglu(Ab[:m0], W1b, W2b)
    dt = time.perf_counter() - t0
    m = int(min(M, max(m0, m0 * target_s / max(dt, 1e-6))))
    m = max(threads, (m // threads) * threads) if m >= threads else m
    m = min(m, M)
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.swiglu(Ab[:m], W1b, W2b)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 0.8 * target_s or m < M:
            break
    return {
        "value": round(reps * flops(m, w.K, w.N) / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(oracle.max_threads()),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": "first %d of %d rows of A, all %d columns (K=%d), %d run(s); %.1f s"
                  % (m, M, w.N, w.K, reps, dt),
    }


def bench_point_fp8(w, M, steps, warmup, stream, prewarm_s=0.0):
    """The FP8 path on the workload's own tensors, quantised per tensor (E4M3,
    scale = amax / 448), over rotated input sets."""
    import numpy as np
    import torch
    import swiglu_gated_mlp_amd as sw
    from swiglu_gated_mlp_amd import inputs
    dev = torch.device("cuda:0")
    K, N = w.K, w.N
    A, W1, W2 = inputs.workload_tensors(w, M)
    A8, sa = inputs.quantize_e4m3(A)
    W18, s1 = inputs.quantize_e4m3(W1)
    W28, s2 = inputs.quantize_e4m3(W2)
    sg = float(np.float32(sa) * np.float32(s1))
    su = float(np.float32(sa) * np.float32(s2))
    R = max(1, math.ceil(2 * MALL_BYTES / fused_bytes_fp8(M, K, N)))
    W18d, W28d = W18.to(dev), W28.to(dev)
    sets = [(A8.to(dev), sw.swiglu_pack_weights_fp8(W18d, W28d),
             torch.empty((M, N), dtype=torch.bfloat16, device=dev)) for _ in range(R)]
    del W18d, W28d
    torch.cuda.synchronize()
    fns = [(lambda s=s: sw.swiglu_fused_packed_fp8(s[0], s[1], N, sg, su, Y=s[2])) for s in sets]
    per = time_gpu(fns, steps, warmup, stream, prewarm_s) / steps
    return {"M": M, "K": K, "N": N, "rotation": R, "per_launch_s": per,
            "tflops": flops(M, K, N) / per / 1e12, "gbs": fused_bytes_fp8(M, K, N) / per / 1e9}


def bench_point(w, M, steps, warmup, variant, stream, prewarm_s=0.0, layout="per-tile", repeats=1,
                graph=False):
    import torch
    import swiglu_gated_mlp_amd as sw
    from swiglu_gated_mlp_amd import inputs
    dev = torch.device("cuda:0")
    K, N = w.K, w.N
    A, W1, W2 = inputs.workload_tensors(w, M)
    W1d, W2d = W1.to(dev), W2.to(dev)
    R = rotation_count(M, K, N)
    sets = []
    pack = sw.swiglu_pack_weights_interleaved if layout == "interleaved" else sw.swiglu_pack_weights
    for r in range(R):
        Wp = pack(W1d, W2d)
        Ad = A.to(dev)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = sw.Workspace(dev)
        sets.append((Ad, Wp, Y, ws))
    del W1d, W2d
    torch.cuda.synchronize()
    v = sw.VARIANTS[variant]
    if layout == "interleaved":
        fns = [(lambda s=s: sw.swiglu_fused_packed_interleaved(s[0], s[1], N, Y=s[2])) for s in sets]
    else:
        fns = [(lambda s=s: sw.swiglu_fused_packed(s[0], s[1], N, Y=s[2], workspace=s[3], variant=v))
               for s in sets]
    sec = time_gpu(fns, steps, warmup, stream, prewarm_s)
    per = sec / steps
    out = {
        "M": M, "K": K, "N": N, "rotation": R, "seconds": sec, "per_launch_s": per,
        "tflops": flops(M, K, N) / per / 1e12,
        "gbs": fused_bytes(M, K, N) / per / 1e9,
        "variant": variant, "resolved_variant": sw.swiglu_choose_variant(M, K, N) if v == 0 else v,
    }
    if repeats > 1:
        # further timed repeats of the same steps (no new warm-up needed);
        # the median is reported with the spread
        pers = [per] + [time_gpu(fns, steps, 0, stream) / steps for _ in range(repeats - 1)]
        pers.sort()
        out.update(per_launch_s=pers[len(pers) // 2], per_min_s=pers[0], per_max_s=pers[-1], repeats=repeats)
        per = out["per_launch_s"]
        out["tflops"] = flops(M, K, N) / per / 1e12
        out["gbs"] = fused_bytes(M, K, N) / per / 1e9
    if graph:
        out["graph_per_launch_s"] = time_gpu_graph(fns, max(R, 32), max(3, steps // 32), stream)
    return out


def bench_rowmajor(w, M, steps, warmup, stream, prewarm_s=0.0):
    """The fused product from row-major W1, W2 (swiglu_fused, no pack) and
    the one-time pack of those weights (swiglu_pack_weights), each over
    rotated sets; returns per-call seconds of both."""
    import torch
    import swiglu_gated_mlp_amd as sw
    from swiglu_gated_mlp_amd import inputs
    dev = torch.device("cuda:0")
    K, N = w.K, w.N
    A, W1, W2 = inputs.workload_tensors(w, M)
    R = rotation_count(M, K, N)
    sets = []
    for _ in range(R):
        W1d, W2d = W1.to(dev), W2.to(dev)
        sets.append((A.to(dev), W1d, W2d, torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                     torch.empty(sw.swiglu_packed_bytes(K, N) // 2, dtype=torch.bfloat16, device=dev)))
    torch.cuda.synchronize()
    fused = [(lambda s=s: sw.swiglu_fused(s[0], s[1], s[2], Y=s[3])) for s in sets]
    pack = [(lambda s=s: sw.swiglu_pack_weights(s[1], s[2], Wp=s[4])) for s in sets]
    tr = time_gpu(fused, steps, warmup, stream, prewarm_s) / steps
    tp = time_gpu(pack, max(3, steps // 4), 2, stream) / max(3, steps // 4)
    return tr, tp


def bench_unfused(w, M, steps, warmup, stream, prewarm_s=0.0):
    """The unfused pipeline on the library's fastest GEMM: W1 and W2 in the
    single-weight pack (packed once, like the fused weights), two GEMM calls
    writing bf16 Gate and Up, then the SiLU * Up kernel reading them back;
    rotated sets like the fused call."""
    import torch
    import swiglu_gated_mlp_amd as sw
    from swiglu_gated_mlp_amd import inputs
    dev = torch.device("cuda:0")
    K, N = w.K, w.N
    A, W1, W2 = inputs.workload_tensors(w, M)
    R = max(1, math.ceil(2 * MALL_BYTES / (fused_bytes(M, K, N) + unfused_extra_bytes(M, K, N))))
    sets = []
    for _ in range(R):
        W1d, W2d = W1.to(dev), W2.to(dev)
        sets.append((A.to(dev), sw.swiglu_gemm_pack_weight(W1d), sw.swiglu_gemm_pack_weight(W2d),
                     torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                     torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                     torch.empty((M, N), dtype=torch.bfloat16, device=dev)))
        del W1d, W2d
    torch.cuda.synchronize()
    fns = [(lambda t=t: sw.swiglu_unfused_packed(t[0], t[1], t[2], N, t[3], t[4], t[5])) for t in sets]
    sec = time_gpu(fns, steps, warmup, stream, prewarm_s)
    return sec / steps


def bench_gemm(w, M, steps, warmup, stream, prewarm_s=0.0):
    """One GEMM of the unfused pipeline alone, C = A @ W1 on the single-weight
    pack, over rotated sets: per-call seconds, TFLOP/s (2 M K N) and GB/s
    (A, W and C once each)."""
    import torch
    import swiglu_gated_mlp_amd as sw
    from swiglu_gated_mlp_amd import inputs
    dev = torch.device("cuda:0")
    K, N = w.K, w.N
    A, W1, _ = inputs.workload_tensors(w, M)
    nbytes = 2.0 * (M * K + K * N + M * N)
    R = max(1, math.ceil(2 * MALL_BYTES / nbytes))
    W1d = W1.to(dev)
    sets = [(A.to(dev), sw.swiglu_gemm_pack_weight(W1d), torch.empty((M, N), dtype=torch.bfloat16, device=dev))
            for _ in range(R)]
    del W1d
    torch.cuda.synchronize()
    fns = [(lambda t=t: sw.swiglu_gemm_packed(t[0], t[1], N, t[2])) for t in sets]
    per = time_gpu(fns, steps, warmup, stream, prewarm_s) / steps
    return {"gemm_us": round(per * 1e6, 2), "gemm_tflops": round(2.0 * M * K * N / per / 1e12, 2),
            "gemm_gbs": round(nbytes / per / 1e9, 1)}


def bench_mlp(w, M, steps, warmup, stream, prewarm_s=0.0):
    """The gated MLP block (SwiGLU product, then the down projection Y @ W3)
    fused and unfused, and the down projection alone, each over rotated
    input sets; returns per-call seconds and the SwiGLU shares of MLP time."""
    import torch
    import swiglu_gated_mlp_amd as sw
    from swiglu_gated_mlp_amd import inputs
    dev = torch.device("cuda:0")
    K, N = w.K, w.N
    A, W1, W2 = inputs.workload_tensors(w, M)
    W3 = inputs.down_weight(w)
    R = max(1, math.ceil(2 * MALL_BYTES / (fused_bytes(M, K, N) + 2 * (N * K + M * K))))
    mk = lambda r, c: torch.empty((r, c), dtype=torch.bfloat16, device=dev)  # noqa: E731
    sets = []
    for _ in range(R):
        W1d, W2d = W1.to(dev), W2.to(dev)
        sets.append(dict(A=A.to(dev), W1g=sw.swiglu_gemm_pack_weight(W1d), W2g=sw.swiglu_gemm_pack_weight(W2d),
                         Wp=sw.swiglu_pack_weights(W1d, W2d), W3g=sw.swiglu_gemm_pack_weight(W3.to(dev)),
                         G=mk(M, N), U=mk(M, N), Y=mk(M, N), Z=mk(M, K), ws=sw.Workspace(dev)))
        del W1d, W2d
    torch.cuda.synchronize()
    fused = [(lambda d=d: sw.swiglu_mlp_packed(d["A"], d["Wp"], d["W3g"], N, Y=d["Y"], Z=d["Z"],
                                               workspace=d["ws"])) for d in sets]
    unfused = [(lambda d=d: sw.swiglu_mlp_unfused(d["A"], d["W1g"], d["W2g"], d["W3g"], N, d["G"], d["U"],
                                                  d["Y"], d["Z"], workspace=d["ws"])) for d in sets]
    down = [(lambda d=d: sw.swiglu_mlp_down(d["Y"], d["W3g"], K, d["Z"], workspace=d["ws"])) for d in sets]
    tf = time_gpu(fused, steps, warmup, stream, prewarm_s) / steps
    tu = time_gpu(unfused, steps, warmup, stream, prewarm_s) / steps
    td = time_gpu(down, steps, warmup, stream, prewarm_s) / steps
    # removed_by_fusion: the share of the unfused MLP's time that fusion takes
    # away (materialised Gate/Up, the separate activation pass, and the
    # difference between the two SwiGLU kernels); gateup_share_*: the share of
    # the gate/up projections plus activation in each MLP (the rest is the
    # down projection)
    return {"workload": w.name, "M": M, "K": K, "N": N, "rotation": R,
            "mlp_fused_us": round(tf * 1e6, 2), "mlp_unfused_us": round(tu * 1e6, 2),
            "down_proj_us": round(td * 1e6, 2), "mlp_speedup": round(tu / tf, 3),
            "removed_by_fusion": round((tu - tf) / tu, 4),
            "gateup_share_unfused": round((tu - td) / tu, 4), "gateup_share_fused": round((tf - td) / tf, 4)}


def ceilings(stream):
    """What the device sustains: MFMA-only loop, streaming read, and the vendor
    library's bf16 GEMM on the same [M,K]x[K,2N] shapes (context only)."""
    import torch
    import swiglu_gated_mlp_amd as sw
    from swiglu_gated_mlp_amd import inputs
    dev = torch.device("cuda:0")
    out = {}
    blocks, iters = 2048, 1000
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    sec = time_gpu([lambda: sw.swiglu_probe_mfma(sink, blocks, iters)], 5, 2, stream)
    out["mfma_bf16_tflops"] = round(blocks * 4 * iters * 8 * 32768 / (sec / 5) / 1e12, 1)
    nbytes = 4 << 30
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev)
    src.fill_(1.0)
    isink = torch.empty(4096 * 256, dtype=torch.int32, device=dev)
    for b in (1024, 2048, 4096):
        sec = time_gpu([lambda b=b: sw.swiglu_probe_read(src, isink, b)], 5, 2, stream)
        out["hbm_read_gbs_blocks%d" % b] = round(nbytes / (sec / 5) / 1e9, 1)
    del src
    dst = torch.empty(nbytes // 4, dtype=torch.bfloat16, device=dev)
    srcc = torch.ones(nbytes // 4, dtype=torch.bfloat16, device=dev)
    sec = time_gpu([lambda: dst.copy_(srcc)], 5, 2, stream)
    out["copy_gbs_read_plus_write"] = round(2 * (nbytes // 2) / (sec / 5) / 1e9, 1)
    del dst, srcc
    for name, m in (("qwen2.5-0.5B-prefill", 4096), ("qwen2.5-7B-prefill", 8192), ("qwen2.5-72B", 4096)):
        w = inputs.BY_NAME[name]
        A = torch.randn(m, w.K, device=dev).to(torch.bfloat16)
        W = (torch.randn(w.K, 2 * w.N, device=dev) * w.K ** -0.5).to(torch.bfloat16)
        sec = time_gpu([lambda: torch.matmul(A, W)], 10, 3, stream)
        out["torch_matmul_%s_tflops" % name] = round(flops(m, w.K, w.N) / (sec / 10) / 1e12, 1)
        del A, W
    log("CEIL " + json.dumps(out))
    return out


def mfma_probe(blocks=2048, iters=1000, calls=3):
    """The MFMA-only loop (no memory traffic) a few times: what the matrix-core
    counters read when the matrix cores are the only busy unit."""
    import torch
    import swiglu_gated_mlp_amd as sw
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(calls):
        sw.swiglu_probe_mfma(sink, blocks, iters)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / calls
    log("mfma probe: %d calls of %d workgroups x %d iterations, %.1f TFLOP/s (host clock)"
        % (calls, blocks, iters, blocks * 4 * iters * 8 * 32768 / dt / 1e12))


def copy_probe(mib):
    """A plain device copy of a known size (the byte-counter calibration run)."""
    import torch
    n = (mib << 20) // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copy probe: 3 copies of %d MiB" % mib)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--prewarm", type=float, default=0.5, metavar="SECONDS",
                    help="untimed calls before the warm-up steps, in seconds of wall time (0 under a profiler)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--m", type=int, default=None, help="token count (default: the workload's largest)")
    ap.add_argument("--variant", default="auto", choices=["auto", "data_parallel", "split_k", "sequential"])
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "fp8"],
                    help="operand type: bf16 (default) or FP8 E4M3 with per-tensor scales (the workload's "
                         "tensors quantised; data-parallel streaming schedule)")
    ap.add_argument("--layout", default="per-tile", choices=["per-tile", "interleaved"],
                    help="packed weight layout: per-128-column-tile [W1|W2] (default) or column-granular "
                         "interleave (the data-parallel streaming schedule only)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--repeats", type=int, default=5,
                    help="--all: timed repeats per point (median and min/max reported)")
    ap.add_argument("--mlp", action="store_true",
                    help="also time the whole gated MLP block (with the down projection), fused and "
                         "unfused, at the workload point (with --all: at every point) (stderr)")
    ap.add_argument("--all", action="store_true",
                    help="also time every workload point and the unfused pipeline (stderr)")
    ap.add_argument("--ceilings", action="store_true",
                    help="also measure the MFMA / HBM / vendor-GEMM ceilings (stderr)")
    ap.add_argument("--unfused", action="store_true",
                    help="only time the unfused pipeline (two GEMM launches, then the SiLU*Up kernel) at "
                         "the workload point, print an UNFUSED line (stderr) and exit (for counter runs)")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only run the MFMA-only loop a few times and exit (matrix-core counter calibration)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (byte-counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the fused SwiGLU product runs on a "
              "single MI355X (no multi-GPU path); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import swiglu_gated_mlp_amd as sw
    from swiglu_gated_mlp_amd import inputs
    from swiglu_gated_mlp_amd import build as hip_build
    if not os.path.exists(hip_build.LIB_PATH):
        hip_build.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sw.lib()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.mfma_probe:
        mfma_probe()
        return
    stream = torch.cuda.current_stream()
    if args.ceilings:
        ceilings(stream)
    w = inputs.BY_NAME[args.workload]
    M = args.m or (DEFAULT_M if w.name == DEFAULT_WORKLOAD else w.m_max)
    if args.unfused:
        tu = bench_unfused(w, M, args.steps, args.warmup, stream, args.prewarm)
        log("UNFUSED " + json.dumps({"workload": w.name, "M": M, "K": w.K, "N": w.N,
                                     "us": round(tu * 1e6, 2),
                                     "model_bytes": fused_bytes(M, w.K, w.N) + unfused_extra_bytes(M, w.K, w.N)}))
        return

    if args.dtype == "fp8":
        res = bench_point_fp8(w, M, args.steps, args.warmup, stream, args.prewarm)
    else:
        res = bench_point(w, M, args.steps, args.warmup, args.variant, stream, args.prewarm, args.layout)
    per = res["per_launch_s"]
    bound = bound_of(M, w.K, w.N, args.dtype)
    if bound == "mfma":
        achieved, unit = res["tflops"], "TFLOP/s"
        peak = MFMA_FP8_PEAK_TFLOPS if args.dtype == "fp8" else MFMA_BF16_PEAK_TFLOPS
    else:
        achieved, peak, unit = res["gbs"], HBM_PEAK_GBS, "GB/s"

    extra = {}
    if args.all:
        log("CONTEXT " + json.dumps(run_context()))
        for ww in inputs.WORKLOADS:
            for mm in ww.ms:
                r = bench_point(ww, mm, max(10, args.steps // 2), 5, args.variant, stream, args.prewarm,
                                args.layout, repeats=args.repeats, graph=mm <= 64)
                tu = bench_unfused(ww, mm, max(5, args.steps // 4), 3, stream, args.prewarm)
                b = bound_of(mm, ww.K, ww.N)
                frac = r["tflops"] / MFMA_BF16_PEAK_TFLOPS if b == "mfma" else r["gbs"] / HBM_PEAK_GBS
                line = {"workload": ww.name, "M": mm, "K": ww.K, "N": ww.N, "bound": b,
                        "us": round(r["per_launch_s"] * 1e6, 2), "tflops": round(r["tflops"], 2),
                        "gbs": round(r["gbs"], 1), "frac": round(frac, 4),
                        "unfused_us": round(tu * 1e6, 2),
                        "speedup_vs_unfused": round(tu / r["per_launch_s"], 3),
                        # time saved against the time the removed traffic (Gate and
                        # Up written and read, A read again) takes at peak HBM
                        "fusion_efficiency": round((tu - r["per_launch_s"]) /
                                                   (unfused_extra_bytes(mm, ww.K, ww.N) / (HBM_PEAK_GBS * 1e9)), 3),
                        "resolved_variant": r["resolved_variant"]}
                if "repeats" in r:
                    line.update(repeats=r["repeats"], us_min=round(r["per_min_s"] * 1e6, 2),
                                us_max=round(r["per_max_s"] * 1e6, 2))
                if "graph_per_launch_s" in r:
                    line["graph_us"] = round(r["graph_per_launch_s"] * 1e6, 2)
                line.update(bench_gemm(ww, mm, max(10, args.steps // 2), 5, stream, args.prewarm))
                # the unpacked entry point (row-major weights) and the one-time
                # pack, reported beside the packed path they stand for
                tr, tp = bench_rowmajor(ww, mm, max(10, args.steps // 4), 3, stream, args.prewarm)
                line.update(rowmajor_us=round(tr * 1e6, 2), rowmajor_tflops=round(flops(mm, ww.K, ww.N) / tr / 1e12, 2),
                            pack_us=round(tp * 1e6, 2))
                log("POINT " + json.dumps(line))
                extra.setdefault("points", []).append(line)
                if args.mlp:
                    log("MLP " + json.dumps(bench_mlp(ww, mm, max(10, args.steps // 2), 5, stream,
                                                      args.prewarm)))
    elif args.mlp:
        log("MLP " + json.dumps(bench_mlp(w, M, args.steps, args.warmup, stream, args.prewarm)))

    cpu = None
    if not args.no_cpu and args.dtype == "bf16":
        log("timing the CPU oracle on a sample of the workload ...")
        cpu = cpu_baseline(w, M)

    out = {
        "metric": "fused SwiGLU TFLOP/s (bf16) at Qwen-2.5 shapes; % of MFMA/HBM roofline",
        "value": round(res["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(per * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic (seeded N(0,1) activations, N(0,1/K) weights)",
        "config": {"workload": "%s M=%d K=%d N=%d" % (w.name, M, w.K, w.N), "M": M, "K": w.K,
                   "N": w.N, "variant": args.variant, "layout": args.layout, "rotation_sets": res["rotation"]},
        "roofline": {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 5),
                     "scope": "one swiglu_fused_packed call, all of its kernel launches",
                     "traffic": (measured_traffic("%s M=%d K=%d N=%d" % (w.name, M, w.K, w.N))
                                 if args.dtype == "bf16" else None)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
