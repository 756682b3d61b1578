#!/usr/bin/env python3
"""Benchmark of the NF4-LoRA linear layer on one MI355X.

The workload is the Llama-7B attention projection: W 4096x4096 (NF4, blocks
of 64, 8-bit scales in groups of 256), 2048 tokens, rank 16, s = 2.  A step is
one pass of the layer: the fused forward (Y and the saved T) and the backward
(dX, dL1, dL2).  The weight is quantized once before the timed region, as in
training, where the frozen base is quantized when it is loaded; the profiling
pass (NF4 quantize with double quantization and the per-layer reconstruction
error from one read of W, then the top-K protected set) runs there too and is
timed on its own.

`value` is the forward+backward algorithmic work F = 4 M h o + 6 M r (h + o)
divided by the wall time of a step.  The JSON line also carries the per-op
breakdown, the profiling pass, the roofline of the dominant kernel timed with
HIP events on the stream it is launched on, and the CPU oracle timed on this
host.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused NF4-LoRA linear fwd+bwd TFLOP/s and % bf16 MFMA peak, 4096² r=16"
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 dense bf16 FLOP/clk/CU
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_nf4_gemm_c2.json")
GEMM_SOURCES = ["quantized_lora_fine_amd/csrc/gemm.hip", "quantized_lora_fine_amd/csrc/common.hpp"]


def kernel_source_hash() -> str:
    """Hash of the fused GEMM's code (comments, trailing spaces and blank lines
    left out, so an edit to comments alone keeps the stored counters valid)."""
    import re
    h = hashlib.sha256()
    for p in GEMM_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            for line in f:
                code = re.sub(r"//.*", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def flops_fwd_bwd(M, h, o, r):
    return 4.0 * M * h * o + 6.0 * M * r * (h + o)


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def blas_threads():
    """(threads, library) of the BLAS numpy calls, as threadpoolctl reports them."""
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            return max(i.get("num_threads", 1) for i in blas), blas[0].get("internal_api", "blas")
    except Exception:  # pragma: no cover
        pass
    return 1, "unknown"


def cpu_baseline(d, s, budget_s=10.0, min_steps=3):
    """The oracle, as it stands, on this host: the step the GPU line times (the
    forward and the backward of the layer, the dequantized weight rebuilt from
    the codes each time, as the fused kernels do), on the same workload, repeated
    until about `budget_s` seconds of work (at least `min_steps` steps); returns
    the fastest step.  The weight is quantized once, before, as on the GPU."""
    import oracle
    q = oracle.quantize(d["W"], 64, 256)
    best, n, t_all = None, 0, time.perf_counter()
    while n < min_steps or time.perf_counter() - t_all < budget_s:
        t0 = time.perf_counter()
        wh = oracle.dequantize(q)
        oracle.fwd(d["X"], wh, d["L1"], d["L2"], s)
        oracle.bwd(d["X"], d["dY"], wh, d["L1"], d["L2"], s)
        dt = time.perf_counter() - t0
        best = dt if best is None else min(best, dt)
        n += 1
    return best, n


# algorithmic bytes per weight of the passes over W: quantize with 8-bit scales
# (read fp32, write 4-bit codes, one 8-bit scale per 64 and one fp32 step per
# 16384 weights) and the layer error (read fp32 only)
QUANT_DQ_BYTES_PER_WEIGHT = 4 + 0.5 + 1 / 64 + 4 / 16384
ERROR_BYTES_PER_WEIGHT = 4.0


def cpu_passes(W, threads, reps=3, rows_per_chunk=64):
    """The oracle's quantize (8-bit scales) and layer error (fp32 scales) over
    all of W in chunks of `rows_per_chunk` rows (whole double-quantization
    groups for rows of 4096 weights) on `threads` threads; numpy releases the
    GIL inside its vector operations.  Best of `reps` for each; returns the
    rates in GB/s of algorithmic bytes."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    chunks = [W[i:i + rows_per_chunk] for i in range(0, W.shape[0], rows_per_chunk)]

    def best(fn):
        t = None
        with ThreadPoolExecutor(max(1, threads)) as ex:
            for _ in range(reps):
                t0 = time.perf_counter()
                list(ex.map(fn, chunks))
                dt = time.perf_counter() - t0
                t = dt if t is None else min(t, dt)
        return t

    tq = best(lambda w: oracle.quantize(w, 64, 256))
    te = best(lambda w: oracle.layer_error(w, 64, 0))
    return {"quantize_dq_GBps": round(W.size * QUANT_DQ_BYTES_PER_WEIGHT / tq / 1e9, 4),
            "layer_error_GBps": round(W.size * ERROR_BYTES_PER_WEIGHT / te / 1e9, 4),
            "sample": f"all {W.size} weights of this W in {len(chunks)} chunks of {rows_per_chunk} rows on "
                      f"{max(1, threads)} threads, best of {reps}",
            "threads": max(1, threads)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 200 for c2, 20 for c3 and c5, 5 for c4-stack)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: 20 for c2, after --settle-ms of untimed steps; "
                         "3 for c3 and c5, 1 for c4-stack)")
    ap.add_argument("--kernel-calls", type=int, default=50,
                    help="c2: back-to-back launches per window of the standalone kernel timings")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="c2: untimed full steps for this long before the warmup steps, so the timed steps run "
                         "at the steady shader clock")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--power-probe", action="store_true",
                    help="c2: also sample socket power and the shader clock (amd-smi, rocm-smi in a child "
                         "process) while the forward GEMM runs back to back, and while a spin kernel runs")
    ap.add_argument("--workload", default="c2", choices=["c2", "c3", "c5", "c4-stack"],
                    help="c2: the 4096x4096 layer (default); c3: the three 7B-shaped MLP linears; c5: the "
                         "70B-shaped up projection; c4-stack: the 280-linear 14B-shaped stack with AQLoRA's "
                         "allocation against QLoRA")
    args = ap.parse_args()
    steps0, warmup0 = {"c2": (200, 20), "c3": (20, 3), "c5": (20, 3), "c4-stack": (5, 1)}[args.workload]
    if args.steps is None:
        args.steps = steps0
    if args.warmup is None:
        args.warmup = warmup0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: measures one GPU only (the layer runs on a single MI355X); "
              "multi-GPU runs are not supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_lora_fine_amd as nf4
    import synth

    if args.workload == "c4-stack":
        return bench_stack(args)
    if args.workload in ("c3", "c5"):
        return bench_layers(args)

    cfg = synth.C2
    M, o, h, r, s = cfg.M, cfg.rows, cfg.cols, cfg.r, cfg.s
    d = synth.layer_inputs(cfg)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"# device {torch.cuda.get_device_name(0)}; workload {cfg.name}", file=sys.stderr, flush=True)

    W = torch.from_numpy(d["W"]).to(dev)
    X, L1, L2, dY = (d[k].to(dev).contiguous() for k in ("X", "L1", "L2", "dY"))
    q = nf4.NF4Weight(o, h, 256, dev)
    err = torch.empty(1, dtype=torch.float64, device=dev)
    idx = torch.empty(1, dtype=torch.int32, device=dev)
    ws_e = torch.empty(nf4.workspace_bytes(nf4.NF4_OP_ERROR, 0, o, h, 1), dtype=torch.uint8, device=dev)
    ws_f = nf4.workspace(nf4.NF4_OP_FWD, M, q, r)
    ws_b = nf4.workspace(nf4.NF4_OP_BWD, M, q, r)
    Y = torch.empty(M, o, dtype=torch.bfloat16, device=dev)
    T = torch.empty(M, r, dtype=torch.bfloat16, device=dev)
    dX = torch.empty(M, h, dtype=torch.bfloat16, device=dev)
    dL1 = torch.empty(h, r, dtype=torch.float32, device=dev)
    dL2 = torch.empty(r, o, dtype=torch.float32, device=dev)

    # ---- once, before the timed region: the profiling pass and the stored weight ----
    prof_ops = [
        ("quantize+error", lambda: nf4.quantize_error(W, 256, 0, out=q, err=err, ws=ws_e)),
        ("topk", lambda: nf4.topk(err, 1, out=idx)),
    ]
    for _, f in prof_ops:
        f()
    torch.cuda.synchronize()

    ops = [
        ("fwd", lambda: nf4.fwd(q, X, L1, L2, s, ws=ws_f, out=Y, T_out=T)),
        ("bwd", lambda: nf4.bwd(q, X, dY, L1, L2, s, T=T, ws=ws_b, outs=(dX, dL1, dL2))),
    ]

    def step():
        for _, f in ops:
            f()

    # ---- clock settle: the shader clock takes tens of ms of work to reach its steady
    # level after the host-side setup (0.201 against 0.182 ms per step over the
    # first 10 steps); full steps run untimed until `settle_ms` of them have passed ----
    t_settle = time.perf_counter()
    n_settle = 0
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        n_settle += 20

    # ---- the timed region: `warmup` untimed steps, then exactly `steps` steps ----
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / max(args.steps, 1)
    F = flops_fwd_bwd(M, h, o, r)
    value = F / (ms_per_step * 1e-3) / 1e12
    print(f"# timed {args.steps} steps: {ms_per_step:.4f} ms/step", file=sys.stderr, flush=True)

    # ---- per-op breakdown: HIP events between the ops of each step (the profiling
    # pass's ops included, in front of the layer, as they ran once before) ----
    stream = torch.cuda.current_stream()
    all_ops = prof_ops + ops
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(all_ops) + 1)] for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record(stream)
        for j, (_, f) in enumerate(all_ops):
            f()
            evs[i][j + 1].record(stream)
    torch.cuda.synchronize()
    op_ms = {}
    for j, (name, _) in enumerate(all_ops):
        op_ms[name] = sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)) / args.steps
    fb_ms = op_ms["fwd"] + op_ms["bwd"]

    # ---- roofline: the fused NF4 GEMMs alone, K launches between two events ----
    RP = (r + 15) // 16 * 16
    g = torch.Generator(device="cpu").manual_seed(0)
    A2f = torch.zeros(M, RP, dtype=torch.bfloat16, device=dev)
    A2f[:, :r] = (torch.randn(M, r, generator=g) * 0.5).to(torch.bfloat16).to(dev)
    B2f = torch.zeros(o, RP, dtype=torch.bfloat16, device=dev)
    B2f[:, :r] = L2.t()
    A2b = torch.zeros(M, RP, dtype=torch.bfloat16, device=dev)
    A2b[:, :r] = (torch.randn(M, r, generator=g) * 0.5).to(torch.bfloat16).to(dev)
    B2b = torch.zeros(h, RP, dtype=torch.bfloat16, device=dev)
    B2b[:, :r] = L1
    Cf = torch.empty(M, o, dtype=torch.bfloat16, device=dev)
    Cb = torch.empty(M, h, dtype=torch.bfloat16, device=dev)
    # Standalone kernel timings: 7 interleaved repetitions across these ops, each a
    # window of `steps` back-to-back launches between HIP events on the launch
    # stream; `us` is the mean of the fastest half, with the median and range.
    n = o * h
    q_bytes = 4 * n + n // 2 + n // 64 + 4 * (n // 64 // 256)
    e_bytes = 4 * n
    Wm = torch.empty(o, h, dtype=torch.bfloat16, device=dev)
    # context for the fused GEMMs: hipBLASLt's plain bf16 GEMM (torch.mm) at the same shapes on the
    # dequantized weight, the unfused stock path (dequantize to bf16, then the base matmul and the two
    # adapter matmuls), and the MFMA-only probe (no memory traffic)
    Wq = nf4.dequantize(q, bf16=True)
    Cf2 = torch.empty(M, o, dtype=torch.bfloat16, device=dev)
    Cb2 = torch.empty(M, h, dtype=torch.bfloat16, device=dev)
    Tst = torch.empty(M, r, dtype=torch.bfloat16, device=dev)

    def stock_fwd():
        nf4.dequantize(q, bf16=True, out=Wm)
        torch.mm(X, Wm.t(), out=Cf2)
        torch.mm(X, L1, out=Tst)
        Cf2.addmm_(Tst, L2, alpha=s)

    # what plain streaming reaches at this size, as context for the passes over W: torch's fp32 copy of W
    # (67 MB read, 67 MB written) and its fp32 sum of W (67 MB read)
    Wc = torch.empty_like(W)
    Wsum = torch.empty((), dtype=torch.float32, device=dev)
    probe_wg, probe_iters = 256, 180
    probe_out = torch.empty(probe_wg * 512, dtype=torch.float32, device=dev)
    probe_flops = probe_wg * 8 * (probe_iters + probe_iters % 2) * 8 * 32768.0
    work = {
        "nf4_gemm_fwd": (lambda: nf4.matmul(q, X, False, A2f, B2f, out=Cf), "flops", 2.0 * M * h * o + 2.0 * M * r * o),
        "nf4_gemm_dx": (lambda: nf4.matmul(q, dY, True, A2b, B2b, out=Cb), "flops", 2.0 * M * h * o + 2.0 * M * r * h),
        "quantize_error_dq": (lambda: nf4.quantize_error(W, 256, 0, out=q, err=err, ws=ws_e), "bytes", q_bytes),
        # the two passes on their own (each reads W once)
        "quantize_dq": (lambda: nf4.quantize(W, 256, out=q), "bytes", q_bytes),
        "layer_error": (lambda: nf4.layer_error(W, 0, out=err, ws=ws_e), "bytes", e_bytes),
        # merge after training (not part of the step): NF4 base -> bf16, fp32 base -> bf16
        "merge_nf4_to_bf16": (lambda: nf4.merge(q, L1, L2, s, bf16=True, out=Wm), "bytes",
                              n // 2 + n // 64 + 4 * (n // 64 // 256) + 2 * n),
        "merge_fp32_to_bf16": (lambda: nf4.merge(W, L1, L2, s, bf16=True, out=Wm), "bytes", 6 * n),
        "torch_copy_fp32_W": (lambda: Wc.copy_(W), "bytes", 8 * n),
        "torch_sum_fp32_W": (lambda: torch.sum(W, dim=(0, 1), out=Wsum), "bytes", 4 * n),
        "hipblaslt_bf16_fwd": (lambda: torch.mm(X, Wq.t(), out=Cf2), "flops", 2.0 * M * h * o),
        "hipblaslt_bf16_dx": (lambda: torch.mm(dY, Wq, out=Cb2), "flops", 2.0 * M * h * o),
        "unfused_stock_fwd": (stock_fwd, "flops", 2.0 * M * h * o + 2.0 * M * r * (h + o)),
        "mfma_only_probe": (lambda: nf4.probe_mfma_peak(probe_iters, probe_wg, probe_out), "flops", probe_flops),
    }
    stats = interleaved_times({k: v[0] for k, v in work.items()}, args.kernel_calls, 7, stream, torch)
    kernels = {}
    for name, (_, kind, amount) in work.items():
        st = stats[name]
        kernels[name] = dict(st)
        if kind == "flops":
            tf = amount / (st["us"] * 1e-6) / 1e12
            kernels[name].update(tflops=round(tf, 1), pct_bf16_peak=round(100 * tf / PEAK_BF16_TFLOPS, 1),
                                 flops_per_launch=amount)
        else:
            gb = amount / (st["us"] * 1e-6) / 1e9
            kernels[name].update(GBps=round(gb, 1), pct_hbm_peak=round(100 * gb / PEAK_HBM_GBS, 1), bytes=amount)
    kernels["timing"] = (f"7 interleaved repetitions of {args.kernel_calls} back-to-back launches per op (HIP events on "
                         f"the launch stream); us = mean of the fastest half")

    # the same weights at identical storage in the other 4-bit codebooks: reconstruction error and quantize time
    codebooks = {}
    for cbn in ("nf4", "int4", "fp4"):
        qc = nf4.NF4Weight(o, h, 256, dev, cbn)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nf4.quantize(W, 256, out=qc)
        e0.record(stream)
        for _ in range(args.steps):
            nf4.quantize(W, 256, out=qc)
        e1.record(stream)
        err_c = nf4.layer_error(W, 256, ws=ws_e, codebook=cbn)
        torch.cuda.synchronize()
        codebooks[cbn] = {"rel_frobenius_error": round(float(err_c.cpu()), 6),
                          "quantize_us": round(1e3 * e0.elapsed_time(e1) / args.steps, 3)}

    # the second NF4 stage over the residual: fwd+bwd with the two-stage weight against one stage
    q_res = nf4.quantize(W, 256, residual=True)
    res_ms = {}
    for name, qq in (("one_stage", q), ("two_stage", q_res)):
        def fb():
            nf4.fwd(qq, X, L1, L2, s, ws=ws_f, out=Y, T_out=T)
            nf4.bwd(qq, X, dY, L1, L2, s, T=T, ws=ws_b, outs=(dX, dL1, dL2))
        for _ in range(args.warmup):
            fb()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fb()
        e1.record(stream)
        torch.cuda.synchronize()
        res_ms[name] = e0.elapsed_time(e1) / args.steps
    residual = {"fwd_bwd_ms_one_stage": round(res_ms["one_stage"], 5),
                "fwd_bwd_ms_two_stage": round(res_ms["two_stage"], 5),
                "overhead_pct": round(100.0 * (res_ms["two_stage"] / res_ms["one_stage"] - 1.0), 2)}
    del q_res

    dom = max(("nf4_gemm_fwd", "nf4_gemm_dx"), key=lambda k: kernels[k]["us"])
    ach = kernels[dom]["tflops"]
    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_source_hash") == kernel_source_hash() and dom in tr.get("kernels", {}):
            traffic = tr["kernels"][dom]["bytes_per_launch"]
    except (OSError, ValueError, KeyError):
        traffic = None
    roofline = {"bound": "mfma", "kernel": dom, "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic}

    power = None
    if args.power_probe:
        power = {"fwd_gemm_back_to_back": power_probe(lambda: nf4.matmul(q, X, False, A2f, B2f, out=Cf), torch),
                 "spin_kernel": power_probe(lambda: torch.cuda._sleep(100000), torch)}

    if args.calib_copy:
        src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    cpu = None
    if not args.no_cpu_baseline:
        threads, blas = blas_threads()
        sec, nsteps = cpu_baseline(d, s)
        cpu = {"value": round(F / sec / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
               "sample": f"{nsteps} full fwd+bwd steps of this workload on the CPU oracle (numpy: fp32 "
                         f"dequantize, fp64 products), fastest {sec:.2f} s/step",
               "host_cpus": os.cpu_count(), "cpu_model": host_cpu_model(), "blas": blas, "blas_threads": threads,
               "passes": cpu_passes(d["W"], threads)}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama7b-attn-proj W 4096x4096 NF4 block 64 + 8-bit DQ/256, M=2048 tokens, r=16, s=2",
                   "step": "fwd+bwd (dX, dL1, dL2); quantize, error and top-K once before the timed region",
                   "tokens": M, "rank": r, "flops_fwd_bwd": F},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "pct_of_target": round(100 * value / (0.6 * PEAK_BF16_TFLOPS), 2),
        "settle": {"steps": n_settle, "ms": args.settle_ms},
        "fwd_bwd_ms_events": round(fb_ms, 5),
        "op_ms": {k: round(v, 5) for k, v in op_ms.items()},
        "profiling_pass": {"quantize_error_ms": round(op_ms["quantize+error"], 5), "topk_ms": round(op_ms["topk"], 5),
                           "quantize_error_GBps": round(q_bytes / (op_ms["quantize+error"] * 1e-3) / 1e9, 1)},
        "kernels": kernels,
        "codebooks": codebooks,
        "residual_stage": residual,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if power is not None:
        out["power_probe"] = power
    print(json.dumps(out), flush=True)


def interleaved_times(fns, calls, reps, stream, torch):
    """Per-launch time of each op in `fns`: `reps` rounds, each timing every op
    in turn over `calls` back-to-back launches (after 2 untimed ones) with HIP
    events on `stream`.  Returns, per op, the mean of the fastest half of the
    rounds (`us`), their median and their range, in microseconds.  Seven
    interleaved runs and the fastest half follow the timing protocol of the
    AQLoRA page (section 4, "Timing protocol")."""
    import statistics
    times = {k: [] for k in fns}
    for _ in range(reps):
        for name, fn in fns.items():
            for _ in range(2):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(calls):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times[name].append(1e3 * e0.elapsed_time(e1) / calls)
    out = {}
    for name, t in times.items():
        t = sorted(t)
        fast = t[:(len(t) + 1) // 2]
        out[name] = {"us": round(sum(fast) / len(fast), 3), "median_us": round(statistics.median(t), 3),
                     "min_us": round(t[0], 3), "max_us": round(t[-1], 3)}
    return out


def power_probe(fn, torch, secs: float = 8.0):
    """Launch `fn` back to back for `secs` seconds; halfway through, read the
    socket power (amd-smi) and the shader clock (rocm-smi) from a child process.
    Returns the readings and the mean time per launch (None for a reading the
    tools do not report)."""
    import re
    import subprocess
    t0 = time.perf_counter()
    proc, n = None, 0
    while time.perf_counter() - t0 < secs:
        for _ in range(50):
            fn()
        torch.cuda.synchronize()
        n += 50
        if proc is None and time.perf_counter() - t0 > secs / 2:
            try:
                proc = subprocess.Popen(["sh", "-c", "amd-smi metric -p; rocm-smi --showclocks"],
                                        stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
            except OSError:
                proc = False
    elapsed = time.perf_counter() - t0
    text = ""
    if proc:
        try:
            text = proc.communicate(timeout=60)[0]
        except subprocess.TimeoutExpired:
            proc.kill()
            text = proc.communicate()[0]
    pw = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", text)
    sc = re.search(r"sclk clock level:[^(]*\((\d+)\s*Mhz\)", text)
    return {"socket_power_w": float(pw.group(1)) if pw else None, "sclk_mhz": int(sc.group(1)) if sc else None,
            "us_per_launch": round(1e6 * elapsed / max(n, 1), 2), "launches": n}


def bench_layers(args):
    """Larger single layers at their full sizes: c3 (gate, up, down of a 7B-shaped
    MLP, M=8192, r=64) or c5 (a 70B-shaped up projection, M=16384, r=64).  Per
    linear: quantize (8-bit DQ scales) and bf16 dequantize as standalone passes,
    and the fused fwd and bwd, each timed with HIP events over `steps` calls after
    `warmup` calls and at least 50 ms of the op's own work.  The value is the fwd+bwd FLOP of all the linears over their summed
    fwd+bwd time.  The CPU oracle is not timed at these sizes (cpu_baseline is
    null); the full-size parity tests check these workloads against it."""
    import torch

    import quantized_lora_fine_amd as nf4
    import synth

    layers = {"c3": [synth.C3_GATE, synth.C3_UP, synth.C3_DOWN], "c5": [synth.C5]}[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    print(f"# device {torch.cuda.get_device_name(0)}; workload {args.workload}", file=sys.stderr, flush=True)

    def timed(fn):
        # untimed calls first: `warmup` of them and at least 50 ms of the op's own work (the clock takes
        # tens of ms to settle after the host-side setup; without this the first op timed the ramp)
        t_end, n = time.perf_counter() + 0.05, 0
        while n < args.warmup or time.perf_counter() < t_end:
            fn()
            torch.cuda.synchronize()
            n += 1
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps  # ms

    per, F_all, ms_all = [], 0.0, 0.0
    for cfg in layers:
        M, o, h, r, s = cfg.M, cfg.rows, cfg.cols, cfg.r, cfg.s
        d = synth.layer_inputs(cfg)
        W = torch.from_numpy(d["W"]).to(dev)
        X, L1, L2, dY = (d[k].to(dev).contiguous() for k in ("X", "L1", "L2", "dY"))
        del d
        q = nf4.NF4Weight(o, h, 256, dev)
        n = o * h
        q_ms = timed(lambda: nf4.quantize(W, 256, out=q))
        Wd = torch.empty(o, h, dtype=torch.bfloat16, device=dev)
        dq_ms = timed(lambda: nf4.dequantize(q, bf16=True, out=Wd))
        # what plain PyTorch elementwise passes over the same weights reach: an fp32 copy (4 B read + 4 B
        # written per weight) and the fp32 -> bf16 conversion (4 + 2 B), the practical streaming rates the
        # quantize (4.5 B) and dequantize (2.5 B) passes are compared with
        Wc = torch.empty_like(W)
        cp_ms = timed(lambda: Wc.copy_(W))
        cv_ms = timed(lambda: Wd.copy_(W))
        del Wd, W, Wc
        ws_f = nf4.workspace(nf4.NF4_OP_FWD, M, q, r)
        ws_b = nf4.workspace(nf4.NF4_OP_BWD, M, q, r)
        Y = torch.empty(M, o, dtype=torch.bfloat16, device=dev)
        T = torch.empty(M, r, dtype=torch.bfloat16, device=dev)
        dX = torch.empty(M, h, dtype=torch.bfloat16, device=dev)
        dL1 = torch.empty(h, r, dtype=torch.float32, device=dev)
        dL2 = torch.empty(r, o, dtype=torch.float32, device=dev)
        f_ms = timed(lambda: nf4.fwd(q, X, L1, L2, s, ws=ws_f, out=Y, T_out=T))
        b_ms = timed(lambda: nf4.bwd(q, X, dY, L1, L2, s, T=T, ws=ws_b, outs=(dX, dL1, dL2)))
        F = flops_fwd_bwd(M, h, o, r)
        F_all += F
        ms_all += f_ms + b_ms
        q_bytes = 4 * n + n // 2 + n // 64 + 4 * (n // 64 // 256)
        dq_bytes = n // 2 + n // 64 + 4 * (n // 64 // 256) + 2 * n
        tf = F / ((f_ms + b_ms) * 1e-3) / 1e12
        per.append({"linear": cfg.name, "o": o, "h": h, "tokens": M, "rank": r, "flops_fwd_bwd": F,
                    "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4), "fwd_bwd_tflops": round(tf, 1),
                    "fwd_bwd_pct_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                    "quantize_us": round(1e3 * q_ms, 2), "quantize_GBps": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
                    "dequantize_bf16_us": round(1e3 * dq_ms, 2),
                    "dequantize_GBps": round(dq_bytes / (dq_ms * 1e-3) / 1e9, 1),
                    "torch_copy_fp32_GBps": round(8 * n / (cp_ms * 1e-3) / 1e9, 1),
                    "torch_fp32_to_bf16_GBps": round(6 * n / (cv_ms * 1e-3) / 1e9, 1)})
        print(f"# {cfg.name}: fwd {f_ms:.3f} ms, bwd {b_ms:.3f} ms ({tf:.1f} TFLOP/s); quantize {1e3 * q_ms:.1f} us, "
              f"dequantize {1e3 * dq_ms:.1f} us", file=sys.stderr, flush=True)
        del q, X, L1, L2, dY, Y, T, dX, dL1, dL2, ws_f, ws_b
        torch.cuda.empty_cache()
    value = F_all / (ms_all * 1e-3) / 1e12
    wl = {"c3": "llama7b MLP gate, up (W 11008x4096) and down (W 4096x11008), NF4 + DQ/256, M=8192, r=64, s=2",
          "c5": "70b up projection W 28672x8192, NF4 + DQ/256, M=16384, r=64, s=2"}[args.workload]
    out = {"metric": f"fused NF4-LoRA linear fwd+bwd TFLOP/s and % bf16 MFMA peak, {args.workload}",
           "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_all, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": wl, "step": "fwd+bwd of each linear", "flops_fwd_bwd": F_all},
           "fwd_bwd_pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
           "linears": per, "roofline": None, "cpu_baseline": None}
    print(json.dumps(out), flush=True)


def bench_stack(args):
    """The 14B-shaped stack: per-linear NF4 error, top-8 protection, then one
    training step's linear work (forward over all 280 linears, backward down
    to the cut) under three allocations:
      qlora     every linear NF4, adapters everywhere, full backward;
      aqlora-q  the 8 largest-error linears in bf16, adapters everywhere;
      aqlora-s  the same protection, adapters on the top 85% of the blocks
                (below them a plain forward), backward stopped at the lowest
                adapted block, whose input-side linears need no dX.
    Activations are synthetic and shared between linears of the same shape
    (the linear work does not depend on their values)."""
    import torch

    import quantized_lora_fine_amd as nf4
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stack = synth.c4_stack()
    n, M, r, s, K = len(stack), synth.C4_TOKENS, 16, 2.0, synth.C4_TOPK
    nblk = synth.C4_LAYERS
    print(f"# device {torch.cuda.get_device_name(0)}; 14B-shaped stack, {n} linears, M={M}", file=sys.stderr,
          flush=True)
    # profiling pass over all 280 weights, resident at once (50.75 GB fp32), then NF4 storage
    t0 = time.perf_counter()
    Ws = [synth.c4_weight(lin, device=dev) for lin in stack]
    errs = torch.empty(n, dtype=torch.float64, device=dev)
    ws_b = torch.empty(nf4.error_batch_workspace_bytes([tuple(W.shape) for W in Ws]), dtype=torch.uint8,
                       device=dev)

    def pass_ms(fn, reps=3):
        # untimed passes for at least 50 ms first, then the median of `reps` timed passes
        t_end = time.perf_counter() + 0.05
        while time.perf_counter() < t_end:
            fn()
            torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return sorted(ts)[len(ts) // 2]

    # one batched call (64 linears per launch pair), and the same pass as 280 calls of nf4_layer_error
    e_ms = pass_ms(lambda: nf4.layer_error_batch(Ws, 0, out=errs, ws=ws_b))
    ws_e = torch.empty(nf4.workspace_bytes(nf4.NF4_OP_ERROR, 0, synth.C4_FFN, synth.C4_HIDDEN, 1),
                       dtype=torch.uint8, device=dev)
    slots = torch.empty(n, 2, dtype=torch.float64, device=dev)

    def per_linear():
        for i, W in enumerate(Ws):
            nf4.layer_error(W, 0, out=slots[i], ws=ws_e)
    e1_ms = pass_ms(per_linear)
    assert torch.equal(errs, slots[:, 0])
    qs = [nf4.quantize(W, 256) for W in Ws]
    del Ws
    top = nf4.topk(errs, K).cpu().numpy().tolist()
    protected = {i: synth.c4_weight(stack[i], device=dev).to(torch.bfloat16).contiguous() for i in top}
    print(f"# stack built in {time.perf_counter() - t0:.1f} s; top-{K} {top}", file=sys.stderr, flush=True)

    g = torch.Generator(device=dev).manual_seed(7)
    acts = {}
    for width in (synth.C4_HIDDEN, synth.C4_FFN):
        acts[("x", width)] = torch.randn(M, width, generator=g, device=dev).to(torch.bfloat16)
        acts[("y", width)] = torch.empty(M, width, dtype=torch.bfloat16, device=dev)
        acts[("dy", width)] = torch.randn(M, width, generator=g, device=dev).to(torch.bfloat16)
        acts[("dx", width)] = torch.empty(M, width, dtype=torch.bfloat16, device=dev)
    adapters = []
    for lin in stack:
        adapters.append({"L1": (torch.randn(lin.cols, r, generator=g, device=dev) * 0.02).to(torch.bfloat16),
                         "L2": (torch.randn(r, lin.rows, generator=g, device=dev) * 0.02).to(torch.bfloat16),
                         "T": torch.empty(M, r, dtype=torch.bfloat16, device=dev),
                         "dL1": torch.empty(lin.cols, r, dtype=torch.float32, device=dev),
                         "dL2": torch.empty(r, lin.rows, dtype=torch.float32, device=dev)})

    def build(protect, alpha):
        first_blk = nblk - int(round(alpha * nblk))  # lowest adapted block
        cut = first_blk * len(synth.C4_LINEARS)
        linears = []
        for lin in stack:
            L = {"X": acts[("x", lin.cols)], "Y": acts[("y", lin.rows)], "dY": acts[("dy", lin.rows)]}
            if protect and lin.index in protected:
                L["w"] = protected[lin.index]
            else:
                L["q"] = qs[lin.index]
            if lin.index >= cut:
                L.update(adapters[lin.index], r=r, s=s)
                # the lowest adapted block's input-side linears feed nothing that needs a gradient
                if not (lin.layer == first_blk and lin.kind in ("q", "k", "v", "gate", "up")):
                    L["dX"] = acts[("dx", lin.cols)]
            linears.append(L)
        return nf4.Stack(linears, M), cut

    flops_fwd = 2.0 * M * sum(l.rows * l.cols for l in stack)
    res = {}
    for name, protect, alpha in (("qlora", False, 1.0), ("aqlora-q", True, 1.0), ("aqlora-s", True, 0.85)):
        st, cut = build(protect, alpha)

        def step():
            st.fwd()
            st.bwd(cut)

        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        ms = 1e3 * (time.perf_counter() - t) / args.steps
        res[name] = {"ms_per_step": round(ms, 3), "cut": cut, "bf16_linears": K if protect else 0}
        print(f"# {name}: {ms:.2f} ms/step (backward cut at linear {cut})", file=sys.stderr, flush=True)
    base = res["qlora"]["ms_per_step"]
    for k in res:
        res[k]["speedup_vs_qlora_pct"] = round(100.0 * (base / res[k]["ms_per_step"] - 1.0), 2)
    out = {
        "metric": "14B-shaped stack training-step linear work, AQLoRA allocation vs QLoRA",
        "value": res["aqlora-s"]["speedup_vs_qlora_pct"], "unit": "% faster than QLoRA", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["aqlora-s"]["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "14B-shaped stack: 40 blocks x {q,k,v,o 5120^2; gate,up 5120->13824; down "
                               "13824->5120}, Student-t weights, NF4 + DQ/256, top-8 bf16, M=4096, r=16",
                   "forward_tflop": round(flops_fwd / 1e12, 2)},
        "error_pass_ms": round(e_ms, 3), "error_pass_GBps": round(4.0 * sum(l.rows * l.cols for l in stack)
                                                                   / (e_ms * 1e-3) / 1e9, 1),
        "error_pass": "nf4_layer_error_batch over all 280 weights (resident), median of 3 passes after 50 ms "
                      "of untimed passes",
        "error_pass_per_linear_ms": round(e1_ms, 3),
        "protected": top, "modes": res,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
