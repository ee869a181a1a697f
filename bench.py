#!/usr/bin/env python3
"""Benchmark of the FLCE forward+backward hot path on one MI355X.

One step = one flce_forward_backward call over the whole synthetic batch
(all token chunks: logits GEMM + LSE epilogue, combine, dlogits in place,
dx GEMM, dW GEMM, loss finalize), inputs already resident in HBM.

Prints ONE JSON line on stdout (diagnostics go to stderr).  Per-kernel
durations come from the library's own HIP events, recorded on the stream the
kernels run on, over the timed region.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FLCE fwd+bwd tokens/s (V=128256,H=4096,bf16); % MFMA peak; peak HBM"
PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}      # MI355X published dense MFMA peaks
PEAK_SCLK_MHZ = 2400.0                               # the engine clock those peaks assume
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """Source text without comments and whitespace runs (the part that decides the kernels)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(csrc: str = None) -> str:
    """Fingerprint of the HIP sources' code (comments and layout excluded), used to tell whether
    stored rocprofv3 traffic counters still describe the kernels."""
    h = hashlib.sha256()
    csrc = csrc or os.path.join(ROOT, "linear_cross_entropy_token_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp")):
            with open(os.path.join(csrc, f), encoding="utf-8") as fh:
                h.update(f.encode() + b"\0" + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, chunk: int):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE runs, if taken on this source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    e = rec.get(f"{workload}/{chunk}/{kernel}")
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(w, seconds_target: float = 15.0):
    """The CPU oracle (fp64, materialised logits) timed on a bounded token sample."""
    import oracle
    from flce_inputs import make_inputs
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    # Inputs are drawn once for the largest sample: seeded draws are prefix-stable in N, so the
    # first n rows are exactly the workload's first n tokens.  Two small samples give the
    # per-token cost without the fixed part (thread start-up); the timed sample is sized from it.
    n_max = min(8192, w.N)
    d = make_inputs(n_max, w.H, w.V, w.dtype, w.seed, w.targets)
    x_all = oracle.widen(d["x"], w.dtype)
    W = oracle.widen(d["W"], w.dtype)
    t_all = d["t"]
    del d

    def run(n):
        t0 = time.perf_counter()
        oracle.flce(x_all[:n], W, t_all[:n])
        return time.perf_counter() - t0

    n_a, n_b = min(128, n_max), min(512, n_max)
    c_a, c_b = run(n_a), run(n_b)
    per_token = max((c_b - c_a) / max(n_b - n_a, 1), 1e-6)
    n = max(n_b, min(n_max, int(seconds_target / per_token) // 64 * 64))
    dt = run(n) if n > n_b else c_b
    return {"value": n / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {n} tokens of the {w.name} workload (full H={w.H}, V={w.V}), "
                      f"fp64 NumPy oracle with materialised logits, {dt:.2f} s",
            "host": host_info()}


def host_info():
    """CPU model, BLAS library and host RAM of the machine the oracle ran on."""
    info = {"cpu_model": None, "blas": None, "host_ram_gb": None}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if blas:
            info["blas"] = f"{blas[0].get('internal_api')} {blas[0].get('version')}"
    except Exception:
        pass
    try:
        info["host_ram_gb"] = round(os.sysconf("SC_PAGE_SIZE") * os.sysconf("SC_PHYS_PAGES") / 1e9, 1)
    except (ValueError, OSError):
        pass
    return info


def materialised_peak(x, W, t):
    """Peak HBM of the plain PyTorch path: logits = x W^T, cross_entropy in fp32, backward."""
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    try:
        xr = x.detach().requires_grad_(True)
        Wr = W.detach().requires_grad_(True)
        loss = torch.nn.functional.cross_entropy((xr @ Wr.T).float(), t)
        loss.backward()
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        del xr, Wr, loss
        torch.cuda.empty_cache()
        return {"extra_gb": peak / 1e9, "status": "ok"}
    except torch.cuda.OutOfMemoryError:
        torch.cuda.empty_cache()
        return {"extra_gb": None, "status": "OOM"}


def hipblaslt_yardstick(x, W, rows: int, reps: int = 10):
    """torch.matmul (hipBLASLt) on one chunk's three products in the layouts the library uses:
    logits x_c W^T, dx G W and dW G^T x_c, with a random G of the chunk's shape; ms and TFLOP/s
    per product, 2 rows V H flops each (a reference point, not part of the step)."""
    import torch
    xc = x[:rows]
    g = torch.randn(rows, W.shape[0], device=x.device, dtype=x.dtype)
    fl = 2.0 * rows * W.shape[0] * W.shape[1]
    res = {}
    for name, fn in (("logits_lse", lambda: xc @ W.T), ("dx", lambda: g @ W), ("dw", lambda: g.T @ xc)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name] = {"avg_ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 1)}
    del g
    torch.cuda.synchronize()
    return res


def fused_record(flce, x, W, t, w, chunk, steps, ignore, reduction, grad_fp32=True):
    """The fused variant (two passes, logits recomputed) on the same inputs: ms per step, credited
    TFLOP/s (6 N H V) and executed (8 N H V: the recompute), peak extra HBM, per-kernel averages.
    fp32 gradients give its fastest form (one pass 2 over all tokens, atomics into dx and dW);
    bf16 gradients are the chunked line's own configuration (pass 2 per chunk, dW stored)."""
    import torch
    dev = x.device
    gdt = torch.float32 if grad_fp32 else x.dtype
    f = flce.FusedLinearCrossEntropy(in_dtype=x.dtype, dx_dtype=gdt, dw_dtype=gdt, variant=flce.FLCE_FUSED)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    dx = torch.empty(x.shape, dtype=gdt, device=dev)
    dW = torch.empty(W.shape, dtype=gdt, device=dev)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    f.reserve(w.N, w.H, w.V, chunk)
    ws = f.workspace_bytes(w.N, w.H, w.V, chunk)
    out = (loss, dx, dW, None)

    def step():
        f.forward_backward(x, W, t, chunk=chunk, out=out, reduction=reduction, ignore_index=ignore)
    step()
    torch.cuda.synchronize()
    f.profile_enable(True)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    stats = f.profile_read()
    peak_extra = torch.cuda.max_memory_allocated() - base + ws
    status = f.check()
    lval = loss.item()
    f.close()
    del dx, dW
    torch.cuda.empty_cache()
    if status != 0 or not math.isfinite(lval):
        raise SystemExit(f"fused bench run is invalid: status {status}, loss {lval}")
    fl = 6.0 * w.N * w.H * w.V
    kernels = {}
    for name, st in stats.items():
        avg = st["total_ms"] / max(st["launches"], 1)
        k = {"launches_per_step": st["launches"] / steps, "avg_ms": round(avg, 4)}
        if st["flops"] > 0:
            k["tflops_executed"] = round(st["flops"] / st["launches"] / (avg * 1e-3) / 1e12, 1)
        kernels[name] = k
    log(f"[bench] fused: {ms:.2f} ms/step, loss {lval:.6f}")
    fb = stats.get("fused_bwd")
    roof = None
    if fb and fb["launches"] > 0:
        avg_s = fb["total_ms"] / fb["launches"] * 1e-3
        ach = fb["flops"] / fb["launches"] / avg_s / 1e12      # executed: recompute + dx + dW products
        eff_chunk = flce.flce_effective_chunk(w.N, w.H, w.V, chunk)
        roof = {"bound": "mfma", "kernel": "fused_bwd", "achieved": round(ach, 1), "peak": PEAK_TFLOPS["bf16"],
                "unit": "TFLOP/s", "frac": round(ach / PEAK_TFLOPS["bf16"], 4),
                "traffic": measured_traffic("fused_bwd", w.name, eff_chunk),
                "flops_per_launch": fb["flops"] / fb["launches"], "avg_launch_ms": round(avg_s * 1e3, 4)}
    return {"variant": "fused", "grad_dtype": "fp32" if grad_fp32 else "bf16", "steps": steps, "warmup": 1,
            "ms_per_step": round(ms, 4),
            "tokens_per_s": round(w.N / (ms * 1e-3), 1),
            "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
            "mfma_peak_frac": round(fl / (ms * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"], 4),
            "tflops_executed": round(8.0 / 6.0 * fl / (ms * 1e-3) / 1e12, 1),
            "peak_extra_gb": round(peak_extra / 1e9, 3), "workspace_gb": round(ws / 1e9, 3),
            "loss": round(lval, 6), "kernels": kernels, "roofline": roof}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="llama3_vocab")
    ap.add_argument("--chunk", type=int, default=0, help="0 = the workload's chunk")
    ap.add_argument("--variant", choices=["chunked", "fused"], default="chunked")
    ap.add_argument("--grad-dtype", choices=["input", "fp32"], default="input",
                    help="dtype of dx and dW (default: the input dtype)")
    ap.add_argument("--forward-only", action="store_true",
                    help="loss only (flce_forward_backward_opt with FLCE_FORWARD_ONLY); credited 2NHV flops")
    ap.add_argument("--reduction", choices=["mean", "sum"], default="mean")
    ap.add_argument("--ignore-frac", type=float, default=0.0,
                    help="set this fraction of the targets (seeded) to -100 and pass ignore_index=-100")
    ap.add_argument("--accumulate", action="store_true", help="add the gradients into dx and dW")
    ap.add_argument("--rmsnorm", action="store_true",
                    help="RMSNorm in front of the head (flce_rmsnorm_forward_backward): the workload's x "
                         "becomes the hidden states, gamma ~ 1 + 0.2 N(0,1) (seeded), eps 1e-6")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-materialised", action="store_true",
                    help="skip the peak-HBM measurement of the materialised-logits PyTorch path")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the fused-variant sub-record (fp32 gradients) of a chunked run")
    ap.add_argument("--fused-steps", type=int, default=5)
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="GIB",
                    help="after the run, copy a buffer of this many GiB once (a plain copy kernel of "
                         "known traffic, to scale rocprofv3 FETCH_SIZE/WRITE_SIZE readings)")
    ap.add_argument("--yardstick", action="store_true",
                    help="also time torch.matmul (hipBLASLt) on the chunk's three products")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU sharding "
              f"of this path is a design, not a built component.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import linear_cross_entropy_token_amd as flce
    from flce_inputs import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    w = WORKLOADS[args.workload]
    chunk = args.chunk or w.chunk
    dev = torch.device("cuda:0")
    log(f"[bench] generating {w.name}: N={w.N} H={w.H} V={w.V} {w.dtype}")
    t0 = time.perf_counter()
    d = make_inputs(w.N, w.H, w.V, w.dtype, w.seed, w.targets)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    if w.dtype == "bf16":
        x = torch.from_numpy(d["x"].view(np.int16)).view(torch.bfloat16).to(dev)
        W = torch.from_numpy(d["W"].view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        x = torch.from_numpy(d["x"]).to(dev)
        W = torch.from_numpy(d["W"]).to(dev)
    if args.ignore_frac > 0:
        rng = np.random.default_rng(w.seed + 7919)
        d["t"] = np.where(rng.random(w.N) < args.ignore_frac, -100, d["t"])
    t = torch.from_numpy(d["t"]).to(dev)
    del d
    ignore = -100 if args.ignore_frac > 0 else None
    if args.forward_only and args.accumulate:
        raise SystemExit("--forward-only and --accumulate exclude each other")
    gamma = None
    if args.rmsnorm:
        g32 = (1.0 + 0.2 * np.random.default_rng(w.seed + 104729).standard_normal(w.H)).astype(np.float32)
        gamma = torch.from_numpy(g32).to(dev).to(x.dtype)
    log(f"[bench] inputs on device in {time.perf_counter() - t0:.1f} s")

    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    variant = flce.FLCE_FUSED if args.variant == "fused" else flce.FLCE_CHUNKED
    gdt = torch.float32 if args.grad_dtype == "fp32" else tdt
    f = flce.FusedLinearCrossEntropy(in_dtype=tdt, dx_dtype=gdt, dw_dtype=gdt, variant=variant)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    dx = torch.empty(x.shape, dtype=gdt, device=dev)
    dW = torch.empty(W.shape, dtype=gdt, device=dev)
    dgamma = torch.empty((w.H,), dtype=gdt, device=dev) if args.rmsnorm else None
    base_alloc = torch.cuda.memory_allocated()
    free0, _ = torch.cuda.mem_get_info()
    if not args.forward_only and not args.rmsnorm:   # the other calls size their workspace themselves
        f.reserve(w.N, w.H, w.V, chunk)
    free1, total_mem = torch.cuda.mem_get_info()
    if args.rmsnorm:
        ws_bytes = flce.flce_rmsnorm_workspace_bytes(
            f.handle, w.N, w.H, w.V, chunk,
            flce._options(args.reduction, None, flce.FLCE_FORWARD_ONLY if args.forward_only else 0))
    else:
        ws_bytes = f.workspace_bytes(w.N, w.H, w.V, chunk, forward_only=args.forward_only)
    eff_chunk = flce.flce_effective_chunk(w.N, w.H, w.V, chunk)

    out = (loss, dx, dW, None)
    stream = torch.cuda.current_stream(dev)
    if args.accumulate:
        dx.zero_()
        dW.zero_()

    def step():
        if args.rmsnorm:
            if args.forward_only:
                return f.rmsnorm_forward(x, gamma, W, t, eps=1e-6, chunk=chunk, reduction=args.reduction,
                                         ignore_index=ignore)
            return f.rmsnorm_forward_backward(x, gamma, W, t, eps=1e-6, chunk=chunk,
                                              out=(loss, dx, dgamma, dW, None), reduction=args.reduction,
                                              ignore_index=ignore, accumulate=args.accumulate)
        if args.forward_only:
            return f.forward(x, W, t, chunk=chunk, reduction=args.reduction, ignore_index=ignore)
        return f.forward_backward(x, W, t, chunk=chunk, out=out, reduction=args.reduction, ignore_index=ignore,
                                  accumulate=args.accumulate)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    f.profile_enable(True)
    # one event between consecutive steps (recorded on the stream, no host synchronisation)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(args.steps):
        res = step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    step_ms = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    stats = f.profile_read()
    f.profile_enable(False)
    if args.forward_only:
        loss = res
    peak_extra = torch.cuda.max_memory_allocated() - base_alloc + ws_bytes
    status = f.check()
    log(f"[bench] {ms:.3f} ms/step, loss {loss.item():.6f}, check status {status}")
    if status != 0 or not math.isfinite(loss.item()):
        raise SystemExit(f"bench run is invalid: status {status}, loss {loss.item()}")

    flops_step = (2.0 if args.forward_only else 6.0) * w.N * w.H * w.V
    tflops = flops_step / (ms * 1e-3) / 1e12
    peak_tf = PEAK_TFLOPS[w.dtype]
    kernels = {}
    for name, s in stats.items():
        avg = s["total_ms"] / max(s["launches"], 1)
        k = {"launches_per_step": s["launches"] / args.steps, "avg_ms": round(avg, 4),
             "ms_per_step": round(s["total_ms"] / args.steps, 4),
             "share": round(s["total_ms"] / args.steps / ms, 4)}
        if s["flops"] > 0:
            k["tflops"] = round(s["flops"] / s["launches"] / (avg * 1e-3) / 1e12, 1)
            if s.get("sclk_mhz"):
                k["sclk_mhz"] = round(s["sclk_mhz"], 1)
        elif s["bytes"] > 0:
            k["gbs"] = round(s["bytes"] / s["launches"] / (avg * 1e-3) / 1e9, 1)
        kernels[name] = k
    gemms = {n: s for n, s in stats.items() if s["flops"] > 0}
    dom = max(gemms, key=lambda n: gemms[n]["total_ms"])
    ds = gemms[dom]
    avg_s = ds["total_ms"] / ds["launches"] * 1e-3
    achieved = ds["flops"] / ds["launches"] / avg_s / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1), "peak": peak_tf,
                "unit": "TFLOP/s", "frac": round(achieved / peak_tf, 4),
                "traffic": measured_traffic(dom, w.name, eff_chunk),
                "flops_per_launch": ds["flops"] / ds["launches"],
                "avg_launch_ms": round(avg_s * 1e3, 4)}
    if ds.get("sclk_mhz"):
        # the same peak scaled to the shader clock the kernel's workgroups ran at (s_memtime
        # against the 100 MHz real-time counter, summed over its workgroups)
        roofline["observed_sclk_mhz"] = round(ds["sclk_mhz"], 1)
        roofline["frac_at_observed_sclk"] = round(achieved / (peak_tf * ds["sclk_mhz"] / PEAK_SCLK_MHZ), 4)

    extra = {"peak_extra_gb": round(peak_extra / 1e9, 3), "peak_extra_gib": round(peak_extra / 2**30, 3),
             "dx_dtype": str(gdt).replace("torch.", ""), "dw_dtype": str(gdt).replace("torch.", ""),
             "workspace_gb": round(ws_bytes / 1e9, 3),
             "free_delta_gb": round((free0 - free1) / 1e9, 3),
             "materialised_fp32_logits_gb": round(w.N * w.V * 4 / 1e9, 2)}
    f.close()
    del dx, dW, dgamma, out
    torch.cuda.empty_cache()
    fused = None
    if args.variant == "chunked" and not args.no_fused and not (args.forward_only or args.rmsnorm or
                                                               args.accumulate or w.dtype != "bf16"):
        log(f"[bench] fused variant, fp32 gradients: {args.fused_steps} timed steps")
        fused = fused_record(flce, x, W, t, w, chunk, args.fused_steps, ignore, args.reduction)
        log(f"[bench] fused variant, bf16 gradients: {args.fused_steps} timed steps")
        fb = fused_record(flce, x, W, t, w, chunk, args.fused_steps, ignore, args.reduction, grad_fp32=False)
        fused["bf16_grads"] = {k: fb[k] for k in ("ms_per_step", "tokens_per_s", "tflops", "mfma_peak_frac",
                                                   "peak_extra_gb", "workspace_gb", "loss")}
    if not args.no_materialised:
        log("[bench] peak HBM of the materialised-logits PyTorch loss")
        extra["materialised_baseline"] = materialised_peak(x, W, t)

    if args.copy_calibration > 0:
        n = int(args.copy_calibration * (1 << 30)) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        extra["copy_calibration_bytes"] = n * 4
        del src, dst

    yard = None
    if args.yardstick:
        log("[bench] timing torch.matmul on the chunk's three products")
        yard = hipblaslt_yardstick(x, W, eff_chunk)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(w)

    rec = {
        "metric": METRIC, "value": round(w.N / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "step_ms": {"median": round(step_ms[len(step_ms) // 2] if len(step_ms) % 2
                                    else 0.5 * (step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2]), 4),
                    "min": round(step_ms[0], 4), "max": round(step_ms[-1], 4)},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded x~N(0,1), W~N(0,0.02^2), targets "
                + ("Zipf(1.1)" if w.targets == "zipf" else "uniform") + ")",
        "config": {"workload": f"{w.name}: N={w.N} H={w.H} V={w.V} {w.dtype}, chunk {eff_chunk}",
                   "N": w.N, "H": w.H, "V": w.V, "chunk": eff_chunk, "variant": args.variant,
                   "grad_dtype": "fp32" if args.grad_dtype == "fp32" else w.dtype,
                   "mode": "forward" if args.forward_only else "forward+backward",
                   "reduction": args.reduction, "ignore_frac": args.ignore_frac,
                   "accumulate": args.accumulate, "rmsnorm": args.rmsnorm, "parallelism": "single GPU"},
        "tflops": round(tflops, 1), "mfma_peak_frac": round(tflops / peak_tf, 4),
        "memory": extra, "kernels": kernels, "roofline": roofline, "cpu_baseline": cpu,
    }
    if fused is not None:
        rec["fused_variant"] = fused
    if yard is not None:
        rec["yardstick_hipblaslt"] = yard
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
