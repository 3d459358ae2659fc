"""Benchmark: attention TFLOP/s of the HIP path on one MI355X.

One step is one ``vitattn_fwd`` call (the whole hot path: work planning, K/V
staging, both MFMA products, online softmax and the epilogue) over one batch of
seeded synthetic input.  The headline workload is the packed variable-length
batch (8 images, 17,408 tokens, 16 heads of 80, bf16); the 912-patch page
(16 heads of 80, bf16), also named by the metric, is timed beside it.  FLOPs are
4 * sum_s L_s^2 * D * H with the true head_dim.  Inputs are resident in HBM before
the timed region starts.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 (and f16) MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
FP32_PEAK_TFLOPS = 157.3   # MI355X dense fp32
HEADLINE = "packed-varlen-8"
SECONDARY = "page-912"
PROFILES = os.path.join(ROOT, "profiles")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def visible_pairs(lengths, causal: bool, window: int) -> int:
    """(query, key) pairs a mask keeps, summed over the sequences (all L^2 without one)."""
    import numpy as np
    total = 0
    for n in lengths:
        i = np.arange(int(n), dtype=np.int64)
        lo = np.maximum(0, i - window + 1) if window > 0 else np.zeros_like(i)
        hi = np.full_like(i, int(n) - 1)
        if window > 0:
            hi = np.minimum(hi, i + window - 1)
        if causal:
            hi = np.minimum(hi, i)
        total += int(np.sum(hi - lo + 1))
    return total


def time_workload(name: str, steps: int, warmup: int, out_f32: bool = False, causal: bool = False,
                  window: int = 0):
    import torch

    import vision_transformer_attention_amd as vta
    from vision_transformer_attention_amd import inputs

    w = inputs.WORKLOADS[name]
    q, k, v, cu, scale = inputs.make(w)
    dev = torch.device("cuda:0")
    q, k, v, cu = q.to(dev), k.to(dev), v.to(dev), cu.to(dev)
    out = torch.empty(q.shape, dtype=torch.float32 if out_f32 else q.dtype, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(warmup):
        vta.fwd(q, k, v, cu, scale, out=out, check_cu=False, causal=causal, window=window)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        vta.fwd(q, k, v, cu, scale, out=out, check_cu=False, causal=causal, window=window)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = start.elapsed_time(end) / steps  # events on the launch stream
    cfg = vta.binding.kernel_config(w.head_dim, q.dtype)
    return w, kernel_ms, wall * 1e3 / steps, cfg


HBM_PEAK_GBS = 8000.0  # MI355X HBM3E


def time_prologue(name: str, steps: int, warmup: int):
    """The qkv prologue (split + per-head RMS norm + rope) on the workload's token count and
    heads; returns (seconds per launch, algorithmic bytes per launch)."""
    import torch

    import vision_transformer_attention_amd as vta
    from vision_transformer_attention_amd import inputs

    w = inputs.WORKLOADS[name]
    d = inputs.prologue_inputs(w.lengths, w.n_heads, w.head_dim, w.dtype, seed=w.seed + 100, n_kv_heads=w.n_kv_heads)
    dev = torch.device("cuda:0")
    mv = lambda x: x.to(dev) if x is not None else None
    args = (mv(d["qkv"]), d["n_heads"], d["n_kv_heads"], mv(d["cos"]), mv(d["sin"]), mv(d["q_weight"]),
            mv(d["k_weight"]))
    out = vta.qkv_prologue(*args)
    for _ in range(warmup):
        vta.qkv_prologue(*args, out=out)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream(dev)
    start.record(stream)
    for _ in range(steps):
        vta.qkv_prologue(*args, out=out)
    end.record(stream)
    torch.cuda.synchronize()
    sec = start.elapsed_time(end) / steps * 1e-3
    es = d["qkv"].element_size()
    t = d["qkv"].shape[0]
    nbytes = 2 * d["qkv"].numel() * es + 2 * t * w.head_dim * 4 + 2 * w.head_dim * 4
    return w, sec, nbytes


def cpu_baseline(name: str, target_s: float = 12.0):
    """The float64 oracle timed on the host's cores on a bounded sample of query rows."""
    import numpy as np

    import oracle
    from vision_transformer_attention_amd import inputs

    w = inputs.WORKLOADS[name]
    q, k, v, cu, scale = inputs.make(w)
    cu_np = cu.numpy()
    lens = np.diff(cu_np)
    seq_of = np.repeat(np.arange(len(lens)), lens)
    rng = np.random.default_rng(123)

    def run(n_rows):
        rows = np.sort(rng.choice(w.total_tokens, size=n_rows, replace=False)).astype(np.int64)
        flops = float(np.sum(4.0 * lens[seq_of[rows]] * w.head_dim * w.n_heads))
        t0 = time.perf_counter()
        oracle.attention_rows(q, k, v, cu, scale, rows)
        return time.perf_counter() - t0, flops, n_rows

    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    run(16)  # warms the oracle's threads and caches
    dt, fl, n = run(128)  # the per-row time of a short pilot sizes the sample
    per_row = max(dt / n, 1e-6)
    n_rows = int(min(w.total_tokens, max(16, target_s / per_row)))
    dt, fl, n = run(n_rows)
    return {
        "value": fl / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.threads(),
        "cpu_model": model,
        "kind": "oracle",
        "sample": f"{n} of {w.total_tokens} query rows of {name} (all {w.n_heads} heads, every key of each row's "
                  f"image), float64, {dt:.1f} s",
    }


def load_traffic(name: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary, or None
    when there is none for this workload or the kernel source changed since it was taken."""
    import hashlib

    path = os.path.join(PROFILES, f"attn_fwd_bf16_d80_{name}_hbm_traffic.json")
    src = os.path.join(ROOT, "vision_transformer_attention_amd", "csrc", "vitattn.hip")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(src, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
        if rec.get("source_sha256") != sha:
            return None
        return rec.get("bytes_per_launch")
    except Exception:
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-secondary", action="store_true", help="time only --workload (for profiling runs)")
    ap.add_argument("--out-dtype", choices=("same", "f32"), default="same",
                    help="output element type: the input's, or float32 (16-bit inputs only)")
    ap.add_argument("--causal", action="store_true", help="aligned causal mask inside each image")
    ap.add_argument("--window", type=int, default=0, help="key window |qi - kj| < W (0: none)")
    ap.add_argument("--prologue", action="store_true",
                    help="time the qkv prologue (split, per-head RMS norm, rope) instead of the attention")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device-to-device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the attention path here is a "
              f"single-GPU build, see DESIGN.md for how it would shard.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.prologue:
        w, sec, nbytes = time_prologue(args.workload, args.steps, args.warmup)
        gbs = nbytes / sec / 1e9
        log(f"[bench] prologue {args.workload}: {sec * 1e6:.1f} us/launch, {gbs:.0f} GB/s")
        print(json.dumps({
            "metric": "qkv prologue GB/s (packed qkv read once, Q/K/V written once, rope tables read once)",
            "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": sec * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": w.dtype, "data": "synthetic (seeded N(0,1) projection output, 2-D rope tables)",
            "config": {"workload": w.name, "tokens": w.total_tokens, "heads": w.n_heads, "kv_heads": w.kv_heads,
                       "head_dim": w.head_dim, "bytes_per_step": nbytes, "rope": True, "norm": True},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None},
        }), flush=True)
        return
    log(f"[bench] timing {args.workload}: warmup {args.warmup}, steps {args.steps}")
    masked = args.causal or args.window > 0
    w, kernel_ms, wall_ms, cfg = time_workload(args.workload, args.steps, args.warmup, args.out_dtype == "f32",
                                               args.causal, args.window)
    # algorithmic FLOPs: 4*D*H per (query, key) pair the mask keeps
    flops = (4.0 * w.head_dim * w.n_heads * visible_pairs(w.lengths, args.causal, args.window)) if masked else w.flops
    tflops = flops / (kernel_ms * 1e-3) / 1e12
    log(f"[bench] {args.workload}: {kernel_ms * 1e3:.1f} us/launch, {tflops:.1f} TFLOP/s")
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {args.copy_calibration_mib} MiB read + written once")
        del src, dst
    sec = None
    if args.workload != SECONDARY and not args.no_secondary and not masked:
        log(f"[bench] timing {SECONDARY}")
        w2, k2, wall2, cfg2 = time_workload(SECONDARY, max(args.steps, 200), args.warmup)
        sec = {"workload": SECONDARY, "value": w2.flops / (k2 * 1e-3) / 1e12, "unit": "TFLOP/s",
               "ms_per_step": k2, "frac_of_bf16_peak": w2.flops / (k2 * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}
        log(f"[bench] {SECONDARY}: {k2 * 1e3:.1f} us/launch, {sec['value']:.1f} TFLOP/s")
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the float64 oracle on the host cores (bounded sample)")
        cpu = cpu_baseline(args.workload)
        log(f"[bench] oracle: {cpu['value'] * 1e3:.3f} GFLOP/s on {cpu['cores']} threads")
    dtype = w.dtype  # the element type the products are computed in: "bf16", "f16" or "f32"
    peak = FP32_PEAK_TFLOPS if w.dtype == "f32" else BF16_PEAK_TFLOPS  # dense f16 MFMA = dense bf16
    rec = {
        "metric": "attention TFLOP/s (4*S^2*D*H summed over sequences)",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": kernel_ms,
        "wall_ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,1) inputs of the workload's shape)",
        "config": {
            "workload": w.name, "lengths": list(w.lengths), "tokens": w.total_tokens, "heads": w.n_heads,
            "head_dim": w.head_dim, "kv_heads": w.kv_heads, "out_dtype": "f32" if args.out_dtype == "f32" else w.dtype,
            "causal": bool(args.causal), "window": args.window,
            "caches": "warm: inputs resident in HBM, launches back to back on one stream",
            "flops_per_step": flops, "block_m": None if masked else cfg["block_m"],
            "block_n": cfg["block_n"], "waves_per_workgroup": cfg["waves"], "grid": cfg["grid"],
        },
        "roofline": {
            "bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s",
            "frac": tflops / peak,
            "traffic": load_traffic(w.name) if args.out_dtype == "same" and not masked else None,
        },
        "secondary": sec,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
