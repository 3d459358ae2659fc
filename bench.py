"""Benchmark: attention TFLOP/s of the HIP path on one MI355X.

One step is one attention call (the whole hot path: work planning, K/V staging, both
MFMA products, online softmax and the epilogue) over one batch of seeded synthetic
input.  The headline workload is the packed variable-length batch (8 images, 17,408
tokens, 16 heads of 80, bf16); every other workload of the metric's family is timed
beside it in ``configs``: the tiny float32 case, the 196-patch ViT image, the 912-patch
page and the 16,384-token sequence.  The three small ones are also replayed from a HIP
graph of 50 captured calls, since their eager launches are bound by the host's enqueue
time (``graph_replay_ms_per_step``).  FLOPs are 4 * sum_s L_s^2 * D * H with the true head_dim.
Inputs are resident in HBM before any timed region starts.

Timing per workload: one call for the library's one-time device set-up, then ``--warmup``
launches timed as a block (the cold figure, reported as ``cold_ms_per_step``), then untimed
launches until ``--settle-ms`` of device time has passed
(the GPU needs about 30 ms of work to reach its steady clock), then exactly ``--steps``
launches between two HIP events on the launch stream.

The CPU leg times the float64 oracle on the host's cores (all of them, then one) on a
bounded sample of the headline workload, and compares each workload's GPU output with
the oracle on a bounded set of rows (``max_abs_err`` in ``configs``).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
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

METRIC = "attention TFLOP/s (4*S^2*D*H) at S=912,D=80 and packed varlen; % bf16 MFMA peak"
BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 (and f16) MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
FP32_PEAK_TFLOPS = 157.3   # MI355X dense fp32
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
PEAK_CLOCK_GHZ = 2.4       # the engine clock of the peak figures
HEADLINE = "packed-varlen-8"
FAMILY = ("tiny-64", "vit-196", "page-912", "packed-varlen-8", "long-16384")
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "vision_transformer_attention_amd", "csrc", "vitattn.hip")
# rows of each workload the oracle recomputes for max_abs_err (None: every row)
ERR_ROWS = {"tiny-64": None, "vit-196": None, "page-912": None, "packed-varlen-8": 2048, "long-16384": 192}
TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 1e-2}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def peak_of(dtype: str) -> float:
    return FP32_PEAK_TFLOPS if dtype == "f32" else BF16_PEAK_TFLOPS  # dense f16 MFMA = dense bf16


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


def timed_launches(call, steps: int, warmup: int, settle_ms: float):
    """(cold ms per launch over the warm-up, settle ms actually run, ms per launch over `steps`)."""
    import torch
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    call()  # the library's one-time device set-up happens outside every timed region
    torch.cuda.synchronize()
    cold = None
    if warmup > 0:
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(warmup):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        cold = a.elapsed_time(b) / warmup
    settled = 0.0
    while settled < settle_ms:  # untimed: until the device has worked settle_ms
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(20):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        settled += a.elapsed_time(b)
    start, end = ev(), ev()
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        call()
    end.record(stream)
    torch.cuda.synchronize()
    return cold, settled, start.elapsed_time(end) / steps


def graph_replay_ms(call, per_graph: int = 50, replays: int = 20) -> float:
    """ms per call when `per_graph` calls are captured into one HIP graph and replayed."""
    import torch
    call()  # device set-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            call()
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(replays):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (replays * per_graph)


def attention_case(name: str, out_f32: bool = False, causal: bool = False, window: int = 0):
    """Device inputs for a workload and a zero-argument call of the binding on them."""
    import torch

    import vision_transformer_attention_amd as vta
    from vision_transformer_attention_amd import inputs

    w = inputs.WORKLOADS[name]
    q, k, v, cu, scale = inputs.make(w)
    dev = torch.device("cuda:0")
    qd, kd, vd, cud = q.to(dev), k.to(dev), v.to(dev), cu.to(dev)
    out = torch.empty(q.shape, dtype=torch.float32 if out_f32 else q.dtype, device=dev)

    def call():
        vta.fwd(qd, kd, vd, cud, scale, out=out, causal=causal, window=window)

    return w, (q, k, v, cu, scale), out, call


def time_workload(name: str, steps: int, warmup: int, settle_ms: float, graph: bool = False, **kw):
    w, host, out, call = attention_case(name, **kw)
    cold, settled, ms = timed_launches(call, steps, warmup, settle_ms)
    rec = {"workload": name, "ms_per_step": ms, "cold_ms_per_step": cold, "settle_ms": settled, "steps": steps}
    if graph:
        rec["graph_replay_ms_per_step"] = graph_replay_ms(call)
    return w, host, out, rec


def time_prologue(name: str, steps: int, warmup: int, settle_ms: float):
    """The qkv prologue (split + per-head RMS norm + rope) on the workload's token count and
    heads; returns (workload, ms per launch, algorithmic bytes per launch)."""
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
    _, _, ms = timed_launches(lambda: vta.qkv_prologue(*args, out=out), steps, warmup, settle_ms)
    es = d["qkv"].element_size()
    t = d["qkv"].shape[0]
    nbytes = 2 * d["qkv"].numel() * es + 2 * t * w.head_dim * 4 + 2 * w.head_dim * 4
    return w, ms, nbytes


def kernel_sha() -> str:
    """Fingerprint of the kernel binary's inputs: the HIP source and the hipcc flags."""
    import __graft_entry__
    h = hashlib.sha256()
    with open(KERNEL_SRC, "rb") as f:
        h.update(f.read())
    h.update(" ".join(__graft_entry__.HIP_FLAGS).encode())
    return h.hexdigest()


def committed_counters(name: str):
    """The committed rocprofv3 counter summary of this workload's attention kernel, when it was
    taken on the current kernel source (else None): MFMA-busy fraction and HBM bytes per launch."""
    path = os.path.join(PROFILES, f"attn_fwd_{name}_counters.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_sha():
        return None
    return rec


# The rocprofv3 runs behind profiles/attn_fwd_<workload>.md, run from the repository root (one
# process each): a kernel trace of the timed bench command, then counter passes of the same
# command with 20 timed launches (the same warm-up and settle before them), the last two with a
# plain copy of known size after the attention launches to calibrate the HBM byte counters.
PMC_PASSES = {
    "p1": ["SQ_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU",
           "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT"],
    "p2": ["SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_WAIT_INST_LDS", "SQ_WAIT_ANY",
           "SQ_INSTS_VALU_TRANS_F32", "SQ_INST_LEVEL_LDS", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_ANY"],
    "p3": ["FETCH_SIZE"],
    "p4": ["WRITE_SIZE"],
}
COPY_MIB = 256


def profile_commands(name: str, out: str = "gpurun_out/prof") -> list:
    """Shell commands (repository root as working directory) that write the raw rocprofv3 output
    that --summarize-profiles reads: <out>/<workload>/<run>/run_*.csv and <out>/<workload>/<run>.json."""
    base = f"python3 bench.py --workload {name} --no-secondary --no-cpu-baseline"
    short = f"{base} --steps 20"  # the same warm-up and settle as the trace run, fewer timed launches
    d = f"{out}/{name}"
    cmds = [f"mkdir -p {d}",
            f"TMPDIR=/tmp timeout -s KILL 300 rocprofv3 --kernel-trace --stats --output-format csv -d {d}/kt -o run "
            f"-- {base} > {d}/kt.json"]
    for run, ctrs in PMC_PASSES.items():
        extra = f" --copy-calibration-mib {COPY_MIB}" if run in ("p3", "p4") else ""
        cmds.append(f"TMPDIR=/tmp timeout -s KILL 300 rocprofv3 --pmc {' '.join(ctrs)} --output-format csv "
                    f"-d {d}/{run} -o run -- {short}{extra} > {d}/{run}.json")
    return cmds


def _read_csv(path: str) -> list:
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def summarize_profiles(root: str, name: str, out_dir: str = PROFILES) -> dict:
    """Reads the rocprofv3 output of profile_commands(name) under `root` and writes
    profiles/attn_fwd_<name>_counters.json and profiles/attn_fwd_<name>.md.  The averages are
    over the timed launches only (the last `steps` attention dispatches of each run)."""
    import statistics

    from vision_transformer_attention_amd import inputs

    w = inputs.WORKLOADS[name]
    d = os.path.join(root, name)
    is_attn = lambda r: "attn_fwd" in r["Kernel_Name"]
    def bench_line(run):  # the JSON line that run's bench.py printed (its last line)
        with open(os.path.join(d, f"{run}.json")) as f:
            return json.loads(f.read().strip().splitlines()[-1])

    bench = {run: bench_line(run) for run in ["kt", *PMC_PASSES]}
    agent = next(r for r in _read_csv(os.path.join(d, "kt", "run_agent_info.csv")) if r["Agent_Type"] == "GPU")
    n_simd, n_se = int(agent["Simd_Count"]), int(agent["Array_Count"])

    # kernel trace: the timed launches are the last `steps` dispatches of the attention kernel
    kt = sorted((r for r in _read_csv(os.path.join(d, "kt", "run_kernel_trace.csv")) if is_attn(r)),
                key=lambda r: int(r["Dispatch_Id"]))
    steps = bench["kt"]["steps"]
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in kt]
    timed = durs[-steps:]
    trace = {"dispatches": len(durs), "timed": len(timed), "mean_us": statistics.fmean(timed),
             "min_us": min(timed), "max_us": max(timed), "all_mean_us": statistics.fmean(durs),
             "kernel": kt[-1]["Kernel_Name"], "bench_us": bench["kt"]["ms_per_step"] * 1e3,
             "bench_cold_us": (bench["kt"].get("cold_ms_per_step") or 0.0) * 1e3}
    stats_rows = _read_csv(os.path.join(d, "kt", "run_kernel_stats.csv"))

    # counter passes: per-dispatch values of the last `steps` attention dispatches
    ctr, spread, dur_ns, calib = {}, {}, {}, {}
    for run, names in PMC_PASSES.items():
        rows = _read_csv(os.path.join(d, run, "run_counter_collection.csv"))
        by = {}
        for r in rows:
            by.setdefault(int(r["Dispatch_Id"]), []).append(r)
        ids = sorted(i for i, rs in by.items() if is_attn(rs[0]))
        n = bench[run]["steps"]
        use = ids[-n:]
        for c in names:
            vals = [sum(float(r["Counter_Value"]) for r in by[i] if r["Counter_Name"] == c) for i in use]
            ctr[c] = statistics.fmean(vals)
            spread[c] = (min(vals), max(vals))
        dur_ns[run] = statistics.fmean(int(by[i][0]["End_Timestamp"]) - int(by[i][0]["Start_Timestamp"]) for i in use)
        if run in ("p3", "p4"):  # the copy dispatches after the last attention launch
            copies = [i for i in by if i > ids[-1] and "copy" in by[i][0]["Kernel_Name"].lower()]
            calib[names[0]] = (sum(float(r["Counter_Value"]) for i in copies for r in by[i]
                                   if r["Counter_Name"] == names[0]), len(copies), by[copies[0]][0]["Kernel_Name"])
    copy_kib = COPY_MIB * 1024.0
    f_scale = copy_kib / calib["FETCH_SIZE"][0]
    w_scale = copy_kib / calib["WRITE_SIZE"][0]
    rd = ctr["FETCH_SIZE"] * f_scale * 1024.0
    wr = ctr["WRITE_SIZE"] * w_scale * 1024.0
    es = 4 if w.dtype == "f32" else 2
    q_rows = w.total_tokens * w.n_heads * w.head_dim
    kv_rows = w.total_tokens * w.kv_heads * w.head_dim
    alg = (2 * q_rows + 2 * kv_rows) * es
    clock_ghz = ctr["SQ_CYCLES"] / n_se / dur_ns["p1"]
    # busy cycles of the matrix pipes over the counter run's own dispatch time at the 2.4 GHz of
    # the peak figures (a lower bound on the fraction when the clock ran lower)
    mfma_busy = ctr["SQ_VALU_MFMA_BUSY_CYCLES"] / (n_simd * dur_ns["p1"] * PEAK_CLOCK_GHZ)
    rec = {
        "kernel": trace["kernel"], "workload": name, "source_sha256": kernel_sha(),
        "trace_mean_us": trace["mean_us"], "trace": trace,
        "counters_mean_per_dispatch": ctr,
        "hbm_bytes_per_launch": rd + wr, "hbm_read_bytes": rd, "hbm_write_bytes": wr,
        "algorithmic_bytes": alg, "fetch_scale": f_scale, "write_scale": w_scale,
        "hbm_gbs": (rd + wr) / (trace["mean_us"] * 1e3),
        "mfma_busy": mfma_busy, "counter_run_clock_ghz": clock_ghz,
        "lds_conflict_cycles_per_lds_inst": ctr["SQ_LDS_BANK_CONFLICT"] / ctr["SQ_INSTS_LDS"],
        "valu_per_mfma": ctr["SQ_INSTS_VALU"] / ctr["SQ_INSTS_MFMA"],
        "profile": f"attn_fwd_{name}.md",
    }
    with open(os.path.join(out_dir, f"attn_fwd_{name}_counters.json"), "w") as f:
        json.dump(rec, f, indent=1)

    tf = w.flops / (trace["mean_us"] * 1e-6) / 1e12
    lines = [
        f"# Attention kernel on {name} ({len(w.lengths)} sequence(s), {w.total_tokens:,} tokens, {w.n_heads} heads "
        f"of {w.head_dim}, {w.dtype})", "",
        f"Kernel fingerprint (sha256 of the HIP source and the hipcc flags): `{rec['source_sha256']}`", "",
        "## Commands (repository root, one MI355X; written by `bench.py --profile-commands "
        f"{name}`, summarised by `bench.py --summarize-profiles gpurun_out/prof --workload {name}`)", "", "```",
        *profile_commands(name), "```", "",
        "## Kernel trace (`kt`)", "",
        f"Kernel: `{trace['kernel']}`", "",
        f"- {trace['dispatches']} dispatches (one set-up call, {bench['kt']['warmup']} cold warm-up launches, "
        f"the settle launches, {steps} timed launches).",
        f"- Timed launches: mean {trace['mean_us']:.2f} us (min {trace['min_us']:.2f}, max {trace['max_us']:.2f}), "
        f"{tf:.1f} TFLOP/s, {tf / peak_of(w.dtype):.1%} of the dense peak.",
        f"- bench.py in the same profiled run: {trace['bench_us']:.2f} us per launch (HIP events around the "
        f"timed launches); cold warm-up {trace['bench_cold_us']:.2f} us per launch.",
        f"- Mean over every dispatch of the run: {trace['all_mean_us']:.2f} us.", "",
        "`--stats` rows:", "", "```",
        *[f"{r['Name'][:90]}: calls {r['Calls']}, average {float(r['AverageNs']) / 1e3:.2f} us, "
          f"min {float(r['MinNs']) / 1e3:.2f}, max {float(r['MaxNs']) / 1e3:.2f}" for r in stats_rows],
        "```", "",
        f"## Counters (mean per timed dispatch of the counter runs: last {bench['p1']['steps']} of each)", "",
        f"Counter runs serialise dispatches; their mean dispatch took {dur_ns['p1'] / 1e3:.2f} us in pass p1"
        + (f", and SQ_CYCLES / ({n_se} shader arrays x duration) puts the shader clock at {clock_ghz:.2f} GHz"
           if dur_ns["p1"] > 1e5 else " (too short for a clock estimate from SQ_CYCLES, which then also counts "
           "cycles outside the dispatch)")
        + ".  The instruction, byte and conflict counts do not depend on the clock.", "",
        "| counter | mean | min | max |", "|---|---|---|---|",
        *[f"| {c} | {v:,.0f} | {spread[c][0]:,.0f} | {spread[c][1]:,.0f} |" for c, v in sorted(ctr.items())], "",
        "## HBM traffic", "",
        f"Calibration: one {COPY_MIB} MiB device-to-device copy after the attention launches "
        f"({calib['FETCH_SIZE'][1]} dispatch(es) of `{calib['FETCH_SIZE'][2][:60]}`) reads FETCH_SIZE "
        f"{calib['FETCH_SIZE'][0]:,.1f} KiB and WRITE_SIZE {calib['WRITE_SIZE'][0]:,.1f} KiB in total against "
        f"{copy_kib:,.0f} KiB moved each way: scale factors {f_scale:.4f} (fetch) and {w_scale:.4f} (write).", "",
        f"Per attention launch: {rd / 1e6:.1f} MB read + {wr / 1e6:.1f} MB written = {(rd + wr) / 1e6:.1f} MB "
        f"against {alg / 1e6:.1f} MB of algorithmic bytes (Q, K, V read once, O written once): "
        f"{(rd + wr) / alg:.2f}x; {rec['hbm_gbs']:.0f} GB/s over the trace mean "
        f"({rec['hbm_gbs'] / HBM_PEAK_GBS:.1%} of {HBM_PEAK_GBS:.0f}).", "",
        "## Derived", "",
        f"- MFMA busy: SQ_VALU_MFMA_BUSY_CYCLES / ({n_simd} SIMDs x {dur_ns['p1'] / 1e3:.2f} us x "
        f"{PEAK_CLOCK_GHZ} GHz) = {mfma_busy:.1%} (the pipes' busy share of the dispatch).",
        f"- VALU instructions per MFMA instruction: {rec['valu_per_mfma']:.2f}; transcendental (exp2) "
        f"{ctr['SQ_INSTS_VALU_TRANS_F32']:,.0f} per dispatch.",
        f"- LDS bank-conflict cycles per LDS instruction: {rec['lds_conflict_cycles_per_lds_inst']:.3f}.",
        f"- VALU/MFMA co-issue: SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES = "
        f"{ctr['SQ_VALU_MFMA_COEXEC_CYCLES'] / ctr['SQ_VALU_MFMA_BUSY_CYCLES']:.1%}.",
        "",
    ]
    with open(os.path.join(out_dir, f"attn_fwd_{name}.md"), "w") as f:
        f.write("\n".join(lines))
    return rec


def cpu_leg(name: str, gpu_outputs: dict, target_s: float = 10.0, one_core_s: float = 8.0):
    """The float64 oracle: timed on the host cores (all, then one) on a bounded sample of the
    headline workload's query rows, and compared with each workload's GPU output on a bounded
    set of rows.  Returns (cpu_baseline record, {workload: error record})."""
    import numpy as np

    import oracle
    from vision_transformer_attention_amd import inputs

    w = inputs.WORKLOADS[name]
    q, k, v, cu, scale = inputs.make(w)
    lens = np.diff(cu.numpy())
    seq_of = np.repeat(np.arange(len(lens)), lens)
    rng = np.random.default_rng(123)

    def run(n_rows):
        rows = np.sort(rng.choice(w.total_tokens, size=n_rows, replace=False)).astype(np.int64)
        flops = float(np.sum(4.0 * lens[seq_of[rows]] * w.head_dim * w.n_heads))
        t0 = time.perf_counter()
        oracle.attention_rows(q, k, v, cu, scale, rows)
        return time.perf_counter() - t0, flops, n_rows

    def timed(budget_s):
        run(16)  # warms the oracle's threads and caches
        dt, _, n = run(128)  # the per-row time of a short pilot sizes the sample
        n_rows = int(min(w.total_tokens, max(16, budget_s / max(dt / n, 1e-6))))
        return run(n_rows)

    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    cores = oracle.threads()
    dt, fl, n = timed(target_s)
    oracle.set_threads(1)
    dt1, fl1, n1 = timed(one_core_s)
    oracle.set_threads(cores)
    base = {
        "value": fl / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "cpu_model": model,
        "kind": "oracle",
        "sample": f"{n} of {w.total_tokens} query rows of {name} (all {w.n_heads} heads, every key of each row's "
                  f"image), float64, {dt:.1f} s on {cores} threads",
        "one_core": {"value": fl1 / dt1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                     "sample": f"{n1} query rows of {name}, {dt1:.1f} s on 1 thread"},
    }
    errs = {}
    for wname, (host, out) in gpu_outputs.items():
        wq, wk, wv, wcu, wscale = host
        ww = inputs.WORKLOADS[wname]
        g = out.float().cpu().numpy().astype(np.float64)
        n_rows = ERR_ROWS.get(wname)
        if n_rows is None or n_rows >= ww.total_tokens:
            ref = oracle.attention(wq, wk, wv, wcu, wscale)
            rows = None
        else:
            rows = np.sort(np.random.default_rng(7).choice(ww.total_tokens, size=n_rows, replace=False))
            ref = oracle.attention_rows(wq, wk, wv, wcu, wscale, rows.astype(np.int64))
            g = g[rows]
        diff = np.abs(g - ref)
        at = np.unravel_index(int(np.argmax(diff)), diff.shape)
        row = int(rows[at[0]]) if rows is not None else int(at[0])
        errs[wname] = {"max_abs_err": float(diff[at]), "at": [row, int(at[1]), int(at[2])],
                       "mean_abs_err": float(diff.mean()), "tol": TOL[ww.dtype],
                       "rows_compared": int(g.shape[0]), "rows": int(ww.total_tokens)}
        log(f"[bench] {wname}: max-abs err {errs[wname]['max_abs_err']:.3e} at {errs[wname]['at']} "
            f"over {g.shape[0]} rows (tol {TOL[ww.dtype]})")
    return base, errs


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed device time run after the warm-up, before the timed launches")
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
    ap.add_argument("--profile-commands", action="store_true",
                    help="print the rocprofv3 commands behind profiles/attn_fwd_<workload>.md and exit")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/attn_fwd_<workload>.md and _counters.json from the rocprofv3 output "
                         "that --profile-commands wrote under DIR, and exit (no GPU needed)")
    args = ap.parse_args()
    if args.profile_commands:
        print("\n".join(profile_commands(args.workload)))
        return
    if args.summarize_profiles:
        rec = summarize_profiles(args.summarize_profiles, args.workload)
        log(f"[bench] wrote profiles/attn_fwd_{args.workload}.md: trace mean {rec['trace_mean_us']:.2f} us, "
            f"MFMA busy {rec['mfma_busy']:.1%}, HBM {rec['hbm_bytes_per_launch'] / 1e6:.1f} MB per launch")
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this attention path is a single-GPU "
              f"build; DESIGN.md describes how it would shard.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.prologue:
        w, ms, nbytes = time_prologue(args.workload, args.steps, args.warmup, args.settle_ms)
        gbs = nbytes / (ms * 1e-3) / 1e9
        log(f"[bench] prologue {args.workload}: {ms * 1e3:.1f} us/launch, {gbs:.0f} GB/s")
        print(json.dumps({
            "metric": "qkv prologue GB/s (packed qkv read once, Q/K/V written once, rope tables read once)",
            "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": w.dtype, "data": "synthetic (seeded N(0,1) projection output, 2-D rope tables)",
            "config": {"workload": w.name, "tokens": w.total_tokens, "heads": w.n_heads, "kv_heads": w.kv_heads,
                       "head_dim": w.head_dim, "bytes_per_step": nbytes, "rope": True, "norm": True},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": None},
        }), flush=True)
        return

    masked = args.causal or args.window > 0
    out_f32 = args.out_dtype == "f32"
    log(f"[bench] {args.workload}: warmup {args.warmup}, settle {args.settle_ms:.0f} ms, steps {args.steps}")
    w, host, out, rec = time_workload(args.workload, args.steps, args.warmup, args.settle_ms, out_f32=out_f32,
                                      causal=args.causal, window=args.window)
    kernel_ms = rec["ms_per_step"]
    # algorithmic FLOPs: 4*D*H per (query, key) pair the mask keeps
    flops = (4.0 * w.head_dim * w.n_heads * visible_pairs(w.lengths, args.causal, args.window)) if masked else w.flops
    tflops = flops / (kernel_ms * 1e-3) / 1e12
    peak = peak_of(w.dtype)
    log(f"[bench] {args.workload}: {kernel_ms * 1e3:.1f} us/launch ({tflops:.1f} TFLOP/s, {tflops / peak:.1%} of "
        f"peak); cold {rec['cold_ms_per_step'] * 1e3 if rec['cold_ms_per_step'] else 0:.1f} us/launch")
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {args.copy_calibration_mib} MiB read + written once")
        del src, dst

    outputs = {}  # workload -> (host inputs, GPU output) for the oracle comparison
    configs = {}
    family = not (args.no_secondary or masked or out_f32) and args.workload in FAMILY
    if family:
        outputs[args.workload] = (host, out)
        for name in FAMILY:
            if name == args.workload:
                r = dict(rec)
                ww = w
            else:
                ww, h2, o2, r = time_workload(name, args.steps if name != "long-16384" else max(10, args.steps // 10),
                                              args.warmup, min(args.settle_ms, 50.0),
                                              graph=name in ("tiny-64", "vit-196", "page-912"))
                outputs[name] = (h2, o2)
            pk = peak_of(ww.dtype)
            r.update({"value": ww.flops / (r["ms_per_step"] * 1e-3) / 1e12, "unit": "TFLOP/s", "dtype": ww.dtype,
                      "lengths": list(ww.lengths) if len(ww.lengths) <= 16 else len(ww.lengths),
                      "heads": ww.n_heads, "head_dim": ww.head_dim, "flops_per_step": ww.flops, "peak": pk})
            r["frac_of_peak"] = r["value"] / pk
            if "graph_replay_ms_per_step" in r:
                r["graph_replay_value"] = ww.flops / (r["graph_replay_ms_per_step"] * 1e-3) / 1e12
            configs[name] = r
            log(f"[bench] {name}: {r['ms_per_step'] * 1e3:.2f} us/launch, {r['value']:.1f} TFLOP/s "
                f"({r['frac_of_peak']:.1%} of {pk})"
                + (f"; graph replay {r['graph_replay_ms_per_step'] * 1e3:.2f} us" if "graph_replay_ms_per_step" in r
                   else ""))

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] the float64 oracle on the host cores (bounded samples)")
        cpu, errs = cpu_leg(args.workload if args.workload in FAMILY else HEADLINE, outputs)
        for name, e in errs.items():
            configs.setdefault(name, {}).update(e)
        log(f"[bench] oracle: {cpu['value'] * 1e3:.3f} GFLOP/s on {cpu['cores']} threads, "
            f"{cpu['one_core']['value'] * 1e3:.3f} on 1")

    counters = committed_counters(w.name) if not (masked or out_f32) else None
    traffic = counters.get("hbm_bytes_per_launch") if counters else None
    result = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": kernel_ms,
        "cold_ms_per_step": rec["cold_ms_per_step"],
        "settle_ms": rec["settle_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs of the workload's shape)",
        "config": {
            "workload": w.name, "lengths": list(w.lengths), "tokens": w.total_tokens, "heads": w.n_heads,
            "head_dim": w.head_dim, "kv_heads": w.kv_heads, "out_dtype": "f32" if out_f32 else w.dtype,
            "causal": bool(args.causal), "window": args.window, "flops_per_step": flops,
            "caches": "warm: inputs resident in HBM, launches back to back on one stream",
        },
        "roofline": {
            "bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s", "frac": tflops / peak,
            "traffic": traffic,
            "traffic_source": (f"profiles/attn_fwd_{w.name}_counters.json: rocprofv3 FETCH_SIZE and WRITE_SIZE "
                               f"of this kernel source, scaled by a plain copy" if traffic else None),
        },
        "counters": ({"source": f"profiles/attn_fwd_{w.name}_counters.json (rocprofv3, this kernel source)",
                      "mfma_busy": counters.get("mfma_busy"), "hbm_gbs": counters.get("hbm_gbs"),
                      "trace_mean_us": counters.get("trace_mean_us")} if counters else None),
        "configs": configs or None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
