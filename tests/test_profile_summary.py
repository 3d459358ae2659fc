"""bench.py's rocprofv3 summariser on a small synthetic output tree (host logic, no GPU).

The tree has the layout that `bench.py --profile-commands` writes: per run a directory of
rocprofv3 CSV files and the bench JSON line.  The figures are chosen so that every derived
number has a hand-computable value: the trace mean over the timed launches only, the counter
means over the last `steps` attention dispatches only, the copy calibration's scale factors,
HBM bytes and the MFMA-busy fraction.
"""
from __future__ import annotations

import csv
import json
import os

import pytest

import bench
from vision_transformer_attention_amd import inputs

NAME = "page-912"
KERNEL = "void attn_fwd_bf16_kernel<...>(...)"
COPY = "__amd_rocclr_copyBuffer"


def write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=list(rows[0]))
        wr.writeheader()
        wr.writerows(rows)


def make_tree(root, steps=4, cold=3):
    d = os.path.join(root, NAME)
    write_csv(os.path.join(d, "kt", "run_agent_info.csv"),
              [{"Agent_Type": "CPU", "Simd_Count": 0, "Array_Count": 0},
               {"Agent_Type": "GPU", "Simd_Count": 1024, "Array_Count": 32}])
    # three cold dispatches of 50 us, then the timed ones: 10, 12, 14 and 16 us
    trace, t = [], 1000
    durs = [50_000] * cold + [10_000 + 2_000 * i for i in range(steps)]
    for i, du in enumerate(durs):
        trace.append({"Dispatch_Id": i + 1, "Kernel_Name": KERNEL, "Start_Timestamp": t, "End_Timestamp": t + du})
        t += du + 500
    trace.append({"Dispatch_Id": len(durs) + 1, "Kernel_Name": "some_other_kernel", "Start_Timestamp": t,
                  "End_Timestamp": t + 999_999})
    write_csv(os.path.join(d, "kt", "run_kernel_trace.csv"), trace)
    write_csv(os.path.join(d, "kt", "run_kernel_stats.csv"),
              [{"Name": KERNEL, "Calls": len(durs), "AverageNs": 1.0, "MinNs": 1.0, "MaxNs": 1.0}])
    for run in ["kt", *bench.PMC_PASSES]:
        with open(os.path.join(d, f"{run}.json"), "w") as f:
            json.dump({"steps": steps, "warmup": cold, "ms_per_step": 0.013, "cold_ms_per_step": 0.05}, f)
    for run, names in bench.PMC_PASSES.items():
        rows, did = [], 0
        for i in range(cold + steps):  # cold dispatches carry huge values that must not count
            did += 1
            for c in names:
                val = 1e12 if i < cold else (1000.0 * (i - cold + 1) if c != "SQ_VALU_MFMA_BUSY_CYCLES" else 0.0)
                if c == "SQ_VALU_MFMA_BUSY_CYCLES" and i >= cold:
                    val = 1024 * 20_000 * bench.PEAK_CLOCK_GHZ * 0.25  # a quarter of 20 us at 2.4 GHz
                if c == "SQ_CYCLES" and i >= cold:
                    val = 32 * 20_000 * 2.0  # 2.0 GHz over 20 us on 32 shader arrays
                rows.append({"Dispatch_Id": did, "Kernel_Name": KERNEL, "Counter_Name": c, "Counter_Value": val,
                             "Start_Timestamp": 0, "End_Timestamp": 20_000})
        if run in ("p3", "p4"):  # one copy of COPY_MIB: fetch counts half the bytes, write all
            did += 1
            kib = bench.COPY_MIB * 1024.0
            rows.append({"Dispatch_Id": did, "Kernel_Name": COPY, "Counter_Name": names[0],
                         "Counter_Value": kib / 2 if names[0] == "FETCH_SIZE" else kib,
                         "Start_Timestamp": 0, "End_Timestamp": 1})
        write_csv(os.path.join(d, run, "run_counter_collection.csv"), rows)
    return d


def test_summary_figures(tmp_path):
    root = tmp_path / "prof"
    out = tmp_path / "out"
    out.mkdir()
    make_tree(str(root))
    rec = bench.summarize_profiles(str(root), NAME, out_dir=str(out))
    # timed launches: the last 4 of the attention kernel, 10..16 us
    assert rec["trace"]["timed"] == 4 and rec["trace_mean_us"] == pytest.approx(13.0)
    assert rec["trace"]["min_us"] == pytest.approx(10.0) and rec["trace"]["max_us"] == pytest.approx(16.0)
    # counter means over the timed dispatches only: 1000, 2000, 3000, 4000 -> 2500
    assert rec["counters_mean_per_dispatch"]["SQ_INSTS_MFMA"] == pytest.approx(2500.0)
    # calibration: fetch counted half the copied bytes -> scale 2; write scale 1
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["hbm_read_bytes"] == pytest.approx(2500.0 * 2.0 * 1024)
    assert rec["hbm_write_bytes"] == pytest.approx(2500.0 * 1024)
    assert rec["hbm_gbs"] == pytest.approx((2500.0 * 3 * 1024) / 13_000.0)
    assert rec["mfma_busy"] == pytest.approx(0.25)
    assert rec["counter_run_clock_ghz"] == pytest.approx(2.0)
    w = inputs.WORKLOADS[NAME]
    assert rec["algorithmic_bytes"] == 2 * 2 * w.total_tokens * w.head_dim * (w.n_heads + w.kv_heads)
    assert rec["source_sha256"] == bench.kernel_sha()
    on_disk = json.loads((out / f"attn_fwd_{NAME}_counters.json").read_text())
    assert on_disk["trace_mean_us"] == rec["trace_mean_us"]
    md = (out / f"attn_fwd_{NAME}.md").read_text()
    for cmd in bench.profile_commands(NAME):
        assert cmd in md  # the summary carries the commands that made it


def test_counters_are_used_only_for_the_same_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    rec = {"source_sha256": bench.kernel_sha(), "hbm_bytes_per_launch": 1.0}
    (tmp_path / f"attn_fwd_{NAME}_counters.json").write_text(json.dumps(rec))
    assert bench.committed_counters(NAME)["hbm_bytes_per_launch"] == 1.0
    rec["source_sha256"] = "0" * 64
    (tmp_path / f"attn_fwd_{NAME}_counters.json").write_text(json.dumps(rec))
    assert bench.committed_counters(NAME) is None
    assert bench.committed_counters("no-such-workload") is None


def test_profile_commands_run_from_the_repository_root():
    for name in ("packed-varlen-8", "page-912", "long-16384"):
        cmds = bench.profile_commands(name)
        assert cmds[0].startswith("mkdir -p ")
        for c in cmds[1:]:
            assert "-- python3 bench.py --workload " + name in c and "cd " not in c
        pmc = [c for c in cmds if "--pmc" in c]
        assert len(pmc) == len(bench.PMC_PASSES)
        for c, names in zip(pmc, bench.PMC_PASSES.values()):
            assert c.split("--pmc ")[1].split(" --output-format")[0].split() == names
