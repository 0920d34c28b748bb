"""Host-side checks of the measurement tooling in bench.py (no GPU needed)."""
from __future__ import annotations

import csv
import json
import os
import subprocess
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for disp, kern, val in rows:
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": kern, "Counter_Name": counter, "Counter_Value": val})


def test_traffic_summary_scales_by_the_copy(tmp_path):
    copy_kib = bench.COPY_BYTES / 1024
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # the copy reads COPY_BYTES but FETCH_SIZE shows half of it: fetch factor 2
    _counter_csv(fetch, "FETCH_SIZE", [
        (1, "void at::native::neg_kernel", copy_kib / 2),
        (2, "void dsa::sparse_mla_fwd_kernel<1, false>(dsa::FwdArgs)", 1000.0),
        (3, "void dsa::sparse_mla_fwd_kernel<1, false>(dsa::FwdArgs)", 1000.0),
        (4, "dsa::sparse_mla_bwd_kernel<1>(dsa::BwdArgs)", 77.0)])
    _counter_csv(write, "WRITE_SIZE", [
        (1, "void at::native::neg_kernel", copy_kib),
        (2, "void dsa::sparse_mla_fwd_kernel<1, false>(dsa::FwdArgs)", 300.0),
        (3, "void dsa::sparse_mla_fwd_kernel<1, false>(dsa::FwdArgs)", 300.0)])
    out = tmp_path / "t.json"
    bench.summarize_traffic("swe", str(fetch), str(write), "cmd", op="fwd", out_path=str(out))
    rec = json.loads(out.read_text())
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    assert rec["fetch_bytes"] == 2 * 1000 * 1024 and rec["write_bytes"] == 300 * 1024
    assert rec["bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
    assert rec["fetch_dispatches"] == 2 and rec["source_hash"] == bench.source_hash("fwd")


def test_source_hash_per_op(tmp_path, monkeypatch):
    """An op's profiles depend only on its kernels and the launch code: a
    change to the backward's kernel leaves the forward's hash alone."""
    csrc = tmp_path / "dsa_sparse_mla_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in sorted(set().union(*bench.OP_SOURCES.values())):
        (csrc / name).write_text(name)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    before = {op: bench.source_hash(op) for op in ("fwd", "bwd", "topk")}
    full = bench.source_hash()
    (csrc / "bwd_dkv_kernel.hpp").write_text("changed")
    after = {op: bench.source_hash(op) for op in ("fwd", "bwd", "topk")}
    assert after["fwd"] == before["fwd"] and after["topk"] == before["topk"]
    assert after["bwd"] != before["bwd"] and bench.source_hash() != full


def test_backward_traffic_sums_the_kernels_of_a_call(tmp_path):
    copy_kib = bench.COPY_BYTES / 1024
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    call = [("void dsa::dkv_zero_kernel(float*, long, long)", 1.0),
            ("void dsa::sparse_mla_bwd_prep_kernel(dsa::BwdArgs, dsa::KvMajorArgs)", 10.0),
            ("void dsa::sparse_mla_bwd_kv_kernel(dsa::BwdArgs, dsa::KvMajorArgs)", 100.0),
            ("void dsa::sparse_mla_bwd_kernel<1>(dsa::BwdArgs)", 5.0)]
    rows = [(1, "void at::native::neg_kernel", copy_kib / 2),
            (2, "void dsa::sparse_mla_fwd_kernel<1, false>(dsa::FwdArgs)", 999.0)]
    rows += [(3 + 4 * c + i, k, v) for c in range(2) for i, (k, v) in enumerate(call)]
    _counter_csv(fetch, "FETCH_SIZE", rows)
    _counter_csv(write, "WRITE_SIZE", [(d, k, 2 * v if "neg" not in k else copy_kib) for d, k, v in rows])
    out = tmp_path / "t.json"
    bench.summarize_traffic("swe", str(fetch), str(write), "cmd", op="bwd", out_path=str(out))
    rec = json.loads(out.read_text())
    assert rec["fetch_dispatches"] == 2 and rec["fetch_kib_kernel"] == 116.0
    assert rec["fetch_bytes"] == 2 * 116 * 1024 and rec["write_bytes"] == 232 * 1024


def test_valid_keys_flat_and_paged():
    idx = torch.tensor([[0, 3, -1, 7], [9, -5, 2, 2]], dtype=torch.int32)
    d = {"kv": torch.zeros((8, 576)), "indices": idx}
    assert bench.valid_keys(d) == 5          # 0, 3, 7 | 2, 2 (9 and -5 are not rows)
    d = {"kv_pages": torch.zeros((2, 4, 576)), "indices": idx, "q_per_seq": 1,
         "seq_lens": torch.tensor([8, 3], dtype=torch.int32)}
    assert bench.valid_keys(d) == 5          # seq 0 holds 8: 0, 3, 7 | seq 1 holds 3: 2, 2


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2 and "one GPU" in res.stderr


def test_flop_and_byte_constants():
    assert bench.FLOP_PER_KEY_HEAD == 2 * (576 + 512)
    assert bench.ROW_BYTES == 1152
    assert bench.BWD_FLOP_PER_KEY_HEAD == 2 * (3 * 576 + 2 * 512)
    assert bench.BWD_BYTES_PER_KEY == 1152
    assert np.isclose(bench.HBM_PEAK_GBPS, 8000.0) and np.isclose(bench.MFMA_BF16_PEAK_TFLOPS, 2500.0)


def test_trace_summary(tmp_path):
    """The kernel-trace summary is written from a rocprofv3 trace directory and
    the script's own JSON line, with the command that made it."""
    import argparse
    d = tmp_path / "kt"
    d.mkdir()
    with open(d / "kt_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        w.writeheader()
        w.writerow({"Name": "void dsa::topk_select_kernel(dsa::TopkArgs)", "Calls": 4, "AverageNs": 50000,
                    "MinNs": 49000, "MaxNs": 51000, "Percentage": 90.0})
    with open(d / "kt_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for i, dur in enumerate((60000, 49000, 50000, 51000)):
            w.writerow({"Kernel_Name": "void dsa::topk_select_kernel(dsa::TopkArgs)",
                        "Start_Timestamp": 10 ** 9 * i, "End_Timestamp": 10 ** 9 * i + dur})
    log = tmp_path / "b.log"
    rec = {"steps": 3, "warmup": 1, "source_hash": "x", "config": {"workload": "w"}, "kernel_ms_avg": 0.05,
           "ms_per_step": 0.06, "roofline": {"bound": "hbm", "achieved": 1, "unit": "GB/s", "peak": 8000, "frac": 0.1}}
    log.write_text("noise\n" + json.dumps(rec) + "\n")
    args = argparse.Namespace(op="topk", workload="wide")
    bench.summarize_trace(args, str(d), str(log), out_dir=str(tmp_path))
    text = (tmp_path / "dsa_topk_wide_kernel_trace.md").read_text()
    assert "--op topk --workload wide --steps 3 --warmup 1" in text
    assert "50.0 us average over the last 3 launches" in text     # the warm-up launch is left out


def test_counter_summary(tmp_path):
    """Counters per dispatch of the op's kernel only; MFMA-busy fraction
    against the SIMD count (from the agent info) x the dispatch's cycles
    (SQ_BUSY_CYCLES over the shader engines), L2 hit fraction from TCC hits
    and misses."""
    import argparse
    with open(tmp_path / "pmc_agent_info.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Agent_Type", "Name", "Simd_Count", "Num_Shader_Banks"])
        w.writeheader()
        w.writerow({"Agent_Type": "CPU", "Name": "host", "Simd_Count": 0, "Num_Shader_Banks": 0})
        w.writerow({"Agent_Type": "GPU", "Name": "gfx950", "Simd_Count": 1024, "Num_Shader_Banks": 32})
    p = tmp_path / "pmc.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for disp in (1, 2, 3):
            k = "void dsa::sparse_mla_fwd_ws_kernel<false>(dsa::FwdArgs)"
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": k, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES",
                        "Counter_Value": 512000})
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": k, "Counter_Name": "SQ_BUSY_CYCLES",
                        "Counter_Value": 32000})
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": k, "Counter_Name": "TCC_HIT_sum", "Counter_Value": 75})
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": k, "Counter_Name": "TCC_MISS_sum", "Counter_Value": 25})
        w.writerow({"Dispatch_Id": 9, "Kernel_Name": "at::neg", "Counter_Name": "SQ_BUSY_CYCLES", "Counter_Value": 5})
    args = argparse.Namespace(op="fwd", workload="wide", traffic_command="cmd")
    bench.summarize_counters(args, [str(p)], out_dir=str(tmp_path))
    out = json.load(open(tmp_path / "counters_fwd_wide.json"))
    assert out["mfma_busy_frac"] == 0.5 and out["l2_hit_frac"] == 0.75
    assert out["dispatches"]["SQ_BUSY_CYCLES"] == 3 and out["cycles_per_dispatch"] == 1000


def test_counter_summary_per_kernel(tmp_path):
    """An op with several kernels per call (the backward): each kernel gets
    its own medians, and the top-level figures are the busiest kernel's."""
    import argparse
    p = tmp_path / "pmc.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for disp, k, busy, mfma in ((1, "dsa::dkv_zero_kernel(float*, long, long)", 3200, 0),
                                    (2, "dsa::sparse_mla_bwd_dkv_kernel(dsa::BwdArgs, dsa::KvMajorArgs)", 320000, 2048000),
                                    (3, "dsa::sparse_mla_bwd_dq_kernel(dsa::BwdArgs, dsa::KvMajorArgs)", 160000, 512000)):
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": k, "Counter_Name": "SQ_BUSY_CYCLES", "Counter_Value": busy})
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": k, "Counter_Name": "SQ_VALU_MFMA_BUSY_CYCLES",
                        "Counter_Value": mfma})
    args = argparse.Namespace(op="bwd", workload="wide", traffic_command="cmd")
    bench.summarize_counters(args, [str(p)], out_dir=str(tmp_path))
    out = json.load(open(tmp_path / "counters_bwd_wide.json"))
    assert "dkv_kernel" in out["kernel"] and out["mfma_busy_frac"] == 0.2   # 2048000 / (1024 * 320000 / 32)
    assert len(out["per_kernel"]) == 3
    assert out["per_kernel"]["dsa::sparse_mla_bwd_dq_kernel(dsa::BwdArgs, dsa::KvMajorArgs)"]["mfma_busy_frac"] == 0.1
