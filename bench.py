"""Benchmark of the DSA sparse MLA forward on one MI355X.

One step = one call of the library's forward (index stage, gather, QK^T,
online softmax, PV, epilogue, and the split merge when the call splits) over
one batch of synthetic inputs already resident in HBM.

Default workload: SWE-like prefill, sq = skv = 2119 tokens, 8 query heads,
dqk 576 / dv 512, topk 2048, bf16 (the shape of "feat: add XTuner TileLang
sparse MLA backend", Performance > Isolated sparse MLA forward).

With --op bwd it times the backward instead (flat workloads): one step is
one backward call (the dkv zero fill, then the token-major kernel, or the
kv-major prepass and pass with the token-major kernel for rows that repeat
an entry), after one forward that supplies out and LSE; `value` then counts
the 1152-byte gathered row per valid key, as for the forward, and `tflops`
5504 flops per valid key and head.

Prints one JSON line. `value` is the gathered-KV bandwidth (1152 bytes per
valid key: one 576-wide bf16 row, shared by every head) over the average step
time; `tflops` counts 2 * H * (576 + 512) flops per valid key. `roofline`
takes the forward kernel's own average duration, from HIP events recorded on
the stream it runs on. `cpu_baseline` times the CPU oracle on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0         # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "sparse MLA fwd TFLOP/s + gathered-KV GB/s (% roofline), topk=2048, dqk576/dv512"
ROW_BYTES = 576 * 2
FLOP_PER_KEY_HEAD = 2 * (576 + 512)
# backward: QK^T (576), dO V^T (512), dQ (576), dK (576), dV (512) per key and head
BWD_METRIC = "sparse MLA bwd TFLOP/s + gathered-KV GB/s (% roofline), topk=2048, dqk576/dv512"
BWD_FLOP_PER_KEY_HEAD = 2 * (3 * 576 + 2 * 512)
# the gathered row, as for the forward: the fp32 gradient row each key
# receives is summed in registers by the kv-major schedule, so it is not
# counted as moved bytes (the counters give what the token-major one moves)
BWD_BYTES_PER_KEY = ROW_BYTES


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dsa_sparse_mla_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(workload: str, op: str = "fwd") -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json" if op == "fwd"
                        else f"traffic_bwd_{workload}.json")


def traffic_for(workload: str, op: str = "fwd"):
    """Measured HBM bytes per launch of the op's main kernel, from the committed
    counter summary, if it was taken on the current kernel sources; otherwise None."""
    path = traffic_path(workload, op)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


COPY_BYTES = 256 << 20   # the calibration copy reads and writes this many bytes
FWD_KERNEL = re.compile(r"sparse_mla_fwd(_ws)?_kernel")   # the forward kernels' names
# the kernels of one backward call: the dkv fill (once per call), the kv-major
# prepass and pass, and the token-major kernel
BWD_KERNEL = re.compile(r"dkv_zero_kernel|sparse_mla_bwd_(prep_|kv_)?kernel")
BWD_CALL_MARK = re.compile(r"dkv_zero_kernel")


def copy_calibration(dev, reps: int = 3):
    """Launch a plain elementwise copy of known size (read COPY_BYTES, write
    COPY_BYTES) so that counter runs can scale FETCH_SIZE / WRITE_SIZE."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def summarize_traffic(workload: str, fetch_csv: str, write_csv: str, command: str, op: str = "fwd",
                      out_path: str | None = None):
    """Turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, then WRITE_SIZE, in
    KiB per dispatch) into HBM bytes per forward launch, each scaled by what
    the same counter reads for the calibration copy, and store the result
    under profiles/ with the kernel-source hash it was taken on."""
    import csv
    import statistics

    def per_dispatch(path, counter):
        vals = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                key = (row["Dispatch_Id"], row["Kernel_Name"])
                vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
        return vals

    out = {"workload": workload, "source_hash": source_hash(), "command": command}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = per_dispatch(path, counter)
        copy = [v for (d, k), v in vals.items() if "neg" in k]
        kern = FWD_KERNEL if op == "fwd" else BWD_KERNEL
        fwd = [v for (d, k), v in vals.items() if kern.search(k)]
        if not copy or not fwd:
            raise SystemExit(f"{path}: no calibration copy or {op} dispatch with {counter}")
        factor = COPY_BYTES / (statistics.median(copy) * 1024.0)
        if op == "fwd":
            # one forward kernel per launch: the median dispatch
            kib, count = statistics.median(fwd), len(fwd)
        else:
            # a backward call launches several kernels: their sum per call
            count = sum(1 for (d, k) in vals if BWD_CALL_MARK.search(k))
            kib = sum(fwd) / max(count, 1)
        tag = counter.split("_")[0].lower()
        out[f"{tag}_kib_copy"] = statistics.median(copy)
        out[f"{tag}_kib_kernel"] = kib
        out[f"{tag}_factor"] = round(factor, 4)
        out[f"{tag}_bytes"] = round(kib * 1024.0 * factor)
        out[f"{tag}_dispatches"] = count
    out["bytes_per_launch"] = out["fetch_bytes"] + out["write_bytes"]
    path = out_path or traffic_path(workload, op)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def valid_keys(d) -> int:
    import torch
    if "kv" in d:
        idx = d["indices"]
        n = d["kv"].shape[0]
        return int(((idx >= 0) & (idx < n)).sum().item())
    idx = d["indices"].long()
    T = idx.shape[0]
    seq = torch.arange(T, device=idx.device) // d["q_per_seq"]
    lens = d["seq_lens"].long()[seq][:, None]
    return int(((idx >= 0) & (idx < lens)).sum().item())   # the decode tables map every position


def cpu_baseline(d, budget_s: float):
    """Time the CPU oracle on the last tokens of the workload until ~budget_s."""
    import numpy as np
    from oracle import sparse_mla_fwd_paged_ref, sparse_mla_fwd_ref
    q = d["q"].float().cpu().numpy()
    idx = d["indices"].cpu().numpy()
    paged = "kv_pages" in d
    if paged:
        kvp = d["kv_pages"].float().cpu().numpy()
        table = d["page_table"].cpu().numpy()
        lens = d["seq_lens"].cpu().numpy()
        Q = d["q_per_seq"]
    else:
        kv = d["kv"].float().cpu().numpy()
    T = q.shape[0]
    done_keys = 0
    done_tokens = 0
    elapsed = 0.0
    chunk = 16
    t_end = T
    while elapsed < budget_s and t_end > 0:
        if paged:
            # whole sequences, so the oracle's token -> sequence map holds
            s1 = (t_end - 1) // Q + 1
            s0 = max(0, s1 - max(1, chunk // Q))
            a, b = s0 * Q, s1 * Q
            t0 = time.perf_counter()
            sparse_mla_fwd_paged_ref(q[a:b], kvp, table[s0:s1], lens[s0:s1], idx[a:b],
                                     d["sm_scale"], Q)
            elapsed += time.perf_counter() - t0
            seq = np.arange(a, b) // Q - s0
            done_keys += int(((idx[a:b] >= 0) & (idx[a:b] < lens[s0:s1][seq][:, None])).sum())
        else:
            a, b = max(0, t_end - chunk), t_end
            t0 = time.perf_counter()
            sparse_mla_fwd_ref(q[a:b], kv, idx[a:b], d["sm_scale"])
            elapsed += time.perf_counter() - t0
            done_keys += int(((idx[a:b] >= 0) & (idx[a:b] < kv.shape[0])).sum())
        done_tokens += b - a
        t_end = a
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {
        "value": round(done_keys * ROW_BYTES / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"last {done_tokens} of {T} tokens ({done_keys} valid keys), numpy float64, "
                  f"{elapsed:.1f} s",
    }


def cpu_baseline_bwd(d, dout, budget_s: float):
    """Time the CPU backward oracle on the last tokens of the workload until ~budget_s."""
    from oracle import sparse_mla_bwd_ref
    q = d["q"].float().cpu().numpy()
    kv = d["kv"].float().cpu().numpy()
    idx = d["indices"].cpu().numpy()
    do = dout.float().cpu().numpy()
    T = q.shape[0]
    done_keys = done_tokens = 0
    elapsed = 0.0
    t_end = T
    while elapsed < budget_s and t_end > 0:
        a, b = max(0, t_end - 16), t_end
        t0 = time.perf_counter()
        sparse_mla_bwd_ref(q[a:b], kv, idx[a:b], d["sm_scale"], do[a:b])
        elapsed += time.perf_counter() - t0
        done_keys += int(((idx[a:b] >= 0) & (idx[a:b] < kv.shape[0])).sum())
        done_tokens += b - a
        t_end = a
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {
        "value": round(done_keys * BWD_BYTES_PER_KEY / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"last {done_tokens} of {T} tokens ({done_keys} valid keys), backward oracle, "
                  f"numpy float64, {elapsed:.1f} s",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="swe",
                    choices=["short", "swe", "wide", "varlen16k", "varlen32k", "decode"])
    ap.add_argument("--op", default="fwd", choices=["fwd", "bwd"],
                    help="fwd (the headline metric) or the backward (flat workloads)")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for cpu_baseline (0 skips it)")
    ap.add_argument("--flush", action="store_true",
                    help="also time launches with a 512 MB scratch write between them (caches cold), "
                         "reported as kernel_ms_flushed")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a copy of known size (for HBM counter scaling)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="host only: store HBM bytes per launch from two counter runs")
    ap.add_argument("--traffic-command", default="",
                    help="the profiling command, recorded with --summarize-traffic")
    args = ap.parse_args()

    if args.summarize_traffic:
        summarize_traffic(args.workload, *args.summarize_traffic, args.traffic_command, args.op)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(this path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import torch

    import dsa_sparse_mla_amd as dsa
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.WORKLOADS[args.workload]
    gen_dev = "cpu" if w.num_tokens * w.num_heads <= 2119 * 8 else "cuda"
    d_host = workloads.make(args.workload, device=gen_dev)
    d = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in d_host.items()}
    H = d["q"].shape[1]
    T = d["q"].shape[0]
    V = valid_keys(d)
    gathered = V * ROW_BYTES
    flops = V * H * FLOP_PER_KEY_HEAD

    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    splits, ws_bytes = dsa.workspace_size(T, H, d["indices"].shape[1], args.num_splits)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    if args.op == "bwd":
        if "kv" not in d:
            print("the backward runs on flat workloads only", file=sys.stderr)
            sys.exit(2)
        g = torch.Generator(device=dev).manual_seed(12345)
        dout = torch.randn((T, H, 512), generator=g, device=dev).to(torch.bfloat16)
        dsa.sparse_mla_fwd(d["q"], d["kv"], d["indices"], d["sm_scale"], out=out, lse=lse, workspace=ws)
        dq = torch.empty((T, H, 576), dtype=torch.float32, device=dev)
        dkv = torch.empty((d["kv"].shape[0], 576), dtype=torch.float32, device=dev)
        bwd_schedule, bwd_ws_bytes = dsa.bwd_workspace_size(T, H, d["kv"].shape[0], d["indices"].shape[1])
        bwd_ws = torch.empty(max(bwd_ws_bytes, 256), dtype=torch.uint8, device=dev)

        def step():
            dsa.sparse_mla_bwd(d["q"], d["kv"], d["indices"], d["sm_scale"], out, lse, dout,
                               dq=dq, dkv=dkv, workspace=bwd_ws)
    elif "kv" in d:
        def step():
            dsa.sparse_mla_fwd(d["q"], d["kv"], d["indices"], d["sm_scale"], out=out, lse=lse,
                               num_splits=args.num_splits, workspace=ws)
    else:
        def step():
            dsa.sparse_mla_fwd_paged(d["q"], d["kv_pages"], d["page_table"], d["seq_lens"],
                                     d["indices"], d["sm_scale"], d["q_per_seq"], out=out, lse=lse,
                                     num_splits=args.num_splits, workspace=ws)

    if args.copy_calibration:
        copy_calibration(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    per_launch_ms.sort()
    avg_ms = sum(per_launch_ms) / len(per_launch_ms)
    med_ms = per_launch_ms[len(per_launch_ms) // 2]
    ms_per_step = wall * 1e3 / args.steps

    flushed_ms = None
    if args.flush:
        # L2 and MALL hold no KV when each launch starts: a 512 MB write
        # between launches, outside the events
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        fl = []
        for i in range(args.steps):
            scratch.fill_(i & 255)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            fl.append(e0.elapsed_time(e1))
        fl.sort()
        flushed_ms = fl[len(fl) // 2]
        del scratch

    if args.op == "bwd":
        gathered = V * BWD_BYTES_PER_KEY
        flops = V * H * BWD_FLOP_PER_KEY_HEAD
    gbps = gathered / (ms_per_step * 1e-3) / 1e9
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    kern_gbps = gathered / (avg_ms * 1e-3) / 1e9
    kern_tflops = flops / (avg_ms * 1e-3) / 1e12
    bound = "hbm" if H <= 16 else "mfma"
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(kern_gbps, 2), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(kern_gbps / HBM_PEAK_GBPS, 4),
                "traffic": traffic_for(args.workload)}
    else:
        roof = {"bound": "mfma", "achieved": round(kern_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(kern_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic_for(args.workload)}

    if args.op == "bwd":
        roof["traffic"] = traffic_for(args.workload, "bwd")
    rec = {
        "metric": METRIC if args.op == "fwd" else BWD_METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.desc, "name": w.name, "num_tokens": T, "num_heads": H,
                   "topk": int(d["indices"].shape[1]), "dqk": 576, "dv": 512,
                   "valid_keys": V, "splits": splits},
        "tflops": round(tflops, 3),
        "gathered_kv_gbps": round(gbps, 2),
        "kernel_ms_avg": round(avg_ms, 5),
        "kernel_ms_median": round(med_ms, 5),
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "pct_mfma_peak": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 3),
        "roofline": roof,
        **({"kernel_ms_flushed": round(flushed_ms, 5),
            "gathered_kv_gbps_flushed": round(gathered / (flushed_ms * 1e-3) / 1e9, 2)}
           if flushed_ms is not None else {}),
        "source_hash": source_hash(),
    }
    if args.op == "bwd":
        rec["config"]["op"] = "bwd"
        rec["config"]["schedule"] = bwd_schedule
        rec["bytes_per_key"] = BWD_BYTES_PER_KEY
    if args.cpu_budget > 0:
        if args.op == "bwd":
            rec["cpu_baseline"] = cpu_baseline_bwd(d_host if gen_dev == "cpu" else d, dout, args.cpu_budget)
        else:
            rec["cpu_baseline"] = cpu_baseline(d_host if gen_dev == "cpu" else d, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
