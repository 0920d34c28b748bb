"""Benchmark of the DSA sparse MLA forward on one MI355X.

One step = one call of the library's forward (index stage, gather, QK^T,
online softmax, PV, epilogue, and the split merge when the call splits) over
one batch of synthetic inputs already resident in HBM.

Default workload: SWE-like prefill, sq = skv = 2119 tokens, 8 query heads,
dqk 576 / dv 512, topk 2048, bf16 (the shape of "feat: add XTuner TileLang
sparse MLA backend", Performance > Isolated sparse MLA forward).

With --op bwd it times the backward instead (flat workloads): one step is
one backward call (the dkv zero fill, then the token-major kernel; or the
prepass, the kv-major pass (up to 16 heads) or the split schedule's dq and
dkv passes, and the token-major kernel for rows that repeat an entry), after
one forward that supplies out and LSE; `value` then counts
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
FP8_ROW_BYTES = 656   # an FP8 MLA cache row: 512 e4m3 + 4 fp32 scales + 64 bf16
FLOP_PER_KEY_HEAD = 2 * (576 + 512)
# backward: QK^T (576), dO V^T (512), dQ (576), dK (576), dV (512) per key and head
BWD_METRIC = "sparse MLA bwd TFLOP/s + gathered-KV GB/s (% roofline), topk=2048, dqk576/dv512"
BWD_FLOP_PER_KEY_HEAD = 2 * (3 * 576 + 2 * 512)
# the gathered row, as for the forward: the fp32 gradient row each key
# receives is summed in registers by the kv-major schedule, so it is not
# counted as moved bytes (the counters give what the token-major one moves)
BWD_BYTES_PER_KEY = ROW_BYTES


# kernel sources behind each op's measurements (the launch code is in the .hip)
OP_SOURCES = {
    "fwd": ("dsa_sparse_mla.hip", "fwd_kernel.hpp", "fwd_kernel_ws.hpp"),
    "bwd": ("dsa_sparse_mla.hip", "fwd_kernel.hpp", "bwd_kernel.hpp", "bwd_dq_kernel.hpp", "bwd_dkv_kernel.hpp"),
    "topk": ("dsa_sparse_mla.hip", "topk_kernel.hpp"),
}


def source_hash(op: str | None = None) -> str:
    """Hash of the kernel sources an op's profiles were taken on (all of
    csrc/ when op is None): a profile stays valid while they are unchanged."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dsa_sparse_mla_amd", "csrc")
    names = sorted(os.listdir(csrc)) if op is None else sorted(OP_SOURCES[op])
    for name in names:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(workload: str, op: str = "fwd") -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json" if op == "fwd"
                        else f"traffic_{op}_{workload}.json")


def traffic_for(workload: str, op: str = "fwd"):
    """Measured HBM bytes per launch of the op's main kernel, from the committed
    counter summary, if it was taken on the current kernel sources; otherwise None."""
    path = traffic_path(workload, op)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(op):
        return None
    return rec.get("bytes_per_launch")


COPY_BYTES = 256 << 20   # the calibration copy reads and writes this many bytes
FWD_KERNEL = re.compile(r"sparse_mla_fwd(_ws)?_kernel")   # the forward kernels' names
# the kernels of one backward call: the dkv fill (once per call), the
# prepass, the kv-major pass or the split schedule's dq and dkv passes, and
# the token-major kernel
BWD_KERNEL = re.compile(r"dkv_zero_kernel|sparse_mla_bwd_(prep_|kv_|dkv_|dq_)?kernel")
BWD_CALL_MARK = re.compile(r"dkv_zero_kernel")
TOPK_KERNEL = re.compile(r"topk_select_kernel")
OP_KERNEL = {"fwd": FWD_KERNEL, "bwd": BWD_KERNEL, "topk": TOPK_KERNEL}
# file-name stem of each op's profiles
OP_STEM = {"fwd": "sparse_mla_fwd", "bwd": "sparse_mla_bwd", "topk": "dsa_topk"}


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

    out = {"workload": workload, "op": op, "source_hash": source_hash(op), "command": command}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = per_dispatch(path, counter)
        copy = [v for (d, k), v in vals.items() if "neg" in k]
        kern = OP_KERNEL[op]
        fwd = [v for (d, k), v in vals.items() if kern.search(k)]
        if not copy or not fwd:
            raise SystemExit(f"{path}: no calibration copy or {op} dispatch with {counter}")
        factor = COPY_BYTES / (statistics.median(copy) * 1024.0)
        if op != "bwd":
            # one kernel per launch: the median dispatch
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


def _bench_line(log_path: str) -> dict:
    with open(log_path) as f:
        lines = [ln for ln in f if ln.startswith("{")]
    if not lines:
        raise SystemExit(f"{log_path}: no JSON line from bench.py")
    return json.loads(lines[-1])


def _profile_args(args, rec) -> str:
    op = "" if args.op == "fwd" else f" --op {args.op}"
    return (f"python bench.py{op} --workload {args.workload} --steps {rec['steps']} --warmup {rec['warmup']} "
            "--cpu-budget 0 --no-legs")


def summarize_trace(args, trace_dir: str, log_path: str, out_dir: str | None = None):
    """Format a rocprofv3 kernel-trace run of this script (-d trace_dir -o kt)
    into profiles/<op>_<workload>_kernel_trace.md: the command, the per-kernel
    statistics, the per-dispatch durations of the timed launches and the
    script's own line from the same run (its HIP-event average must agree)."""
    import csv
    import statistics
    rec = _bench_line(log_path)
    steps = rec["steps"]
    stats = list(csv.DictReader(open(os.path.join(trace_dir, "kt_kernel_stats.csv"))))
    trace = list(csv.DictReader(open(os.path.join(trace_dir, "kt_kernel_trace.csv"))))
    cmd = (f"rocprofv3 --kernel-trace --stats --output-format csv -d {trace_dir} -o kt -- "
           + _profile_args(args, rec))
    cfg = rec["config"]

    def short(n):
        return n if len(n) <= 70 else n[:67] + "..."
    out = [f"# {OP_STEM[args.op]} kernel trace: {cfg['workload']}", "",
           "MI355X (gfx950), one GPU. Command (from the repository root):", "", "```", cmd, "```", "",
           f"Kernel sources hash (bench.py `source_hash`): `{rec['source_hash']}`", "",
           "| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for r in stats[:8]:
        out.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    out += ["", "The calls include the warm-up launches; torch kernels are input generation.",
            "Per-dispatch durations of the library's kernels, timed launches only (`kt_kernel_trace.csv`):", ""]
    by = {}
    for r in trace:
        by.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    for k, v in by.items():
        if "dsa::" in k:
            t = v[-steps:]
            out.append(f"* `{short(k)}`: {statistics.mean(t):.1f} us average over the last {len(t)} launches "
                       f"(min {min(t):.1f}, max {max(t):.1f})")
    r = rec["roofline"]
    out += ["", "bench.py's line from the same run (HIP events on the launch stream, timed steps only):", "",
            f"* event average {rec['kernel_ms_avg'] * 1e3:.1f} us per step, wall {rec['ms_per_step'] * 1e3:.1f} us per step",
            f"* configuration: `{json.dumps(cfg)}`",
            f"* roofline: {r['bound']} {r['achieved']} {r['unit']} of {r['peak']} = {r['frac']}"]
    if "tflops" in rec:
        out.append(f"* {rec['gathered_kv_gbps']} GB/s of gathered rows, {rec['tflops']} TFLOP/s (wall time)")
    tp = traffic_path(args.workload, args.op)
    if os.path.exists(tp):
        t = json.load(open(tp))
        if t["source_hash"] == rec["source_hash"]:
            out += ["", f"HBM traffic per call (`profiles/{os.path.basename(tp)}`, two counter runs scaled by a "
                    f"copy of known size): fetch {t['fetch_bytes'] / 1e6:.1f} MB, write {t['write_bytes'] / 1e6:.1f} MB."]
    name = f"{OP_STEM[args.op]}_{args.workload}_kernel_trace.md"
    with open(os.path.join(out_dir or os.path.join(ROOT, "profiles"), name), "w") as f:
        f.write("\n".join(out) + "\n")
    print("wrote " + name)


def summarize_counters(args, csv_paths, out_dir: str | None = None):
    """Median per dispatch of every counter in rocprofv3 --pmc CSVs, per
    kernel of the op, into profiles/counters_<op>_<workload>.json, with
    derived MFMA-busy, L2 hit and LDS bank-conflict fractions. The top-level
    figures are those of the kernel with the most busy cycles (an op such as
    the backward launches several kernels per call).

    SQ counters are summed over the shader engines, so a dispatch's cycles
    are SQ_BUSY_CYCLES / Num_Shader_Banks (32 on MI355X), and the MFMA-busy
    fraction is SQ_VALU_MFMA_BUSY_CYCLES / (Simd_Count x those cycles), both
    counts from the run's pmc_agent_info.csv (defaults 1024 SIMDs, 32
    engines)."""
    import csv
    import statistics
    kern = OP_KERNEL[args.op]
    per = {}   # kernel -> counter -> dispatch -> value
    for path in csv_paths:
        with open(path) as f:
            for row in csv.DictReader(f):
                name = row.get("Kernel_Name", "")
                if not kern.search(name):
                    continue
                key = (path, row["Dispatch_Id"])
                c = row["Counter_Name"]
                d = per.setdefault(name, {}).setdefault(c, {})
                d[key] = d.get(key, 0.0) + float(row["Counter_Value"])
    if not per:
        raise SystemExit("no dispatch of the op's kernel in the counter files")
    simds, engines = 1024, 32
    for path in csv_paths:
        info = os.path.join(os.path.dirname(path), "pmc_agent_info.csv")
        if os.path.exists(info):
            with open(info) as f:
                for row in csv.DictReader(f):
                    if row.get("Agent_Type", "").upper().endswith("GPU") or "gfx" in row.get("Name", ""):
                        simds = int(row.get("Simd_Count") or simds)
                        engines = int(row.get("Num_Shader_Banks") or engines)
                        break
            break

    def derive(counters):
        med = {c: statistics.median(v.values()) for c, v in counters.items()}
        out = {"dispatches": {c: len(v) for c, v in counters.items()}, "counters": med}
        if "SQ_VALU_MFMA_BUSY_CYCLES" in med and med.get("SQ_BUSY_CYCLES"):
            cycles = med["SQ_BUSY_CYCLES"] / engines
            out["cycles_per_dispatch"] = cycles
            out["mfma_busy_frac"] = round(med["SQ_VALU_MFMA_BUSY_CYCLES"] / (simds * cycles), 4)
        hit, miss = med.get("TCC_HIT_sum"), med.get("TCC_MISS_sum")
        if hit is not None and miss is not None and hit + miss > 0:
            out["l2_hit_frac"] = round(hit / (hit + miss), 4)
        if med.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in med:
            out["lds_conflict_frac"] = round(med["SQ_LDS_BANK_CONFLICT"] / med["SQ_LDS_IDX_ACTIVE"], 4)
        return out

    kernels = {name: derive(c) for name, c in per.items()}
    main = max(kernels, key=lambda n: kernels[n]["counters"].get("SQ_BUSY_CYCLES", 0.0))
    out = {"workload": args.workload, "op": args.op, "source_hash": source_hash(args.op),
           "kernel": main, **kernels[main], "simds": simds, "shader_engines": engines,
           "command": args.traffic_command}
    if len(kernels) > 1:
        out["per_kernel"] = kernels
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), f"counters_{args.op}_{args.workload}.json")
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


def cpu_baseline(d, budget_s: float, dtype="float64"):
    """Time the CPU oracle on the last tokens of the workload until ~budget_s."""
    import numpy as np
    from oracle import sparse_mla_fwd_paged_fp8_ref, sparse_mla_fwd_paged_ref, sparse_mla_fwd_ref
    import torch
    q = d["q"].float().cpu().numpy()
    idx = d["indices"].cpu().numpy()
    paged = "kv_pages" in d
    fp8 = paged and d["kv_pages"].dtype == torch.uint8
    row_bytes = FP8_ROW_BYTES if fp8 else ROW_BYTES
    if paged:
        # FP8 rows stay raw (the oracle dequantises the pages a chunk uses)
        kvp = d["kv_pages"].cpu().numpy() if fp8 else d["kv_pages"].float().cpu().numpy()
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
            if fp8:
                # only this chunk's pages, renumbered
                tab = table[s0:s1]
                used = np.unique(tab[tab >= 0])
                remap = np.full(kvp.shape[0], -1, dtype=np.int64)
                remap[used] = np.arange(used.size)
                small = np.where(tab >= 0, remap[np.maximum(tab, 0)], -1).astype(np.int32)
                sparse_mla_fwd_paged_fp8_ref(q[a:b], kvp[used], small, lens[s0:s1], idx[a:b],
                                             d["sm_scale"], Q, dtype=getattr(np, dtype))
            else:
                sparse_mla_fwd_paged_ref(q[a:b], kvp, table[s0:s1], lens[s0:s1], idx[a:b],
                                         d["sm_scale"], Q, dtype=getattr(np, dtype))
            elapsed += time.perf_counter() - t0
            seq = np.arange(a, b) // Q - s0
            done_keys += int(((idx[a:b] >= 0) & (idx[a:b] < lens[s0:s1][seq][:, None])).sum())
        else:
            a, b = max(0, t_end - chunk), t_end
            t0 = time.perf_counter()
            sparse_mla_fwd_ref(q[a:b], kv, idx[a:b], d["sm_scale"], dtype=getattr(np, dtype))
            elapsed += time.perf_counter() - t0
            done_keys += int(((idx[a:b] >= 0) & (idx[a:b] < kv.shape[0])).sum())
        done_tokens += b - a
        t_end = a
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {
        "value": round(done_keys * row_bytes / elapsed / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"last {done_tokens} of {T} tokens ({done_keys} valid keys), numpy {dtype}, "
                  f"{elapsed:.1f} s",
    }


def host_info():
    """CPU model, usable cores and the BLAS pool the oracle runs on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    blas = None
    try:
        import numpy as np
        from threadpoolctl import threadpool_info
        np.ones((64, 64)) @ np.ones((64, 64))   # loads the BLAS pool
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if pools:
            blas = {"library": pools[0].get("internal_api"), "threads": pools[0].get("num_threads")}
    except Exception:
        pass
    return {"cpu_model": model, "cores": cores, "blas": blas}


def cpu_baseline_full(d, budget_s: float):
    """The oracle as it stands: float64 on all host cores (the reported value),
    then float32, then float64 on one BLAS thread (a per-core rate), each over
    a bounded sample of the workload's last tokens."""
    rec = cpu_baseline(d, budget_s)
    rec.update(host_info())
    rec["fp32"] = cpu_baseline(d, budget_s / 3, dtype="float32")
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"):
            one = cpu_baseline(d, budget_s / 3)
        one["cores"] = 1
        rec["single_thread"] = one
    except ImportError:
        pass
    rec["cores"] = rec["blas"]["threads"] if rec.get("blas") else rec["cores"]
    return rec


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


def gpu_info(dev):
    """Device name, its maximum shader clock, and the current one as the
    amdgpu driver reports it in sysfs (the level marked '*' in pp_dpm_sclk;
    a file read, so nothing is started from this process)."""
    import glob
    import torch
    p = torch.cuda.get_device_properties(dev)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "cus": p.multi_processor_count,
            "sclk_max_mhz": round(getattr(p, "clock_rate", 0) / 1000) or None}
    levels = []
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                cur = [ln.split(":", 1)[1].replace("*", "").strip() for ln in f if ln.rstrip().endswith("*")]
            if cur:
                levels.append(cur[0])
        except (OSError, IndexError):
            pass
    if levels:
        # one entry per card the host exposes; with one GPU there is one
        info["sclk_now"] = levels[0] if len(set(levels)) == 1 else levels
    return info


def time_steps(step, steps: int, warmup: int, stream):
    """W untimed steps, then K steps, each between HIP events on `stream`.
    Returns (average event ms, median event ms, wall ms per step)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return sum(ms) / len(ms), ms[len(ms) // 2], wall * 1e3 / steps


def time_flushed(step, steps: int, dev, stream, dirty: bool = False):
    """Median event ms of launches that each start with no KV in L2 or the
    MALL. Between launches, outside the events, a 512 MB write evicts the
    caches, and a read of another 512 MB then evicts the written lines, so
    their write-back to HBM happens before the launch and the caches hold
    clean, unrelated lines. With dirty=True the read is left out: the launch
    then starts with the L2s and the MALL full of dirty lines and pays their
    write-back inside the events (the cold case behind a writing kernel)."""
    import torch
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    clean = None if dirty else torch.ones(128 << 20, dtype=torch.int32, device=dev)
    fl = []
    for i in range(steps):
        scratch.fill_(i & 255)
        if clean is not None:
            clean.sum()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        fl.append(e0.elapsed_time(e1))
    del scratch, clean
    fl.sort()
    return fl[len(fl) // 2]


def fwd_setup(name: str, dev, num_splits: int = 0):
    """Inputs of a workload on the GPU and one forward step over them."""
    import torch
    import dsa_sparse_mla_amd as dsa
    import workloads
    w = workloads.WORKLOADS[name]
    gen_dev = "cpu" if w.kind == "flat" and w.num_tokens * w.num_heads <= 2119 * 8 else "cuda"
    fp8 = w.kind == "paged_fp8"
    d_host = workloads.make(name, device=gen_dev)
    d = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in d_host.items()}
    T, H = d["q"].shape[:2]
    topk = int(d["indices"].shape[1])
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    splits, ws_bytes = dsa.workspace_size(T, H, topk, num_splits)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    if "kv" in d:
        def step():
            dsa.sparse_mla_fwd(d["q"], d["kv"], d["indices"], d["sm_scale"], out=out, lse=lse,
                               num_splits=num_splits, workspace=ws)
    else:
        fwd = dsa.sparse_mla_fwd_paged_fp8 if fp8 else dsa.sparse_mla_fwd_paged

        def step():
            fwd(d["q"], d["kv_pages"], d["page_table"], d["seq_lens"], d["indices"], d["sm_scale"],
                d["q_per_seq"], out=out, lse=lse, num_splits=num_splits, workspace=ws)
    return {"row_bytes": FP8_ROW_BYTES if fp8 else ROW_BYTES, "w": w, "d": d, "d_host": d_host if gen_dev == "cpu" else d, "T": T, "H": H, "topk": topk,
            "splits": splits, "out": out, "lse": lse, "ws": ws, "step": step, "V": valid_keys(d)}


def fwd_leg(name: str, dev, stream, steps: int, warmup: int, flush: bool):
    """A second forward workload timed inside the same run: kernel time and its
    rate against the roofline that bounds it (MFMA above 16 heads, HBM at or
    below), warm and, with flush, with cold caches."""
    import torch
    f = fwd_setup(name, dev)
    V, H = f["V"], f["H"]
    flops = V * H * FLOP_PER_KEY_HEAD
    gathered = V * f["row_bytes"]
    avg, med, wall = time_steps(f["step"], steps, warmup, stream)
    rec = {"workload": f["w"].desc, "num_tokens": f["T"], "num_heads": H, "valid_keys": V,
           "splits": f["splits"], "kernel_ms_avg": round(avg, 5), "kernel_ms_median": round(med, 5),
           "tflops": round(flops / (avg * 1e-3) / 1e12, 2),
           "gathered_kv_gbps": round(gathered / (avg * 1e-3) / 1e9, 1)}
    if H > 16:
        rec["mfma_frac"] = round(rec["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)
    else:
        rec["hbm_frac"] = round(rec["gathered_kv_gbps"] / HBM_PEAK_GBPS, 4)
    if flush:
        fl = time_flushed(f["step"], steps, dev, stream)
        rec["kernel_ms_flushed"] = round(fl, 5)
        rec["gathered_kv_gbps_flushed"] = round(gathered / (fl * 1e-3) / 1e9, 1)
        rec["hbm_frac_flushed"] = round(rec["gathered_kv_gbps_flushed"] / HBM_PEAK_GBPS, 4)
        fd = time_flushed(f["step"], steps, dev, stream, dirty=True)
        rec["kernel_ms_flushed_dirty"] = round(fd, 5)
        rec["hbm_frac_flushed_dirty"] = round(gathered / (fd * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
    t = traffic_for(name)
    if t is not None:
        rec["hbm_traffic_bytes"] = t
    del f
    torch.cuda.empty_cache()
    return rec


def topk_setup(name: str, dev):
    """Index-selection inputs shaped like a workload: prefill rows select from
    their causal prefix (their document's, when packed), decode rows from
    their context; N(0,1) stand-in scores."""
    import numpy as np
    import torch
    import workloads
    w = workloads.WORKLOADS[name]
    if w.kind == "paged":
        lens = workloads.decode_lengths()
        Q = w.extra["q_per_seq"]
        T = lens.shape[0] * Q
        ke = torch.tensor([int(lens[t // Q]) - Q + (t % Q) + 1 for t in range(T)], dtype=torch.int32)
        ks = torch.zeros(T, dtype=torch.int32)
        C = int(lens.max())
    else:
        T = w.num_tokens
        cu = workloads.varlen_cu_seqlens(name) if name.startswith("varlen") else None
        ks, ke = workloads.causal_ranges(cu, T)
        C = T
    scores = workloads.index_scores(T, C, seed=w.seed + 500, device=dev)
    n = np.maximum(ke.numpy().astype(np.int64) - ks.numpy(), 0)
    scored = int(n[n > w.topk].sum())
    return {"w": w, "T": T, "C": C, "ks": ks.to(dev), "ke": ke.to(dev), "scores": scores, "topk": w.topk,
            "scored": scored, "rows_scored": int((n > w.topk).sum())}


def cpu_baseline_topk(tk, budget_s: float):
    """Time the selection oracle on the last rows until ~budget_s."""
    import numpy as np
    from oracle import topk_indices_ref
    ks, ke = tk["ks"].cpu().numpy(), tk["ke"].cpu().numpy()
    T, k = tk["T"], tk["topk"]
    done = rows = 0
    elapsed = 0.0
    t_end = T
    while elapsed < budget_s and t_end > 0:
        a, b = max(0, t_end - 16), t_end
        sc = tk["scores"][a:b].cpu().numpy()
        t0 = time.perf_counter()
        topk_indices_ref(sc, ks[a:b], ke[a:b], k, num_cols=tk["C"])
        elapsed += time.perf_counter() - t0
        n = np.maximum(ke[a:b].astype(np.int64) - ks[a:b], 0)
        done += int(n[n > k].sum())
        rows += b - a
        t_end = a
    info = host_info()
    return {"value": round(done * 4 / elapsed / 1e9, 4), "unit": "GB/s",
            "cores": info["blas"]["threads"] if info.get("blas") else info["cores"], "kind": "oracle",
            "sample": f"last {rows} of {T} rows ({done} scored candidates), numpy lexsort, {elapsed:.1f} s",
            "cpu_model": info["cpu_model"]}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="swe",
                    choices=["short", "swe", "wide", "varlen16k", "varlen32k", "decode", "decode_fp8"])
    ap.add_argument("--op", default="fwd", choices=["fwd", "bwd", "topk"],
                    help="fwd (the headline metric), the backward (flat workloads), or the top-k "
                         "index selection over the workload's candidate ranges")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for cpu_baseline (0 skips it)")
    ap.add_argument("--flush", action="store_true",
                    help="also time launches with cold caches: kernel_ms_flushed after a 512 MB write "
                         "and a 512 MB read between launches (clean caches), kernel_ms_flushed_dirty "
                         "after the write alone (its dirty lines are written back inside the launch)")
    ap.add_argument("--no-legs", action="store_true",
                    help="fwd only: skip the wide-head and flushed-decode legs (for profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a copy of known size (for HBM counter scaling)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="host only: store HBM bytes per launch from two counter runs")
    ap.add_argument("--traffic-command", default="",
                    help="the profiling command, recorded with --summarize-traffic")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_LOG"),
                    help="host only: write profiles/<op>_<workload>_kernel_trace.md from a rocprofv3 "
                         "--kernel-trace --stats run of this script (its -d directory, -o kt) and its output")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="host only: write profiles/counters_<op>_<workload>.json from rocprofv3 --pmc runs")
    args = ap.parse_args()

    if args.summarize_traffic:
        summarize_traffic(args.workload, *args.summarize_traffic, args.traffic_command, args.op)
        return
    if args.summarize_trace:
        summarize_trace(args, *args.summarize_trace)
        return
    if args.summarize_counters:
        summarize_counters(args, args.summarize_counters)
        return

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(this path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import torch

    import dsa_sparse_mla_amd as dsa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    if args.op == "topk":
        tk = topk_setup(args.workload, dev)
        idx = torch.empty((tk["T"], tk["topk"]), dtype=torch.int32, device=dev)

        def step():
            dsa.topk_indices(tk["scores"], tk["ks"], tk["ke"], tk["topk"], indices=idx)

        if args.copy_calibration:
            copy_calibration(dev)
        avg, med, wall = time_steps(step, args.steps, args.warmup, stream)
        moved = tk["scored"] * 4 + tk["T"] * (4 * tk["topk"] + 8)
        gbps = moved / (wall * 1e-3) / 1e9
        kern = moved / (avg * 1e-3) / 1e9
        rec = {"metric": "DSA top-k index selection GB/s (scores read + index rows written, % HBM)",
               "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
               "warmup": args.warmup, "ms_per_step": round(wall, 5), "higher_is_better": True,
               "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
               "config": {"workload": f"top-k over {tk['w'].desc} candidate ranges", "name": tk["w"].name,
                          "op": "topk", "num_tokens": tk["T"], "num_cols": tk["C"], "topk": tk["topk"],
                          "rows_scored": tk["rows_scored"], "scored_candidates": tk["scored"]},
               "kernel_ms_avg": round(avg, 5), "kernel_ms_median": round(med, 5),
               "roofline": {"bound": "hbm", "achieved": round(kern, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": round(kern / HBM_PEAK_GBPS, 4), "traffic": traffic_for(args.workload, "topk")},
               "source_hash": source_hash("topk")}
        if args.cpu_budget > 0:
            rec["cpu_baseline"] = cpu_baseline_topk(tk, args.cpu_budget)
        print(json.dumps(rec), flush=True)
        return

    f = fwd_setup(args.workload, dev, args.num_splits)
    d, T, H, V = f["d"], f["T"], f["H"], f["V"]
    gathered = V * f["row_bytes"]
    flops = V * H * FLOP_PER_KEY_HEAD
    step = f["step"]

    if args.op == "bwd":
        if "kv" not in d:
            print("the backward runs on flat workloads only", file=sys.stderr)
            sys.exit(2)
        g = torch.Generator(device=dev).manual_seed(12345)
        dout = torch.randn((T, H, 512), generator=g, device=dev).to(torch.bfloat16)
        f["step"]()   # the forward supplies out and LSE
        out, lse = f["out"], f["lse"]
        dq = torch.empty((T, H, 576), dtype=torch.float32, device=dev)
        dkv = torch.empty((d["kv"].shape[0], 576), dtype=torch.float32, device=dev)
        bwd_schedule, bwd_ws_bytes = dsa.bwd_workspace_size(T, H, d["kv"].shape[0], f["topk"])
        bwd_ws = torch.empty(max(bwd_ws_bytes, 256), dtype=torch.uint8, device=dev)

        def step():
            dsa.sparse_mla_bwd(d["q"], d["kv"], d["indices"], d["sm_scale"], out, lse, dout,
                               dq=dq, dkv=dkv, workspace=bwd_ws)

    if args.copy_calibration:
        copy_calibration(dev)
    avg_ms, med_ms, ms_per_step = time_steps(step, args.steps, args.warmup, stream)
    flushed_ms = time_flushed(step, args.steps, dev, stream) if args.flush else None
    flushed_dirty_ms = time_flushed(step, args.steps, dev, stream, dirty=True) if args.flush else None

    if args.op == "bwd":
        gathered = V * BWD_BYTES_PER_KEY
        flops = V * H * BWD_FLOP_PER_KEY_HEAD
    gbps = gathered / (ms_per_step * 1e-3) / 1e9
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    kern_gbps = gathered / (avg_ms * 1e-3) / 1e9
    kern_tflops = flops / (avg_ms * 1e-3) / 1e12
    traffic = traffic_for(args.workload, args.op)
    if H <= 16:
        roof = {"bound": "hbm", "achieved": round(kern_gbps, 2), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(kern_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic}
        if traffic is not None:
            # the counters' bytes beyond the L2 over the same launch time: at or
            # near the gathered rate only when the rows really come from HBM
            roof["traffic_gbps"] = round(traffic / (avg_ms * 1e-3) / 1e9, 1)
            roof["traffic_frac"] = round(roof["traffic_gbps"] / HBM_PEAK_GBPS, 4)
            if traffic < 0.25 * gathered:
                roof["served_from"] = ("L2/MALL: the gathered rows are cache-resident (counter traffic is "
                                       f"{100 * traffic / gathered:.1f}% of the gathered bytes); "
                                       "decode_flushed is the HBM-bound case")
    else:
        roof = {"bound": "mfma", "achieved": round(kern_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(kern_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic}

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
        "config": {"workload": f["w"].desc, "name": f["w"].name, "num_tokens": T, "num_heads": H,
                   "topk": f["topk"], "dqk": 576, "dv": 512, "valid_keys": V, "splits": f["splits"]},
        "tflops": round(tflops, 3),
        "gathered_kv_gbps": round(gbps, 2),
        "kernel_ms_avg": round(avg_ms, 5),
        "kernel_ms_median": round(med_ms, 5),
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "pct_mfma_peak": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 3),
        "roofline": roof,
        **({"kernel_ms_flushed": round(flushed_ms, 5),
            "gathered_kv_gbps_flushed": round(gathered / (flushed_ms * 1e-3) / 1e9, 2),
            "kernel_ms_flushed_dirty": round(flushed_dirty_ms, 5)}
           if flushed_ms is not None else {}),
        "source_hash": source_hash(args.op),
    }
    if args.op == "bwd":
        rec["config"]["op"] = "bwd"
        rec["config"]["schedule"] = bwd_schedule
        rec["bytes_per_key"] = BWD_BYTES_PER_KEY
    cpu_src = f["d_host"]
    del f
    if args.op == "fwd" and not args.no_legs and args.workload == "swe":
        # the other half of the metric (TFLOP/s at 64 heads) and the HBM-bound
        # 8-head case with cold caches, measured in the same run
        legs_steps = max(3, min(args.steps, 10))
        torch.cuda.empty_cache()
        rec["wide"] = fwd_leg("wide", dev, stream, legs_steps, 2, flush=False)
        rec["decode_flushed"] = fwd_leg("decode", dev, stream, legs_steps, 2, flush=True)
        rec["decode_fp8_flushed"] = fwd_leg("decode_fp8", dev, stream, legs_steps, 2, flush=True)
    rec["gpu"] = gpu_info(dev)
    if args.cpu_budget > 0:
        if args.op == "bwd":
            rec["cpu_baseline"] = cpu_baseline_bwd(cpu_src, dout, args.cpu_budget)
        else:
            rec["cpu_baseline"] = cpu_baseline_full(cpu_src, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
