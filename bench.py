"""Throughput of the rank-local TSP layer forward on one MI355X.

Default workload: one decoder layer of the 7B dense model the TSP pages
validate (hidden 4096, 32 heads of 128, MLP 16384, bf16) at S = 131072 tokens
on a folded axis of D = 8, rank 0: 16384 local zigzag tokens, all 8 weight
shards applied in delivery order, attention against the full gathered K/V
(the other ranks' rows are seeded N(0,1) inputs). One step = one
tsp_layer_fwd call; inputs are resident in HBM before timing starts.

Prints ONE JSON line: local tokens/s, ms per step, the fraction of bf16 MFMA
peak over the layer, the roofline entry of the dominant kernel (attention,
timed per launch with HIP events on the launching stream) and the CPU oracle
timed on a bounded sample of the same workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload layer|mlp|attn]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "local tokens/s per GPU, 7B TSP layer fwd D=8 S=128K; % bf16 MFMA peak"
PEAK_BF16 = 2.5e15   # MI355X dense bf16/fp16 MFMA, flop/s
PEAK_HBM = 8.0e12    # bytes/s


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def attn_pairs(S, D, r):
    """Unmasked (query, key) pairs of rank r: sum over local rows of pos + 1."""
    C = S // (2 * D)
    pos0 = r * C + np.arange(C, dtype=np.int64)
    pos1 = (2 * D - 1 - r) * C + np.arange(C, dtype=np.int64)
    return int((pos0 + 1).sum() + (pos1 + 1).sum())


def layer_flops(sh, r):
    N = sh.N
    qkv = 2 * N * sh.h * (sh.H + 2 * sh.kv_heads) * sh.Dh
    attn = 4 * sh.Dh * sh.H * attn_pairs(sh.S, sh.D, r)
    outp = 2 * N * sh.h * sh.h
    mlp = (3 if sh.mlp == "swiglu" else 2) * 2 * N * sh.h * sh.F  # gated: gate, up and down products
    return {"qkv": qkv, "attention": attn, "outproj": outp, "mlp": mlp, "total": qkv + attn + outp + mlp}


# Kernel classes of the layer step whose HBM bytes the traffic summary
# records: (class, substring of the kernel name, which dispatch of that name
# within a step when one name serves two classes, source file).
# Names appear demangled or mangled in the counter files, so a class is
# matched by substrings that must all be present.
TRAFFIC_KERNELS = (
    ("attention", ("attn_bf16_kernel<128, false, true",), None, "attention.hip"),
    ("qkv", ("gemm_bf16_kernel", "EpiQKV"), None, "gemm.hip"),
    ("outproj", ("gemm_bf16_kernel", "EpiAddF32"), 0, "gemm.hip"),
    ("mlp_down", ("gemm_bf16_kernel", "EpiAddF32"), 1, "gemm.hip"),
    ("mlp_up", ("gemm_bf16_kernel", "EpiGelu"), None, "gemm.hip"),
    ("rmsnorm", ("rmsnorm_kernelIDF16bDF16b",), None, "rows.hip"),
)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "layer7b_hbm_traffic.txt")
TRAFFIC_PASSES = (
    "TCC_BUBBLE_sum TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_DRAM_32B_sum GRBM_GUI_ACTIVE",
    "TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_64B_sum TCC_EA0_WRREQ_WRITE_DRAM_32B_sum GRBM_GUI_ACTIVE",
)


def _src_sha(name):
    return hashlib.sha256(open(os.path.join(ROOT, "tsp_rank_local_amd", "csrc", name), "rb").read()).hexdigest()


def traffic_from_profile():
    """{kernel class: HBM bytes per launch} from the committed counter
    summary, for the classes whose kernel source is unchanged since the
    counters were taken (the others are left out)."""
    if not os.path.exists(TRAFFIC_FILE):
        return {}
    out, sha = {}, {}
    for line in open(TRAFFIC_FILE):
        if line.startswith("source_sha256 "):
            _, name, h = line.split()
            sha[name] = h
        elif line.startswith("hbm_bytes "):
            _, cls, v = line.split()
            out[cls] = float(v)
    srcs = {cls: src for cls, _, _, src in TRAFFIC_KERNELS}
    return {cls: v for cls, v in out.items() if cls in srcs and sha.get(srcs[cls]) == _src_sha(srcs[cls])}


SQ_FILE = os.path.join(ROOT, "profiles", "layer7b_sq_counters.txt")


def sq_from_profile():
    """{kernel class: {"sclk_ghz", "mfma_busy"}} from the committed shader
    counter summary of the layer step, for the classes of TRAFFIC_KERNELS
    whose source is unchanged since the counters were taken. The output
    projection and the MLP down product share one kernel name there, so
    they get the average of the two."""
    if not os.path.exists(SQ_FILE):
        return {}
    sha, rows = {}, []
    for line in open(SQ_FILE):
        if line.startswith("source_sha256 "):
            _, name, h = line.split()
            sha[name] = h
        elif " | " in line and not line.startswith(("#", "kernel |")):
            rows.append([c.strip() for c in line.split(" | ")])
    out = {}
    for cls, subs, _, src in TRAFFIC_KERNELS:
        if sha.get(src) != _src_sha(src):
            continue
        for r in rows:
            if all(x in r[0] for x in subs) and r[1] != "-" and r[2] != "-":
                out[cls] = {"sclk_ghz": float(r[1]), "mfma_busy": float(r[2])}
                break
    return out


def summarize_traffic(csvs, copy_mib):
    """HBM bytes per launch of the layer step's kernels from the L2-to-memory
    request counters of rocprofv3 (two passes, TRAFFIC_PASSES).

    Reads: the requests the L2 sends to the data fabric, by size, give
    FETCH_SIZE (128-byte requests x 128 + 64-byte x 64 + 32-byte x 32); the
    requests due to DRAM, counted in 32-byte units whatever their size, give
    the DRAM read bytes. Writes: WRITE_SIZE (64-byte requests x 64, the rest
    x 32) and the DRAM write requests in 32-byte units. The plain device copy
    of copy_mib MiB that --copy-mib runs before warmup calibrates each: its
    known bytes divided by what the counter reads. The bytes recorded per
    kernel are the DRAM counts times their copy factors."""
    import csv
    per = {}  # (kernel, dispatch) -> {counter: value}
    order = {}
    for path in csvs:
        for row in csv.DictReader(open(path)):
            key = (row["Kernel_Name"], int(row["Dispatch_Id"]))
            per.setdefault(key, {})[row["Counter_Name"]] = float(row["Counter_Value"])
    for name, disp in sorted(per, key=lambda k: k[1]):
        order.setdefault(name, []).append(disp)

    def derived(c):
        d = {}
        if "TCC_EA0_RDREQ_sum" in c:
            b, rq, r32 = c.get("TCC_BUBBLE_sum", 0.0), c["TCC_EA0_RDREQ_sum"], c.get("TCC_EA0_RDREQ_32B_sum", 0.0)
            d["fetch"] = b * 128 + (rq - b - r32) * 64 + r32 * 32
            d["req128"], d["req32"], d["req"] = b, r32, rq
        if "FETCH_SIZE" in c:  # the derived counter itself (KiB)
            d.setdefault("fetch", 1024 * c["FETCH_SIZE"])
        if "WRITE_SIZE" in c:
            d.setdefault("write", 1024 * c["WRITE_SIZE"])
        if "TCC_EA0_RDREQ_DRAM_32B_sum" in c:
            d["dram_rd"] = 32 * c["TCC_EA0_RDREQ_DRAM_32B_sum"]
        if "TCC_EA0_WRREQ_sum" in c:
            w, w64 = c["TCC_EA0_WRREQ_sum"], c.get("TCC_EA0_WRREQ_64B_sum", 0.0)
            d["write"] = (w - w64) * 32 + w64 * 64
        if "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum" in c:
            d["dram_wr"] = 32 * c["TCC_EA0_WRREQ_WRITE_DRAM_32B_sum"]
        return d

    # the copy: the largest dispatch of the runtime's copy kernel in each pass
    copy = {}
    for (name, disp), c in per.items():
        if "copyBuffer" not in name:
            continue
        for k, v in derived(c).items():
            copy[k] = max(copy.get(k, 0.0), v)
    nbytes = float(copy_mib) * (1 << 20)
    scale = {k: nbytes / copy[k] for k in ("fetch", "dram_rd", "write", "dram_wr") if copy.get(k)}

    def avg(dicts, k):
        v = [d[k] for d in dicts if k in d]
        return sum(v) / len(v) if v else None

    lines = [
        "# HBM traffic per launch of the 7B layer step's kernels (rank 0 of D=8, S=131072), from rocprofv3 counters.",
        "# Made by (one step each; the 1 GiB device copy run before warmup calibrates the counters):",
    ]
    for i, ctrs in enumerate(TRAFFIC_PASSES):
        lines.append(f"#   rocprofv3 --pmc {ctrs} -d <dir{i + 1}> -o run --output-format csv -- "
                     "python bench.py --steps 1 --warmup 0 --cpu-rows 0 --copy-mib 1024")
    lines += [
        "#   python bench.py --summarize-traffic <dir1>/run_counter_collection.csv <dir2>/run_counter_collection.csv",
        "# fetch: L2->fabric read requests by size (128/64/32 B); dram_rd, dram_wr: DRAM requests in 32-byte units;",
        "# write: write requests (64 B or 32 B). Copy factor = copy bytes / counter bytes for the 1 GiB copy.",
        "# hbm_bytes <class> = dram_rd x its copy factor + dram_wr x its copy factor (per launch).",
    ]
    for k in ("fetch", "dram_rd", "write", "dram_wr"):
        if k in copy:
            lines.append(f"copy {k}: {copy[k]:.6g} bytes for {nbytes:.6g}; factor {scale.get(k, float('nan')):.4f}")
    for cls, key, which, src in TRAFFIC_KERNELS:
        names = [n for n in order if all(k in n for k in key)]
        if len(names) != 1:
            continue
        disps = order[names[0]]
        if which is not None:  # dispatch `which` of every step (dispatches alternate between the classes)
            disps = disps[which::2]
        rows = [derived(per[(names[0], d)]) for d in disps]
        f, dr, w, dw = avg(rows, "fetch"), avg(rows, "dram_rd"), avg(rows, "write"), avg(rows, "dram_wr")
        r128, r32, rq = avg(rows, "req128"), avg(rows, "req32"), avg(rows, "req")
        split = (f"{100 * r128 / rq:.1f}/{100 * (rq - r128 - r32) / rq:.1f}/{100 * r32 / rq:.1f}"
                 if rq else "-")
        lines.append(f"kernel {cls}: {names[0][:90]}")
        g = (lambda x: "-" if x is None else f"{x:.6g}")  # noqa: E731
        lines.append(f"  fetch {g(f)}  dram_rd {g(dr)}  write {g(w)}  dram_wr {g(dw)}  "
                     f"read requests 128/64/32 B (%) {split}")
        if dr is not None and dw is not None and "dram_rd" in scale and "dram_wr" in scale:
            lines.append(f"hbm_bytes {cls} {dr * scale['dram_rd'] + dw * scale['dram_wr']:.6g}")
    for src in sorted({t[3] for t in TRAFFIC_KERNELS}):
        lines.append(f"source_sha256 {src} {_src_sha(src)}")
    with open(TRAFFIC_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


KTRACE_WORKLOADS = {
    # workload -> (title, summary file, bench arguments)
    "layer": ("one 7B TSP layer forward (rank 0 of D=8, S=131072, 16384 local tokens, bf16)",
              "attn_layer7b_kernel_stats.md", ""),
    "layer_bwd": ("one 7B TSP layer backward, both halves (rank 0 of D=8, S=131072, 16384 local tokens, bf16)",
                  "layer_bwd_7b_kernel_stats.md", "--workload layer_bwd --steps 5 --warmup 1"),
    "train": ("one 7B TSP layer training step: the forward keeping the attention output and statistics, both "
              "halves of the backward from them (rank 0 of D=8, S=131072, 16384 local tokens, bf16)",
              "train_7b_kernel_stats.md", "--workload train --steps 5 --warmup 1"),
    "attn_bwd": ("the 7B zigzag attention backward, statistics recomputed, P and dS as hi + lo (rank 0 of D=8, "
                 "S=131072, 32 heads x 128, bf16)", "attn_bwd_7b_kernel_stats.md",
                 "--workload attn_bwd --steps 3 --warmup 1"),
    "attn_bwd_lse": ("the 7B zigzag attention backward from the forward's statistics, P and dS as hi + lo (rank 0 of "
                     "D=8, S=131072, 32 heads x 128, bf16)", "attn_bwd_lse_7b_kernel_stats.md",
                     "--workload attn_bwd_lse --steps 3 --warmup 1"),
    "attn_bwd_lse_plain": ("the 7B zigzag attention backward from the forward's statistics, P and dS rounded once to "
                           "bf16, the layer backward's call (rank 0 of D=8, S=131072, 32 heads x 128, bf16)",
                           "attn_bwd_lse_plain_7b_kernel_stats.md",
                           "--workload attn_bwd_lse --plain-pds --steps 3 --warmup 1"),
    "mlp_bwd": ("the 7B MLP ring backward, Z recomputed (16384 tokens, h 4096, F 16384, D=8, bf16)",
                "mlp_bwd_7b_kernel_stats.md", "--workload mlp_bwd --steps 10 --warmup 2"),
    "mlp_bwd_z": ("the 7B MLP ring backward from the forward's Z (16384 tokens, h 4096, F 16384, D=8, bf16)",
                  "mlp_bwd_z_7b_kernel_stats.md", "--workload mlp_bwd_z --steps 10 --warmup 2"),
}


def summarize_ktrace(stats_csv, bench_json, workload="layer"):
    """Markdown summary of a rocprofv3 --kernel-trace --stats run of the
    benchmark: per-kernel launches and durations from the profiler, beside
    the same run's own HIP-event figures (its JSON line)."""
    import csv
    title, fname, bench_args = KTRACE_WORKLOADS[workload]
    rows = list(csv.DictReader(open(stats_csv)))
    b = json.loads([ln for ln in open(bench_json).read().splitlines() if ln.startswith("{")][-1])
    cmd = ("rocprofv3 --kernel-trace --stats -d <dir> -o run --output-format csv -- python bench.py" +
           (f" {bench_args}" if bench_args else ""))
    lines = [f"# Kernel time, {title}", "", "Command (run from the repository root on one MI355X):", "",
             f"    {cmd}", "",
             f"`run_kernel_stats.csv` ({b['warmup']} warmup + {b['steps']} timed + {b['steps']} per-step steps):", "",
             "| kernel | calls | avg ms | min ms | max ms | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['Name'][:110]} | {r['Calls']} | {float(r['AverageNs']) / 1e6:.3f} | "
                     f"{float(r['MinNs']) / 1e6:.3f} | {float(r['MaxNs']) / 1e6:.3f} | {float(r['Percentage']):.1f}% |")
    k = b.get("kernels", {})
    lines += ["", "Same run, bench.py's HIP events on the launching stream:", ""]
    lines.append(f"- step: {b['ms_per_step']:.3f} ms, {b['value']:,.0f} local tokens/s, "
                 f"{b['pct_bf16_mfma_peak']:.1f}% of the 2.5 PF bf16 peak over the step")
    for name, v in k.items():
        extra = f", {v['hbm_gb_s']:.0f} GB/s of HBM traffic" if "hbm_gb_s" in v else ""
        lines.append(f"- {name}: {v['ms_per_launch']:.3f} ms per launch, {v['launches_per_step']:g} per step{extra}")
    rf = b.get("roofline") or {}
    if rf:
        lines.append(f"- roofline ({rf['kernel']}): {rf['achieved']:.0f} {rf['unit']} of {rf['peak']:.0f}, "
                     f"frac {rf['frac']:.3f}; traffic {rf['traffic']}")
    bwd = [r for r in rows if "attn_bwd_" in r["Name"]]
    if bwd and "attn_bwd" in k:
        b_ms = sum(float(r["AverageNs"]) for r in bwd) / 1e6
        lines.append(f"- attention backward: profiler averages of its kernels add to {b_ms:.3f} ms vs HIP events "
                     f"{k['attn_bwd']['ms_per_launch']:.3f} ms per call "
                     f"({100 * (k['attn_bwd']['ms_per_launch'] / b_ms - 1):+.1f}%)")
    att = [r for r in rows if "attn_bf16_kernel" in r["Name"]]
    if att and "attention" in k:
        a_ms = float(att[0]["AverageNs"]) / 1e6
        lines.append(f"- attention: profiler average {a_ms:.3f} ms vs HIP events {k['attention']['ms_per_launch']:.3f} "
                     f"ms ({100 * (k['attention']['ms_per_launch'] / a_ms - 1):+.1f}%)")
    out = os.path.join(ROOT, "profiles", fname)
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:  # pragma: no cover
        pass
    return len(os.sched_getaffinity(0))


SQ_PASSES = (
    "SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU_TRANS_F32 "
    "SQ_ACTIVE_INST_LDS SQ_WAIT_INST_LDS GRBM_GUI_ACTIVE",
    "SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_WAIT_ANY SQ_ACTIVE_INST_ANY SQ_BUSY_CU_CYCLES "
    "GRBM_GUI_ACTIVE",
)


# workload -> (title, summary file, the bench arguments of the counter runs)
SQ_WORKLOADS = {
    "layer": ("the default layer step (7B, rank 0 of D=8, S=131072)", "layer7b_sq_counters.txt",
              "--steps 1 --warmup 0 --cpu-rows 0"),
    "attn_bwd": ("the 7B zigzag attention backward (rank 0 of D=8, S=131072)", "attn_bwd_7b_sq_counters.txt",
                 "--workload attn_bwd --steps 1 --warmup 0"),
    "mlp_bwd": ("the 7B MLP ring backward (16384 tokens, D=8)", "mlp_bwd_7b_sq_counters.txt",
                "--workload mlp_bwd --steps 1 --warmup 0"),
    "layer_bwd": ("the 7B layer backward, both halves (rank 0 of D=8, S=131072)", "layer_bwd_7b_sq_counters.txt",
                  "--workload layer_bwd --steps 1 --warmup 0"),
}


def summarize_sq(csvs, workload="layer"):
    """Per-kernel shader counters of one workload's step: fractions of the
    kernel's cycles per SIMD (cycles = GRBM_GUI_ACTIVE / 8 XCDs, 1024 SIMDs),
    instruction mixes per MFMA. One line per kernel, averaged over dispatches."""
    title, fname, bench_args = SQ_WORKLOADS[workload]
    import csv
    per = {}  # (kernel, dispatch) -> {counter: value}
    for path in csvs:
        for row in csv.DictReader(open(path)):
            key = (path, row["Kernel_Name"], row["Dispatch_Id"])
            per.setdefault(key, {})[row["Counter_Name"]] = float(row["Counter_Value"])
            per[key]["_ns"] = float(row["End_Timestamp"]) - float(row["Start_Timestamp"])
    kern = {}
    for (_, name, _), c in per.items():
        if "GRBM_GUI_ACTIVE" not in c or "copyBuffer" in name:
            continue
        simd = 1024.0 * c["GRBM_GUI_ACTIVE"] / 8.0
        f = {}

        def put(key, num, den=1.0, scale=1.0):
            if num in c and (den == 1.0 or den in c):
                f[key] = scale * c[num] / (simd if den == 1.0 else max(c[den], 1.0))

        # effective shader clock: the kernel's cycles (per XCD) over its duration
        if c.get("_ns", 0.0) > 0:
            f["sclk_ghz"] = c["GRBM_GUI_ACTIVE"] / 8.0 / c["_ns"]
        put("mfma_busy", "SQ_VALU_MFMA_BUSY_CYCLES")
        put("valu_active", "SQ_ACTIVE_INST_VALU", scale=4.0)
        put("mfma_valu_coexec", "SQ_VALU_MFMA_COEXEC_CYCLES")
        put("lds_active", "SQ_ACTIVE_INST_LDS", scale=4.0)
        put("lds_wait", "SQ_WAIT_INST_LDS")
        if c.get("SQ_INSTS_MFMA", 0.0) > 0:
            put("trans_per_mfma", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_MFMA")
        put("bank_conflicts_per_lds_inst", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS")
        for k, n in (("_mfma", "SQ_INSTS_MFMA"), ("_valu", "SQ_INSTS_VALU"), ("_salu", "SQ_INSTS_SALU"),
                     ("_lds", "SQ_INSTS_LDS")):
            if n in c:
                f[k] = c[n]
        kern.setdefault(name, []).append(f)
    lines = [f"# Shader counters of {title}, per kernel.",
             "# Made by (one step, two passes, each within one pass's counter limits):"]
    for i, ctrs in enumerate(SQ_PASSES):
        lines.append(f"#   rocprofv3 --pmc {ctrs} -d <dir{i + 1}> -o run --output-format csv -- "
                     f"python bench.py {bench_args}")
    wl = "" if workload == "layer" else f" --workload {workload}"
    lines += [f"#   python bench.py --summarize-sq <dir1>/run_counter_collection.csv <dir2>/run_counter_collection.csv{wl}",
              "# Fractions are of the kernel's cycles per SIMD (GRBM_GUI_ACTIVE / 8 XCDs, x 1024 SIMDs);",
              "# SQ_ACTIVE_INST_* count 4-cycle units. Instruction ratios are per MFMA instruction.",
              "# sclk: effective shader clock, GRBM_GUI_ACTIVE / 8 XCDs / the dispatch's duration (GHz);",
              "# mfma_tflops: mfma_busy x sclk x 256 CUs x 4096 flop per CU-cycle (dense bf16 rate at that busy share).",
              "kernel | sclk | mfma_busy | mfma_tflops | valu_active | coexec | lds_active | lds_wait | valu/mfma | "
              "salu/mfma | lds/mfma | trans/mfma | bank_conflicts/lds"]
    order = sorted(kern, key=lambda n: -len(kern[n]))
    for name in order:
        rows = kern[name]

        def avg(k):
            v = [r[k] for r in rows if k in r]
            return sum(v) / len(v) if v else None

        mf, va, sa, ld = avg("_mfma"), avg("_valu"), avg("_salu"), avg("_lds")
        ratio = (lambda x: f"{x / mf:.2f}" if (x is not None and mf) else "-")

        def fmt(k):
            v = avg(k)
            return "-" if v is None else f"{v:.3f}"

        mb, ck = avg("mfma_busy"), avg("sclk_ghz")
        tf = f"{mb * ck * 1e9 * 256 * 4096 / 1e12:.0f}" if (mb is not None and ck is not None) else "-"
        lines.append(f"{name[:80]} | {fmt('sclk_ghz')} | {fmt('mfma_busy')} | {tf} | {fmt('valu_active')} | "
                     f"{fmt('mfma_valu_coexec')} | "
                     f"{fmt('lds_active')} | {fmt('lds_wait')} | {ratio(va)} | {ratio(sa)} | {ratio(ld)} | "
                     f"{fmt('trans_per_mfma')} | {fmt('bank_conflicts_per_lds_inst')}")
    # the kernel sources the counters were taken on (bench.py reads a
    # kernel's clock from here only while its source is unchanged)
    for src in ("attention.hip", "attention_bwd.hip", "gemm.hip", "lead.hip", "rows.hip"):
        lines.append(f"source_sha256 {src} {_src_sha(src)}")
    out = os.path.join(ROOT, "profiles", fname)
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", choices=["layer", "mlp", "attn", "layers32", "mlp_bwd", "mlp_bwd_z", "attn_bwd",
                                           "attn_bwd_lse", "layer_bwd", "train"], default="layer")
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--rope-base", type=float, default=0.0,
                    help="rotary embedding base for the layer workloads (0 = none, the pages' model)")
    ap.add_argument("--hkv", type=int, default=0,
                    help="K/V heads for the layer and attention workloads (grouped-query attention; 0 = 32, "
                         "multi-head as in the pages' model)")
    ap.add_argument("--mlp", choices=["gelu", "swiglu"], default="gelu",
                    help="MLP form for the layer and MLP workloads (gelu: the pages' two-matrix MLP)")
    ap.add_argument("--plain-pds", action="store_true",
                    help="attention backward workloads: P and dS rounded once to bf16 (TSP_ATTN_BWD_PLAIN_PDS) "
                         "instead of the hi + lo pair")
    ap.add_argument("--cpu-rows", type=int, default=384, help="rows in the CPU oracle sample (0 = skip)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="before warmup, run one plain device-to-device copy of this many MiB (a known-size "
                         "reference for rocprofv3 HBM byte counters)")
    ap.add_argument("--summarize-ktrace", nargs=2, metavar=("STATS_CSV", "BENCH_JSON"),
                    help="write the kernel-time summary of the workload under profiles/ from a rocprofv3 "
                         "--kernel-trace --stats run of bench.py (its run_kernel_stats.csv and JSON line)")
    ap.add_argument("--summarize-sq", nargs="+", metavar="CSV",
                    help="write profiles/layer7b_sq_counters.txt from rocprofv3 shader-counter csv files")
    ap.add_argument("--summarize-traffic", nargs="+", metavar="CSV",
                    help="write profiles/layer7b_hbm_traffic.txt from the rocprofv3 counter_collection.csv files of "
                         "the two traffic passes of a run with --copy-mib, then exit")
    args = ap.parse_args()
    if args.summarize_traffic:
        summarize_traffic(args.summarize_traffic, copy_mib=args.copy_mib or 1024)
        return
    if args.summarize_ktrace:
        summarize_ktrace(*args.summarize_ktrace, args.workload + ("_plain" if args.plain_pds else ""))
        return
    if args.summarize_sq:
        summarize_sq(args.summarize_sq, args.workload)
        return
    if args.gpus != 1:
        sys.exit(f"bench.py: only --gpus 1 is supported; this build measures one rank's share on one GPU "
                 f"(asked for {args.gpus}).")

    import torch

    import synth
    import tsp_rank_local_amd as tsp

    assert torch.cuda.is_available(), "needs a GPU"
    tsp.lib()
    mem0 = torch.cuda.memory_allocated()
    sh = dataclasses.replace(synth.SEVEN_B, Hkv=args.hkv, mlp=args.mlp)
    r = args.rank
    N = sh.N
    seed = 4
    t_gen = time.perf_counter()
    log(f"generating inputs: S={sh.S} D={sh.D} r={r} h={sh.h} H={sh.H} Hkv={sh.kv_heads} Dh={sh.Dh} F={sh.F}")
    shape = tsp.make_shape(sh.S, sh.D, r, sh.h, sh.H, sh.Dh, sh.F, eps=sh.eps, dtype="bf16",
                           rope_base=args.rope_base, Hkv=args.hkv, mlp=args.mlp)
    kv_note = f", {sh.kv_heads} K/V heads" if sh.kv_heads != sh.H else ""
    mlp_note = "SwiGLU FFN" if sh.mlp == "swiglu" else "FFN"
    stream = torch.cuda.current_stream()
    flops = layer_flops(sh, r)

    if args.workload in ("layer", "mlp", "mlp_bwd", "mlp_bwd_z", "layer_bwd", "train"):
        w = synth.layer_weights(sh, seed=seed)
        wd = {k: ([tsp.to_device(a, "bf16") for a in v] if isinstance(v, list) else tsp.to_device(v, "bf16"))
              for k, v in w.items()}
    if args.workload == "layer":
        x = synth.activations(N, sh.h, seed=seed)
        k_rem, v_rem = synth.remote_kv(sh, seed=seed)
        xd = tsp.to_device(x, "f32")
        kf, vf = tsp.to_device(k_rem, "bf16"), tsp.to_device(v_rem, "bf16")
        y = torch.empty((N, sh.h), dtype=torch.float32, device="cuda")
        ws = torch.empty(tsp.workspace_size(shape, tsp.TSP_WS_LAYER), dtype=torch.uint8, device="cuda")

        def step():
            tsp.tsp_layer_fwd(shape, wd, xd, kf, vf, y, tsp.TSP_PHASE_ALL, ws)
        step_flops = flops["total"]
        step_exps = sh.H * attn_pairs(sh.S, sh.D, r)
        workload = (f"tsp_layer_fwd: one 7B dense decoder layer (h=4096, 32x128 heads{kv_note}, {mlp_note} 16384, bf16) on "
                    f"rank {r} of D=8 at S=131072, 16384 local zigzag tokens")
    elif args.workload == "layer_bwd":
        # both halves of one rank's layer backward; the summed K/V-row
        # gradients the second half takes are seeded values (the
        # reduce-scatter that would deliver them is not on one GPU)
        x = synth.activations(N, sh.h, seed=seed)
        dy = synth.activations(N, sh.h, seed=seed, tid=synth.TID_DY)
        k_rem, v_rem = synth.remote_kv(sh, seed=seed)
        dkl = synth.normal((N, sh.kv_heads, sh.Dh), seed, synth.TID_DK_LOC, std=0.05)
        dvl = synth.normal((N, sh.kv_heads, sh.Dh), seed, synth.TID_DV_LOC, std=0.05)
        xd, dyd = tsp.to_device(x, "f32"), tsp.to_device(dy, "f32")
        kf, vf = tsp.to_device(k_rem, "bf16"), tsp.to_device(v_rem, "bf16")
        dkld, dvld = tsp.to_device(dkl, "f32"), tsp.to_device(dvl, "f32")
        dkf = torch.empty((sh.S, sh.kv_heads, sh.Dh), dtype=torch.float32, device="cuda")
        dvf = torch.empty_like(dkf)
        dx = torch.empty((N, sh.h), dtype=torch.float32, device="cuda")
        grads = {k: [torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in wd[k]]
                 for k in ("wqkv", "wo", "w1", "w2")}
        grads.update(g_attn=torch.empty(sh.h, dtype=torch.float32, device="cuda"),
                     g_mlp=torch.empty(sh.h, dtype=torch.float32, device="cuda"))
        ws = torch.empty(tsp.workspace_size(shape, tsp.TSP_WS_LAYER_BWD), dtype=torch.uint8, device="cuda")

        def step():
            tsp.tsp_layer_bwd(shape, wd, xd, kf, vf, dyd, dkf, dvf, None, None, None, grads, tsp.TSP_BWD_ATTN, ws)
            tsp.tsp_layer_bwd(shape, wd, xd, None, None, None, None, None, dkld, dvld, dx, grads, tsp.TSP_BWD_QKV,
                              ws)
        # algorithmic: the chain rule's products only, twice each forward GEMM
        # (input and weight gradient) and 2.5x the attention; the forward
        # recomputation (RMSNorms, Q, attention with its statistics, output
        # projection, the MLP's Z) is extra work, not counted
        step_flops = 2.0 * (flops["qkv"] + flops["outproj"] + flops["mlp"]) + 2.5 * flops["attention"]
        step_exps = 2 * sh.H * attn_pairs(sh.S, sh.D, r)
        workload = (f"tsp_layer_bwd: backward of one 7B dense decoder layer (h=4096, 32x128 heads{kv_note}, FFN 16384, "
                    f"bf16) on rank {r} of D=8 at S=131072, 16384 local zigzag tokens, both halves (forward "
                    f"recomputed from x; dx, dK/dV of every key row and all weight and gain gradients in fp32)")
    elif args.workload == "train":
        # one training step of the layer on one rank: the forward that keeps
        # the attention output and statistics and the MLP pre-activation, then
        # both halves of the backward that take them (no second attention
        # forward, no second MLP up product); the summed
        # K/V-row gradients of the second half are seeded values as above
        x = synth.activations(N, sh.h, seed=seed)
        dy = synth.activations(N, sh.h, seed=seed, tid=synth.TID_DY)
        k_rem, v_rem = synth.remote_kv(sh, seed=seed)
        dkl = synth.normal((N, sh.kv_heads, sh.Dh), seed, synth.TID_DK_LOC, std=0.05)
        dvl = synth.normal((N, sh.kv_heads, sh.Dh), seed, synth.TID_DV_LOC, std=0.05)
        xd, dyd = tsp.to_device(x, "f32"), tsp.to_device(dy, "f32")
        kf, vf = tsp.to_device(k_rem, "bf16"), tsp.to_device(v_rem, "bf16")
        dkld, dvld = tsp.to_device(dkl, "f32"), tsp.to_device(dvl, "f32")
        y = torch.empty((N, sh.h), dtype=torch.float32, device="cuda")
        o_sv = torch.empty((N, sh.H, sh.Dh), dtype=torch.float32, device="cuda")
        lse_sv = torch.empty((sh.H, N), dtype=torch.float32, device="cuda")
        z_sv = torch.empty((N, sh.F), dtype=torch.bfloat16, device="cuda")
        dkf = torch.empty((sh.S, sh.kv_heads, sh.Dh), dtype=torch.float32, device="cuda")
        dvf = torch.empty_like(dkf)
        dx = torch.empty((N, sh.h), dtype=torch.float32, device="cuda")
        grads = {k: [torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in wd[k]]
                 for k in ("wqkv", "wo", "w1", "w2")}
        grads.update(g_attn=torch.empty(sh.h, dtype=torch.float32, device="cuda"),
                     g_mlp=torch.empty(sh.h, dtype=torch.float32, device="cuda"))
        ws_f = torch.empty(tsp.workspace_size(shape, tsp.TSP_WS_LAYER), dtype=torch.uint8, device="cuda")
        ws = torch.empty(tsp.workspace_size(shape, tsp.TSP_WS_LAYER_BWD), dtype=torch.uint8, device="cuda")

        def step():
            tsp.tsp_layer_fwd_save(shape, wd, xd, kf, vf, y, o_sv, lse_sv, tsp.TSP_PHASE_ALL, ws_f, z_save=z_sv)
            tsp.tsp_layer_bwd_ex(shape, wd, xd, kf, vf, dyd, o_sv, lse_sv, dkf, dvf, None, None, None, grads,
                                 tsp.TSP_BWD_ATTN, ws, z_saved=z_sv)
            tsp.tsp_layer_bwd_ex(shape, wd, xd, None, None, None, None, None, None, None, dkld, dvld, dx, grads,
                                 tsp.TSP_BWD_QKV, ws)
        # algorithmic: the forward's flops and the backward's chain-rule products
        step_flops = flops["total"] + 2.0 * (flops["qkv"] + flops["outproj"] + flops["mlp"]) + 2.5 * flops["attention"]
        step_exps = 3 * sh.H * attn_pairs(sh.S, sh.D, r)
        workload = (f"tsp_layer_fwd_save + tsp_layer_bwd_ex: one training step of one 7B dense decoder layer (h=4096, "
                    f"32x128 heads{kv_note}, FFN 16384, bf16) on rank {r} of D=8 at S=131072, 16384 local zigzag "
                    f"tokens: the forward keeping the attention output and statistics and the MLP pre-activation, "
                    f"both halves of the backward from them")
    elif args.workload == "mlp":
        x = synth.activations(N, sh.h, seed=2, dtype="bf16")
        xd = tsp.to_device(x, "bf16")
        y = torch.empty((N, sh.h), dtype=torch.float32, device="cuda")
        ws = torch.empty(tsp.workspace_size(shape, tsp.TSP_WS_MLP), dtype=torch.uint8, device="cuda")

        def step():
            tsp.tsp_mlp_ring(shape, xd, wd["w1"], wd["w2"], None, y, ws)
        step_flops = flops["mlp"]
        step_exps = 0
        workload = (f"tsp_mlp_ring: 7B MLP ring ({mlp_note}), 16384x4096 bf16 local X, D=8 shards of "
                    f"{2 if sh.mlp == 'swiglu' else 1}x2048x4096 and 4096x2048")
    elif args.workload in ("mlp_bwd", "mlp_bwd_z"):
        x = synth.activations(N, sh.h, seed=2, dtype="bf16")
        dy = synth.activations(N, sh.h, seed=2, tid=synth.TID_DY, dtype="bf16")
        xd, dyd = tsp.to_device(x, "bf16"), tsp.to_device(dy, "bf16")
        fd = sh.F // sh.D
        dx = torch.empty((N, sh.h), dtype=torch.float32, device="cuda")
        dw1 = [torch.empty((fd, sh.h), dtype=torch.float32, device="cuda") for _ in range(sh.D)]
        dw2 = [torch.empty((sh.h, fd), dtype=torch.float32, device="cuda") for _ in range(sh.D)]
        ws = torch.empty(tsp.workspace_size(shape, tsp.TSP_WS_MLP_BWD), dtype=torch.uint8, device="cuda")

        if args.workload == "mlp_bwd_z":
            # the forward's pre-activation, made once before timing
            z_f = torch.empty((N, sh.F), dtype=torch.bfloat16, device="cuda")
            ws_f = torch.empty(tsp.workspace_size(shape, tsp.TSP_WS_MLP), dtype=torch.uint8, device="cuda")
            tsp.tsp_mlp_ring_z(shape, xd, wd["w1"], wd["w2"], None, dx, z_f, ws_f)

            def step():
                tsp.tsp_mlp_ring_bwd_z(shape, xd, z_f, wd["w1"], wd["w2"], dyd, None, dx, dw1, dw2, ws)
        else:
            def step():
                tsp.tsp_mlp_ring_bwd(shape, xd, wd["w1"], wd["w2"], dyd, None, dx, dw1, dw2, ws)
        # algorithmic: the four products of the chain rule (dy W2, dZ W1, dZ^T x,
        # dy^T GELU(Z)); the recomputation of Z = x W1^T is extra work, not counted
        step_flops = 4 * 2.0 * N * sh.h * sh.F
        step_exps = 0
        workload = (f"{'tsp_mlp_ring_bwd_z' if args.workload == 'mlp_bwd_z' else 'tsp_mlp_ring_bwd'}: backward of the "
                    "7B MLP ring (FFN), 16384x4096 bf16 local x and dy, D=8 shards of 2048x4096 and 4096x2048; dx, dW1, "
                    "dW2 in fp32 " + ("(Z from the forward)" if args.workload == "mlp_bwd_z" else "(Z recomputed)"))
    elif args.workload in ("attn_bwd", "attn_bwd_lse"):
        q = synth.attn_queries(sh, seed=3)
        k_rem, v_rem = synth.remote_kv(sh, seed=3)
        dout = synth.normal((N, sh.H, sh.Dh), 3, synth.TID_DY, 0, dtype="bf16")
        qd, dod = tsp.to_device(q, "bf16"), tsp.to_device(dout, "bf16")
        kf, vf = tsp.to_device(k_rem, "bf16"), tsp.to_device(v_rem, "bf16")
        dq = torch.empty((N, sh.H, sh.Dh), dtype=torch.float32, device="cuda")
        dk = torch.empty((sh.S, sh.kv_heads, sh.Dh), dtype=torch.float32, device="cuda")
        dv = torch.empty_like(dk)
        ws = torch.empty(tsp.workspace_size(shape, tsp.TSP_WS_ATTN_BWD), dtype=torch.uint8, device="cuda")

        if args.workload == "attn_bwd_lse":
            # the forward's fp32 O and row log-sum-exp, made once before timing
            o_f = torch.empty((N, sh.H, sh.Dh), dtype=torch.float32, device="cuda")
            lse_f = torch.empty((sh.H, N), dtype=torch.float32, device="cuda")
            tsp.tsp_zigzag_attn_lse(shape, qd, kf, vf, o_f, lse_f)

            def step():
                if args.plain_pds:
                    tsp.tsp_zigzag_attn_bwd_ex(shape, qd, kf, vf, o_f, lse_f, dod, dq, dk, dv,
                                               tsp.TSP_ATTN_BWD_PLAIN_PDS, ws)
                else:
                    tsp.tsp_zigzag_attn_bwd_lse(shape, qd, kf, vf, o_f, lse_f, dod, dq, dk, dv, ws)
        else:
            def step():
                if args.plain_pds:
                    tsp.tsp_zigzag_attn_bwd_ex(shape, qd, kf, vf, None, None, dod, dq, dk, dv,
                                               tsp.TSP_ATTN_BWD_PLAIN_PDS, ws)
                else:
                    tsp.tsp_zigzag_attn_bwd(shape, qd, kf, vf, dod, dq, dk, dv, ws)
        # algorithmic: 2.5 x the forward's 4*Dh flops per unmasked (query, key)
        # pair and head (S recomputed, dP, dV, dK, dQ)
        step_flops = 2.5 * flops["attention"]
        step_exps = sh.H * attn_pairs(sh.S, sh.D, r)
        workload = (f"{'tsp_zigzag_attn_bwd_lse' if args.workload == 'attn_bwd_lse' else 'tsp_zigzag_attn_bwd'}: "
                    f"32x128 heads{kv_note}, S=131072, 16384 zigzag queries of rank {r} of D=8; dq, dk, dv in fp32"
                    + ("; the forward's fp32 O and log-sum-exp given" if args.workload == "attn_bwd_lse" else "")
                    + ("; P and dS rounded once to bf16" if args.plain_pds else "; P and dS as bf16 hi + lo"))
    elif args.workload == "layers32":
        # 32 layers resident in HBM (82 GB of weights and K/V), each with its
        # own weights and remote K/V, generated on the GPU from a fixed seed:
        # N(0, 0.02^2) bf16 weights, unit gains, N(0, 1) bf16 K/V and fp32 x
        n_layers = 32
        gen = torch.Generator(device="cuda")
        gen.manual_seed(seed)

        def rnd(shape_, std, dtype):
            return (torch.randn(shape_, generator=gen, device="cuda", dtype=torch.float32) * std).to(dtype)

        hd, fd = sh.h // sh.D, sh.F // sh.D
        hkd = sh.kv_heads * sh.Dh // sh.D
        f1 = (2 if sh.mlp == "swiglu" else 1) * fd
        layers = []
        for _ in range(n_layers):
            wl = {"g_attn": torch.ones(sh.h, dtype=torch.bfloat16, device="cuda"),
                  "g_mlp": torch.ones(sh.h, dtype=torch.bfloat16, device="cuda"),
                  "wqkv": [rnd((hd + 2 * hkd, sh.h), 0.02, torch.bfloat16) for _ in range(sh.D)],
                  "wo": [rnd((sh.h, hd), 0.02, torch.bfloat16) for _ in range(sh.D)],
                  "w1": [rnd((f1, sh.h), 0.02, torch.bfloat16) for _ in range(sh.D)],
                  "w2": [rnd((sh.h, fd), 0.02, torch.bfloat16) for _ in range(sh.D)]}
            kl = rnd((sh.S, sh.kv_heads, sh.Dh), 1.0, torch.bfloat16)
            vl = rnd((sh.S, sh.kv_heads, sh.Dh), 1.0, torch.bfloat16)
            layers.append((wl, kl, vl))
        xbuf = [rnd((N, sh.h), 1.0, torch.float32), torch.empty((N, sh.h), dtype=torch.float32, device="cuda"),
                torch.empty((N, sh.h), dtype=torch.float32, device="cuda")]
        ws = torch.empty(tsp.workspace_size(shape, tsp.TSP_WS_LAYER), dtype=torch.uint8, device="cuda")

        def step():
            # x0 stays untouched; layer outputs alternate between two buffers
            src = xbuf[0]
            for i, (wl, kl, vl) in enumerate(layers):
                dst = xbuf[1 + (i & 1)]
                tsp.tsp_layer_fwd(shape, wl, src, kl, vl, dst, tsp.TSP_PHASE_ALL, ws)
                src = dst
        step_flops = n_layers * flops["total"]
        step_exps = n_layers * sh.H * attn_pairs(sh.S, sh.D, r)
        N = N * n_layers  # value = layer-tokens/s, comparable with the one-layer figure
        workload = (f"32 x tsp_layer_fwd: 32-layer 7B dense forward (each layer h=4096, 32x128 heads{kv_note}, {mlp_note} 16384, "
                    f"bf16, own weights and remote K/V, all resident) on rank {r} of D=8 at S=131072, "
                    f"16384 local zigzag tokens; value counts layer-tokens (16384 x 32 per step)")
    else:
        q = synth.attn_queries(sh, seed=3)
        k_rem, v_rem = synth.remote_kv(sh, seed=3)
        qd = tsp.to_device(q, "bf16")
        kf, vf = tsp.to_device(k_rem, "bf16"), tsp.to_device(v_rem, "bf16")
        o = torch.empty((N, sh.H, sh.Dh), dtype=torch.float32, device="cuda")

        def step():
            tsp.tsp_zigzag_attn(shape, qd, kf, vf, o, tsp.TSP_F32)
        step_flops = flops["attention"]
        step_exps = sh.H * attn_pairs(sh.S, sh.D, r)
        workload = f"tsp_zigzag_attn: 32x128 heads{kv_note}, S=131072, 16384 zigzag queries of rank {r} of D=8"
    torch.cuda.synchronize()
    mem_inputs = torch.cuda.memory_allocated() - mem0
    log(f"inputs resident in HBM ({time.perf_counter() - t_gen:.1f} s, {mem_inputs / 1e9:.3f} GB); "
        f"warmup {args.warmup}")

    if args.copy_mib > 0:
        n = args.copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"reference copy: {n} bytes read, {n} bytes written")
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done; timing {args.steps} steps")

    tsp.profile_reset()
    tsp.profile_enable(True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tsp.profile_enable(False)
    ms_step = ev0.elapsed_time(ev1) / args.steps
    kernels = {}
    for name in tsp.KERNEL_CLASSES:
        ms, n = tsp.profile_read(name)
        if n:
            kernels[name] = {"ms_per_launch": ms / n, "launches_per_step": n / args.steps}
    log(f"timed: {ms_step:.3f} ms/step (wall {wall * 1e3 / args.steps:.3f} ms/step)")

    # second pass, outside the timed region above: the same steps, each
    # bracketed by its own events, for the per-step minimum and median
    per = []
    for _ in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        per.append((a, b))
    torch.cuda.synchronize()
    per_ms = [a.elapsed_time(b) for a, b in per]
    ms_min, ms_median = min(per_ms), statistics.median(per_ms)
    log(f"per step: min {ms_min:.3f} ms, median {ms_median:.3f} ms")

    tokens_per_s = N / (ms_step * 1e-3)
    # dominant kernel: attention (73% of the layer's algorithmic flops)
    # HBM bytes per launch from the committed counter summary (taken on the
    # default layer: rank 0, 32 K/V heads, GELU MLP, no rotation), and the
    # bandwidth they give at this run's launch times
    default_layer = (args.workload == "layer" and r == 0 and sh.kv_heads == sh.H and sh.mlp == "gelu"
                     and args.rope_base == 0.0)
    hbm = traffic_from_profile() if default_layer else {}
    for cls, nbytes in hbm.items():
        if cls in kernels:
            kernels[cls]["hbm_bytes"] = nbytes
            kernels[cls]["hbm_gb_s"] = nbytes / (kernels[cls]["ms_per_launch"] * 1e-3) / 1e9
    # effective shader clock and MFMA-busy share per kernel from the committed
    # shader-counter summary of the same step (when the source is unchanged)
    sq = sq_from_profile() if default_layer else {}
    for cls, v in sq.items():
        if cls in kernels:
            kernels[cls].update(v)
    roofline = None
    if args.workload in ("layer_bwd", "train") and "attn_bwd" in kernels:
        # the attention backward: 4.40e13 of the step's 5.72e13 algorithmic flops
        t_b = kernels["attn_bwd"]["ms_per_launch"] * 1e-3
        achieved = 2.5 * flops["attention"] / t_b / 1e12
        roofline = {"kernel": "attn_bwd_stats_kernel + attn_bwd_dq_lds_kernel<128> + attn_bwd_dkv_kernel<128>",
                    "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                    "frac": achieved * 1e12 / PEAK_BF16, "traffic": None}
    elif "attention" in kernels:
        t_attn = kernels["attention"]["ms_per_launch"] * 1e-3
        achieved = flops["attention"] / t_attn / 1e12
        roofline = {"kernel": "attn_bf16_kernel<128>", "bound": "mfma", "achieved": achieved,
                    "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s", "frac": achieved * 1e12 / PEAK_BF16,
                    "traffic": hbm.get("attention")}
        if "attention" in sq:
            # the published peak is at 2.4 GHz; the counters give the clock the
            # kernel actually ran at
            roofline["sclk_ghz"] = sq["attention"]["sclk_ghz"]
            roofline["frac_of_peak_at_sclk"] = roofline["frac"] * 2.4 / sq["attention"]["sclk_ghz"]
    elif "attn_bwd" in kernels:
        t_b = kernels["attn_bwd"]["ms_per_launch"] * 1e-3
        achieved = 2.5 * flops["attention"] / t_b / 1e12
        names = ("attn_bwd_dq_kernel<128> + attn_bwd_dkv_kernel<128>" if args.workload == "attn_bwd" else
                 "attn_bwd_stats_kernel + attn_bwd_dq_lds_kernel<128> + attn_bwd_dkv_kernel<128>")
        roofline = {"kernel": names, "bound": "mfma", "achieved": achieved,
                    "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s", "frac": achieved * 1e12 / PEAK_BF16, "traffic": None}
    elif "bwd_gemm" in kernels:
        # launches of one product size each (Z recomputation unless Z is given, dZ, dW1, dW2, dx)
        t_g = kernels["bwd_gemm"]["ms_per_launch"] * 1e-3
        achieved = 2.0 * N * sh.h * sh.F / t_g / 1e12
        roofline = {"kernel": "gemm_bf16_kernel (MLP backward products)", "bound": "mfma", "achieved": achieved,
                    "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s", "frac": achieved * 1e12 / PEAK_BF16, "traffic": None}
    elif "mlp_up" in kernels:
        # one launch covers the up products of all D ring steps
        t_up = kernels["mlp_up"]["ms_per_launch"] * 1e-3
        f_up = (2 if sh.mlp == "swiglu" else 1) * 2 * N * sh.h * sh.F
        achieved = f_up / t_up / 1e12
        roofline = {"kernel": "gemm_bf16_kernel<EpiSwiGLU>" if sh.mlp == "swiglu" else "gemm_bf16_kernel<EpiGelu>",
                    "bound": "mfma", "achieved": achieved,
                    "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s", "frac": achieved * 1e12 / PEAK_BF16, "traffic": None}

    memory = None
    if args.workload in ("layer", "layers32"):
        memory = memory_report(sh, r, args, mem_inputs)

    cpu = None
    if args.cpu_rows > 0 and args.workload == "layer":
        cpu = cpu_baseline(sh, r, x, w, k_rem, v_rem, args.cpu_rows, args.rope_base)

    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_min": ms_min,
        "ms_per_step_median": ms_median,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload, "S": sh.S, "D": sh.D, "r": r, "h": sh.h, "H": sh.H, "Dh": sh.Dh,
                   "F": sh.F, "local_tokens": sh.N, "layers": 32 if args.workload == "layers32" else 1,
                   "parallelism": "one rank of a D=8 folded TP+SP axis", "rope_base": args.rope_base,
                   "Hkv": sh.kv_heads, "mlp": sh.mlp},
        "pct_bf16_mfma_peak": 100.0 * step_flops / (ms_step * 1e-3) / PEAK_BF16,
        "algorithmic_tflop_per_step": step_flops / 1e12,
        "softmax_exps_per_step": step_exps,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "memory": memory,
        "kernels": kernels,
        "gpu": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)


def memory_report(sh, r, args, allocated):
    """Device bytes the workload's inputs, outputs and workspace took (the
    allocator's count) beside the analytic model of the same allocations,
    and the model's per-rank footprint of the distributed 32-layer forward
    (and of training under its stated assumptions) at this shape; the pages'
    38.8 GB per GPU (8 x MI300X, 128K tokens) is context, not a target."""
    from tsp_rank_local_amd import memory as mm

    layers = 32 if args.workload == "layers32" else 1
    m = mm.Model(S=sh.S, D=sh.D, r=r, h=sh.h, H=sh.H, Dh=sh.Dh, F=sh.F, layers=layers, Hkv=sh.Hkv, mlp=sh.mlp,
                 rope_base=args.rope_base)
    model = mm.single_gpu_bytes(m, "layer" if layers == 1 else "layers")
    m32 = dataclasses.replace(m, layers=32)
    fwd, trn = mm.rank_memory(m32), mm.rank_memory(m32, train=True)
    return {"allocated_bytes": allocated, "model_bytes": model, "model_vs_allocated": model / allocated,
            "rank_forward_32_layers_gb": {k: round(v / 1e9, 3) for k, v in fwd.items()},
            "rank_train_32_layers_gb": round(trn["total"] / 1e9, 3),
            "pages_tsp_gb_per_gpu": 38.8}


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(sh, r, x, w, k_rem, v_rem, m, rope_base=0.0):
    """Time the fp64 oracle on m evenly strided local rows of the same layer:
    each row's RMSNorm, Q/K/V projection, causal attention over its prefix of
    the gathered K/V, output projection, RMSNorm and MLP. The rate scales
    linearly with rows (every row's work is independent once K/V are
    gathered), so tokens/s = m / t."""
    import oracle
    import synth

    log(f"cpu baseline: oracle on {m} of {sh.N} local rows")
    w64 = {k: ([synth.as_f32(a, "bf16").astype(np.float64) for a in v] if isinstance(v, list)
               else synth.as_f32(v, "bf16").astype(np.float64)) for k, v in w.items()}
    k32, v32 = synth.as_f32(k_rem, "bf16"), synth.as_f32(v_rem, "bf16")
    rows = np.linspace(0, sh.N - 1, m).round().astype(np.int64)
    pos = oracle.zigzag_positions(sh.S, sh.D, r)[rows]
    t0 = time.perf_counter()
    oracle.local_kv(x[rows], w64, sh.H, sh.Dh, sh.eps, pos, rope_base, Hkv=sh.kv_heads)
    oracle.layer_rows(x[rows], pos, w64, k32, v32, sh.H, sh.Dh, sh.eps, sh.scale, rope_base, Hkv=sh.kv_heads,
                      gated=sh.mlp == "swiglu")
    t = time.perf_counter() - t0
    log(f"cpu baseline: {t:.1f} s")
    return {"value": m / t, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{m} evenly strided local rows of the same layer (per-row Q/K/V projection, causal attention "
                      f"over the gathered K/V prefix, output projection, MLP) in numpy float64; {t:.1f} s; "
                      f"BLAS threads as cores, exp/erf single-threaded"}


if __name__ == "__main__":
    main()
