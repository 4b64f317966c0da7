"""Write the text summaries under profiles/ from rocprofv3 CSV output.

Usage (repository root, after the GPU runs listed in each summary wrote gpurun_out/):
    python profiles/make_summaries.py gpurun_out
Reads <dir>/prof_trace/run_kernel_trace.csv + run_kernel_stats.csv + prof_trace.log (the
bench JSON line printed under the profiler), <dir>/pmc_{fetch,write,copy_fetch,copy_write} and
<dir>/pmc_clock, and <dir>/prof_hbm (the standalone HBM-bound steps).
"""

from __future__ import annotations

import collections
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ATTN = "attention_kernel<128>"
FLOP = 4 * 9828 * 32760 * 128 * 12
ALGO_BYTES = 9828 * 1536 * 2 + 2 * 32760 * 1536 * 2 + 9828 * 1536 * 2


def _short(name):
    return name.split("(")[0].replace("void ", "")


def trace_summary(d):
    stats = list(csv.DictReader(open(os.path.join(d, "prof_trace", "run_kernel_stats.csv"))))
    trace = list(csv.DictReader(open(os.path.join(d, "prof_trace", "run_kernel_trace.csv"))))
    bench = None
    log = os.path.join(d, "prof_trace.log")
    if os.path.exists(log):
        for line in open(log):
            if line.startswith("{"):
                bench = json.loads(line)
    warm = int(bench["warmup"]) if bench else 3
    durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in trace if ATTN in r["Kernel_Name"]]
    timed = durs[warm:] if len(durs) > warm else durs
    out = [
        "# rocprofv3 kernel-trace summary: pruned layer step, wan13b workload",
        "# (N=32760 tokens, D=1536, 12 heads x 128, 30% active = 9828 queries)",
        "# command (repository root, one MI355X):",
        "#   rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_trace -o run -- \\",
        "#       python3 bench.py --steps 10 --warmup 3 --no-cpu-baseline --no-dense --no-hbm",
        "# summary written by: python profiles/make_summaries.py gpurun_out",
        "",
        f"{'kernel':48s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}",
    ]
    for r in stats:
        out.append(f"{_short(r['Name'])[:48]:48s} {r['Calls']:>6s} {float(r['AverageNs'])/1e3:10.1f} "
                   f"{float(r['MinNs'])/1e3:10.1f} {float(r['MaxNs'])/1e3:10.1f} {float(r['Percentage']):6.2f}")
    avg_t = sum(timed) / len(timed) / 1e3
    out += ["", f"# {ATTN}: {len(durs)} dispatches; the {len(timed)} of the timed steps average {avg_t:.1f} us",
            f"#   -> {FLOP / (avg_t * 1e-6) / 1e12:.1f} TFLOP/s = {FLOP / (avg_t * 1e-6) / 1e12 / 2500 * 100:.1f}% of 2500 TFLOP/s"]
    if bench:
        out.append(f"# bench.py under the profiler (HIP events on the launch stream): attention "
                   f"{bench['kernel_ms']['attention_scatter']['mean']*1e3:.1f} us (mean; median {bench['kernel_ms']['attention_scatter']['median']*1e3:.1f} us), roofline.achieved {bench['roofline']['achieved']} TFLOP/s")
    return "\n".join(out) + "\n"


def _per_kernel(d, counter):
    f = glob.glob(os.path.join(d, "*counter_collection.csv"))[0]
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(f)):
        if r["Counter_Name"] == counter:
            agg[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in agg.items()}


def traffic_summary(d):
    fetch = _per_kernel(os.path.join(d, "pmc_fetch"), "FETCH_SIZE")
    write = _per_kernel(os.path.join(d, "pmc_write"), "WRITE_SIZE")
    cf = _per_kernel(os.path.join(d, "pmc_copy_fetch"), "FETCH_SIZE")["__amd_rocclr_copyBuffer"]
    cw = _per_kernel(os.path.join(d, "pmc_copy_write"), "WRITE_SIZE")["__amd_rocclr_copyBuffer"]
    sf, sw = 2 ** 20 / cf, 2 ** 20 / cw
    src = hashlib.sha256(open(os.path.join(ROOT, "token_sparse_attention_rel_amd", "csrc", "attention.hip"), "rb").read()).hexdigest()
    a = next(k for k in fetch if ATTN in k)
    hb = fetch[a] * sf * 1024 + write[a] * sw * 1024
    out = [
        "# HBM traffic per launch from rocprofv3 counters, wan13b pruned layer step",
        "# commands (repository root, one MI355X; one counter per run):",
        "#   timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc_fetch -o run -- python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-dense --no-hbm",
        "#   timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc_write -o run -- python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-dense --no-hbm",
        "# calibration: the same two counters over `python3 bench.py --copy-calibration` (a plain 1 GiB",
        "#   device copy, __amd_rocclr_copyBuffer, reading and writing exactly 1048576 KiB per launch):",
        f"#   FETCH_SIZE reads {cf:.1f} KiB per copy -> scale {sf:.4f};  WRITE_SIZE reads {cw:.1f} KiB -> scale {sw:.4f}",
        "# summary written by: python profiles/make_summaries.py gpurun_out",
        "# per-kernel averages over dispatches (KiB as reported, then scaled bytes):",
        "",
    ]
    for k in fetch:
        if k.startswith("at::"):
            continue
        fb, wb = fetch[k] * sf * 1024, write.get(k, 0) * sw * 1024
        out.append(f"# {k[:40]:40s} FETCH {fetch[k]:12.1f} KiB  WRITE {write.get(k, 0):12.1f} KiB  -> read {fb/1e6:9.1f} MB  write {wb/1e6:8.1f} MB")
    out += ["", "# attention kernel: algorithmic bytes per launch = Q_a + K + V + O",
            f"#   = 9828*1536*2 + 2*32760*1536*2 + 9828*1536*2 = {ALGO_BYTES/1e6:.1f} MB;"
            f" measured/algorithmic = {hb / ALGO_BYTES:.2f}",
            f"kernel: {ATTN}", f"kernel_source_sha256: {src}",
            f"fetch_kib_per_dispatch: {fetch[a]:.3f}", f"write_kib_per_dispatch: {write[a]:.3f}",
            f"fetch_scale: {sf:.5f}", f"write_scale: {sw:.5f}", f"hbm_bytes_per_launch: {hb:.0f}"]
    return "\n".join(out) + "\n"


def clock_summary(d):
    """Shader clock and MFMA activity of the attention kernel from one counter run."""
    f = glob.glob(os.path.join(d, "pmc_clock", "*counter_collection.csv"))[0]
    per = collections.defaultdict(dict)
    for r in csv.DictReader(open(f)):
        if ATTN in _short(r["Kernel_Name"]):
            e = per[r["Dispatch_Id"]]
            e[r["Counter_Name"]] = float(r["Counter_Value"])
            e["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    rows = [e for e in per.values() if "GRBM_GUI_ACTIVE" in e]
    src = hashlib.sha256(open(os.path.join(ROOT, "token_sparse_attention_rel_amd", "csrc", "attention.hip"), "rb").read()).hexdigest()
    out = [
        "# Shader clock and MFMA activity of the attention kernel, wan13b pruned layer step",
        "# command (repository root, one MI355X):",
        "#   timeout -s KILL 120 rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_WAVES "
        "--output-format csv -d gpurun_out/pmc_clock -o run -- python3 bench.py --steps 3 --warmup 1 "
        "--no-cpu-baseline --no-dense --no-hbm",
        "# summary written by: python profiles/make_summaries.py gpurun_out",
        "# GRBM_GUI_ACTIVE counts busy GPU cycles on each of the 8 XCDs (summed): cycles = value / 8;",
        "# sclk = cycles / kernel duration.  MFMA utilisation at that clock = algorithmic FLOP /",
        "# (duration x sclk x 4096 FLOP/clk/CU x 256 CUs); SQ_VALU_MFMA_BUSY_CYCLES per SIMD-cycle agrees.",
        "",
        f"{'dispatch_us':>12s} {'sclk_GHz':>9s} {'util_at_sclk':>13s} {'MFMA_busy_per_SIMD':>19s} {'SQ_WAVES':>9s}",
    ]
    sclks, utils = [], []
    for e in rows:
        cyc = e["GRBM_GUI_ACTIVE"] / 8.0
        sclk = cyc / e["ns"]
        util = FLOP / (e["ns"] * 1e-9 * sclk * 1e9 * 4096 * 256)
        sclks.append(sclk)
        utils.append(util)
        mb = e.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cyc * 1024)  # per SIMD (4 per CU)
        out.append(f"{e['ns'] / 1e3:12.1f} {sclk:9.3f} {util:13.3f} {mb:19.3f} {e.get('SQ_WAVES', 0):9.0f}")
    sclks.sort()
    utils.sort()
    med = sclks[len(sclks) // 2]
    out += ["", f"kernel: {ATTN}", f"kernel_source_sha256: {src}", f"sclk_ghz_median: {med:.3f}",
            f"mfma_util_at_sclk_median: {utils[len(utils) // 2]:.3f}"]
    return "\n".join(out) + "\n"


def stats_summary(d, sub, title, command):
    """Per-kernel statistics of one rocprofv3 --kernel-trace --stats run."""
    stats = list(csv.DictReader(open(os.path.join(d, sub, "run_kernel_stats.csv"))))
    out = [f"# rocprofv3 kernel-trace summary: {title}", "# command (repository root, one MI355X):",
           f"#   {command}", "# summary written by: python profiles/make_summaries.py gpurun_out", "",
           f"{'kernel':48s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}"]
    for r in stats:
        out.append(f"{_short(r['Name'])[:48]:48s} {r['Calls']:>6s} {float(r['AverageNs'])/1e3:10.1f} "
                   f"{float(r['MinNs'])/1e3:10.1f} {float(r['MaxNs'])/1e3:10.1f} {float(r['Percentage']):6.2f}")
    return "\n".join(out) + "\n"


def hbm_summary(d):
    """Kernel durations of the standalone HBM-bound steps (the bench's flushed repetitions)."""
    trace = list(csv.DictReader(open(os.path.join(d, "prof_hbm", "run_kernel_trace.csv"))))
    n, dim, k = 32760, 1536, 9828
    kernels = [
        ("a1 score", "score_kernel<", 2 * n * dim * 2 + 4 * n),
        ("a4 gather", "gather_rows_kernel<false", k * dim * 4),
        ("a6 cache sync", "copy_rows_kernel<true", 4 * k * dim * 2),
        ("a8 scatter", "copy_rows_kernel<false", 2 * k * dim * 2),
    ]
    out = ["# rocprofv3 kernel-trace summary: HBM-bound steps alone, wan13b workload",
           "# (N=32760, D=1536, 9828 active rows; the 256 MB MALL flushed before each repetition)",
           "# command (repository root, one MI355X):",
           "#   rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_hbm -o run -- \\",
           "#       python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-dense",
           "# summary written by: python profiles/make_summaries.py gpurun_out",
           "# median kernel time of the last 20 dispatches (the bench's flushed repetitions),",
           "# algorithmic bytes as in bench.py, against 8000 GB/s", "",
           f"{'step':14s} {'kernel':40s} {'median_us':>10s} {'GB/s':>8s} {'frac':>6s}"]
    for label, key, nbytes in kernels:
        durs = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in trace if key in r["Kernel_Name"]]
        if not durs:
            continue
        last = sorted(durs[-20:])
        med = last[len(last) // 2] / 1e3
        name = _short([r["Kernel_Name"] for r in trace if key in r["Kernel_Name"]][0])
        out.append(f"{label:14s} {name[:40]:40s} {med:10.1f} {nbytes / med / 1e3:8.1f} {nbytes / med / 1e3 / 8000:6.3f}")
    return "\n".join(out) + "\n"


EXTRA = [
    ("prof_hsa_loop", "hsa_loop_wan13b_kernel_trace.txt",
     "HSA sampling loop (Euler update, phase window), N=32760, D=1536, 12 x 128, T=8",
     "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_hsa_loop -o run -- "
     "python3 bench.py --workload hsa_loop --steps 8 --warmup 1 --no-dense"),
    ("prof_lipar_lif", "lipar_lif_kernel_trace.txt",
     "LIPAR pass with the long/short-term mask + restoration, 33x45x80 -> N=118800, D=3072, 24 x 128",
     "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_lipar_lif -o run -- "
     "python3 bench.py --workload lipar_lif --steps 10 --warmup 1"),
    ("prof_tr", "timeripple_reuse_kernel_trace.txt",
     "dense pass with Timeripple partial-score reuse, 21x30x52 -> N=32760, D=1536, 12 x 128 "
     "(bench pass with reuse + pass without reuse + the reuse kernels timed alone; the 512 MB "
     "reduce is the bench's MALL flush)",
     "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_tr -o run -- "
     "python3 bench.py --workload timeripple --steps 10 --warmup 2"),
    ("prof_rc", "layer_step_wan13b_rope_causal_kernel_trace.txt",
     "pruned layer step with 3D RoPE and frame-causal attention, 21x30x52 -> N=32760, D=1536, 12 x 128",
     "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof_rc -o run -- "
     "python3 bench.py --workload wan13b_rc --steps 10 --warmup 3 --no-cpu-baseline --no-dense --no-hbm"),
]


def main(argv):
    d = argv[1] if len(argv) > 1 else "gpurun_out"
    here = os.path.dirname(os.path.abspath(__file__))
    open(os.path.join(here, "layer_step_wan13b_kernel_trace.txt"), "w").write(trace_summary(d))
    open(os.path.join(here, "attention_wan13b_traffic.txt"), "w").write(traffic_summary(d))
    if glob.glob(os.path.join(d, "pmc_clock", "*counter_collection.csv")):
        open(os.path.join(here, "attention_wan13b_clock.txt"), "w").write(clock_summary(d))
    if os.path.exists(os.path.join(d, "prof_hbm", "run_kernel_trace.csv")):
        open(os.path.join(here, "hbm_kernels_wan13b_kernel_trace.txt"), "w").write(hbm_summary(d))
    for sub, fname, title, cmd in EXTRA:
        if os.path.exists(os.path.join(d, sub, "run_kernel_stats.csv")):
            open(os.path.join(here, fname), "w").write(stats_summary(d, sub, title, cmd))
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
