"""Benchmark of the pruned attention layer step on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
score + top-k select + compaction, QKV of the active tokens with the fused
KV-cache sync, attention of the active queries over all N cached keys with
the fused scatter back to token order.  Inputs are resident in HBM before
the timed region starts.

Prints ONE JSON line.  ``value`` is the effective layer throughput in
TFLOP/s = 4 * N_active * N * head_dim * heads / step time.  Extra fields give
tokens/s, the per-kernel times (median / p10 / p90 over the timed steps), the
attention kernel's roofline, the HBM-bound steps timed standalone against the
HBM peak, the dense layer and the CPU oracle measured on a bounded sample of
the same workload.  Step labels (a1 score ... a8 scatter) follow
include/tsa.h.

Other workloads (``--workload``): ``large`` and ``tiny`` (the same step),
``hsa`` (the T-step schedule loop), ``hsa_loop`` (the sampling loop with the
cached Euler update and phase window), ``lipar`` (the inter-frame sweep over
active fractions) and ``lipar_lif`` (the pass with the long/short-term mask and
restoration); each prints its own JSON line.
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

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "pruned-attn layer TFLOP/s + tokens/s at N=32760, 30% active; % MFMA peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_wan13b_traffic.txt")
CLOCK_FILE = os.path.join(ROOT, "profiles", "attention_wan13b_clock.txt")
SPEC_SCLK_GHZ = 2.4
ATTN_SRC = os.path.join(ROOT, "token_sparse_attention_rel_amd", "csrc", "attention.hip")


def parse_args(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="wan13b")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample-rows", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-hbm", action="store_true", help="skip the standalone HBM-kernel timings")
    ap.add_argument("--attn-schedule", choices=("split", "tile"), default="split",
                    help="attention: split the last, partly filled round of query tiles into key "
                         "ranges (default) or run one workgroup per query tile throughout")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (HBM counter calibration)")
    return ap.parse_args(argv)


def copy_calibration():
    """A plain device-to-device copy of known size, to calibrate the HBM byte counters:
    each launch reads and writes exactly 2**30 bytes."""
    import torch

    a = torch.ones(2 ** 29, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read_per_launch": 2 ** 30,
                      "copy_calibration_bytes_written_per_launch": 2 ** 30}), flush=True)
    return 0


def attention_kernel_label(cfg, split: bool, causal: bool) -> str:
    """The attention kernel(s) the roofline object times, named as the profiler reports them."""
    hd = cfg.head_dim
    big = "true" if ((cfg.n - 1) * cfg.dim + hd) * 2 > 0x7FFFFFFF else "false"  # caches past one buffer range
    if causal:
        return (f"attention_causal_kernel<{hd}, {big}> (active queries x the keys of their frames and "
                "earlier, fused scatter)")
    if split:
        return (f"attention_split_kernel<{hd}, {big}> + attention_merge_kernel<{hd}> (active queries x all "
                "cached K/V, fused scatter; timed together)")
    return f"attention_kernel<{hd}, {big}> (active queries x all cached K/V, fused scatter)"


def _src_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _profile_value(path, key):
    """A value from a committed rocprofv3 summary of the attention kernel, or None when the
    summary is missing or the kernel source changed since it was taken."""
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    try:
        if vals.get("kernel_source_sha256") != _src_hash(ATTN_SRC):
            return None
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def attention_traffic():
    """HBM bytes per attention launch (FETCH_SIZE + WRITE_SIZE counter summary)."""
    return _profile_value(TRAFFIC_FILE, "hbm_bytes_per_launch")


def attention_sclk():
    """Median shader clock (GHz) during the attention kernel (GRBM_GUI_ACTIVE summary)."""
    return _profile_value(CLOCK_FILE, "sclk_ghz_median")


def cpu_baseline(cfg, inp, n_sample):
    """The CPU oracle on a bounded sample of the same step: scores + selection over all N,
    projections + cache sync of all active tokens, attention of n_sample active queries;
    the attention time is scaled by N_active / n_sample."""
    import numpy as np

    from oracle import reference as ref

    try:
        from threadpoolctl import threadpool_info

        blas = max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        blas = os.cpu_count() or 1
    xp = inp["x_prev"].double().numpy()
    xc = inp["x_cur"].double().numpy()
    w = inp["w_qkv"].double().numpy()
    kc, vc = ref.init_kv_cache(xp, w)  # state before the step: not timed
    k = cfg.n_active
    t0 = time.perf_counter()
    s = ref.token_scores(xc, xp)
    mask = ref.select_topk(s, k)
    idx, _ = ref.compact(mask)
    p = ref.project(xc[idx], w, "kv")
    ref.kv_cache_sync(kc, vc, idx, p["k"], p["v"])
    t1 = time.perf_counter()
    rows = np.sort(np.random.default_rng(0).choice(idx.size, min(n_sample, idx.size), replace=False))
    q = ref.project(xc[idx[rows]], w, "q")["q"]
    ref.attention(q, kc, vc, cfg.heads)
    t2 = time.perf_counter()
    t_step = (t1 - t0) + (t2 - t1) * idx.size / rows.size
    return {
        "value": cfg.attn_flops(k) / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": int(blas),
        "kind": "oracle",
        "sample": (f"numpy fp64 oracle: scores/top-k/compaction over all {cfg.n} tokens and QKV + cache sync "
                   f"of all {k} active tokens ({t1 - t0:.2f} s), attention of {rows.size} sampled active "
                   f"queries ({t2 - t1:.2f} s) scaled x{idx.size / rows.size:.2f}; step estimate {t_step:.2f} s"),
        "step_seconds_estimate": t_step,
        "host_cpus": os.cpu_count(),
        "affinity": len(os.sched_getaffinity(0)),
    }


class EventTimer:
    """Per-repetition HIP event pairs on one stream; statistics in milliseconds."""

    def __init__(self, torch, stream):
        self.torch, self.stream, self.pairs = torch, stream, []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.pairs.append([e, None])

    def stop(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.pairs[-1][1] = e

    def times(self):
        return [a.elapsed_time(b) for a, b in self.pairs]


def stats(ms):
    """median / p10 / p90 / mean of a list of times (ms)."""
    import numpy as np

    a = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 5), "p10": round(float(np.percentile(a, 10)), 5),
            "p90": round(float(np.percentile(a, 90)), 5), "mean": round(float(a.mean()), 5), "reps": int(a.size)}


def roofline_entry(kind, work, st, unit):
    """Algorithmic work per launch over the median launch time, against the MI355X peak."""
    t = st["median"] * 1e-3
    if kind == "hbm":
        achieved = work / t / 1e9
        return {"bound": "hbm", "algorithmic_bytes": int(work), "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "ms": st}
    achieved = work / t / 1e12
    return {"bound": "mfma", "algorithmic_flop": int(work), "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": unit, "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "ms": st}


def hbm_kernels(tsa, torch, cfg, layer, xc, xp, sets=12, launches=20, reps=5):
    """The HBM-bound steps timed standalone: a1 score (all N rows of X_cur and X_ref read),
    a4 gather, a6 cache sync and a8 scatter of the N_a active rows (fused into the QKV and
    attention kernels on the layer path).  Protocol: `launches` back-to-back launches per
    event pair, cycling over `sets` copies of the inputs at distinct addresses (together more
    than twice the 256 MB MALL, so each launch reads HBM), the median over `reps` pairs; per
    launch = pair time / launches.  Beside each, a plain device copy of the same byte count
    (half read, half written) timed the same way: the read+write rate the chip reaches on a
    copy, for scale."""
    n, d, k = cfg.n, cfg.dim, cfg.n_active
    dev = xc.device
    stream = torch.cuda.current_stream()
    esz = xc.element_size()
    g = torch.Generator(device="cpu").manual_seed(1)
    xs = [(xc.clone(), xp.clone()) for _ in range(sets)]
    idxs = [torch.randperm(n, generator=g)[:k].sort().values.to(torch.int32).to(dev) for _ in range(sets)]
    kvs = [(layer.k_cache[:k].clone(), layer.v_cache[:k].clone()) for _ in range(sets)]
    caches = [(layer.k_cache.clone(), layer.v_cache.clone()) for _ in range(sets)]
    scores = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(sets)]
    dsts = [torch.empty(k, d, dtype=xc.dtype, device=dev) for _ in range(sets)]
    ops = {
        "a1_score": (lambda i: tsa.token_scores(xs[i][0], xs[i][1], scores[i]), 2 * n * d * esz + 4 * n),
        "a4_gather": (lambda i: tsa.gather_rows(xs[i][0], idxs[i], k, dsts[i]), k * d * (esz + 2)),
        "a6_cache_sync": (lambda i: tsa.kv_cache_sync(kvs[i][0], kvs[i][1], idxs[i], k, caches[i][0], caches[i][1]),
                          4 * k * d * 2),
        "a8_scatter": (lambda i: tsa.scatter_out(kvs[i][0], idxs[i], k, caches[i][0]), 2 * k * d * 2),
    }
    if xc.dtype != torch.bfloat16:
        # fp32 token rows (the tiny workload) enter the projection directly; the standalone
        # gather moves bf16 rows only
        del ops["a4_gather"]

    def per_launch_ms(fn):
        for i in range(sets):
            fn(i)
        torch.cuda.synchronize()
        tm = EventTimer(torch, stream)
        for _ in range(reps):
            tm.start()
            for j in range(launches):
                fn(j % sets)
            tm.stop()
        torch.cuda.synchronize()
        return stats([t / launches for t in tm.times()])

    res = {}
    for name, (fn, nbytes) in ops.items():
        st = per_launch_ms(fn)
        half = nbytes // 2 // 2 * 2
        src = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(sets)]
        dst = [torch.empty_like(t) for t in src]
        cst = per_launch_ms(lambda i: dst[i].copy_(src[i]))
        del src, dst
        e = roofline_entry("hbm", nbytes, st, "GB/s")
        e["protocol"] = f"{launches} back-to-back launches per event pair over {sets} rotated input sets"
        e["plain_copy_same_bytes"] = roofline_entry("hbm", 2 * half, cst, "GB/s")
        res[name] = e
    del xs, kvs, caches
    return res


def bench_step(args, torch, tsa, cfg):
    """One pruned layer step (score + top-k + compaction, QKV + cache sync, attention +
    scatter), K timed steps; the JSON line of the headline workload."""
    from workloads import generate

    dev = torch.device("cuda:0")
    inp = generate.step_inputs(cfg, args.seed)
    layer = tsa.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, inp["w_qkv"].to(dev), device=dev,
                                     split_attention=args.attn_schedule == "split",
                                     rope=(cfg.height, cfg.width, 10000.0) if cfg.rope else None,
                                     causal_frame_tokens=cfg.hw if cfg.causal else None)
    xp = inp["x_prev"].to(dev)
    xc = inp["x_cur"].to(dev)
    layer.init_cache(xp)
    k = cfg.n_active
    stream = torch.cuda.current_stream()
    attn_ws = layer.attention_workspace(k)

    for _ in range(args.warmup):
        layer.step_topk(xc, xp, k)
    torch.cuda.synchronize()

    t_sel, t_qkv, t_att, t_step = (EventTimer(torch, stream) for _ in range(4))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        t_step.start()
        t_sel.start()
        layer.select(xc, xp, k=k)
        t_sel.stop()
        t_qkv.start()
        layer._qkv(xc, layer.idx, k, q_out=layer.q_a, k_out=layer.k_cache, v_out=layer.v_cache,
                   out_is_cache=True, n_cache=cfg.n)
        t_qkv.stop()
        t_att.start()
        if cfg.causal:
            tsa.frame_causal_attention(layer.q_a, layer.k_cache, layer.v_cache, k, cfg.heads, cfg.head_dim,
                                       layer.idx, cfg.hw, layer.out, out_rows=layer.idx)
        else:
            tsa.sparse_query_attention(layer.q_a, layer.k_cache, layer.v_cache, k, cfg.heads,
                                       cfg.head_dim, layer.out, out_rows=layer.idx, workspace=attn_ws)
        t_att.stop()
        t_step.stop()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    s_sel, s_qkv, s_att, s_step = (stats(t.times()) for t in (t_sel, t_qkv, t_att, t_step))
    t_att_mean = s_att["mean"]

    flops = cfg.attn_flops(k)
    if cfg.causal:
        # algorithmic work of the frame-causal attention: each query's visible keys only
        import numpy as np

        fr = layer.idx[:k].cpu().numpy().astype(np.int64) // cfg.hw
        visible = np.minimum((fr + 1) * cfg.hw, cfg.n)
        flops = int(4 * visible.sum() * cfg.head_dim * cfg.heads)
    dense = None
    if not args.no_dense:
        # dense layer: the same QKV and attention kernels over every token, no selection;
        # each repetition synchronised on its own so that host-side gaps between
        # repetitions are not timed
        layer.dense_forward(xc)
        torch.cuda.synchronize()
        td = EventTimer(torch, stream)
        for _ in range(max(20, args.steps)):
            td.start()
            layer.dense_forward(xc)
            td.stop()
            torch.cuda.synchronize()
        dense = stats(td.times())
        layer.init_cache(xp)

    hbm = None if args.no_hbm else hbm_kernels(tsa, torch, cfg, layer, xc, xp)
    achieved = flops / (t_att_mean * 1e-3) / 1e12
    # the clock summary covers the wan13b attention kernel only
    sclk = attention_sclk() if cfg.name == "wan13b" else None
    rec = {
        "metric": METRIC if cfg.name == "wan13b" else f"pruned-attn layer TFLOP/s + tokens/s ({cfg.name})",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded generator; random-init projection weights)",
        "config": {
            "workload": f"{cfg.name}: F={cfg.frames} H={cfg.height} W={cfg.width} -> N={cfg.n} tokens, "
                        f"D={cfg.dim}, {cfg.heads} heads x d={cfg.head_dim}, {cfg.active_pct}% active "
                        f"(k={k}), {cfg.static_pct}% static tokens, "
                        + ("3D rotary positions on Q/K, frame-causal attention" if cfg.rope or cfg.causal
                           else "full bidirectional attention"),
            "n_tokens": cfg.n,
            "n_active": k,
            "dim": cfg.dim,
            "heads": cfg.heads,
            "head_dim": cfg.head_dim,
            "seed": args.seed,
            "rope": cfg.rope,
            "frame_causal": cfg.causal,
        },
        "attention_schedule": ("one workgroup per query tile, last round split into key ranges"
                               if attn_ws is not None else "one workgroup per query tile"),
        "tokens_per_s": round(cfg.n / (ms_step * 1e-3), 1),
        "active_tokens_per_s": round(k / (ms_step * 1e-3), 1),
        "step_ms_events": s_step,
        "attn_tflops": round(achieved, 3),
        "attn_frac_of_mfma_peak": round(achieved / PEAK_BF16_TFLOPS, 4),
        "kernel_ms": {"score_select_compact": s_sel, "qkv_gather_cache_sync": s_qkv,
                      "attention_scatter": s_att},
        "qkv": roofline_entry("mfma", cfg.qkv_flops(k), s_qkv, "TFLOP/s"),
        "hbm_kernels": hbm,
        "dense_layer_ms": dense,
        "speedup_vs_dense": None if dense is None else round(dense["median"] / s_step["median"], 3),
        "roofline": {
            "bound": "mfma",
            "kernel": attention_kernel_label(cfg, attn_ws is not None, cfg.causal),
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            # the counter summary covers the wan13b attention kernel only
            "traffic": attention_traffic() if cfg.name == "wan13b" else None,
            "algorithmic_flop_per_launch": flops,
            # the shader clock the profiled attention kernel ran at (power-limited under full
            # MFMA load) and the fraction of the peak at that clock, next to the spec-clock frac
            "sclk_ghz_profiled": sclk,
            "frac_at_profiled_sclk": None if sclk is None else round(achieved / (PEAK_BF16_TFLOPS * sclk / SPEC_SCLK_GHZ), 4),
            "launch_ms_mean_events": round(t_att_mean, 5),
        },
    }
    if cfg.causal:
        rec["attention_schedule"] = "one workgroup per query tile, key loop bounded by its queries' frames"
    if not args.no_cpu_baseline and not (cfg.rope or cfg.causal):
        rec["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample_rows)
    return rec


def bench_hsa(args, torch, tsa, cfg):
    """HSA schedule loop: T global steps on X_1..X_T, groups ranked once at step 0 by the
    change between X_1 and X_0; every step syncs the cache for its active set.  Reports
    per-step and total throughput and the same T steps run dense."""
    from workloads import generate

    dev = torch.device("cuda:0")
    inp = generate.hsa_inputs(cfg, args.seed)
    xs = [x.to(dev) for x in inp["xs"]]
    layer = tsa.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, inp["w_qkv"].to(dev), device=dev)
    counts, gper = cfg.group_counts(), cfg.group_periods()
    period = torch.empty(cfg.n, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def run(timers=None, dense=False):
        layer.init_cache(xs[0])
        layer.select(xs[1], xs[0], k=1)
        tsa.assign_groups(layer.scores, counts, gper, period, layer.workspace)
        for i in range(cfg.steps):
            if timers:
                timers[i].start()
            if dense:
                layer.dense_forward(xs[i + 1])
            else:
                layer.select(None, periods=period, step=i)
                layer.forward_active(xs[i + 1], tsa.hsa_active_count(counts, gper, i))
            if timers:
                timers[i].stop()

    for _ in range(max(1, args.warmup // 4)):
        run()
    reps = max(3, args.steps // 8)
    tm = [EventTimer(torch, stream) for _ in range(cfg.steps)]
    for _ in range(reps):
        run(tm)
    td = [EventTimer(torch, stream) for _ in range(cfg.steps)]
    if not args.no_dense:
        for _ in range(reps):
            run(td, dense=True)
    torch.cuda.synchronize()
    per_step, total_ms, total_flops = [], 0.0, 0
    for i in range(cfg.steps):
        n_act = tsa.hsa_active_count(counts, gper, i)
        st = stats(tm[i].times())
        total_ms += st["median"]
        total_flops += cfg.attn_flops(n_act)
        per_step.append({"step": i, "n_active": n_act, "ms": st,
                         "attn_tflops_effective": round(cfg.attn_flops(n_act) / (st["median"] * 1e-3) / 1e12, 2)})
    dense_ms = None if args.no_dense else sum(stats(t.times())["median"] for t in td)
    return {
        "metric": "HSA schedule loop: effective TFLOP/s and token-steps/s over T steps",
        "value": round(total_flops / (total_ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic (seeded generator; random-init projection weights)",
        "config": {"workload": f"{cfg.name}: N={cfg.n}, D={cfg.dim}, {cfg.heads}x{cfg.head_dim}, T={cfg.steps}, "
                               f"groups {cfg.group_pcts}% with budgets {cfg.group_budgets}", "seed": args.seed},
        "loop_ms": round(total_ms, 4),
        "token_steps_per_s": round(cfg.n * cfg.steps / (total_ms * 1e-3), 1),
        "per_step": per_step,
        "dense_loop_ms": None if dense_ms is None else round(dense_ms, 4),
        "speedup_vs_dense": None if dense_ms is None else round(dense_ms / total_ms, 3),
        "repetitions": reps,
    }


def bench_hsa_loop(args, torch, tsa, cfg):
    """The sampling loop with the cached Euler update and the phase window (fp32 state)."""
    from workloads import generate

    dev = torch.device("cuda:0")
    inp = generate.hsa_inputs(cfg, args.seed)
    x0, x1 = inp["xs"][0].to(dev), inp["xs"][1].to(dev)
    layer = tsa.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, inp["w_qkv"].to(dev), device=dev)
    counts, gper = cfg.group_counts(), cfg.group_periods()
    sig = cfg.sigmas()
    period = torch.empty(cfg.n, dtype=torch.uint8, device=dev)
    layer.select(x1, x0, k=1)
    tsa.assign_groups(layer.scores, counts, gper, period, layer.workspace)
    stream = torch.cuda.current_stream()
    x = torch.empty(cfg.n, cfg.dim, dtype=torch.float32, device=dev)

    def run(window, t_loop=None):
        x.copy_(x0)
        if t_loop:
            t_loop.start()
        layer.hsa_run(x, period, sig, window, counts, gper)
        if t_loop:
            t_loop.stop()

    run(cfg.window)
    reps = max(3, args.steps // 8)
    t_loop = EventTimer(torch, stream)
    for _ in range(reps):
        run(cfg.window, t_loop)
    t_dense = EventTimer(torch, stream)
    if not args.no_dense:
        for _ in range(reps):
            run(cfg.steps, t_dense)
    # the Euler kernel alone: read x (fp32) and v_hat (bf16), write x
    t_eu = EventTimer(torch, stream)
    flush = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device=dev)
    for _ in range(20):
        flush.max()
        t_eu.start()
        tsa.euler_update(x, layer.out, -1.0 / cfg.steps)
        t_eu.stop()
    torch.cuda.synchronize()
    loop = stats(t_loop.times())
    counts_per_step = [cfg.n if (i < cfg.window or i >= cfg.steps - cfg.window)
                       else tsa.hsa_active_count(counts, gper, i) for i in range(cfg.steps)]
    flops = sum(cfg.attn_flops(c) for c in counts_per_step)
    dense = None if args.no_dense else stats(t_dense.times())
    return {
        "metric": "HSA sampling loop (Euler update, phase window): effective TFLOP/s over T steps",
        "value": round(flops / (loop["median"] * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "higher_is_better": True,
        "dtype": "bf16 (fp32 latent state)",
        "data": "synthetic (seeded generator; random-init projection weights)",
        "config": {"workload": f"{cfg.name}: N={cfg.n}, D={cfg.dim}, {cfg.heads}x{cfg.head_dim}, T={cfg.steps}, "
                               f"window={cfg.window}, linear sigmas, groups {cfg.group_pcts}% budgets "
                               f"{cfg.group_budgets}", "seed": args.seed},
        "active_per_step": counts_per_step,
        "loop_ms": loop,
        "token_steps_per_s": round(cfg.n * cfg.steps / (loop["median"] * 1e-3), 1),
        "dense_loop_ms": dense,
        "speedup_vs_dense": None if dense is None else round(dense["median"] / loop["median"], 3),
        "euler": roofline_entry("hbm", cfg.n * cfg.dim * (4 + 2 + 4), stats(t_eu.times()), "GB/s"),
    }


def bench_lipar(args, torch, tsa, cfg):
    """LIPAR inter-frame sweep: one pruned pass over the whole clip per active fraction."""
    from workloads import generate

    dev = torch.device("cuda:0")
    inp = generate.lipar_inputs(cfg, args.seed)
    x = inp["x"].to(dev)
    layer = tsa.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, inp["w_qkv"].to(dev), device=dev)
    stream = torch.cuda.current_stream()
    points = []
    reps = max(3, args.steps // 10)
    for p, (pct, k) in enumerate(zip(cfg.sweep_pcts, cfg.sweep_counts())):
        eps = generate.lipar_eps(cfg, args.seed, p).to(dev)
        layer.step_lipar(x, eps, cfg.hw, k, cfg.sigma)
        tm = EventTimer(torch, stream)
        for _ in range(reps):
            tm.start()
            layer.step_lipar(x, eps, cfg.hw, k, cfg.sigma)
            tm.stop()
        torch.cuda.synchronize()
        st = stats(tm.times())
        fl = cfg.attn_flops(k)
        points.append({"active_pct": pct, "n_active": k, "ms": st,
                       "attn_tflops_effective": round(fl / (st["median"] * 1e-3) / 1e12, 2),
                       "tokens_per_s": round(cfg.n / (st["median"] * 1e-3), 1)})
        del eps
    full = points[-1]["ms"]["median"]
    for pt in points:
        pt["speedup_vs_100pct"] = round(full / pt["ms"]["median"], 3)
    return {
        "metric": "LIPAR inter-frame sweep: pass time, effective TFLOP/s and tokens/s per active fraction",
        "value": points[0]["attn_tflops_effective"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic (seeded generator; random-init projection weights)",
        "config": {"workload": f"{cfg.name}: F={cfg.frames} H={cfg.height} W={cfg.width} -> N={cfg.n}, "
                               f"D={cfg.dim}, {cfg.heads}x{cfg.head_dim}, sigma={cfg.sigma}", "seed": args.seed},
        "points": points,
        "repetitions": reps,
    }


def bench_lipar_lif(args, torch, tsa, cfg):
    """LIPAR pass with the long/short-term mask and the restoration of pruned frames."""
    from workloads import generate

    dev = torch.device("cuda:0")
    inp = generate.lipar_inputs(cfg, args.seed)
    x = inp["x"].to(dev)
    eps = generate.lipar_eps(cfg, args.seed, 0).to(dev)
    layer = tsa.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, inp["w_qkv"].to(dev), device=dev)
    stream = torch.cuda.current_stream()
    k = layer.step_lipar_lif(x, eps, cfg.frames, cfg.hw, cfg.tau_short, cfg.tau_long, cfg.sigma)
    reps = max(3, args.steps // 10)
    t_pass = EventTimer(torch, stream)
    for _ in range(reps):
        t_pass.start()
        layer.step_lipar_lif(x, eps, cfg.frames, cfg.hw, cfg.tau_short, cfg.tau_long, cfg.sigma)
        t_pass.stop()
    mask = torch.empty(cfg.n, dtype=torch.uint8, device=dev)
    flush = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device=dev)
    t_mask, t_rest = EventTimer(torch, stream), EventTimer(torch, stream)
    for _ in range(20):
        flush.max()
        t_mask.start()
        tsa.lif_mask(x, cfg.frames, cfg.hw, cfg.tau_short, cfg.tau_long, mask)
        t_mask.stop()
        flush.max()
        t_rest.start()
        tsa.restore_frames(layer.out, mask, cfg.frames, cfg.hw)
        t_rest.stop()
    torch.cuda.synchronize()
    st = stats(t_pass.times())
    fl = cfg.attn_flops(k)
    row = cfg.dim * 2
    return {
        "metric": "LIPAR pass with long/short-term mask + restoration: effective TFLOP/s and tokens/s",
        "value": round(fl / (st["median"] * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic (seeded generator; random-init projection weights)",
        "config": {"workload": f"{cfg.name}: F={cfg.frames} H={cfg.height} W={cfg.width} -> N={cfg.n}, "
                               f"D={cfg.dim}, {cfg.heads}x{cfg.head_dim}, abs L1 thresholds short "
                               f"{cfg.tau_short} / long {cfg.tau_long}, sigma={cfg.sigma}", "seed": args.seed},
        "n_active": k,
        "active_frac": round(k / cfg.n, 4),
        "pass_ms": st,
        "tokens_per_s": round(cfg.n / (st["median"] * 1e-3), 1),
        "lif_mask": roofline_entry("hbm", cfg.n * row + cfg.n, stats(t_mask.times()), "GB/s"),
        "restore": roofline_entry("hbm", cfg.n * row + cfg.n, stats(t_rest.times()), "GB/s"),
        "repetitions": reps,
    }


def bench_reuse(args, torch, tsa, cfg):
    """Timeripple partial-score reuse (Timeripple page, Metodología §2) over a frame-correlated
    clip: the dense pass with reuse (rotated QKV of every token, reuse on Q and K, attention of
    the effective vectors) against the same pass without reuse, the share of partial scores
    reused, and the reuse kernels alone against HBM."""
    import numpy as np

    from workloads import generate

    dev = torch.device("cuda:0")
    inp = generate.lipar_inputs(cfg, args.seed)
    x = inp["x"].to(dev)
    layer = tsa.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, inp["w_qkv"].to(dev), device=dev,
                                     rope=(cfg.height, cfg.width, 10000.0))
    th = cfg.reuse_theta
    stream = torch.cuda.current_stream()
    for _ in range(max(1, args.warmup // 5)):
        layer.reuse_forward(x, th, th)
        layer.dense_forward(x)
    torch.cuda.synchronize()
    reps = max(3, args.steps // 10)
    t_pass, t_dense = EventTimer(torch, stream), EventTimer(torch, stream)
    for _ in range(reps):
        t_pass.start()
        layer.reuse_forward(x, th, th)
        t_pass.stop()
        t_dense.start()
        layer.dense_forward(x)
        t_dense.stop()
    layer.reuse_forward(x, th, th)
    torch.cuda.synchronize()
    # the reuse kernels alone (Q then K rows of the last pass), MALL flushed before each repetition
    flush = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device=dev)
    t_reuse = EventTimer(torch, stream)
    for _ in range(20):
        flush.max()
        t_reuse.start()
        tsa.timeripple_reuse(layer.q_a, cfg.heads, cfg.head_dim, cfg.height, cfg.width, th, layer._q_eff,
                             layer._reuse_ws)
        t_reuse.stop()
    torch.cuda.synchronize()
    ident = np.arange(cfg.n)[:, None]
    d_t = cfg.head_dim - 2 * 2 * (cfg.head_dim // 6)
    sizes = np.array([d_t, 2 * (cfg.head_dim // 6), 2 * (cfg.head_dim // 6)], dtype=np.float64)
    reuse = {}
    for name, src in (("q", layer.src_q), ("k", layer.src_k)):
        sh = src.cpu().numpy()
        used = sh != ident[:, :, None]
        per_group = used.mean(axis=(0, 1))
        reuse[name] = {"entries_reused": {a: round(float(per_group[i]), 4) for i, a in enumerate("tyx")},
                       "partial_score_share_reused": round(float((per_group * sizes).sum() / sizes.sum()), 4)}
    st, sd = stats(t_pass.times()), stats(t_dense.times())
    fl = 4 * cfg.n * cfg.n * cfg.head_dim * cfg.heads
    reuse_bytes = 2 * cfg.n * cfg.dim * 2 + 2 * cfg.n * cfg.heads * 3 * 4
    return {
        "metric": "Timeripple partial-score reuse: dense pass with reuse, effective TFLOP/s and share of "
                  "partial scores reused",
        "value": round(fl / (st["median"] * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic (seeded frame-correlated clip; random-init projection weights)",
        "config": {"workload": f"{cfg.name}: F={cfg.frames} H={cfg.height} W={cfg.width} -> N={cfg.n}, "
                               f"D={cfg.dim}, {cfg.heads}x{cfg.head_dim}, rotary Q/K, thresholds "
                               f"(t, y, x) = {tuple(cfg.reuse_theta)} on Q and K", "seed": args.seed},
        "pass_ms": st,
        "dense_pass_without_reuse_ms": sd,
        "reuse": reuse,
        "reuse_kernels_one_tensor": roofline_entry("hbm", reuse_bytes, stats(t_reuse.times()), "GB/s"),
        "note": "reused partial scores are taken as effective Q/K channels; the attention kernel "
                "computes every score, so the pass costs what the dense pass costs plus the reuse kernels",
        "repetitions": reps,
    }


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the pruned layer runs unsharded on a single MI355X "
              "(multi-GPU sharding is design-only). Run with --gpus 1.", file=sys.stderr)
        return 2

    if args.copy_calibration:
        return copy_calibration()

    import torch

    import token_sparse_attention_rel_amd as tsa
    from workloads import configs

    cfg = configs.get_config(args.workload)
    torch.cuda.set_device(0)
    fn = {"step": bench_step, "hsa": bench_hsa, "hsa_loop": bench_hsa_loop, "lipar": bench_lipar,
          "lipar_lif": bench_lipar_lif, "reuse": bench_reuse}[cfg.kind]
    rec = fn(args, torch, tsa, cfg)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
