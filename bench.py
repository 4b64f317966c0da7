"""Benchmark of the pruned attention layer step on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
score + top-k select + compaction, QKV of the active tokens with the fused
KV-cache sync, attention of the active queries over all N cached keys with
the fused scatter back to token order.  Inputs are resident in HBM before
the timed region starts.

Prints ONE JSON line.  ``value`` is the effective layer throughput in
TFLOP/s = 4 * N_active * N * head_dim * heads / step time.  Extra fields give
tokens/s, the per-kernel times, the attention kernel's roofline and the CPU
oracle measured on a bounded sample of the same workload.
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
ATTN_SRC = os.path.join(ROOT, "token_sparse_attention_rel_amd", "csrc", "attention.hip")


def parse_args(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan13b")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample-rows", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
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


ATTN_KERNELS = {
    False: "attention_kernel<128> (active queries x all cached K/V, fused scatter)",
    True: "attention_split_kernel<128> + attention_merge_kernel<128> (active queries x all cached "
          "K/V, fused scatter; timed together)",
}


def _src_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def attention_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 counter summary,
    or None when it is missing or the kernel source changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    try:
        if vals.get("kernel_source_sha256") != _src_hash(ATTN_SRC):
            return None
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


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
    from workloads import configs, generate

    cfg = configs.get_config(args.workload)
    if cfg.kind != "step":
        raise SystemExit("bench.py times single-step workloads (tiny, wan13b, large)")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = generate.step_inputs(cfg, args.seed)
    layer = tsa.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, inp["w_qkv"].to(dev), device=dev,
                                     split_attention=args.attn_schedule == "split")
    xp = inp["x_prev"].to(dev)
    xc = inp["x_cur"].to(dev)
    layer.init_cache(xp)
    k = cfg.n_active
    stream = torch.cuda.current_stream()
    attn_ws = layer.attention_workspace(k)

    for _ in range(args.warmup):
        layer.step_topk(xc, xp, k)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        e = ev[i]
        e[0].record(stream)
        layer.select(xc, xp, k=k)
        e[1].record(stream)
        tsa.qkv_active(xc, layer.idx, k, layer.w_qkv, q_out=layer.q_a, k_out=layer.k_cache,
                       v_out=layer.v_cache, out_is_cache=True, n_cache=cfg.n)
        e[2].record(stream)
        tsa.sparse_query_attention(layer.q_a, layer.k_cache, layer.v_cache, k, cfg.heads,
                                   cfg.head_dim, layer.out, out_rows=layer.idx, workspace=attn_ws)
        e[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    t_sel = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    t_qkv = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    t_att = sum(e[2].elapsed_time(e[3]) for e in ev) / args.steps

    flops = cfg.attn_flops(k)
    dense_ms = None
    if not args.no_dense:
        dl = tsa.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, layer.w_qkv, device=dev)
        dl.init_cache(xp)
        for _ in range(2):
            dl.step_topk(xc, xp, cfg.n)
        torch.cuda.synchronize()
        nd = max(3, args.steps // 4)
        td = time.perf_counter()
        for _ in range(nd):
            dl.step_topk(xc, xp, cfg.n)
        torch.cuda.synchronize()
        dense_ms = (time.perf_counter() - td) * 1e3 / nd
        del dl

    achieved = flops / (t_att * 1e-3) / 1e12
    rec = {
        "metric": METRIC,
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
                        f"(k={k}), {cfg.static_pct}% static tokens, full bidirectional attention",
            "n_tokens": cfg.n,
            "n_active": k,
            "dim": cfg.dim,
            "heads": cfg.heads,
            "head_dim": cfg.head_dim,
            "seed": args.seed,
        },
        "attention_schedule": ("one workgroup per query tile, last round split into key ranges"
                               if attn_ws is not None else "one workgroup per query tile"),
        "tokens_per_s": round(cfg.n / (ms_step * 1e-3), 1),
        "active_tokens_per_s": round(k / (ms_step * 1e-3), 1),
        "attn_tflops": round(achieved, 3),
        "attn_frac_of_mfma_peak": round(achieved / PEAK_BF16_TFLOPS, 4),
        "kernel_ms": {"score_select_compact": round(t_sel, 4), "qkv_gather_cache_sync": round(t_qkv, 4),
                      "attention_scatter": round(t_att, 4)},
        "qkv_tflops": round(cfg.qkv_flops(k) / (t_qkv * 1e-3) / 1e12, 3),
        "dense_layer_ms": None if dense_ms is None else round(dense_ms, 4),
        "speedup_vs_dense": None if dense_ms is None else round(dense_ms / ms_step, 3),
        "roofline": {
            "bound": "mfma",
            "kernel": ATTN_KERNELS[attn_ws is not None],
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": attention_traffic(),
            "algorithmic_flop_per_launch": flops,
        },
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample_rows)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
