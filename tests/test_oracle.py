"""The CPU oracle against facts other than itself (closed forms, library routines, brute force)."""

from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import pins
from oracle import brute
from oracle import reference as ref
from workloads import configs, generate


def load_golden_schedule(root):
    rows = []
    with open(os.path.join(root, "tests", "golden", "hsa_schedule_T8.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            vals = [int(v) for v in line.split()]
            rows.append((vals[0], vals[1], vals[2:]))
    return rows


# ------------------------------------------------------------ bf16 rounding

def test_round_bf16_matches_torch_conversion():
    r = np.random.default_rng(0)
    # wide exponent range, random mantissas, both signs
    x = (r.standard_normal(200000) * np.exp2(r.integers(-140, 126, 200000))).astype(np.float32)
    # exact ties (low 16 bits 0x8000) and near-ties
    bits = r.integers(0, 2 ** 31, 20000, dtype=np.uint64).astype(np.uint32)
    ties = ((bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    near = ((bits & np.uint32(0xFFFF0000)) | np.uint32(0x7FFF)).view(np.float32)
    sub = (r.standard_normal(5000) * 2.0 ** -130).astype(np.float32)
    big = np.float32([3.3895e38, 3.39e38, -3.395e38, 1e38])
    for arr in (x, ties, near, sub, big):
        arr = arr[np.isfinite(arr)]
        want = torch.from_numpy(arr).to(torch.bfloat16).to(torch.float64).numpy()
        got = ref.round_bf16(arr.astype(np.float64))
        assert np.array_equal(got, want)


def test_round_bf16_float64_ties_and_brute():
    # 1 + 2**-8 is exactly halfway between 1 and 1 + 2**-7: ties to the even neighbour, 1
    assert ref.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert ref.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    # just above the halfway point rounds up (a fp64 value that a fp32 detour would get wrong)
    assert ref.round_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -40]))[0] == 1 + 2.0 ** -7
    r = np.random.default_rng(1)
    x = r.standard_normal(3000) * np.exp2(r.integers(-60, 60, 3000))
    assert np.array_equal(ref.round_bf16(x), np.array([brute.bf16(v) for v in x]))


# ------------------------------------------------------------- step by step

def test_scores_pinned():
    pins.check_scores(ref.token_scores)


def test_topk_pinned():
    pins.check_topk(ref.select_topk)


def test_threshold_pinned():
    pins.check_threshold(ref.select_threshold)


def test_compact_pinned():
    pins.check_compact(ref.compact)


def test_schedule_pinned(root):
    pins.check_periods(ref.assign_periods, ref.schedule_mask, load_golden_schedule(root))


def test_recovery_pinned():
    pins.check_recover(ref.recover_rows)


def test_projection_pinned():
    pins.check_project(ref.project)


def test_attention_pinned():
    pins.check_attention(ref.attention)


# ------------------------------------------------------------- whole layer

def _tiny(seed=0, n=48, dim=64, heads=2):
    r = np.random.default_rng(seed)
    x_prev = pins.bf16_values(r.standard_normal((n, dim)))
    scale = np.where(r.random(n) < 0.7, 0.01, 0.5)
    x_cur = pins.bf16_values(x_prev + scale[:, None] * r.standard_normal((n, dim)))
    w = pins.bf16_values(r.standard_normal((3 * dim, dim)) / np.sqrt(dim))
    return x_prev, x_cur, w


def test_layer_step_matches_brute_force():
    heads = 2
    x_prev, x_cur, w = _tiny()
    n, dim = x_cur.shape
    kc, vc = ref.init_kv_cache(x_prev, w)
    out = np.zeros((n, dim))
    res = ref.layer_step(x_cur, w, heads, kc, vc, out, x_ref=x_prev, k=12)

    bkc = [list(rw) for rw in brute.project(x_prev.tolist(), w.tolist(), "k")]
    bvc = [list(rw) for rw in brute.project(x_prev.tolist(), w.tolist(), "v")]
    assert np.array_equal(np.array(bkc), ref.init_kv_cache(x_prev, w)[0])
    bout = [[0.0] * dim for _ in range(n)]
    b = brute.layer_step(x_cur.tolist(), x_prev.tolist(), w.tolist(), heads, bkc, bvc, bout, 12)
    assert list(res["idx"]) == b["idx"]
    assert np.array_equal(kc, np.array(bkc)) and np.array_equal(vc, np.array(bvc))
    assert np.allclose(out, np.array(bout), rtol=1e-12, atol=1e-13)


def test_full_activity_equals_dense_attention():
    heads = 2
    x_prev, x_cur, w = _tiny(1)
    n, dim = x_cur.shape
    kc, vc = ref.init_kv_cache(x_prev, w)
    out = np.zeros((n, dim))
    ref.layer_step(x_cur, w, heads, kc, vc, out, x_ref=x_prev, k=n)
    p = ref.project(x_cur, w)
    assert np.array_equal(kc, p["k"]) and np.array_equal(vc, p["v"])
    assert np.allclose(out, pins.sdpa64(p["q"], p["k"], p["v"], heads), rtol=1e-12, atol=1e-12)


def test_unchanged_tokens_leave_cache_and_output_untouched():
    heads = 2
    x_prev, _, w = _tiny(2)
    n, dim = x_prev.shape
    kc, vc = ref.init_kv_cache(x_prev, w)
    k0, v0 = kc.copy(), vc.copy()
    out = np.full((n, dim), 7.0)
    res = ref.layer_step(x_prev.copy(), w, heads, kc, vc, out, x_ref=x_prev, tau=1e-6)
    assert res["idx"].size == 0
    assert np.array_equal(kc, k0) and np.array_equal(vc, v0) and np.all(out == 7.0)


def test_inactive_rows_keep_stale_cache_and_output():
    heads = 2
    x_prev, x_cur, w = _tiny(3)
    n, dim = x_cur.shape
    kc, vc = ref.init_kv_cache(x_prev, w)
    k0, v0 = kc.copy(), vc.copy()
    out = np.full((n, dim), -3.0)
    res = ref.layer_step(x_cur, w, heads, kc, vc, out, x_ref=x_prev, k=10)
    keep = res["pidx"]
    assert np.array_equal(kc[keep], k0[keep]) and np.array_equal(vc[keep], v0[keep])
    assert np.all(out[keep] == -3.0)
    # active queries see the stale rows: equal to attention over the mixed cache
    mixed_k = k0.copy()
    mixed_k[res["idx"]] = res["k"]
    mixed_v = v0.copy()
    mixed_v[res["idx"]] = res["v"]
    assert np.allclose(out[res["idx"]], pins.sdpa64(res["q"], mixed_k, mixed_v, heads), rtol=1e-12, atol=1e-12)


def test_lipar_full_activity_is_dense_and_recovery_feeds_pruned_rows():
    heads, hw = 2, 8
    r = np.random.default_rng(4)
    n, dim = 40, 32
    x = pins.bf16_values(r.standard_normal((n, dim)))
    eps = pins.bf16_values(r.standard_normal((n, dim)))
    w = pins.bf16_values(r.standard_normal((3 * dim, dim)) / np.sqrt(dim))
    kc, vc, out = np.zeros((n, dim)), np.zeros((n, dim)), np.zeros((n, dim))
    ref.lipar_step(x, eps, w, heads, hw, n, 0.6, kc, vc, out)
    p = ref.project(x, w)
    assert np.allclose(out, pins.sdpa64(p["q"], p["k"], p["v"], heads), rtol=1e-12, atol=1e-12)
    kc, vc, out = np.zeros((n, dim)), np.zeros((n, dim)), np.zeros((n, dim))
    res = ref.lipar_step(x, eps, w, heads, hw, 20, 0.6, kc, vc, out)
    assert set(range(hw)) <= set(res["idx"].tolist())  # first frame has no reference: always kept
    rb = np.array(brute.recover(x.tolist(), eps.tolist(), res["pidx"].tolist(), hw, 0.6))
    kp = np.array(brute.project(rb.tolist(), w.tolist(), "k"))
    assert np.array_equal(kc[res["pidx"]], kp)
    # sampled query rows agree with the full pass
    kc2, vc2, out2 = np.zeros((n, dim)), np.zeros((n, dim)), np.zeros((n, dim))
    res2 = ref.lipar_step(x, eps, w, heads, hw, 20, 0.6, kc2, vc2, out2, query_rows=[0, 5, 19])
    assert np.allclose(res2["o_a"], res["o_a"][[0, 5, 19]], rtol=1e-13, atol=1e-13)


# -------------------------------------------------------------- generator

def test_generator_deterministic_and_structured():
    cfg = configs.get_config("tiny")
    a = generate.step_inputs(cfg, 0)
    b = generate.step_inputs(cfg, 0)
    c = generate.step_inputs(cfg, 1)
    for key in ("x_prev", "x_cur", "w_qkv", "static"):
        assert torch.equal(a[key], b[key])
    assert not torch.equal(a["x_cur"], c["x_cur"])
    assert int(a["static"].sum()) == cfg.n_static == 179
    assert a["x_cur"].dtype == torch.float32 and a["w_qkv"].dtype == torch.bfloat16
    # static tokens barely change, moving tokens change by ~0.5
    d = (a["x_cur"] - a["x_prev"]).abs().mean(1)
    assert float(d[a["static"]].max()) < 0.02 and float(d[~a["static"]].min()) > 0.2


def test_config_counts_are_exact():
    c = configs.CONFIGS
    assert (c["tiny"].n, c["tiny"].n_active) == (256, 64)
    assert (c["wan13b"].n, c["wan13b"].n_active, c["wan13b"].n_static) == (32760, 9828, 22932)
    assert (c["large"].n, c["large"].n_active, c["large"].n_static) == (75600, 15120, 60480)
    assert c["hsa"].group_counts() == (8190, 8190, 16380) and c["hsa"].group_periods() == (1, 2, 4)
    assert c["lipar"].n == 118800 and c["lipar"].sweep_counts() == (5940, 11880, 29700, 59400, 118800)
    assert c["lipar"].n_static == 2700
    assert c["wan13b"].attn_flops(9828) == 4 * 9828 * 32760 * 128 * 12


def test_oracle_on_tiny_workload_is_consistent():
    cfg = configs.get_config("tiny")
    inp = generate.step_inputs(cfg, 0)
    x_prev = inp["x_prev"].double().numpy()
    x_cur = inp["x_cur"].double().numpy()
    w = inp["w_qkv"].double().numpy()
    kc, vc = ref.init_kv_cache(x_prev, w)
    out = np.zeros((cfg.n, cfg.dim))
    res = ref.layer_step(x_cur, w, cfg.heads, kc, vc, out, x_ref=x_prev, k=cfg.n_active)
    # the 64 active tokens are all moving tokens (77 moving, clear score gap)
    static = inp["static"].numpy()
    assert res["idx"].size == 64 and not static[res["idx"]].any()
    assert np.isfinite(out).all()


# ------------------------------------------------ f1 / f2 (steps beside the layer)

def test_euler_pinned():
    pins.check_euler(ref.euler_update)


def test_phase_window_pinned():
    pins.check_window(ref.step_is_dense)


def test_hsa_run_pinned():
    pins.check_hsa_run(ref.hsa_run, ref.schedule_mask)


def test_lif_mask_pinned():
    pins.check_lif_mask(ref.lif_mask, ref.token_scores, ref.select_threshold)


def test_restore_pinned():
    pins.check_restore(ref.restore_frames)


# -------------------------------------------- f3: rotary positions, frame-causal attention

def test_rope_pinned():
    pins.check_rope(ref.rope3d, ref.rope_split, ref.token_position)


def test_project_rope_pinned():
    pins.check_project_rope(ref.project_rope, ref.project, ref.rope3d)


def test_frame_causal_pinned():
    pins.check_frame_causal(ref.attention_frame_causal, ref.attention)


def test_layer_step_rope_causal_matches_brute_force():
    r = np.random.default_rng(19)
    n, dim, heads, h, w = 24, 16, 2, 2, 3
    x = pins.bf16_values(r.standard_normal((n, dim)))
    w_qkv = pins.bf16_values(r.standard_normal((3 * dim, dim)) / np.sqrt(dim))
    mask = r.random(n) < 0.5
    mask[[0, n - 1]] = True
    kc, vc = ref.init_kv_cache(x, w_qkv)
    out = np.zeros((n, dim))
    res = ref.layer_step(x, w_qkv, heads, kc, vc, out, mask=mask, rope=(h, w, 10000.0),
                         causal_frame_tokens=h * w)
    idx = res["idx"]
    # brute force: exact projections, rotated, rounded; cache rows replaced; causal attention
    xb = [[brute.bf16(v) for v in row] for row in x[idx].tolist()]
    exact = {p: brute.matmul_t(xb, w_qkv[i * dim:(i + 1) * dim].tolist()) for i, p in enumerate("qkv")}
    rq = [[brute.bf16(v) for v in row] for row in brute.rope(exact["q"], idx.tolist(), h, w, heads)]
    rk = [[brute.bf16(v) for v in row] for row in brute.rope(exact["k"], idx.tolist(), h, w, heads)]
    rv = [[brute.bf16(v) for v in row] for row in exact["v"]]
    kb, vb = ref.init_kv_cache(x, w_qkv)
    kb, vb = kb.tolist(), vb.tolist()
    for j, t in enumerate(idx):
        kb[t], vb[t] = rk[j], rv[j]
    o = brute.attention_frame_causal(rq, kb, vb, heads, idx.tolist(), h * w)
    assert np.array_equal(res["q"], np.array(rq))
    assert np.allclose(kc, np.array(kb), rtol=0, atol=0)
    assert np.allclose(res["o_a"], np.array(o), rtol=1e-12, atol=1e-12)


def test_reuse_pinned():
    pins.check_reuse(ref.reuse_deltas, ref.reuse_sources, ref.reuse_effective, ref.axis_neighbors,
                     ref.reuse_groups, ref.rope3d)


def test_timeripple_attention_pinned():
    pins.check_timeripple_attention(ref.timeripple_attention, ref.attention, ref.rope3d)
