"""End-to-end GPU parity of the pruned layer step against the CPU oracle.

Small workloads are compared element by element; the full-size workloads are
run exactly as the benchmark runs them and compared on the whole index lists,
the whole cache and a seeded sample of output rows (rows are independent
given the cache, so the oracle computes just those).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_util as G
from oracle import reference as ref
from workloads import configs, generate
from workloads.configs import scaled

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    G.need_gpu()


def tsa():
    import token_sparse_attention_rel_amd as t
    return t


def _step_case(cfg, seed=0, fused=True, sample=None):
    """Run one top-k step on the GPU and the oracle; compare."""
    t = tsa()
    print(f"  case {cfg.name} N={cfg.n} D={cfg.dim} H={cfg.heads} k={cfg.n_active} seed={seed}", flush=True)
    inp = generate.step_inputs(cfg, seed)
    x_prev, x_cur, w = inp["x_prev"], inp["x_cur"], inp["w_qkv"]
    layer = t.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, G.dev(w))
    xp, xc = G.dev(x_prev), G.dev(x_cur)
    layer.init_cache(xp)
    torch.cuda.synchronize()
    k_init, v_init = G.host64(layer.k_cache), G.host64(layer.v_cache)
    layer.step_topk(xc, xp, cfg.n_active, fused=fused)
    torch.cuda.synchronize()

    xp64, xc64, w64 = G.host64(x_prev), G.host64(x_cur), G.host64(w)
    kc, vc = ref.init_kv_cache(xp64, w64)
    d = cfg.dim
    # elementwise bound on a seeded sample of rows (all rows for the small workloads)
    chk = np.arange(cfg.n) if cfg.n <= 40000 else np.sort(np.random.default_rng(7).choice(cfg.n, 4096, replace=False))
    axp = np.abs(ref.round_bf16(xp64[chk]))
    wk, wv = np.abs(w64[d:2 * d]), np.abs(w64[2 * d:])
    G.assert_projection_close(k_init[chk], kc[chk], axp @ wk.T, d, "initial K cache")
    G.assert_projection_close(v_init[chk], vc[chk], axp @ wv.T, d, "initial V cache")
    G.assert_close(k_init, kc, "initial K cache (all rows)", mabs=np.inf)
    scores = ref.token_scores(xc64, xp64)
    mask = ref.select_topk(scores, cfg.n_active)
    gm = layer.mask.cpu().numpy().astype(bool)
    flips = G.mask_mismatch_ok(gm, mask, scores, cfg.n_active)
    print(f"  near-threshold mask flips: {flips}", flush=True)
    assert flips == 0  # the static/moving gap leaves no token near the threshold here
    idx, pidx = ref.compact(mask)
    assert np.array_equal(layer.idx.cpu().numpy()[:idx.size], idx)
    assert np.array_equal(layer.pidx.cpu().numpy()[:pidx.size], pidx)
    assert int(layer.n_active.item()) == idx.size
    gs = G.host64(layer.scores)
    fin = np.isfinite(scores)
    assert np.max(np.abs(gs[fin] - scores[fin]) / np.maximum(scores[fin], 1e-30)) <= G.SCORE_RTOL

    p = ref.project(xc64[idx], w64, "kv")
    ref.kv_cache_sync(kc, vc, idx, p["k"], p["v"])
    gk, gv = G.host64(layer.k_cache), G.host64(layer.v_cache)
    # fresh rows: elementwise bound (sampled for the large workloads)
    fr = idx if idx.size <= 20000 else np.sort(np.random.default_rng(8).choice(idx, 4096, replace=False))
    axc = np.abs(ref.round_bf16(xc64[fr]))
    G.assert_projection_close(gk[fr], kc[fr], axc @ wk.T, d, "K cache (fresh rows)")
    G.assert_projection_close(gv[fr], vc[fr], axc @ wv.T, d, "V cache (fresh rows)")
    G.assert_close(gk, kc, "K cache (all rows)", mabs=np.inf)
    G.assert_close(gv, vc, "V cache (all rows)", mabs=np.inf)
    # stale rows are bit-identical to what the cache held before the step
    assert np.array_equal(gk[pidx], k_init[pidx]) and np.array_equal(gv[pidx], v_init[pidx])

    go = G.host64(layer.out)
    assert np.all(go[pidx] == 0.0)  # inactive rows untouched (zero-initialised)
    rows = np.arange(idx.size) if sample is None else np.sort(np.random.default_rng(seed).choice(idx.size, sample, replace=False))
    q = ref.project(xc64[idx[rows]], w64, "q")["q"]
    o = ref.attention(q, kc, vc, cfg.heads)
    G.assert_close(go[idx[rows]], o, "output rows")
    return layer


def test_tiny_step_full_parity():
    _step_case(configs.get_config("tiny"))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_wan_shape_scaled_step(seed):
    cfg = scaled(configs.get_config("wan13b"), frames=3, height=10, width=52)
    _step_case(cfg, seed)


def test_head_dim_64_scaled_step():
    cfg = scaled(configs.get_config("wan13b"), frames=2, height=15, width=40, dim=512, heads=8)
    _step_case(cfg, 0)


def test_fused_and_unfused_paths_bit_identical():
    t = tsa()
    cfg = scaled(configs.get_config("wan13b"), frames=2, height=20, width=52)
    inp = generate.step_inputs(cfg, 0)
    outs = []
    for fused in (True, False):
        layer = t.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, G.dev(inp["w_qkv"]))
        xp, xc = G.dev(inp["x_prev"]), G.dev(inp["x_cur"])
        layer.init_cache(xp)
        layer.step_topk(xc, xp, cfg.n_active, fused=fused)
        outs.append((layer.out.clone(), layer.k_cache.clone(), layer.v_cache.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_concurrent_streams_match_sequential_steps():
    """The library keeps no per-call state: two layers stepping at the same time on two
    streams (default priority) give the bits they give one after the other, with the split
    attention schedule and its workspace on both."""
    t = tsa()
    cfgs = [scaled(configs.get_config("wan13b"), frames=3, height=20, width=52),
            scaled(configs.get_config("wan13b"), frames=2, height=30, width=40)]
    layers, xs = [], []
    for i, cfg in enumerate(cfgs):
        inp = generate.step_inputs(cfg, i)
        layers.append(t.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, G.dev(inp["w_qkv"]),
                                             split_attention=True))
        xs.append((G.dev(inp["x_prev"]), G.dev(inp["x_cur"])))

    def run(streams):
        outs = []
        for layer, (xp, xc), cfg, st in zip(layers, xs, cfgs, streams):
            with torch.cuda.stream(st):
                layer.init_cache(xp)
                for _ in range(3):
                    layer.step_topk(xc, xp, cfg.n_active)
        torch.cuda.synchronize()
        for layer in layers:
            outs.append((layer.out.clone(), layer.k_cache.clone(), layer.idx.clone(), layer.mask.clone()))
        return outs

    cur = torch.cuda.current_stream()
    seq = run([cur, cur])
    par = run([torch.cuda.Stream(), torch.cuda.Stream()])
    for a, b in zip(seq, par):
        for x, y in zip(a, b):
            assert torch.equal(x, y)


def test_threshold_step_on_a_side_stream_reads_its_own_count():
    """step_threshold on a stream other than the current one: the active count is read back
    after the selection queued on that stream (which starts late behind a long product), so
    the step uses the count of this selection, not whatever the buffer held."""
    t = tsa()
    cfg = scaled(configs.get_config("wan13b"), frames=2, height=20, width=52)
    inp = generate.step_inputs(cfg, 3)
    xp64, xc64 = G.host64(inp["x_prev"]), G.host64(inp["x_cur"])
    tau = 0.1  # between the static (about 0.01) and the moving (about 0.5) scores
    want = ref.select_threshold(ref.token_scores(xc64, xp64), tau)
    layer = t.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, G.dev(inp["w_qkv"]))
    xp, xc = G.dev(inp["x_prev"]), G.dev(inp["x_cur"])
    layer.init_cache(xp)
    layer.n_active.fill_(-5)
    big = torch.randn(4096, 4096, device="cuda")
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        for _ in range(8):
            big = big @ big.T / 64.0  # keeps the side stream busy before the selection
    n_act = layer.step_threshold(xc, xp, tau, stream=side)
    torch.cuda.synchronize()
    assert n_act == int(want.sum())
    idx, _ = ref.compact(want)
    assert np.array_equal(layer.idx.cpu().numpy()[:n_act], idx)


def test_threshold_step_zero_change_leaves_state():
    t = tsa()
    cfg = scaled(configs.get_config("wan13b"), frames=2, height=10, width=16)
    inp = generate.step_inputs(cfg, 0)
    layer = t.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, G.dev(inp["w_qkv"]))
    xp = G.dev(inp["x_prev"])
    layer.init_cache(xp)
    layer.out.fill_(3.0)
    k0, v0 = layer.k_cache.clone(), layer.v_cache.clone()
    n_active = layer.step_threshold(xp.clone(), xp, tau=1e-6)
    torch.cuda.synchronize()
    assert n_active == 0
    assert torch.equal(layer.k_cache, k0) and torch.equal(layer.v_cache, v0)
    assert bool((layer.out == 3.0).all())


def test_full_activity_is_dense_attention():
    t = tsa()
    cfg = scaled(configs.get_config("wan13b"), frames=2, height=10, width=26)
    inp = generate.step_inputs(cfg, 1)
    layer = t.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, G.dev(inp["w_qkv"]))
    xp, xc = G.dev(inp["x_prev"]), G.dev(inp["x_cur"])
    layer.init_cache(xp)
    layer.step_topk(xc, xp, cfg.n)
    torch.cuda.synchronize()
    p = ref.project(G.host64(inp["x_cur"]), G.host64(inp["w_qkv"]))
    G.assert_close(G.host64(layer.out), ref.attention(p["q"], p["k"], p["v"], cfg.heads), "dense")


def test_hsa_schedule_loop_scaled():
    t = tsa()
    cfg = scaled(configs.get_config("hsa"), frames=2, height=12, width=52)
    inp = generate.hsa_inputs(cfg, 0)
    xs, w = inp["xs"], inp["w_qkv"]
    counts, periods = cfg.group_counts(), cfg.group_periods()
    assert sum(counts) == cfg.n
    layer = t.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, G.dev(w))
    xds = [G.dev(x) for x in xs]
    layer.init_cache(xds[0])
    # rank once at step 0 from the change between x_1 and x_0
    layer.select(xds[1], xds[0], k=1)
    period = torch.empty(cfg.n, dtype=torch.uint8, device="cuda")
    t.assign_groups(layer.scores, counts, periods, period, layer.workspace)

    w64 = G.host64(w)
    x64 = [G.host64(x) for x in xs]
    kc, vc = ref.init_kv_cache(x64[0], w64)
    out = np.zeros((cfg.n, cfg.dim))
    s0 = ref.token_scores(x64[1], x64[0])
    per = ref.assign_periods(s0, counts, periods)
    assert np.array_equal(period.cpu().numpy(), per)
    for i in range(cfg.steps):
        n_act = t.hsa_active_count(counts, periods, i)
        layer.select(None, periods=period, step=i)
        layer.forward_active(xds[i + 1], n_act)
        torch.cuda.synchronize()
        res = ref.layer_step(x64[i + 1], w64, cfg.heads, kc, vc, out, mask=ref.schedule_mask(per, i))
        assert res["idx"].size == n_act
        assert np.array_equal(layer.idx.cpu().numpy()[:n_act], res["idx"])
        G.assert_close(G.host64(layer.out), out, f"step {i} out")
        G.assert_close(G.host64(layer.k_cache), kc, f"step {i} K cache", mabs=np.inf)
        fresh = res["idx"]
        ax = np.abs(x64[i + 1][fresh])
        G.assert_projection_close(G.host64(layer.k_cache)[fresh], kc[fresh],
                                  ax @ np.abs(w64[cfg.dim:2 * cfg.dim]).T, cfg.dim, f"step {i} fresh K")


def test_debug_layer_checks_the_host_count():
    """With debug=True a step given the wrong active count raises before any kernel runs
    with it; the right count runs as usual."""
    t = tsa()
    cfg = scaled(configs.get_config("hsa"), frames=2, height=6, width=20)
    inp = generate.hsa_inputs(cfg, 0)
    layer = t.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, G.dev(inp["w_qkv"]), debug=True)
    xs = [G.dev(x) for x in inp["xs"]]
    layer.init_cache(xs[0])
    layer.select(xs[1], xs[0], k=1)
    counts, periods = cfg.group_counts(), cfg.group_periods()
    period = torch.empty(cfg.n, dtype=torch.uint8, device="cuda")
    t.assign_groups(layer.scores, counts, periods, period, layer.workspace)
    layer.select(None, periods=period, step=1)
    right = t.hsa_active_count(counts, periods, 1)
    out0 = layer.out.clone()
    with pytest.raises(ValueError):
        layer.forward_active(xs[2], right + 1)
    torch.cuda.synchronize()
    assert torch.equal(layer.out, out0)
    layer.forward_active(xs[2], right)
    torch.cuda.synchronize()


def _lipar_case(cfg, pct_index, seed=0, sample=None):
    t = tsa()
    inp = generate.lipar_inputs(cfg, seed)
    x, w = inp["x"], inp["w_qkv"]
    eps = generate.lipar_eps(cfg, seed, pct_index)
    k = cfg.sweep_counts()[pct_index]
    print(f"  case {cfg.name} N={cfg.n} D={cfg.dim} k={k}", flush=True)
    layer = t.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, G.dev(w))
    xd = G.dev(x)
    layer.step_lipar(xd, G.dev(eps), cfg.hw, k, cfg.sigma)
    torch.cuda.synchronize()
    x64, w64, e64 = G.host64(x), G.host64(w), G.host64(eps)
    kc = np.zeros((cfg.n, cfg.dim))
    vc = np.zeros((cfg.n, cfg.dim))
    out = np.zeros((cfg.n, cfg.dim))
    rows = None
    if sample is not None:
        rows = np.sort(np.random.default_rng(seed).choice(k, min(sample, k), replace=False))
    res = ref.lipar_step(x64, e64, w64, cfg.heads, cfg.hw, k, cfg.sigma, kc, vc, out, query_rows=rows)
    gm = layer.mask.cpu().numpy().astype(bool)
    flips = G.mask_mismatch_ok(gm, res["mask"], res["scores"], k)
    print(f"  near-threshold mask flips: {flips}", flush=True)
    if flips:
        # compare downstream with the oracle's own mask fed to the GPU (MASK mode)
        layer.k_cache.zero_()
        layer.v_cache.zero_()
        layer.out.zero_()
        mask_d = G.dev(torch.from_numpy(res["mask"].astype(np.uint8)))
        layer.select(None, mask=mask_d)
        from token_sparse_attention_rel_amd import _binding as B
        B.qkv_active(xd, layer.idx, k, layer.w_qkv, q_out=layer.q_a, k_out=layer.k_cache,
                     v_out=layer.v_cache, out_is_cache=True, n_cache=cfg.n)
        if cfg.n - k:
            B.qkv_active(xd, layer.pidx, cfg.n - k, layer.w_qkv, k_out=layer.k_cache,
                         v_out=layer.v_cache, out_is_cache=True, n_cache=cfg.n, eps=G.dev(eps),
                         src_row_offset=cfg.hw, sigma=cfg.sigma)
        B.sparse_query_attention(layer.q_a, layer.k_cache, layer.v_cache, k, cfg.heads,
                                 cfg.dim // cfg.heads, layer.out, out_rows=layer.idx)
        torch.cuda.synchronize()
    idx = res["idx"]
    assert np.array_equal(layer.idx.cpu().numpy()[:k], idx)
    gk, gv = G.host64(layer.k_cache), G.host64(layer.v_cache)
    pidx = res["pidx"]
    # rows of active tokens: same bf16 inputs as the oracle -> rounding + fp32 summation bound
    sm = idx if idx.size <= 20000 else np.sort(np.random.default_rng(9).choice(idx, 4096, replace=False))
    ax = np.abs(x64[sm])
    d = cfg.dim
    G.assert_projection_close(gk[sm], kc[sm], ax @ np.abs(w64[d:2 * d]).T, d, "K cache (active rows)")
    G.assert_projection_close(gv[sm], vc[sm], ax @ np.abs(w64[2 * d:]).T, d, "V cache (active rows)")
    G.assert_close(gk[idx], kc[idx], "K cache (all active rows)", mabs=np.inf)
    G.assert_close(gv[idx], vc[idx], "V cache (all active rows)", mabs=np.inf)
    if pidx.size:
        # rows from recovered inputs: those inputs carry their own fp32 rounding, so compare
        # with the layer tolerance, max-abs taken relative to max(1, |value|)
        for name, a, b in (("K", gk[pidx], kc[pidx]), ("V", gv[pidx], vc[pidx])):
            rf = G.rel_frob(a, b)
            rel_abs = float(np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b))))
            print(f"  {name} cache (recovered rows): rel_frob={rf:.3e} scaled max_abs={rel_abs:.3e}", flush=True)
            assert rf <= G.REL_FROB and rel_abs <= G.MAX_ABS
    go = G.host64(layer.out)
    if rows is None:
        G.assert_close(go[idx], res["o_a"], "output rows")
    else:
        G.assert_close(go[idx[rows]], res["o_a"], "sampled output rows")
    return flips


@pytest.mark.parametrize("pct_index", [0, 1, 2, 3, 4])
def test_lipar_sweep_scaled(pct_index):
    cfg = scaled(configs.get_config("lipar"), frames=5, height=9, width=16, dim=256, heads=2)
    _lipar_case(cfg, pct_index)


# ----------------------------------------------------------- full size

@pytest.mark.slow
def test_wan13b_full_size_sampled():
    _step_case(configs.get_config("wan13b"), 0, sample=96)


@pytest.mark.slow
def test_large_full_size_sampled():
    _step_case(configs.get_config("large"), 0, sample=48)


@pytest.mark.slow
@pytest.mark.parametrize("pct_index", [0, 1, 2, 3, 4])
def test_lipar_full_size_sampled(pct_index):
    """LIPAR sweep at full size (N = 118800, D = 3072, 24 heads): 5 / 10 / 25 / 50 / 100 %
    active; 100 % is the dense check (every row projected from its own latent)."""
    _lipar_case(configs.get_config("lipar"), pct_index, sample=48)


@pytest.mark.slow
def test_hsa_schedule_full_size_every_step():
    """The HSA 8-step schedule at full size (N = 32760, D = 1536, 12 heads; per-step active
    counts N, N/4, N/2, N/4, N, N/4, N/2, N/4): the period of every token and the whole active
    list of every step bit for bit; the whole K/V cache after every step against the oracle's
    (fresh rows within the projection bound on a sample, stale rows bit-identical to the
    previous step); a seeded sample of the step's output rows against the oracle's attention
    over its own cache; output rows of skipped tokens bit-identical to the previous step."""
    t = tsa()
    cfg = configs.get_config("hsa")
    print(f"  case {cfg.name} N={cfg.n} D={cfg.dim} H={cfg.heads} T={cfg.steps}", flush=True)
    inp = generate.hsa_inputs(cfg, 0)
    xs, w = inp["xs"], inp["w_qkv"]
    counts, periods = cfg.group_counts(), cfg.group_periods()
    d = cfg.dim
    layer = t.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, G.dev(w))
    layer.init_cache(G.dev(xs[0]))
    layer.select(G.dev(xs[1]), G.dev(xs[0]), k=1)
    period = torch.empty(cfg.n, dtype=torch.uint8, device="cuda")
    t.assign_groups(layer.scores, counts, periods, period, layer.workspace)
    torch.cuda.synchronize()

    w64 = G.host64(w)
    wk, wv = np.abs(w64[d:2 * d]), np.abs(w64[2 * d:])
    kc, vc = ref.init_kv_cache(G.host64(xs[0]), w64)
    per = ref.assign_periods(ref.token_scores(G.host64(xs[1]), G.host64(xs[0])), counts, periods)
    assert np.array_equal(period.cpu().numpy(), per)
    prev_k, prev_v = G.host64(layer.k_cache), G.host64(layer.v_cache)
    prev_out = G.host64(layer.out)
    rng = np.random.default_rng(17)
    for i in range(cfg.steps):
        n_act = t.hsa_active_count(counts, periods, i)
        layer.select(None, periods=period, step=i)
        layer.forward_active(G.dev(xs[i + 1]), n_act)
        torch.cuda.synchronize()
        mask = ref.schedule_mask(per, i)
        idx, pidx = ref.compact(mask)
        print(f"  step {i}: {idx.size} active", flush=True)
        assert idx.size == n_act
        assert np.array_equal(layer.idx.cpu().numpy()[:n_act], idx)
        assert np.array_equal(layer.pidx.cpu().numpy()[:pidx.size], pidx)
        assert int(layer.n_active.item()) == n_act
        x64 = G.host64(xs[i + 1])
        p = ref.project(x64[idx], w64, "kv")
        ref.kv_cache_sync(kc, vc, idx, p["k"], p["v"])
        gk, gv, go = G.host64(layer.k_cache), G.host64(layer.v_cache), G.host64(layer.out)
        G.assert_close(gk, kc, f"step {i} K cache (all rows)", mabs=np.inf)
        G.assert_close(gv, vc, f"step {i} V cache (all rows)", mabs=np.inf)
        fr = idx if idx.size <= 8192 else np.sort(rng.choice(idx, 8192, replace=False))
        ax = np.abs(ref.round_bf16(x64[fr]))
        G.assert_projection_close(gk[fr], kc[fr], ax @ wk.T, d, f"step {i} K cache (fresh rows)")
        G.assert_projection_close(gv[fr], vc[fr], ax @ wv.T, d, f"step {i} V cache (fresh rows)")
        assert np.array_equal(gk[pidx], prev_k[pidx]) and np.array_equal(gv[pidx], prev_v[pidx])
        assert np.array_equal(go[pidx], prev_out[pidx])  # skipped tokens keep their output
        rows = np.sort(rng.choice(idx.size, 48, replace=False))
        q = ref.project(x64[idx[rows]], w64, "q")["q"]
        G.assert_close(go[idx[rows]], ref.attention(q, kc, vc, cfg.heads), f"step {i} sampled output rows")
        prev_k, prev_v, prev_out = gk, gv, go
