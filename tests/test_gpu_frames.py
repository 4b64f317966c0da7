"""GPU parity of the steps beside the layer against the CPU oracle: the cached Euler update
and the sampling loop with its phase window (HSA page §2.3-§2.4), the long/short-term
pruning mask and the restoration of pruned frames (LIPAR page §2.B, Dutch page §2.D)."""

from __future__ import annotations

from dataclasses import replace

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


# ------------------------------------------------------------------ Euler

def _ulp(values, fmt):
    """Spacing of the float32 / bfloat16 grid at |values| (normal range)."""
    a = np.abs(np.asarray(values, np.float64))
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    bits = 24 if fmt == "f32" else 8
    return np.ldexp(1.0, e - bits)


@pytest.mark.parametrize("state", ["f32", "bf16"])
@pytest.mark.parametrize("n,dim,dt", [(1, 8, -0.125), (37, 200, 0.3), (1000, 1536, -0.0625),
                                      (4099, 3072, -0.1234567), (3, 16, 0.0), (32760, 1536, -0.125)])
def test_euler_matches_oracle(state, n, dim, dt):
    t = tsa()
    g = torch.Generator().manual_seed(n + dim)
    x = torch.randn(n, dim, generator=g)
    if state == "bf16":
        x = x.to(torch.bfloat16)
    v = torch.randn(n, dim, generator=g).to(torch.bfloat16)
    xd = G.dev(x)
    t.euler_update(xd, G.dev(v), dt)
    got = G.host64(xd)
    want = ref.euler_update(G.host64(x), G.host64(v), float(np.float32(dt)), store=state)
    # one fused multiply-add: the exact value rounded once to fp32 (then to bf16 for a bf16
    # state), as the oracle does.  The oracle's float64 sum is exact unless the exponents of
    # x and dt*v differ by more than ~21; a float64 rounding can then move a value onto an
    # fp32 tie: allow one ulp on a tiny fraction of elements.
    off = got != want
    assert np.all(np.abs(got - want) <= _ulp(want, state)), "more than one ulp from the oracle"
    frac = off.mean()
    print(f"  {state} n={n} dim={dim}: {off.sum()} elements one ulp off ({frac:.2e})", flush=True)
    assert frac <= 1e-6
    if dt == 0.0:
        assert np.array_equal(got, G.host64(x))


# ------------------------------------------------------- pruning mask

def _lif_cfg(frames, height, width, dim, heads, dtype="bf16"):
    base = configs.get_config("lipar_lif")
    cfg = scaled(base, frames=frames, height=height, width=width, dim=dim, heads=heads)
    # the per-frame change of a token grows with the row length: scale the thresholds
    return replace(cfg, dtype=dtype, tau_short=base.tau_short * dim / base.dim,
                   tau_long=base.tau_long * dim / base.dim)


def _margin(res, tau_s, tau_l):
    """Smallest relative distance of any finite change score from its threshold."""
    def m(s, tau):
        s = s[np.isfinite(s)]
        return float(np.min(np.abs(s - tau) / tau)) if s.size else np.inf
    return min(m(res["short"], tau_s), m(res["long"], tau_l))


@pytest.mark.parametrize("frames,height,width,dim,dtype,kind", [
    (8, 6, 10, 256, "bf16", "abs"), (12, 5, 7, 1000, "bf16", "abs"), (9, 4, 9, 512, "fp32", "abs"),
    (10, 7, 5, 3072, "bf16", "abs"), (7, 3, 11, 264, "bf16", "rel"), (1, 4, 4, 64, "bf16", "abs"),
])
def test_lif_mask_matches_oracle(frames, height, width, dim, dtype, kind):
    t = tsa()
    cfg = _lif_cfg(frames, height, width, dim, 2 if dim % 256 else dim // 128, dtype)
    x = generate.lipar_inputs(cfg, 0)["x"]
    x64 = G.host64(x)
    rel = kind == "rel"
    tau_s, tau_l = cfg.tau_short, cfg.tau_long
    if rel:  # relative changes: thresholds on the relative scale of this clip
        s = ref.token_scores(x64, None, cfg.hw, relative=True)
        tau_s = 4.0 * float(np.median(s[cfg.hw:]))
        tau_l = 2.5 * float(np.min(s[cfg.hw:]))
    want = ref.lif_mask(x64, frames, cfg.hw, tau_s, tau_l, relative=rel)
    # the inputs keep every score clear of the thresholds, so both sides must agree exactly
    assert _margin(want, tau_s, tau_l) > 1e-4
    mask = torch.empty(cfg.n, dtype=torch.uint8, device="cuda")
    so = torch.empty(cfg.n, dtype=torch.float32, device="cuda")
    lo = torch.empty(cfg.n, dtype=torch.float32, device="cuda")
    t.lif_mask(G.dev(x), frames, cfg.hw, tau_s, tau_l, mask, short_out=so, long_out=lo,
               score_kind=t.SCORE_REL_L1 if rel else t.SCORE_ABS_L1)
    gm = mask.cpu().numpy().astype(bool)
    assert np.array_equal(gm, want["mask"])
    kept = gm.reshape(frames, -1)
    print(f"  kept {gm.sum()} of {gm.size}; refresh of static locations seen: "
          f"{bool(kept[1:].any())}", flush=True)
    # fp32 sums of `dim` non-negative terms: relative error below dim * 2^-24
    rtol = (dim + 2) * 2.0 ** -24
    for name, g_, w_ in (("short", so, want["short"]), ("long", lo, want["long"])):
        g = g_.cpu().numpy().astype(np.float64)
        fin = np.isfinite(w_)
        assert np.array_equal(np.isfinite(g), fin), name
        assert np.all(np.abs(g[fin] - w_[fin]) <= rtol * np.abs(w_[fin]) + 1e-30), name


# ----------------------------------------------------------- restoration

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("frames,hw,dim", [(6, 7, 64), (33, 90, 3072), (2, 1, 8), (1, 5, 16)])
def test_restore_matches_oracle(dtype, frames, hw, dim):
    t = tsa()
    g = torch.Generator().manual_seed(frames * hw + dim)
    buf = torch.randn(frames * hw, dim, generator=g).to(dtype)
    mask = (torch.rand(frames * hw, generator=g) < 0.4).to(torch.uint8)
    mask[: hw // 2] = 1  # part of frame 0 kept, part pruned (left as it is)
    bd = G.dev(buf)
    t.restore_frames(bd, G.dev(mask), frames, hw)
    want = ref.restore_frames(G.host64(buf), mask.numpy().astype(bool), frames, hw)
    assert np.array_equal(G.host64(bd), want)


# ------------------------------------------------------ sampling loop

def test_hsa_loop_scaled():
    t = tsa()
    cfg = scaled(configs.get_config("hsa_loop"), frames=2, height=12, width=26, dim=512, heads=4)
    inp = generate.hsa_inputs(cfg, 0)
    x0, x1, w = inp["xs"][0], inp["xs"][1], inp["w_qkv"]
    counts, gper = cfg.group_counts(), cfg.group_periods()
    sig = cfg.sigmas()
    print(f"  case {cfg.name} N={cfg.n} D={cfg.dim} T={cfg.steps} window={cfg.window}", flush=True)
    layer = t.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, G.dev(w))
    # groups ranked once from the change between two latents (as the HSA schedule test does)
    layer.select(G.dev(x1), G.dev(x0), k=1)
    period = torch.empty(cfg.n, dtype=torch.uint8, device="cuda")
    t.assign_groups(layer.scores, counts, gper, period, layer.workspace)
    x64, w64 = G.host64(x0), G.host64(w)
    per = ref.assign_periods(ref.token_scores(G.host64(x1), x64), counts, gper)
    assert np.array_equal(period.cpu().numpy(), per)
    hist = ref.hsa_run(x64, w64, cfg.heads, per, sig, cfg.window)

    x = G.dev(x0.float())
    seen = []

    def check(i):
        torch.cuda.synchronize()
        h = hist[i]
        dense = ref.step_is_dense(i, cfg.steps, cfg.window)
        if not dense:
            n_act = t.hsa_active_count(counts, gper, i)
            assert np.array_equal(layer.idx.cpu().numpy()[:n_act], h["idx"]), i
        G.assert_close(G.host64(layer.out), h["v_hat"], f"step {i} v_hat")
        G.assert_close(G.host64(x) - x64, h["x"] - x64, f"step {i} displacement")
        seen.append(i)

    layer.hsa_run(x, period, sig, cfg.window, counts, gper, on_step=check)
    assert seen == list(range(cfg.steps))


# ------------------------------------------- inter-frame pass with restoration

def test_lipar_lif_pass_scaled():
    t = tsa()
    cfg = _lif_cfg(6, 6, 10, 256, 2)
    inp = generate.lipar_inputs(cfg, 0)
    x, w = inp["x"], inp["w_qkv"]
    eps = generate.lipar_eps(cfg, 0, 0)
    x64, w64, e64 = G.host64(x), G.host64(w), G.host64(eps)
    lm = ref.lif_mask(x64, cfg.frames, cfg.hw, cfg.tau_short, cfg.tau_long)
    assert _margin(lm, cfg.tau_short, cfg.tau_long) > 1e-4
    mask = lm["mask"]
    k = int(mask.sum())
    print(f"  case {cfg.name} N={cfg.n} D={cfg.dim} kept={k}", flush=True)
    layer = t.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, G.dev(w))
    got_k = layer.step_lipar_lif(G.dev(x), G.dev(eps), cfg.frames, cfg.hw, cfg.tau_short,
                                 cfg.tau_long, cfg.sigma)
    torch.cuda.synchronize()
    assert got_k == k
    kc = np.zeros((cfg.n, cfg.dim))
    vc = np.zeros((cfg.n, cfg.dim))
    out = np.zeros((cfg.n, cfg.dim))
    res = ref.lipar_step(x64, e64, w64, cfg.heads, cfg.hw, k, cfg.sigma, kc, vc, out, mask=mask)
    restored = ref.restore_frames(out, mask, cfg.frames, cfg.hw)
    assert np.array_equal(layer.idx.cpu().numpy()[:k], res["idx"])
    assert np.array_equal(layer.pidx.cpu().numpy()[:cfg.n - k], res["pidx"])
    G.assert_close(G.host64(layer.k_cache), kc, "K cache", mabs=np.inf)
    G.assert_close(G.host64(layer.out), restored, "restored output")
    # restored rows repeat the previous frame's row of the GPU output exactly
    o = G.host64(layer.out).reshape(cfg.frames, cfg.hw, -1)
    m = mask.reshape(cfg.frames, cfg.hw)
    for f in range(1, cfg.frames):
        assert np.array_equal(o[f][~m[f]], o[f - 1][~m[f]])


def _mask_flips_near_threshold(gm, want, cfg):
    """Locations whose GPU mask (frames x hw) differs from the oracle's; the first frame that
    differs at each must have a change score within 1e-5 (relative) of its threshold (later
    frames follow from it through the long-term reference).  Returns their number."""
    wm = want["mask"].reshape(cfg.frames, cfg.hw)
    ws = want["short"].reshape(cfg.frames, cfg.hw)
    wl = want["long"].reshape(cfg.frames, cfg.hw)
    gm = gm.reshape(cfg.frames, cfg.hw)
    flips = 0
    for loc in np.flatnonzero((gm != wm).any(axis=0)):
        f = int(np.argmax(gm[:, loc] != wm[:, loc]))
        near = min(abs(ws[f, loc] - cfg.tau_short) / cfg.tau_short,
                   abs(wl[f, loc] - cfg.tau_long) / cfg.tau_long)
        assert near <= G.NEAR_THRESHOLD, (loc, f, ws[f, loc], wl[f, loc])
        flips += 1
    return flips


@pytest.mark.slow
def test_lipar_lif_pass_full_size():
    """The long/short-term pass on the whole 33x45x80 clip (N = 118800, D = 3072, 24 heads):
    mask, active and pruned lists bit for bit; the whole K/V cache (active rows projected from
    their latent, pruned rows from their recovered rows) within the layer tolerance; 48 sampled
    kept output rows and 48 sampled restored rows (each the output of the last kept frame at its
    location) against the oracle, and each restored row bit-identical to its source row.
    Where the masks differ (change scores within 1e-5 of a threshold) the pass after the mask
    is rerun on the GPU with the oracle's mask."""
    t = tsa()
    cfg = configs.get_config("lipar_lif")
    inp = generate.lipar_inputs(cfg, 0)
    x, w = inp["x"], inp["w_qkv"]
    eps = generate.lipar_eps(cfg, 0, 0)
    print(f"  case {cfg.name} N={cfg.n} D={cfg.dim} heads={cfg.heads} frames={cfg.frames}", flush=True)
    layer = t.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, G.dev(w))
    xd, ed = G.dev(x), G.dev(eps)
    got_k = layer.step_lipar_lif(xd, ed, cfg.frames, cfg.hw, cfg.tau_short, cfg.tau_long, cfg.sigma)
    torch.cuda.synchronize()
    x64, w64, e64 = G.host64(x), G.host64(w), G.host64(eps)
    lm = ref.lif_mask(x64, cfg.frames, cfg.hw, cfg.tau_short, cfg.tau_long)
    mask = lm["mask"]
    k = int(mask.sum())
    flips = _mask_flips_near_threshold(layer._lif_mask.cpu().numpy().astype(bool), lm, cfg)
    print(f"  kept {k} of {cfg.n}; GPU kept {got_k}; near-threshold locations: {flips}", flush=True)
    if flips:
        md = G.dev(torch.from_numpy(mask.astype(np.uint8)))
        for buf in (layer.k_cache, layer.v_cache, layer.out):
            buf.zero_()
        layer.select(None, mask=md)
        layer._lipar_forward(xd, ed, cfg.hw, k, cfg.sigma, None)
        t.restore_frames(layer.out, md, cfg.frames, cfg.hw)
        torch.cuda.synchronize()
    else:
        assert got_k == k
    idx, pidx = np.flatnonzero(mask), np.flatnonzero(~mask)
    rng = np.random.default_rng(5)
    kept_s = np.sort(rng.choice(idx, 48, replace=False))
    pruned_s = np.sort(rng.choice(pidx[pidx >= cfg.hw], 48, replace=False))
    m2 = mask.reshape(cfg.frames, cfg.hw)

    def source(tok):  # the last kept frame at the token's location (frame 0 is always kept)
        f, loc = divmod(int(tok), cfg.hw)
        while not m2[f, loc]:
            f -= 1
        return f * cfg.hw + loc

    src_s = np.array([source(p) for p in pruned_s])
    need = np.unique(np.concatenate([kept_s, src_s]))
    kc = np.zeros((cfg.n, cfg.dim))
    vc = np.zeros((cfg.n, cfg.dim))
    out = np.zeros((cfg.n, cfg.dim))
    print(f"  oracle: projections of all {cfg.n} rows, attention of {need.size} queries", flush=True)
    res = ref.lipar_step(x64, e64, w64, cfg.heads, cfg.hw, k, cfg.sigma, kc, vc, out,
                         query_rows=np.searchsorted(idx, need), mask=mask)
    out[need] = res["o_a"]
    restored = ref.restore_frames(out, mask, cfg.frames, cfg.hw)
    assert np.array_equal(layer.idx.cpu().numpy()[:k], res["idx"])
    assert np.array_equal(layer.pidx.cpu().numpy()[:cfg.n - k], res["pidx"])
    gk, gv = G.host64(layer.k_cache), G.host64(layer.v_cache)
    G.assert_close(gk[idx], kc[idx], "K cache (active rows)", mabs=np.inf)
    G.assert_close(gv[idx], vc[idx], "V cache (active rows)", mabs=np.inf)
    for name, a, b in (("K", gk[pidx], kc[pidx]), ("V", gv[pidx], vc[pidx])):
        rf = G.rel_frob(a, b)
        rel_abs = float(np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b))))
        print(f"  {name} cache (recovered rows): rel_frob={rf:.3e} scaled max_abs={rel_abs:.3e}", flush=True)
        assert rf <= G.REL_FROB and rel_abs <= G.MAX_ABS
    del gk, gv
    go = G.host64(layer.out)
    G.assert_close(go[kept_s], restored[kept_s], "kept output rows")
    G.assert_close(go[pruned_s], restored[pruned_s], "restored output rows")
    assert np.array_equal(go[pruned_s], go[src_s])


@pytest.mark.slow
def test_lif_mask_full_size():
    """The 33x45x80 clip at D=3072: masks compared location by location up to the first
    disagreement, which must be a change score within 1e-5 (relative) of its threshold."""
    t = tsa()
    cfg = configs.get_config("lipar_lif")
    x = generate.lipar_inputs(cfg, 0)["x"]
    print(f"  case {cfg.name} N={cfg.n} D={cfg.dim}", flush=True)
    mask = torch.empty(cfg.n, dtype=torch.uint8, device="cuda")
    so = torch.empty(cfg.n, dtype=torch.float32, device="cuda")
    lo = torch.empty(cfg.n, dtype=torch.float32, device="cuda")
    t.lif_mask(G.dev(x), cfg.frames, cfg.hw, cfg.tau_short, cfg.tau_long, mask, short_out=so, long_out=lo)
    torch.cuda.synchronize()
    want = ref.lif_mask(G.host64(x), cfg.frames, cfg.hw, cfg.tau_short, cfg.tau_long)
    gm = mask.cpu().numpy().astype(bool).reshape(cfg.frames, cfg.hw)
    wm = want["mask"].reshape(cfg.frames, cfg.hw)
    ws = want["short"].reshape(cfg.frames, cfg.hw)
    wl = want["long"].reshape(cfg.frames, cfg.hw)
    gl = lo.cpu().numpy().astype(np.float64).reshape(cfg.frames, cfg.hw)
    flips = _mask_flips_near_threshold(gm, want, cfg)
    print(f"  kept {wm.sum()} of {wm.size}; near-threshold locations: {flips}", flush=True)
    same = ~(gm != wm).cumsum(axis=0).astype(bool)  # frames before the first disagreement
    fin = np.isfinite(wl) & same
    rtol = (cfg.dim + 2) * 2.0 ** -24
    assert np.all(np.abs(gl[fin] - wl[fin]) <= rtol * wl[fin])
