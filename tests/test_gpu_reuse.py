"""GPU parity of the Timeripple partial-score reuse (similarity checks, sources, effective
rows) and of attention over the effective Q/K, against the CPU oracle."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import gpu_util as G
from oracle import reference as ref

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    G.need_gpu()


def tsa():
    import token_sparse_attention_rel_amd as t
    return t


def _clip_rows(frames, height, width, heads, hd, seed, static_frac=0.75, drift=0.01, moving=0.5):
    """Rotary Q- or K-like rows of a clip: per location a content row that drifts slowly
    (static locations) or fast (moving ones) from frame to frame, rotated by each token's
    3D position, rounded to bf16."""
    r = np.random.default_rng(seed)
    hw = height * width
    dim = heads * hd
    static = r.random(hw) < static_frac
    scale = np.where(static, drift, moving)[:, None]
    rows = [r.standard_normal((hw, dim))]
    for _ in range(1, frames):
        rows.append(rows[-1] + scale * r.standard_normal((hw, dim)))
    content = np.concatenate(rows, axis=0)
    n = frames * hw
    return ref.round_bf16(ref.rope3d(content, np.arange(n), height, width, heads))


def _run(v64, heads, hd, height, width, thetas):
    t = tsa()
    n = v64.shape[0]
    v = G.dev(torch.from_numpy(v64), torch.bfloat16)
    eff = torch.empty_like(v)
    src = torch.empty(n, heads, 3, dtype=torch.int32, device="cuda")
    delta = torch.empty(n, heads, 3, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, t.reuse_workspace_bytes(n, heads)), dtype=torch.uint8, device="cuda")
    t.timeripple_reuse(v, heads, hd, height, width, thetas, eff, ws, src_out=src, delta_out=delta)
    torch.cuda.synchronize()
    return eff, src.cpu().numpy().astype(np.int64), delta.cpu().numpy().astype(np.float64)


def _check_against_oracle(v64, heads, hd, height, width, thetas, what):
    eff, src, delta = _run(v64, heads, hd, height, width, thetas)
    want_delta = ref.reuse_deltas(v64, heads, height, width)
    # fp32 sums of squares vs fp64: relative agreement, the same infinities
    fin = np.isfinite(want_delta)
    assert np.array_equal(np.isfinite(delta), fin), what
    err = np.abs(delta[fin] - want_delta[fin]) / np.maximum(want_delta[fin], 1e-30)
    print(f"  {what}: delta max rel err {float(err.max()) if err.size else 0.0:.2e}", flush=True)
    assert err.size == 0 or err.max() <= 1e-5, what
    # the decisions, taken on the kernel's fp32 deltas against fp32 thresholds, agree exactly
    th32 = [float(np.float32(x)) for x in thetas]
    want_src = ref.reuse_sources(delta, th32, height, width)
    assert np.array_equal(src, want_src), what
    # and against the oracle's own fp64 deltas, except where a delta lies within 1e-5 of its threshold
    own = ref.reuse_sources(want_delta, th32, height, width)
    near = np.zeros(src.shape[:2], dtype=bool)
    for a in range(3):
        if np.isfinite(th32[a]):
            near |= np.abs(want_delta[:, :, a] - th32[a]) <= 1e-5 * max(th32[a], 1e-30)
    differ = (own != src).any(axis=2)
    assert not (differ & ~near).any(), what
    # effective rows: copies of the resolved sources' channels, bit for bit
    want_eff = ref.reuse_effective(v64, src, heads)
    assert np.array_equal(G.host64(eff), want_eff), what
    return src


@pytest.mark.parametrize("frames,height,width,heads,hd,thetas", [
    (4, 5, 6, 2, 128, (0.05, 0.05, 0.05)),
    (3, 7, 9, 3, 64, (0.05, 0.3, 0.3)),
    (5, 1, 8, 2, 128, (0.1, 1.0, 1.5)),
    (6, 4, 1, 1, 64, (0.02, 1.5, 0.0)),
    (3, 6, 7, 2, 128, (np.inf, 0.0, 0.0)),
])
def test_reuse_matches_oracle(frames, height, width, heads, hd, thetas):
    v64 = _clip_rows(frames, height, width, heads, hd, seed=frames * 100 + width)
    src = _check_against_oracle(v64, heads, hd, height, width, thetas, f"{frames}x{height}x{width} d{hd} {thetas}")
    reused = (src != np.arange(v64.shape[0])[:, None, None]).mean()
    print(f"  reused (token, head, group) entries: {reused:.3f}", flush=True)


def test_reuse_edge_cases():
    frames, height, width, heads, hd = 3, 4, 5, 2, 128
    n = frames * height * width
    v64 = _clip_rows(frames, height, width, heads, hd, seed=7)
    ident = np.arange(n)[:, None, None]
    # thresholds 0: nothing reused, the rows are copied unchanged
    eff, src, _ = _run(v64, heads, hd, height, width, (0.0, 0.0, 0.0))
    assert np.array_equal(src, np.broadcast_to(ident, src.shape))
    assert np.array_equal(G.host64(eff), v64)
    # every check passing: closed-form chain roots (frame start, row start of frame 0, column of frame 0)
    eff, src, _ = _run(v64, heads, hd, height, width, (np.inf,) * 3)
    e = G.host64(eff)
    groups = ref.reuse_groups(hd)
    hw = height * width
    for t in range(n):
        f, y, x = t // hw, (t // width) % height, t % width
        roots = (f * hw, y * width, x)
        for h in range(heads):
            for g, (s, end) in enumerate(groups):
                assert np.array_equal(e[t, h * hd + s:h * hd + end], v64[roots[g], h * hd + s:h * hd + end])
    # rotary rows of one content row: exact zero differences, reuse everywhere, rows unchanged
    u = np.repeat(np.random.default_rng(3).standard_normal((1, heads * hd)), n, axis=0)
    rv = ref.round_bf16(ref.rope3d(u, np.arange(n), height, width, heads))
    _check_against_oracle(rv, heads, hd, height, width, (1e-6, 1e-6, 1e-6), "rotary constant rows")
    # one token: no neighbours
    eff, src, delta = _run(v64[:1], heads, hd, 1, 1, (1.0, 1.0, 1.0))
    assert (src == 0).all() and np.isinf(delta).all() and np.array_equal(G.host64(eff), v64[:1])


def test_timeripple_attention_matches_oracle():
    t = tsa()
    frames, height, width, heads, hd = 4, 6, 8, 2, 128
    n = frames * height * width
    q64 = _clip_rows(frames, height, width, heads, hd, seed=11)
    k64 = _clip_rows(frames, height, width, heads, hd, seed=12)
    v64 = ref.round_bf16(np.random.default_rng(13).standard_normal((n, heads * hd)))
    th_q, th_k = (0.05, 0.05, 0.05), (0.08, 0.04, 0.04)
    q_eff, src_q, _ = _run(q64, heads, hd, height, width, th_q)
    k_eff, src_k, _ = _run(k64, heads, hd, height, width, th_k)
    out = torch.empty(n, heads * hd, dtype=torch.bfloat16, device="cuda")
    t.sparse_query_attention(q_eff, k_eff, G.dev(torch.from_numpy(v64), torch.bfloat16), n, heads, hd, out)
    torch.cuda.synchronize()
    # the oracle's attention over the effective rows resolved from the kernel's decisions
    want = ref.attention(ref.reuse_effective(q64, src_q, heads), ref.reuse_effective(k64, src_k, heads), v64, heads)
    G.assert_close(G.host64(out), want, "attention of the effective Q/K")
    full = ref.timeripple_attention(q64, k64, v64, heads, height, width, th_q, th_k)
    same = np.array_equal(full["src_q"], src_q) and np.array_equal(full["src_k"], src_k)
    print(f"  kernel decisions equal the oracle's own: {same}", flush=True)
    assert (src_q != np.arange(n)[:, None, None]).any() and (src_k != np.arange(n)[:, None, None]).any()


@pytest.mark.slow
def test_reuse_full_size_wan_grid():
    """21 x 30 x 52 tokens, 12 heads of 128 (the headline grid): all deltas and decisions,
    effective rows of sampled (token, head) pairs by following the kernel's sources."""
    frames, height, width, heads, hd = 21, 30, 52, 12, 128
    n = frames * height * width
    v64 = _clip_rows(frames, height, width, heads, hd, seed=21)
    thetas = (0.05, 0.05, 0.05)
    eff, src, delta = _run(v64, heads, hd, height, width, thetas)
    want_delta = ref.reuse_deltas(v64, heads, height, width)
    fin = np.isfinite(want_delta)
    assert np.array_equal(np.isfinite(delta), fin)
    assert (np.abs(delta[fin] - want_delta[fin]) / np.maximum(want_delta[fin], 1e-30)).max() <= 1e-5
    assert np.array_equal(src, ref.reuse_sources(delta, [float(np.float32(x)) for x in thetas], height, width))
    e = G.host64(eff)
    groups = ref.reuse_groups(hd)
    rng = np.random.default_rng(0)
    for t in rng.choice(n, 400, replace=False):
        for h in range(heads):
            for g, (s, end) in enumerate(groups):
                r = int(t)
                while src[r, h, g] != r:
                    r = int(src[r, h, g])
                assert np.array_equal(e[t, h * hd + s:h * hd + end], v64[r, h * hd + s:h * hd + end])
    reused = (src != np.arange(n)[:, None, None]).mean()
    print(f"  reused (token, head, group) entries: {reused:.3f}", flush=True)
    assert 0.3 < reused < 0.8


def test_layer_reuse_forward_scaled():
    """The layer's dense pass with reuse: rotated QKV of every token, reuse on Q and K,
    attention of the effective vectors, outputs in token order."""
    from workloads import configs, generate
    from workloads.configs import scaled

    t = tsa()
    cfg = scaled(configs.get_config("timeripple"), frames=4, height=6, width=10, dim=256, heads=2)
    inp = generate.lipar_inputs(cfg, 0)
    x, w = inp["x"], inp["w_qkv"]
    rope = (cfg.height, cfg.width, 10000.0)
    layer = t.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, G.dev(w), rope=rope)
    th_q, th_k = (0.05, 0.05, 0.05), (0.05, 0.05, 0.05)
    layer.reuse_forward(G.dev(x), th_q, th_k)
    torch.cuda.synchronize()
    toks = np.arange(cfg.n)
    p = ref.project_rope(G.host64(x), toks, G.host64(w), cfg.heads, *rope)
    src_q = layer.src_q.cpu().numpy().astype(np.int64)
    src_k = layer.src_k.cpu().numpy().astype(np.int64)
    assert (src_q != toks[:, None, None]).mean() > 0.2
    # the oracle's own decisions on its Q/K agree away from the thresholds
    own_q = ref.reuse_sources(ref.reuse_deltas(p["q"], cfg.heads, cfg.height, cfg.width), th_q, cfg.height, cfg.width)
    print(f"  Q sources equal to the oracle's own: {(own_q == src_q).mean():.4f}", flush=True)
    assert (own_q == src_q).mean() > 0.99
    want = ref.attention(ref.reuse_effective(p["q"], src_q, cfg.heads), ref.reuse_effective(p["k"], src_k, cfg.heads),
                         p["v"], cfg.heads)
    G.assert_close(G.host64(layer.out), want, "layer pass with reuse")
