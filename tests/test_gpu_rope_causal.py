"""GPU parity of the rotary-position and frame-causal variants (3D RoPE of Q/K fused into
the QKV projection; block-causal attention per frame) against the CPU oracle."""

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


def _pairsum(a):
    """Each channel pair's two entries replaced by their sum (the pair a rotation mixes)."""
    s = a[:, 0::2] + a[:, 1::2]
    return np.repeat(s, 2, axis=1)


def _assert_rotated_close(got, want, exact, abs_dot, k_terms, what):
    """Rotated projections: the fp32 accumulation error of both channels of a pair, the fp32
    rotation (angle and sine/cosine error below 1e-5 of the pair's size), and the two bf16
    roundings."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    bound = (0.5 * (G.bf16_ulp_of(got) + G.bf16_ulp_of(want)) + k_terms * 2.0 ** -24 * _pairsum(abs_dot)
             + 1e-5 * _pairsum(np.abs(exact)))
    err = np.abs(got - want)
    print(f"  {what}: rel_frob={G.rel_frob(got, want):.3e}, max err/bound {float(np.max(err / bound)):.3f}",
          flush=True)
    assert G.rel_frob(got, want) <= G.REL_FROB and np.all(err <= bound), what


@pytest.mark.parametrize("n_x,n,dim,heads,hw,gather,xdt", [
    (240, 97, 256, 2, (6, 10), True, torch.bfloat16),
    (1000, 333, 512, 4, (10, 25), True, torch.bfloat16),
    (300, 300, 128, 2, (5, 6), False, torch.bfloat16),
    (260, 130, 768, 12, (4, 13), True, torch.float32),
])
def test_qkv_rope_matches_oracle(n_x, n, dim, heads, hw, gather, xdt):
    t = tsa()
    g = torch.Generator().manual_seed(n_x + dim)
    x = torch.randn(n_x, dim, generator=g).to(xdt)
    w = (torch.randn(3 * dim, dim, generator=g) / dim ** 0.5).to(torch.bfloat16)
    rows = np.sort(np.random.default_rng(n).choice(n_x, n, replace=False)).astype(np.int32) if gather else None
    toks = rows if gather else np.arange(n)
    q = torch.empty(n, dim, dtype=torch.bfloat16, device="cuda")
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    h, wd = hw
    t.qkv_active_rope(G.dev(x), G.dev(torch.from_numpy(rows)) if gather else None, n, G.dev(w), heads, h, wd,
                      q_out=q, k_out=k, v_out=v)
    x64 = G.host64(x)[toks]
    w64 = G.host64(w)
    want = ref.project_rope(x64, toks, w64, heads, h, wd)
    xb = ref.round_bf16(x64)
    ax = np.abs(xb)
    for name, part, got in (("q", 0, q), ("k", 1, k)):
        wp = w64[part * dim:(part + 1) * dim]
        exact = ref.rope3d(xb @ wp.T, toks, h, wd, heads)
        _assert_rotated_close(G.host64(got), want[name], exact, ax @ np.abs(wp).T, dim, f"rotated {name}")
    G.assert_projection_close(G.host64(v), want["v"], ax @ np.abs(w64[2 * dim:]).T, dim, "v (not rotated)")


def test_qkv_rope_cache_rows_and_identity():
    """K/V written to cache rows; a grid of one token per frame rotates by the frame index only."""
    t = tsa()
    g = torch.Generator().manual_seed(5)
    n_x, dim, heads = 64, 256, 2
    x = torch.randn(n_x, dim, generator=g).to(torch.bfloat16)
    w = (torch.randn(3 * dim, dim, generator=g) / dim ** 0.5).to(torch.bfloat16)
    rows = np.array([0, 5, 17, 40, 63], dtype=np.int32)
    kc = torch.zeros(n_x, dim, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    q = torch.empty(rows.size, dim, dtype=torch.bfloat16, device="cuda")
    t.qkv_active_rope(G.dev(x), G.dev(torch.from_numpy(rows)), rows.size, G.dev(w), heads, 1, 1, q_out=q,
                      k_out=kc, v_out=vc, out_is_cache=True, n_cache=n_x)
    want = ref.project_rope(G.host64(x)[rows], rows, G.host64(w), heads, 1, 1)
    others = np.setdiff1d(np.arange(n_x), rows)
    kh = G.host64(kc)
    assert np.all(kh[others] == 0)
    G.assert_close(kh[rows], want["k"], "cache rows of rotated K", mabs=np.inf)
    # token 0 sits at the origin: its rotated Q equals the plain projection bit for bit
    plain = torch.empty_like(q)
    t.qkv_active(G.dev(x), G.dev(torch.from_numpy(rows)), rows.size, G.dev(w), q_out=plain,
                 k_out=torch.empty_like(q), v_out=torch.empty_like(q))
    assert torch.equal(q[0], plain[0])


@pytest.mark.parametrize("n_q,n_kv,heads,hd,ft,order", [
    (300, 1000, 2, 128, 100, "sorted"), (777, 2085, 4, 64, 139, "sorted"), (129, 5000, 1, 128, 1000, "sorted"),
    (50, 200, 2, 64, 1, "sorted"), (400, 1200, 3, 128, 240, "shuffled"), (1000, 1000, 2, 128, 1000, "sorted"),
])
def test_frame_causal_attention_matches_oracle(n_q, n_kv, heads, hd, ft, order):
    t = tsa()
    g = torch.Generator().manual_seed(n_q + n_kv + ft)
    dim = heads * hd
    rng = np.random.default_rng(n_q)
    toks = np.sort(rng.choice(n_kv, n_q, replace=False)).astype(np.int32)
    if order == "shuffled":
        toks = rng.permutation(toks).astype(np.int32)
    q = torch.randn(n_q, dim, generator=g).to(torch.bfloat16)
    k = torch.randn(n_kv, dim, generator=g).to(torch.bfloat16)
    v = torch.randn(n_kv, dim, generator=g).to(torch.bfloat16)
    out = torch.empty(n_q, dim, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(heads, n_q, dtype=torch.float32, device="cuda")
    t.frame_causal_attention(G.dev(q), G.dev(k), G.dev(v), n_q, heads, hd, G.dev(torch.from_numpy(toks)), ft, out,
                             lse_out=lse)
    want, want_lse = ref.attention_frame_causal(G.host64(q), G.host64(k), G.host64(v), heads, toks, ft,
                                                return_lse=True)
    G.assert_close(G.host64(out), want, f"frame-causal {n_q}x{n_kv} h{heads} d{hd} ft{ft} {order}")
    assert np.max(np.abs(G.host64(lse) - want_lse)) <= 1e-3 * max(1.0, np.abs(want_lse).max())


def _rope_causal_case(cfg, seed=0, sample=None):
    t = tsa()
    hw = cfg.height * cfg.width
    rope = (cfg.height, cfg.width, 10000.0)
    print(f"  case {cfg.name} N={cfg.n} D={cfg.dim} H={cfg.heads} k={cfg.n_active} rope+causal", flush=True)
    inp = generate.step_inputs(cfg, seed)
    x_prev, x_cur, w = inp["x_prev"], inp["x_cur"], inp["w_qkv"]
    layer = t.PrunedAttentionLayer(cfg.n, cfg.dim, cfg.heads, G.dev(w), rope=rope, causal_frame_tokens=hw)
    layer.init_cache(G.dev(x_prev))
    layer.step_topk(G.dev(x_cur), G.dev(x_prev), cfg.n_active)
    torch.cuda.synchronize()
    xp64, xc64, w64 = G.host64(x_prev), G.host64(x_cur), G.host64(w)
    all_toks = np.arange(cfg.n)
    init = ref.project_rope(xp64, all_toks, w64, cfg.heads, *rope, parts="kv")
    kc, vc = init["k"], init["v"]
    mask = ref.select_topk(ref.token_scores(xc64, xp64), cfg.n_active)
    idx, _ = ref.compact(mask)
    assert np.array_equal(layer.idx.cpu().numpy()[:idx.size], idx)
    p = ref.project_rope(xc64[idx], idx, w64, cfg.heads, *rope, parts="kv")
    ref.kv_cache_sync(kc, vc, idx, p["k"], p["v"])
    G.assert_close(G.host64(layer.k_cache), kc, "rotated K cache", mabs=np.inf)
    rows = np.arange(idx.size) if sample is None else np.sort(np.random.default_rng(seed).choice(idx.size, sample, replace=False))
    q = ref.project_rope(xc64[idx[rows]], idx[rows], w64, cfg.heads, *rope, parts="q")["q"]
    o = ref.attention_frame_causal(q, kc, vc, cfg.heads, idx[rows], hw)
    G.assert_close(G.host64(layer.out)[idx[rows]], o, "output rows (rope + frame-causal)")


def test_rope_causal_layer_scaled():
    _rope_causal_case(scaled(configs.get_config("wan13b"), frames=3, height=10, width=26, dim=512, heads=4))


def test_rope_causal_layer_head_dim_64():
    _rope_causal_case(scaled(configs.get_config("wan13b"), frames=4, height=6, width=20, dim=256, heads=4))


@pytest.mark.slow
def test_rope_causal_wan13b_full_size_sampled():
    _rope_causal_case(configs.get_config("wan13b"), sample=96)
