"""Seeded random shapes and argument mixes through the C ABI against the CPU oracle: each case
draws its sizes, dtypes and options (ragged tails, scatter rows, workspaces, recovery rows,
rotary positions, frame-causal limits, selection modes) from its seed, so the combinations that
the hand-picked cases of the other files leave out are covered too.  Same tolerances as there."""

from __future__ import annotations

import math

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


def _bf16(g, *shape, scale=1.0):
    return (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16)


def _sorted_rows(rng, n_from, n):
    return np.sort(rng.choice(n_from, n, replace=False)).astype(np.int32)


@pytest.mark.parametrize("seed", range(24))
def test_attention_fuzz(seed):
    """Random n_q, n_kv, heads, head_dim, query scale; compact or scattered outputs; with or
    without the split workspace; bidirectional or frame-causal; default or explicit scale."""
    t = tsa()
    rng = np.random.default_rng(1000 + seed)
    g = torch.Generator().manual_seed(1000 + seed)
    hd = int(rng.choice([64, 128]))
    heads = int(rng.integers(1, 7))
    n_q = int(rng.integers(1, 900))
    n_kv = int(rng.integers(1, 5000))
    dim = heads * hd
    qs = float(rng.choice([0.5, 1.0, 3.0]))
    scale = float(rng.choice([0.0, 0.05, 0.2]))
    causal = rng.random() < 0.3
    scatter = rng.random() < 0.5
    q = _bf16(g, n_q, dim, scale=qs)
    k = _bf16(g, n_kv, dim)
    v = _bf16(g, n_kv, dim)
    n_out = n_q + int(rng.integers(0, 400)) if scatter else n_q
    rows = _sorted_rows(rng, n_out, n_q) if scatter else None
    out = _bf16(g, n_out, dim)
    before = out.clone()
    od = G.dev(out)
    kw = dict(out_rows=G.dev(torch.from_numpy(rows)) if scatter else None, scale=scale)
    sc = scale if scale > 0 else None
    print(f"  seed {seed}: n_q={n_q} n_kv={n_kv} heads={heads} hd={hd} causal={causal} scatter={scatter} "
          f"scale={scale} q_scale={qs}", flush=True)
    q64, k64, v64 = G.host64(q), G.host64(k), G.host64(v)
    if causal:
        frame = int(rng.integers(1, n_kv + 1))
        q_tokens = np.sort(rng.integers(0, n_kv + frame, n_q)).astype(np.int32)
        t.frame_causal_attention(G.dev(q), G.dev(k), G.dev(v), n_q, heads, hd,
                                 G.dev(torch.from_numpy(q_tokens)), frame, od, **kw)
        want = ref.attention_frame_causal(q64, k64, v64, heads, q_tokens, frame, scale=sc)
    else:
        ws_bytes = t.attention_workspace_bytes(n_q, n_kv, heads, hd)
        ws = None
        if ws_bytes and rng.random() < 0.5:
            ws = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device="cuda")
        t.sparse_query_attention(G.dev(q), G.dev(k), G.dev(v), n_q, heads, hd, od, workspace=ws, **kw)
        want = ref.attention(q64, k64, v64, heads, scale=sc)
    torch.cuda.synchronize()
    got = G.host64(od)
    if scatter:
        G.assert_close(got[rows], want, f"fuzz attention {seed}")
        others = np.setdiff1d(np.arange(n_out), rows)
        assert torch.equal(od.cpu()[others], before[others])
    else:
        G.assert_close(got, want, f"fuzz attention {seed}")


def _rope_heads(rng, dim):
    """A head count whose head size is even and at least 6, or 0 (no rotary positions)."""
    ok = [h for h in range(1, dim // 6 + 1) if dim % h == 0 and (dim // h) % 2 == 0 and dim // h >= 6]
    return int(rng.choice(ok)) if ok and rng.random() < 0.4 else 0


@pytest.mark.parametrize("seed", range(24))
def test_qkv_fuzz(seed):
    """Random token counts and widths (multiples of 64), bf16 / fp32 / recovery rows, gathered
    or contiguous rows, compact outputs or cache rows, with or without Q, rotary positions."""
    t = tsa()
    rng = np.random.default_rng(2000 + seed)
    g = torch.Generator().manual_seed(2000 + seed)
    dim = 64 * int(rng.integers(1, 25))
    n_x = int(rng.integers(1, 4000))
    m = int(rng.integers(1, n_x + 1))
    src = str(rng.choice(["bf16", "f32", "recover"]))
    gathered = rng.random() < 0.8 or src == "recover"
    to_cache = gathered and rng.random() < 0.5
    with_q = not to_cache or rng.random() < 0.5
    heads = _rope_heads(rng, dim)
    height = int(rng.integers(1, 40))
    width = int(rng.integers(1, 60))
    print(f"  seed {seed}: n_x={n_x} m={m} dim={dim} src={src} gathered={gathered} cache={to_cache} "
          f"q={with_q} rope_heads={heads} ({height}x{width})", flush=True)
    x = torch.randn(n_x, dim, generator=g)
    if src != "f32":
        x = x.to(torch.bfloat16)
    w = (torch.randn(3 * dim, dim, generator=g) / math.sqrt(dim)).to(torch.bfloat16)
    rows = _sorted_rows(rng, n_x, m) if gathered else np.arange(m, dtype=np.int32)
    rd = G.dev(torch.from_numpy(rows)) if gathered else None
    n_out = n_x if to_cache else m
    qo = torch.empty(m, dim, dtype=torch.bfloat16, device="cuda") if with_q else None
    ko = G.dev(_bf16(g, n_out, dim))
    vo = G.dev(_bf16(g, n_out, dim))
    k_before, v_before = ko.cpu(), vo.cpu()
    kw = dict(q_out=qo, k_out=ko, v_out=vo, out_is_cache=to_cache, n_cache=n_x if to_cache else 0)
    off, sigma = int(rng.integers(0, n_x + 1)), float(rng.uniform(0.1, 0.9))
    if src == "recover":
        eps = _bf16(g, n_x, dim)
        kw.update(eps=G.dev(eps), src_row_offset=off, sigma=sigma)
        a_rows = ref.recover_rows(G.host64(x), G.host64(eps), rows, off, sigma)
    else:
        a_rows = G.host64(x)[rows]
    if heads:
        t.qkv_active_rope(G.dev(x), rd, m, G.dev(w), heads, height, width, **kw)
        want = ref.project_rope(a_rows, rows, G.host64(w), heads, height, width)
    else:
        t.qkv_active(G.dev(x), rd, m, G.dev(w), **kw)
        want = ref.project(a_rows, G.host64(w))
    torch.cuda.synchronize()
    dst = rows if to_cache else np.arange(m)
    outs = [("k", ko), ("v", vo)] + ([("q", qo)] if with_q else [])
    for name, buf in outs:
        got = G.host64(buf)[np.arange(m) if name == "q" else dst]
        if src == "recover" or heads:
            # recovered rows carry their own fp32 rounding; rotations their own fp32 arithmetic
            G.assert_close(got, want[name], f"fuzz qkv {seed} {name}")
        else:
            part = "qkv".index(name)
            wp = np.abs(G.host64(w)[part * dim:(part + 1) * dim])
            G.assert_projection_close(got, want[name], np.abs(ref.round_bf16(a_rows)) @ wp.T, dim,
                                      f"fuzz qkv {seed} {name}")
    if to_cache:
        others = np.setdiff1d(np.arange(n_x), rows)
        assert torch.equal(ko.cpu()[others], k_before[others]) and torch.equal(vo.cpu()[others], v_before[others])


@pytest.mark.parametrize("seed", range(16))
def test_select_fuzz(seed):
    """Random token counts, widths, dtypes, score kinds, inter-frame offsets and selection modes
    (top-k with k from 0 to N, threshold, given mask): the mask, both index lists and the count
    bit for bit, except tokens whose score lies within 1e-5 of the deciding value."""
    t = tsa()
    rng = np.random.default_rng(3000 + seed)
    g = torch.Generator().manual_seed(3000 + seed)
    n = int(rng.integers(1, 70000))
    dim = 8 * int(rng.integers(1, 65))
    dtype = torch.bfloat16 if rng.random() < 0.7 else torch.float32
    rel = rng.random() < 0.6
    mode = str(rng.choice(["topk", "threshold", "mask"]))
    inter = rng.random() < 0.3
    off = int(rng.integers(1, max(2, n // 4))) if inter else 0
    x_ref = torch.randn(n, dim, generator=g)
    step = torch.where(torch.rand(n, generator=g) < 0.7, 0.01, 0.5)
    x_cur = (x_ref + step[:, None] * torch.randn(n, dim, generator=g)).to(dtype)
    x_ref = x_ref.to(dtype)
    print(f"  seed {seed}: n={n} dim={dim} dtype={dtype} rel={rel} mode={mode} offset={off}", flush=True)
    xc = G.dev(x_cur)
    xr = None if inter else G.dev(x_ref)
    scores = ref.token_scores(G.host64(x_cur), None if inter else G.host64(x_ref), off, relative=rel)
    kind = t.SCORE_REL_L1 if rel else t.SCORE_ABS_L1
    mask_d = torch.empty(n, dtype=torch.uint8, device="cuda")
    idx = torch.empty(n, dtype=torch.int32, device="cuda")
    pidx = torch.empty(n, dtype=torch.int32, device="cuda")
    na = torch.empty(1, dtype=torch.int32, device="cuda")
    sd = torch.empty(n, dtype=torch.float32, device="cuda")
    kw = dict(score_kind=kind, scores_out=sd, mask_out=mask_d, idx_out=idx, pidx_out=pidx, n_active_out=na)
    near = None
    if mode == "topk":
        k = int(rng.choice([0, n, int(rng.integers(0, n + 1))]))
        t.select_active(xc, xr, off, t.SELECT_TOPK, k=k, **kw)
        want = ref.select_topk(scores, k)
    elif mode == "threshold":
        fin = scores[np.isfinite(scores)]
        tau = float(np.quantile(fin, rng.uniform(0.05, 0.95))) if fin.size else 1.0
        tau = float(np.float32(tau)) * (1 + 3e-5)  # off any score, as an fp32 value
        t.select_active(xc, xr, off, t.SELECT_THRESHOLD, tau=tau, **kw)
        want = ref.select_threshold(scores, tau)
        near = np.abs(scores - tau) <= G.NEAR_THRESHOLD * abs(tau)
    else:
        m_in = rng.random(n) < rng.uniform(0, 1)
        t.select_active(xc, xr, off, t.SELECT_MASK, aux_in=G.dev(torch.from_numpy(m_in.astype(np.uint8))), **kw)
        want = m_in
    torch.cuda.synchronize()
    gm = mask_d.cpu().numpy().astype(bool)
    if mode == "topk" and 0 < k < n:
        flips = G.mask_mismatch_ok(gm, want, scores, k)
    elif near is not None:
        assert np.all(near[gm != want]), "threshold mask differs away from tau"
        flips = int((gm != want).sum())
    else:
        flips = 0
        assert np.array_equal(gm, want)
    ref_mask = want if flips == 0 else gm  # with flips: the lists must still be those of the mask given back
    i_w, p_w = ref.compact(ref_mask)
    n_act = int(na.item())
    assert n_act == i_w.size
    assert np.array_equal(idx.cpu().numpy()[:n_act], i_w)
    assert np.array_equal(pidx.cpu().numpy()[:n - n_act], p_w)
    if mode != "mask":
        got_s = G.host64(sd)
        fin = np.isfinite(scores)
        assert np.array_equal(np.isfinite(got_s), fin)
        err = np.abs(got_s[fin] - scores[fin]) / np.maximum(np.abs(scores[fin]), 1e-30)
        assert err.size == 0 or err.max() <= G.SCORE_RTOL


@pytest.mark.parametrize("seed", range(12))
def test_row_movers_fuzz(seed):
    """Random row counts and widths (multiples of 8): gather (plain and recovery rows), the
    two-buffer cache sync and the scatter, bit for bit against the oracle's row operations."""
    t = tsa()
    rng = np.random.default_rng(4000 + seed)
    g = torch.Generator().manual_seed(4000 + seed)
    dim = 8 * int(rng.integers(1, 700))
    n = int(rng.integers(1, 5000))
    m = int(rng.integers(1, n + 1))
    rows = _sorted_rows(rng, n, m)
    rd = G.dev(torch.from_numpy(rows))
    print(f"  seed {seed}: n={n} m={m} dim={dim}", flush=True)
    x = _bf16(g, n, dim)
    eps = _bf16(g, n, dim)
    off, sigma = int(rng.integers(0, n + 1)), float(rng.uniform(0.1, 0.9))
    dst = torch.empty(m, dim, dtype=torch.bfloat16, device="cuda")
    t.gather_rows(G.dev(x), rd, m, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), x[torch.from_numpy(rows).long()])
    t.gather_rows(G.dev(x), rd, m, dst, eps=G.dev(eps), src_row_offset=off, sigma=sigma)
    torch.cuda.synchronize()
    want = ref.recover_rows(G.host64(x), G.host64(eps), rows, off, sigma)
    # fp32 evaluation of (1 - s) c + s e: one bf16 ulp of the result plus the fp32 rounding of
    # the two products (as in the fixed-shape gather test)
    srcr = rows.astype(np.int64) - off
    clean = np.where((srcr >= 0)[:, None], G.host64(x)[np.maximum(srcr, 0)], 0.0)
    e = G.host64(eps)[rows]
    bound = G.bf16_ulp_of(want) + 2.0 ** -22 * ((1 - sigma) * np.abs(clean) + sigma * np.abs(e))
    assert np.all(np.abs(G.host64(dst) - want) <= bound)
    ka, va = _bf16(g, m, dim), _bf16(g, m, dim)
    kc, vc = _bf16(g, n, dim), _bf16(g, n, dim)
    kcd, vcd = G.dev(kc), G.dev(vc)
    t.kv_cache_sync(G.dev(ka), G.dev(va), rd, m, kcd, vcd)
    kw_, vw_ = G.host64(kc), G.host64(vc)
    ref.kv_cache_sync(kw_, vw_, rows, G.host64(ka), G.host64(va))
    out = G.dev(kc)
    t.scatter_out(G.dev(ka), rd, m, out)
    torch.cuda.synchronize()
    assert np.array_equal(G.host64(kcd), kw_) and np.array_equal(G.host64(vcd), vw_)
    ow = G.host64(kc)
    ref.scatter(ow, rows, G.host64(ka))
    assert np.array_equal(G.host64(out), ow)
