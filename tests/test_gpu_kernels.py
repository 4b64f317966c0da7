"""Per-stage GPU parity against the CPU oracle (through the C ABI)."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import gpu_util as G
import pins
from oracle import reference as ref

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    G.need_gpu()


def tsa():
    import token_sparse_attention_rel_amd as t
    return t


def _randn_bf16(gen, *shape, scale=1.0):
    return (torch.randn(*shape, generator=gen) * scale).to(torch.bfloat16)


# ------------------------------------------------------------------ scores

@pytest.mark.parametrize("dtype,n,dim", [(torch.float32, 256, 128), (torch.bfloat16, 1000, 1536),
                                         (torch.bfloat16, 77, 5120), (torch.float32, 300, 768),
                                         (torch.bfloat16, 130, 512)])
def test_scores_match_oracle(dtype, n, dim):
    t = tsa()
    g = torch.Generator().manual_seed(n + dim)
    x_ref = torch.randn(n, dim, generator=g).to(dtype)
    scale = torch.where(torch.rand(n, generator=g) < 0.7, 0.01, 0.5)
    x_cur = (x_ref.float() + scale[:, None] * torch.randn(n, dim, generator=g)).to(dtype)
    x_cur[3] = x_ref[3]           # unchanged token -> 0
    x_ref[5] = 0
    x_cur[5] = 0                  # 0 / 0 -> 0
    x_ref[6] = 0                  # x / 0 -> inf
    xc, xr = G.dev(x_cur), G.dev(x_ref)
    scores = torch.empty(n, device="cuda")
    mask = torch.empty(n, dtype=torch.uint8, device="cuda")
    idx = torch.empty(n, dtype=torch.int32, device="cuda")
    na = torch.empty(1, dtype=torch.int32, device="cuda")
    for kind, rel in ((t.SCORE_REL_L1, True), (t.SCORE_ABS_L1, False)):
        t.select_active(xc, xr, 0, t.SELECT_TOPK, k=n // 4, score_kind=kind, scores_out=scores,
                        mask_out=mask, idx_out=idx, n_active_out=na)
        got = G.host64(scores)
        want = ref.token_scores(G.host64(x_cur), G.host64(x_ref), 0, relative=rel)
        fin = np.isfinite(want)
        assert np.array_equal(np.isfinite(got), fin)
        assert np.all(np.isinf(got[~fin]))
        err = np.abs(got[fin] - want[fin]) / np.maximum(np.abs(want[fin]), 1e-30)
        print(f"  kind={kind} max rel err {err.max():.2e}", flush=True)
        assert err.max() <= G.SCORE_RTOL
        if rel:
            assert got[3] == 0.0 and got[5] == 0.0 and math.isinf(got[6])


def test_scores_interframe_offset():
    t = tsa()
    g = torch.Generator().manual_seed(5)
    hw, frames, dim = 40, 5, 256
    x = torch.randn(hw * frames, dim, generator=g).to(torch.bfloat16)
    n = x.shape[0]
    scores = torch.empty(n, device="cuda")
    mask = torch.empty(n, dtype=torch.uint8, device="cuda")
    idx = torch.empty(n, dtype=torch.int32, device="cuda")
    na = torch.empty(1, dtype=torch.int32, device="cuda")
    t.select_active(G.dev(x), None, hw, t.SELECT_TOPK, k=50, scores_out=scores, mask_out=mask,
                    idx_out=idx, n_active_out=na)
    got = G.host64(scores)
    want = ref.token_scores(G.host64(x), None, hw)
    assert np.all(np.isinf(got[:hw])) and np.all(np.isfinite(got[hw:]))
    assert np.max(np.abs(got[hw:] - want[hw:]) / want[hw:]) <= G.SCORE_RTOL


# ------------------------------------------------------------------ select

def _exact_score_rows(values, dim=64, seed=0):
    """fp32 token pairs whose relative L1 score is exactly `values[i]` (a power of two or 0):
    x_cur = x_ref * (1 + v), exact in fp32 for bf16-valued x_ref."""
    g = torch.Generator().manual_seed(seed)
    x_ref = torch.randn(len(values), dim, generator=g).to(torch.bfloat16).float()
    v = torch.tensor(values, dtype=torch.float32)
    x_cur = x_ref * (1.0 + v[:, None])
    return x_cur, x_ref


@pytest.mark.parametrize("n", [1, 7, 100, 4096, 4099, 12000, 20000, 32760, 32768, 32769, 40000, 100001])
def test_topk_select_and_compact_bit_exact_with_ties(n):
    t = tsa()
    r = np.random.default_rng(n)
    # scores drawn from a few exact powers of two -> heavy ties at the k-th value
    vals = (2.0 ** -r.integers(1, 6, n)).astype(np.float64)
    vals[r.random(n) < 0.05] = 0.0
    x_cur, x_ref = _exact_score_rows(vals.tolist(), seed=n)
    want_scores = ref.token_scores(x_cur.double().numpy(), x_ref.double().numpy())
    assert np.array_equal(want_scores, vals)  # the construction is exact
    xc, xr = G.dev(x_cur), G.dev(x_ref)
    scores = torch.empty(n, device="cuda")
    mask = torch.empty(n, dtype=torch.uint8, device="cuda")
    idx = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    pidx = torch.full((n,), -7, dtype=torch.int32, device="cuda")
    na = torch.empty(1, dtype=torch.int32, device="cuda")
    for k in sorted({0, 1, n // 3, n // 2, n - 1, n}):
        if k < 0:
            continue
        t.select_active(xc, xr, 0, t.SELECT_TOPK, k=k, scores_out=scores, mask_out=mask,
                        idx_out=idx, pidx_out=pidx, n_active_out=na)
        torch.cuda.synchronize()
        assert np.array_equal(G.host64(scores), vals)
        want = ref.select_topk(vals, k)
        wi, wp = ref.compact(want)
        assert np.array_equal(mask.cpu().numpy().astype(bool), want), k
        assert int(na.item()) == k
        assert np.array_equal(idx.cpu().numpy()[:k], wi)
        assert np.array_equal(pidx.cpu().numpy()[:n - k], wp)


@pytest.mark.parametrize("n,k", [(32760, 9828), (100001, 30000), (118800, 45619), (65536, 1), (1000003, 333333)])
def test_topk_distinct_scores_multi_chunk(n, k):
    """Continuous scores (no ties): the selected set is the top k of the kernel's own fp32
    scores, decided by the oracle on those same values."""
    t = tsa()
    g = torch.Generator().manual_seed(n)
    x_ref = torch.randn(n, 64, generator=g).to(torch.bfloat16)
    x_cur = (x_ref.float() + 0.3 * torch.randn(n, 64, generator=g)).to(torch.bfloat16)
    scores = torch.empty(n, device="cuda")
    mask = torch.empty(n, dtype=torch.uint8, device="cuda")
    idx = torch.empty(n, dtype=torch.int32, device="cuda")
    pidx = torch.empty(n, dtype=torch.int32, device="cuda")
    na = torch.empty(1, dtype=torch.int32, device="cuda")
    t.select_active(G.dev(x_cur), G.dev(x_ref), 0, t.SELECT_TOPK, k=k, scores_out=scores, mask_out=mask,
                    idx_out=idx, pidx_out=pidx, n_active_out=na)
    torch.cuda.synchronize()
    s64 = G.host64(scores)
    want = ref.select_topk(s64, k)
    wi, wp = ref.compact(want)
    assert np.array_equal(mask.cpu().numpy().astype(bool), want)
    assert int(na.item()) == k
    assert np.array_equal(idx.cpu().numpy()[:k], wi)
    assert np.array_equal(pidx.cpu().numpy()[:n - k], wp)


@pytest.mark.parametrize("n", [5, 1023, 4096, 30001, 70001])
def test_threshold_mask_schedule_modes_bit_exact(n):
    t = tsa()
    r = np.random.default_rng(7 + n)
    vals = (2.0 ** -r.integers(1, 8, n)).astype(np.float64)
    x_cur, x_ref = _exact_score_rows(vals.tolist(), seed=n)
    xc, xr = G.dev(x_cur), G.dev(x_ref)
    scores = torch.empty(n, device="cuda")
    mask = torch.empty(n, dtype=torch.uint8, device="cuda")
    idx = torch.empty(n, dtype=torch.int32, device="cuda")
    pidx = torch.empty(n, dtype=torch.int32, device="cuda")
    na = torch.empty(1, dtype=torch.int32, device="cuda")

    def check(want):
        torch.cuda.synchronize()
        wi, wp = ref.compact(want)
        assert np.array_equal(mask.cpu().numpy().astype(bool), want)
        assert int(na.item()) == wi.size
        assert np.array_equal(idx.cpu().numpy()[:wi.size], wi)
        assert np.array_equal(pidx.cpu().numpy()[:wp.size], wp)

    for tau in (2.0 ** -3, 2.0 ** -3 + 1e-4, 1.0, 0.0):  # exact equality s == tau is active
        t.select_active(xc, xr, 0, t.SELECT_THRESHOLD, tau=tau, scores_out=scores, mask_out=mask,
                        idx_out=idx, pidx_out=pidx, n_active_out=na)
        check(ref.select_threshold(vals, tau))
    m = r.random(n) < 0.3
    t.select_active(None, None, 0, t.SELECT_MASK, aux_in=G.dev(torch.from_numpy(m.astype(np.uint8))),
                    mask_out=mask, idx_out=idx, pidx_out=pidx, n_active_out=na, n_rows=n)
    check(m)
    periods = r.choice([1, 2, 4, 0], n).astype(np.uint8)
    pd = G.dev(torch.from_numpy(periods))
    for step in range(9):
        t.select_active(None, None, 0, t.SELECT_SCHEDULE, aux_in=pd, step=step, mask_out=mask,
                        idx_out=idx, pidx_out=pidx, n_active_out=na, n_rows=n)
        want = (periods != 0) & (step % np.maximum(periods, 1) == 0)
        check(want)


def test_assign_groups_bit_exact():
    t = tsa()
    n = 5000
    r = np.random.default_rng(3)
    vals = (2.0 ** -r.integers(1, 5, n)).astype(np.float64)
    x_cur, x_ref = _exact_score_rows(vals.tolist(), seed=3)
    scores = torch.empty(n, device="cuda")
    mask = torch.empty(n, dtype=torch.uint8, device="cuda")
    idx = torch.empty(n, dtype=torch.int32, device="cuda")
    na = torch.empty(1, dtype=torch.int32, device="cuda")
    t.select_active(G.dev(x_cur), G.dev(x_ref), 0, t.SELECT_TOPK, k=1, scores_out=scores,
                    mask_out=mask, idx_out=idx, n_active_out=na)
    period = torch.empty(n, dtype=torch.uint8, device="cuda")
    ws = torch.empty(t.select_workspace_bytes(n) + n, dtype=torch.uint8, device="cuda")
    for counts, periods in (((1250, 1250, 2500), (1, 2, 4)), ((n,), (3,)), ((0, 4999, 1), (1, 2, 8))):
        t.assign_groups(scores, counts, periods, period, ws)
        want = ref.assign_periods(vals, counts, periods)
        assert np.array_equal(period.cpu().numpy(), want)


# -------------------------------------------------------------- row movers

@pytest.mark.parametrize("n,dim,na_", [(3000, 1536, 901), (700, 512, 333), (400, 3072, 97), (300, 5120, 77),
                                       (64, 1536, 1)])
def test_gather_cache_sync_scatter_bit_exact(n, dim, na_):
    """Row widths for each loader shape (2 or 4 slices per lane with two rows per wave, 8 with
    one, rows longer than one pass) and odd row counts (a wave with one live row)."""
    t = tsa()
    g = torch.Generator().manual_seed(11)
    x = _randn_bf16(g, n, dim)
    rows = torch.from_numpy(np.sort(np.random.default_rng(1).choice(n, na_, replace=False)).astype(np.int32))
    xd, rd = G.dev(x), G.dev(rows)
    dst = torch.empty(na_, dim, dtype=torch.bfloat16, device="cuda")
    t.gather_rows(xd, rd, na_, dst)
    assert torch.equal(dst.cpu(), x[rows.long()])
    # recovery rows: (1 - sigma) x[t - off] + sigma eps[t], first rows have no previous row
    eps = _randn_bf16(g, n, dim)
    off = min(500, n // 3)
    for sigma in (0.0, 1.0, 0.6):
        t.gather_rows(xd, rd, na_, dst, eps=G.dev(eps), src_row_offset=off, sigma=sigma)
        want = ref.recover_rows(G.host64(x), G.host64(eps), rows.numpy(), off, sigma)
        got = G.host64(dst)
        if sigma in (0.0, 1.0):
            assert np.array_equal(got, want)
        else:
            # fp32 evaluation of (1 - s) c + s e: one bf16 ulp of the result plus the fp32
            # rounding of the two products, which dominates where the terms cancel
            src = rows.numpy() - off
            clean = np.where((src >= 0)[:, None], G.host64(x)[np.maximum(src, 0)], 0.0)
            e = G.host64(eps)[rows.numpy()]
            ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 2.0 ** -126))) - 7)
            bound = ulp + 2.0 ** -22 * ((1 - sigma) * np.abs(clean) + sigma * np.abs(e))
            err = np.abs(got - want)
            print(f"  recovery sigma={sigma}: {(err > 0).sum()} of {got.size} differ, "
                  f"max err/bound {np.max(err / bound):.3f}", flush=True)
            assert np.all(err <= bound)
    # cache sync: listed rows overwritten, all others bit-identical
    kc, vc = _randn_bf16(g, n, dim), _randn_bf16(g, n, dim)
    ka, va = _randn_bf16(g, na_, dim), _randn_bf16(g, na_, dim)
    kcd, vcd = G.dev(kc), G.dev(vc)
    t.kv_cache_sync(G.dev(ka), G.dev(va), rd, na_, kcd, vcd)
    wk, wv = kc.clone(), vc.clone()
    wk[rows.long()] = ka
    wv[rows.long()] = va
    assert torch.equal(kcd.cpu(), wk) and torch.equal(vcd.cpu(), wv)
    # scatter
    out = _randn_bf16(g, n, dim)
    od = G.dev(out)
    t.scatter_out(G.dev(ka), rd, na_, od)
    wo = out.clone()
    wo[rows.long()] = ka
    assert torch.equal(od.cpu(), wo)
    # n = 0 touches nothing
    t.kv_cache_sync(G.dev(ka), G.dev(va), rd, 0, kcd, vcd)
    t.scatter_out(G.dev(ka), rd, 0, od)
    assert torch.equal(kcd.cpu(), wk) and torch.equal(od.cpu(), wo)


# -------------------------------------------------------------- projection

def test_qkv_layout_exact_with_identity_weights():
    t = tsa()
    g = torch.Generator().manual_seed(2)
    n, dim = 300, 128
    x = _randn_bf16(g, n, dim)
    perm = torch.randperm(dim, generator=g)
    w = torch.zeros(3 * dim, dim)
    w[:dim] = torch.eye(dim)
    w[dim:2 * dim] = 2 * torch.eye(dim)
    w[2 * dim + torch.arange(dim), perm] = 1.0
    rows = torch.arange(0, n, 3, dtype=torch.int32)
    m = rows.numel()
    q = torch.empty(m, dim, dtype=torch.bfloat16, device="cuda")
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    t.qkv_active(G.dev(x), G.dev(rows), m, G.dev(w.to(torch.bfloat16)), q_out=q, k_out=k, v_out=v)
    xs = x[rows.long()]
    assert torch.equal(q.cpu(), xs)
    assert torch.equal(k.cpu(), (2 * xs.float()).to(torch.bfloat16))
    assert torch.equal(v.cpu(), xs[:, perm])


@pytest.mark.parametrize("n_x,m,dim,src", [(256, 64, 128, "f32"), (3000, 901, 1536, "bf16"),
                                           (700, 131, 5120, "bf16"), (2000, 777, 3072, "recover"),
                                           (500, 500, 192, "bf16")])
def test_qkv_matches_oracle(n_x, m, dim, src):
    t = tsa()
    g = torch.Generator().manual_seed(m)
    x = torch.randn(n_x, dim, generator=g)
    x = x if src == "f32" else x.to(torch.bfloat16)
    w = (torch.randn(3 * dim, dim, generator=g) / math.sqrt(dim)).to(torch.bfloat16)
    rows = np.sort(np.random.default_rng(m).choice(n_x, m, replace=False)).astype(np.int32)
    rd = G.dev(torch.from_numpy(rows))
    q = torch.empty(m, dim, dtype=torch.bfloat16, device="cuda")
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    eps = None
    off, sigma = n_x // 10, 0.6
    if src == "recover":
        eps = _randn_bf16(g, n_x, dim)
        t.qkv_active(G.dev(x), rd, m, G.dev(w), q_out=q, k_out=k, v_out=v, eps=G.dev(eps),
                     src_row_offset=off, sigma=sigma)
        a_rows = ref.recover_rows(G.host64(x), G.host64(eps), rows, off, sigma)
    else:
        t.qkv_active(G.dev(x), rd, m, G.dev(w), q_out=q, k_out=k, v_out=v)
        a_rows = G.host64(x)[rows]
    want = ref.project(a_rows, G.host64(w))
    for name, got in (("q", q), ("k", k), ("v", v)):
        gh = G.host64(got)
        if src == "recover":
            # the recovered input rows carry their own fp32 rounding (see the gather test)
            G.assert_close(gh, want[name], f"{src} {name}")
        else:
            part = "qkv".index(name)
            wp = np.abs(G.host64(w)[part * dim:(part + 1) * dim])
            G.assert_projection_close(gh, want[name], np.abs(ref.round_bf16(a_rows)) @ wp.T, dim,
                                      f"{src} {name}")
    # K/V only, written into cache rows (fused cache sync); other rows untouched
    kc = _randn_bf16(g, n_x, dim)
    vc = _randn_bf16(g, n_x, dim)
    kcd, vcd = G.dev(kc), G.dev(vc)
    if src == "recover":
        t.qkv_active(G.dev(x), rd, m, G.dev(w), k_out=kcd, v_out=vcd, out_is_cache=True,
                     n_cache=n_x, eps=G.dev(eps), src_row_offset=off, sigma=sigma)
    else:
        t.qkv_active(G.dev(x), rd, m, G.dev(w), k_out=kcd, v_out=vcd, out_is_cache=True, n_cache=n_x)
    others = np.setdiff1d(np.arange(n_x), rows)
    kch, vch = kcd.cpu(), vcd.cpu()
    assert torch.equal(kch[others], kc[others]) and torch.equal(vch[others], vc[others])
    assert torch.equal(kch[rows], k.cpu()) and torch.equal(vch[rows], v.cpu())


def _qkv_rows_up_to(n_x, src, seed):
    """Token rows at the end of an input of n_x rows of 1536 (bf16 or fp32 rows, or LIPAR's
    recovery rows from clean and noise rows of the same size): sampled rows against the oracle,
    K/V written into caches of n_x rows, untouched cache rows left zero."""
    t = tsa()
    dim = 1536
    gen = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randn(n_x, dim, device="cuda", generator=gen)
    if src != "f32":
        x = x.to(torch.bfloat16)
    w = (torch.randn(3 * dim, dim, device="cuda", generator=gen) / math.sqrt(dim)).to(torch.bfloat16)
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([np.arange(16), np.arange(n_x - 300, n_x),
                                     rng.choice(n_x, 700, replace=False)])).astype(np.int32)
    m = rows.size
    print(f"  n_x={n_x} ({n_x * dim * x.element_size()} bytes of {src} rows), {m} rows", flush=True)
    rd = G.dev(torch.from_numpy(rows))
    q = torch.empty(m, dim, dtype=torch.bfloat16, device="cuda")
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    kc = torch.zeros(n_x, dim, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    x_rows = G.host64(x[torch.from_numpy(rows).long().cuda()])
    if src == "recover":
        eps = torch.randn(n_x, dim, device="cuda", generator=gen).to(torch.bfloat16)
        off, sigma = 3600, 0.6
        kw = dict(eps=eps, src_row_offset=off, sigma=sigma)
        # the recovery rows of the sampled tokens, from the gathered clean and noise rows
        srcr = rows.astype(np.int64) - off
        ok = srcr >= 0
        clean = np.zeros((m, dim))
        clean[ok] = G.host64(x[torch.from_numpy(srcr[ok]).cuda()])
        a_rows = ref.recover_rows(clean, G.host64(eps[torch.from_numpy(rows).long().cuda()]), np.arange(m), 0, sigma)
    else:
        kw = {}
        a_rows = x_rows
    t.qkv_active(x, rd, m, w, q_out=q, k_out=k, v_out=v, **kw)
    t.qkv_active(x, rd, m, w, k_out=kc, v_out=vc, out_is_cache=True, n_cache=n_x, **kw)
    torch.cuda.synchronize()
    want = ref.project(a_rows, G.host64(w))
    for name, got in (("q", q), ("k", k), ("v", v)):
        gh = G.host64(got)
        if src == "recover":
            G.assert_close(gh, want[name], f"{n_x} rows {src} {name}")
        else:
            part = "qkv".index(name)
            wp = np.abs(G.host64(w)[part * dim:(part + 1) * dim])
            G.assert_projection_close(gh, want[name], np.abs(ref.round_bf16(a_rows)) @ wp.T, dim,
                                      f"{n_x} rows {src} {name}")
    rl = torch.from_numpy(rows).long().cuda()
    assert torch.equal(kc[rl], k) and torch.equal(vc[rl], v)
    others = torch.from_numpy(np.setdiff1d(rng.choice(n_x, 2000, replace=False), rows)).long().cuda()
    assert not kc[others].any() and not vc[others].any()


@pytest.mark.slow
@pytest.mark.parametrize("src", ["bf16", "recover"])
def test_qkv_at_the_buffer_range_limit(src):
    """The largest bf16 input one 32-bit buffer range holds (n_x * dim * 2 bytes just under
    2**31, 699050 rows of 1536): the 32-bit offsets of the row loads (and of the noise rows)
    run at their limit."""
    _qkv_rows_up_to((2 ** 31 - 1) // (1536 * 2), src, 7)


@pytest.mark.slow
@pytest.mark.parametrize("src", ["bf16", "recover", "f32"])
def test_qkv_past_the_buffer_range_limit(src):
    """800000 token rows of 1536 (2.46 GB of bf16 rows, 4.9 GB of fp32 ones): bf16 rows take
    the kernels that address every row with a 64-bit pointer (LDS-direct copies from global
    addresses; plain loads of the clean and noise rows for the recovery), with sampled rows
    past the 2 GiB mark."""
    _qkv_rows_up_to(800_000, src, 8)


@pytest.mark.slow
def test_rows_to_cache_past_the_buffer_range_limit():
    """tsa_qkv_rows_to_cache with 800000 compact rows of 1536 (2.46 GB) into caches of 1000000
    rows: the compact rows past the 2 GiB mark are read through 64-bit addresses; sampled rows
    against the oracle, their cache rows bit-identical to the compact projection's."""
    t = tsa()
    dim, n, n_cache = 1536, 800_000, 1_000_000
    gen = torch.Generator(device="cuda").manual_seed(9)
    a = torch.randn(n, dim, device="cuda", generator=gen).to(torch.bfloat16)
    w = (torch.randn(3 * dim, dim, device="cuda", generator=gen) / math.sqrt(dim)).to(torch.bfloat16)
    rng = np.random.default_rng(9)
    rows = np.sort(rng.choice(n_cache, n, replace=False)).astype(np.int32)
    kc = torch.zeros(n_cache, dim, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    t.qkv_rows_to_cache(a, G.dev(torch.from_numpy(rows)), n, w, kc, vc)
    torch.cuda.synchronize()
    sample = np.unique(np.concatenate([np.arange(8), np.arange(n - 200, n), rng.choice(n, 500, replace=False)]))
    a_rows = G.host64(a[torch.from_numpy(sample).long().cuda()])
    want = ref.project(a_rows, G.host64(w), parts="kv")
    cr = torch.from_numpy(rows[sample]).long().cuda()
    for name, cache in (("k", kc), ("v", vc)):
        part = "qkv".index(name)
        wp = np.abs(G.host64(w)[part * dim:(part + 1) * dim])
        G.assert_projection_close(G.host64(cache[cr]), want[name], np.abs(a_rows) @ wp.T, dim,
                                  f"rows_to_cache past 2 GiB {name}")
    # the same rows through the compact projection: bit-identical
    sub = torch.from_numpy(sample.astype(np.int32))
    ks = torch.empty(sample.size, dim, dtype=torch.bfloat16, device="cuda")
    vs = torch.empty_like(ks)
    t.qkv_active(a, G.dev(sub), sample.size, w, k_out=ks, v_out=vs)
    assert torch.equal(kc[cr], ks) and torch.equal(vc[cr], vs)


@pytest.mark.parametrize("src", ["bf16", "recover", "f32"])
def test_qkv_large_tile_sampled(src):
    """A grid of at least 1024 256x256 tiles takes the large-tile kernel: checked on sampled
    rows (two per 256-row token tile plus the ragged tail) against the oracle."""
    t = tsa()
    n_x, m, dim = 9000, 7461, 3072  # 30 token tiles x 36 feature tiles
    g = torch.Generator().manual_seed(len(src))
    x = torch.randn(n_x, dim, generator=g)
    x = x if src == "f32" else x.to(torch.bfloat16)
    w = (torch.randn(3 * dim, dim, generator=g) / math.sqrt(dim)).to(torch.bfloat16)
    rows = np.sort(np.random.default_rng(5).choice(n_x, m, replace=False)).astype(np.int32)
    rd = G.dev(torch.from_numpy(rows))
    q = torch.empty(m, dim, dtype=torch.bfloat16, device="cuda")
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    off, sigma = 900, 0.6
    eps = _randn_bf16(g, n_x, dim) if src == "recover" else None
    t.qkv_active(G.dev(x), rd, m, G.dev(w), q_out=q, k_out=k, v_out=v,
                 eps=None if eps is None else G.dev(eps), src_row_offset=off, sigma=sigma)
    rng = np.random.default_rng(6)
    sample = np.unique(np.concatenate([np.arange(0, m, 256)[:, None] + rng.integers(0, 256, (m // 256 + 1, 2)),
                                       np.arange(m - 5, m)[:, None]], axis=None))
    sample = sample[sample < m]
    if src == "recover":
        a_rows = ref.recover_rows(G.host64(x), G.host64(eps), rows[sample], off, sigma)
    else:
        a_rows = G.host64(x)[rows[sample]]
    w64 = G.host64(w)
    want = ref.project(a_rows, w64)
    for name, got in (("q", q), ("k", k), ("v", v)):
        gh = G.host64(got)[sample]
        if src == "recover":
            G.assert_close(gh, want[name], f"large tile {src} {name}")
        else:
            part = "qkv".index(name)
            wp = np.abs(w64[part * dim:(part + 1) * dim])
            G.assert_projection_close(gh, want[name], np.abs(ref.round_bf16(a_rows)) @ wp.T, dim,
                                      f"large tile {src} {name}")
    # K/V into cache rows: the same values, other rows untouched
    kc = torch.zeros(n_x, dim, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    t.qkv_active(G.dev(x), rd, m, G.dev(w), k_out=kc, v_out=vc, out_is_cache=True, n_cache=n_x,
                 eps=None if eps is None else G.dev(eps), src_row_offset=off, sigma=sigma)
    others = torch.from_numpy(np.setdiff1d(np.arange(n_x), rows)).cuda()
    rl = rd.long()
    assert torch.equal(kc[rl], k) and torch.equal(vc[rl], v)
    assert not kc[others].any() and not vc[others].any()


@pytest.mark.parametrize("kv_only,rope", [(False, None), (True, None), (False, (30, 40))])
def test_qkv_large_and_small_tiles_agree_bit_for_bit(kv_only, rope):
    """Grids of at least 1024 256x256 tiles run the large tile; a call on a few of the same
    rows runs the 128x128 tile.  Both accumulate every output in the same order (ascending
    16-deep K chunks in fp32), so the rows agree bit for bit -- here with the ragged last
    token tile, K/V written into cache rows (features from D on), and 3D rotary positions in
    the epilogue."""
    t = tsa()
    n_x, m, dim, heads = 12000, 11001, 3072, 24  # K/V only: 24 x 43 large tiles
    g = torch.Generator().manual_seed(11)
    x = G.dev(_randn_bf16(g, n_x, dim))
    w = G.dev((torch.randn(3 * dim, dim, generator=g) / math.sqrt(dim)).to(torch.bfloat16))
    rows = np.sort(np.random.default_rng(12).choice(n_x, m, replace=False)).astype(np.int32)
    pick = np.unique(np.concatenate([np.arange(0, m, 997), np.arange(m - 40, m)]))
    assert (3 * dim // 256) * ((m + 255) // 256) >= 1024 and (2 * dim // 256) * ((m + 255) // 256) >= 1024
    assert (3 * dim // 256) * ((len(pick) + 255) // 256) < 1024

    def run(r):
        n = len(r)
        rd = G.dev(torch.from_numpy(r))
        if kv_only:
            kc = torch.zeros(n_x, dim, dtype=torch.bfloat16, device="cuda")
            vc = torch.zeros_like(kc)
            t.qkv_active(x, rd, n, w, k_out=kc, v_out=vc, out_is_cache=True, n_cache=n_x)
            rl = rd.long()
            return [kc[rl], vc[rl]]
        out = [torch.empty(n, dim, dtype=torch.bfloat16, device="cuda") for _ in range(3)]
        if rope is None:
            t.qkv_active(x, rd, n, w, q_out=out[0], k_out=out[1], v_out=out[2])
        else:
            t.qkv_active_rope(x, rd, n, w, heads, rope[0], rope[1], q_out=out[0], k_out=out[1], v_out=out[2])
        return out

    full = run(rows)
    few = run(rows[pick])
    torch.cuda.synchronize()
    pk = torch.from_numpy(pick).cuda()
    for a, b in zip(full, few):
        assert torch.equal(a[pk], b)


@pytest.mark.parametrize("n_x,m,dim,rope", [(3000, 2049, 1536, None), (12000, 11001, 3072, None),
                                            (1500, 901, 768, (5, 12, 4))])
def test_qkv_register_staged_and_lds_direct_agree_bit_for_bit(n_x, m, dim, rope):
    """bf16 token rows go HBM -> LDS directly (qkv_gemm_lds_kernel); fp32 rows go through
    registers and are converted on the way (qkv_gemm_kernel).  Fed the same values (fp32
    rows that are exactly bf16), both kernels accumulate every output in the same order, so
    Q, K and V (here written into cache rows, with rotary positions in one case) agree bit
    for bit -- on the small-tile grid and, for 12000 x 3072, the large-tile grid."""
    t = tsa()
    g = torch.Generator().manual_seed(n_x)
    xb = _randn_bf16(g, n_x, dim)
    w = G.dev((torch.randn(3 * dim, dim, generator=g) / math.sqrt(dim)).to(torch.bfloat16))
    rows = G.dev(torch.from_numpy(np.sort(np.random.default_rng(m).choice(n_x, m, replace=False)).astype(np.int32)))
    heads = dim // 128 if dim % 128 == 0 else dim // 64
    outs = []
    for x in (G.dev(xb), G.dev(xb.float())):
        q = torch.empty(m, dim, dtype=torch.bfloat16, device="cuda")
        kc = torch.zeros(n_x, dim, dtype=torch.bfloat16, device="cuda")
        vc = torch.zeros_like(kc)
        if rope is None:
            t.qkv_active(x, rows, m, w, q_out=q, k_out=kc, v_out=vc, out_is_cache=True, n_cache=n_x)
        else:
            t.qkv_active_rope(x, rows, m, w, heads, rope[0], rope[1], q_out=q, k_out=kc, v_out=vc,
                              out_is_cache=True, n_cache=n_x)
        torch.cuda.synchronize()
        outs.append((q, kc, vc))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("n_x,m,dim,rope", [(2000, 777, 1536, None), (9000, 7461, 3072, None),
                                            (1200, 500, 512, (6, 10, 4))])
def test_rows_to_cache_equals_fused_recovery(n_x, m, dim, rope):
    """Recovered rows gathered once and projected into their cache rows equal the fused
    recovery projection bit for bit (the same blend, the same GEMM arithmetic)."""
    t = tsa()
    g = torch.Generator().manual_seed(m)
    x = _randn_bf16(g, n_x, dim)
    eps = _randn_bf16(g, n_x, dim)
    w = (torch.randn(3 * dim, dim, generator=g) / math.sqrt(dim)).to(torch.bfloat16)
    rows = G.dev(torch.from_numpy(np.sort(np.random.default_rng(m).choice(n_x, m, replace=False)).astype(np.int32)))
    off, sigma = n_x // 7, 0.6
    caches = [torch.zeros(n_x, dim, dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    xd, ed, wd = G.dev(x), G.dev(eps), G.dev(w)
    if rope is None:
        t.qkv_active(xd, rows, m, wd, k_out=caches[0], v_out=caches[1], out_is_cache=True, n_cache=n_x, eps=ed,
                     src_row_offset=off, sigma=sigma)
    else:
        h, wd_, heads = rope
        t.qkv_active_rope(xd, rows, m, wd, heads, h, wd_, k_out=caches[0], v_out=caches[1], out_is_cache=True,
                          n_cache=n_x, eps=ed, src_row_offset=off, sigma=sigma)
    rec = torch.empty(m, dim, dtype=torch.bfloat16, device="cuda")
    t.gather_rows(xd, rows, m, rec, eps=ed, src_row_offset=off, sigma=sigma)
    if rope is None:
        t.qkv_rows_to_cache(rec, rows, m, wd, caches[2], caches[3])
    else:
        t.qkv_rows_to_cache(rec, rows, m, wd, caches[2], caches[3], rope=(h, wd_, 10000.0), heads=heads)
    torch.cuda.synchronize()
    assert torch.equal(caches[0], caches[2]) and torch.equal(caches[1], caches[3])
    others = torch.from_numpy(np.setdiff1d(np.arange(n_x), rows.cpu().numpy())).cuda()
    assert not caches[2][others].any() and caches[2][rows.long()].any()


# --------------------------------------------------------------- attention

@pytest.mark.parametrize("n_q,n_kv,heads,hd", [(1, 1, 1, 64), (37, 53, 3, 64), (128, 64, 2, 128),
                                               (300, 1000, 2, 128), (1000, 4099, 4, 128),
                                               (777, 2085, 4, 64), (129, 20000, 1, 128)])
def test_attention_matches_oracle(n_q, n_kv, heads, hd):
    t = tsa()
    g = torch.Generator().manual_seed(n_q * 7 + n_kv)
    dim = heads * hd
    q = _randn_bf16(g, n_q, dim)
    k = _randn_bf16(g, n_kv, dim)
    v = _randn_bf16(g, n_kv, dim)
    out = torch.empty(n_q, dim, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(heads, n_q, dtype=torch.float32, device="cuda")
    t.sparse_query_attention(G.dev(q), G.dev(k), G.dev(v), n_q, heads, hd, out, lse_out=lse)
    want, want_lse = ref.attention(G.host64(q), G.host64(k), G.host64(v), heads, return_lse=True)
    G.assert_close(G.host64(out), want, f"attn {n_q}x{n_kv} h{heads} d{hd}")
    assert np.max(np.abs(G.host64(lse) - want_lse)) <= 1e-3 * max(1.0, np.abs(want_lse).max())


@pytest.mark.parametrize("hd", [128, 64])
def test_attention_every_tile_count_up_to_40(hd):
    """K/V tiles (32 keys) are staged two per barrier, with the loop's first, last and
    next-to-last iterations specialised: every cache length from one tile to 40 tiles, whole
    and ragged, for both head widths, against the oracle (and the split schedule too)."""
    t = tsa()
    heads, n_q = 2, 70
    dim = heads * hd
    g = torch.Generator().manual_seed(hd)
    lengths = sorted({1, 2, 31, 32, 33} | {32 * nt + r for nt in range(1, 41) for r in (0, 7)})
    k_all = _randn_bf16(g, max(lengths), dim)
    v_all = _randn_bf16(g, max(lengths), dim)
    q = _randn_bf16(g, n_q, dim, scale=2.0)
    qd = G.dev(q)
    for n_kv in lengths:
        kd, vd = G.dev(k_all[:n_kv]), G.dev(v_all[:n_kv])
        want = ref.attention(G.host64(q), G.host64(k_all[:n_kv]), G.host64(v_all[:n_kv]), heads)
        out = torch.empty(n_q, dim, dtype=torch.bfloat16, device="cuda")
        t.sparse_query_attention(qd, kd, vd, n_q, heads, hd, out)
        got = G.host64(out)
        ws_bytes = t.attention_workspace_bytes(n_q, n_kv, heads, hd)
        if ws_bytes:
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
            out2 = torch.empty_like(out)
            t.sparse_query_attention(qd, kd, vd, n_q, heads, hd, out2, workspace=ws)
            G.assert_close(G.host64(out2), want, f"split n_kv={n_kv} d={hd}")
        assert G.rel_frob(got, want) <= G.REL_FROB, n_kv
        assert np.max(np.abs(got - want) / np.maximum(1.0, np.abs(want))) <= G.MAX_ABS, n_kv
    print(f"  {len(lengths)} cache lengths from {lengths[0]} to {lengths[-1]} keys", flush=True)


@pytest.mark.slow
def test_attention_at_the_buffer_range_limit():
    """The largest K/V the ABI accepts for one head of 128: n_kv * 128 * 2 bytes just under
    2**31 (8388607 keys, 2 GiB each for K and V), so the 32-bit buffer offsets of the K/V
    loads and the range check of the prefetches past the last key run at their limit.
    Whole tiles and the split schedule, sampled query rows against the oracle."""
    t = tsa()
    heads, hd = 1, 128
    n_kv = (2 ** 31 - 1) // (heads * hd * 2)
    n_q = 300
    gen = torch.Generator(device="cuda").manual_seed(31)
    q = (3.0 * torch.randn(n_q, hd, device="cuda", generator=gen)).to(torch.bfloat16)
    k = torch.randn(n_kv, hd, device="cuda", generator=gen).to(torch.bfloat16)
    v = torch.randn(n_kv, hd, device="cuda", generator=gen).to(torch.bfloat16)
    rows = np.array([0, 1, 150, 255, 256, 299])
    print(f"  n_kv={n_kv} ({n_kv * hd * 2} bytes per cache); oracle on rows {rows.tolist()}", flush=True)
    want = ref.attention(G.host64(q)[rows], G.host64(k), G.host64(v), heads)
    ws_bytes = t.attention_workspace_bytes(n_q, n_kv, heads, hd)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    for name, w in (("whole tiles", None), ("split", ws if ws_bytes > 0 else None)):
        out = torch.empty(n_q, hd, dtype=torch.bfloat16, device="cuda")
        t.sparse_query_attention(q, k, v, n_q, heads, hd, out, workspace=w)
        torch.cuda.synchronize()
        G.assert_close(G.host64(out)[rows], want, f"attention at the range limit, {name}")


@pytest.mark.slow
@pytest.mark.parametrize("heads,hd", [(1, 128), (2, 64)])
def test_attention_past_the_buffer_range_limit(heads, hd):
    """K/V caches of 12000000 keys of 128 bf16 (3.07 GB each): the kernels for caches past one
    32-bit buffer range, which place the range at every key tile's first row.  The keys past the
    2 GiB mark (30 % of them) carry +3 on channel 0 of each head and their values +2, and the
    queries +-2 on that channel, so every output depends on reading those rows right.  Whole
    tiles, the split schedule, and the frame-causal variant with frames of 4000000 keys (queries
    of frames 0 and 1 see no key past the mark, those of frame 2 all of them); sampled query rows
    against the oracle."""
    t = tsa()
    dim = heads * hd
    n_kv, n_q, frame = 12_000_000, 300, 4_000_000
    mark = 2 ** 31 // (dim * 2)  # first key row at or past 2 GiB
    gen = torch.Generator(device="cuda").manual_seed(41 + hd)
    ch0 = torch.arange(heads, device="cuda") * hd
    q = torch.randn(n_q, dim, device="cuda", generator=gen)
    q[:, ch0] = torch.where(torch.arange(n_q, device="cuda") % 2 == 0, 2.0, -2.0)[:, None]
    q = q.to(torch.bfloat16)
    k = torch.randn(n_kv, dim, device="cuda", generator=gen)
    k[mark:, ch0] += 3.0
    k = k.to(torch.bfloat16)
    v = torch.randn(n_kv, dim, device="cuda", generator=gen)
    v[mark:] += 2.0
    v = v.to(torch.bfloat16)
    rows = np.array([0, 1, 2, 150, 255, 256, 298, 299])
    q_tokens = (np.arange(n_q) % 3) * frame + np.arange(n_q)  # frames 0, 1, 2 in turn
    print(f"  heads={heads} hd={hd} n_kv={n_kv} ({n_kv * dim * 2} bytes per cache, mark at key {mark}); "
          f"oracle on rows {rows.tolist()}", flush=True)
    k64, v64 = G.host64(k), G.host64(v)
    q64 = G.host64(q)[rows]
    want = ref.attention(q64, k64, v64, heads)
    want_c = ref.attention_frame_causal(q64, k64, v64, heads, q_tokens[rows], frame)
    del k64, v64
    ws_bytes = t.attention_workspace_bytes(n_q, n_kv, heads, hd)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    for name, w in (("whole tiles", None), ("split", ws if ws_bytes > 0 else None)):
        out = torch.empty(n_q, dim, dtype=torch.bfloat16, device="cuda")
        t.sparse_query_attention(q, k, v, n_q, heads, hd, out, workspace=w)
        torch.cuda.synchronize()
        G.assert_close(G.host64(out)[rows], want, f"attention past 2 GiB, {name}")
    out = torch.empty(n_q, dim, dtype=torch.bfloat16, device="cuda")
    t.frame_causal_attention(q, k, v, n_q, heads, hd, G.dev(torch.from_numpy(q_tokens.astype(np.int32))),
                             frame, out)
    torch.cuda.synchronize()
    G.assert_close(G.host64(out)[rows], want_c, "frame-causal attention past 2 GiB")


# Split schedule: shapes whose last round of query tiles (256 queries for head_dim 128, 128
# for 64) leaves a 256-CU GPU partly idle, ragged in queries and keys, so that tiles are cut
# into key ranges and merged; fewer tiles than compute units (all tiles cut), tails of
# a few tiles and of many, key counts of a few tiles and many.
SPLIT_CASES = [(1100, 700, 60, 128), (300, 3000, 12, 64), (2000, 2085, 33, 128), (300, 5000, 3, 128),
               (1030, 700, 52, 128), (1300, 1111, 60, 128), (129, 20000, 1, 128), (777, 4099, 4, 64)]


@pytest.mark.parametrize("n_q,n_kv,heads,hd", SPLIT_CASES)
def test_attention_split_matches_oracle(n_q, n_kv, heads, hd):
    t = tsa()
    ws_bytes = t.attention_workspace_bytes(n_q, n_kv, heads, hd)
    assert ws_bytes > 0, "no split for this shape on this GPU"
    g = torch.Generator().manual_seed(n_q + 3 * n_kv + heads)
    dim = heads * hd
    q = _randn_bf16(g, n_q, dim)
    k = _randn_bf16(g, n_kv, dim)
    v = _randn_bf16(g, n_kv, dim)
    want, want_lse = ref.attention(G.host64(q), G.host64(k), G.host64(v), heads, return_lse=True)
    qd, kd, vd = G.dev(q), G.dev(k), G.dev(v)
    ws = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN bytes
    lse = torch.empty(heads, n_q, dtype=torch.float32, device="cuda")
    for rep in range(2):  # the workspace keeps the first call's partials
        out = torch.empty(n_q, dim, dtype=torch.bfloat16, device="cuda")
        t.sparse_query_attention(qd, kd, vd, n_q, heads, hd, out, lse_out=lse, workspace=ws)
        G.assert_close(G.host64(out), want, f"split attn {n_q}x{n_kv} h{heads} d{hd} call {rep}")
        assert np.max(np.abs(G.host64(lse) - want_lse)) <= 1e-3 * max(1.0, np.abs(want_lse).max())
    # without a workspace: one workgroup per tile, the same result to rounding
    o_plain = torch.empty(n_q, dim, dtype=torch.bfloat16, device="cuda")
    t.sparse_query_attention(qd, kd, vd, n_q, heads, hd, o_plain)
    G.assert_close(G.host64(o_plain), want, "plain path")
    with pytest.raises(t.TsaError):
        t.sparse_query_attention(qd, kd, vd, n_q, heads, hd, out, workspace=ws[:ws_bytes - 16])


def test_attention_split_fused_scatter():
    t = tsa()
    g = torch.Generator().manual_seed(21)
    n, heads, hd = 3000, 64, 128
    dim = heads * hd
    rows = np.sort(np.random.default_rng(5).choice(n, 1111, replace=False)).astype(np.int32)
    ws = torch.empty(t.attention_workspace_bytes(rows.size, n, heads, hd), dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0
    q = _randn_bf16(g, rows.size, dim)
    k = _randn_bf16(g, n, dim)
    v = _randn_bf16(g, n, dim)
    base = _randn_bf16(g, n, dim)
    out = G.dev(base)
    t.sparse_query_attention(G.dev(q), G.dev(k), G.dev(v), rows.size, heads, hd, out,
                             out_rows=G.dev(torch.from_numpy(rows)), workspace=ws)
    oh = out.cpu()
    others = np.setdiff1d(np.arange(n), rows)
    assert torch.equal(oh[others], base[others])
    want = ref.attention(G.host64(q), G.host64(k), G.host64(v), heads)
    G.assert_close(G.host64(oh)[rows], want, "split fused scatter")


def test_attention_no_split_when_last_round_is_full():
    """A tile count that is a multiple of the resident workgroups needs no split."""
    t = tsa()
    assert t.attention_workspace_bytes(256 * 256, 4096, 1, 128) == 0
    assert t.attention_workspace_bytes(100, 5000, 3, 128) > 0


def test_attention_scaled_inputs_and_scale_argument():
    """Large logits (sharp softmax) and an explicit scale."""
    t = tsa()
    g = torch.Generator().manual_seed(9)
    n_q, n_kv, heads, hd = 200, 700, 2, 128
    q = _randn_bf16(g, n_q, heads * hd, scale=3.0)
    k = _randn_bf16(g, n_kv, heads * hd, scale=3.0)
    v = _randn_bf16(g, n_kv, heads * hd)
    out = torch.empty(n_q, heads * hd, dtype=torch.bfloat16, device="cuda")
    for scale in (0.0, 0.05):
        t.sparse_query_attention(G.dev(q), G.dev(k), G.dev(v), n_q, heads, hd, out, scale=scale)
        want = ref.attention(G.host64(q), G.host64(k), G.host64(v), heads,
                             scale=None if scale == 0.0 else scale)
        G.assert_close(G.host64(out), want, f"scale={scale}")


def test_attention_special_cases():
    t = tsa()
    g = torch.Generator().manual_seed(10)
    n_q, n_kv, heads, hd = 100, 333, 2, 64
    dim = heads * hd
    q = _randn_bf16(g, n_q, dim)
    k = _randn_bf16(g, n_kv, dim)
    # value rows all equal c -> output c
    c = _randn_bf16(g, 1, dim)
    out = torch.empty(n_q, dim, dtype=torch.bfloat16, device="cuda")
    t.sparse_query_attention(G.dev(q), G.dev(k), G.dev(c.repeat(n_kv, 1)), n_q, heads, hd, out)
    G.assert_close(G.host64(out), np.tile(G.host64(c), (n_q, 1)), "constant V", rel=4e-3, mabs=1e-2)
    # all key rows equal -> mean of V
    v = _randn_bf16(g, n_kv, dim)
    t.sparse_query_attention(G.dev(q), G.dev(k[:1].repeat(n_kv, 1)), G.dev(v), n_q, heads, hd, out)
    G.assert_close(G.host64(out), np.tile(G.host64(v).mean(0), (n_q, 1)), "equal K")


def test_attention_fused_scatter_leaves_other_rows():
    t = tsa()
    g = torch.Generator().manual_seed(12)
    n, heads, hd = 900, 2, 128
    dim = heads * hd
    rows = np.sort(np.random.default_rng(2).choice(n, 250, replace=False)).astype(np.int32)
    q = _randn_bf16(g, rows.size, dim)
    k = _randn_bf16(g, n, dim)
    v = _randn_bf16(g, n, dim)
    base = _randn_bf16(g, n, dim)
    out = G.dev(base)
    t.sparse_query_attention(G.dev(q), G.dev(k), G.dev(v), rows.size, heads, hd, out,
                             out_rows=G.dev(torch.from_numpy(rows)))
    oh = out.cpu()
    others = np.setdiff1d(np.arange(n), rows)
    assert torch.equal(oh[others], base[others])
    want = ref.attention(G.host64(q), G.host64(k), G.host64(v), heads)
    G.assert_close(G.host64(oh)[rows], want, "fused scatter")


def test_attention_deterministic():
    t = tsa()
    g = torch.Generator().manual_seed(13)
    n_q, n_kv, heads, hd = 500, 3000, 3, 128
    q, k, v = (G.dev(_randn_bf16(g, s, heads * hd)) for s in (n_q, n_kv, n_kv))
    o1 = torch.empty(n_q, heads * hd, dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty_like(o1)
    t.sparse_query_attention(q, k, v, n_q, heads, hd, o1)
    t.sparse_query_attention(q, k, v, n_q, heads, hd, o2)
    assert torch.equal(o1, o2)
    # split schedule: the same cut points every call, so also bitwise repeatable
    n_q, heads = 1100, 60
    q, k, v = (G.dev(_randn_bf16(g, s, heads * hd)) for s in (n_q, 700, 700))
    ws = torch.empty(t.attention_workspace_bytes(n_q, 700, heads, hd), dtype=torch.uint8, device="cuda")
    o1 = torch.empty(n_q, heads * hd, dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty_like(o1)
    t.sparse_query_attention(q, k, v, n_q, heads, hd, o1, workspace=ws)
    t.sparse_query_attention(q, k, v, n_q, heads, hd, o2, workspace=ws)
    assert torch.equal(o1, o2)
