"""Property-based agreement of the numpy oracle with the pure-Python brute force over many
small random shapes (hypothesis, derandomized so the suite is reproducible): the two share
no code, so a slip in either -- an axis, an offset, a tie order, a rounding point -- shows
up as a disagreement on some shape.  Values are bf16-exact draws, ties and zero rows are
planted on purpose."""

from __future__ import annotations

import math

import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import brute
from oracle import reference as ref

SETTINGS = settings(max_examples=150, deadline=None, derandomize=True, database=None)


def _rows(seed, n, d, scale=1.0, zero_rows=()):
    r = np.random.default_rng(seed)
    x = ref.round_bf16(scale * r.standard_normal((n, d)))
    for i in zero_rows:
        if i < n:
            x[i] = 0.0
    return x


@SETTINGS
@given(seed=st.integers(0, 10 ** 6), n=st.integers(1, 24), d=st.sampled_from([4, 8, 16]),
       off=st.integers(0, 6), relative=st.booleans())
def test_scores(seed, n, d, off, relative):
    x = _rows(seed, n, d, zero_rows=(1,))
    y = ref.round_bf16(x + 0.25 * np.random.default_rng(seed + 1).standard_normal(x.shape))
    y[min(2, n - 1)] = x[min(2, n - 1)]  # an unchanged token
    got = ref.token_scores(y, x, relative=relative)
    want = brute.scores(y.tolist(), x.tolist(), relative=relative)
    assert np.allclose(got, want, rtol=1e-12, atol=0.0, equal_nan=False)
    got = ref.token_scores(y, None, off, relative=relative)
    want = brute.scores(y.tolist(), None, relative=relative, ref_row_offset=off)
    assert np.array_equal(np.isinf(got), np.isinf(want))
    fin = ~np.isinf(got)
    assert np.allclose(got[fin], np.asarray(want)[fin], rtol=1e-12, atol=0.0)


@SETTINGS
@given(seed=st.integers(0, 10 ** 6), n=st.integers(1, 40), levels=st.integers(1, 6), kfrac=st.floats(0, 1))
def test_topk_and_compact(seed, n, levels, kfrac):
    # few distinct values: many ties, taken in ascending token order
    s = np.random.default_rng(seed).integers(0, levels, n).astype(np.float64) / levels
    k = int(round(kfrac * n))
    m = ref.select_topk(s, k)
    assert np.array_equal(m, np.array(brute.topk(s.tolist(), k)))
    idx, pidx = ref.compact(m)
    bi, bp = brute.compact(m.tolist())
    assert idx.tolist() == bi and pidx.tolist() == bp


@SETTINGS
@given(seed=st.integers(0, 10 ** 6), nq=st.integers(1, 9), nk=st.integers(1, 12), heads=st.sampled_from([1, 2, 3]),
       d=st.sampled_from([2, 4, 8]), scale=st.sampled_from([0.5, 1.0, 3.0]))
def test_attention(seed, nq, nk, heads, d, scale):
    dim = heads * d
    q = _rows(seed, nq, dim, scale)
    k = _rows(seed + 1, nk, dim, scale)
    v = _rows(seed + 2, nk, dim)
    got = ref.attention(q, k, v, heads)
    want = np.array(brute.attention(q.tolist(), k.tolist(), v.tolist(), heads))
    assert np.allclose(got, want, rtol=1e-10, atol=1e-12)


@SETTINGS
@given(seed=st.integers(0, 10 ** 6), frames=st.integers(1, 5), hw=st.integers(1, 4), d=st.sampled_from([4, 8]),
       drift=st.sampled_from([0.0, 0.02, 0.3]), relative=st.booleans())
def test_lif_mask_and_restore(seed, frames, hw, d, drift, relative):
    r = np.random.default_rng(seed)
    base = r.standard_normal((hw, d))
    rows = [base]
    for _ in range(1, frames):
        rows.append(rows[-1] + drift * r.standard_normal((hw, d)))
    x = ref.round_bf16(np.concatenate(rows))
    tau_s, tau_l = (0.1, 0.25) if relative else (0.3, 0.8)
    got = ref.lif_mask(x, frames, hw, tau_s, tau_l, relative=relative)["mask"]
    want = brute.lif_mask(x.tolist(), frames, hw, tau_s, tau_l, relative=relative)
    assert got.tolist() == want
    buf = _rows(seed + 3, frames * hw, d)
    assert np.array_equal(ref.restore_frames(buf, got, frames, hw),
                          np.array(brute.restore(buf.tolist(), got.tolist(), frames, hw)))


@SETTINGS
@given(seed=st.integers(0, 10 ** 6), frames=st.integers(1, 3), height=st.integers(1, 3), width=st.integers(1, 3),
       heads=st.sampled_from([1, 2]), theta=st.sampled_from([0.0, 0.05, 0.3, math.inf]))
def test_reuse(seed, frames, height, width, heads, theta):
    d = 12
    n = frames * height * width
    r = np.random.default_rng(seed)
    content = np.repeat(r.standard_normal((1, heads * d)), n, axis=0) + 0.05 * r.standard_normal((n, heads * d))
    v = ref.round_bf16(ref.rope3d(content, np.arange(n), height, width, heads))
    thetas = (theta, theta, theta)
    src = ref.reuse_sources(ref.reuse_deltas(v, heads, height, width), thetas, height, width)
    eff = ref.reuse_effective(v, src, heads)
    bsrc, beff = brute.reuse(v.tolist(), heads, height, width, thetas)
    assert np.array_equal(src, np.array(bsrc)) and np.array_equal(eff, np.array(beff))
