"""Checks that pin the oracle to facts other than itself.

Each ``check_*`` takes the implementation under test as arguments, so the same
check runs on the real oracle (tests/test_oracle.py) and on copies of it with
a planted mistake (tests/test_oracle_mutations.py), where it must fail.
Every check raises AssertionError on a mismatch.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from oracle import brute


def rng(seed=0):
    return np.random.default_rng(seed)


def bf16_values(a):
    """float64 array holding bf16-representable values (RNE via torch, a library routine)."""
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


# ------------------------------------------------------------------ scores

def check_scores(token_scores):
    r = rng(1)
    x = bf16_values(r.standard_normal((48, 96)))
    # identical tokens -> 0
    assert np.all(token_scores(x, x) == 0.0)
    # doubling every element (exact in bf16) -> relative change exactly 1
    assert np.all(token_scores(2.0 * x, x) == 1.0)
    # x_cur = -x_ref -> sum|2r| / sum|r| = 2 exactly
    assert np.all(token_scores(-x, x) == 2.0)
    # a power-of-two rescale of both inputs leaves the relative score bit-identical
    y = bf16_values(x + 0.3 * r.standard_normal(x.shape))
    assert np.array_equal(token_scores(y, x), token_scores(8.0 * y, 8.0 * x))
    # absolute mode scales with the data
    assert np.allclose(token_scores(8.0 * y, 8.0 * x, relative=False), 8.0 * token_scores(y, x, relative=False))
    # zero reference rows: 0/0 -> 0, x/0 -> inf
    z = np.zeros((2, 96))
    s = token_scores(np.stack([np.zeros(96), np.ones(96)]), z)
    assert s[0] == 0.0 and math.isinf(s[1])
    # one planted change of size c in one element of row 5
    u = x.copy()
    u[5, 7] += 0.5
    expect = abs(u[5, 7] - x[5, 7]) / np.abs(x[5]).sum()
    s = token_scores(u, x)
    assert abs(s[5] - expect) <= 1e-15 * expect and np.all(np.delete(s, 5) == 0.0)
    # inter-frame mode: reference is the row hw earlier, first frame is +inf
    hw = 12
    s = token_scores(y, None, hw)
    assert np.all(np.isinf(s[:hw]))
    expect = [math.fsum(abs(a - b) for a, b in zip(y[i], y[i - hw])) / math.fsum(abs(b) for b in y[i - hw])
              for i in range(hw, y.shape[0])]
    assert np.allclose(s[hw:], expect, rtol=1e-14, atol=0)
    # brute force
    bs = brute.scores(y.tolist(), x.tolist())
    assert np.allclose(token_scores(y, x), bs, rtol=1e-14, atol=0)


# ------------------------------------------------------------------ select

def check_topk(select_topk):
    r = rng(2)
    s = r.random(64)
    s[[3, 17, 40]] = 0.5  # planted ties
    s[[8, 9]] = np.inf
    for k in (0, 1, 2, 5, 20, 63, 64):
        m = select_topk(s, k)
        assert m.dtype == bool and m.sum() == k
        assert np.array_equal(m, np.array(brute.topk(s.tolist(), k)))
        if 0 < k < 64:
            assert s[m].min() >= s[~m].max()
    # ties are taken in ascending token order
    eq = np.full(10, 0.25)
    assert np.array_equal(np.flatnonzero(select_topk(eq, 4)), [0, 1, 2, 3])
    tie = np.array([0.1, 0.5, 0.5, 0.9, 0.5, 0.2])
    assert np.array_equal(np.flatnonzero(select_topk(tie, 3)), [1, 2, 3])


def check_threshold(select_threshold):
    s = np.array([0.0, 0.1, 0.2, 0.2, 0.3, np.inf])
    assert np.array_equal(select_threshold(s, 0.2), [False, False, True, True, True, True])
    assert not select_threshold(np.zeros(5), 1e-9).any()


def check_compact(compact):
    r = rng(3)
    for n in (0, 1, 63, 200):
        m = r.random(n) < 0.3
        idx, pidx = compact(m)
        bi, bp = brute.compact(m.tolist())
        assert list(idx) == bi and list(pidx) == bp
        assert np.array_equal(np.sort(np.concatenate([idx, pidx])), np.arange(n))


def check_periods(assign_periods, schedule_mask, golden_rows):
    # rank groups: 25% / 25% / 50% with periods 1 / 2 / 4
    r = rng(4)
    n = 64
    s = r.random(n)
    s[[5, 6]] = 0.7
    per = assign_periods(s, (16, 16, 32), (1, 2, 4))
    assert list(per) == brute.periods_by_rank(s.tolist(), (16, 16, 32), (1, 2, 4))
    # the golden schedule table (budget, period, activity per step)
    for budget, period, acts in golden_rows:
        for i, a in enumerate(acts):
            assert bool(schedule_mask(np.array([period]), i)[0]) == bool(a), (budget, i)
    # closed-form per-step counts on a 25/25/50 split of N
    n = 32760
    periods = np.repeat([1, 2, 4], [n // 4, n // 4, n // 2])
    counts = [int(schedule_mask(periods, i).sum()) for i in range(8)]
    assert counts == [n, n // 4, n // 2, n // 4, n, n // 4, n // 2, n // 4]
    assert sum(counts) == 4 * n


# ---------------------------------------------------------------- recovery

def check_recover(recover_rows):
    r = rng(5)
    x0 = bf16_values(r.standard_normal((30, 16)))
    eps = bf16_values(r.standard_normal((40, 16)))
    rows = np.array([10, 11, 25, 39])
    off = 10
    # sigma = 0 -> exact clean copy of the previous-frame row; sigma = 1 -> exactly the fresh noise
    assert np.array_equal(recover_rows(x0, eps, rows, off, 0.0), x0[rows - off])
    assert np.array_equal(recover_rows(x0, eps, rows, off, 1.0), eps[rows])
    got = recover_rows(x0, eps, rows, off, 0.6)
    want = brute.recover(x0.tolist(), eps.tolist(), rows.tolist(), off, 0.6)
    assert np.array_equal(got, np.array(want))
    # a row with no previous frame keeps only the noise term
    got = recover_rows(x0, eps, np.array([3]), off, 0.5)
    assert np.array_equal(got, np.array(brute.recover(x0.tolist(), eps.tolist(), [3], off, 0.5)))


# -------------------------------------------------------------- projection

def check_project(project):
    r = rng(6)
    d = 32
    x = bf16_values(r.standard_normal((20, d)))
    perm = r.permutation(d)
    w = np.zeros((3 * d, d))
    w[:d] = np.eye(d)
    w[d:2 * d] = 2.0 * np.eye(d)
    w[2 * d + np.arange(d), perm] = 1.0  # row j of W_v picks input column perm[j]
    p = project(x, w, "qkv")
    assert np.array_equal(p["q"], x)
    assert np.array_equal(p["k"], 2.0 * x)
    assert np.array_equal(p["v"], x[:, perm])
    # a general weight vs pure-Python brute force (same storage rounding)
    w = bf16_values(r.standard_normal((3 * d, d)) / math.sqrt(d))
    p = project(x, w, "qkv")
    for part in "qkv":
        assert np.array_equal(p[part], np.array(brute.project(x.tolist(), w.tolist(), part))), part


# --------------------------------------------------------------- attention

def sdpa64(q, k, v, heads):
    """torch's scaled_dot_product_attention in float64 on the CPU (a library routine)."""
    n_q, dim = q.shape
    d = dim // heads
    tq = torch.from_numpy(q).reshape(n_q, heads, d).permute(1, 0, 2)
    tk = torch.from_numpy(k).reshape(k.shape[0], heads, d).permute(1, 0, 2)
    tv = torch.from_numpy(v).reshape(v.shape[0], heads, d).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    return o.permute(1, 0, 2).reshape(n_q, dim).numpy()


def check_attention(attention):
    r = rng(7)
    heads, d = 3, 16
    dim = heads * d
    q = bf16_values(r.standard_normal((37, dim)))
    k = bf16_values(r.standard_normal((53, dim)))
    v = bf16_values(r.standard_normal((53, dim)))
    o = attention(q, k, v, heads)
    assert np.allclose(o, sdpa64(q, k, v, heads), rtol=1e-12, atol=1e-12)
    # value rows all equal c -> output c (rows of softmax sum to one)
    c = r.standard_normal(dim)
    assert np.allclose(attention(q, k, np.tile(c, (53, 1)), heads), np.tile(c, (37, 1)), rtol=0, atol=1e-12)
    # all key rows equal -> uniform weights -> column mean of V
    ke = np.tile(k[0], (53, 1))
    assert np.allclose(attention(q, ke, v, heads), np.tile(v.mean(0), (37, 1)), rtol=0, atol=1e-12)
    # one-hot value columns expose the softmax matrix of head 0: rows sum to 1
    v1 = np.zeros((53, dim))
    v1[np.arange(d), np.arange(d)] = 1.0
    p = attention(q, k, v1, heads)[:, :d]
    s = (q[:, :d] @ k[:d, :d].T) / math.sqrt(d)
    full = (q[:, :d] @ k[:, :d].T) / math.sqrt(d)
    expect = np.exp(s - full.max(1, keepdims=True)) / np.exp(full - full.max(1, keepdims=True)).sum(1, keepdims=True)
    assert np.allclose(p, expect, rtol=1e-12, atol=1e-14)
    _, lse = attention(q, k, v, heads, return_lse=True)
    for h in range(heads):
        sh = (q[:, h * d:(h + 1) * d] @ k[:, h * d:(h + 1) * d].T) / math.sqrt(d)
        mx = sh.max(1)
        assert np.allclose(lse[h], mx + np.log(np.exp(sh - mx[:, None]).sum(1)), rtol=1e-13, atol=1e-13)
    # permutation equivariance: no positional term
    pk = r.permutation(53)
    pq = r.permutation(37)
    assert np.allclose(attention(q[pq], k[pk], v[pk], heads), o[pq], rtol=1e-12, atol=1e-12)
    # brute force on a tiny case
    qs, ks, vs = q[:5], k[:9], v[:9]
    assert np.allclose(attention(qs, ks, vs, heads), brute.attention(qs.tolist(), ks.tolist(), vs.tolist(), heads),
                       rtol=1e-12, atol=1e-13)


# ------------------------------------------------------ f1: cached Euler update

def check_euler(euler_update):
    r = rng(11)
    x = r.standard_normal((7, 24)).astype(np.float32).astype(np.float64)
    v = bf16_values(r.standard_normal((7, 24)))
    # no step or no velocity: the state is unchanged, bit for bit
    assert np.array_equal(euler_update(x, v, 0.0), x)
    assert np.array_equal(euler_update(x, np.zeros_like(v), -0.125), x)
    # from zero, a power-of-two step scales the velocity exactly
    assert np.array_equal(euler_update(np.zeros_like(x), v, 0.5), 0.5 * v)
    # dt = +-1 reduces to one float32 addition / subtraction (numpy's float32 arithmetic)
    x32, v32 = x.astype(np.float32), v.astype(np.float32)
    assert np.array_equal(euler_update(x, v, 1.0), (x32 + v32).astype(np.float64))
    assert np.array_equal(euler_update(x, v, -1.0), (x32 - v32).astype(np.float64))
    # a general step: the exact value rounded once (pure-Python brute force)
    dt = float(np.float32(-0.1234567))
    assert np.array_equal(euler_update(x, v, dt), np.array(brute.euler(x.tolist(), v.tolist(), dt)))
    # kept exact ('f64'): x + dt * v
    assert np.array_equal(euler_update(x, v, dt, store="f64"), x + dt * v)
    # a bf16 state stores the fp32 result rounded to bf16 (torch's float32 -> bfloat16)
    xb = bf16_values(x)
    f32res = euler_update(xb, v, dt)
    want = torch.from_numpy(f32res.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(euler_update(xb, v, dt, store="bf16"), want)


def check_window(step_is_dense):
    assert [step_is_dense(i, 8, 2) for i in range(8)] == [True, True] + [False] * 4 + [True, True]
    assert not any(step_is_dense(i, 8, 0) for i in range(8))
    assert all(step_is_dense(i, 8, 4) for i in range(8))
    assert [step_is_dense(i, 5, 1) for i in range(5)] == [True, False, False, False, True]


def _hsa_tiny(seed=12, n=20, dim=16, heads=2):
    r = rng(seed)
    x0 = r.standard_normal((n, dim)).astype(np.float32).astype(np.float64)
    w = bf16_values(r.standard_normal((3 * dim, dim)) / np.sqrt(dim))
    periods = r.choice([1, 2, 4], size=n)
    sigmas = [float(np.cos(np.pi * i / 16)) for i in range(9)]  # unequal steps
    return x0, w, heads, periods, sigmas


def check_hsa_run(hsa_run, schedule_mask):
    x0, w, heads, periods, sigmas = _hsa_tiny()
    steps = len(sigmas) - 1
    window = 2
    hist = hsa_run(x0, w, heads, periods, sigmas, window)
    bh = brute.hsa_run(x0.tolist(), w.tolist(), heads, periods.tolist(), sigmas, window)
    for i, (a, b) in enumerate(zip(hist, bh)):
        assert list(a["idx"]) == b["idx"], i
        assert np.allclose(a["v_hat"], np.array(b["v_hat"]), rtol=1e-12, atol=1e-12), i
        # float32 states: equal up to a rounding flip caused by last-bit differences of v_hat
        assert np.allclose(a["x"], np.array(b["x"]), rtol=2.0 ** -23, atol=1e-12), i
    n = x0.shape[0]
    prev = None
    for i, h in enumerate(hist):
        # active set: everyone in the window, the period schedule in between
        want = np.arange(n) if i < window or i >= steps - window else np.flatnonzero(schedule_mask(periods, i))
        assert np.array_equal(h["idx"], want), i
        # skipped tokens keep the velocity of their last active step, bit for bit
        if prev is not None:
            skipped = np.setdiff1d(np.arange(n), h["idx"])
            assert np.array_equal(h["v_hat"][skipped], prev["v_hat"][skipped]), i
        prev = h
    # exact state: the displacement telescopes to sum_i (sigma_{i+1} - sigma_i) v_hat_i
    hx = hsa_run(x0, w, heads, periods, sigmas, window, store="f64")
    disp = sum(float(np.float32(sigmas[i + 1] - sigmas[i])) * hx[i]["v_hat"] for i in range(steps))
    assert np.allclose(hx[-1]["x"] - x0, disp, rtol=0, atol=1e-12)
    # a window covering every step makes every step dense
    assert all(h["idx"].size == n for h in hsa_run(x0, w, heads, periods, sigmas, steps // 2))


# ------------------------------- f2: long/short-term pruning mask, restoration

def _drift_clip(frames=10, hw=3, d=8):
    """Location 0 static, location 1 drifting by a fixed exact step per frame, location 2 random."""
    r = rng(13)
    base = bf16_values(r.standard_normal((hw, d)))
    step = np.full(d, 2.0 ** -6)
    x = np.zeros((frames, hw, d))
    for f in range(frames):
        x[f, 0] = base[0]
        x[f, 1] = base[1] + f * step
        x[f, 2] = bf16_values(r.standard_normal(d))
    return x.reshape(frames * hw, d), float(np.abs(step).sum())


def check_lif_mask(lif_mask, token_scores, select_threshold):
    frames, hw = 10, 3
    x, c = _drift_clip(frames, hw)
    # strict comparison: thresholds of 0 keep everything; infinite thresholds keep frame 0 only
    assert lif_mask(x, frames, hw, 0.0, 0.0)["mask"].all()
    m = lif_mask(x, frames, hw, np.inf, np.inf)["mask"].reshape(frames, hw)
    assert m[0].all() and not m[1:].any()
    # slow drift below the per-frame threshold: the long-term change forces a refresh every
    # ceil(tau_long / c) frames; the static location is never refreshed
    res = lif_mask(x, frames, hw, 1.5 * c, 2.5 * c)
    m = res["mask"].reshape(frames, hw)
    assert list(np.flatnonzero(m[:, 1])) == [0, 3, 6, 9]
    assert list(np.flatnonzero(m[:, 0])) == [0]
    assert np.allclose(res["short"].reshape(frames, hw)[1:, 1], c, rtol=0, atol=0)
    assert list(res["long"].reshape(frames, hw)[1:4, 1]) == [c, 2 * c, 3 * c]
    # without a long-term limit it is the plain threshold rule on the previous-frame change
    r = rng(14)
    y = bf16_values(r.standard_normal((6 * 5, 12)))
    s = token_scores(y, None, 5, relative=False)
    tau = float(np.median(s[5:]))
    assert np.array_equal(lif_mask(y, 6, 5, tau, np.inf)["mask"], select_threshold(s, tau))
    # brute force, absolute and relative changes
    for rel in (False, True):
        tau_s = float(np.quantile(token_scores(y, None, 5, relative=rel)[5:], 0.6))
        got = lif_mask(y, 6, 5, tau_s, 1.7 * tau_s, relative=rel)["mask"]
        assert list(got) == brute.lif_mask(y.tolist(), 6, 5, tau_s, 1.7 * tau_s, relative=rel)


def check_restore(restore_frames):
    r = rng(15)
    frames, hw, d = 6, 4, 8
    buf = bf16_values(r.standard_normal((frames * hw, d)))
    assert np.array_equal(restore_frames(buf, np.ones(frames * hw, bool), frames, hw), buf)
    only0 = np.zeros(frames * hw, bool)
    only0[:hw] = True
    assert np.array_equal(restore_frames(buf, only0, frames, hw), np.tile(buf[:hw], (frames, 1)))
    mask = r.random(frames * hw) < 0.5
    mask[:hw] = True
    got = restore_frames(buf, mask, frames, hw)
    assert np.array_equal(got[mask], buf[mask])
    assert np.array_equal(got, np.array(brute.restore(buf.tolist(), mask.tolist(), frames, hw)))


# ------------------------------------ f3: 3D rotary positions, frame-causal attention

def check_rope(rope3d, rope_split, token_position):
    assert rope_split(128) == (44, 42, 42) and rope_split(64) == (24, 20, 20)
    h, w = 3, 5
    f, y, x = token_position(np.array([0, 4, 5, 14, 15, 37]), h, w)
    assert list(f) == [0, 0, 0, 0, 1, 2] and list(y) == [0, 0, 1, 2, 0, 1] and list(x) == [0, 4, 0, 4, 0, 2]
    r = rng(16)
    heads, d = 2, 24
    dt, dy, dx = rope_split(d)
    xrows = r.standard_normal((6, heads * d))
    toks = np.array([0, 7, 15, 16, 44, 59])
    # token 0 sits at the origin: no rotation
    assert np.array_equal(rope3d(xrows[:1], [0], h, w, heads), xrows[:1])
    # closed form: a unit vector on pair i of the width group of head 1, token at column 1
    for i in range(dx // 2):
        e = np.zeros((1, heads * d))
        e[0, d + dt + dy + 2 * i] = 1.0
        got = rope3d(e, [1], h, w, heads, base=100.0)
        phi = 100.0 ** (-2.0 * i / dx)
        want = np.zeros_like(e)
        want[0, d + dt + dy + 2 * i] = np.cos(phi)
        want[0, d + dt + dy + 2 * i + 1] = np.sin(phi)
        assert np.allclose(got, want, rtol=0, atol=1e-15)
    # closed form: pair 0 of the time group turns by the frame index (frequency 1)
    e = np.zeros((1, heads * d))
    e[0, 0] = 1.0
    got = rope3d(e, [2 * h * w], h, w, heads)
    assert np.allclose(got[0, :2], [np.cos(2.0), np.sin(2.0)], rtol=0, atol=1e-15)
    # rotations: every channel pair keeps its length
    out = rope3d(xrows, toks, h, w, heads)
    assert np.allclose(out[:, 0::2] ** 2 + out[:, 1::2] ** 2, xrows[:, 0::2] ** 2 + xrows[:, 1::2] ** 2,
                       rtol=1e-13, atol=0)
    # scores depend only on the offset between the two positions (shift both along each axis)
    q, k = r.standard_normal((1, heads * d)), r.standard_normal((1, heads * d))
    for a, b, shift in ((3, 8, 1), (0, 16, 15), (6, 21, 5)):  # column, row (w), frame (h*w) shifts
        s0 = rope3d(q, [a], h, w, heads) @ rope3d(k, [b], h, w, heads).T
        s1 = rope3d(q, [a + shift], h, w, heads) @ rope3d(k, [b + shift], h, w, heads).T
        assert np.allclose(s0, s1, rtol=1e-12, atol=1e-12)
    # brute force
    assert np.allclose(out, np.array(brute.rope(xrows.tolist(), toks.tolist(), h, w, heads)), rtol=1e-13, atol=1e-13)


def check_project_rope(project_rope, project, rope3d):
    r = rng(17)
    heads, d = 2, 24
    x = bf16_values(r.standard_normal((5, heads * d)))
    w = bf16_values(r.standard_normal((3 * heads * d, heads * d)) / np.sqrt(heads * d))
    toks = np.array([0, 3, 19, 20, 41])
    p = project_rope(x, toks, w, heads, 4, 5)
    plain = project(x, w, "qkv")
    # V is not rotated; a token at the origin is not rotated at all
    assert np.array_equal(p["v"], plain["v"])
    assert np.array_equal(p["q"][0], plain["q"][0]) and np.array_equal(p["k"][0], plain["k"][0])
    # rotation of the exact projection, rounded once
    for name, part in (("q", 0), ("k", 1)):
        exact = x.astype(np.float64) @ w[part * heads * d:(part + 1) * heads * d].T
        want = rope3d(exact, toks, 4, 5, heads)
        assert np.allclose(p[name], want, rtol=2.0 ** -8, atol=1e-12)
        assert np.array_equal(p[name], bf16_values(want))


def check_frame_causal(attention_frame_causal, attention):
    r = rng(18)
    heads, d, ft = 2, 8, 6
    n_kv = 27
    k = r.standard_normal((n_kv, heads * d))
    v = r.standard_normal((n_kv, heads * d))
    toks = np.array([0, 2, 5, 6, 11, 13, 20, 26])
    q = r.standard_normal((toks.size, heads * d))
    out = attention_frame_causal(q, k, v, heads, toks, ft)
    # one frame covering the whole cache: plain attention
    assert np.allclose(attention_frame_causal(q, k, v, heads, toks, n_kv + 5), attention(q, k, v, heads),
                       rtol=1e-14, atol=1e-14)
    # a frame-0 query equals attention over the first frame's keys only; the last frame sees all
    assert np.allclose(out[:3], attention(q[:3], k[:ft], v[:ft], heads), rtol=1e-14, atol=1e-14)
    assert np.allclose(out[-1:], attention(q[-1:], k, v, heads), rtol=1e-14, atol=1e-14)
    # keys of later frames do not matter (change them arbitrarily)
    k2, v2 = k.copy(), v.copy()
    k2[12:] = r.standard_normal(k2[12:].shape) * 5
    v2[12:] = r.standard_normal(v2[12:].shape) * 5
    mid = toks < 12
    assert np.allclose(attention_frame_causal(q[mid], k2, v2, heads, toks[mid], ft), out[mid], rtol=1e-14, atol=1e-14)
    # brute force
    want = brute.attention_frame_causal(q.tolist(), k.tolist(), v.tolist(), heads, toks.tolist(), ft)
    assert np.allclose(out, np.array(want), rtol=1e-12, atol=1e-12)


# --------------------------------------------- f4: Timeripple partial-score reuse

def _grid_pos(n, height, width):
    hw = height * width
    return [(t // hw, (t // width) % height, t % width) for t in range(n)]


def check_reuse(reuse_deltas, reuse_sources, reuse_effective, axis_neighbors, reuse_groups, rope3d):
    assert reuse_groups(128) == [(0, 44), (44, 86), (86, 128)]
    assert reuse_groups(64) == [(0, 24), (24, 44), (44, 64)]
    frames, height, width = 3, 3, 4
    n = frames * height * width
    nb = axis_neighbors(n, height, width)
    for t, (f, y, x) in enumerate(_grid_pos(n, height, width)):
        assert nb[0, t] == (t - height * width if f else -1)
        assert nb[1, t] == (t - width if y else -1)
        assert nb[2, t] == (t - 1 if x else -1)
    r = rng(19)
    heads, d = 2, 12
    groups = reuse_groups(d)
    v = r.standard_normal((n, heads * d))
    v[height * width:] = v[:-height * width] + 0.05 * r.standard_normal((n - height * width, heads * d))
    ident = np.arange(n)[:, None, None]
    # thresholds 0: nothing is reused, the vectors are unchanged
    s0 = reuse_sources(reuse_deltas(v, heads, height, width), (0.0, 0.0, 0.0), height, width)
    assert np.array_equal(s0, np.broadcast_to(ident, s0.shape))
    assert np.array_equal(reuse_effective(v, s0, heads), v)
    # rotary vectors of one content row: moving along an axis leaves the other two groups'
    # channels exactly equal, so every check passes at any positive threshold; the sources
    # follow the axis order and the effective vectors equal the originals
    u = np.repeat(r.standard_normal((1, heads * d)), n, axis=0)
    rv = rope3d(u, np.arange(n), height, width, heads)
    dr = reuse_deltas(rv, heads, height, width)
    for t, (f, y, x) in enumerate(_grid_pos(n, height, width)):
        for a, has in enumerate((f > 0, y > 0, x > 0)):
            assert (dr[t, :, a] == 0.0).all() if has else np.isinf(dr[t, :, a]).all()
    sr = reuse_sources(dr, (1e-12, 1e-12, 1e-12), height, width)
    for t, (f, y, x) in enumerate(_grid_pos(n, height, width)):
        back = (t - height * width if f else None, t - width if y else None, t - 1 if x else None)
        for g in range(3):
            want = next((back[a] for a in range(3) if a != g and back[a] is not None), t)
            assert (sr[t, :, g] == want).all(), (t, g)
    assert np.array_equal(reuse_effective(rv, sr, heads), rv)
    # every check passing: chains end at the frame's first token (time group), the first token
    # of the row in frame 0 (height group) and of the column in frame 0 (width group)
    sinf = reuse_sources(reuse_deltas(v, heads, height, width), (np.inf,) * 3, height, width)
    eff = reuse_effective(v, sinf, heads)
    for t, (f, y, x) in enumerate(_grid_pos(n, height, width)):
        roots = (f * height * width, y * width, x)
        for h in range(heads):
            for g, (s, e) in enumerate(groups):
                assert np.array_equal(eff[t, h * d + s:h * d + e], v[roots[g], h * d + s:h * d + e])
    # the threshold is strict: a relative difference of exactly 0.5 is not below 0.5
    w2 = np.zeros((2 * 1 * 1, d))
    w2[0, groups[1][0]] = 1.0
    w2[1, groups[1][0]] = 2.0  # |2 - 1| / |2| = 0.5 over the height and width groups
    d2 = reuse_deltas(w2, 1, 1, 1)
    assert d2[1, 0, 0] == 0.5
    assert (reuse_sources(d2, (0.5, 0.0, 0.0), 1, 1)[1, 0] == 1).all()
    assert list(reuse_sources(d2, (0.5000001, 0.0, 0.0), 1, 1)[1, 0]) == [1, 0, 0]
    # relative: a power-of-two rescale leaves every difference and decision unchanged
    dv = reuse_deltas(v, heads, height, width)
    assert np.array_equal(reuse_deltas(v * 2.0 ** 9, heads, height, width), dv)
    th = (0.3, 1.2, 0.9)
    sv = reuse_sources(dv, th, height, width)
    assert np.array_equal(reuse_sources(reuse_deltas(v * 2.0 ** -7, heads, height, width), th, height, width), sv)
    assert 0 < (sv != ident).mean() < 1
    # brute force
    bs, be = brute.reuse(v.tolist(), heads, height, width, th)
    assert np.array_equal(sv, np.array(bs))
    assert np.array_equal(reuse_effective(v, sv, heads), np.array(be))


def check_timeripple_attention(timeripple_attention, attention, rope3d):
    r = rng(20)
    frames, height, width, heads, d = 2, 3, 3, 2, 12
    n = frames * height * width
    q = r.standard_normal((n, heads * d))
    k = r.standard_normal((n, heads * d))
    v = r.standard_normal((n, heads * d))
    zero = (0.0, 0.0, 0.0)
    # no reuse: plain attention
    res = timeripple_attention(q, k, v, heads, height, width, zero, zero)
    assert np.allclose(res["out"], attention(q, k, v, heads), rtol=1e-14, atol=1e-14)
    # the output is the attention of the effective vectors, each side reused independently
    th = (0.9, 1.3, 1.1)
    res = timeripple_attention(q, k, v, heads, height, width, th, zero)
    assert np.array_equal(res["k_eff"], k) and not np.array_equal(res["q_eff"], q)
    assert np.allclose(res["out"], attention(res["q_eff"], k, v, heads), rtol=1e-14, atol=1e-14)
    res = timeripple_attention(q, k, v, heads, height, width, zero, th)
    assert np.array_equal(res["q_eff"], q) and not np.array_equal(res["k_eff"], k)
    assert np.allclose(res["out"], attention(q, res["k_eff"], v, heads), rtol=1e-14, atol=1e-14)
    # rotary keys of one content row are reproduced exactly by any reuse: output unchanged
    kr = rope3d(np.repeat(k[:1], n, axis=0), np.arange(n), height, width, heads)
    res = timeripple_attention(q, kr, v, heads, height, width, zero, (1e-9, 1e-9, 1e-9))
    assert np.array_equal(res["k_eff"], kr) and (res["src_k"] != np.arange(n)[:, None, None]).any()
    assert np.allclose(res["out"], attention(q, kr, v, heads), rtol=1e-14, atol=1e-14)
