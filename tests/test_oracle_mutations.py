"""Planted mistakes in copies of the oracle must fail the pins (the pins are not vacuous)."""

from __future__ import annotations

import numpy as np
import pytest

import pins
from oracle import reference as ref
from test_oracle import load_golden_schedule


def _fails(check, *args):
    with pytest.raises(AssertionError):
        check(*args)


# ------------------------------------------------------------------ scores

def _scores_wrong_denominator(x_cur, x_ref=None, ref_row_offset=0, relative=True):
    s = ref.token_scores(x_cur, x_ref, ref_row_offset, relative=False)
    if not relative:
        return s
    x_cur = np.asarray(x_cur, np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        return s / np.abs(x_cur).sum(1)  # divides by the current row instead of the reference


def _scores_no_abs(x_cur, x_ref=None, ref_row_offset=0, relative=True):
    x_cur = np.asarray(x_cur, np.float64)
    r = x_cur if x_ref is None else np.asarray(x_ref, np.float64)
    out = np.full(x_cur.shape[0], np.inf)
    rows = np.arange(ref_row_offset, x_cur.shape[0])
    num = (x_cur[rows] - r[rows - ref_row_offset]).sum(1)  # dropped |.|
    den = np.abs(r[rows - ref_row_offset]).sum(1)
    with np.errstate(divide="ignore", invalid="ignore"):
        out[rows] = np.where(den == 0, np.where(num == 0, 0.0, np.inf), num / den) if relative else num
    return out


def _scores_wrong_offset(x_cur, x_ref=None, ref_row_offset=0, relative=True):
    return ref.token_scores(x_cur, x_ref, max(ref_row_offset - 1, 0), relative)


@pytest.mark.parametrize("bad", [_scores_wrong_denominator, _scores_no_abs, _scores_wrong_offset])
def test_score_mutations_caught(bad):
    _fails(pins.check_scores, bad)


# ------------------------------------------------------------------ select

def _topk_ties_descending(scores, k):
    n = len(scores)
    order = np.lexsort((-np.arange(n), -np.asarray(scores)))
    m = np.zeros(n, bool)
    m[order[:k]] = True
    return m


def _topk_lowest(scores, k):
    n = len(scores)
    order = np.lexsort((np.arange(n), np.asarray(scores)))
    m = np.zeros(n, bool)
    m[order[:k]] = True
    return m


@pytest.mark.parametrize("bad", [_topk_ties_descending, _topk_lowest])
def test_topk_mutations_caught(bad):
    _fails(pins.check_topk, bad)


def test_threshold_strict_caught():
    _fails(pins.check_threshold, lambda s, tau: np.asarray(s) > tau)


def test_compact_mutation_caught():
    def bad(mask):
        idx, pidx = ref.compact(mask)
        return idx[::-1], pidx  # descending order
    _fails(pins.check_compact, bad)


def test_schedule_mutations_caught(root):
    golden = load_golden_schedule(root)
    _fails(pins.check_periods, ref.assign_periods, lambda p, i: ((i + 1) % np.asarray(p)) == 0, golden)

    def periods_ascending(scores, counts, periods):
        return ref.assign_periods(-np.asarray(scores), counts, periods)
    _fails(pins.check_periods, periods_ascending, ref.schedule_mask, golden)


# ---------------------------------------------------------------- recovery

def test_recovery_mutations_caught():
    def swapped(x0, eps, rows, off, sigma):
        return ref.recover_rows(x0, eps, rows, off, 1.0 - sigma)
    _fails(pins.check_recover, swapped)

    def no_offset(x0, eps, rows, off, sigma):
        return ref.recover_rows(x0, eps, rows, 0, sigma)
    _fails(pins.check_recover, no_offset)


# -------------------------------------------------------------- projection

def test_projection_mutations_caught():
    def untransposed(x_rows, w_qkv, parts="qkv"):
        x = ref.round_bf16(np.asarray(x_rows, np.float64))
        d = w_qkv.shape[1]
        return {n: ref.round_bf16(x @ w_qkv[i * d:(i + 1) * d]) for i, n in enumerate("qkv") if n in parts}
    _fails(pins.check_project, untransposed)

    def unrounded(x_rows, w_qkv, parts="qkv"):
        x = np.asarray(x_rows, np.float64)
        d = w_qkv.shape[1]
        return {n: x @ w_qkv[i * d:(i + 1) * d].T for i, n in enumerate("qkv") if n in parts}
    _fails(pins.check_project, unrounded)

    def kv_swapped(x_rows, w_qkv, parts="qkv"):
        p = ref.project(x_rows, w_qkv, "qkv")
        p["k"], p["v"] = p["v"], p["k"]
        return {n: p[n] for n in parts}
    _fails(pins.check_project, kv_swapped)


# --------------------------------------------------------------- attention

def _attn_no_scale(q, k, v, heads, scale=None, block=256, return_lse=False):
    return ref.attention(q, k, v, heads, scale=1.0, block=block, return_lse=return_lse)


def _attn_head0_keys(q, k, v, heads, scale=None, block=256, return_lse=False):
    d = q.shape[1] // heads
    k2 = np.tile(np.asarray(k)[:, :d], (1, heads))  # every head uses head 0's keys
    return ref.attention(q, k2, v, heads, scale, block, return_lse)


def _attn_softmax_wrong_axis(q, k, v, heads, scale=None, block=256, return_lse=False):
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    d = q.shape[1] // heads
    out = np.zeros_like(q)
    lse = np.zeros((heads, q.shape[0]))
    for h in range(heads):
        c = slice(h * d, (h + 1) * d)
        s = q[:, c] @ k[:, c].T / np.sqrt(d)
        p = np.exp(s - s.max(0, keepdims=True))
        p /= p.sum(0, keepdims=True)  # normalised over queries instead of keys
        out[:, c] = p @ v[:, c]
        lse[h] = np.log(np.exp(s).sum(1))
    return (out, lse) if return_lse else out


def _attn_no_max_shift_lse(q, k, v, heads, scale=None, block=256, return_lse=False):
    out, lse = ref.attention(q, k, v, heads, scale, block, True)
    return (out, lse - 1.0) if return_lse else out


@pytest.mark.parametrize("bad", [_attn_no_scale, _attn_head0_keys, _attn_softmax_wrong_axis, _attn_no_max_shift_lse])
def test_attention_mutations_caught(bad):
    _fails(pins.check_attention, bad)


# ------------------------------------------------ f1: Euler update and loop

def _euler_wrong_sign(x, v_hat, dt, store="f32"):
    return ref.euler_update(x, v_hat, -dt, store)


def _euler_no_rounding(x, v_hat, dt, store="f32"):
    return ref.euler_update(x, v_hat, dt, "f64")


@pytest.mark.parametrize("bad", [_euler_wrong_sign, _euler_no_rounding])
def test_euler_mutations_caught(bad):
    _fails(pins.check_euler, bad)


def test_window_off_by_one_caught():
    _fails(pins.check_window, lambda i, steps, window: i <= window or i >= steps - window)


def _hsa_with(**patch):
    """hsa_run with one of its steps replaced (a planted mistake)."""
    def run(x0, w, heads, periods, sigmas, window, store="f32"):
        saved = {k: getattr(ref, k) for k in patch}
        try:
            for k, f in patch.items():
                setattr(ref, k, f)
            return ref.hsa_run(x0, w, heads, periods, sigmas, window, store)
        finally:
            for k, f in saved.items():
                setattr(ref, k, f)
    return run


def _dt_previous_interval(sigmas, step):
    return float(np.float32(float(sigmas[max(step, 1)]) - float(sigmas[max(step, 1) - 1])))


def _layer_step_forgets_velocity(x_cur, w_qkv, heads, k_cache, v_cache, out, **kw):
    out[:] = 0.0  # skipped tokens lose their cached velocity
    return _orig_layer_step(x_cur, w_qkv, heads, k_cache, v_cache, out, **kw)


_orig_layer_step = ref.layer_step


@pytest.mark.parametrize("patch", [
    {"euler_dt": _dt_previous_interval},
    {"layer_step": _layer_step_forgets_velocity},
    {"step_is_dense": lambda i, steps, window: i < window},
])
def test_hsa_run_mutations_caught(patch):
    _fails(pins.check_hsa_run, _hsa_with(**patch), ref.schedule_mask)


# ----------------------------------- f2: long/short-term mask, restoration

def _lif_previous_frame_only(x, frames, hw, tau_short, tau_long, relative=False):
    """long-term reference taken as the previous frame (no tracking of the last kept frame)"""
    s = ref.token_scores(x, None, hw, relative=relative)
    keep = ~((s < tau_short) & (s < tau_long))
    keep[:hw] = True
    return {"mask": keep, "short": s, "long": s}


def _lif_not_strict(x, frames, hw, tau_short, tau_long, relative=False):
    return ref.lif_mask(x, frames, hw, np.nextafter(tau_short, np.inf), np.nextafter(tau_long, np.inf),
                        relative)


@pytest.mark.parametrize("bad", [_lif_previous_frame_only, _lif_not_strict])
def test_lif_mask_mutations_caught(bad):
    _fails(pins.check_lif_mask, bad, ref.token_scores, ref.select_threshold)


def _restore_from_original(buf, mask, frames, hw):
    """copies the previous frame's original row instead of its restored value"""
    b = np.array(buf, dtype=np.float64).reshape(frames, hw, -1)
    src = b.copy()
    m = np.asarray(mask, bool).reshape(frames, hw)
    for f in range(1, frames):
        b[f, ~m[f]] = src[f - 1, ~m[f]]
    return b.reshape(frames * hw, -1)


def test_restore_mutation_caught():
    _fails(pins.check_restore, _restore_from_original)


# ------------------------------------ f3: rotary positions, frame-causal attention

def _rope_generic(x_rows, tokens, height, width, heads, base=10000.0, sign=1.0, halves=False, swap_xy=False):
    x = np.asarray(x_rows, dtype=np.float64)
    d = x.shape[1] // heads
    d_t, d_y, d_x = ref.rope_split(d)
    f, y, xx = ref.token_position(tokens, height, width)
    if swap_xy:
        y, xx = xx, y
    out = x.copy()
    for h in range(heads):
        for off, d_a, pos in ((0, d_t, f), (d_t, d_y, y), (d_t + d_y, d_x, xx)):
            i = np.arange(d_a // 2)
            ang = pos[:, None] * (base ** (-2.0 * i / d_a))[None, :]
            c, s = np.cos(ang), sign * np.sin(ang)
            ev = h * d + off + (i if halves else 2 * i)
            od = ev + (d_a // 2 if halves else 1)
            a, b = x[:, ev], x[:, od]
            out[:, ev] = a * c - b * s
            out[:, od] = a * s + b * c
    return out


@pytest.mark.parametrize("kw", [{"sign": -1.0}, {"halves": True}, {"swap_xy": True}])
def test_rope_mutations_caught(kw):
    _fails(pins.check_rope, lambda *a, **k: _rope_generic(*a, **{**k, **kw}), ref.rope_split, ref.token_position)


def test_project_rope_mutation_caught():
    def rotate_after_rounding(x_rows, tokens, w_qkv, heads, height, width, base=10000.0, parts="qkv"):
        p = ref.project(x_rows, w_qkv, parts)
        return {n: (ref.round_bf16(ref.rope3d(p[n], tokens, height, width, heads, base)) if n in "qk" else p[n])
                for n in p}
    _fails(pins.check_project_rope, rotate_after_rounding, ref.project, ref.rope3d)


def _causal_shifted(shift):
    def run(q, k, v, heads, q_tokens, frame_tokens, scale=None, return_lse=False):
        frames = np.asarray(q_tokens) // frame_tokens
        out = np.zeros_like(np.asarray(q, np.float64))
        for f in np.unique(frames):
            rows = np.flatnonzero(frames == f)
            lim = max(1, min(len(k), (int(f) + 1 + shift) * frame_tokens))
            out[rows] = ref.attention(np.asarray(q)[rows], np.asarray(k)[:lim], np.asarray(v)[:lim], heads, scale)
        return out
    return run


@pytest.mark.parametrize("shift", [1, -1])
def test_frame_causal_mutations_caught(shift):
    _fails(pins.check_frame_causal, _causal_shifted(shift), ref.attention)


# ------------------------------------------- f4: Timeripple partial-score reuse

def _deltas_generic(v, heads, height, width, all_channels=False, absolute=False, neighbour_den=False,
                    swap_xy=False):
    v = np.asarray(v, np.float64)
    n, dim = v.shape
    d = dim // heads
    groups = ref.reuse_groups(d)
    nb = ref.axis_neighbors(n, height, width)
    if swap_xy:
        nb = nb[[0, 2, 1]]
    out = np.full((n, heads, 3), np.inf)
    for a in range(3):
        chans = np.concatenate([np.arange(s, e) for g, (s, e) in enumerate(groups) if all_channels or g != a])
        rows = np.flatnonzero(nb[a] >= 0)
        for h in range(heads):
            cols = h * d + chans
            own = v[np.ix_(rows, cols)]
            other = v[np.ix_(nb[a, rows], cols)]
            num = np.sqrt(((own - other) ** 2).sum(1))
            den = np.sqrt(((other if neighbour_den else own) ** 2).sum(1))
            with np.errstate(divide="ignore", invalid="ignore"):
                rel = np.where(den == 0, np.where(num == 0, 0.0, np.inf), num / den)
            out[rows, h, a] = num if absolute else rel
    return out


@pytest.mark.parametrize("kw", [{"all_channels": True}, {"absolute": True}, {"neighbour_den": True},
                                {"swap_xy": True}])
def test_reuse_delta_mutations_caught(kw):
    _fails(pins.check_reuse, lambda *a: _deltas_generic(*a, **kw), ref.reuse_sources, ref.reuse_effective,
           ref.axis_neighbors, ref.reuse_groups, ref.rope3d)


def _sources_generic(deltas, thetas, height, width, order=(0, 1, 2), every_axis=False, non_strict=False):
    deltas = np.asarray(deltas, np.float64)
    n, heads, _ = deltas.shape
    nb = ref.axis_neighbors(n, height, width)
    src = np.broadcast_to(np.arange(n)[:, None, None], (n, heads, 3)).copy()
    for g in range(3):
        axes = [a for a in order if a != g]
        passes = [(deltas[:, :, a] <= thetas[a]) if non_strict else (deltas[:, :, a] < thetas[a]) for a in axes]
        if every_axis:
            allp = np.logical_and.reduce(passes)
            src[:, :, g] = np.where(allp, nb[axes[0]][:, None], src[:, :, g])
            continue
        decided = np.zeros((n, heads), dtype=bool)
        for a, ok in zip(axes, passes):
            ok = ok & ~decided
            src[:, :, g] = np.where(ok, nb[a][:, None], src[:, :, g])
            decided |= ok
    return src


@pytest.mark.parametrize("kw", [{"order": (2, 1, 0)}, {"every_axis": True}, {"non_strict": True}])
def test_reuse_source_mutations_caught(kw):
    _fails(pins.check_reuse, ref.reuse_deltas, lambda *a: _sources_generic(*a, **kw), ref.reuse_effective,
           ref.axis_neighbors, ref.reuse_groups, ref.rope3d)


def _effective_from_originals(v, src, heads):
    v = np.asarray(v, np.float64)
    d = v.shape[1] // heads
    eff = v.copy()
    for t in range(v.shape[0]):
        for h in range(heads):
            for g, (s, e) in enumerate(ref.reuse_groups(d)):
                j = int(src[t, h, g])
                eff[t, h * d + s:h * d + e] = v[j, h * d + s:h * d + e]  # the source's own values, not resolved
    return eff


def test_reuse_effective_mutation_caught():
    _fails(pins.check_reuse, ref.reuse_deltas, ref.reuse_sources, _effective_from_originals,
           ref.axis_neighbors, ref.reuse_groups, ref.rope3d)


def test_timeripple_attention_mutation_caught():
    def keys_not_reused(q, k, v, heads, height, width, thetas_q, thetas_k, scale=None):
        res = ref.timeripple_attention(q, k, v, heads, height, width, thetas_q, (0.0, 0.0, 0.0), scale)
        res["src_k"] = ref.reuse_sources(ref.reuse_deltas(k, heads, height, width), thetas_k, height, width)
        return res
    _fails(pins.check_timeripple_attention, keys_not_reused, ref.attention, ref.rope3d)
