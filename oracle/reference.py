"""Plain numpy float64 oracle of the token-pruned attention layer.

TEST INFRASTRUCTURE ONLY (see the package docstring): slow, obviously
correct, one function per step, in the order the method runs them.

Step labels in the section headers: a1 score, a2 select, a3 compact,
a4 gather / recovery rows, a5 projection, a6 cache sync, a7 attention,
a8 scatter; f1 cached Euler update, f2 long/short-term pruning mask and
restoration, f3 3D rotary positions and frame-causal attention, f4
Timeripple partial-score reuse.

Conventions
-----------
* Token rows are row-major ``[N, D]``; inside Q/K/V, column ``h*d + j`` is
  dimension ``j`` of head ``h``.
* ``w_qkv`` is ``[3*D, D]``: rows ``[0, D)`` project to Q, ``[D, 2D)`` to K,
  ``[2D, 3D)`` to V, and ``y = x @ w_part.T``.
* Inputs arrive as float64 arrays holding bf16 (or fp32) values exactly.
  Values the method stores (Q, K, V, recovered rows) are rounded to bf16 at
  the point where they are stored; scores, softmax and outputs stay float64.
"""

from __future__ import annotations

import numpy as np

# Largest finite bfloat16: (2 - 2**-7) * 2**127.
_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16, ties to even (storage rounding).

    bfloat16 keeps 8 significant bits, so a value in [2**(e-1), 2**e) is
    rounded to a multiple of 2**(e-8); below the smallest normal 2**-126 the
    spacing stays 2**-133.  Results beyond the largest finite bf16 become
    +-inf.  Pinned against torch's float32 -> bfloat16 conversion.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x) & (x != 0.0)
    v = x[fin]
    _, e = np.frexp(v)
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(v, -q)), q)
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, r), r)
    out[fin] = r
    return out


# ---------------------------------------------------------------- a1: score

def token_scores(x_cur, x_ref=None, ref_row_offset: int = 0, relative: bool = True) -> np.ndarray:
    """Per-token change score.

    HSA page §2.1 ("Selección Dinámica"): tokens are ranked by the relative L1
    change of each token; LIPAR page §2.B: a latent patch is compared by L1
    norm with the patch at the same spatial location in the previous frame.

    The reference row of token n is ``ref[n - ref_row_offset]`` where ``ref``
    is ``x_ref`` if given, else ``x_cur`` itself (the inter-frame case, with
    the offset equal to one frame's H*W tokens).  Tokens without a reference
    row score +inf (always kept).  Relative score = sum|x - r| / sum|r|, with
    0/0 -> 0 and x/0 -> +inf; ``relative=False`` returns sum|x - r|.
    """
    x_cur = np.asarray(x_cur, dtype=np.float64)
    ref = x_cur if x_ref is None else np.asarray(x_ref, dtype=np.float64)
    n = x_cur.shape[0]
    scores = np.full(n, np.inf)
    rows = np.arange(max(ref_row_offset, 0), min(n, ref.shape[0] + ref_row_offset))
    if rows.size == 0:
        return scores
    r = ref[rows - ref_row_offset]
    num = np.abs(x_cur[rows] - r).sum(axis=1)
    if not relative:
        scores[rows] = num
        return scores
    den = np.abs(r).sum(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = num / den
    s = np.where(den == 0.0, np.where(num == 0.0, 0.0, np.inf), s)
    scores[rows] = s
    return scores


# --------------------------------------------------------------- a2: select

def select_topk(scores, k: int) -> np.ndarray:
    """Mask of the k highest scores; equal scores are taken in ascending token order."""
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    if not 0 <= k <= n:
        raise ValueError("k out of range")
    order = np.lexsort((np.arange(n), -scores))
    mask = np.zeros(n, dtype=bool)
    mask[order[:k]] = True
    return mask


def select_threshold(scores, tau: float) -> np.ndarray:
    """LIPAR page §2.B: a token whose change is below tau is redundant (pruned); s >= tau stays active."""
    return np.asarray(scores, dtype=np.float64) >= tau


def assign_periods(scores, group_counts, group_periods) -> np.ndarray:
    """HSA page §2.1: split tokens into disjoint groups by score rank, highest change first.

    Group g receives the next ``group_counts[g]`` tokens in (score descending,
    index ascending) order and the activity period ``group_periods[g]``
    (= T / s_g, the total step count over the group's step budget).
    """
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    if sum(group_counts) != n:
        raise ValueError("group counts must cover all tokens")
    order = np.lexsort((np.arange(n), -scores))
    periods = np.empty(n, dtype=np.int64)
    start = 0
    for count, period in zip(group_counts, group_periods):
        periods[order[start:start + count]] = period
        start += count
    return periods


def schedule_mask(periods, step: int) -> np.ndarray:
    """HSA page §2.1: a token of period p = T/s_k is active at global step i iff i mod p == 0."""
    return (step % np.asarray(periods, dtype=np.int64)) == 0


# -------------------------------------------------------------- a3: compact

def compact(mask) -> tuple[np.ndarray, np.ndarray]:
    """Ascending indices of the active tokens and of the pruned complement (HSA page §2.2, item 1)."""
    mask = np.asarray(mask, dtype=bool)
    return np.flatnonzero(mask).astype(np.int64), np.flatnonzero(~mask).astype(np.int64)


# ------------------------------------------------------- a4: recovery rows

def recover_rows(x0_prev, eps, rows, src_row_offset: int, sigma: float) -> np.ndarray:
    """LIPAR page §2.C, noise-aware duplication: a pruned token's context is rebuilt from the
    clean previous latent at the same location plus fresh noise, R = (1 - sigma) * x0_prev + sigma * eps.

    For token p the clean previous latent is ``x0_prev[p - src_row_offset]``
    and the noise is ``eps[p]``; a token with no previous row takes 0 for the
    clean term.  The result is stored, so it is rounded to bf16.
    """
    x0_prev = np.asarray(x0_prev, dtype=np.float64)
    eps = np.asarray(eps, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    src = rows - src_row_offset
    ok = (src >= 0) & (src < x0_prev.shape[0])
    clean = np.zeros((rows.size, eps.shape[1]))
    clean[ok] = x0_prev[src[ok]]
    return round_bf16((1.0 - sigma) * clean + sigma * eps[rows])


# ----------------------------------------------------------- a5: projection

def project(x_rows, w_qkv, parts: str = "qkv") -> dict:
    """HSA page §2.2, item 1: only the active tokens go through the Q/K/V projections.

    Returns bf16-rounded ``x_rows @ W_part.T`` for each requested part
    ('q', 'k', 'v').  The input rows are rounded to bf16 first (fp32 tokens
    enter the projection as bf16).
    """
    x = round_bf16(np.asarray(x_rows, dtype=np.float64))
    w = np.asarray(w_qkv, dtype=np.float64)
    d = w.shape[1]
    if w.shape[0] != 3 * d or x.shape[1] != d:
        raise ValueError("w_qkv must be [3*D, D] and rows [n, D]")
    out = {}
    for i, name in enumerate("qkv"):
        if name in parts:
            out[name] = round_bf16(x @ w[i * d:(i + 1) * d].T)
    return out


# --------------------------------------------------------- a6: cache sync

def kv_cache_sync(k_cache, v_cache, rows, k_rows, v_rows) -> None:
    """HSA page §2.2, item 2: fresh K/V of the given tokens overwrite their rows of the
    per-layer cache in place; every other row keeps its (stale but valid) entry."""
    rows = np.asarray(rows, dtype=np.int64)
    k_cache[rows] = k_rows
    v_cache[rows] = v_rows


# ----------------------------------------------------------- a7: attention

def attention(q, k, v, heads: int, scale: float | None = None, block: int = 256,
              return_lse: bool = False):
    """HSA page §2.2, items 3-4: active queries attend over the full cached K/V.

    Per head h: O_h = softmax(Q_h K_h^T * scale) V_h with scale = 1/sqrt(d),
    no mask (bidirectional).  Float64 throughout; query rows are processed in
    blocks only to bound memory.  ``lse`` is the natural-log normaliser
    log(sum_j exp(S_ij)) per (head, query).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_q, dim = q.shape
    d = dim // heads
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((n_q, dim))
    lse = np.zeros((heads, n_q))
    for h in range(heads):
        cols = slice(h * d, (h + 1) * d)
        kh = k[:, cols]
        vh = v[:, cols]
        for r0 in range(0, n_q, block):
            s = (q[r0:r0 + block, cols] @ kh.T) * scale
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            z = p.sum(axis=1, keepdims=True)
            out[r0:r0 + block, cols] = (p @ vh) / z
            lse[h, r0:r0 + block] = (m + np.log(z))[:, 0]
    if return_lse:
        return out, lse
    return out


# ------------------------------------------------------------ a8: scatter

def scatter(out, rows, o_rows) -> None:
    """Outputs of the active tokens go back to their token rows; other rows keep their
    previous value (HSA page §2.3: skipped tokens reuse what was cached)."""
    out[np.asarray(rows, dtype=np.int64)] = o_rows


# --------------------------------------------------------- whole-layer steps

def init_kv_cache(x, w_qkv) -> tuple[np.ndarray, np.ndarray]:
    """Cache at the start of a run: K/V projections of every token of the previous latent."""
    p = project(x, w_qkv, "kv")
    return p["k"], p["v"]


def layer_step(x_cur, w_qkv, heads: int, k_cache, v_cache, out, *, mask=None, x_ref=None,
               ref_row_offset: int = 0, k: int | None = None, tau: float | None = None,
               relative: bool = True, rope=None, causal_frame_tokens: int | None = None) -> dict:
    """One pruned layer step (HSA page §2.2): score, select, compact, project the active
    tokens, sync their K/V into the cache, attend, scatter.  Updates the cache and ``out``
    in place and returns the intermediate results.

    Selection: ``mask`` if given, else top-``k`` if ``k`` is given, else ``s >= tau``.
    Variants: ``rope = (height, width, base)`` rotates Q and K by their tokens' 3D
    positions before storage (project_rope); ``causal_frame_tokens`` restricts every query
    to the keys of frames up to its own (attention_frame_causal).
    """
    scores = None
    if mask is None:
        scores = token_scores(x_cur, x_ref, ref_row_offset, relative)
        mask = select_topk(scores, k) if k is not None else select_threshold(scores, tau)
    idx, pidx = compact(mask)
    res = {"scores": scores, "mask": np.asarray(mask, bool), "idx": idx, "pidx": pidx}
    if idx.size == 0:
        res["o_a"] = np.zeros((0, out.shape[1]))
        return res
    xa = np.asarray(x_cur, dtype=np.float64)[idx]
    if rope is None:
        p = project(xa, w_qkv, "qkv")
    else:
        p = project_rope(xa, idx, w_qkv, heads, *rope, parts="qkv")
    kv_cache_sync(k_cache, v_cache, idx, p["k"], p["v"])
    if causal_frame_tokens is None:
        o_a = attention(p["q"], k_cache, v_cache, heads)
    else:
        o_a = attention_frame_causal(p["q"], k_cache, v_cache, heads, idx, causal_frame_tokens)
    scatter(out, idx, o_a)
    res.update(q=p["q"], k=p["k"], v=p["v"], o_a=o_a)
    return res


def lipar_step(x, eps, w_qkv, heads: int, hw: int, k: int, sigma: float,
               k_cache, v_cache, out, query_rows=None, mask=None) -> dict:
    """One inter-frame pruned pass over a whole clip (LIPAR page §2.B and §2.C).

    Tokens are scored against the same location one frame earlier (offset
    ``hw``; first-frame tokens score +inf), the top-``k`` stay active; active
    tokens are projected from their own latent, pruned tokens get K/V from the
    recovered row (1 - sigma) * x0_prev + sigma * eps.  Every cache row is
    rewritten; active queries attend over the whole cache.

    ``query_rows`` (positions into the active list) restricts the attention to a
    sample of active queries; rows are independent given the cache.  A given
    ``mask`` (e.g. lif_mask's long/short-term mask) replaces the top-k choice.
    """
    scores = token_scores(x, None, hw)
    mask = select_topk(scores, k) if mask is None else np.asarray(mask, dtype=bool)
    idx, pidx = compact(mask)
    res = {"scores": scores, "mask": mask, "idx": idx, "pidx": pidx}
    xa = np.asarray(x, dtype=np.float64)[idx]
    pa = project(xa, w_qkv, "kv")
    kv_cache_sync(k_cache, v_cache, idx, pa["k"], pa["v"])
    if pidx.size:
        r = recover_rows(x, eps, pidx, hw, sigma)
        pp = project(r, w_qkv, "kv")
        kv_cache_sync(k_cache, v_cache, pidx, pp["k"], pp["v"])
        res.update(r=r, k_p=pp["k"], v_p=pp["v"])
    if query_rows is not None:
        xa = xa[np.asarray(query_rows)]
    q = project(xa, w_qkv, "q")["q"]
    o_a = attention(q, k_cache, v_cache, heads)
    if query_rows is None:
        scatter(out, idx, o_a)
    res.update(q=q, k=pa["k"], v=pa["v"], o_a=o_a)
    return res


# ------------------------------------------- f1: cached Euler update, phase window

def round_f32(x) -> np.ndarray:
    """Round float64 values to the nearest float32, ties to even (storage rounding of an
    fp32 state)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def euler_update(x, v_hat, dt: float, store: str = "f32") -> np.ndarray:
    """HSA page §2.3: every token, active or skipped, advances by the same Euler increment
    dt = sigma_{i+1} - sigma_i along its cached velocity v_hat (the velocity of its most
    recent active step).  One elementwise operation over all N tokens.

    Precision points (the page fixes none): the update is one fp32 operation, so the exact
    x + dt * v_hat is rounded once to fp32; a bf16 state then stores that fp32 value rounded
    to nearest even.  store: 'f32', 'bf16', or 'f64' (kept exact, for checks).
    """
    y = np.asarray(x, dtype=np.float64) + float(dt) * np.asarray(v_hat, dtype=np.float64)
    if store == "f32":
        return round_f32(y)
    if store == "bf16":
        return round_bf16(round_f32(y))
    if store == "f64":
        return y
    raise ValueError(f"unknown store {store!r}")


def step_is_dense(step: int, steps: int, window: int) -> bool:
    """HSA page §2.4: the first and the last ``window`` of the ``steps`` global steps run
    full, uncached passes for every token; caching is confined to the middle."""
    return step < window or step >= steps - window


def euler_dt(sigmas, step: int) -> float:
    """sigma_{i+1} - sigma_i, handed to the update as an fp32 value."""
    return float(np.float32(float(sigmas[step + 1]) - float(sigmas[step])))


def hsa_run(x0, w_qkv, heads: int, periods, sigmas, window: int, store: str = "f32") -> list:
    """HSA page §2.1-§2.4: the sampling loop around the pruned layer.

    T = len(sigmas) - 1 global steps.  At step i the active set is every token when i
    lies in the phase window (step_is_dense), else the tokens whose period p divides i
    (schedule_mask).  The layer step (layer_step: projection of the active tokens, KV
    cache sync, attention over the whole cache, scatter) refreshes the velocity cache
    v_hat at the active rows -- the layer output stands for the velocity prediction --
    and then every token advances: x <- euler_update(x, v_hat, sigma_{i+1} - sigma_i).
    The cache, v_hat and x start at zero, x0 and zero; the state x is stored as
    ``store``.  Returns one record per step: active indices, v_hat and x after it.
    """
    steps = len(sigmas) - 1
    x = np.array(x0, dtype=np.float64)
    n, d = x.shape
    k_cache = np.zeros((n, d))
    v_cache = np.zeros((n, d))
    v_hat = np.zeros((n, d))
    periods = np.asarray(periods)
    hist = []
    for i in range(steps):
        if step_is_dense(i, steps, window):
            mask = np.ones(n, dtype=bool)
        else:
            mask = schedule_mask(periods, i)
        res = layer_step(x, w_qkv, heads, k_cache, v_cache, v_hat, mask=mask)
        x = euler_update(x, v_hat, euler_dt(sigmas, i), store)
        hist.append({"idx": res["idx"], "v_hat": v_hat.copy(), "x": x.copy()})
    return hist


# ------------------------------ f2: long/short-term pruning mask, restoration

def _l1_change(a, b, relative: bool) -> np.ndarray:
    num = np.abs(a - b).sum(axis=-1)
    if not relative:
        return num
    den = np.abs(b).sum(axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = num / den
    s = np.where(den == 0.0, np.where(num == 0.0, 0.0, np.inf), s)
    return s


def lif_mask(x, frames: int, hw: int, tau_short: float, tau_long: float,
             relative: bool = False) -> dict:
    """LIPAR page §2.B (detection and its improvement): a latent token is compared with the
    same spatial location in the previous frame (short-term change) and in the most recent
    frame where that location was kept (long-term change, so that slow drift that stays
    under the per-frame threshold still forces a refresh).  It is pruned only when both
    changes are below their thresholds (strictly); frame 0 is always kept.  Changes are L1
    norms of the row difference (``relative``: divided by the reference row's L1 norm).
    Frames are processed in order, since the long-term reference depends on the earlier
    decisions.  Returns the mask (True = kept) and both change scores (+inf on frame 0).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[1]
    xf = x.reshape(frames, hw, d)
    keep = np.zeros((frames, hw), dtype=bool)
    short = np.full((frames, hw), np.inf)
    long_ = np.full((frames, hw), np.inf)
    keep[0] = True
    last = np.zeros(hw, dtype=np.int64)  # frame of the last kept token at each location
    loc = np.arange(hw)
    for f in range(1, frames):
        short[f] = _l1_change(xf[f], xf[f - 1], relative)
        long_[f] = _l1_change(xf[f], xf[last, loc], relative)
        keep[f] = ~((short[f] < tau_short) & (long_[f] < tau_long))
        last = np.where(keep[f], f, last)
    return {"mask": keep.reshape(-1), "short": short.reshape(-1), "long": long_.reshape(-1)}


def restore_frames(buf, mask, frames: int, hw: int) -> np.ndarray:
    """Dutch LIPAR page §2.D (restoration): after denoising, every pruned token is filled in
    by duplicating the same location of the previous frame, so the decoder receives the
    full token sequence.  Along the frame axis this carries the most recent kept token
    forward.  Kept rows are unchanged; a pruned row in frame 0 (no previous frame) is left
    as it is.
    """
    b = np.array(buf, dtype=np.float64).reshape(frames, hw, -1)
    m = np.asarray(mask, dtype=bool).reshape(frames, hw)
    for f in range(1, frames):
        pruned = ~m[f]
        b[f, pruned] = b[f - 1, pruned]
    return b.reshape(frames * hw, -1)


# ------------------------------------- f3: 3D rotary positions, frame-causal attention

def rope_split(head_dim: int) -> tuple:
    """Channels of one head given to the time, height and width axes: the two spatial axes
    take 2 * floor(d / 6) each and the time axis the rest (d = 128: 44 / 42 / 42)."""
    s = 2 * (head_dim // 6)
    return head_dim - 2 * s, s, s


def token_position(tokens, height: int, width: int) -> tuple:
    """(frame, row, column) of frame-major token indices."""
    t = np.asarray(tokens, dtype=np.int64)
    return t // (height * width), (t // width) % height, t % width


def rope3d(x_rows, tokens, height: int, width: int, heads: int, base: float = 10000.0) -> np.ndarray:
    """Rotary position embedding over the three latent axes.  The Timeripple page
    (Metodología, §1, structured encoding) describes the RoPE of video DiTs as splitting a
    head's channels into a temporal group and two spatial groups (x and y); LIPAR page §2.C
    requires the pruned path to respect those rotations.  Q and K are rotated by their own
    tokens' positions.  Each head's channels are split into time / height / width groups
    (rope_split; the page gives no group sizes, so these are a reading of it); inside the
    group of axis a, of size d_a, the channel pair
    (2i, 2i+1), read as the complex number x_2i + i x_2i+1, is multiplied by
    exp(i p_a base^(-2i/d_a)), p_a being the token's coordinate along a.  Float64, not rounded.
    """
    x = np.asarray(x_rows, dtype=np.float64)
    dim = x.shape[1]
    d = dim // heads
    d_t, d_y, d_x = rope_split(d)
    f, y, xx = token_position(tokens, height, width)
    out = x.copy()
    for h in range(heads):
        for off, d_a, pos in ((0, d_t, f), (d_t, d_y, y), (d_t + d_y, d_x, xx)):
            i = np.arange(d_a // 2)
            ang = pos[:, None].astype(np.float64) * (float(base) ** (-2.0 * i / d_a))[None, :]
            c, s = np.cos(ang), np.sin(ang)
            ev = h * d + off + 2 * i
            a, b = x[:, ev], x[:, ev + 1]
            out[:, ev] = a * c - b * s
            out[:, ev + 1] = a * s + b * c
    return out


def project_rope(x_rows, tokens, w_qkv, heads: int, height: int, width: int, base: float = 10000.0,
                 parts: str = "qkv") -> dict:
    """project() with Q and K rotated (rope3d) by the positions of their tokens before they are
    stored: the exact projection is rotated, then rounded to bf16 once.  V is not rotated."""
    x = round_bf16(np.asarray(x_rows, dtype=np.float64))
    w = np.asarray(w_qkv, dtype=np.float64)
    d = w.shape[1]
    out = {}
    for i, name in enumerate("qkv"):
        if name in parts:
            y = x @ w[i * d:(i + 1) * d].T
            if name in "qk":
                y = rope3d(y, tokens, height, width, heads, base)
            out[name] = round_bf16(y)
    return out


def attention_frame_causal(q, k, v, heads: int, q_tokens, frame_tokens: int, scale: float | None = None,
                           return_lse: bool = False):
    """Frame-causal variant of attention() for causal video models (LIPAR page §3 and §4: the
    method serves causal models such as Self-Forcing as well as bidirectional ones): the
    query of token t sees only the keys of the frames up to its own,
    j < (t // frame_tokens + 1) * frame_tokens (a block-causal mask, one block per frame).  Queries of one frame share a key range, so each group is
    plain attention() over that prefix of the cache."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    frames = np.asarray(q_tokens, dtype=np.int64) // frame_tokens
    out = np.zeros_like(q)
    lse = np.zeros((heads, q.shape[0]))
    for f in np.unique(frames):
        rows = np.flatnonzero(frames == f)
        lim = min(k.shape[0], (int(f) + 1) * frame_tokens)
        o, l = attention(q[rows], k[:lim], v[:lim], heads, scale, return_lse=True)
        out[rows] = o
        lse[:, rows] = l
    return (out, lse) if return_lse else out


# ------------------------------------------ f4: Timeripple partial-score reuse

# Axis order of the reuse checks and of the channel groups: time (frames), height (rows),
# width (columns) -- the order of rope_split.
REUSE_AXES = ("t", "y", "x")


def reuse_groups(head_dim: int) -> list:
    """Channel ranges [start, end) of the time / height / width groups of one head: the
    rotary groups of the Timeripple page (Metodología §1, structured encoding)."""
    d_t, d_y, d_x = rope_split(head_dim)
    return [(0, d_t), (d_t, d_t + d_y), (d_t + d_y, head_dim)]


def axis_neighbors(n_tokens: int, height: int, width: int) -> np.ndarray:
    """[3, n]: the token one step back along time / height / width (frame-major layout):
    same location one frame earlier, one row up, one column left; -1 where there is none."""
    t = np.arange(n_tokens, dtype=np.int64)
    f, y, x = token_position(t, height, width)
    nb = np.full((3, n_tokens), -1, dtype=np.int64)
    nb[0] = np.where(f > 0, t - height * width, -1)
    nb[1] = np.where(y > 0, t - width, -1)
    nb[2] = np.where(x > 0, t - 1, -1)
    return nb


def reuse_deltas(v, heads: int, height: int, width: int) -> np.ndarray:
    """Timeripple page, Metodología §2 (similarity checks along the time, x and y axes):
    for token n, head h and axis a, the relative RMS difference between the token and its
    neighbour along a over C_a, the channels of the two groups that axis a does not rotate
    (moving along a leaves their rotary phase unchanged, Metodología §1):
        delta[n, h, a] = ||v[n, h, C_a] - v[nb_a(n), h, C_a]||_2 / ||v[n, h, C_a]||_2
    (0/0 -> 0, x/0 -> inf); +inf without a neighbour.  Float64."""
    v = np.asarray(v, dtype=np.float64)
    n, dim = v.shape
    d = dim // heads
    groups = reuse_groups(d)
    nb = axis_neighbors(n, height, width)
    out = np.full((n, heads, 3), np.inf)
    for a in range(3):
        chans = np.concatenate([np.arange(s, e) for g, (s, e) in enumerate(groups) if g != a])
        has = nb[a] >= 0
        rows = np.flatnonzero(has)
        for h in range(heads):
            cols = h * d + chans
            own = v[np.ix_(rows, cols)]
            diff = own - v[np.ix_(nb[a, rows], cols)]
            num = np.sqrt((diff * diff).sum(1))
            den = np.sqrt((own * own).sum(1))
            with np.errstate(divide="ignore", invalid="ignore"):
                out[rows, h, a] = np.where(den == 0, np.where(num == 0, 0.0, np.inf), num / den)
    return out


def reuse_sources(deltas, thetas, height: int, width: int) -> np.ndarray:
    """Reuse decision (Metodología §2): a token is reusable along axis a when its delta is
    below theta_a (strictly); any reusable axis suffices.  Channel group g of token n, head h
    then takes its partial scores from the neighbour along the first reusable axis a != g in
    the order time, height, width; otherwise from the token itself.  Returns
    src[n, h, g] (a token index, = n when computed)."""
    deltas = np.asarray(deltas, dtype=np.float64)
    n, heads, _ = deltas.shape
    nb = axis_neighbors(n, height, width)
    src = np.broadcast_to(np.arange(n, dtype=np.int64)[:, None, None], (n, heads, 3)).copy()
    for g in range(3):
        decided = np.zeros((n, heads), dtype=bool)
        for a in range(3):
            if a == g:
                continue
            ok = (deltas[:, :, a] < float(thetas[a])) & ~decided
            src[:, :, g] = np.where(ok, nb[a][:, None], src[:, :, g])
            decided |= ok
    return src


def reuse_effective(v, src, heads: int) -> np.ndarray:
    """Aggregation (Metodología §2): the partial scores of group g of token n are the
    neighbour's own (computed or themselves reused), i.e. the group's channels of the
    source token's effective vector; sources precede their tokens, so one pass in token
    order resolves every chain.  Reusing the partial score q_g . k_g of a token is the same
    as taking its group-g channels from the source, so the attention map is that of the
    effective vectors."""
    v = np.asarray(v, dtype=np.float64)
    n, dim = v.shape
    d = dim // heads
    groups = reuse_groups(d)
    eff = v.copy()
    for t in range(n):
        for h in range(heads):
            for g, (s, e) in enumerate(groups):
                j = int(src[t, h, g])
                if j != t:
                    eff[t, h * d + s:h * d + e] = eff[j, h * d + s:h * d + e]
    return eff


def timeripple_attention(q, k, v, heads: int, height: int, width: int, thetas_q, thetas_k,
                         scale: float | None = None) -> dict:
    """Attention with Timeripple's partial-score reuse applied independently to the queries
    and the keys of all N tokens (Metodología §2: checks for Q and K tokens); V unchanged."""
    sq = reuse_sources(reuse_deltas(q, heads, height, width), thetas_q, height, width)
    sk = reuse_sources(reuse_deltas(k, heads, height, width), thetas_k, height, width)
    q_eff = reuse_effective(q, sq, heads)
    k_eff = reuse_effective(k, sk, heads)
    return {"src_q": sq, "src_k": sk, "q_eff": q_eff, "k_eff": k_eff,
            "out": attention(q_eff, k_eff, v, heads, scale)}
