"""Second, independent implementation of the layer in pure Python (lists, math.fsum, math.exp).

TEST INFRASTRUCTURE ONLY.  Written without numpy so that a mistake shared by
numpy idioms in ``reference`` (an axis, a transpose, a broadcast) cannot hide
in both.  Only for tiny inputs (N <= 64 tokens).
"""

from __future__ import annotations

import math
import struct


def bf16(x: float) -> float:
    """Nearest bfloat16 (8 significant bits), ties to even, via Python's round-half-even."""
    if x == 0.0 or math.isinf(x) or math.isnan(x):
        return x
    m, e = math.frexp(x)  # x = m * 2**e, 0.5 <= |m| < 1
    quantum_exp = max(e - 8, -133)
    r = round(x / 2.0 ** quantum_exp) * 2.0 ** quantum_exp
    if abs(r) > (2.0 - 2.0 ** -7) * 2.0 ** 127:
        return math.copysign(math.inf, r)
    return r


def scores(x_cur, x_ref, relative=True, ref_row_offset=0):
    n = len(x_cur)
    ref = x_cur if x_ref is None else x_ref
    out = []
    for i in range(n):
        j = i - ref_row_offset
        if j < 0 or j >= len(ref):
            out.append(math.inf)
            continue
        num = math.fsum(abs(a - b) for a, b in zip(x_cur[i], ref[j]))
        if not relative:
            out.append(num)
            continue
        den = math.fsum(abs(b) for b in ref[j])
        if den == 0.0:
            out.append(0.0 if num == 0.0 else math.inf)
        else:
            out.append(num / den)
    return out


def topk(s, k):
    ranked = sorted(range(len(s)), key=lambda i: (-s[i], i))
    chosen = set(ranked[:k])
    return [i in chosen for i in range(len(s))]


def compact(mask):
    return [i for i, m in enumerate(mask) if m], [i for i, m in enumerate(mask) if not m]


def matmul_t(x, w_rows):
    """x @ w.T for lists of rows."""
    return [[math.fsum(a * b for a, b in zip(row, wr)) for wr in w_rows] for row in x]


def project(x_rows, w_qkv, part):
    d = len(w_qkv[0])
    off = "qkv".index(part) * d
    xb = [[bf16(v) for v in row] for row in x_rows]
    return [[bf16(v) for v in row] for row in matmul_t(xb, w_qkv[off:off + d])]


def attention(q, k, v, heads, scale=None):
    dim = len(q[0])
    d = dim // heads
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = [[0.0] * dim for _ in q]
    for h in range(heads):
        c0 = h * d
        for i, qi in enumerate(q):
            s = [scale * math.fsum(qi[c0 + t] * kj[c0 + t] for t in range(d)) for kj in k]
            mx = max(s)
            p = [math.exp(x - mx) for x in s]
            z = math.fsum(p)
            for t in range(d):
                out[i][c0 + t] = math.fsum(p[j] * k_v[c0 + t] for j, k_v in enumerate(v)) / z
    return out


def layer_step(x_cur, x_ref, w_qkv, heads, k_cache, v_cache, out, k):
    """Score, top-k, compact, project, cache sync, attention, scatter -- all in lists."""
    s = scores(x_cur, x_ref)
    mask = topk(s, k)
    idx, pidx = compact(mask)
    xa = [x_cur[i] for i in idx]
    q = project(xa, w_qkv, "q")
    ka = project(xa, w_qkv, "k")
    va = project(xa, w_qkv, "v")
    for r, i in enumerate(idx):
        k_cache[i] = list(ka[r])
        v_cache[i] = list(va[r])
    o = attention(q, k_cache, v_cache, heads)
    for r, i in enumerate(idx):
        out[i] = list(o[r])
    return {"scores": s, "mask": mask, "idx": idx, "pidx": pidx, "q": q, "k": ka, "v": va, "o_a": o}


def recover(x0_prev, eps, rows, src_row_offset, sigma):
    res = []
    for p in rows:
        j = p - src_row_offset
        clean = x0_prev[j] if 0 <= j < len(x0_prev) else [0.0] * len(eps[p])
        res.append([bf16((1.0 - sigma) * a + sigma * b) for a, b in zip(clean, eps[p])])
    return res


def periods_by_rank(s, counts, periods):
    ranked = sorted(range(len(s)), key=lambda i: (-s[i], i))
    out = [0] * len(s)
    pos = 0
    for c, p in zip(counts, periods):
        for i in ranked[pos:pos + c]:
            out[i] = p
        pos += c
    return out


def f32(x: float) -> float:
    """Nearest float32, ties to even (the struct module's conversion)."""
    return struct.unpack("f", struct.pack("f", x))[0]


def euler(x, v, dt):
    """x + dt * v per element, the exact value rounded once to float32 (fsum keeps it exact)."""
    return [[f32(math.fsum([a, dt * b])) for a, b in zip(xr, vr)] for xr, vr in zip(x, v)]


def hsa_run(x0, w_qkv, heads, periods, sigmas, window):
    """The sampling loop: dense steps in the window, schedule elsewhere, Euler update after each."""
    steps = len(sigmas) - 1
    n, d = len(x0), len(x0[0])
    x = [list(r) for r in x0]
    k_cache = [[0.0] * d for _ in range(n)]
    v_cache = [[0.0] * d for _ in range(n)]
    v_hat = [[0.0] * d for _ in range(n)]
    hist = []
    for i in range(steps):
        dense = i < window or i >= steps - window
        idx = [t for t in range(n) if dense or i % periods[t] == 0]
        xa = [x[t] for t in idx]
        q = project(xa, w_qkv, "q")
        ka = project(xa, w_qkv, "k")
        va = project(xa, w_qkv, "v")
        for r, t in enumerate(idx):
            k_cache[t] = list(ka[r])
            v_cache[t] = list(va[r])
        o = attention(q, k_cache, v_cache, heads)
        for r, t in enumerate(idx):
            v_hat[t] = list(o[r])
        dt = f32(sigmas[i + 1] - sigmas[i])
        x = euler(x, v_hat, dt)
        hist.append({"idx": idx, "v_hat": [list(r) for r in v_hat], "x": [list(r) for r in x]})
    return hist


def lif_mask(x, frames, hw, tau_short, tau_long, relative=False):
    """Frame-by-frame scan per location with short- and long-term L1 changes."""
    def change(a, b):
        num = math.fsum(abs(p - r) for p, r in zip(a, b))
        if not relative:
            return num
        den = math.fsum(abs(r) for r in b)
        if den == 0.0:
            return 0.0 if num == 0.0 else math.inf
        return num / den
    keep = [True] * hw + [False] * ((frames - 1) * hw)
    for loc in range(hw):
        last = 0
        for f in range(1, frames):
            cur = x[f * hw + loc]
            s = change(cur, x[(f - 1) * hw + loc])
            lt = change(cur, x[last * hw + loc])
            k = not (s < tau_short and lt < tau_long)
            keep[f * hw + loc] = k
            if k:
                last = f
    return keep


def restore(buf, mask, frames, hw):
    """Pruned token (f, loc) takes the value of the nearest earlier kept frame at loc."""
    out = [list(r) for r in buf]
    for loc in range(hw):
        for f in range(1, frames):
            t = f * hw + loc
            if not mask[t]:
                src = f - 1
                while src > 0 and not mask[src * hw + loc]:
                    src -= 1
                out[t] = list(buf[src * hw + loc])  # a kept frame, or frame 0
    return out


def rope(x_rows, tokens, height, width, heads, base=10000.0):
    """Rotate each adjacent channel pair of every head by its axis position times the pair's
    frequency; time / height / width channel groups of sizes d - 4*(d//6), 2*(d//6), 2*(d//6)."""
    dim = len(x_rows[0])
    d = dim // heads
    g = 2 * (d // 6)
    groups = [(0, d - 2 * g, 0), (d - 2 * g, g, 1), (d - g, g, 2)]
    out = []
    for row, t in zip(x_rows, tokens):
        pos = (t // (height * width), (t // width) % height, t % width)
        r = list(row)
        for h in range(heads):
            for start, size, axis in groups:
                for i in range(size // 2):
                    theta = pos[axis] * base ** (-2.0 * i / size)
                    j = h * d + start + 2 * i
                    a, b = row[j], row[j + 1]
                    r[j] = a * math.cos(theta) - b * math.sin(theta)
                    r[j + 1] = a * math.sin(theta) + b * math.cos(theta)
        out.append(r)
    return out


def attention_frame_causal(q, k, v, heads, q_tokens, frame_tokens, scale=None):
    """Query of token t sees keys j with j // frame_tokens <= t // frame_tokens."""
    dim = len(q[0])
    d = dim // heads
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = [[0.0] * dim for _ in q]
    for i, (qi, t) in enumerate(zip(q, q_tokens)):
        keys = [j for j in range(len(k)) if j // frame_tokens <= t // frame_tokens]
        for h in range(heads):
            c0 = h * d
            s = [scale * math.fsum(qi[c0 + u] * k[j][c0 + u] for u in range(d)) for j in keys]
            mx = max(s)
            p = [math.exp(x - mx) for x in s]
            z = math.fsum(p)
            for u in range(d):
                out[i][c0 + u] = math.fsum(pj * v[j][c0 + u] for pj, j in zip(p, keys)) / z
    return out


def reuse(v_rows, heads, height, width, thetas):
    """Timeripple partial-score reuse, token by token: for each axis (time, height, width) the
    neighbour one step back, the relative RMS difference over the channels of the two groups
    that axis does not rotate, the first axis (in that order, not the group's own) whose
    difference is below its threshold gives each channel group its source; the group's
    channels are copied from the source's already resolved vector.  Returns (src, eff)."""
    n = len(v_rows)
    dim = len(v_rows[0])
    d = dim // heads
    g = 2 * (d // 6)
    bounds = [(0, d - 2 * g), (d - 2 * g, d - g), (d - g, d)]
    hw = height * width
    eff = [list(r) for r in v_rows]
    src = [[[t] * 3 for _ in range(heads)] for t in range(n)]
    for t in range(n):
        f, y, x = t // hw, (t // width) % height, t % width
        nbs = [t - hw if f > 0 else None, t - width if y > 0 else None, t - 1 if x > 0 else None]
        for h in range(heads):
            deltas = []
            for a in range(3):
                j = nbs[a]
                if j is None:
                    deltas.append(math.inf)
                    continue
                chans = [h * d + c for gi, (s, e) in enumerate(bounds) if gi != a for c in range(s, e)]
                num = math.sqrt(math.fsum((v_rows[t][c] - v_rows[j][c]) ** 2 for c in chans))
                den = math.sqrt(math.fsum(v_rows[t][c] ** 2 for c in chans))
                deltas.append((0.0 if num == 0 else math.inf) if den == 0 else num / den)
            for gi, (s, e) in enumerate(bounds):
                for a in range(3):
                    if a != gi and deltas[a] < thetas[a]:
                        src[t][h][gi] = nbs[a]
                        for c in range(h * d + s, h * d + e):
                            eff[t][c] = eff[nbs[a]][c]
                        break
    return src, eff
