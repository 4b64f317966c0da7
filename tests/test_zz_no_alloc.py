"""tsa_timeripple_reuse_noalloc (the library's static scratch instead of a caller's
workspace) against tsa_timeripple_reuse with a workspace: bit for bit, on calls in a
row of different sizes (each call overwrites what the previous one left in the
scratch), up to the largest accepted size; sizes above it are refused."""

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


def _rows(frames, height, width, heads, hd, seed):
    """Rotary rows of a clip whose locations drift slowly (75 %) or fast, rounded to bf16."""
    r = np.random.default_rng(seed)
    hw = height * width
    scale = np.where(r.random(hw) < 0.75, 0.01, 0.5)[:, None]
    rows = [r.standard_normal((hw, heads * hd))]
    for _ in range(1, frames):
        rows.append(rows[-1] + scale * r.standard_normal((hw, heads * hd)))
    content = np.concatenate(rows, axis=0)
    v = ref.round_bf16(ref.rope3d(content, np.arange(frames * hw), height, width, heads))
    return G.dev(torch.from_numpy(v), torch.bfloat16)


def _both(v, heads, hd, height, width, thetas):
    t = tsa()
    n = v.shape[0]
    outs = []
    for noalloc in (False, True):
        eff = torch.full_like(v, 7.0)
        src = torch.full((n, heads, 3), -9, dtype=torch.int32, device="cuda")
        delta = torch.full((n, heads, 3), -9.0, dtype=torch.float32, device="cuda")
        if noalloc:
            t.timeripple_reuse_noalloc(v, heads, hd, height, width, thetas, eff, src_out=src, delta_out=delta)
        else:
            ws = torch.empty(t.reuse_workspace_bytes(n, heads), dtype=torch.uint8, device="cuda")
            t.timeripple_reuse(v, heads, hd, height, width, thetas, eff, ws, src_out=src, delta_out=delta)
        torch.cuda.synchronize()
        outs.append((eff, src, delta))
    return outs


@pytest.mark.parametrize("order", ["large_then_small", "small_then_large"])
def test_noalloc_reuse_equals_workspace_reuse(order):
    cases = [(9, 10, 24, 4, 128, (0.05, 0.05, 0.05), 1), (5, 7, 11, 2, 64, (0.2, 0.0, float("inf")), 2)]
    if order == "small_then_large":
        cases = cases[::-1]
    for frames, h, w, heads, hd, th, seed in cases + cases[:1]:
        print(f"  noalloc reuse: {frames}x{h}x{w} heads={heads} d={hd} thetas={th}", flush=True)
        v = _rows(frames, h, w, heads, hd, seed)
        (e0, s0, d0), (e1, s1, d1) = _both(v, heads, hd, h, w, th)
        assert torch.equal(e0, e1) and torch.equal(s0, s1) and torch.equal(d0, d1)
        assert int((s1 >= 0).sum()) > 0  # every entry written


def test_noalloc_reuse_at_the_size_limit_and_above():
    t = tsa()
    lim = t.reuse_noalloc_max_token_heads()
    assert lim == 1 << 20
    heads, hd, h, w = 4, 64, 64, 64
    n = lim // heads  # 64 frames of 64 x 64
    print(f"  noalloc reuse at the limit: n={n} heads={heads}", flush=True)
    g = torch.Generator().manual_seed(3)
    v = (torch.randn(n, heads * hd, generator=g)).to(torch.bfloat16).cuda()
    (e0, s0, d0), (e1, s1, d1) = _both(v, heads, hd, h, w, (0.3, 0.3, 0.3))
    assert torch.equal(e0, e1) and torch.equal(s0, s1) and torch.equal(d0, d1)
    v2 = torch.zeros(n + 1, heads * hd, dtype=torch.bfloat16, device="cuda")
    eff2 = torch.empty_like(v2)
    with pytest.raises(t.TsaError) as err:
        t.timeripple_reuse_noalloc(v2, heads, hd, h, w, (0.3, 0.3, 0.3), eff2)
    assert err.value.status == 2  # TSA_ERR_SHAPE, nothing launched
