"""Seeded input generators (CPU, torch's mt19937 CPU generator).

Each named tensor is drawn from its own generator, seeded by a stable hash of
(seed, tensor name).  So a tensor never depends on which other tensors were
drawn before it, and large per-sweep-point tensors can be drawn lazily.

Recipe shared by all workloads:

* a random static set (a permutation of tokens, or of spatial locations for
  the inter-frame workload); static tokens change with std ``static_scale``,
  the others with std ``moving_scale``;
* latents ~ N(0, 1), rounded to the storage type (bf16 round-to-nearest-even,
  or kept fp32 for the tiny workload);
* one fused projection weight ``w_qkv`` of shape [3*D, D] (rows 0..D-1 are the
  query projection, then key, then value; output = x @ w_part.T), entries
  ~ N(0, 1/D), stored bf16.

Returned tensors live on the CPU; callers move them where they are needed.
"""

from __future__ import annotations

import hashlib

import torch

from .configs import Config

_STORE = {"bf16": torch.bfloat16, "fp32": torch.float32}


def _gen(seed: int, tag: str) -> torch.Generator:
    h = hashlib.blake2b(f"tsa:{seed}:{tag}".encode(), digest_size=8).digest()
    return torch.Generator().manual_seed(int.from_bytes(h, "little") & ((1 << 63) - 1))


def _randn(seed: int, tag: str, *shape: int) -> torch.Tensor:
    return torch.randn(*shape, generator=_gen(seed, tag), dtype=torch.float32)


def _store(x: torch.Tensor, dtype: str) -> torch.Tensor:
    return x.to(_STORE[dtype]).contiguous()


def _weights(cfg: Config, seed: int) -> torch.Tensor:
    w = _randn(seed, "w_qkv", 3 * cfg.dim, cfg.dim) * (cfg.dim ** -0.5)
    return w.to(torch.bfloat16).contiguous()


def _token_scale(cfg: Config, seed: int, count: int, n_static: int) -> tuple[torch.Tensor, torch.Tensor]:
    perm = torch.randperm(count, generator=_gen(seed, "static"))
    static = torch.zeros(count, dtype=torch.bool)
    static[perm[:n_static]] = True
    scale = torch.where(static, torch.tensor(cfg.static_scale), torch.tensor(cfg.moving_scale))
    return static, scale.to(torch.float32)


def step_inputs(cfg: Config, seed: int = 0) -> dict:
    """One layer step: x_prev, x_cur = store(x_prev + s_n * z), w_qkv, static mask."""
    n, d = cfg.n, cfg.dim
    static, scale = _token_scale(cfg, seed, n, cfg.n_static)
    x_prev = _store(_randn(seed, "x_prev", n, d), cfg.dtype)
    z = _randn(seed, "z", n, d)
    x_cur = _store(x_prev.float() + scale[:, None] * z, cfg.dtype)
    del z
    return {"x_prev": x_prev, "x_cur": x_cur, "w_qkv": _weights(cfg, seed), "static": static}


def hsa_inputs(cfg: Config, seed: int = 0) -> dict:
    """T+1 latents x_0..x_T with x_{i+1} = store(x_i + s_n * z_i); step i runs on x_{i+1}."""
    n, d = cfg.n, cfg.dim
    static, scale = _token_scale(cfg, seed, n, cfg.n_static)
    xs = [_store(_randn(seed, "x_prev", n, d), cfg.dtype)]
    for i in range(cfg.steps):
        z = _randn(seed, f"z{i}", n, d)
        xs.append(_store(xs[-1].float() + scale[:, None] * z, cfg.dtype))
        del z
    return {"xs": xs, "w_qkv": _weights(cfg, seed), "static": static}


def lipar_inputs(cfg: Config, seed: int = 0) -> dict:
    """Clean per-frame latents x0_f = store(x0_{f-1} + s_loc * z_f), frames stacked to [F*H*W, D]."""
    hw, d = cfg.hw, cfg.dim
    static, scale = _token_scale(cfg, seed, hw, cfg.n_static)
    frames = [_store(_randn(seed, "x0_0", hw, d), cfg.dtype)]
    for f in range(1, cfg.frames):
        z = _randn(seed, f"z{f}", hw, d)
        frames.append(_store(frames[-1].float() + scale[:, None] * z, cfg.dtype))
        del z
    x = torch.cat(frames, dim=0).contiguous()
    del frames
    return {"x": x, "w_qkv": _weights(cfg, seed), "static_loc": static}


def lipar_eps(cfg: Config, seed: int, point: int) -> torch.Tensor:
    """Fresh Gaussian noise [N, D] for sweep point ``point`` (drawn anew for every point)."""
    return _store(_randn(seed, f"eps{point}", cfg.n, cfg.dim), cfg.dtype)
