"""Workload shapes for the pruned-attention layer.

Every count below is an exact integer (a percentage of N is taken as
``pct * N // 100``), so no float rounding decides how many tokens are static or
active.  The shapes stand in for the video-DiT latent grids the pages run on
(LIPAR: DAVIS clips through Self-Forcing / Time-to-Move; HSA: Wan-2.1-1.3B,
Wan-2.2-A14B, LTX-2).  None of those datasets or models is used.
"""

from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Config:
    name: str
    kind: str  # "step" (one layer step), "hsa" (T-step schedule), "hsa_loop" (sampling loop with
    # Euler update and phase window), "lipar" (inter-frame sweep), "lipar_lif" (long/short-term mask)
    frames: int
    height: int
    width: int
    dim: int
    heads: int
    head_dim: int
    dtype: str  # storage type of the latent tokens: "fp32" or "bf16"
    static_pct: int  # percent of tokens (or spatial locations, for "lipar") that barely change
    active_pct: int = 0  # "step": percent of tokens kept active (top-k by score)
    static_scale: float = 0.01  # std of the per-step change of a static token
    moving_scale: float = 0.5  # std of the per-step change of a moving token
    steps: int = 0  # "hsa": T
    group_pcts: tuple = ()  # "hsa": group sizes in percent of N, highest change first
    group_budgets: tuple = ()  # "hsa": step budget s_k of each group (divides T)
    sigma: float = 0.0  # "lipar": re-noising level of the recovered pruned tokens
    sweep_pcts: tuple = field(default_factory=tuple)  # "lipar": active percentages swept
    window: int = 0  # "hsa_loop": the first and last `window` steps run dense
    tau_short: float = 0.0  # "lipar_lif": threshold on the L1 change against the previous frame
    tau_long: float = 0.0  # "lipar_lif": threshold on the L1 change against the last kept frame
    rope: bool = False  # "step": 3D rotary positions on Q and K (base 10000)
    causal: bool = False  # "step": frame-causal attention (a query sees the frames up to its own)
    reuse_theta: tuple = ()  # "reuse": thresholds (time, height, width) of the partial-score reuse of Q and K

    @property
    def n(self) -> int:
        return self.frames * self.height * self.width

    @property
    def hw(self) -> int:
        return self.height * self.width

    @property
    def n_static(self) -> int:
        if self.kind.startswith("lipar") or self.kind == "reuse":
            return self.static_pct * self.hw // 100
        return self.static_pct * self.n // 100

    @property
    def n_active(self) -> int:
        return self.active_pct * self.n // 100

    def group_counts(self) -> tuple:
        return tuple(p * self.n // 100 for p in self.group_pcts)

    def group_periods(self) -> tuple:
        return tuple(self.steps // b for b in self.group_budgets)

    def sweep_counts(self) -> tuple:
        return tuple(p * self.n // 100 for p in self.sweep_pcts)

    def sigmas(self) -> list:
        """Noise levels sigma_0..sigma_T of the sampling loop: linear from 1 to 0."""
        return [1.0 - i / self.steps for i in range(self.steps + 1)]

    def attn_flops(self, n_active: int) -> int:
        """Algorithmic attention work of one layer step: 4 * N_a * N * d * H."""
        return 4 * n_active * self.n * self.head_dim * self.heads

    def qkv_flops(self, n_active: int) -> int:
        return 2 * n_active * self.dim * 3 * self.dim


CONFIGS = {
    # 4x8x8 latent grid, fp32 tokens, 25% active.
    "tiny": Config("tiny", "step", 4, 8, 8, 128, 2, 64, "fp32", static_pct=70, active_pct=25),
    # Wan-1.3B-like grid 21x30x52, 30% active (the headline workload).
    "wan13b": Config("wan13b", "step", 21, 30, 52, 1536, 12, 128, "bf16", static_pct=70, active_pct=30),
    # The headline grid with 3D rotary positions and frame-causal attention.
    "wan13b_rc": Config("wan13b_rc", "step", 21, 30, 52, 1536, 12, 128, "bf16", static_pct=70, active_pct=30,
                        rope=True, causal=True),
    # 21x45x80 grid at model dim 5120, 20% active.
    "large": Config("large", "step", 21, 45, 80, 5120, 40, 128, "bf16", static_pct=80, active_pct=20),
    # HSA schedule loop on the Wan-1.3B-like grid: T=8, groups 25/25/50 % with budgets 8/4/2.
    "hsa": Config(
        "hsa", "hsa", 21, 30, 52, 1536, 12, 128, "bf16", static_pct=70,
        steps=8, group_pcts=(25, 25, 50), group_budgets=(8, 4, 2),
    ),
    # The HSA schedule inside its sampling loop: Euler update after every step, the first and
    # last step dense.
    "hsa_loop": Config(
        "hsa_loop", "hsa_loop", 21, 30, 52, 1536, 12, 128, "bf16", static_pct=70,
        steps=8, group_pcts=(25, 25, 50), group_budgets=(8, 4, 2), window=1,
    ),
    # Timeripple partial-score reuse over a 21x30x52 clip (75% static locations drifting by 1%
    # per frame): dense attention of all tokens with rotated Q/K whose channel groups are
    # reused from the neighbouring token when their relative RMS difference is below 5%.
    "timeripple": Config("timeripple", "reuse", 21, 30, 52, 1536, 12, 128, "bf16", static_pct=75,
                         reuse_theta=(0.05, 0.05, 0.05)),
    # LIPAR inter-frame sweep on a 33x45x80 grid, 75% static locations, sigma = 0.6.
    "lipar": Config(
        "lipar", "lipar", 33, 45, 80, 3072, 24, 128, "bf16", static_pct=75,
        sigma=0.6, sweep_pcts=(5, 10, 25, 50, 100),
    ),
    # The same clip pruned by the long/short-term mask (absolute L1 changes): a static location
    # changes by about 24 per frame and drifts past 60 after 5-7 frames; a moving one changes
    # by about 1200 per frame.
    "lipar_lif": Config(
        "lipar_lif", "lipar_lif", 33, 45, 80, 3072, 24, 128, "bf16", static_pct=75,
        sigma=0.6, tau_short=100.0, tau_long=60.0,
    ),
}


def get_config(name: str) -> Config:
    try:
        return CONFIGS[name]
    except KeyError as exc:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}") from exc


def scaled(cfg: Config, frames: int | None = None, height: int | None = None,
           width: int | None = None, dim: int | None = None, heads: int | None = None) -> Config:
    """A smaller copy of a workload with the same structure (for tests the oracle finishes quickly)."""
    from dataclasses import replace

    kw = {}
    if frames is not None:
        kw["frames"] = frames
    if height is not None:
        kw["height"] = height
    if width is not None:
        kw["width"] = width
    if dim is not None:
        kw["dim"] = dim
    if heads is not None:
        kw["heads"] = heads
    if dim is not None or heads is not None:
        d = kw.get("dim", cfg.dim)
        h = kw.get("heads", cfg.heads)
        if d % h:
            raise ValueError("dim must be a multiple of heads")
        kw["head_dim"] = d // h
    return replace(cfg, name=cfg.name + "_scaled", **kw)
