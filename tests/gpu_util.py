"""Helpers for the GPU parity tests (comparison metrics, transfers)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

# Output tolerance of the layer (attention outputs and written K/V):
# relative Frobenius error <= 5e-3 and max abs error <= 2e-2 against the fp64 oracle.
REL_FROB = 5e-3
MAX_ABS = 2e-2
# Scores: fp32 accumulation of D terms vs fp64; relative error bound used by the tests.
SCORE_RTOL = 2e-6
# Tokens whose score lies within this relative distance of the k-th score may flip.
NEAR_THRESHOLD = 1e-5


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_sparse_attention_rel_amd  # noqa: F401  (raises if libtsa.so is missing)


def dev(t, dtype=None):
    t = torch.as_tensor(t)
    if dtype is not None:
        t = t.to(dtype)
    return t.contiguous().cuda()


def host64(t) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def rel_frob(got, want) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


def max_abs(got, want) -> float:
    d = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
    return float(d.max()) if d.size else 0.0


def assert_close(got, want, what="", rel=REL_FROB, mabs=MAX_ABS):
    """Layer output tolerance: relative Frobenius error <= rel, and elementwise
    |got - want| <= mabs * max(1, |want|).  The max-abs bound is scaled for |want| > 1
    because the outputs are stored as bf16, whose rounding alone (half an ulp,
    2**-9 |want|) exceeds a fixed 2e-2 once |want| >= 8 (one ulp flip once |want| >= 4)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    rf, ma = rel_frob(got, want), max_abs(got, want)
    sc = float(np.max(np.abs(got - want) / np.maximum(1.0, np.abs(want)))) if got.size else 0.0
    # elements whose unscaled error exceeds the fixed 2e-2 (those sit where |want| > 1)
    n_over = int(np.count_nonzero(np.abs(got - want) > MAX_ABS))
    print(f"  {what}: rel_frob={rf:.3e} max_abs={ma:.3e} scaled_max_abs={sc:.3e} "
          f"above_{MAX_ABS:g}={n_over} of {got.size}", flush=True)
    assert rf <= rel and sc <= mabs, f"{what}: rel_frob={rf:.3e} max_abs={ma:.3e} scaled={sc:.3e}"


def bf16_ulp_mismatch(got, want) -> tuple[int, int]:
    """(#elements differing, #differing by more than one bf16 ulp) between two bf16-valued arrays."""
    d = ulp_distance(got, want)
    return int((d != 0).sum()), int((d > 1).sum())


def mask_mismatch_ok(gpu_mask, ora_mask, ora_scores, k) -> int:
    """Check a top-k mask against the oracle's: tokens may differ only when their score is
    within NEAR_THRESHOLD (relative) of the oracle's k-th score.  Returns the count."""
    diff = np.flatnonzero(np.asarray(gpu_mask, bool) != np.asarray(ora_mask, bool))
    if diff.size == 0:
        return 0
    thr = np.sort(ora_scores)[::-1][k - 1]
    rel = np.abs(ora_scores[diff] - thr) / max(abs(thr), 1e-30)
    assert np.all(rel <= NEAR_THRESHOLD), f"mask differs far from the threshold: {rel.max():.3e}"
    return int(diff.size)


def _ordered_bf16(a) -> np.ndarray:
    """bf16 bit patterns mapped to integers in value order (so differences count ulps)."""
    b = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16)
    u = b.to(torch.int32) & 0xFFFF
    mag = u & 0x7FFF
    return torch.where(u >= 0x8000, -mag, mag).numpy()


def ulp_distance(got, want) -> np.ndarray:
    """Distance in bf16 ulps between two bf16-valued arrays."""
    return np.abs(_ordered_bf16(got).astype(np.int64) - _ordered_bf16(want).astype(np.int64))


def assert_bf16_close(got, want, what=""):
    """Stored bf16 values (K/V, projections): within one bf16 ulp of the oracle's rounding of the
    exact value (the fp32-accumulated product can land on the other side of a rounding
    boundary), mismatches counted, and the relative Frobenius bound of the layer."""
    d = ulp_distance(got, want)
    rf = rel_frob(got, want)
    print(f"  {what}: rel_frob={rf:.3e}, {int((d == 1).sum())} of {d.size} one-ulp differences, "
          f"max {int(d.max()) if d.size else 0} ulp", flush=True)
    assert rf <= REL_FROB and (d.size == 0 or d.max() <= 1), what


def bf16_ulp_of(v) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (2**(e-7) for |v| in [2**e, 2**(e+1)))."""
    a = np.maximum(np.abs(np.asarray(v, np.float64)), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def assert_projection_close(got, want, abs_dot, k_terms, what=""):
    """bf16 results of a length-k dot product accumulated in fp32, against the oracle's
    bf16 rounding of the exact value:  |got - want| <= ulp(got)/2 + ulp(want)/2 + k * 2**-24 * sum|x||w|
    (two roundings to bf16 plus the classic bound on fp32 summation error), elementwise;
    plus the relative Frobenius bound of the layer."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    bound = 0.5 * (bf16_ulp_of(got) + bf16_ulp_of(want)) + k_terms * 2.0 ** -24 * np.asarray(abs_dot)
    err = np.abs(got - want)
    rf = rel_frob(got, want)
    d = ulp_distance(got, want)
    print(f"  {what}: rel_frob={rf:.3e}, {int((d > 0).sum())} of {d.size} differ, "
          f"max err/bound {float(np.max(err / bound)) if err.size else 0:.3f}", flush=True)
    assert rf <= REL_FROB and np.all(err <= bound), what
