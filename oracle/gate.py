"""The graded elementwise accuracy rule (test infrastructure only).

TEST INFRASTRUCTURE ONLY; never imported by the library.

An output element u passes against the reference value r iff
    |u - r| <= 2e-3   OR   |u - r| <= 2e-2 * |r|
(devpost "optimized-gpu-kernels-for-transformer-layers", Inspiration: the
absolute-or-relative rule; devpost "transformerkernel ... Tesla T4",
Inspiration: the same rule with "<=" on every output element).

Readings: the relative rail is taken in the multiplied form so it is defined
at r = 0; the comparison is done in float64; a NaN or infinite u fails where r
is finite; where r is -inf (a row with no visible key, lse only) u must be
exactly -inf.
"""

from __future__ import annotations

import numpy as np

ATOL = 2e-3
RTOL = 2e-2

__all__ = ["gate", "budget_fraction", "ATOL", "RTOL"]


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def gate(u, r):
    """Elementwise pass mask (numpy bool array, shape of r)."""
    u, r = _f64(u), _f64(r)
    if u.shape != r.shape:
        raise ValueError(f"shape mismatch {u.shape} vs {r.shape}")
    finite_r = np.isfinite(r)
    with np.errstate(invalid="ignore"):
        d = np.abs(u - r)
        ok = (d <= ATOL) | (d <= RTOL * np.abs(r))
    ok &= np.isfinite(u) | ~finite_r
    # infinite reference values must be matched exactly (same sign)
    ok = np.where(finite_r, ok, u == r)
    return ok


def budget_fraction(u, r) -> float:
    """max over elements of min(|u-r| / 2e-3, |u-r| / (2e-2 |r|)); <= 1 passes.

    Elements where r is infinite contribute 0 if matched exactly, inf if not.
    A NaN or infinite u against a finite r counts as inf.
    """
    u, r = _f64(u), _f64(r)
    if r.size == 0:
        return 0.0
    finite_r = np.isfinite(r)
    with np.errstate(invalid="ignore", divide="ignore"):
        d = np.abs(u - r)
        fa = d / ATOL
        fr = np.where(r != 0, d / (RTOL * np.abs(r)), np.inf)
        f = np.minimum(fa, fr)
    f = np.where(np.isfinite(u) | ~finite_r, f, np.inf)
    f = np.where(finite_r, f, np.where(u == r, 0.0, np.inf))
    f = np.where(np.isnan(f), np.inf, f)
    return float(f.max())
