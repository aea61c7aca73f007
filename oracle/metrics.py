"""Acceptance metrics for a GEMM result against the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The required bar for BF16 outputs is a per-element relative error of at most
1e-2 and a global similarity defect 1 - 2*sum(xy)/sum(x^2 + y^2) below 1e-3.
The pages state no tolerance of their own; they only say that FP8 tensor-core
accumulation is imprecise and is compensated by promotion (GeekNews topic
19444, opening bullets).

Reading of "per-element relative error <= 1e-2": taken literally it cannot
hold where X cancels to ~0, since any accumulation in any order is off by up
to the rounding bound below.  The per-element test is therefore

    |y - X| <= 1e-2 * |X| + eps,   eps = (2^-14 + 2^-24 * (Kb + 3)) * S

The first term is the matrix core's own sum of a 128-term slice.  The pages
say only that FP8 accumulation inside the matrix core is imprecise and that
promotion at every 128 elements compensates; they give no figure.  Reading:
each slice's partial is within 2^-14 of the slice's magnitude sum(|a*b|)
(the slice magnitudes, times their scales, add up to S).  gfx950's FP8 MFMA
is not a sequence of IEEE fp32 additions: on a one-slice problem it was
measured up to 162 * 2^-24 of S away from the exact sum, beyond the 127
fp32 roundings of a sequential sum; 2^-14 leaves a factor of about 6.  The
second term is fp32 outside the matrix core: one rounding for the scale
product sa*sb, one per slice promotion FMA (Kb of them), one for an addend
and one of slack, each bounded by 2^-24 times a partial sum of magnitudes
<= S.  The final bf16 rounding (relative 2^-8) sits inside the 1e-2 term.
The literal count is reported too, for information.
"""

from __future__ import annotations

import numpy as np

U32 = 2.0 ** -24
SLICE_SUM = 2.0 ** -14  # matrix-core error of one slice, relative to its magnitude


def accumulation_bound(S: np.ndarray, Kb: int) -> np.ndarray:
    """eps per element for a K of Kb 128-slices."""
    return (SLICE_SUM + U32 * (Kb + 3)) * np.asarray(S, np.float64)


def similarity_defect(y, x) -> float:
    """1 - 2*sum(x*y) / sum(x^2 + y^2) over the given elements (float64)."""
    y = np.asarray(y, np.float64).ravel()
    x = np.asarray(x, np.float64).ravel()
    den = float(np.sum(x * x + y * y))
    if den == 0.0:
        return 0.0
    return 1.0 - 2.0 * float(np.sum(x * y)) / den


def check_result(y, X, S, Kb: int, rel: float = 1e-2, sim_max: float = 1e-3) -> dict:
    """Compare a device result y (float64 values of its BF16 output) with X.

    Returns a report dict with ``ok`` True when every element meets the
    per-element bound and the similarity defect is below ``sim_max``.
    """
    y = np.asarray(y, np.float64)
    X = np.asarray(X, np.float64)
    err = np.abs(y - X)
    bound = rel * np.abs(X) + accumulation_bound(S, Kb)
    bad = ~(err <= bound)  # NaN in y counts as bad
    strict_bad = ~(err <= rel * np.abs(X))
    sim = similarity_defect(y, X)
    with np.errstate(divide="ignore", invalid="ignore"):
        relerr = np.where(X != 0, err / np.abs(X), np.where(err == 0, 0.0, np.inf))
    return {
        "ok": bool((not bad.any()) and sim < sim_max),
        "n": int(X.size),
        "n_bad": int(bad.sum()),
        "n_strict_bad": int(strict_bad.sum()),
        "similarity_defect": sim,
        "max_abs_err": float(err.max()) if err.size else 0.0,
        "max_rel_err": float(np.nanmax(relerr)) if relerr.size else 0.0,
    }
