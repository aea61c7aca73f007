"""Acceptance metrics for a GEMM result against the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The required bar for BF16 outputs is a per-element relative error of at most
1e-2 and a global similarity defect 1 - 2*sum(xy)/sum(x^2 + y^2) below 1e-3.
The pages state no tolerance of their own; they only say that FP8 tensor-core
accumulation is imprecise and is compensated by promotion (GeekNews topic
19444, opening bullets).

Reading of "per-element relative error <= 1e-2": taken literally it cannot
hold where X cancels to ~0, since any fp32 accumulation in any order is off
by up to the rounding bound below.  The per-element test is therefore

    |y - X| <= 1e-2 * |X| + eps,   eps = 2^-24 * (128 + Kb + 2) * S

eps is the first-order worst case of fp32 accumulation: up to 127 roundings
inside a 128-term slice sum, one for the scale product sa*sb, one per slice
promotion FMA (Kb of them), and one more of slack; each rounding is bounded
by 2^-24 times a partial sum of magnitudes <= S.  The final bf16 rounding
(relative 2^-8) sits inside the 1e-2 term.  The literal count is reported
too, for information.
"""

from __future__ import annotations

import numpy as np

U32 = 2.0 ** -24


def accumulation_bound(S: np.ndarray, Kb: int) -> np.ndarray:
    """eps per element for a K of Kb 128-slices."""
    return U32 * (128 + Kb + 2) * np.asarray(S, np.float64)


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
