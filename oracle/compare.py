"""Error measures used when a result is compared with the oracle.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

wkv_t is a convex combination of zero-mean values, so it crosses zero and a
plain |y - y_ref| / |y_ref| is unbounded near those crossings.  The guarded
relative error divides by max(|y_ref|, g), with the guard g the RMS of the
values v the outputs are averages of (about 1 for every workload here).
"""
from __future__ import annotations

import numpy as np


def rms(x) -> float:
    x = np.asarray(x, dtype=np.float64)
    return float(np.sqrt(np.mean(x * x))) if x.size else 1.0


def guarded_rel_err(y, y_ref, guard: float) -> float:
    """max_i |y_i - y_ref_i| / max(|y_ref_i|, guard); 0 for empty inputs."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y.size == 0:
        return 0.0
    den = np.maximum(np.abs(y_ref), guard)
    return float(np.max(np.abs(y - y_ref) / den))


def rel_err_where_large(y, y_ref, guard: float) -> float:
    """Plain relative error over the outputs with |y_ref| >= guard."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    sel = np.abs(y_ref) >= guard
    if not sel.any():
        return 0.0
    return float(np.max(np.abs(y[sel] - y_ref[sel]) / np.abs(y_ref[sel])))


def prefix_hull_violation(y, v, slack_rel: float = 0.0) -> float:
    """Largest distance by which y[:, t, :] leaves [min v[:, :t+1, :], max v[:, :t+1, :]].

    The bound is widened by slack_rel * max(|bound|) to allow for the rounding
    of the stored output.  Returns 0 when every output is inside its hull.
    """
    y = np.asarray(y, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lo = np.minimum.accumulate(v, axis=1)
    hi = np.maximum.accumulate(v, axis=1)
    lo = lo - slack_rel * np.abs(lo)
    hi = hi + slack_rel * np.abs(hi)
    below = np.maximum(lo - y, 0.0)
    above = np.maximum(y - hi, 0.0)
    if y.size == 0:
        return 0.0
    return float(max(below.max(), above.max()))


def state_mismatch(state, state_ref, guard: float = 1.0) -> tuple:
    """Compare two (a, b, p) states that may use different exponents p.

    Both are brought to the reference exponent: a * e^{p - p_ref}.  Returns
    (max relative error of the rescaled a, of the rescaled b, max |p - p_ref|).
    Entries where the reference is the empty history (p_ref = -inf) are
    compared on p only.
    """
    a, b, p = (np.asarray(s, dtype=np.float64) for s in state)
    ar, br, pr = (np.asarray(s, dtype=np.float64) for s in state_ref)
    live = np.isfinite(pr) & (pr > -1e30)
    with np.errstate(all="ignore"):
        scale = np.exp(np.where(live, p - pr, 0.0))
        a_s = a * scale
        b_s = b * scale
        ea = np.abs(a_s - ar) / np.maximum(np.abs(ar), guard * np.maximum(br, 1e-300))
        eb = np.abs(b_s - br) / np.maximum(np.abs(br), 1e-300)
        ep = np.abs(p - pr)
    ea = float(np.max(ea[live])) if live.any() else 0.0
    eb = float(np.max(eb[live])) if live.any() else 0.0
    ep = float(np.max(ep[live])) if live.any() else 0.0
    return ea, eb, ep
