"""Known answers for the error measures every parity test relies on.

CPU only.  oracle/compare.py turns a GPU result and an oracle result into the
numbers the tests hold against their bars, so a slip in it (dividing by the
result instead of the reference, dropping the guard, a hull without the
prefix, a state compared without its exponent) would make every parity test
vacuous.  Each measure is checked here against values worked out by hand,
and copies of compare.py with such slips planted in them must fail at least
one of those checks.
"""
import math
import os
import types

import numpy as np
import pytest

from oracle import compare

SRC = os.path.join(os.path.dirname(compare.__file__), "compare.py")


def _battery(m):
    """Run the known-answer checks against the measures of module-like `m`;
    return the names of the checks that fail."""
    failed = []

    def check(name, got, want, tol=1e-12):
        if not (abs(got - want) <= tol):
            failed.append(name)

    # guarded_rel_err: |y - y_ref| / max(|y_ref|, g)
    #   y_ref 0    -> 0.5 / max(0, 1) = 0.5   (the guard takes over at 0)
    #   y_ref 2    -> 0.2 / 2 = 0.1
    #   y_ref -4   -> 0.4 / 4 = 0.1
    check("guarded_basic", m.guarded_rel_err([0.5, 2.2, -4.4], [0.0, 2.0, -4.0], 1.0), 0.5)
    # below the guard the error is absolute over g: 0.1 / 1 (not 0.1 / 0.5)
    check("guarded_below_guard", m.guarded_rel_err([0.6], [0.5], 1.0), 0.1)
    # above it, relative to the reference: 0.3 / 3 (not 0.3 / 3.3)
    check("guarded_reference_scale", m.guarded_rel_err([3.3], [3.0], 1.0), 0.1)
    # the guard scales: g = 4 makes 0.3 / 4
    check("guarded_guard_value", m.guarded_rel_err([3.3], [3.0], 4.0), 0.075)
    # the maximum over elements, whatever their order and shape
    check("guarded_max_2d", m.guarded_rel_err([[1.0, 5.0], [2.0, 9.0]], [[1.0, 4.0], [2.0, 10.0]], 1.0),
          0.25)
    check("guarded_empty", m.guarded_rel_err([], [], 1.0), 0.0)
    check("guarded_exact", m.guarded_rel_err([1.5, -2.0], [1.5, -2.0], 1.0), 0.0)

    # rel_err_where_large: plain relative error over |y_ref| >= g only
    check("large_selects", m.rel_err_where_large([5.0, 2.2, -4.2], [0.1, 2.0, -4.0], 1.0), 0.1)
    check("large_none_selected", m.rel_err_where_large([5.0], [0.1], 1.0), 0.0)
    check("large_boundary_included", m.rel_err_where_large([1.5], [1.0], 1.0), 0.5)

    # prefix_hull_violation over [B, T, C] along T
    v = np.array([1.0, 3.0, 2.0]).reshape(1, 3, 1)
    # the prefix hull at t = 0 is [1, 1]: y = 2 leaves it by 1 (the hull of
    # the whole sequence, [1, 3], would not see it)
    check("hull_prefix", m.prefix_hull_violation(np.full((1, 3, 1), 2.0), v), 1.0)
    # above and below: t=1 hull [1, 3], y = 3.25 -> 0.25; t=2 hull [1, 3], y = 0.5 -> 0.5
    check("hull_both_sides", m.prefix_hull_violation(np.array([1.0, 3.25, 0.5]).reshape(1, 3, 1), v), 0.5)
    check("hull_inside", m.prefix_hull_violation(np.array([1.0, 2.0, 3.0]).reshape(1, 3, 1), v), 0.0)
    # slack widens each bound by slack * |bound|: [1 - 0.5, 1 + 0.5] at t = 0
    check("hull_slack", m.prefix_hull_violation(np.full((1, 3, 1), 2.0), v, 0.5), 0.5)
    # and below: y = 0 at t = 0 against [0.5, 1.5]
    check("hull_slack_below", m.prefix_hull_violation(np.array([0.0, 2.0, 2.0]).reshape(1, 3, 1), v, 0.5),
          0.5)
    # hulls are per batch row and channel, not pooled
    v2 = np.array([[[0.0, 10.0]], [[5.0, -5.0]]])          # [B=2, T=1, C=2]
    y2 = np.array([[[0.0, 10.0]], [[0.0, -5.0]]])          # row 1 channel 0 leaves [5, 5] by 5
    check("hull_per_column", m.prefix_hull_violation(y2, v2), 5.0)

    # state_mismatch: (a, b, p) states compared at the reference's exponent
    ref = (np.array([2.0]), np.array([1.0]), np.array([0.0]))
    # the same accumulators e^p a, e^p b written with p shifted by 1: no mismatch in a, b
    same = (np.array([2.0 / math.e]), np.array([1.0 / math.e]), np.array([1.0]))
    ea, eb, ep = m.state_mismatch(same, ref)
    check("state_equivalent_a", ea, 0.0, 1e-15)
    check("state_equivalent_b", eb, 0.0, 1e-15)
    check("state_equivalent_p", ep, 1.0)
    # a 10% larger a: |2.2 - 2| / max(2, 1 * 1) = 0.1, at either exponent
    ea, eb, ep = m.state_mismatch((np.array([2.2]), np.array([1.0]), np.array([0.0])), ref)
    check("state_a_error", ea, 0.1, 1e-15)
    check("state_a_error_b_clean", eb, 0.0)
    ea, eb, ep = m.state_mismatch((np.array([2.2 / math.e]), np.array([1.0 / math.e]),
                                   np.array([1.0])), ref)
    check("state_a_error_shifted", ea, 0.1, 1e-15)
    # b 25% small: |0.75 - 1| / 1
    ea, eb, ep = m.state_mismatch((np.array([2.0]), np.array([0.75]), np.array([0.0])), ref)
    check("state_b_error", eb, 0.25, 1e-15)
    # a near 0: the guard g * b_ref takes over (0.1 / max(0.01, 2 * 1) = 0.05)
    ea, _, _ = m.state_mismatch((np.array([0.11]), np.array([1.0]), np.array([0.0])),
                                (np.array([0.01]), np.array([1.0]), np.array([0.0])), guard=2.0)
    check("state_a_guard", ea, 0.05, 1e-15)
    # an empty reference entry (p_ref = -inf) is compared on nothing but is not an error;
    # the live entry still counts
    h = math.exp(-0.5)
    ea, eb, ep = m.state_mismatch((np.array([5.0, 2.0 * h]), np.array([3.0, h]), np.array([7.0, 0.5])),
                                  (np.array([0.0, 2.0]), np.array([0.0, 1.0]),
                                   np.array([-np.inf, 0.0])))
    check("state_empty_skipped_a", ea, 0.0, 1e-15)
    check("state_empty_live_p", ep, 0.5)
    return failed


def test_known_answers():
    assert _battery(compare) == []


# Slips planted in copies of compare.py: (old text, new text).  Each copy
# must fail at least one known answer.
MUTANTS = {
    # divide by the result instead of the reference
    "divide_by_result": ("den = np.maximum(np.abs(y_ref), guard)",
                         "den = np.maximum(np.abs(y), guard)"),
    # drop the guard
    "no_guard": ("den = np.maximum(np.abs(y_ref), guard)", "den = np.abs(y_ref) + 1e-300"),
    # guard replaces the reference scale everywhere
    "guard_only": ("den = np.maximum(np.abs(y_ref), guard)", "den = np.full_like(y_ref, guard)"),
    # mean instead of max
    "mean_not_max": ("return float(np.max(np.abs(y - y_ref) / den))",
                     "return float(np.mean(np.abs(y - y_ref) / den))"),
    # vacuous measure
    "returns_zero": ("return float(np.max(np.abs(y - y_ref) / den))", "return 0.0"),
    # where-large selects the small outputs
    "large_inverted": ("sel = np.abs(y_ref) >= guard", "sel = np.abs(y_ref) < guard"),
    # hull of the whole sequence instead of the prefix
    "hull_not_prefix": ("lo = np.minimum.accumulate(v, axis=1)\n    hi = np.maximum.accumulate(v, axis=1)",
                        "lo = np.broadcast_to(v.min(axis=1, keepdims=True), v.shape)\n"
                        "    hi = np.broadcast_to(v.max(axis=1, keepdims=True), v.shape)"),
    # hull taken along the channels
    "hull_wrong_axis": ("lo = np.minimum.accumulate(v, axis=1)\n    hi = np.maximum.accumulate(v, axis=1)",
                        "lo = np.minimum.accumulate(v, axis=2)\n    hi = np.maximum.accumulate(v, axis=2)"),
    # one side of the hull only
    "hull_one_side": ("return float(max(below.max(), above.max()))", "return float(above.max())"),
    # the slack ignored
    "hull_no_slack": ("lo = lo - slack_rel * np.abs(lo)", "lo = lo"),
    # state compared without bringing it to the reference exponent
    "state_no_rescale": ("scale = np.exp(np.where(live, p - pr, 0.0))", "scale = np.ones_like(p)"),
    # exponent difference with the wrong sign
    "state_rescale_sign": ("scale = np.exp(np.where(live, p - pr, 0.0))",
                           "scale = np.exp(np.where(live, pr - p, 0.0))"),
    # a compared without its guard
    "state_a_no_guard": ("ea = np.abs(a_s - ar) / np.maximum(np.abs(ar), guard * np.maximum(br, 1e-300))",
                         "ea = np.abs(a_s - ar) / np.maximum(np.abs(ar), 1e-300)"),
    # b never compared
    "state_b_ignored": ("eb = float(np.max(eb[live])) if live.any() else 0.0", "eb = 0.0"),
}


def _mutant_module(name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"{name}: the text to replace is not unique in compare.py"
    mod = types.ModuleType(f"compare_mutant_{name}")
    exec(compile(src.replace(old, new), f"<compare mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_slip_is_caught(name):
    old, new = MUTANTS[name]
    failed = _battery(_mutant_module(name, old, new))
    assert failed, f"the slip {name} in compare.py passes every known answer"
