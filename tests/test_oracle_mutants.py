"""The pins catch plausible mistakes planted in copies of the oracle.

CPU only.  Each mutant is wkv_oracle.c with one slip substituted in (a wrong
decay sign, a dropped bonus, a transposed operand, ...), built with gcc into
a temporary directory.  The check battery below is a subset of the pins in
test_oracle_pins.py; every mutant must fail at least one of them.  The real
oracle passes them all.
"""
import json
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import build as oracle_build

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")

MUTANTS = {
    # fold-in decays with the wrong sign (the negative-w convention applied to positive w)
    "decay_sign": ("scaled_weights(*p - w, k, &hist, &cur)", "scaled_weights(*p + w, k, &hist, &cur)"),
    # read-out forgets the current-token bonus
    "no_bonus": ("scaled_weights(*p, u + k, &hist, &cur)", "scaled_weights(*p, k, &hist, &cur)"),
    # read-out decays the history once too often
    "extra_decay": ("scaled_weights(*p, u + k, &hist, &cur)", "scaled_weights(*p - w, u + k, &hist, &cur)"),
    # numerator takes a where v belongs
    "transposed_av": ("double y = (hist * *a + cur * v)", "double y = (hist * v + cur * *a)"),
    # state update adds the bonus too
    "bonus_in_state": ("scaled_weights(*p - w, k, &hist, &cur)", "scaled_weights(*p - w, u + k, &hist, &cur)"),
    # the common scale is not the larger exponent (the ratio survives, the state's p does not)
    "scale_not_max": ("double m = fmax(x1, x2);", "double m = x2;"),
    # denominator drops the history
    "den_no_history": ("/ (hist * *b + cur);", "/ (cur);"),
    # decay per channel read with the batch index
    "wrong_param_index": ("stabilised_token(&a, &b, &p, k[i], v[i], w[c], u[c])",
                          "stabilised_token(&a, &b, &p, k[i], v[i], w[bb], u[c])"),
}


def _checks_fail():
    """Run the check battery on whatever library the oracle is bound to; return
    the names of the checks that fail."""
    with open(GOLDEN) as f:
        g = json.load(f)
    failed = []
    i = g["inputs"]
    k = np.array(i["k"]).reshape(1, 3, 1)
    v = np.array(i["v"]).reshape(1, 3, 1)
    y, _ = oracle.forward(k, v, np.array([i["w"]]), np.array([i["u"]]))
    if abs(y[0, 2, 0] - g["printed"]["wkv_3"]) > g["half_ulp_of_print"]:
        failed.append("worked_example")
    for T in (1, 2):
        _, (a, b, p) = oracle.forward(k[:, :T], v[:, :T], np.array([i["w"]]), np.array([i["u"]]))
        if abs(np.exp(p[0, 0]) * a[0, 0] - g["printed"]["naive_a"][T - 1]) > 5e-5:
            failed.append("worked_example_state")
    rng = np.random.default_rng(5)
    B, T, C = 2, 24, 3
    w = np.exp(rng.uniform(-3, 1, size=C))
    u = rng.normal(0, 0.5, size=C)
    kk = rng.normal(0, 3, size=(B, T, C))
    vv = rng.normal(size=(B, T, C))
    y, (a, b, p) = oracle.forward(kk, vv, w, u)
    if not np.allclose(y, oracle.direct_np(kk, vv, w, u), rtol=1e-10, atol=1e-10):
        failed.append("summed_form")
    expo = kk - (T - 1 - np.arange(T))[None, :, None] * w[None, None, :]
    if not np.allclose(p, expo.max(axis=1), rtol=0, atol=1e-10):
        failed.append("state_closed_form")
    return failed


def _build_mutant(tmp_path, name, old, new):
    src = open(oracle_build.SRC).read()
    assert src.count(old) == 1, name
    mpath = tmp_path / f"mut_{name}.c"
    mpath.write_text(src.replace(old, new))
    lib = tmp_path / f"libmut_{name}.so"
    subprocess.run(["gcc", *oracle_build.CFLAGS, "-w", "-o", str(lib), str(mpath), "-lm"],
                   check=True)
    return str(lib)


def test_real_oracle_passes_the_battery():
    assert _checks_fail() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    lib = _build_mutant(tmp_path, name, old, new)
    with oracle.library(lib):
        failed = _checks_fail()
    assert failed, f"mutant {name} passed every pin"


# ---------------------------------------------------------------------------
# the receptance gate's logistic function (NumPy side of the oracle)
# ---------------------------------------------------------------------------

SIGMOID_MUTANTS = {
    "negated_argument": lambda r: 1.0 / (1.0 + np.exp(r)),
    "tanh": np.tanh,
    "missing_one": lambda r: np.exp(r),
    "half_slope": lambda r: 1.0 / (1.0 + np.exp(-r / 2)),
    "shifted": lambda r: 1.0 / (1.0 + np.exp(-(r + 0.1))),
}


def _sigmoid_checks_fail(sig):
    """The closed-form pins of test_oracle_pins.py, applied to `sig`."""
    failed = []
    if sig(np.float64(0.0)) != 0.5:
        failed.append("half_at_zero")
    if abs(sig(np.log(3.0)) - 0.75) > 1e-15:
        failed.append("three_quarters_at_ln3")
    r = np.linspace(-30.0, 30.0, 601)
    if np.max(np.abs(sig(r) + sig(-r) - 1.0)) > 4.5e-16:
        failed.append("symmetry")
    h = 1e-5
    rr = np.linspace(-8.0, 8.0, 65)
    d = (sig(rr + h) - sig(rr - h)) / (2 * h)
    s = sig(rr)
    if not np.allclose(d, s * (1 - s), rtol=1e-6, atol=1e-10):
        failed.append("derivative")
    return failed


def test_real_sigmoid_passes_its_pins():
    assert _sigmoid_checks_fail(oracle.sigmoid) == []


@pytest.mark.parametrize("name", sorted(SIGMOID_MUTANTS))
def test_sigmoid_mutant_is_caught(name):
    with np.errstate(over="ignore", invalid="ignore"):
        assert _sigmoid_checks_fail(SIGMOID_MUTANTS[name]), name
