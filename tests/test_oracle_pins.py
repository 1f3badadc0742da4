"""Pins that tie the fp64 oracle to what the pages and the mathematics fix.

CPU only.  Each test names the passage (page and section) it rests on.  Taken
together they are meant to fail for any plausible slip in the oracle: a
dropped bonus u, a decay with the wrong sign or offset, a transposed k/v, a
wrong running-max update, a lost prior state.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from oracle.compare import prefix_hull_violation, state_mismatch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _col(x):
    return np.asarray(x, dtype=np.float64).reshape(1, -1, 1)


def _rand_case(rng, B, T, C, k_scale=3.0, w_range=(-5, 1)):
    w = np.exp(rng.uniform(*w_range, size=C))
    u = rng.normal(0, 0.5, size=C)
    k = rng.normal(0, k_scale, size=(B, T, C))
    v = rng.normal(0, 1, size=(B, T, C))
    return k, v, w, u


# ---------------------------------------------------------------------------
# P-1: the worked example (tm_rwkv_math, "A worked example, one channel")
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _example(g):
    i = g["inputs"]
    return _col(i["k"]), _col(i["v"]), np.array([i["w"]]), np.array([i["u"]])


def test_worked_example_output(golden):
    k, v, w, u = _example(golden)
    tol = golden["half_ulp_of_print"]
    y_rec, _ = oracle.forward(k, v, w, u)
    y_dir, _ = oracle.direct(k, v, w, u)
    y_np = oracle.direct_np(k, v, w, u)
    for y in (y_rec, y_dir, y_np):
        assert abs(y[0, 2, 0] - golden["printed"]["wkv_3"]) <= tol
        lo, hi = golden["printed"]["hull"]
        assert lo <= y[0, 2, 0] <= hi


def test_worked_example_terms(golden):
    """The printed terms of wkv_3 follow from the definition's exponents."""
    i = golden["inputs"]
    w, u, k, v = i["w"], i["u"], i["k"], i["v"]
    tol = golden["half_ulp_of_print"]
    assert abs(np.exp(-w) - golden["printed"]["exp_neg_w"]) <= tol
    expo = [-(3 - 1 - 1) * w + k[0], -(3 - 1 - 2) * w + k[1], u + k[2]]
    for x, ww, vv, prod in zip(expo, golden["printed"]["term_weights_at_t3"], v,
                               golden["printed"]["term_products_at_t3"]):
        assert abs(np.exp(x) - ww) <= tol
        assert abs(np.exp(x) * vv - prod) <= tol
    num = sum(np.exp(x) * vv for x, vv in zip(expo, v))
    den = sum(np.exp(x) for x in expo)
    assert abs(num - golden["printed"]["numerator_t3"]) <= tol
    assert abs(den - golden["printed"]["denominator_t3"]) <= 1.5e-4   # rounded-term sum
    # the oracle's output is exactly this ratio
    k3, v3, w3, u3 = _example(golden)
    y, _ = oracle.forward(k3, v3, w3, u3)
    assert y[0, 2, 0] == pytest.approx(num / den, rel=1e-14)


def test_worked_example_naive_state(golden):
    k, v, w, u = _example(golden)
    tol = golden["half_ulp_of_print"]
    _, a_hist, b_hist = oracle.naive(k, v, w, u, np.float64)
    for t in range(2):
        assert abs(a_hist[0, t, 0] - golden["printed"]["naive_a"][t]) <= tol
        assert abs(b_hist[0, t, 0] - golden["printed"]["naive_b"][t]) <= tol


def test_worked_example_stabilised_state(golden):
    """e^p a and e^p b of the stabilised state are the naive accumulators
    (tm_rwkv_math, "Numerical stability: carry the exponent")."""
    k, v, w, u = _example(golden)
    tol = golden["half_ulp_of_print"]
    for T in (1, 2):
        _, (a, b, p) = oracle.forward(k[:, :T], v[:, :T], w, u)
        assert abs(np.exp(p[0, 0]) * a[0, 0] - golden["printed"]["naive_a"][T - 1]) <= tol
        assert abs(np.exp(p[0, 0]) * b[0, 0] - golden["printed"]["naive_b"][T - 1]) <= tol
    # the running maximum after two tokens is max(k1 - w, k2) = max(0.3, 0.0)
    _, (_, _, p) = oracle.forward(k[:, :2], v[:, :2], w, u)
    assert p[0, 0] == pytest.approx(0.3, abs=1e-15)


# ---------------------------------------------------------------------------
# P-2: recurrence == summed form on tiny inputs ("the same arithmetic,
# regrouped": aiwiki, "Why it is both parallel and recurrent")
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_recurrence_equals_summed_form(seed):
    rng = np.random.default_rng(100 + seed)
    T = [1, 2, 7, 33, 64, 50][seed]
    k, v, w, u = _rand_case(rng, 2, T, 5, k_scale=[1, 3, 10, 20, 3, 50][seed])
    y_rec, st_rec = oracle.forward(k, v, w, u)
    y_dir, st_dir = oracle.direct(k, v, w, u)
    y_np = oracle.direct_np(k, v, w, u)
    np.testing.assert_allclose(y_rec, y_dir, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y_np, y_dir, rtol=1e-12, atol=1e-12)
    ea, eb, ep = state_mismatch(st_rec, st_dir)
    assert ea < 1e-12 and eb < 1e-12 and ep < 1e-12


def test_recurrence_equals_summed_form_with_prior_state():
    rng = np.random.default_rng(7)
    k, v, w, u = _rand_case(rng, 3, 40, 4)
    a0 = rng.normal(0, 2, size=(3, 4))
    b0 = rng.uniform(1, 5, size=(3, 4))
    p0 = rng.normal(0, 5, size=(3, 4))
    y_rec, st_rec = oracle.forward(k, v, w, u, state=(a0, b0, p0))
    y_dir, st_dir = oracle.direct(k, v, w, u, state=(a0, b0, p0))
    np.testing.assert_allclose(y_rec, y_dir, rtol=1e-12, atol=1e-12)
    ea, eb, ep = state_mismatch(st_rec, st_dir)
    assert ea < 1e-12 and eb < 1e-12 and ep < 1e-12


def test_sampled_columns_of_workloads_match_summed_form():
    """P-2 at the real sequence lengths of the two smaller workloads, on a few columns."""
    import synth
    for wl, ncols in ((synth.TINY, 64), (synth.SMALL_LM, 4)):
        x = synth.make_forward_inputs(wl)
        cols = np.linspace(0, wl.C - 1, ncols).astype(int)
        k = x.k[:1, :, cols]
        v = x.v[:1, :, cols]
        y_rec, _ = oracle.forward(k, v, x.w[cols], x.u[cols])
        y_dir, _ = oracle.direct(k, v, x.w[cols], x.u[cols])
        np.testing.assert_allclose(y_rec, y_dir, rtol=1e-11, atol=1e-11)


# ---------------------------------------------------------------------------
# P-3: T = 1 returns v exactly (the current token is the only term)
# ---------------------------------------------------------------------------

def test_single_token_returns_v_exactly():
    rng = np.random.default_rng(3)
    k, v, w, u = _rand_case(rng, 4, 1, 33, k_scale=30)
    y, (a, b, p) = oracle.forward(k, v, w, u)
    assert np.array_equal(y, v)
    assert np.array_equal(a, v[:, 0, :]) and np.all(b == 1.0) and np.array_equal(p, k[:, 0, :])


# ---------------------------------------------------------------------------
# P-4: convex combination => inside the prefix hull of v
# (tm_rwkv_math, "The WKV operator": numerator and denominator share weights)
# ---------------------------------------------------------------------------

def test_prefix_hull():
    import synth
    x = synth.make_forward_inputs(synth.TINY)
    y, _ = oracle.forward(x.k, x.v, x.w, x.u)
    assert prefix_hull_violation(y, x.v, 1e-15) == 0.0
    rng = np.random.default_rng(4)
    k, v, w, u = _rand_case(rng, 2, 300, 16, k_scale=20)
    y, _ = oracle.forward(k, v, w, u)
    assert prefix_hull_violation(y, v, 1e-15) == 0.0


# ---------------------------------------------------------------------------
# P-5: the naive form overflows; the stabilised form does not
# (tm_rwkv_math, "Numerical stability"; aiwiki, note under the wkv_step code)
# ---------------------------------------------------------------------------

def _spiky(T, C, spike, seed):
    rng = np.random.default_rng(seed)
    k = rng.normal(0, 1, size=(1, T, C))
    v = rng.normal(0, 1, size=(1, T, C))
    k[:, ::17, :] = spike
    w = np.exp(rng.uniform(-5, 1, size=C))
    u = rng.normal(0, 0.5, size=C)
    return k, v, w, u


def test_naive_overflows_where_stabilised_does_not():
    # fp16: e^40 is far past the largest half (65504 = e^11.09)
    k, v, w, u = _spiky(256, 8, 40.0, 11)
    y16, _, _ = oracle.naive(k, v, w, u, np.float16)
    assert not np.all(np.isfinite(y16))
    # fp32: e^40 = 2.35e17 is still finite, so the pages' "k = 40" does not
    # overflow fp32; e^89 is past FLT_MAX = e^88.72 and does
    y32_40, _, _ = oracle.naive(k, v, w, u, np.float32)
    assert np.all(np.isfinite(y32_40))
    k89, v89, w89, u89 = _spiky(256, 8, 89.0, 12)
    y32, _, _ = oracle.naive(k89, v89, w89, u89, np.float32)
    assert not np.all(np.isfinite(y32))
    # fp64: past e^709.78
    k1k, v1k, w1k, u1k = _spiky(64, 4, 40.0, 13)
    y64, _, _ = oracle.naive(k1k + 1000.0, v1k, w1k, u1k, np.float64)
    assert not np.all(np.isfinite(y64))
    for kk, vv, ww, uu in ((k, v, w, u), (k89, v89, w89, u89), (k1k + 1000.0, v1k, w1k, u1k)):
        y, st = oracle.forward(kk, vv, ww, uu)
        assert np.all(np.isfinite(y)) and all(np.all(np.isfinite(s)) for s in st)
        assert prefix_hull_violation(y, vv, 1e-15) == 0.0
    # where it does not overflow, the naive fp64 form agrees with the oracle
    y_n, _, _ = oracle.naive(k, v, w, u, np.float64)
    y_s, _ = oracle.forward(k, v, w, u)
    np.testing.assert_allclose(y_n, y_s, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# P-6: special cases with independent closed forms
# ---------------------------------------------------------------------------

def test_no_decay_no_bonus_is_causal_softmax_mean():
    """w = 0, u = 0: every past and current token weighs e^{k_i}, so wkv_t is
    the softmax(k_1..k_t)-weighted mean of v_1..v_t."""
    rng = np.random.default_rng(21)
    T, C = 40, 6
    k = rng.normal(0, 4, size=(1, T, C))
    v = rng.normal(0, 1, size=(1, T, C))
    y, _ = oracle.forward(k, v, np.zeros(C), np.zeros(C))
    for t in range(T):
        wts = softmax(k[0, :t + 1, :], axis=0)
        np.testing.assert_allclose(y[0, t], (wts * v[0, :t + 1]).sum(axis=0), rtol=1e-12, atol=1e-13)


def test_constant_values_are_reproduced():
    rng = np.random.default_rng(22)
    k, _, w, u = _rand_case(rng, 2, 50, 7, k_scale=10)
    v = np.full_like(k, 1.75)
    y, _ = oracle.forward(k, v, w, u)
    np.testing.assert_allclose(y, 1.75, rtol=1e-14)


def test_huge_bonus_returns_current_value():
    rng = np.random.default_rng(23)
    k, v, w, _ = _rand_case(rng, 1, 30, 5)
    y, _ = oracle.forward(k, v, w, np.full(5, 1e3))
    np.testing.assert_allclose(y, v, rtol=0, atol=1e-12)


def test_huge_decay_is_two_term_softmax():
    """w = 1e3 wipes everything but the previous token (distance 0 in the
    decay, weight e^{k_{t-1}}) and the current one (weight e^{u+k_t})."""
    rng = np.random.default_rng(24)
    k, v, _, u = _rand_case(rng, 1, 30, 5)
    y, _ = oracle.forward(k, v, np.full(5, 1e3), u)
    for t in range(1, 30):
        z = np.stack([k[0, t - 1], u + k[0, t]])
        wts = softmax(z, axis=0)
        np.testing.assert_allclose(y[0, t], wts[0] * v[0, t - 1] + wts[1] * v[0, t], rtol=1e-12)


def test_constant_keys_no_decay_is_prefix_mean():
    rng = np.random.default_rng(25)
    v = rng.normal(size=(1, 64, 3))
    y, _ = oracle.forward(np.full_like(v, 0.3), v, np.zeros(3), np.zeros(3))
    np.testing.assert_allclose(y, np.cumsum(v, axis=1) / np.arange(1, 65)[None, :, None],
                               rtol=1e-12)


def test_nonzero_bonus_weights_only_the_current_token():
    """With w = 0 and u != 0 the current token weighs e^{u+k_t}, past ones e^{k_i}."""
    rng = np.random.default_rng(26)
    T = 20
    k = rng.normal(0, 2, size=(1, T, 1))
    v = rng.normal(size=(1, T, 1))
    u = 0.8
    y, _ = oracle.forward(k, v, np.zeros(1), np.array([u]))
    for t in range(T):
        wts = np.exp(k[0, :t + 1, 0])
        wts[t] *= np.exp(u)
        assert y[0, t, 0] == pytest.approx((wts * v[0, :t + 1, 0]).sum() / wts.sum(), rel=1e-12)


# ---------------------------------------------------------------------------
# P-7: metamorphic relations
# ---------------------------------------------------------------------------

def test_key_shift_invariance():
    rng = np.random.default_rng(31)
    k, v, w, u = _rand_case(rng, 2, 80, 6)
    y0, (a0, b0, p0) = oracle.forward(k, v, w, u)
    y1, (a1, b1, p1) = oracle.forward(k + 1000.0, v, w, u)
    np.testing.assert_allclose(y1, y0, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(p1 - p0, 1000.0, rtol=0, atol=1e-9)
    np.testing.assert_allclose(a1, a0, rtol=1e-10)
    np.testing.assert_allclose(b1, b0, rtol=1e-10)


def test_value_affine_equivariance():
    rng = np.random.default_rng(32)
    k, v, w, u = _rand_case(rng, 2, 80, 6)
    y0, _ = oracle.forward(k, v, w, u)
    y1, _ = oracle.forward(k, -2.5 * v + 0.75, w, u)
    np.testing.assert_allclose(y1, -2.5 * y0 + 0.75, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("split", [0, 1, 17, 63, 64])
def test_split_and_resume_equals_single_run(split):
    """Serialising the (a,b,p) state and resuming reproduces the single run
    (multigrid.ai, "Prefill, decode, ...": a session resumes from its state)."""
    rng = np.random.default_rng(33)
    k, v, w, u = _rand_case(rng, 2, 64, 5)
    y, st = oracle.forward(k, v, w, u)
    y1, st1 = oracle.forward(k[:, :split], v[:, :split], w, u)
    y2, st2 = oracle.forward(k[:, split:], v[:, split:], w, u, state=st1)
    np.testing.assert_array_equal(np.concatenate([y1, y2], axis=1), y)
    for s, s_ref in zip(st2, st):
        np.testing.assert_array_equal(s, s_ref)


# ---------------------------------------------------------------------------
# P-8: closed form of the state
# ---------------------------------------------------------------------------

def test_state_closed_form():
    rng = np.random.default_rng(41)
    k, v, w, u = _rand_case(rng, 1, 50, 4, k_scale=5)
    for T in (1, 2, 10, 50):
        _, (a, b, p) = oracle.forward(k[:, :T], v[:, :T], w, u)
        i = np.arange(T)
        expo = k[0, :T, :] - (T - 1 - i)[:, None] * w[None, :]
        p_ref = expo.max(axis=0)
        np.testing.assert_allclose(p[0], p_ref, rtol=0, atol=1e-12)
        wts = np.exp(expo - p_ref)
        np.testing.assert_allclose(b[0], wts.sum(axis=0), rtol=1e-12)
        np.testing.assert_allclose(a[0], (wts * v[0, :T]).sum(axis=0), rtol=1e-12, atol=1e-12)
        assert np.all(b[0] >= 1.0 - 1e-15) and np.all(b[0] <= T + 1e-12)


# ---------------------------------------------------------------------------
# Decode step and token shift
# ---------------------------------------------------------------------------

def test_step_chain_equals_forward():
    """Decode (one step per token) and the training form agree (aiwiki, "Why
    it is both parallel and recurrent"); per-layer w,u are indexed by layer."""
    rng = np.random.default_rng(51)
    L, S, C, T = 3, 4, 5, 12
    w = np.exp(rng.uniform(-5, 1, size=(L, C)))
    u = rng.normal(0, 0.5, size=(L, C))
    k = rng.normal(0, 3, size=(L, S, T, C))
    v = rng.normal(size=(L, S, T, C))
    st = (np.zeros((L, S, C)), np.zeros((L, S, C)), np.full((L, S, C), -np.inf))
    ys = []
    for t in range(T):
        y, st = oracle.step(st, k[:, :, t], v[:, :, t], w, u)
        ys.append(y)
    ys = np.stack(ys, axis=2)
    for l in range(L):
        y_ref, st_ref = oracle.forward(k[l], v[l], w[l], u[l])
        np.testing.assert_array_equal(ys[l], y_ref)
        for s, s_ref in zip(st, st_ref):
            np.testing.assert_array_equal(s[l], s_ref)


def test_token_shift_closed_forms():
    """mu = 1 keeps x_t, mu = 0 reads x_{t-1} (tm_rwkv_math, "Token shift")."""
    rng = np.random.default_rng(61)
    B, T, C = 2, 9, 4
    x = rng.normal(size=(B, T, C))
    xp = rng.normal(size=(B, C))
    ones, zeros = np.ones(C), np.zeros(C)
    mu = rng.uniform(0, 1, size=C)
    xr, xk, xv, last = oracle.token_shift(x, ones, zeros, mu, x_prev=xp)
    np.testing.assert_array_equal(xr, x)
    prev = np.concatenate([xp[:, None, :], x[:, :-1, :]], axis=1)
    np.testing.assert_array_equal(xk, prev)
    np.testing.assert_allclose(xv, mu * x + (1 - mu) * prev, rtol=1e-15)
    np.testing.assert_array_equal(last, x[:, -1, :])
    _, xk0, _, _ = oracle.token_shift(x, ones, zeros, mu)
    assert np.all(xk0[:, 0, :] == 0.0)


def test_empty_sequence_passes_state_through():
    rng = np.random.default_rng(71)
    k = np.zeros((2, 0, 3))
    st = (rng.normal(size=(2, 3)), rng.uniform(1, 2, size=(2, 3)), rng.normal(size=(2, 3)))
    y, st_out = oracle.forward(k, k, np.ones(3), np.zeros(3), state=st)
    assert y.shape == (2, 0, 3)
    for s, s_ref in zip(st_out, st):
        np.testing.assert_array_equal(s, s_ref)


# ---------------------------------------------------------------------------
# receptance gate (aicassindra.com tm_rwkv_math, "Receptance: the gate on the
# way out"): o = sigmoid(r) * wkv, sigmoid the logistic function
# ---------------------------------------------------------------------------

def test_sigmoid_closed_forms():
    """Values fixed by the logistic function's definition, which a swapped
    sign, a tanh or a missing 1 would each break."""
    assert oracle.sigmoid(0.0) == 0.5
    # 1 / (1 + e^{-ln 3}) = 1 / (1 + 1/3) = 3/4 and its mirror 1/4
    assert abs(oracle.sigmoid(np.log(3.0)) - 0.75) < 1e-15
    assert abs(oracle.sigmoid(-np.log(3.0)) - 0.25) < 1e-15
    r = np.linspace(-60.0, 60.0, 2401)
    s = oracle.sigmoid(r)
    np.testing.assert_allclose(s + oracle.sigmoid(-r), 1.0, rtol=0, atol=4.5e-16)   # symmetry
    assert np.all(np.diff(s) >= 0) and np.all(s > 0) and np.all(s <= 1)
    # no overflow far out; the limits
    with np.errstate(over="raise", invalid="raise"):
        big = oracle.sigmoid(np.array([-1000.0, 1000.0]))
    assert big[0] == 0.0 and big[1] == 1.0


def test_sigmoid_derivative_identity():
    """sigma' = sigma (1 - sigma), checked by central differences."""
    r = np.linspace(-8.0, 8.0, 65)
    h = 1e-5
    d = (oracle.sigmoid(r + h) - oracle.sigmoid(r - h)) / (2 * h)
    s = oracle.sigmoid(r)
    np.testing.assert_allclose(d, s * (1 - s), rtol=1e-6, atol=1e-10)


def test_gated_forward_special_cases():
    """r = 0 halves the output, r -> +inf passes it, r -> -inf mutes it; the
    state is the plain recurrence's."""
    rng = np.random.default_rng(77)
    B, T, C = 2, 40, 5
    k = rng.normal(0, 2, (B, T, C))
    v = rng.normal(0, 1, (B, T, C))
    w = np.exp(rng.uniform(-3, 1, C))
    u = rng.normal(0, 0.5, C)
    y, st = oracle.forward(k, v, w, u)
    o0, st0 = oracle.forward_gated(k, v, np.zeros_like(k), w, u)
    np.testing.assert_array_equal(o0, y / 2)
    for a, b in zip(st0, st):
        np.testing.assert_array_equal(a, b)
    op, _ = oracle.forward_gated(k, v, np.full_like(k, 50.0), w, u)
    np.testing.assert_allclose(op, y, rtol=1e-20, atol=1e-20 + 2e-22 * np.abs(y).max())
    om, _ = oracle.forward_gated(k, v, np.full_like(k, -800.0), w, u)
    assert np.all(om == 0.0)
    # a gate is applied per element: mixing r between two positions mixes only them
    r = rng.normal(0, 2, (B, T, C))
    o, _ = oracle.forward_gated(k, v, r, w, u)
    np.testing.assert_allclose(o, y / (1 + np.exp(-r)), rtol=1e-15, atol=0)


def test_gated_step_chain_equals_gated_forward():
    rng = np.random.default_rng(78)
    B, T, C = 3, 25, 4
    k = rng.normal(0, 2, (B, T, C))
    v = rng.normal(0, 1, (B, T, C))
    r = rng.normal(0, 2, (B, T, C))
    w = np.exp(rng.uniform(-3, 1, C))
    u = rng.normal(0, 0.5, C)
    o_f, st_f = oracle.forward_gated(k, v, r, w, u)
    st = (np.zeros((1, B, C)), np.zeros((1, B, C)), np.full((1, B, C), -np.inf))
    outs = []
    for t in range(T):
        o_t, st = oracle.step_gated(st, k[None, :, t], v[None, :, t], r[None, :, t], w[None], u[None])
        outs.append(o_t[0])
    np.testing.assert_allclose(np.stack(outs, axis=1), o_f, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# backward: the gradients of the summed definition, pinned by central finite
# differences of the stabilised forward (the C recurrence, a separate code
# path) and by closed forms
# ---------------------------------------------------------------------------

def _loss(k, v, w, u, g):
    y, _ = oracle.forward(k, v, w, u)
    return float((y * g).sum())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_backward_matches_finite_differences(seed):
    rng = np.random.default_rng(300 + seed)
    B, T, C = 2, 9, 3
    k = rng.normal(0, 2, (B, T, C))
    v = rng.normal(0, 1, (B, T, C))
    w = np.exp(rng.uniform(-2, 1, C))
    u = rng.normal(0, 0.7, C)
    g = rng.normal(0, 1, (B, T, C))
    gk, gv, gw, gu = oracle.backward(k, v, w, u, g)
    h = 1e-6
    for arr, grad in ((k, gk), (v, gv)):
        for idx in [(0, 0, 0), (1, 4, 2), (0, 8, 1), (1, 3, 0), (0, 5, 2)]:
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            args_p = (ap, v, w, u, g) if arr is k else (k, ap, w, u, g)
            args_m = (am, v, w, u, g) if arr is k else (k, am, w, u, g)
            fd = (_loss(*args_p) - _loss(*args_m)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-7 * max(1.0, abs(fd)), (idx, fd, grad[idx])
    for c in range(C):
        for arr, grad in ((w, gw), (u, gu)):
            ap, am = arr.copy(), arr.copy()
            ap[c] += h
            am[c] -= h
            args_p = (k, v, ap, u, g) if arr is w else (k, v, w, ap, g)
            args_m = (k, v, am, u, g) if arr is w else (k, v, w, am, g)
            fd = (_loss(*args_p) - _loss(*args_m)) / (2 * h)
            assert abs(fd - grad[c]) <= 1e-7 * max(1.0, abs(fd)), (c, fd, grad[c])


def test_backward_closed_forms():
    """One token: wkv_0 = v_0 whatever k, u, w are.  Constant values: wkv is
    that constant, so nothing but v has a gradient, and gv sums to sum(g)
    (each output's weights sum to one)."""
    rng = np.random.default_rng(310)
    k = rng.normal(0, 2, (3, 1, 4))
    v = rng.normal(0, 1, (3, 1, 4))
    g = rng.normal(0, 1, (3, 1, 4))
    w = np.exp(rng.uniform(-2, 1, 4))
    u = rng.normal(0, 0.5, 4)
    gk, gv, gw, gu = oracle.backward(k, v, w, u, g)
    np.testing.assert_array_equal(gk, 0.0)
    np.testing.assert_allclose(gv, g, rtol=1e-15)
    np.testing.assert_array_equal(gw, 0.0)
    np.testing.assert_array_equal(gu, 0.0)
    B, T, C = 2, 12, 3
    k = rng.normal(0, 2, (B, T, C))
    v = np.full((B, T, C), 0.625)
    g = rng.normal(0, 1, (B, T, C))
    gk, gv, gw, gu = oracle.backward(k, v, w[:C], u[:C], g)
    np.testing.assert_allclose(gk, 0.0, atol=1e-14)
    np.testing.assert_allclose(gw, 0.0, atol=1e-13)
    np.testing.assert_allclose(gu, 0.0, atol=1e-13)
    np.testing.assert_allclose(gv.sum(axis=1), g.sum(axis=1), rtol=1e-12)


def test_backward_magnitude_bounds_and_closed_forms():
    """The term-magnitude sums bound the signed gradients; with gy >= 0 the
    value magnitudes are the signed gv; with constant positive values c
    (wkv = c everywhere) the key magnitude is 2 c gv; one token: gy_0 * 2|v_0|."""
    rng = np.random.default_rng(320)
    B, T, C = 2, 11, 3
    k = rng.normal(0, 2, (B, T, C))
    v = rng.normal(0, 1, (B, T, C))
    w = np.exp(rng.uniform(-2, 1, C))
    u = rng.normal(0, 0.7, C)
    g = rng.normal(0, 1, (B, T, C))
    signed = oracle.backward(k, v, w, u, g)
    mag = oracle.backward(k, v, w, u, g, magnitude=True)
    for s_, m_ in zip(signed, mag):
        assert np.all(m_ >= np.abs(s_) - 1e-13)
    assert np.all(mag[2] > 0) and np.all(mag[3] > 0)
    gpos = np.abs(g)
    np.testing.assert_allclose(oracle.backward(k, v, w, u, gpos, magnitude=True)[1],
                               oracle.backward(k, v, w, u, gpos)[1], rtol=1e-13)
    vc = np.full((B, T, C), 0.625)
    gv_c = oracle.backward(k, vc, w, u, gpos)[1]
    np.testing.assert_allclose(oracle.backward(k, vc, w, u, gpos, magnitude=True)[0],
                               2 * 0.625 * gv_c, rtol=1e-13)
    k1, v1, g1 = k[:, :1], v[:, :1], g[:, :1]
    mk, mv, mw, mu = oracle.backward(k1, v1, w, u, g1, magnitude=True)
    np.testing.assert_allclose(mk, np.abs(g1) * 2 * np.abs(v1), rtol=1e-15)
    np.testing.assert_allclose(mv, np.abs(g1), rtol=1e-15)
    np.testing.assert_array_equal(mw, 0.0)
    np.testing.assert_allclose(mu, (np.abs(g1) * 2 * np.abs(v1)).sum(axis=(0, 1)), rtol=1e-14)
