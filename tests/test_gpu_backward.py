"""GPU parity of wkv_backward (gradients of sum(gy * wkv) from the empty
history) against the fp64 oracle, and of wkv_backward_saved, which starts
from the states wkv_forward_save kept instead of recomputing them (the
`saved` cases).

Error measure: each gradient is a sum of terms gy_t alpha[t,i] (v_i - y_t)
(or without the last factor, or weighted by the age t-1-i), so the rounding
error of any fp32 evaluation order is bounded by a small multiple of eps32
times the sum of the terms' magnitudes, which the oracle returns with
magnitude=True.  The measure is max |x - ref| / max(magnitude, 1e-30) (the
floor only covers contributions below fp32's range).  The bar is the
forward's: 1e-4 for fp32 storage; for bf16 storage gk, gv are also rounded
to bf16 once (2^-9 of their magnitude), so 2e-2 as for bf16 outputs; gw, gu
are fp32 outputs in either case and keep 1e-4.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
TOL_WU = 1e-4
FLOOR = 1e-30


def _torch():
    import torch
    return torch


def to_dev(x, dev, bf16_bits=None):
    torch = _torch()
    if bf16_bits is not None:
        return torch.from_numpy(np.ascontiguousarray(bf16_bits).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)


def host(t):
    return t.float().cpu().numpy()


def scaled_err(x, ref, mag):
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0:
        return 0.0
    return float(np.max(np.abs(x - ref) / np.maximum(mag, FLOOR)))


def bf16_exact(a):
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.asarray(a, dtype=np.float32)))


def run_backward(k, v, w, u, g, dtype, dev, saved=False):
    """k, v, g: fp32 arrays (bf16-exact when dtype is bf16).  saved: the
    states from forward_save, then backward from them."""
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    bits = (lambda a: synth.f32_to_bf16_bits(a)) if dtype == "bf16" else (lambda a: None)
    kd, vd, gd = (to_dev(a, dev, bits(a)) for a in (k, v, g))
    wd, ud = to_dev(w, dev), to_dev(u, dev)
    states = wkv.forward_save(kd, vd, wd, ud)[1] if saved else None
    out = wkv.backward(kd, vd, wd, ud, gd, states=states)
    torch.cuda.synchronize()
    return tuple(host(t) for t in out)


SAVED = pytest.mark.parametrize("saved", [False, True], ids=["recompute", "saved"])


def check(k, v, w, u, g, dtype, dev, label="", saved=False):
    got = run_backward(k, v, w, u, g, dtype, dev, saved)
    ref = oracle.backward(k, v, w, u, g)
    mag = oracle.backward(k, v, w, u, g, magnitude=True)
    errs = {}
    for name, x, r, m, tol in zip(("gk", "gv", "gw", "gu"), got, ref, mag,
                                  (TOL[dtype], TOL[dtype], TOL_WU, TOL_WU)):
        assert np.all(np.isfinite(x)), (label, name)
        errs[name] = scaled_err(x, r, m)
        assert errs[name] <= tol, f"{label} {name}: scaled err {errs[name]:.3e} > {tol}"
    return got, errs


def workload_inputs(wl):
    x = synth.make_forward_inputs(wl)
    g, _ = synth.make_output_grad(wl)
    return x.k, x.v, x.w, x.u, g


# ---------------------------------------------------------------------------
# the workload recipes at oracle-sized shapes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,wl", [
    ("tiny", synth.TINY),
    ("small_lm", synth.SMALL_LM.resized(B=2, T=300, C=96)),
    ("bf16_main", synth.BF16_MAIN.resized(B=2, T=512, C=128)),
    ("long_ctx", synth.LONG_CTX.resized(B=1, T=1500, C=40)),
])
@SAVED
def test_workload_recipes(device, name, wl, saved):
    _, errs = check(*workload_inputs(wl), wl.dtype, device, name, saved)
    print(name, {k: f"{v:.2e}" for k, v in errs.items()})


SHAPES = [(1, 1, 1), (1, 2, 3), (3, 17, 5), (1, 16, 256), (2, 33, 257), (1, 129, 64),
          (2, 255, 31), (4, 64, 100)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@SAVED
def test_ragged_shapes(device, shape, dtype, saved):
    B, T, C = shape
    base = synth.BF16_MAIN if dtype == "bf16" else synth.TINY
    wl = base.resized(B=B, T=T, C=C, seed=3000 + B * T + C)
    check(*workload_inputs(wl), dtype, device, f"{shape}", saved)


# ---------------------------------------------------------------------------
# degenerate and stressing inputs
# ---------------------------------------------------------------------------

def test_empty_sequence_zeroes_gw_gu(device):
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    B, C = 2, 300
    k = torch.empty((B, 0, C), device=device)
    w = torch.ones(C, device=device)
    u = torch.zeros(C, device=device)
    gw = torch.full((C,), float("nan"), device=device)
    gu = torch.full((C,), float("nan"), device=device)
    wkv.backward(k, k.clone(), w, u, k.clone(), out=(k.clone(), k.clone(), gw, gu))
    torch.cuda.synchronize()
    assert torch.all(gw == 0) and torch.all(gu == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_token_closed_form(device, dtype):
    """wkv_0 = v_0, so gv = gy and k, w, u get no gradient.  The kernel forms
    the read-out as (c v) (1/c) with c = e^{u-w} (the fold's weights reused),
    so y_0 is v_0 within three roundings (one of them the reciprocal's, within
    1 ulp): |gv - gy| <= 3 * 2^-24 |gy| and |gk|, |gu| <= 4 * 2^-24 |gy v|
    (per element, and summed over the batch for gu).  Rounded to bf16, gv is
    gy exactly (gy is a bf16 value and the error is far below half its ulp).
    gw has no term at all with an empty history: exactly 0."""
    rng = np.random.default_rng(11)
    B, C = 3, 70
    k = rng.normal(0, 3, (B, 1, C)).astype(np.float32)
    v = rng.normal(0, 1, (B, 1, C)).astype(np.float32)
    g = rng.normal(0, 1, (B, 1, C)).astype(np.float32)
    if dtype == "bf16":
        k, v, g = bf16_exact(k), bf16_exact(v), bf16_exact(g)
    w = np.exp(rng.uniform(-5, 1, C)).astype(np.float32)
    u = rng.normal(0, 0.5, C).astype(np.float32)
    gk, gv, gw, gu = run_backward(k, v, w, u, g, dtype, device)
    ulp = 2.0 ** -24
    gd, vd = g.astype(np.float64), v.astype(np.float64)
    if dtype == "bf16":
        np.testing.assert_array_equal(gv, g)
    else:
        assert np.all(np.abs(gv - gd) <= 3 * ulp * np.abs(gd))
    assert np.all(np.abs(gk) <= 4 * ulp * np.abs(gd * vd) * (1 + 2.0 ** -8))
    assert np.all(np.abs(gu) <= 4 * ulp * np.abs(gd * vd).sum(axis=(0, 1)) * (1 + 1e-6))
    np.testing.assert_array_equal(gw, 0.0)


def _cols(B, T, C, seed):
    rng = np.random.default_rng(seed)
    return rng, (rng.normal(0, 1, (B, T, C)).astype(np.float32),
                 rng.normal(0, 1, (B, T, C)).astype(np.float32))


@SAVED
def test_monotone_keys_move_the_anchor_every_token_or_never(device, saved):
    """Rising keys (k_t = 0.5 t) make each token the new maximum, in both
    passes' stabilisation; falling keys never do."""
    B, T, C = 2, 200, 64
    rng, (v, g) = _cols(B, T, C, 12)
    ramp = (0.5 * np.arange(T, dtype=np.float32))[None, :, None]
    w = np.exp(rng.uniform(-5, 1, C)).astype(np.float32)
    u = rng.normal(0, 0.5, C).astype(np.float32)
    for k in (np.broadcast_to(ramp, (B, T, C)).copy(), np.broadcast_to(-ramp, (B, T, C)).copy()):
        check(k, v, w, u, g, "f32", device, "ramp", saved)


@pytest.mark.parametrize("omega", [-8.0, 0.0, 2.0, 3.7, 4.0])
@SAVED
def test_decay_extremes(device, omega, saved):
    """w from e^-8 (a window of thousands of tokens) to e^4 = 55 (only the
    current and the previous token matter; |u - w| > 44 takes the read-out
    with its own exponential)."""
    B, T, C = 1, 700, 48
    rng, (v, g) = _cols(B, T, C, 13)
    k = rng.normal(0, 2, (B, T, C)).astype(np.float32)
    w = np.full(C, np.exp(omega), dtype=np.float32)
    u = rng.normal(0, 0.5, C).astype(np.float32)
    check(k, v, w, u, g, "f32", device, f"omega={omega}", saved)


@SAVED
def test_mixed_read_out_forms(device, saved):
    """Column groups whose channels all have |u - w| <= 44 reuse the fold's
    exponential for the read-out; a group with any other channel takes the
    separate read-out.  Here the first 64 channels have w = e^4 (and the
    next 64 a bonus u = 50), the rest ordinary values, in both dtypes'
    channel grouping."""
    B, T, C = 2, 150, 300
    rng, (v, g) = _cols(B, T, C, 16)
    k = rng.normal(0, 2, (B, T, C)).astype(np.float32)
    w = np.exp(rng.uniform(-5, 1, C)).astype(np.float32)
    u = rng.normal(0, 0.5, C).astype(np.float32)
    w[:64] = np.float32(np.exp(4.0))
    u[64:128] = 50.0
    check(k, v, w, u, g, "f32", device, "mixed f32", saved)
    check(bf16_exact(k), bf16_exact(v), w, u, bf16_exact(g), "bf16", device, "mixed bf16", saved)


@SAVED
def test_keys_far_outside_exp_range(device, saved):
    """k ~ N(0, 30): e^k overflows fp32 for a third of the keys; every
    exponential the kernels take has a non-positive argument."""
    B, T, C = 2, 300, 64
    rng, (v, g) = _cols(B, T, C, 14)
    k = rng.normal(0, 30, (B, T, C)).astype(np.float32)
    w = np.exp(rng.uniform(-5, 1, C)).astype(np.float32)
    u = rng.normal(0, 0.5, C).astype(np.float32)
    check(k, v, w, u, g, "f32", device, "wide keys", saved)


def test_zero_output_gradient_gives_zero(device):
    B, T, C = 2, 100, 40
    rng, (v, _) = _cols(B, T, C, 15)
    k = rng.normal(0, 3, (B, T, C)).astype(np.float32)
    w = np.exp(rng.uniform(-5, 1, C)).astype(np.float32)
    u = rng.normal(0, 0.5, C).astype(np.float32)
    out = run_backward(k, v, w, u, np.zeros_like(v), "f32", device)
    for x in out:
        np.testing.assert_array_equal(x, 0.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unaligned_tensors(device, dtype):
    """k, v, gy, gk, gv at odd element offsets: the kernels read and write
    one element per lane and assume no alignment beyond the element's."""
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    base = synth.BF16_MAIN if dtype == "bf16" else synth.TINY
    wl = base.resized(B=2, T=90, C=70, seed=41)
    k, v, w, u, g = workload_inputs(wl)
    bits = (lambda a: synth.f32_to_bf16_bits(a)) if dtype == "bf16" else (lambda a: None)
    dev = device

    def odd(a):
        t = to_dev(a, dev, bits(a))
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=dev)
        o = buf[1:].view(t.shape)
        o.copy_(t)
        return o

    kd, vd, gd = odd(k), odd(v), odd(g)
    gk, gv = odd(np.zeros_like(k)), odd(np.zeros_like(k))
    gw = torch.empty(wl.C, device=dev)
    gu = torch.empty(wl.C, device=dev)
    wkv.backward(kd, vd, to_dev(w, dev), to_dev(u, dev), gd, out=(gk, gv, gw, gu))
    torch.cuda.synchronize()
    ref = oracle.backward(k, v, w, u, g)
    mag = oracle.backward(k, v, w, u, g, magnitude=True)
    for x, r, m, tol in zip((gk, gv, gw, gu), ref, mag, (TOL[dtype], TOL[dtype], TOL_WU, TOL_WU)):
        assert scaled_err(host(x), r, m) <= tol


@SAVED
def test_deterministic_and_graph_replay(device, saved):
    """Two eager calls agree bit for bit (gw, gu are reduced over the batch
    in a fixed order), and a captured HIP graph replays the same bits."""
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    wl = synth.BF16_MAIN.resized(B=4, T=300, C=200, seed=43)
    k, v, w, u, g = workload_inputs(wl)
    bits = synth.f32_to_bf16_bits
    kd, vd, gd = (to_dev(a, device, bits(a)) for a in (k, v, g))
    wd, ud = to_dev(w, device), to_dev(u, device)
    st = wkv.forward_save(kd, vd, wd, ud)[1] if saved else None
    need = (wkv.backward_saved_workspace_size(wl.B, wl.C) if saved
            else wkv.backward_workspace_size(wl.B, wl.T, wl.C))
    ws = torch.empty(need, dtype=torch.uint8, device=device)
    first = [t.clone() for t in wkv.backward(kd, vd, wd, ud, gd, workspace=ws, states=st)]
    second = wkv.backward(kd, vd, wd, ud, gd, workspace=ws, states=st)
    torch.cuda.synchronize()
    for a, b in zip(first, second):
        assert torch.equal(a, b)
    outs = tuple(torch.empty_like(t) for t in first)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            wkv.backward(kd, vd, wd, ud, gd, out=outs, workspace=ws, states=st)
    torch.cuda.current_stream().wait_stream(s)
    for _ in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(first, outs):
            assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# the full-size workload: B=16, T=4096, C=2048 bf16, sampled columns
# ---------------------------------------------------------------------------

@SAVED
def test_bf16_main_full_size_sampled(device, saved):
    """The bf16 workload at its full size, in the launch bench.py times.
    gk, gv are checked on whole columns (b, c) and gw, gu on one channel
    (all 16 batch rows), each against the oracle run on those columns alone."""
    wl = synth.BF16_MAIN
    k, v, w, u, g = workload_inputs(wl)
    gk, gv, gw, gu = run_backward(k, v, w, u, g, "bf16", device, saved)
    c0 = 1234
    sl = (slice(None), slice(None), slice(c0, c0 + 1))
    ref = oracle.backward(k[sl], v[sl], w[c0:c0 + 1], u[c0:c0 + 1], g[sl])
    mag = oracle.backward(k[sl], v[sl], w[c0:c0 + 1], u[c0:c0 + 1], g[sl], magnitude=True)
    errs = [scaled_err(gk[sl], ref[0], mag[0]), scaled_err(gv[sl], ref[1], mag[1]),
            scaled_err(gw[c0:c0 + 1], ref[2], mag[2]), scaled_err(gu[c0:c0 + 1], ref[3], mag[3])]
    print("channel", c0, [f"{e:.2e}" for e in errs])
    assert errs[0] <= TOL["bf16"] and errs[1] <= TOL["bf16"]
    assert errs[2] <= TOL_WU and errs[3] <= TOL_WU
    for b, c in ((0, 0), (15, 2047), (7, 1023)):
        s1 = (slice(b, b + 1), slice(None), slice(c, c + 1))
        r1 = oracle.backward(k[s1], v[s1], w[c:c + 1], u[c:c + 1], g[s1])
        m1 = oracle.backward(k[s1], v[s1], w[c:c + 1], u[c:c + 1], g[s1], magnitude=True)
        assert scaled_err(gk[s1], r1[0], m1[0]) <= TOL["bf16"], (b, c)
        assert scaled_err(gv[s1], r1[1], m1[1]) <= TOL["bf16"], (b, c)
