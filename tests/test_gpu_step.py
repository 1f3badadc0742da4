"""GPU parity of wkv_step and wkv_token_shift against the fp64 oracle, and of
the device input generator against the host one."""
import numpy as np
import pytest

import oracle
import synth
from oracle.compare import guarded_rel_err, state_mismatch

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def dev_f32(x, dev):
    return _torch().from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)


def host(t):
    return t.float().cpu().numpy()


def _decode_case(rng, Ln, S, C):
    w = np.exp(rng.uniform(-5, 1, (Ln, C))).astype(np.float32)
    u = rng.normal(0, 0.5, (Ln, C)).astype(np.float32)
    return w, u


@pytest.mark.parametrize("C", [4, 64, 4096, 7, 130])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_matches_oracle(device, C, dtype):
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    rng = np.random.default_rng(C)
    Ln, S = 3, 5
    w, u = _decode_case(rng, Ln, S, C)
    st = tuple(torch.full((Ln, S, C), f, device=device) for f in (0.0, 0.0, float("-inf")))
    st_o = (np.zeros((Ln, S, C)), np.zeros((Ln, S, C)), np.full((Ln, S, C), -np.inf))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for t in range(20):
        k = torch.from_numpy(rng.normal(0, 3, (Ln, S, C)).astype(np.float32)).to(device).to(tdt)
        v = torch.from_numpy(rng.normal(0, 1, (Ln, S, C)).astype(np.float32)).to(device).to(tdt)
        y, st = wkv.step(st, k, v, dev_f32(w, device), dev_f32(u, device))
        y_o, st_o = oracle.step(st_o, host(k), host(v), w, u)
        torch.cuda.synchronize()
        tol = 2e-2 if dtype == "bf16" else 1e-4
        assert guarded_rel_err(host(y), y_o, 1.0) <= tol, t
        # the decode state keeps its own anchor: compared at the oracle's exponent
        ea, eb, _ = state_mismatch(tuple(host(s) for s in st), st_o)
        assert ea <= 1e-4 and eb <= 1e-4


def test_step_in_place(device):
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    rng = np.random.default_rng(3)
    Ln, S, C = 2, 4, 256
    w, u = _decode_case(rng, Ln, S, C)
    wd, ud = dev_f32(w, device), dev_f32(u, device)
    st = tuple(torch.full((Ln, S, C), f, device=device) for f in (0.0, 0.0, float("-inf")))
    st_copy = tuple(s.clone() for s in st)
    for t in range(10):
        k = torch.randn(Ln, S, C, device=device)
        v = torch.randn(Ln, S, C, device=device)
        y0, st_copy = wkv.step(st_copy, k, v, wd, ud)
        y1, st_ret = wkv.step(st, k, v, wd, ud, inplace=True)
        torch.cuda.synchronize()
        assert st_ret[0].data_ptr() == st[0].data_ptr()
        assert torch.equal(y0, y1)
        for a, b in zip(st, st_copy):
            assert torch.equal(a, b)


@pytest.mark.parametrize("path", ["serial", "chained", "chunked"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_chain_matches_forward(device, dtype, path):
    """A chain of decode steps reproduces wkv_forward's outputs and final state
    (1e-5 guarded relative for fp32 storage; bf16 outputs may sit one bf16
    rounding apart)."""
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    B, T, C = 6, 300, 192
    x = synth.make_forward_inputs(synth.SMALL_LM.resized(B=B, T=T, C=C, seed=21,
                                                         dtype=dtype))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    k = torch.from_numpy(x.k).to(device).to(tdt)
    v = torch.from_numpy(x.v).to(device).to(tdt)
    w, u = dev_f32(x.w, device), dev_f32(x.u, device)
    y_f, st_f = wkv.forward(k, v, w, u, path=path, return_state=True)
    # decode layout [L=1, S=B, C]
    wl, ul = w[None].contiguous(), u[None].contiguous()
    st = tuple(torch.full((1, B, C), f, device=device) for f in (0.0, 0.0, float("-inf")))
    ys = []
    for t in range(T):
        y, st = wkv.step(st, k[:, t][None].contiguous(), v[:, t][None].contiguous(), wl, ul)
        ys.append(y[0])
    torch.cuda.synchronize()
    y_chain = torch.stack(ys, dim=1)
    tol = 1e-5 if dtype == "f32" else 2.0 ** -7
    assert guarded_rel_err(host(y_chain), host(y_f), 1.0) <= tol
    # the chain's state keeps its own anchor: compared at the forward's exponent
    ea, eb, _ = state_mismatch(tuple(host(s[0]) for s in st), tuple(host(s) for s in st_f))
    assert ea <= 1e-4 and eb <= 1e-4, (ea, eb)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1, 4), (2, 33, 64), (3, 100, 130), (1, 70, 7), (2, 0, 8),
                                   (2, 41, 24), (2, 19, 12), (1, 9, 8)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("with_prev", [False, True])
def test_token_shift_matches_oracle(device, shape, dtype, with_prev):
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    B, T, C = shape
    rng = np.random.default_rng(B * 1000 + T * 10 + C)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.from_numpy(rng.normal(0, 1, (B, T, C)).astype(np.float32)).to(device).to(tdt)
    xp = torch.from_numpy(rng.normal(0, 1, (B, C)).astype(np.float32)).to(device).to(tdt) if with_prev else None
    mus = [rng.uniform(0, 1, C).astype(np.float32) for _ in range(3)]
    xr, xk, xv, last = wkv.token_shift(x, *(dev_f32(m, device) for m in mus), x_prev=xp,
                                       return_last=True)
    torch.cuda.synchronize()
    ref = oracle.token_shift(host(x), *mus, x_prev=None if xp is None else host(xp))
    tol = 2.0 ** -8 if dtype == "bf16" else 1e-6
    for got, want in zip((xr, xk, xv), ref[:3]):
        assert guarded_rel_err(host(got), want, 1.0) <= tol
    np.testing.assert_array_equal(host(last), ref[3])



@pytest.mark.parametrize("offset", [1, 2, 4])
def test_token_shift_on_unaligned_views(device, offset):
    """Arrays that start 2, 4 or 8 bytes past a 16-byte boundary take the
    narrower lane accesses (1, 2 or 4 channels); results match the oracle."""
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    B, T, C = 2, 37, 64
    rng = np.random.default_rng(77 + offset)
    n = B * T * C
    flat = torch.from_numpy(rng.normal(0, 1, n + offset).astype(np.float32)).to(device).to(torch.bfloat16)
    x = flat[offset:].view(B, T, C)
    mus = [rng.uniform(0, 1, C).astype(np.float32) for _ in range(3)]
    outs = [torch.empty(n + offset, device=device, dtype=torch.bfloat16) for _ in range(3)]
    out = tuple(o[offset:].view(B, T, C) for o in outs)
    wkv.token_shift(x, *(dev_f32(m, device) for m in mus), out=out)
    torch.cuda.synchronize()
    ref = oracle.token_shift(host(x), *mus)
    for got, want in zip(out, ref[:3]):
        assert guarded_rel_err(host(got), want, 1.0) <= 2.0 ** -8


def test_device_generator_matches_host(device):
    import synth.device as sd
    torch = _torch()
    wl = synth.DECODE
    out_k = torch.empty((2, wl.L, wl.S, 64), device=device)
    out_v = torch.empty_like(out_k)
    # two decode steps, first 64 channels of each (layer, seq)
    dims = (2, wl.L, wl.S, 64)
    S, Tt, C = wl.S, wl.total_T, wl.C
    strides = (C, S * Tt * C, Tt * C, 1)
    base = (wl.prefill_T + 5) * C
    sd.fill_normal(out_k, dims, strides, base, synth.STREAM_K, wl.seed)
    sd.fill_normal(out_v, dims, strides, base, synth.STREAM_V, wl.seed)
    torch.cuda.synchronize()
    lay = np.arange(wl.L)[None, :, None, None]
    seq = np.arange(wl.S)[None, None, :, None]
    tok = (wl.prefill_T + 5 + np.arange(2))[:, None, None, None]
    ch = np.arange(64)[None, None, None, :]
    ctr = synth.decode_counter(wl, lay, seq, tok, ch)
    np.testing.assert_array_equal(out_k.cpu().numpy(), synth.philox_normal(ctr, synth.STREAM_K, wl.seed))
    np.testing.assert_array_equal(out_v.cpu().numpy(), synth.philox_normal(ctr, synth.STREAM_V, wl.seed))


# ---------------------------------------------------------------------------
# the decode chain on keys the pages warn about: 1% of keys at +40
# ([tm-math] "Numerical stability: carry the exponent"), long enough for the
# state's exponent to sit behind a large key for hundreds of tokens
# ---------------------------------------------------------------------------

def _spiky_chain(device, B, T, C, seed, gated):
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    x = synth.make_forward_inputs(synth.TINY.resized(B=B, T=T, C=C, seed=seed))
    k, v = dev_f32(x.k, device), dev_f32(x.v, device)
    w, u = dev_f32(x.w, device), dev_f32(x.u, device)
    r_host = rd = None
    if gated:
        r_host, _ = synth.make_receptance(synth.TINY.resized(B=B, T=T, C=C, seed=seed))
        rd = dev_f32(r_host, device)
    y_f, st_f = wkv.forward(k, v, w, u, return_state=True, r=rd)
    wl, ul = w[None].contiguous(), u[None].contiguous()
    st = tuple(torch.full((1, B, C), f, device=device) for f in (0.0, 0.0, float("-inf")))
    ys = []
    for t in range(T):
        rt = None if rd is None else rd[:, t][None].contiguous()
        y, st = wkv.step(st, k[:, t][None].contiguous(), v[:, t][None].contiguous(), wl, ul, r=rt)
        ys.append(y[0])
    torch.cuda.synchronize()
    y_chain = host(torch.stack(ys, dim=1))
    if gated:
        y_ref, st_ref = oracle.forward_gated(x.k, x.v, r_host, x.w, x.u)
    else:
        y_ref, st_ref = oracle.forward(x.k, x.v, x.w, x.u)
    assert np.all(np.isfinite(y_chain))
    e_fwd = guarded_rel_err(y_chain, host(y_f), 1.0)
    e_orc = guarded_rel_err(y_chain, y_ref, 1.0)
    e_fwd_orc = guarded_rel_err(host(y_f), y_ref, 1.0)
    ea, eb, _ = state_mismatch(tuple(host(s[0]) for s in st), st_ref)
    print(f"spiky chain B={B} T={T} C={C} gated={gated}: chain vs forward {e_fwd:.2e}, "
          f"chain vs oracle {e_orc:.2e}, forward vs oracle {e_fwd_orc:.2e}, state {ea:.2e} {eb:.2e}")
    return e_fwd, e_orc, ea, eb


@pytest.mark.parametrize("gated", [False, True], ids=["plain", "gated"])
@pytest.mark.parametrize("shape", [(4, 256, 64), (2, 1024, 256)], ids=["T256", "T1024"])
def test_step_chain_on_spiky_keys(device, shape, gated):
    """The decode chain follows wkv_forward to 1e-5 (guarded relative) and the
    oracle to 1e-4 on the overflow-probe recipe, where a key of +40 dominates
    the history for hundreds of tokens; the chain's final state equals the
    oracle's to 1e-4 (compared at the oracle's exponent: the decode state
    keeps its own anchor, which need not be the running maximum)."""
    B, T, C = shape
    e_fwd, e_orc, ea, eb = _spiky_chain(device, B, T, C, 300 + T, gated)
    assert e_fwd <= 1e-5
    assert e_orc <= 1e-4
    assert ea <= 1e-4 and eb <= 1e-4
