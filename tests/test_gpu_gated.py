"""GPU parity of the receptance-gated forms (o = sigmoid(r) * wkv, the gate
of aicassindra.com tm_rwkv_math, "Receptance: the gate on the way out")
against the fp64 oracle: every forward path, both storage types, ragged
shapes, the decode step, and the gate's limits.

Bar: guarded relative error (oracle/compare.py) <= 1e-4 for fp32 storage,
<= 2e-2 for bf16; the state outputs equal the ungated call's bit for bit
(the gate does not enter the recurrence)."""
import numpy as np
import pytest

import oracle
import synth
from oracle.compare import guarded_rel_err, rms, state_mismatch

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _torch():
    import torch
    return torch


def host(t):
    return t.float().cpu().numpy()


def _inputs(dev, wl):
    torch = _torch()
    x = synth.make_forward_inputs(wl)
    r, r_bits = synth.make_receptance(wl)
    if wl.dtype == "bf16":
        to = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
        k, v, rd = to(x.k_bits), to(x.v_bits), to(r_bits)
    else:
        k, v, rd = (torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in (x.k, x.v, r))
    return x, r, k, v, rd, torch.from_numpy(x.w).to(dev), torch.from_numpy(x.u).to(dev)


SHAPES = [(1, 1, 64), (2, 33, 128), (3, 100, 130), (1, 700, 256), (2, 257, 192), (1, 40, 7)]


@pytest.mark.parametrize("path", ["serial", "chained", "chunked"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_gated_forward_matches_oracle(device, path, dtype, shape):
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    B, T, C = shape
    wl = synth.SMALL_LM.resized(B=B, T=T, C=C, seed=50 + T + C, dtype=dtype)
    x, r, k, v, rd, w, u = _inputs(device, wl)
    o, st = wkv.forward(k, v, w, u, r=rd, path=path, return_state=True)
    y, st_plain = wkv.forward(k, v, w, u, path=path, return_state=True)
    torch.cuda.synchronize()
    o_ref, st_ref = oracle.forward_gated(x.k, x.v, r, x.w, x.u)
    err = guarded_rel_err(host(o), o_ref, rms(x.v))
    assert err <= TOL[dtype], f"path={path} gated rel err {err:.3e}"
    ea, eb, ep = state_mismatch(tuple(host(s) for s in st), st_ref)
    assert ea <= 1e-4 and eb <= 1e-4 and ep <= 1e-4, (ea, eb, ep)
    if path != "chunked":   # timing-independent paths: the same state as the plain call
        for a, b in zip(st, st_plain):
            assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gated_bf16_main_workload(device, dtype):
    """The bf16 B=16 T=4096 C=2048 workload (and its fp32 twin at a quarter
    of the rows), gated, in the default launch configuration."""
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    wl = synth.BF16_MAIN if dtype == "bf16" else synth.BF16_MAIN.resized(B=4, dtype="f32")
    x, r, k, v, rd, w, u = _inputs(device, wl)
    o = wkv.forward(k, v, w, u, r=rd)
    torch.cuda.synchronize()
    o_ref, _ = oracle.forward_gated(x.k, x.v, r, x.w, x.u)
    err = guarded_rel_err(host(o), o_ref, rms(x.v))
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("path", ["serial", "chained", "chunked"])
def test_gate_limits(device, path):
    """r = 0 halves the plain output exactly; r = +200 passes it unchanged;
    r = -200 mutes it to 0."""
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    wl = synth.SMALL_LM.resized(B=2, T=300, C=192, seed=61)
    x, _, k, v, _, w, u = _inputs(device, wl)
    y = wkv.forward(k, v, w, u, path=path)
    o0 = wkv.forward(k, v, w, u, r=torch.zeros_like(k), path=path)
    op = wkv.forward(k, v, w, u, r=torch.full_like(k, 200.0), path=path)
    om = wkv.forward(k, v, w, u, r=torch.full_like(k, -200.0), path=path)
    torch.cuda.synchronize()
    if path == "chunked":
        tol = lambda a, b: guarded_rel_err(host(a), host(b), 1.0) <= 1e-6
        assert tol(o0, y / 2) and tol(op, y)
    else:
        assert torch.equal(o0, y / 2)
        assert torch.equal(op, y)
    assert bool((om == 0).all())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("C", [64, 130])
def test_gated_step_matches_oracle_and_forward(device, dtype, C):
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    B, T = 3, 120
    wl = synth.SMALL_LM.resized(B=B, T=T, C=C, seed=70 + C, dtype=dtype)
    x, r, k, v, rd, w, u = _inputs(device, wl)
    o_f = wkv.forward(k, v, w, u, r=rd)
    wl_, ul_ = w[None].contiguous(), u[None].contiguous()
    st = tuple(torch.full((1, B, C), f, device=device) for f in (0.0, 0.0, float("-inf")))
    st_o = (np.zeros((1, B, C)), np.zeros((1, B, C)), np.full((1, B, C), -np.inf))
    outs = []
    for t in range(T):
        kt, vt, rt = (a[:, t][None].contiguous() for a in (k, v, rd))
        o_t, st = wkv.step(st, kt, vt, wl_, ul_, r=rt)
        outs.append(o_t[0])
        if t < 8:
            o_ref, st_o = oracle.step_gated(st_o, x.k[None, :, t], x.v[None, :, t], r[None, :, t],
                                            x.w[None], x.u[None])
            torch.cuda.synchronize()
            assert guarded_rel_err(host(o_t), o_ref, 1.0) <= TOL[dtype], t
    torch.cuda.synchronize()
    chain = torch.stack(outs, dim=1)
    tol = 1e-5 if dtype == "f32" else 2.0 ** -7
    assert guarded_rel_err(host(chain), host(o_f), 1.0) <= tol


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("dtype,C", [("f32", 768), ("bf16", 1536)])
def test_chunked_wide_tiles_match_oracle(device, dtype, C, gated):
    """96 column groups over 1000 tokens: 384 tiles of 8 waves would outnumber
    the 256 CUs while 192 tiles of 16 waves do not, so the chunked path takes
    the 16-wave tiles (a ragged last tile included); plain and gated outputs
    and the final state against the oracle."""
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    wl = synth.SMALL_LM.resized(B=8, T=1000, C=C, seed=71, dtype=dtype)
    x, r, k, v, rd, w, u = _inputs(device, wl)
    out, st = wkv.forward(k, v, w, u, r=rd if gated else None, path="chunked", return_state=True)
    torch.cuda.synchronize()
    if gated:
        ref, st_ref = oracle.forward_gated(x.k, x.v, r, x.w, x.u)
    else:
        ref, st_ref = oracle.forward(x.k, x.v, x.w, x.u)
    err = guarded_rel_err(host(out), ref, rms(x.v))
    assert np.all(np.isfinite(host(out)))
    assert err <= TOL[dtype], f"rel err {err:.3e}"
    ea, eb, ep = state_mismatch(tuple(host(s) for s in st), st_ref)
    assert ea <= 1e-4 and eb <= 1e-4 and ep <= 1e-4, (ea, eb, ep)
