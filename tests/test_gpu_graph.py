"""wkv_forward, wkv_step and wkv_token_shift recorded once in a HIP graph and
replayed several times, with eager launches (sharing the forward workspace)
between the replays: each replay matches an eager launch on the same inputs
(bit for bit where the path's result does not depend on timing, else within
the oracle tolerance)."""
import numpy as np
import pytest

import oracle
import synth
from oracle.compare import guarded_rel_err, rms

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _capture(fn):
    torch = _torch()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    torch.cuda.synchronize()
    return g, out


def _inputs(dev, dtype, seed, B, T, C):
    torch = _torch()
    x = synth.make_forward_inputs(synth.SMALL_LM.resized(B=B, T=T, C=C, seed=seed, dtype=dtype))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    k = torch.from_numpy(x.k).to(dev).to(tdt)
    v = torch.from_numpy(x.v).to(dev).to(tdt)
    return x, k, v, torch.from_numpy(x.w).to(dev), torch.from_numpy(x.u).to(dev)


@pytest.mark.parametrize("path", ["serial", "chained", "chunked"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_forward_graph_replay(device, path, dtype):
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    B, T, C = 2, 700, 256
    x, k, v, w, u = _inputs(device, dtype, 31, B, T, C)
    _, k2, v2, _, _ = _inputs(device, dtype, 32, B, T, C)
    y = torch.empty_like(k)
    st = tuple(torch.empty((B, C), device=device) for _ in range(3))
    run = lambda: wkv.forward(k, v, w, u, out=y, state_out=st, path=path)
    run()
    torch.cuda.synchronize()
    y_eager = y.clone()
    st_eager = tuple(s.clone() for s in st)
    y_ref, _ = oracle.forward(x.k, x.v, x.w, x.u)
    tol = 2e-2 if dtype == "bf16" else 1e-4
    g, _ = _capture(run)
    for rep in range(3):
        y.zero_()
        for s in st:
            s.zero_()
        g.replay()
        torch.cuda.synchronize()
        if path == "chunked":
            # the look-back groups its combines by timing: compare with the oracle
            assert guarded_rel_err(y.float().cpu().numpy(), y_ref, rms(x.v)) <= tol, rep
        else:
            assert torch.equal(y, y_eager), rep
            assert all(torch.equal(a, b) for a, b in zip(st, st_eager)), rep
        if rep == 1:
            # eager work on other inputs between two replays (same workspace and
            # stream); replays 0 and 1 run back to back
            y2 = wkv.forward(k2, v2, w, u, path=path)
            torch.cuda.synchronize()
            assert bool(torch.isfinite(y2.float()).all())


def test_step_graph_replay(device):
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    rng = np.random.default_rng(41)
    Ln, S, C = 3, 8, 512
    w = torch.from_numpy(np.exp(rng.uniform(-5, 1, (Ln, C))).astype(np.float32)).to(device)
    u = torch.from_numpy(rng.normal(0, 0.5, (Ln, C)).astype(np.float32)).to(device)
    ks = torch.from_numpy(rng.normal(0, 2, (4, Ln, S, C)).astype(np.float32)).to(device)
    vs = torch.from_numpy(rng.normal(0, 1, (4, Ln, S, C)).astype(np.float32)).to(device)
    st0 = (torch.zeros(Ln, S, C, device=device), torch.zeros(Ln, S, C, device=device),
           torch.full((Ln, S, C), float("-inf"), device=device))
    st = tuple(s.clone() for s in st0)
    y = torch.empty(Ln, S, C, device=device)

    def run():
        for j in range(4):
            wkv.step(st, ks[j], vs[j], w, u, out=y, inplace=True)

    # eager reference from the initial state
    run()
    torch.cuda.synchronize()
    y_eager, st_eager = y.clone(), tuple(s.clone() for s in st)
    g, _ = _capture(run)
    for rep in range(3):
        for s, s0 in zip(st, st0):
            s.copy_(s0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), rep
        assert all(torch.equal(a, b) for a, b in zip(st, st_eager)), rep
        wkv.step(tuple(s.clone() for s in st0), ks[0], vs[0], w, u)   # eager work between
        torch.cuda.synchronize()


def test_token_shift_graph_replay(device):
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    g0 = torch.Generator(device="cpu").manual_seed(7)
    x = torch.randn((2, 300, 384), generator=g0).to(torch.bfloat16).to(device)
    mus = [torch.rand(384, generator=g0).to(device) for _ in range(3)]
    ref = wkv.token_shift(x, *mus, return_last=True)
    torch.cuda.synchronize()
    g, out = _capture(lambda: wkv.token_shift(x, *mus, return_last=True))
    for rep in range(3):
        for t in out:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(out, ref)), rep
        wkv.token_shift(x.flip(1).contiguous(), *mus)
        torch.cuda.synchronize()


@pytest.mark.parametrize("path", ["chunked", "tokenwise"])
def test_mat_forward_graph_replay(device, path):
    """The matrix-valued-state forward recorded once and replayed three
    times, with eager launches on other inputs in between: every replay
    equals the eager result bit for bit (no timing-dependent order)."""
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    wl = synth.MAT_MAIN.resized(B=2, T=77, H=2, seed=41)
    x = synth.make_mat_inputs(wl)
    dev_b = lambda n: torch.from_numpy(x.bits[n].view(np.int16)).to(device).view(torch.bfloat16)
    r, k, v, z = (dev_b(n) for n in ("r", "k", "v", "z"))
    y = torch.empty_like(k)
    s_out = torch.empty((2, 2, 64, 64), device=device)
    run = lambda: wkv.mat_forward(r, k, v, z, out=y, state_out=s_out, path=path)
    run()
    torch.cuda.synchronize()
    y_eager, s_eager = y.clone(), s_out.clone()
    g, _ = _capture(run)
    other = synth.make_mat_inputs(wl.resized(seed=42))
    r2, k2, v2, z2 = (torch.from_numpy(other.bits[n].view(np.int16)).to(device).view(torch.bfloat16)
                      for n in ("r", "k", "v", "z"))
    for _ in range(3):
        wkv.mat_forward(r2, k2, v2, z2, out=torch.empty_like(k2), path=path)
        y.zero_()
        s_out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager) and torch.equal(s_out, s_eager)


def test_mat_step_graph_replay(device):
    """Four decode steps recorded in one graph (state updated in place) and
    replayed from the same starting state: bit for bit the eager chain."""
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    g_ = torch.Generator(device="cpu").manual_seed(43)
    Ln, S, H = 2, 3, 2
    C = 64 * H
    toks = [tuple(torch.randn((Ln, S, C), generator=g_).to(device) for _ in range(4)) for _ in range(4)]
    st0 = (torch.randn((Ln, S, H, 64, 64), generator=g_) * 0.3).to(device)
    st = st0.clone()
    y = torch.empty((Ln, S, C), device=device)

    def run():
        for r, k, v, z in toks:
            wkv.mat_step(st, r, k, v, z, out=y, inplace=True)

    run()
    torch.cuda.synchronize()
    y_eager, st_eager = y.clone(), st.clone()
    st.copy_(st0)
    g, _ = _capture(run)   # the capture warm-up also runs the steps once
    for _ in range(3):
        st.copy_(st0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager) and torch.equal(st, st_eager)


def test_step_graph_replay_full_size(device):
    """The decode step at the decode workload's size ([32, 256, 4096], state
    updated in place, 4 steps in one graph): each replay equals the eager
    chain bit for bit.  The step stores its outputs at device scope; this
    is the shape at which the chain's bytes far exceed the caches."""
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    Ln, S, C = 32, 256, 4096
    gen = torch.Generator(device="cpu").manual_seed(47)
    w = torch.exp(torch.empty(Ln, C).uniform_(-5, 1, generator=gen)).to(device)
    u = (torch.randn(Ln, C, generator=gen) * 0.5).to(device)
    ks = [(torch.randn(Ln, S, C, generator=gen) * 2).to(device) for _ in range(4)]
    vs = [torch.randn(Ln, S, C, generator=gen).to(device) for _ in range(4)]
    st0 = (torch.rand(Ln, S, C, generator=gen).to(device), torch.rand(Ln, S, C, generator=gen).to(device) + 1,
           torch.randn(Ln, S, C, generator=gen).to(device))
    st = tuple(s.clone() for s in st0)
    y = torch.empty(Ln, S, C, device=device)

    def run():
        for j in range(4):
            wkv.step(st, ks[j], vs[j], w, u, out=y, inplace=True)

    run()
    torch.cuda.synchronize()
    y_eager, st_eager = y.clone(), tuple(s.clone() for s in st)
    assert torch.isfinite(y_eager).all()
    g, _ = _capture(run)
    for rep in range(2):
        for s, s0 in zip(st, st0):
            s.copy_(s0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), rep
        assert all(torch.equal(a, b) for a, b in zip(st, st_eager)), rep


def test_mat_step_graph_replay_full_size(device):
    """The matrix-state step at the matrix decode workload's size (32 x 64
    rows of 64 heads, 2.1 GB of state updated in place, 4 steps in one graph):
    each replay equals the eager chain bit for bit."""
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    Ln, S, H = 32, 64, 64
    C = 64 * H
    gen = torch.Generator(device="cpu").manual_seed(53)
    toks = [tuple(torch.randn((Ln, S, C), generator=gen).to(device) for _ in range(4)) for _ in range(4)]
    st0 = torch.empty((Ln, S, H, 64, 64), device=device).normal_(0.0, 0.3)
    st = st0.clone()
    y = torch.empty((Ln, S, C), device=device)

    def run():
        for r, k, v, z in toks:
            wkv.mat_step(st, r, k, v, z, out=y, inplace=True)

    run()
    torch.cuda.synchronize()
    y_eager, st_eager = y.clone(), st.clone()
    assert torch.isfinite(y_eager).all()
    st.copy_(st0)
    g, _ = _capture(run)
    for rep in range(2):
        st.copy_(st0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), rep
        assert torch.equal(st, st_eager), rep
