"""Session save and resume ([multigrid] = multigrid.ai rwkv, "The state, in
bytes": a session's state can be serialised and resumed elsewhere at full
fidelity): the state of one sequence of a decode batch goes to host bytes and
back into another slot (or another batch), and decoding continues exactly as
if it had never stopped."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_save_load_round_trip_and_resume(device, dtype):
    import linear_attention_rnn_forward_amd as wkv
    torch = _torch()
    rng = np.random.default_rng(91)
    Ln, S, C, T = 3, 4, 192, 40
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    w = torch.from_numpy(np.exp(rng.uniform(-4, 1, (Ln, C))).astype(np.float32)).to(device)
    u = torch.from_numpy(rng.normal(0, 0.5, (Ln, C)).astype(np.float32)).to(device)
    ks = torch.from_numpy(rng.normal(0, 2, (T, Ln, S, C)).astype(np.float32)).to(device).to(tdt)
    vs = torch.from_numpy(rng.normal(0, 1, (T, Ln, S, C)).astype(np.float32)).to(device).to(tdt)
    empty = lambda: tuple(torch.full((Ln, S, C), f, device=device) for f in (0.0, 0.0, float("-inf")))

    # an uninterrupted run of T steps
    st = empty()
    ys = []
    for t in range(T):
        y, st = wkv.step(st, ks[t], vs[t], w, u)
        ys.append(y)
    torch.cuda.synchronize()

    # half the steps, then sequence 1 is saved (with a shifted-token array
    # standing in for the token-shift state) and resumed in slot 3 of a fresh
    # batch whose other sequences are left as they are
    st2 = empty()
    for t in range(T // 2):
        _, st2 = wkv.step(st2, ks[t], vs[t], w, u)
    shift = ks[T // 2 - 1].clone()
    blob = wkv.save_session(st2, 1, shifts=(shift,))
    assert len(blob) == wkv.session_bytes(Ln, C, wkv.BF16 if dtype == "bf16" else wkv.F32, 1)
    fresh = empty()
    fresh_shift = torch.zeros_like(shift)
    untouched = fresh[0][:, 0].clone()
    wkv.load_session(blob, fresh, 3, shifts=(fresh_shift,))
    for a, b in zip(fresh, st2):
        assert torch.equal(a[:, 3], b[:, 1])
    assert torch.equal(fresh_shift[:, 3], shift[:, 1])
    assert torch.equal(fresh[0][:, 0], untouched)
    # continue: the resumed slot 3 fed sequence 1's tokens equals the uninterrupted run
    perm = [0, 2, 3, 1]   # slot 3 <- sequence 1
    for t in range(T // 2, T):
        y, fresh = wkv.step(fresh, ks[t][:, perm].contiguous(), vs[t][:, perm].contiguous(), w, u)
        torch.cuda.synchronize()
        assert torch.equal(y[:, 3], ys[t][:, 1]), t
