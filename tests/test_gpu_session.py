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


def _decode_blob(blob, Ln, C):
    """a, b, p [L, C] from a session blob: a 64-byte header (magic "WKVS",
    version, L, C, dtype, number of shift arrays), then a, b, p as fp32
    [L][C] each, little-endian."""
    raw = bytes(blob)
    assert raw[:4] == b"WKVS"
    L_, C_ = np.frombuffer(raw[8:24], dtype="<i8")
    assert (L_, C_) == (Ln, C)
    body = np.frombuffer(raw[64:64 + 12 * Ln * C], dtype="<f4").reshape(3, Ln, C)
    return tuple(body[i].astype(np.float64) for i in range(3))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_resume_matches_the_oracle(device, dtype):
    """A resumed session continues as the oracle does: the oracle, started
    from the a, b, p read back out of the saved bytes, and the oracle run
    without a break both give the resumed slot's outputs (1e-4 guarded
    relative for fp32 storage, 2e-2 for bf16), on keys with 1% at +40."""
    import linear_attention_rnn_forward_amd as wkv
    import oracle
    from oracle.compare import guarded_rel_err
    torch = _torch()
    rng = np.random.default_rng(93)
    Ln, S, C, T = 2, 3, 130, 64
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    w = np.exp(rng.uniform(-5, 1, (Ln, C))).astype(np.float32)
    u = rng.normal(0, 0.5, (Ln, C)).astype(np.float32)
    kh = rng.normal(0, 1, (T, Ln, S, C)).astype(np.float32)
    kh[rng.random(kh.shape) < 0.01] = 40.0
    vh = rng.normal(0, 1, (T, Ln, S, C)).astype(np.float32)
    ks = torch.from_numpy(kh).to(device).to(tdt)
    vs = torch.from_numpy(vh).to(device).to(tdt)
    kh, vh = ks.float().cpu().numpy(), vs.float().cpu().numpy()   # as stored
    wd, ud = torch.from_numpy(w).to(device), torch.from_numpy(u).to(device)
    st = tuple(torch.full((Ln, S, C), f, device=device) for f in (0.0, 0.0, float("-inf")))
    half = T // 2
    for t in range(half):
        _, st = wkv.step(st, ks[t], vs[t], wd, ud)
    blob = wkv.save_session(st, 2)
    torch.cuda.synchronize()
    # resume sequence 2 in slot 0 of a fresh batch
    fresh = tuple(torch.full((Ln, S, C), f, device=device) for f in (0.0, 0.0, float("-inf")))
    wkv.load_session(blob, fresh, 0)
    perm = [2, 0, 1]
    got = []
    for t in range(half, T):
        y, fresh = wkv.step(fresh, ks[t][:, perm].contiguous(), vs[t][:, perm].contiguous(), wd, ud)
        got.append(y[:, 0].float().cpu().numpy())
    torch.cuda.synchronize()
    got = np.stack(got)                                    # [T - half, L, C]
    tol = 2e-2 if dtype == "bf16" else 1e-4
    # the oracle from the saved bytes
    st_o = tuple(x[:, None, :] for x in _decode_blob(blob, Ln, C))   # [L, 1, C]
    ref = []
    for t in range(half, T):
        y_o, st_o = oracle.step(st_o, kh[t][:, 2:3], vh[t][:, 2:3], w, u)
        ref.append(y_o[:, 0])
    ref = np.stack(ref)
    assert guarded_rel_err(got, ref, 1.0) <= tol
    # the oracle without a break (its forward over all T tokens, per layer)
    for l in range(Ln):
        y_full, _ = oracle.forward(kh[:, l, 2][None], vh[:, l, 2][None], w[l], u[l])
        assert guarded_rel_err(got[:, l], y_full[0, half:], 1.0) <= tol, l
