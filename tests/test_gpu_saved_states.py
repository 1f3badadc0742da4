"""wkv_forward_save: its output is the chained forward's, bit for bit (the
same kernel, with the carries stored besides), and its states are the
recurrence's state before every 16-token sub-chunk, checked against the
oracle's state after the same prefix ([tm-math] "Numerical stability: carry
the exponent": the state is the pair of sums scaled by e^{-p}; only
a e^p, b e^p are fixed, so the comparison is on those, state_mismatch).
The backward from these states is checked in test_gpu_backward.py."""
import numpy as np
import pytest

import oracle
import synth
from oracle.compare import state_mismatch

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1, 3), (2, 16, 64), (2, 33, 130), (1, 200, 257), (3, 97, 128)]


def _inputs(B, T, C, dtype, seed):
    base = synth.BF16_MAIN if dtype == "bf16" else synth.TINY
    wl = base.resized(B=B, T=T, C=C, seed=seed)
    x = synth.make_forward_inputs(wl)
    return x, wl


def _dev(x, bits, device):
    import torch
    if bits is not None:
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_forward_save_output_and_states(device, shape, dtype):
    import torch
    import linear_attention_rnn_forward_amd as wkv
    B, T, C = shape
    x, wl = _inputs(B, T, C, dtype, 5000 + B * T + C)
    kd = _dev(x.k, x.k_bits, device)
    vd = _dev(x.v, x.v_bits, device)
    wd, ud = _dev(x.w, None, device), _dev(x.u, None, device)
    y_ref = wkv.forward(kd, vd, wd, ud, path="chained")
    y, st = wkv.forward_save(kd, vd, wd, ud)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    st = st.cpu().numpy().astype(np.float64)          # [B, nsub, 2, C]: r, q
    assert st.shape == (B, (T + 15) // 16, 2, C)
    # sub-chunk 0 starts from the empty history: r = 0, q at the empty exponent
    assert np.all(st[:, 0, 0] == 0) and np.all(st[:, 0, 1] <= -1e37)
    for s in range(1, st.shape[1]):
        _, ref = oracle.forward(x.k[:, :16 * s], x.v[:, :16 * s], x.w, x.u)
        # the history sums are r e^q and e^q: the state (a, b, p) = (r, 1, q)
        r, q = st[:, s, 0], st[:, s, 1]
        ea, eb, _ = state_mismatch((r, np.ones_like(r), q), ref)
        assert ea <= 1e-4 and eb <= 1e-4, (s, ea, eb)


def test_forward_save_checks_the_states_shape(device):
    """forward_save checks the states' shape before it launches."""
    import torch
    import linear_attention_rnn_forward_amd as wkv
    k = torch.zeros((1, 20, 8), device=device)
    w = torch.ones(8, device=device)
    with pytest.raises(ValueError):
        wkv.forward_save(k, k.clone(), w, w.clone(), states=torch.empty((1, 1, 4, 8), device=device))
