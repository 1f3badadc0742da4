"""wkv_forward_noalloc (the entry point for callers that cannot allocate)
gives wkv_forward's results, on two calls in a row whose second input is
smaller, both on the chunked path that uses the library's fixed scratch
array.  Bar: 1e-4 guarded relative for fp32 storage, 2e-2 for bf16, between
the two entry points and against the fp64 oracle; the chunked path's
look-back combines in a timing-dependent order, so the two entry points
agree to rounding, not bit for bit."""
import numpy as np
import pytest

import oracle
import synth
from oracle.compare import guarded_rel_err, rms, state_mismatch

pytestmark = pytest.mark.gpu


def _case(device, wl):
    import torch
    x = synth.make_forward_inputs(wl)
    if wl.dtype == "bf16":
        k = torch.from_numpy(x.k_bits.view(np.int16)).to(device).view(torch.bfloat16)
        v = torch.from_numpy(x.v_bits.view(np.int16)).to(device).view(torch.bfloat16)
    else:
        k = torch.from_numpy(x.k).to(device)
        v = torch.from_numpy(x.v).to(device)
    return x, k, v, torch.from_numpy(x.w).to(device), torch.from_numpy(x.u).to(device)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_noalloc_matches_forward_on_two_calls(device, dtype):
    import torch
    import linear_attention_rnn_forward_amd as wkv
    base = synth.LONG_CTX if dtype == "f32" else synth.BF16_MAIN
    tol = 1e-4 if dtype == "f32" else 2e-2
    code = wkv.F32 if dtype == "f32" else wkv.BF16
    for shape in ((1, 20000, 1024), (2, 3000, 256)):          # the second call smaller
        B, T, C = shape
        wl = base.resized(B=B, T=T, C=C, seed=500 + T)
        assert wkv.auto_path(B, T, C, code) == "chunked"
        assert 0 < wkv.workspace_size(B, T, C, code) <= 40 << 20
        x, k, v, w, u = _case(device, wl)
        y_ref, st_ref = wkv.forward(k, v, w, u, return_state=True)
        y = torch.full_like(k, float("nan"))
        st = tuple(torch.full((B, C), float("nan"), device=device) for _ in range(3))
        wkv.forward_noalloc(k, v, w, u, out=y, state_out=st)
        torch.cuda.synchronize()
        yh = y.float().cpu().numpy()
        assert np.all(np.isfinite(yh))
        e_entry = guarded_rel_err(yh, y_ref.float().cpu().numpy(), rms(x.v))
        y_o, st_o = oracle.forward(x.k, x.v, x.w, x.u)
        e_oracle = guarded_rel_err(yh, y_o, rms(x.v))
        ea, eb, _ = state_mismatch(tuple(s.cpu().numpy() for s in st), st_o)
        print(f"noalloc {dtype} {shape}: vs wkv_forward {e_entry:.2e}, vs oracle {e_oracle:.2e}, "
              f"state {ea:.2e} {eb:.2e}")
        assert e_entry <= tol and e_oracle <= tol
        assert ea <= 1e-4 and eb <= 1e-4
