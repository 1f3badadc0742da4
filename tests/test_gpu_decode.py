"""The decode workload at full size: 32 layers x 256 sequences x 4096 channels,
a 512-token prefill per layer with wkv_forward, then 1024 wkv_step calls.

Inputs come from the counter-based generator (device side for the GPU, host
side for the oracle; bit-identical).  The oracle checks a deterministic
sample of (layer, sequence) columns over all 1536 tokens; the step chain is
also compared with one wkv_forward over the same 1536 tokens (1e-5)."""
import numpy as np
import pytest

import oracle
import synth
from oracle.compare import guarded_rel_err

pytestmark = pytest.mark.gpu

SAMPLE_PAIRS = [(0, 0), (5, 17), (13, 255), (21, 128), (31, 3), (31, 200)]
SAMPLE_CHANNELS = np.linspace(0, 4095, 384).astype(np.int64)
BLOCK = 64


def test_decode_workload_full_size(device):
    import torch

    import linear_attention_rnn_forward_amd as wkv
    import synth.device as sd
    wl = synth.DECODE
    Ln, S, C = wl.L, wl.S, wl.C
    w_h, u_h = synth.decode_params(wl)
    w = torch.from_numpy(w_h).to(device)
    u = torch.from_numpy(u_h).to(device)
    st = tuple(torch.empty((Ln, S, C), dtype=torch.float32, device=device) for _ in range(3))

    # prefill, one layer at a time (B = S sequences, T = 512)
    kp = torch.empty((S, wl.prefill_T, C), device=device)
    vp = torch.empty_like(kp)
    pre_y = {}
    for l in range(Ln):
        sd.decode_prefill_kv(wl, l, kp, vp)
        y, _ = wkv.forward(kp, vp, w[l], u[l], return_state=True,
                           state_out=(st[0][l], st[1][l], st[2][l]))
        for (ll, s) in SAMPLE_PAIRS:
            if ll == l:
                pre_y[(l, s)] = y[s][:, SAMPLE_CHANNELS].cpu().numpy()
    torch.cuda.synchronize()
    print("prefill done", flush=True)

    # decode
    kb = torch.empty((BLOCK, Ln, S, C), device=device)
    vb = torch.empty_like(kb)
    li = torch.tensor([p[0] for p in SAMPLE_PAIRS], device=device)
    si = torch.tensor([p[1] for p in SAMPLE_PAIRS], device=device)
    ys = []                     # sampled pairs, every channel: [steps, pairs, C]
    y = torch.empty((Ln, S, C), device=device)
    for b0 in range(0, wl.steps, BLOCK):
        sd.decode_step_kv(wl, b0, BLOCK, kb, vb)
        for i in range(BLOCK):
            wkv.step(st, kb[i], vb[i], w, u, out=y, inplace=True)
            ys.append(y[li, si])
        if b0 % 256 == 0:
            print(f"decode step {b0}", flush=True)
    y_chain = torch.stack(ys).cpu().numpy()          # [steps, pairs, C]
    assert np.all(np.isfinite(y_chain))

    # oracle on the sampled columns (host generator, identical inputs)
    for pi, (l, s) in enumerate(SAMPLE_PAIRS):
        kh, vh = synth.decode_kv_column(wl, l, s, SAMPLE_CHANNELS)        # [1536, n]
        y_ref, _ = oracle.forward(kh[None], vh[None], w_h[l, SAMPLE_CHANNELS], u_h[l, SAMPLE_CHANNELS])
        y_ref = y_ref[0]
        e_pre = guarded_rel_err(pre_y[(l, s)], y_ref[:wl.prefill_T], 1.0)
        e_dec = guarded_rel_err(y_chain[:, pi, SAMPLE_CHANNELS], y_ref[wl.prefill_T:], 1.0)
        print(f"pair {(l, s)}: prefill err {e_pre:.2e}, decode err {e_dec:.2e}", flush=True)
        assert e_pre <= 1e-4 and e_dec <= 1e-4

    # the step chain against one forward over all 1536 tokens (every channel)
    kf = torch.empty((1, 1, wl.total_T, C), device=device)
    vf = torch.empty_like(kf)
    for pi, (l, s) in enumerate(SAMPLE_PAIRS):
        base = (l * S + s) * wl.total_T * C
        dims = (1, 1, wl.total_T, C)
        strides = (0, 0, C, 1)
        sd.fill_normal(kf, dims, strides, base, synth.STREAM_K, wl.seed)
        sd.fill_normal(vf, dims, strides, base, synth.STREAM_V, wl.seed)
        y_fwd = wkv.forward(kf[0], vf[0], w[l], u[l])
        e = guarded_rel_err(y_chain[:, pi, :], y_fwd[0, wl.prefill_T:].cpu().numpy(), 1.0)
        print(f"pair {(l, s)}: chain vs forward {e:.2e}", flush=True)
        assert e <= 1e-5
