"""GPU parity past 32-bit element and byte offsets.

Inputs of more than 2^31 elements (more than 4 GiB per bf16 array) are made
on the device by the counter-based generator of synth.device, and sampled
channels are made again on the host from the same counters, so that the fp64
oracle can run on those channels over the whole sequence.  Every kernel
forms its addresses from 64-bit bases and 32-bit offsets inside a tile or
chunk; these tests run the paths on arrays where a 32-bit element or byte
offset over the whole array would wrap.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import matrix_state as ms
from oracle.compare import guarded_rel_err

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


def _torch():
    import torch
    return torch


def _wkv():
    import linear_attention_rnn_forward_amd as wkv
    return wkv


def device_normal_bf16(n_rows, C, stream, seed, device, scale=1.0, offset=None):
    """[n_rows, C] bf16 on the device: element (t, c) is philox_normal of
    counter t * C + c (times scale, plus offset[c] when given)."""
    import synth.device as sd
    torch = _torch()
    tmp = torch.empty((n_rows, C), dtype=torch.float32, device=device)
    sd.fill_normal(tmp, (1, 1, n_rows, C), (0, 0, C, 1), 0, stream, seed)
    if scale != 1.0:
        tmp.mul_(scale)
    if offset is not None:
        tmp.add_(torch.from_numpy(offset).to(device)[None, :])
    out = tmp.to(torch.bfloat16)
    del tmp
    return out


def device_normal_f32(shape, stream, seed, device):
    """fp32 on the device: element n (row-major) is philox_normal of counter n."""
    import synth.device as sd
    torch = _torch()
    n_rows = int(np.prod(shape[:-1]))
    out = torch.empty(shape, dtype=torch.float32, device=device)
    sd.fill_normal(out, (1, 1, n_rows, shape[-1]), (0, 0, shape[-1], 1), 0, stream, seed)
    return out


def host_columns_bf16(n_rows, C, channels, stream, seed, scale=1.0, offset=None):
    """The same values for the given channels, [n_rows, len(channels)], as the
    device rounds them: fp32 value (scaled, offset) rounded to bf16."""
    t = np.arange(n_rows, dtype=np.uint64)[:, None]
    ch = np.asarray(channels, dtype=np.uint64)[None, :]
    x = synth.philox_normal(t * np.uint64(C) + ch, stream, seed)
    if scale != 1.0:
        x = (x * np.float32(scale)).astype(np.float32)
    if offset is not None:
        x = (x + offset[np.asarray(channels)][None, :].astype(np.float32)).astype(np.float32)
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))


@pytest.mark.parametrize("path,dtype", [("auto", "bf16"), ("chained", "bf16"), ("auto", "f32")])
def test_forward_past_32_bit_offsets(device, path, dtype):
    """[1, 2^20 + 37, 2304]: 2.42e9 elements, 4.8 GB per bf16 array (9.7 GB
    in fp32)."""
    torch = _torch()
    T, C, seed = (1 << 20) + 37, 2304, 77
    assert T * C > 2 ** 31 and 2 * T * C > 2 ** 32
    if dtype == "bf16":
        k = device_normal_bf16(T, C, synth.STREAM_K, seed, device)
        v = device_normal_bf16(T, C, synth.STREAM_V, seed, device)
    else:
        k = device_normal_f32((T, C), synth.STREAM_K, seed, device)
        v = device_normal_f32((T, C), synth.STREAM_V, seed, device)
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(-5.0, 1.0, C)).astype(np.float32)
    u = rng.normal(0.0, 0.5, C).astype(np.float32)
    y, (a, b, p) = _wkv().forward(k.view(1, T, C), v.view(1, T, C), torch.from_numpy(w).to(device),
                                  torch.from_numpy(u).to(device), return_state=True, path=path)
    cs = [0, 1, 127, 128, 1151, 2048, 2302, 2303]   # lanes, strips, the last channels
    idx = torch.tensor(cs, device=device)
    ys = y[0].index_select(1, idx).float().cpu().numpy()
    state = [s[0].index_select(0, idx).cpu().numpy() for s in (a, b, p)]
    del y, k, v
    torch.cuda.synchronize()
    if dtype == "bf16":
        kh = host_columns_bf16(T, C, cs, synth.STREAM_K, seed)
        vh = host_columns_bf16(T, C, cs, synth.STREAM_V, seed)
    else:
        t = np.arange(T, dtype=np.uint64)[:, None] * np.uint64(C) + np.asarray(cs, dtype=np.uint64)[None, :]
        kh = synth.philox_normal(t, synth.STREAM_K, seed)
        vh = synth.philox_normal(t, synth.STREAM_V, seed)
    tol = TOL_BF16 if dtype == "bf16" else 1e-4
    y_ref, (a_ref, b_ref, p_ref) = oracle.forward(kh[None], vh[None], w[cs], u[cs])
    err = guarded_rel_err(ys, y_ref[0], 1.0)
    print(f"path={path} {dtype}: {ys.shape[0]} tokens x {ys.shape[1]} channels, y err {err:.3e}")
    assert err <= tol, f"path={path}: y err {err:.3e}"
    # the final state, in the form that does not depend on the anchor
    for got, want in ((state[0] * np.exp(state[2] - p_ref[0]), a_ref[0]),
                      (state[1] * np.exp(state[2] - p_ref[0]), b_ref[0])):
        assert np.max(np.abs(got - want) / np.maximum(np.abs(want), 1.0)) <= tol
    torch.cuda.empty_cache()


def test_mat_forward_past_32_bit_offsets(device):
    """Finch bf16 [1, 2^15 + 5, 1024 heads] (C = 65536): 2.15e9 elements; two
    sampled heads against the fp64 oracle over the whole sequence."""
    torch = _torch()
    T, H, seed = (1 << 15) + 5, 1024, 91
    C = 64 * H
    assert T * C > 2 ** 31
    rng = np.random.default_rng(seed)
    zc = rng.uniform(-5.0, 2.0, C).astype(np.float32)
    r = device_normal_bf16(T, C, 0, seed, device)
    k = device_normal_bf16(T, C, 1, seed, device, scale=0.125)
    v = device_normal_bf16(T, C, 2, seed, device)
    z = device_normal_bf16(T, C, 3, seed, device, scale=0.5, offset=zc)
    y, s_out = _wkv().mat_forward(r.view(1, T, C), k.view(1, T, C), v.view(1, T, C), z.view(1, T, C),
                                  return_state=True)
    heads = [0, H - 1]
    cols = [64 * h + i for h in heads for i in range(64)]
    idx = torch.tensor(cols, device=device)
    ys = y[0].index_select(1, idx).float().cpu().numpy()
    ss = s_out[0, heads].cpu().numpy()
    del y, r, k, v, z
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    rh = host_columns_bf16(T, C, cols, 0, seed)
    kh = host_columns_bf16(T, C, cols, 1, seed, scale=0.125)
    vh = host_columns_bf16(T, C, cols, 2, seed)
    zh = host_columns_bf16(T, C, cols, 3, seed, scale=0.5, offset=zc)
    y_ref, s_ref = ms.forward(rh[None], kh[None], vh[None], zh[None])
    y_mag, s_mag = ms.forward(rh[None], kh[None], vh[None], zh[None], magnitude=True)
    ey = float(np.max(np.abs(ys - y_ref[0]) / np.maximum(y_mag[0], 1e-30)))
    es = float(np.max(np.abs(ss - s_ref[0]) / np.maximum(s_mag[0], 1e-30)))
    print(f"{ys.shape[0]} tokens x {ys.shape[1]} channels: y err {ey:.3e}, state err {es:.3e}")
    assert ey <= TOL_BF16 and es <= TOL_BF16, (ey, es)


def test_step_past_32_bit_offsets(device):
    """One decode step over fp32 [L=8, S=8200, C=32768] (2.15e9 elements per
    array), the state updated in place; sampled rows against the oracle."""
    torch = _torch()
    Ln, S, C, seed = 8, 8200, 32768, 93
    shape = (Ln, S, C)
    assert Ln * S * C > 2 ** 31
    k = device_normal_f32(shape, 0, seed, device)
    v = device_normal_f32(shape, 1, seed, device)
    a = device_normal_f32(shape, 2, seed, device)
    b = device_normal_f32(shape, 3, seed, device).abs_().add_(1.0)
    p = device_normal_f32(shape, 4, seed, device)
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(-5.0, 1.0, (Ln, C))).astype(np.float32)
    u = rng.normal(0.0, 0.5, (Ln, C)).astype(np.float32)
    y, _ = _wkv().step((a, b, p), k, v, torch.from_numpy(w).to(device), torch.from_numpy(u).to(device),
                       inplace=True)
    # sampled (layer, sequence) rows, every channel of each: the last row of
    # the array among them
    rows = [(0, 0), (3, 4097), (Ln - 1, S - 1)]
    got = {name: np.stack([t[l, s].cpu().numpy() for l, s in rows]) for name, t in
           (("y", y), ("a", a), ("b", b), ("p", p))}
    del k, v, a, b, p, y
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    flat = [(l * S + s) * C for l, s in rows]
    cnt = np.array(flat, dtype=np.uint64)[:, None] + np.arange(C, dtype=np.uint64)[None, :]
    kh, vh, ah, bh, ph = (synth.philox_normal(cnt, st, seed) for st in range(5))
    bh = np.abs(bh) + np.float32(1.0)
    lay = [l for l, _ in rows]
    y_ref, (a_ref, b_ref, p_ref) = oracle.step((ah[:, None], bh[:, None], ph[:, None]), kh[:, None], vh[:, None],
                                               w[lay], u[lay])
    # the state (exponent p) is compared in the form that does not depend on it
    err_y = guarded_rel_err(got["y"], y_ref[:, 0], 1.0)
    print(f"{len(rows)} rows x {C} channels: y err {err_y:.3e}")
    assert err_y <= 1e-4, err_y
    sc = np.exp(got["p"].astype(np.float64) - p_ref[:, 0])
    for g, r in ((got["a"] * sc, a_ref[:, 0]), (got["b"] * sc, b_ref[:, 0])):
        assert np.max(np.abs(g - r) / np.maximum(np.abs(r), 1.0)) <= 1e-4


def test_token_shift_past_32_bit_offsets(device):
    """Token shift over bf16 [1, 2^20 + 37, 2304]; sampled channels against
    the oracle over the whole sequence."""
    torch = _torch()
    T, C, seed = (1 << 20) + 37, 2304, 95
    assert T * C > 2 ** 31
    x = device_normal_bf16(T, C, 0, seed, device)
    rng = np.random.default_rng(seed)
    mus = [rng.uniform(0.0, 1.0, C).astype(np.float32) for _ in range(3)]
    outs = _wkv().token_shift(x.view(1, T, C), *(torch.from_numpy(m).to(device) for m in mus),
                              return_last=True)
    cs = [0, 3, 4, 1151, 2300, 2303]
    idx = torch.tensor(cs, device=device)
    got = [o[0].index_select(1, idx).float().cpu().numpy() for o in outs[:3]]
    last = outs[3][0].index_select(0, idx).float().cpu().numpy()
    del x, outs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    xh = host_columns_bf16(T, C, cs, 0, seed)
    ref = oracle.token_shift(xh[None], *(m[cs] for m in mus))
    for g, r in zip(got, ref[:3]):
        err = float(np.max(np.abs(g - r[0]) / np.maximum(np.abs(r[0]), 1.0)))
        assert err <= 2.0 ** -8, err
    np.testing.assert_array_equal(last, ref[3][0])


def test_mat_step_past_32_bit_offsets(device):
    """One matrix-state decode step, fp32, [L=8, S=128, H=520]: a state of
    2.18e9 elements updated in place; three sampled heads against the oracle."""
    torch = _torch()
    Ln, S, H, seed = 8, 128, 520, 97
    C = 64 * H
    assert Ln * S * H * 64 * 64 > 2 ** 31
    import synth.device as sd
    st = torch.empty((Ln, S, H, 64, 64), dtype=torch.float32, device=device)
    sd.fill_normal(st, (1, 1, Ln * S * H * 64, 64), (0, 0, 64, 1), 0, 4, seed)
    st.mul_(0.3)
    r, k, v = (device_normal_f32((Ln, S, C), s_, seed, device) for s_ in range(3))
    k.mul_(0.125)
    z = device_normal_f32((Ln, S, C), 3, seed, device)
    _wkv().mat_step(st, r, k, v, z, inplace=True)
    picks = [(0, 0, 0), (3, 77, 259), (Ln - 1, S - 1, H - 1)]
    got_s = np.stack([st[l, s, h].cpu().numpy() for l, s, h in picks])
    del st
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    # the same inputs on the host for the picked heads
    def host_f32(stream, flat_start, n):
        cnt = np.uint64(flat_start) + np.arange(n, dtype=np.uint64)
        return synth.philox_normal(cnt, stream, seed)
    for i, (l, s, h) in enumerate(picks):
        row = l * S + s
        s0 = (host_f32(4, ((row * H + h) * 64) * 64, 64 * 64) * np.float32(0.3)).astype(np.float32)
        rr, kk, vv, zz = (host_f32(st_, row * C + 64 * h, 64) for st_ in range(4))
        kk = (kk * np.float32(0.125)).astype(np.float32)
        _, s_ref = ms.step(s0.reshape(1, 64, 64), rr, kk, vv, zz)
        _, s_mag = ms.step(np.abs(s0).reshape(1, 64, 64), np.abs(rr), np.abs(kk), np.abs(vv), zz)
        err = float(np.max(np.abs(got_s[i] - s_ref.reshape(64, 64)) / np.maximum(s_mag.reshape(64, 64), 1e-30)))
        print(f"head {(l, s, h)}: state err {err:.3e}")
        assert err <= 1e-4, (l, s, h, err)


def test_gated_forward_past_32_bit_offsets(device):
    """The receptance-gated forward over bf16 [1, 2^20 + 37, 2304] (auto path);
    sampled channels against the oracle's forward_gated."""
    torch = _torch()
    T, C, seed = (1 << 20) + 37, 2304, 99
    assert T * C > 2 ** 31
    k = device_normal_bf16(T, C, 0, seed, device)
    v = device_normal_bf16(T, C, 1, seed, device)
    r = device_normal_bf16(T, C, 2, seed, device)
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(-5.0, 1.0, C)).astype(np.float32)
    u = rng.normal(0.0, 0.5, C).astype(np.float32)
    o = _wkv().forward(k.view(1, T, C), v.view(1, T, C), torch.from_numpy(w).to(device),
                       torch.from_numpy(u).to(device), r=r.view(1, T, C))
    cs = [0, 2, 129, 1151, 2303]
    idx = torch.tensor(cs, device=device)
    os_ = o[0].index_select(1, idx).float().cpu().numpy()
    del o, k, v, r
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    kh, vh, rh = (host_columns_bf16(T, C, cs, st, seed) for st in range(3))
    o_ref, _ = oracle.forward_gated(kh[None], vh[None], rh[None], w[cs], u[cs])
    err = guarded_rel_err(os_, o_ref[0], 1.0)
    print(f"gated: {os_.shape[0]} tokens x {os_.shape[1]} channels, err {err:.3e}")
    assert err <= TOL_BF16, err


def test_backward_past_32_bit_offsets(device):
    """The backward over bf16 [1, 2^20 + 37, 2304] with gy non-zero in the
    first 96 tokens only: every gradient then comes from those tokens, so
    gk, gv of the first 96 and gw, gu match the oracle on that prefix (sampled
    channels), and gk, gv of every later token -- up to the end of arrays
    past 4 GiB -- are exactly zero."""
    torch = _torch()
    T, C, seed, P = (1 << 20) + 37, 2304, 101, 96
    assert T * C > 2 ** 31
    k = device_normal_bf16(T, C, 0, seed, device)
    v = device_normal_bf16(T, C, 1, seed, device)
    gy = torch.zeros((T, C), dtype=torch.bfloat16, device=device)
    gy[:P] = device_normal_bf16(P, C, 2, seed, device)
    rng = np.random.default_rng(seed)
    w = np.exp(rng.uniform(-5.0, 1.0, C)).astype(np.float32)
    u = rng.normal(0.0, 0.5, C).astype(np.float32)
    gk, gv, gw, gu = _wkv().backward(k.view(1, T, C), v.view(1, T, C), torch.from_numpy(w).to(device),
                                     torch.from_numpy(u).to(device), gy.view(1, T, C))
    cs = [0, 1, 255, 1152, 2303]
    idx = torch.tensor(cs, device=device)
    head = [g[0, :P].index_select(1, idx).float().cpu().numpy() for g in (gk, gv)]
    tail_nonzero = [int(torch.count_nonzero(g[0, P:]).item()) for g in (gk, gv)]
    gwu = [g.index_select(0, idx).cpu().numpy() for g in (gw, gu)]
    del k, v, gy, gk, gv
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    assert tail_nonzero == [0, 0], tail_nonzero
    kh, vh, gh = (host_columns_bf16(P, C, cs, st, seed) for st in range(3))
    gk_ref, gv_ref, gw_ref, gu_ref = oracle.backward(kh[None], vh[None], w[cs], u[cs], gh[None])
    mags = oracle.backward(kh[None], vh[None], w[cs], u[cs], gh[None], magnitude=True)
    # gw, gu are fp32 sums (the bar of the backward's own tests)
    for name, got, ref, mag, tol in (("gk", head[0], gk_ref[0], mags[0][0], TOL_BF16),
                                     ("gv", head[1], gv_ref[0], mags[1][0], TOL_BF16),
                                     ("gw", gwu[0], gw_ref, mags[2], 1e-4), ("gu", gwu[1], gu_ref, mags[3], 1e-4)):
        err = float(np.max(np.abs(got - ref) / np.maximum(mag, 1e-30)))
        print(f"backward {name}: err {err:.3e}")
        assert err <= tol, (name, err)
