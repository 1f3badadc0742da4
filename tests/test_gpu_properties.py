"""Properties of the operator checked on the GPU path itself, every execution
path and storage type.

- Shifting every key by c leaves the output unchanged and moves the state's
  exponent by c: all weights e^{k_i - ...} share the factor e^c, which cancels
  in the ratio ([tm-math] "Numerical stability: carry the exponent": only
  exponent differences matter).
- v -> alpha v + beta maps y -> alpha y + beta: y is a weighted mean of the
  values with weights that do not involve v ([tm-math] "The WKV operator").
- Seeded random small shapes (ragged B, T, C, including T = 0) against the
  fp64 oracle.

Inputs sit on a coarse grid (multiples of 1/4 for keys, of 1/64 for values)
so that the shifted and scaled inputs are exact in fp32 and in bf16 and any
difference comes from the kernels' own rounding.
"""
import numpy as np
import pytest

import oracle
from oracle.compare import guarded_rel_err, rms, state_mismatch

pytestmark = pytest.mark.gpu

PATHS = ["serial", "chained", "chunked"]
TOL = {"f32": 1e-4, "bf16": 2e-2}


def _dev(x, device, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def _grid_inputs(rng, B, T, C):
    k = np.round(rng.normal(0, 2, (B, T, C)) * 4) / 4          # multiples of 1/4
    k = np.clip(k, -8, 7.75)
    k[rng.random((B, T, C)) < 0.01] = 7.75                     # a few large keys
    v = np.clip(np.round(rng.normal(0, 1, (B, T, C)) * 64) / 64, -3.0, 3.0)
    w = np.exp(rng.uniform(-5, 1, C)).astype(np.float32)
    u = rng.normal(0, 0.5, C).astype(np.float32)
    return k.astype(np.float32), v.astype(np.float32), w, u


def _run(device, k, v, w, u, dtype, path):
    import torch
    import linear_attention_rnn_forward_amd as wkv
    y, st = wkv.forward(_dev(k, device, dtype), _dev(v, device, dtype), _dev(w, device, "f32"),
                        _dev(u, device, "f32"), return_state=True, path=path)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), tuple(s.cpu().numpy() for s in st)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("path", PATHS)
def test_key_shift_invariance(device, path, dtype):
    rng = np.random.default_rng(41)
    k, v, w, u = _grid_inputs(rng, 2, 700, 192)
    c = 16.0                                                    # k + c exact in both storages
    y0, st0 = _run(device, k, v, w, u, dtype, path)
    y1, st1 = _run(device, k + c, v, w, u, dtype, path)
    assert np.all(np.isfinite(y1))
    # outputs: both are the same ratio up to the kernels' rounding (bf16
    # outputs may round to neighbouring values)
    err = guarded_rel_err(y1, y0, rms(v))
    assert err <= (1e-5 if dtype == "f32" else 2.0 ** -7), err
    # the state: the same sums with the exponent moved by c
    ea, eb, _ = state_mismatch((st1[0], st1[1], st1[2] - c), st0)
    assert ea <= 1e-5 and eb <= 1e-5, (ea, eb)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("path", PATHS)
def test_value_affine_equivariance(device, path, dtype):
    rng = np.random.default_rng(43)
    k, v, w, u = _grid_inputs(rng, 2, 700, 192)
    alpha, beta = 2.0, 0.5                                      # exact on the grid
    y0, _ = _run(device, k, v, w, u, dtype, path)
    y1, _ = _run(device, k, alpha * v + beta, w, u, dtype, path)
    err = guarded_rel_err(y1, alpha * y0 + beta, alpha * rms(v) + beta)
    assert err <= (1e-5 if dtype == "f32" else 2.0 ** -7), err


def _random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(rng.integers(1, 4))
        T = int(rng.choice([0, 1, int(rng.integers(2, 40)), int(rng.integers(40, 600))]))
        C = int(rng.integers(1, 300))
        out.append((B, T, C, PATHS[int(rng.integers(0, 3))], ["f32", "bf16"][int(rng.integers(0, 2))],
                    int(rng.integers(0, 1 << 30))))
    return out


@pytest.mark.parametrize("B,T,C,path,dtype,seed", _random_shapes(24, 2024),
                         ids=lambda x: str(x))
def test_random_small_shapes_against_oracle(device, B, T, C, path, dtype, seed):
    import torch
    import linear_attention_rnn_forward_amd as wkv
    rng = np.random.default_rng(seed)
    k = rng.normal(0, 2, (B, T, C)).astype(np.float32)
    k[rng.random((B, T, C)) < 0.02] = 40.0
    v = rng.normal(0, 1, (B, T, C)).astype(np.float32)
    w = np.exp(rng.uniform(-6, 2, C)).astype(np.float32)
    u = rng.normal(0, 0.5, C).astype(np.float32)
    kd, vd = _dev(k, device, dtype), _dev(v, device, dtype)
    # the oracle sees the inputs as stored
    kh, vh = kd.float().cpu().numpy(), vd.float().cpu().numpy()
    y, st = wkv.forward(kd, vd, _dev(w, device, "f32"), _dev(u, device, "f32"), return_state=True,
                        path=path)
    torch.cuda.synchronize()
    y_ref, st_ref = oracle.forward(kh, vh, w, u)
    yh = y.float().cpu().numpy()
    assert yh.shape == (B, T, C) and np.all(np.isfinite(yh))
    assert guarded_rel_err(yh, y_ref, 1.0) <= TOL[dtype]
    ea, eb, _ = state_mismatch(tuple(s.cpu().numpy() for s in st), st_ref)
    assert ea <= 1e-4 and eb <= 1e-4
