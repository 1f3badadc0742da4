"""Device-side generation of the decode workload's inputs (libwkv_synth.so).

Same generator and transform as synth.philox_normal on the host, evaluated on
the GPU for arrays too large to create on the host.  Input generation only.
"""
from __future__ import annotations

import ctypes
import os

from . import IH8_SCALE, KEY_HI, STREAM_K, STREAM_V, DecodeWorkload

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwkv_synth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        i64 = ctypes.c_int64
        L.synth_fill_normal.restype = ctypes.c_int
        L.synth_fill_normal.argtypes = ([ctypes.c_void_p] + [i64] * 8 +
                                        [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                         ctypes.c_uint32, ctypes.c_float, ctypes.c_void_p])
        _lib = L
    return _lib


def fill_normal(out, dims, strides, base: int, stream_id: int, seed: int) -> None:
    """out: contiguous float32 CUDA tensor of shape `dims` (4 entries); element
    (i0..i3) gets the value of counter base + sum(i_d * strides[d])."""
    import torch
    assert out.is_cuda and out.is_contiguous() and out.dtype == torch.float32
    assert tuple(out.shape) == tuple(dims) or out.numel() == dims[0] * dims[1] * dims[2] * dims[3]
    stream = torch.cuda.current_stream(out.device).cuda_stream
    rc = lib().synth_fill_normal(ctypes.c_void_p(out.data_ptr()), *dims, *strides, base, stream_id,
                                 seed & 0xFFFFFFFF, KEY_HI, float(IH8_SCALE),
                                 ctypes.c_void_p(stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill_normal failed with {rc}")


def decode_prefill_kv(wl: DecodeWorkload, layer: int, k_out, v_out) -> None:
    """k, v of the prompt for one layer: [S, prefill_T, C]."""
    S, Tt, C = wl.S, wl.total_T, wl.C
    dims = (1, S, wl.prefill_T, C)
    strides = (0, Tt * C, C, 1)
    base = layer * S * Tt * C
    fill_normal(k_out, dims, strides, base, STREAM_K, wl.seed)
    fill_normal(v_out, dims, strides, base, STREAM_V, wl.seed)


def decode_step_kv(wl: DecodeWorkload, first_step: int, nsteps: int, k_out, v_out) -> None:
    """k, v of decode steps first_step .. first_step+nsteps-1: [nsteps, L, S, C]."""
    S, Tt, C = wl.S, wl.total_T, wl.C
    dims = (nsteps, wl.L, S, C)
    strides = (C, S * Tt * C, Tt * C, 1)
    base = (wl.prefill_T + first_step) * C
    fill_normal(k_out, dims, strides, base, STREAM_K, wl.seed)
    fill_normal(v_out, dims, strides, base, STREAM_V, wl.seed)
