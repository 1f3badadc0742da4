"""Seeded synthetic inputs for the WKV workloads.

This module is shared by both sides of every parity check -- the HIP library's
callers (tests, bench) and the fp64 oracle -- and therefore holds none of the
WKV arithmetic: only shapes, value distributions, seeds, the bf16 rounding of
stored inputs, and one counter-based random generator (Philox4x32-10) with a
fixed transform to approximately standard-normal values.

The pages publish no benchmark or dataset for the operator; the workloads are
synthetic stand-ins shaped like the pages' setting (per-channel decay
w = exp(omega) > 0, bonus u, keys and values of unit scale, and the
overflow-provoking large keys the pages warn about).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

# ----------------------------------------------------------------------------
# Workload definitions
# ----------------------------------------------------------------------------


@dataclass(frozen=True)
class ForwardWorkload:
    """One wkv_forward workload: k, v [B,T,C]; w, u [C]."""
    name: str
    B: int
    T: int
    C: int
    dtype: str                 # storage type of k, v, y: "f32" or "bf16"
    seed: int
    omega: tuple               # w = fl32(exp(omega)), omega ~ U(lo, hi)
    u_std: float               # u ~ N(0, u_std)   (second argument = std dev)
    k_std: float               # k ~ N(0, k_std)
    spike_p: float             # i.i.d. Bernoulli(spike_p) per element of k ...
    spike_value: float         # ... replaced by +spike_value or +-spike_value
    spike_sign: str            # "plus" or "plusminus" (fair coin per spike)

    def resized(self, **kw) -> "ForwardWorkload":
        """Same recipe and seed at another shape (for oracle-sized parity runs)."""
        return replace(self, **kw)

    @property
    def elems(self) -> int:
        return self.B * self.T * self.C


@dataclass(frozen=True)
class DecodeWorkload:
    """Prefill with wkv_forward, then `steps` wkv_step calls over [L,S,C]."""
    name: str
    L: int
    S: int
    C: int
    prefill_T: int
    steps: int
    seed: int
    omega: tuple
    u_std: float

    @property
    def total_T(self) -> int:
        return self.prefill_T + self.steps


TINY = ForwardWorkload("wkv_forward B=1 T=256 C=64 fp32, 1% of k = +40", 1, 256, 64, "f32", 1,
                       (-5.0, 1.0), 0.5, 1.0, 0.01, 40.0, "plus")
SMALL_LM = ForwardWorkload("wkv_forward B=8 T=1024 C=768 fp32", 8, 1024, 768, "f32", 2,
                           (-5.0, 1.0), 0.5, 1.0, 0.0, 0.0, "plus")
BF16_MAIN = ForwardWorkload("wkv_forward B=16 T=4096 C=2048 bf16 k/v/y, fp32 w/u/state", 16, 4096,
                            2048, "bf16", 3, (-6.0, 2.0), 0.5, 3.0, 0.001, 40.0, "plusminus")
LONG_CTX = ForwardWorkload("wkv_forward B=1 T=65536 C=4096 fp32, 1% of k = +40", 1, 65536, 4096,
                           "f32", 4, (-5.0, 1.0), 0.5, 1.0, 0.01, 40.0, "plus")
DECODE = DecodeWorkload("wkv_step L=32 S=256 C=4096 fp32 state, 512-token prefill + 1024 steps",
                        32, 256, 4096, 512, 1024, 5, (-5.0, 1.0), 0.5)

FORWARD_WORKLOADS = {"tiny": TINY, "small_lm": SMALL_LM, "bf16_main": BF16_MAIN,
                     "long_ctx": LONG_CTX}

# ----------------------------------------------------------------------------
# bf16 storage
# ----------------------------------------------------------------------------


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits.

    Inputs here are finite.
    """
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = bits + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to fp32 exactly (a 16-bit shift)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# Forward workload inputs (numpy.random.default_rng)
# ----------------------------------------------------------------------------


@dataclass
class ForwardInputs:
    w: np.ndarray              # [C] fp32
    u: np.ndarray              # [C] fp32
    k: np.ndarray              # [B,T,C] fp32 values as stored (bf16-exact when bf16)
    v: np.ndarray              # [B,T,C] fp32
    k_bits: np.ndarray | None  # [B,T,C] uint16 when the storage type is bf16
    v_bits: np.ndarray | None


def decay_and_bonus(rng: np.random.Generator, shape, omega, u_std):
    omega_v = rng.uniform(omega[0], omega[1], size=shape)
    w = np.exp(omega_v).astype(np.float32)
    u = (rng.standard_normal(size=shape) * u_std).astype(np.float32)
    return w, u


def make_forward_inputs(wl: ForwardWorkload) -> ForwardInputs:
    """Draw w, u, k, v for `wl` in a fixed order from default_rng(wl.seed)."""
    rng = np.random.default_rng(wl.seed)
    B, T, C = wl.B, wl.T, wl.C
    w, u = decay_and_bonus(rng, (C,), wl.omega, wl.u_std)
    k = rng.standard_normal(size=(B, T, C), dtype=np.float32)
    if wl.k_std != 1.0:
        k *= np.float32(wl.k_std)
    if wl.spike_p > 0:
        mask = rng.random(size=(B, T, C), dtype=np.float32) < np.float32(wl.spike_p)
        n = int(mask.sum())
        if wl.spike_sign == "plusminus":
            sign = np.where(rng.integers(0, 2, size=n) == 0, 1.0, -1.0).astype(np.float32)
        else:
            sign = np.ones(n, dtype=np.float32)
        k[mask] = sign * np.float32(wl.spike_value)
        del mask
    v = rng.standard_normal(size=(B, T, C), dtype=np.float32)
    k_bits = v_bits = None
    if wl.dtype == "bf16":
        k_bits = f32_to_bf16_bits(k)
        v_bits = f32_to_bf16_bits(v)
        k = bf16_bits_to_f32(k_bits)
        v = bf16_bits_to_f32(v_bits)
    return ForwardInputs(w, u, k, v, k_bits, v_bits)


# The receptance r of the gated form: r ~ N(0, RECEPTANCE_STD) from its own
# generator (seed offset below), so the k, v, w, u of a workload are the same
# with or without the gate.
RECEPTANCE_STD = 2.0
RECEPTANCE_SEED_OFFSET = 1000


def make_receptance(wl: ForwardWorkload):
    """r [B,T,C] for `wl`: fp32 values as stored, and the uint16 bits when the
    storage type is bf16 (else None)."""
    rng = np.random.default_rng(wl.seed + RECEPTANCE_SEED_OFFSET)
    r = rng.standard_normal(size=(wl.B, wl.T, wl.C), dtype=np.float32)
    r *= np.float32(RECEPTANCE_STD)
    if wl.dtype == "bf16":
        bits = f32_to_bf16_bits(r)
        return bf16_bits_to_f32(bits), bits
    return r, None


# The output gradient gy of a backward workload: gy ~ N(0, 1) from its own
# generator, so k, v, w, u are those of the forward workload of the same name.
OUTPUT_GRAD_SEED_OFFSET = 2000


def make_output_grad(wl: ForwardWorkload):
    """gy [B,T,C] for `wl`: fp32 values as stored, and the uint16 bits when
    the storage type is bf16 (else None)."""
    rng = np.random.default_rng(wl.seed + OUTPUT_GRAD_SEED_OFFSET)
    g = rng.standard_normal(size=(wl.B, wl.T, wl.C), dtype=np.float32)
    if wl.dtype == "bf16":
        bits = f32_to_bf16_bits(g)
        return bf16_bits_to_f32(bits), bits
    return g, None


def decode_params(wl: DecodeWorkload):
    """Per-layer decay and bonus [L,C] for the decode workload."""
    rng = np.random.default_rng(wl.seed)
    return decay_and_bonus(rng, (wl.L, wl.C), wl.omega, wl.u_std)


# ----------------------------------------------------------------------------
# Counter-based generator for inputs too large to hold (the decode workload)
#
# Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
# as 1, 2, 3", SC 2011): 10 rounds of the 4x32 Philox S-box with the published
# multipliers and Weyl key increments.  The device side (synth/philox_fill.hip)
# implements the same definition; tests check the two agree bit for bit.
#
# Normal transform: the 4 output words give 8 16-bit integers h_j; their sum
# S is centred and scaled, z = fl32(S - 262140) * fl32(sqrt(1.5) / 65536).
# This is the standardised Irwin-Hall(8) distribution (mean 0, variance 1,
# |z| <= 4.9), an approximation of N(0,1) whose every step is exact integer
# arithmetic plus one correctly rounded fp32 multiply, so host and device
# produce identical bits without transcendental functions.
# ----------------------------------------------------------------------------

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
IH8_CENTER = 262140                                  # 8 * (65535 / 2)
IH8_SCALE = np.float32(np.sqrt(1.5) / 65536.0)       # 1 / (65536 * sqrt(8/12))
KEY_HI = 0x52574B56                                  # second key word, fixed
STREAM_K = 0
STREAM_V = 1


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32-10 on uint32 arrays (vectorised); returns four uint32 arrays."""
    mask = 0xFFFFFFFF
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint32) for c in (c0, c1, c2, c3))
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    s32 = np.uint64(32)
    for r in range(10):
        if r:
            k0 = (k0 + PHILOX_W0) & mask
            k1 = (k1 + PHILOX_W1) & mask
        p0 = c0.astype(np.uint64) * m0
        p1 = c2.astype(np.uint64) * m1
        hi0 = (p0 >> s32).astype(np.uint32)
        lo0 = p0.astype(np.uint32)
        hi1 = (p1 >> s32).astype(np.uint32)
        lo1 = p1.astype(np.uint32)
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint32(k0), lo1, hi0 ^ c3 ^ np.uint32(k1), lo0)
    return c0, c1, c2, c3


def philox_normal(counter: np.ndarray, stream: int, seed: int) -> np.ndarray:
    """Approximately N(0,1) fp32 values for 64-bit counters (see above)."""
    n = np.asarray(counter, dtype=np.uint64)
    lo = (n & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    hi = (n >> np.uint64(32)).astype(np.uint32)
    x = philox4x32_10(lo, hi, np.full_like(lo, stream), np.zeros_like(lo), seed & 0xFFFFFFFF,
                      KEY_HI)
    s = np.zeros(lo.shape, dtype=np.int64)
    for word in x:
        s += (word & np.uint32(0xFFFF)).astype(np.int64)
        s += (word >> np.uint32(16)).astype(np.int64)
    return (s - IH8_CENTER).astype(np.float32) * IH8_SCALE


def decode_counter(wl: DecodeWorkload, layer, seq, token, channel):
    """Counter of element (layer, seq, token, channel) of the decode workload's
    k or v stream; tokens 0..prefill_T-1 are the prompt, then one per step."""
    layer, seq, token, channel = (np.asarray(x, dtype=np.uint64)
                                  for x in (layer, seq, token, channel))
    S, Tt, C = np.uint64(wl.S), np.uint64(wl.total_T), np.uint64(wl.C)
    return ((layer * S + seq) * Tt + token) * C + channel


def decode_kv_column(wl: DecodeWorkload, layer: int, seq: int, channels) -> tuple:
    """Host copy of k, v for one (layer, seq) over all tokens: [total_T, len(channels)]."""
    ch = np.asarray(channels, dtype=np.uint64)[None, :]
    tok = np.arange(wl.total_T, dtype=np.uint64)[:, None]
    ctr = decode_counter(wl, layer, seq, tok, ch)
    return philox_normal(ctr, STREAM_K, wl.seed), philox_normal(ctr, STREAM_V, wl.seed)


# ----------------------------------------------------------------------------
# Matrix-valued state (RWKV-5 Eagle / RWKV-6 Finch) workloads
#
# r, k, v, z [B,T,C] with C = 64 H.  The pages give no distributions for this
# variant; the recipe keeps every term of unit scale: r ~ N(0, 1), v ~ N(0, 1),
# k ~ N(0, 1/8) so that r.k over a 64-channel head has unit variance, and the
# decay argument z = w_c + N(0, z_token_std) with w_c ~ U(z_lo, z_hi) per
# channel (d = 1 / (1 + e^z) from 0.99 to 0.07 at the channel means, the span
# of the RWKV-4 workloads' e^{-w}).  Eagle has no token term: z = w_c [C].
# ----------------------------------------------------------------------------


@dataclass(frozen=True)
class MatWorkload:
    """One matrix-state forward workload (decode: B = L * S rows of one token)."""
    name: str
    B: int
    T: int
    H: int
    dtype: str                 # storage of r, k, v, y (and of z when per token)
    seed: int
    per_token_z: bool          # Finch (True) or Eagle (False)
    z_range: tuple = (-5.0, 2.0)
    z_token_std: float = 0.5
    k_std: float = 0.125

    def resized(self, **kw) -> "MatWorkload":
        return replace(self, **kw)

    @property
    def C(self) -> int:
        return 64 * self.H

    @property
    def elems(self) -> int:
        return self.B * self.T * self.C


MAT_MAIN = MatWorkload("wkv_mat_forward (Finch) B=16 T=4096 H=32 (C=2048) bf16 r/k/v/z/y, fp32 state",
                       16, 4096, 32, "bf16", 21, True)
MAT_EAGLE = MatWorkload("wkv_mat_forward (Eagle) B=16 T=4096 H=32 (C=2048) bf16 r/k/v/y, fp32 z and state",
                        16, 4096, 32, "bf16", 22, False)


@dataclass(frozen=True)
class MatDecodeWorkload:
    """wkv_mat_step over [L,S] rows of H heads, a pool of `pool` tokens of
    inputs replayed in turn."""
    name: str
    L: int
    S: int
    H: int
    dtype: str
    seed: int
    pool: int

    @property
    def C(self) -> int:
        return 64 * self.H


MAT_DECODE = MatDecodeWorkload("wkv_mat_step (Finch) L=32 S=64 H=64 (C=4096) fp32 r/k/v/z and state",
                               32, 64, 64, "f32", 23, 4)


@dataclass
class MatInputs:
    r: np.ndarray              # [B,T,C] fp32 values as stored (bf16-exact when bf16)
    k: np.ndarray
    v: np.ndarray
    z: np.ndarray              # [B,T,C] (per token) or [C] fp32
    bits: dict | None          # uint16 bits of r, k, v (and z when per token) for bf16


def make_mat_inputs(wl: MatWorkload) -> MatInputs:
    """Draw w_c, r, k, v, z for `wl` in a fixed order from default_rng(wl.seed)."""
    rng = np.random.default_rng(wl.seed)
    B, T, C = wl.B, wl.T, wl.C
    wc = rng.uniform(wl.z_range[0], wl.z_range[1], size=C).astype(np.float32)
    r = rng.standard_normal(size=(B, T, C), dtype=np.float32)
    k = rng.standard_normal(size=(B, T, C), dtype=np.float32) * np.float32(wl.k_std)
    v = rng.standard_normal(size=(B, T, C), dtype=np.float32)
    if wl.per_token_z:
        z = rng.standard_normal(size=(B, T, C), dtype=np.float32) * np.float32(wl.z_token_std)
        z += wc
    else:
        z = wc
    bits = None
    if wl.dtype == "bf16":
        bits = {}
        names = ("r", "k", "v", "z") if wl.per_token_z else ("r", "k", "v")
        arrs = {"r": r, "k": k, "v": v, "z": z}
        for n in names:
            bits[n] = f32_to_bf16_bits(arrs[n])
            arrs[n] = bf16_bits_to_f32(bits[n])
        r, k, v, z = arrs["r"], arrs["k"], arrs["v"], arrs["z"]
    return MatInputs(r, k, v, z, bits)


def make_mat_decode_pool(wl: MatDecodeWorkload) -> MatInputs:
    """`pool` tokens of r, k, v, z for every row: arrays [pool, L, S, C] fp32."""
    rng = np.random.default_rng(wl.seed)
    shape = (wl.pool, wl.L, wl.S, wl.C)
    wc = rng.uniform(-5.0, 2.0, size=(wl.L, 1, wl.C)).astype(np.float32)
    r = rng.standard_normal(size=shape, dtype=np.float32)
    k = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(0.125)
    v = rng.standard_normal(size=shape, dtype=np.float32)
    z = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(0.5) + wc
    return MatInputs(r, k, v, z, None)
