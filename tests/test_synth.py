"""Input generators: the published Philox known answers, bf16 rounding, recipes.

CPU only.
"""
import numpy as np
import pytest

import synth


@pytest.mark.parametrize("ctr,key,expect", [
    # known-answer vectors published with the Random123 library for philox4x32_10
    ((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff,) * 4, (0xffffffff,) * 2, (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
])
def test_philox_known_answers(ctr, key, expect):
    out = synth.philox4x32_10(*[np.array([c], dtype=np.uint32) for c in ctr], *key)
    assert tuple(int(o[0]) for o in out) == expect


def test_philox_normal_moments_and_bounds():
    z = synth.philox_normal(np.arange(2_000_000, dtype=np.uint64), synth.STREAM_K, 5)
    assert z.dtype == np.float32
    assert abs(float(z.mean())) < 3e-3
    assert abs(float(z.std()) - 1.0) < 3e-3
    assert float(np.abs(z).max()) <= 4 * np.sqrt(1.5) + 1e-6
    z2 = synth.philox_normal(np.arange(1000, dtype=np.uint64), synth.STREAM_V, 5)
    assert not np.array_equal(z[:1000], z2)


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, -2.5, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, 40.0, -40.0],
                 dtype=np.float32)
    bits = synth.f32_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(bits)
    # ties go to the even mantissa, anything above a tie rounds up
    np.testing.assert_array_equal(back, np.array([1.0, -2.5, 1.0, 1.0 + 4 * 2 ** -8,
                                                  1.0 + 2 ** -7, 40.0, -40.0], dtype=np.float32))
    assert bits[0] == 0x3F80


def test_forward_recipe_is_seeded_and_shaped():
    a = synth.make_forward_inputs(synth.TINY)
    b = synth.make_forward_inputs(synth.TINY)
    assert np.array_equal(a.k, b.k) and np.array_equal(a.w, b.w)
    assert a.k.shape == (1, 256, 64) and a.w.dtype == np.float32
    frac = float((a.k == 40.0).mean())
    assert 0.003 < frac < 0.02
    assert np.all(a.w > 0)
    s = synth.make_forward_inputs(synth.BF16_MAIN.resized(B=1, T=512, C=256))
    assert s.k_bits is not None and np.array_equal(synth.bf16_bits_to_f32(s.k_bits), s.k)
    assert set(np.unique(s.k[np.abs(s.k) == 40.0])) <= {-40.0, 40.0}
