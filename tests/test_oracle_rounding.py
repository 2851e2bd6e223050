"""Pins of the oracle's rounding helpers against hand-computed values and the
definition 'nearest representable value, ties to even' (brute force)."""
import numpy as np

from oracle.rounding import round_bf16, round_f16, bf16_bits, bf16_from_bits


def test_bf16_hand_values():
    # spacing of bf16 at 1.0 is 2**-7
    assert round_bf16(1.0 + 2**-8) == 1.0                  # tie -> even
    assert round_bf16(1.0 + 3 * 2**-8) == 1.0 + 2**-6      # tie -> even
    assert round_bf16(1.0 + 2**-8 + 2**-30) == 1.0 + 2**-7
    assert round_bf16(0.3) == 0.30078125                   # 153.6 quanta of 2**-9 -> 154
    assert round_bf16(-0.3) == -0.30078125
    assert round_bf16(0.0) == 0.0
    assert np.isinf(round_bf16(3.5e38))


def test_bf16_is_nearest_by_brute_force():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))
    r = round_bf16(x)
    # r must be representable
    bits = r.astype(np.float32).view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    assert np.all(r.astype(np.float32).astype(np.float64) == r)
    # neighbours one bf16 step up and down are not closer
    up = (bits.astype(np.uint64) + 0x10000).astype(np.uint32).view(np.float32).astype(np.float64)
    dn = (bits.astype(np.uint64) - 0x10000).astype(np.uint32).view(np.float32).astype(np.float64)
    d = np.abs(x - r)
    assert np.all(d <= np.abs(x - up))
    assert np.all(d <= np.abs(x - dn))


def test_f16_hand_values():
    assert round_f16(np.float32(1.0) / np.float32(7.0)) == 0.142822265625
    # subnormal binary16 grid is 2**-24: 1e-7 / 2**-24 = 1.68 -> 2 quanta
    assert round_f16(np.float32(1e-7)) == 2 * 2.0**-24
    assert round_f16(np.float32(2.0**-26)) == 0.0           # below half a quantum
    assert round_f16(np.float32(3 * 2.0**-26)) == 2.0**-24  # 0.75 quanta -> 1
    assert round_f16(np.float32(65520.0)) == np.inf         # rounds past max


def test_bf16_bits_roundtrip():
    v = np.array([1.0, -2.5, 0.30078125, 0.0])
    assert np.all(bf16_from_bits(bf16_bits(v)) == v)
    assert bf16_bits(np.array([1.0]))[0] == 0x3F80
