"""Pins of the oracle's bf16 codec against a library routine and exact rationals."""

from fractions import Fraction

import numpy as np
import torch

import oracle
from exact import is_bf16_rne, f64_to_bf16_bits_intmath


def _torch_bf16_bits(f32):
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_f32_to_bf16_matches_torch_all_high_halves():
    """Every sign/exponent/top-fraction pattern (all 65536 high halves) crossed
    with the low halves that decide rounding (0, 1, just below/at/above the
    tie, all ones, quarter points)."""
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0x0000, 0x0001, 0x4000, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFF], dtype=np.uint32)
    pats = (hi[:, None] | lows[None, :]).ravel()
    f = pats.view(np.float32)
    ours = oracle.bf16_from_f32(f)
    ref = _torch_bf16_bits(f)
    nan = np.isnan(f)
    assert np.all(np.isnan(oracle.bf16_bits_to_f32(ours[nan])))
    assert np.array_equal(ours[~nan], ref[~nan])


def test_f32_to_bf16_matches_torch_random():
    rng = np.random.default_rng(7)
    pats = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    f = pats.view(np.float32)
    ours = oracle.bf16_from_f32(f)
    ref = _torch_bf16_bits(f)
    nan = np.isnan(f)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all(ours[nan] == 0x7FC0)


def test_f64_to_bf16_is_nearest_even_exact_rationals():
    """fp64 -> bf16 is a single rounding: checked on exact rationals for random
    values across the whole range (normal, subnormal, overflow edge) and on
    constructed ties and near-ties, where going through fp32 first would round
    twice."""
    rng = np.random.default_rng(11)
    vals = list(rng.standard_normal(3000) * np.exp2(rng.integers(-140, 128, 3000)))
    vals += list(rng.standard_normal(500) * 1e-41)            # bf16 subnormal range
    vals += [3.3895313892515355e38, 3.3961775292304947e38, 3.40e38, 1e39, -1e39]
    # exact ties between consecutive bf16 values, and one fp64 ulp either side
    for m in rng.integers(0x0080, 0x7F7F, 400):
        lo = _val(int(m))
        hi = _val(int(m) + 1)
        mid = (lo + hi) / 2.0
        vals += [mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf), -mid]
    # double-rounding trap: a value just above a bf16 tie whose fp32 rounding lands on the tie
    base = 1.0 + 2.0 ** -8          # tie between 1.0 and 1.0078125
    vals += [base + 2.0 ** -30, base - 2.0 ** -30]
    x = np.array(vals, dtype=np.float64)
    bits = oracle.bf16_from_f64(x)
    for v, b in zip(x, bits):
        assert is_bf16_rne(Fraction(float(v)), int(b)), (v, hex(int(b)))
    # the trap itself: one rounding gives 1.0078125, two would give 1.0
    assert oracle.bf16_from_f64(np.array([base + 2.0 ** -30]))[0] == 0x3F81


def _val(m):
    return float(oracle.bf16_bits_to_f64(np.array([m], dtype=np.uint16))[0])


def test_f64_to_bf16_matches_integer_bit_rounding():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(200000) * np.exp2(rng.integers(-100, 100, 200000))
    assert np.array_equal(oracle.bf16_from_f64(x), f64_to_bf16_bits_intmath(x))


def test_specials():
    x = np.array([0.0, -0.0, np.inf, -np.inf, np.nan], dtype=np.float64)
    b = oracle.bf16_from_f64(x)
    assert list(b) == [0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0]


def test_decode_roundtrip_all_patterns():
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = oracle.bf16_bits_to_f32(pats)
    back = oracle.bf16_from_f32(f)
    finite = ~np.isnan(f)
    assert np.array_equal(back[finite], pats[finite])
