"""Pins of the oracle's W4A16 linear layer: exact-rational brute force on tiny
shapes, and the unit-scale case against torch's float64 matmul."""

from fractions import Fraction

import numpy as np
import torch

import gen
import oracle
from exact import exact_bf16_rne


def _exact_linear_bits(x_bits, codes, scale_bits):
    x = oracle.bf16_bits_to_f64(x_bits)
    s = oracle.bf16_bits_to_f64(scale_bits)
    M, K = x.shape
    N = codes.shape[0]
    out = np.zeros((M, N), dtype=np.uint16)
    for m in range(M):
        xf = [Fraction(float(v)) for v in x[m]]
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += xf[k] * Fraction(float(s[n, k // 32])) * int(codes[n, k])
            out[m, n] = exact_bf16_rne(acc)
    return out


def test_dequant_exact():
    rng = gen.rng_for(901, 1)
    codes = gen.codes_uniform(rng, (8, 64))
    sb = gen.scales_loguniform(rng, (8, 2))
    d = oracle.dequant_f32(codes, sb)
    s = oracle.bf16_bits_to_f64(sb)
    for n in range(8):
        for k in range(64):
            assert Fraction(float(d[n, k])) == Fraction(float(s[n, k // 32])) * int(codes[n, k])


def test_brute_force_tiny_matmuls():
    for seed, (M, K, N) in enumerate([(1, 32, 4), (2, 64, 8), (4, 64, 3), (3, 32, 8)]):
        rng = gen.rng_for(901, 10 + seed)
        x = gen.bf16_normal(rng, (M, K))
        codes = gen.codes_uniform(rng, (N, K))
        sb = gen.scales_loguniform(rng, (N, K // 32))
        assert np.array_equal(oracle.linear(x, codes, sb), _exact_linear_bits(x, codes, sb))


def test_brute_force_wide_exponents():
    """Scales and activations spread over many binades, so the fp64 sums carry
    real cancellation; still bit-identical to exact rational rounding."""
    rng = gen.rng_for(901, 30)
    M, K, N = 3, 64, 6
    x = oracle.bf16_from_f64(rng.standard_normal((M, K)) * np.exp2(rng.integers(-20, 20, (M, K))))
    codes = gen.codes_uniform(rng, (N, K))
    sb = oracle.bf16_from_f64(np.exp2(rng.uniform(-30, 10, (N, K // 32))))
    assert np.array_equal(oracle.linear(x, codes, sb), _exact_linear_bits(x, codes, sb))


def test_unit_scales_reduce_to_integer_matmul():
    rng = gen.rng_for(901, 40)
    M, K, N = 16, 512, 64
    x = gen.bf16_normal(rng, (M, K))
    codes = gen.codes_uniform(rng, (N, K))
    ones = np.full((N, K // 32), 0x3F80, dtype=np.uint16)
    ours = oracle.linear_f64(x, codes, ones)
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    qt = torch.from_numpy(codes.astype(np.float64))
    ref = (xt @ qt.T).numpy()
    assert np.allclose(ours, ref, rtol=1e-13, atol=1e-13)


def test_scale_linearity():
    """Doubling every scale doubles the output exactly (power-of-two scaling)."""
    rng = gen.rng_for(901, 50)
    x = gen.bf16_normal(rng, (4, 256))
    codes = gen.codes_uniform(rng, (32, 256))
    sb = gen.scales_loguniform(rng, (32, 8))
    s2 = oracle.bf16_from_f64(2.0 * oracle.bf16_bits_to_f64(sb))
    y1 = oracle.bf16_bits_to_f64(oracle.linear(x, codes, sb))
    y2 = oracle.bf16_bits_to_f64(oracle.linear(x, codes, s2))
    assert np.array_equal(2.0 * y1, y2)
