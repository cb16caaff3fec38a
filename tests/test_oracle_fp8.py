"""Pins of the FP8 (W8A8) comparison oracle (oracle/fp8.py), CPU only.

The E4M3 codec is checked against what fixes it independently of its own
arithmetic: torch's float8_e4m3fn type (a separate implementation of the same
OCP format), brute-force nearest-value search over the 254 finite values,
the ordering of the codes, and the midpoints between neighbours.  The matmul
is checked against exact integer arithmetic, and the MoE layer on one expert
against a dense composition built from torch float64 operations and torch's
own fp8 conversion.
"""

import numpy as np
import pytest
import torch

import gen
import oracle
from oracle import fp8


def _torch_decode_all():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_torch_float8_for_every_code():
    ref = _torch_decode_all()
    ours = fp8.e4m3_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.flatnonzero(nan)) == set(fp8.E4M3_NAN_CODES)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))   # -0.0 at 0x80


def test_decode_landmarks_and_order():
    v = fp8.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6 and v[0x38] == 1.0
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)            # codes 0x00..0x7E increase strictly
    assert np.array_equal(v[0x80:0xFF], -pos)  # sign bit mirrors


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in fp8.E4M3_NAN_CODES], dtype=np.uint8)
    back = fp8.e4m3_encode(fp8.e4m3_decode(codes))
    assert np.array_equal(back, codes)


def test_encode_midpoints_go_to_the_even_code():
    v = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    for c in range(0x7E):
        mid = (v[c] + v[c + 1]) / 2.0          # exact in fp64
        even = c if c % 2 == 0 else c + 1
        assert fp8.e4m3_encode(mid) == even, c
        assert fp8.e4m3_encode(np.nextafter(mid, 0.0)) == c, c
        assert fp8.e4m3_encode(np.nextafter(mid, 1e9)) == c + 1, c
        assert fp8.e4m3_encode(-mid) == (even | 0x80), c


def test_encode_is_the_nearest_value_by_brute_force():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.uniform(-448, 448, 4000),
        np.ldexp(rng.uniform(-1, 1, 4000), rng.integers(-12, 9, 4000)),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 2000),
    ]).astype(np.float32).astype(np.float64)
    finite = np.array([c for c in range(256) if c not in fp8.E4M3_NAN_CODES])
    vals = fp8.e4m3_decode(finite.astype(np.uint8))
    got = fp8.e4m3_encode(x)
    for xi, gi in zip(x, got):
        d = np.abs(vals - xi)
        best = finite[d == d.min()]
        if len(best) > 1:                       # a tie: the even fraction wins (+0 over -0)
            best = [b for b in best if b % 2 == 0 and not (xi >= 0 and b & 0x80)][:1] or best[:1]
        assert fp8.e4m3_decode(gi) == fp8.e4m3_decode(best[0]), (xi, gi, best)


def test_encode_agrees_with_torch_float8_conversion():
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.uniform(-448, 448, 20000),
                        np.ldexp(rng.uniform(-1, 1, 20000), rng.integers(-14, 9, 20000))]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.e4m3_encode(x), ref)


def test_encode_saturates_above_448():
    assert fp8.e4m3_encode(np.array([448.0, 463.9, 1e9, -1e9])).tolist() == [0x7E, 0x7E, 0x7E, 0xFE]


def test_quantize_rows_scale_and_extremes():
    x = np.array([[1.0, -2.0, 0.5, 4.0],
                  [0.0, 0.0, 0.0, 0.0],
                  [-3.0, 0.0, 1.5, 0.75]], dtype=np.float32)
    bits = oracle.bf16_from_f32(x)
    q, s = fp8.quantize_rows(bits)
    assert s.dtype == np.float32
    assert s[0] == np.float32(4.0) / np.float32(448.0) and s[2] == np.float32(3.0) / np.float32(448.0)
    assert s[1] == 1.0 and not q[1].any()
    assert q[0, 3] == 0x7E and q[2, 0] == 0xFE      # the largest magnitude lands on +-448
    # every code is the E4M3 rounding of the fp32 quotient (torch's conversion)
    r = (x / s[:, None]).astype(np.float32)
    ref = torch.from_numpy(np.clip(r, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)


def test_linear_exact_on_integer_codes():
    # codes of the integers -8..8 are exact; with unit scales the product is
    # the integer matmul
    ints = np.arange(-8, 9)
    codes = {int(i): int(fp8.e4m3_encode(float(i))) for i in ints}
    rng = np.random.default_rng(9)
    a = rng.integers(-8, 9, (3, 64))
    b = rng.integers(-8, 9, (5, 64))
    aq = np.vectorize(codes.get)(a).astype(np.uint8)
    bq = np.vectorize(codes.get)(b).astype(np.uint8)
    y = fp8.linear(aq, np.ones(3, np.float32), bq, np.ones(5, np.float32))
    ref = [[sum(int(a[r, k]) * int(b[n, k]) for k in range(64)) for n in range(5)] for r in range(3)]
    assert np.array_equal(y, np.array(ref, dtype=np.float64))
    # scales multiply row- and column-wise
    sa = np.array([0.5, 2.0, -1.0], np.float32)
    sb = np.array([1.0, 0.25, 4.0, 8.0, 0.125], np.float32)
    y2 = fp8.linear(aq, sa, bq, sb)
    assert np.array_equal(y2, np.array(ref) * sa[:, None].astype(np.float64) * sb[None, :].astype(np.float64))


def test_moe_layer_single_expert_is_the_dense_fp8_mlp():
    """E = 1, k = 1: the layer is the dense gated MLP, composed here from
    torch's float8 conversion, float64 matmuls and GELU."""
    rng = np.random.default_rng(10)
    T, d, I = 6, 64, 32
    x = gen.bf16_normal(rng, (T, d))
    logits = np.zeros((T, 1), np.float32)
    w1q = gen.fp8_codes(rng, (1, 2 * I, d))
    w2q = gen.fp8_codes(rng, (1, d, I))
    w1s = gen.fp8_scales(rng, (1, 2 * I))
    w2s = gen.fp8_scales(rng, (1, d))
    out = fp8.moe_layer(x, logits, w1q, w1s, w2q, w2s, k=1)

    def tq(bits):   # per-row quantization through torch's fp8 type
        v = torch.from_numpy(oracle.bf16_bits_to_f32(bits))
        s = torch.where(v.abs().amax(1) > 0, v.abs().amax(1) / torch.tensor(448.0), torch.tensor(1.0))
        q = torch.clamp(v / s[:, None], -448, 448).to(torch.float8_e4m3fn)
        return q.to(torch.float64), s.to(torch.float64)

    def tw(codes, scale):
        return torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64) * torch.from_numpy(scale).double()[:, None]

    xq, xs = tq(x)
    h = (xq @ tw(w1q[0], w1s[0]).T) * xs[:, None]
    h = torch.from_numpy(oracle.bf16_bits_to_f64(oracle.bf16_from_f64(h.numpy())))
    a = torch.nn.functional.gelu(h[:, :I], approximate="tanh") * h[:, I:]
    a_bits = oracle.bf16_from_f64(a.numpy())
    aq, as_ = tq(a_bits)
    o = (aq @ tw(w2q[0], w2s[0]).T) * as_[:, None]
    y = oracle.bf16_from_f64(o.numpy())            # weight softmax(one logit) = 1
    assert np.array_equal(out["y"], y)
