"""GPU parity of w4a16_linear against the oracle (normwise max-rel <= 1e-2,
RMS-rel <= 2e-3; bit-exact where the exact result is representable)."""

import numpy as np
import pytest
import torch

import gen
import int4_group_quantized_q4_amd as w4
import oracle
from gpu_util import bf16_dev, bits_host, linear_weights, say, to_dev

pytestmark = pytest.mark.gpu


def run_linear(x_bits, packed, scale_bits, N):
    M, K = x_bits.shape
    say("[linear] M=%d K=%d N=%d" % (M, K, N))
    y = w4.linear(bf16_dev(x_bits), to_dev(packed), bf16_dev(scale_bits), N)
    torch.cuda.synchronize()
    return bits_host(y)


def check_linear(M, K, N, seed, label):
    rng = gen.rng_for(920, seed)
    packed, sct, codes, sc = linear_weights(rng, N, K)
    x = gen.bf16_normal(rng, (M, K))
    y = run_linear(x, packed, sct, N)
    ref = oracle.linear(x, codes, sc)
    ok, mx, rms = oracle.within_tolerance(oracle.bf16_bits_to_f64(y), oracle.bf16_bits_to_f64(ref))
    say("  %s: max_rel %.2e rms_rel %.2e, bf16-identical %.4f" % (label, mx, rms, np.mean(y == ref)))
    assert ok, (label, mx, rms)


def test_linear_dense_tiny():
    cfg = gen.DENSE_TINY
    check_linear(cfg["M"], cfg["K"], cfg["N"], 1, "dense-tiny")


@pytest.mark.parametrize("M", [1, 8, 16])
def test_linear_dense_decode_full_size(M):
    cfg = gen.DENSE_DECODE
    check_linear(M, cfg["K"], cfg["N"], 100 + M, "dense-decode M=%d" % M)


def test_linear_dense_prefill_full_size():
    """M = 4096 rows through the prefill (MFMA) kernel; 24 sampled rows, every
    column, against the oracle (the whole product would take the oracle
    minutes), plus the row-scale edge: one row 2^20 times larger than the rest
    and one 2^-20 times smaller."""
    cfg = gen.DENSE_PREFILL
    M, K, N = cfg["M"], cfg["K"], cfg["N"]
    rng = gen.rng_for(921, 1)
    packed, sct, codes, sc = linear_weights(rng, N, K)
    x = gen.bf16_normal(rng, (M, K))
    xs = oracle.bf16_bits_to_f64(x)
    xs[5] *= 2.0 ** 20
    xs[M - 2] *= 2.0 ** -20
    x = oracle.bf16_from_f64(xs)
    y = run_linear(x, packed, sct, N)
    rows = np.unique(np.concatenate([[0, 5, M - 2, M - 1], rng.choice(M, 20, replace=False)]))
    ref = oracle.linear(x[rows], codes, sc)
    worst = (0.0, 0.0)
    for i, row in enumerate(rows):   # row by row: the scaled rows would hide the others' errors
        ok, mx, rms = oracle.within_tolerance(oracle.bf16_bits_to_f64(y[row]), oracle.bf16_bits_to_f64(ref[i]))
        worst = (max(worst[0], mx), max(worst[1], rms))
        assert ok, (row, mx, rms)
    say("  dense-prefill %d rows: worst max_rel %.2e rms_rel %.2e" % (len(rows), worst[0], worst[1]))


@pytest.mark.parametrize("M,K,N", [(1, 32, 16), (2, 96, 48), (3, 704, 32), (5, 2816, 64), (17, 256, 128),
                                   (33, 512, 64), (64, 160, 16), (100, 1024, 48), (300, 128, 32)])
def test_linear_ragged_shapes(M, K, N):
    check_linear(M, K, N, 200 + M + K + N, "ragged %dx%dx%d" % (M, K, N))


def test_linear_exact_integer_case():
    """Unit scales and small-integer activations: every product and partial sum
    is an integer below 2^24, so the fp32 result is exact and the bf16 output
    must be bit-identical to the oracle."""
    rng = gen.rng_for(920, 5)
    M, K, N = 8, 512, 256
    packed, _, codes, _ = linear_weights(rng, N, K)
    sc = np.full((N, K // 32), 0x3F80, dtype=np.uint16)
    x = oracle.bf16_from_f64(rng.integers(-8, 9, (M, K)).astype(np.float64))
    y = run_linear(x, packed, sc.reshape(-1), N)
    assert np.array_equal(y, oracle.linear(x, codes, sc))


def test_linear_empty_M():
    rng = gen.rng_for(920, 6)
    packed, sc, _, _ = linear_weights(rng, 32, 64)
    y = torch.full((0, 32), 7.0, dtype=torch.bfloat16, device="cuda")
    w4.w4a16_linear(torch.empty(0, 64, dtype=torch.bfloat16, device="cuda"), to_dev(packed), bf16_dev(sc), 32, y)
    torch.cuda.synchronize()


# Split-K kernel (M <= 16, K over 1024 columns, with a workspace): a last
# slice holding only the partial block (K = 1088, 1056), 1..3 tail groups,
# tile groups with idle waves (N/16 not a multiple of 8), several slices.
@pytest.mark.parametrize("M,K,N", [(1, 1088, 48), (16, 1056, 32), (7, 4096, 144), (16, 2816, 16),
                                   (9, 9216, 64), (3, 1120, 128), (16, 4096, 14336), (2, 4064, 80),
                                   (1, 96, 16), (5, 704, 48), (16, 6144, 32)])
def test_linear_splitk_shapes(M, K, N):
    check_linear(M, K, N, 300 + M + K + N, "split-K %dx%dx%d" % (M, K, N))


def test_linear_splitk_agrees_with_streaming():
    """The same call under W4_KERNEL_STREAM runs the streaming kernel: both
    match the oracle and each other (they differ in fp32 summation order
    only)."""
    rng = gen.rng_for(920, 9)
    M, K, N = 16, 4096, 256
    packed, sct, codes, sc = linear_weights(rng, N, K)
    x = gen.bf16_normal(rng, (M, K))
    xd, qd, sd = bf16_dev(x), to_dev(packed), bf16_dev(sct)
    y_split = w4.linear(xd, qd, sd, N)
    y_stream = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    with w4.gemm_kernel(w4.W4_KERNEL_STREAM):
        w4.w4a16_linear(xd, qd, sd, N, y_stream)
    torch.cuda.synchronize()
    ref = oracle.bf16_bits_to_f64(oracle.linear(x, codes, sc))
    for y in (y_split, y_stream):
        ok, mx, rms = oracle.within_tolerance(oracle.bf16_bits_to_f64(bits_host(y)), ref)
        say("  max_rel %.2e rms_rel %.2e" % (mx, rms))
        assert ok
    ok, _, _ = oracle.within_tolerance(oracle.bf16_bits_to_f64(bits_host(y_split)),
                                       oracle.bf16_bits_to_f64(bits_host(y_stream)))
    assert ok


def test_linear_fused_splitk_matches_two_kernel_sum_order():
    """K <= 4096 runs the fused split-K kernel (slices summed in LDS in slice
    order), larger K the two-kernel path (partial sums in the workspace, then
    a slice-order sum).  The same matrix padded to K = 4128 with zero codes
    and zero activations has the same four 1024-column slices plus a fifth
    that adds +0, so the two outputs agree bit for bit."""
    import layout
    rng = gen.rng_for(920, 11)
    M, K, N = 4, 4096, 128
    codes = rng.integers(-8, 8, (N, K)).astype(np.int8)
    sc = gen.scales_loguniform(rng, (N, K // 32))
    x = gen.bf16_normal(rng, (M, K))
    Kp = K + 32
    codes_p = np.zeros((N, Kp), dtype=np.int8)
    codes_p[:, :K] = codes
    sc_p = np.concatenate([sc, sc[:, :1]], axis=1)
    x_p = np.zeros((M, Kp), dtype=np.uint16)
    x_p[:, :K] = x
    y4k = run_linear(x, layout.encode(codes), layout.encode_scales(sc), N)
    y_pad = run_linear(x_p, layout.encode(codes_p), layout.encode_scales(sc_p), N)
    ref = oracle.linear(x, codes, sc)
    ok, mx, rms = oracle.within_tolerance(oracle.bf16_bits_to_f64(y4k), oracle.bf16_bits_to_f64(ref))
    assert ok, (mx, rms)
    assert np.array_equal(y4k, y_pad)


def test_linear_dense_prefill_with_zero_groups_full_size():
    """All-zero groups as the repack emits them (codes 0, scale +0: ±0 is
    outside fp16's exact range for s*q, so every block holding one
    recomputes its tile on the exact path, in the same launch) scattered over
    1% of the groups of the full prefill-shaped matrix: the exact path at
    full size, 24 sampled rows against the oracle."""
    import layout
    cfg = gen.DENSE_PREFILL
    M, K, N = cfg["M"], cfg["K"], cfg["N"]
    rng = gen.rng_for(921, 2)
    codes = rng.integers(-8, 8, (N, K)).astype(np.int8)
    sc = gen.scales_loguniform(rng, (N, K // 32))
    zero = rng.random((N, K // 32)) < 0.01
    sc[zero] = 0
    codes.reshape(N, K // 32, 32)[zero] = 0
    x = gen.bf16_normal(rng, (M, K))
    xd, qd, sd = bf16_dev(x), to_dev(layout.encode(codes)), bf16_dev(layout.encode_scales(sc))
    y = w4.linear(xd, qd, sd, N)   # warm-up and result
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    w4.linear(xd, qd, sd, N)
    t1.record()
    torch.cuda.synchronize()
    say("  dense-prefill with %d zero groups: %.0f us per call (every block redone exactly)"
        % (int(zero.sum()), t0.elapsed_time(t1) * 1e3))
    yb = bits_host(y)
    rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 22, replace=False)]))
    ref = oracle.linear(x[rows], codes, sc)
    for i, row in enumerate(rows):
        ok, mx, rms = oracle.within_tolerance(oracle.bf16_bits_to_f64(yb[row]), oracle.bf16_bits_to_f64(ref[i]))
        assert ok, (row, mx, rms)
