"""GPU parity of the LDS-tiled MFMA grouped matmul (the prefill kernel) against
the oracle, with the kernel forced through w4a16_set_gemm_kernel.  Shapes span
several 128-row tiles per expert with ragged tails, empty experts, K with and
without a partial last 4-group block (and K below one block), column blocks
with idle waves, and both gated epilogues."""

import numpy as np
import pytest
import torch

import gen
import int4_group_quantized_q4_amd as w4
import oracle
from gpu_util import bf16_dev, bits_host, expert_weights, linear_weights, say, to_dev

pytestmark = pytest.mark.gpu


def gmm_case(E, R, K, N, seed, counts=None):
    rng = gen.rng_for(950, seed)
    if counts is None:
        counts = rng.integers(0, 2 * R // E + 1, E)
        counts[::3] = 0
    counts = np.asarray(counts)
    R = int(counts.sum())
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    x_rows = max(1, R // 2 + 3)
    x = gen.bf16_normal(rng, (x_rows, K))
    row_index = rng.integers(0, x_rows, R).astype(np.int32)
    packed, sct, codes, sc = expert_weights(rng, E, N, K)
    return offsets, R, x, row_index, packed, sct, codes, sc


def run_gmm(kernel, offsets, R, x, row_index, packed, sct, E, K, N, epi, out_dtype):
    cols = N if epi == w4.W4_EPI_NONE else N // 2
    tdt = torch.float32 if out_dtype == w4.W4_OUT_F32 else torch.bfloat16
    out = torch.full((R, cols), float("nan"), dtype=tdt, device="cuda")
    with w4.gemm_kernel(kernel):
        w4.moe_gmm(bf16_dev(x), to_dev(row_index), to_dev(offsets), E, R, K, N, to_dev(packed),
                         bf16_dev(sct), epi, out, out_dtype)
    torch.cuda.synchronize()
    if out_dtype == w4.W4_OUT_F32:
        return out.cpu().numpy().astype(np.float64)
    return oracle.bf16_bits_to_f64(bits_host(out))


def ref_gmm(offsets, x, row_index, codes, sc, E, N, epi):
    R = int(offsets[-1])
    if epi == w4.W4_EPI_NONE:
        ref = np.zeros((R, N))
    else:
        ref = np.zeros((R, N // 2))
        fn = oracle.gelu_tanh if epi == w4.W4_EPI_GEGLU_TANH else oracle.moe.silu
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        if epi == w4.W4_EPI_NONE:
            ref[lo:hi] = oracle.linear_f64(x[row_index[lo:hi]], codes[e], sc[e])
        else:
            h = oracle.bf16_bits_to_f64(oracle.linear(x[row_index[lo:hi]], codes[e], sc[e]))
            ref[lo:hi] = fn(h[:, :N // 2]) * h[:, N // 2:]
    return ref


@pytest.mark.parametrize("E,R,K,N", [
    (5, 700, 704, 192),     # K: 5 full blocks + 2 tail groups; 12 tiles -> 1 column block, 3 waves busy
    (3, 400, 96, 64),       # K below one block (3 groups only)
    (4, 530, 160, 320),     # 1 full block + 1 tail group; 20 tiles -> 2 column blocks, idle waves
    (2, 300, 2816, 256),    # long K, 16 tiles = one full column block
    (9, 1200, 512, 1024),   # many row tiles and column blocks
])
def test_tiled_gmm_f32(E, R, K, N):
    offsets, R, x, row_index, packed, sct, codes, sc = gmm_case(E, R, K, N, E + R + K + N)
    say("[tiled gmm f32] E=%d R=%d K=%d N=%d counts=%s" % (E, R, K, N, np.diff(offsets).tolist()))
    got = run_gmm(w4.W4_KERNEL_TILED, offsets, R, x, row_index, packed, sct, E, K, N, w4.W4_EPI_NONE,
                  w4.W4_OUT_F32)
    ref = ref_gmm(offsets, x, row_index, codes, sc, E, N, w4.W4_EPI_NONE)
    ok, mx, rms = oracle.within_tolerance(got, ref)
    say("  max_rel %.2e rms_rel %.2e" % (mx, rms))
    assert ok and not np.isnan(got).any()


def test_tiled_gmm_bf16_out_and_exact_counts():
    # counts on and around multiples of the 128-row tile, one expert empty
    E, K, N = 6, 256, 128
    counts = [128, 0, 129, 127, 256, 1]
    offsets, R, x, row_index, packed, sct, codes, sc = gmm_case(E, 0, K, N, 5, counts)
    say("[tiled gmm bf16] counts=%s" % counts)
    got = run_gmm(w4.W4_KERNEL_TILED, offsets, R, x, row_index, packed, sct, E, K, N, w4.W4_EPI_NONE,
                  w4.W4_OUT_BF16)
    ref = ref_gmm(offsets, x, row_index, codes, sc, E, N, w4.W4_EPI_NONE)
    ok, mx, rms = oracle.within_tolerance(got, ref)
    say("  max_rel %.2e rms_rel %.2e" % (mx, rms))
    assert ok


@pytest.mark.parametrize("act", [w4.W4_EPI_GEGLU_TANH, w4.W4_EPI_SWIGLU])
@pytest.mark.parametrize("E,R,K,N", [(6, 600, 256, 128), (3, 500, 704, 512), (2, 400, 2816, 1408)])
def test_tiled_gmm_gated(act, E, R, K, N):
    offsets, R, x, row_index, packed, sct, codes, sc = gmm_case(E, R, K, N, 60 + act + N)
    say("[tiled gmm gated] act=%d E=%d R=%d K=%d N=%d" % (act, E, R, K, N))
    got = run_gmm(w4.W4_KERNEL_TILED, offsets, R, x, row_index, packed, sct, E, K, N, act, w4.W4_OUT_BF16)
    ref = ref_gmm(offsets, x, row_index, codes, sc, E, N, act)
    ok, mx, rms = oracle.within_tolerance(got, ref)
    say("  max_rel %.2e rms_rel %.2e" % (mx, rms))
    assert ok


def test_tiled_and_streaming_agree():
    """Both kernels on one prefill-shaped case: each within tolerance of the
    oracle and of each other (they differ only in fp32 summation order)."""
    E, K, N = 8, 704, 2816
    offsets, R, x, row_index, packed, sct, codes, sc = gmm_case(E, 900, K, N, 9)
    say("[tiled vs streaming] E=%d R=%d K=%d N=%d" % (E, R, K, N))
    a = run_gmm(w4.W4_KERNEL_TILED, offsets, R, x, row_index, packed, sct, E, K, N, w4.W4_EPI_NONE, w4.W4_OUT_F32)
    b = run_gmm(w4.W4_KERNEL_STREAM, offsets, R, x, row_index, packed, sct, E, K, N, w4.W4_EPI_NONE,
                w4.W4_OUT_F32)
    ref = ref_gmm(offsets, x, row_index, codes, sc, E, N, w4.W4_EPI_NONE)
    for got in (a, b):
        ok, mx, rms = oracle.within_tolerance(got, ref)
        say("  max_rel %.2e rms_rel %.2e" % (mx, rms))
        assert ok
    ok, mx, rms = oracle.within_tolerance(a, b)
    assert ok


# One weight matrix: items in groups of 8 row tiles of 128 (10 row tiles:
# groups of 8 and 2; 18: 8, 8 and 2), and fewer row tiles than a group.
@pytest.mark.parametrize("M,K,N", [(1, 256, 64), (300, 2816, 512), (129, 704, 2816), (1200, 256, 512),
                                   (2200, 128, 1024)])
def test_tiled_linear(M, K, N):
    rng = gen.rng_for(951, M + K + N)
    packed, sct, codes, sc = linear_weights(rng, N, K)
    x = gen.bf16_normal(rng, (M, K))
    say("[tiled linear] M=%d K=%d N=%d" % (M, K, N))
    with w4.gemm_kernel(w4.W4_KERNEL_TILED):
        y = w4.linear(bf16_dev(x), to_dev(packed), bf16_dev(sct), N)
    torch.cuda.synchronize()
    ref = oracle.linear(x, codes, sc)
    ok, mx, rms = oracle.within_tolerance(oracle.bf16_bits_to_f64(bits_host(y)), oracle.bf16_bits_to_f64(ref))
    say("  max_rel %.2e rms_rel %.2e" % (mx, rms))
    assert ok


def test_tiled_linear_exact_integer_case():
    """Unit scales and small-integer activations make every partial sum an
    exact fp32 integer: the tiled kernel's bf16 output is bit-identical to the
    oracle's."""
    rng = gen.rng_for(951, 7)
    M, K, N = 200, 512, 256
    packed, _, codes, _ = linear_weights(rng, N, K)
    sc = np.full((N, K // 32), 0x3F80, dtype=np.uint16)
    import layout
    x = oracle.bf16_from_f64(rng.integers(-8, 9, (M, K)).astype(np.float64))
    with w4.gemm_kernel(w4.W4_KERNEL_TILED):
        y = w4.linear(bf16_dev(x), to_dev(packed), bf16_dev(layout.encode_scales(sc)), N)
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(y), oracle.linear(x, codes, sc))


@pytest.mark.parametrize("kind", ["zero", "tiny", "huge"])
def test_tiled_gmm_scales_outside_fp16_range(kind):
    """Blocks whose scales fall outside [2^-14, 2^13) (zero groups, tiny or huge
    scales) are recomputed by the exact kernel; the others keep the fp16 path.
    Both must match the oracle."""
    E, K, N = 4, 704, 256
    offsets, R, x, row_index, packed, sct, codes, sc = gmm_case(E, 600, K, N, 70 + len(kind))
    import layout
    sc = sc.copy()
    value = {"zero": 0x0000, "tiny": oracle.bf16_from_f64(np.array([3e-6]))[0],
             "huge": oracle.bf16_from_f64(np.array([2.0e4]))[0]}[kind]
    sc[1, 5:9, 3] = value          # expert 1: a few groups of a few rows
    sc[3, 200, :] = value          # expert 3: a whole row
    sct = np.concatenate([layout.encode_scales(sc[e]) for e in range(E)])
    say("[tiled gmm out-of-range scales] %s" % kind)
    got = run_gmm(w4.W4_KERNEL_TILED, offsets, R, x, row_index, packed, sct, E, K, N, w4.W4_EPI_NONE, w4.W4_OUT_F32)
    ref = ref_gmm(offsets, x, row_index, codes, sc, E, N, w4.W4_EPI_NONE)
    ok, mx, rms = oracle.within_tolerance(got, ref)
    say("  max_rel %.2e rms_rel %.2e" % (mx, rms))
    assert ok and not np.isnan(got).any()
