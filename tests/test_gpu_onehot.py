"""Bit-exact checks of each matmul kernel's nibble unpack, scale placement and
output mapping.

With one-hot activation rows (row m is bf16 1.0 at column k_m, zero elsewhere)
the product has a single term: y[m][n] = s[n][k_m/32] * q[n][k_m], exact in
fp32 (8-bit times 4-bit significands).  So every kernel -- weight-streaming
decode, short-K, split-K, the tiled prefill kernel and its exact-range
fallback -- must reproduce the oracle's product bit for bit: fp32 outputs equal
the oracle's fp64 value, bf16 outputs its single rounding.  The rows cover
every column of K, so every nibble position, group, block and partial last
block (1, 2 or 3 groups) is read by some lane.

The gated epilogue is checked element by element in the negative tail of the
gate (gate values in [-6, -3]), where a GELU formed as 1 + tanh cancels."""

import numpy as np
import pytest
import torch

import gen
import int4_group_quantized_q4_amd as w4
import layout
import oracle
from gpu_util import bf16_dev, bits_host, say, to_dev

pytestmark = pytest.mark.gpu

ONE = 0x3F80   # bf16 1.0


def onehot(ks, K):
    x = np.zeros((len(ks), K), dtype=np.uint16)
    x[np.arange(len(ks)), ks] = ONE
    return x


def weights(rng, E, N, K, scale_bits=None):
    """Stacked experts: packed codes and tile16 scales for the GPU, logical
    codes [E, N, K] and plain scales [E, N, K/32] for the oracle."""
    codes = gen.codes_uniform(rng, (E, N, K))
    sc = gen.scales_loguniform(rng, (E, N, K // 32)) if scale_bits is None else scale_bits
    packed = np.concatenate([layout.encode(codes[e]) for e in range(E)])
    tiled = np.concatenate([layout.encode_scales(sc[e]) for e in range(E)])
    return packed, tiled, codes, sc


def expect_f64(x, codes, sc):
    return oracle.linear_f64(x, codes, sc)


def check_exact(got, x, codes, sc, out_dtype, label):
    ref = expect_f64(x, codes, sc)
    if out_dtype == w4.W4_OUT_F32:
        ok = np.array_equal(got.astype(np.float64), ref)
    else:
        ok = np.array_equal(got, oracle.bf16_from_f64(ref))
    say("  %s: %s" % (label, "bit-exact" if ok else "MISMATCH"))
    assert ok, label


def run_gmm_onehot(rng, E, K, N, counts, out_dtype, kernel, label, scale_bits=None):
    """Rows of expert e are one-hot at consecutive columns; R = sum(counts)."""
    R = int(sum(counts))
    ks = np.arange(R) % K
    x = onehot(ks, K)
    packed, tiled, codes, sc = weights(rng, E, N, K, scale_bits)
    offs = np.zeros(E + 1, dtype=np.int32)
    offs[1:] = np.cumsum(counts)
    perm = rng.permutation(R).astype(np.int32)        # gather through row_index
    xg = np.empty_like(x)
    xg[perm] = x                                       # x rows stored permuted
    out = torch.empty(R, N, dtype=torch.float32 if out_dtype == w4.W4_OUT_F32 else torch.bfloat16, device="cuda")
    say("[onehot gmm] %s E=%d K=%d N=%d R=%d" % (label, E, K, N, R))
    with w4.gemm_kernel(kernel):
        w4.moe_gmm(bf16_dev(xg), to_dev(perm), to_dev(offs), E, R, K, N, to_dev(packed), bf16_dev(tiled),
                   w4.W4_EPI_NONE, out, out_dtype)
    torch.cuda.synchronize()
    got = out.cpu().numpy() if out_dtype == w4.W4_OUT_F32 else bits_host(out)
    for e in range(E):
        lo, hi = offs[e], offs[e + 1]
        if hi > lo:
            check_exact(got[lo:hi], x[lo:hi], codes[e], sc[e], out_dtype, "%s expert %d" % (label, e))


# weight-streaming decode kernel (K > 1024, plain epilogue): 12 rows per expert
# (one 16-row tile per pass) and 40 (two tiles per pass; a second pass of one)
@pytest.mark.parametrize("K", [1056, 1088, 1120, 2816])
@pytest.mark.parametrize("rpe", [12, 40])
@pytest.mark.parametrize("out_dtype", [w4.W4_OUT_F32, w4.W4_OUT_BF16])
def test_onehot_streaming_kernel(K, rpe, out_dtype):
    rng = gen.rng_for(960, K + rpe + out_dtype)
    E = (K + rpe - 1) // rpe
    counts = np.full(E, rpe)
    counts[-1] = K - rpe * (E - 1)
    run_gmm_onehot(rng, E, K, 48, counts, out_dtype, w4.W4_KERNEL_STREAM, "stream rpe=%d" % rpe)


# short-K decode kernel (K <= 1024, plain epilogue): several passes of 16 rows
@pytest.mark.parametrize("K", [96, 160, 704, 992, 1024])
@pytest.mark.parametrize("out_dtype", [w4.W4_OUT_F32, w4.W4_OUT_BF16])
def test_onehot_short_k_kernel(K, out_dtype):
    rng = gen.rng_for(961, K + out_dtype)
    E = max(2, K // 8)
    counts = np.full(E, K // E)
    counts[0] += K - int(counts.sum())
    counts[1] += 17                                     # a multi-pass expert
    run_gmm_onehot(rng, E, K, 64, counts, out_dtype, w4.W4_KERNEL_STREAM, "short-K")


# tiled prefill kernel (fp16 MFMA on exact s*q), through the MoE entry point
@pytest.mark.parametrize("K", [96, 160, 704, 1120])
@pytest.mark.parametrize("out_dtype", [w4.W4_OUT_F32, w4.W4_OUT_BF16])
def test_onehot_tiled_kernel(K, out_dtype):
    rng = gen.rng_for(962, K + out_dtype)
    E = 3
    counts = np.array([K // 2, 1, K - K // 2 - 1])      # a one-row expert between two large ones
    run_gmm_onehot(rng, E, K, 128, counts, out_dtype, w4.W4_KERNEL_TILED, "tiled")


def test_onehot_tiled_exact_range_fallback():
    """Scales outside fp16's exact range (2^-20, 2^14, zero) send blocks to the
    fallback kernel, which scales each group's fp32 sum instead: still exact."""
    rng = gen.rng_for(963, 1)
    E, K, N = 2, 256, 64
    sc = gen.scales_loguniform(rng, (E, N, K // 32))
    sc[0, 3, 2] = 0x3580            # 2^-20
    sc[1, 40, 7] = 0x4680           # 2^14
    sc[1, 17, 0] = 0x0000           # zero
    run_gmm_onehot(rng, E, K, N, np.array([K // 2, K // 2]), w4.W4_OUT_F32, w4.W4_KERNEL_TILED, "tiled-exact", sc)


# split-K dense decode kernel (w4a16_linear, M <= 16, K over 1024): 16 rows per call
@pytest.mark.parametrize("K", [1088, 1120, 2080])
def test_onehot_splitk_kernel(K):
    rng = gen.rng_for(964, K)
    N = 48
    packed, tiled, codes, sc = weights(rng, 1, N, K)
    qd, sd = to_dev(packed), bf16_dev(tiled)
    ws = torch.empty(max(16, w4.w4a16_linear_workspace(16, K, N)), dtype=torch.uint8, device="cuda")
    say("[onehot split-K] K=%d N=%d" % (K, N))
    ys = []
    for k0 in range(0, K, 16):
        x = onehot(np.arange(k0, k0 + 16), K)
        y = torch.empty(16, N, dtype=torch.bfloat16, device="cuda")
        w4.w4a16_linear(bf16_dev(x), qd, sd, N, y, ws)
        ys.append(y)
    torch.cuda.synchronize()
    got = np.concatenate([bits_host(y) for y in ys])
    check_exact(got, onehot(np.arange(K), K), codes[0], sc[0], w4.W4_OUT_BF16, "split-K K=%d" % K)


def test_onehot_dense_prefill_linear():
    """w4a16_linear over many rows (the tiled kernel, E = 1, no gather)."""
    rng = gen.rng_for(965, 1)
    K, N = 1056, 256
    packed, tiled, codes, sc = weights(rng, 1, N, K)
    x = onehot(np.arange(K), K)
    say("[onehot dense prefill] M=%d K=%d N=%d" % (K, K, N))
    y = w4.linear(bf16_dev(x), to_dev(packed), bf16_dev(tiled), N)
    torch.cuda.synchronize()
    check_exact(bits_host(y), x, codes[0], sc[0], w4.W4_OUT_BF16, "dense prefill")


# gated epilogue in the gate's negative tail
@pytest.mark.parametrize("kernel,E,R", [(w4.W4_KERNEL_STREAM, 4, 64), (w4.W4_KERNEL_TILED, 2, 512)])
def test_geglu_negative_tail_elementwise(kernel, E, R):
    """Gate pre-activations s*q in [-6, -3] (q = -8, s in [0.375, 0.75]), up
    projection 1.0: a = bf16(gelu_tanh(gate)) must be within one bf16 step of
    the oracle's fp64 value at every element."""
    rng = gen.rng_for(966, kernel)
    K, I = 256, 64
    N = 2 * I
    codes = np.empty((E, N, K), dtype=np.int8)
    codes[:, :I] = -8
    codes[:, I:] = 1
    sc = np.empty((E, N, K // 32), dtype=np.uint16)
    sc[:, :I] = gen.to_bf16_bits(rng.uniform(0.375, 0.75, (E, I, K // 32)).astype(np.float32))
    sc[:, I:] = ONE
    packed = np.concatenate([layout.encode(codes[e]) for e in range(E)])
    tiled = np.concatenate([layout.encode_scales(sc[e]) for e in range(E)])
    ks = np.arange(R) % K
    x = onehot(ks, K)
    offs = np.linspace(0, R, E + 1).astype(np.int32)
    out = torch.empty(R, I, dtype=torch.bfloat16, device="cuda")
    say("[geglu tail] kernel=%d E=%d R=%d" % (kernel, E, R))
    with w4.gemm_kernel(kernel):
        w4.moe_gmm(bf16_dev(x), None, to_dev(offs), E, R, K, N, to_dev(packed), bf16_dev(tiled),
                   w4.W4_EPI_GEGLU_TANH, out, w4.W4_OUT_BF16)
    torch.cuda.synchronize()
    got = oracle.bf16_bits_to_f64(bits_host(out))
    ref = np.empty((R, I))
    for e in range(E):
        lo, hi = offs[e], offs[e + 1]
        h = oracle.bf16_bits_to_f64(oracle.bf16_from_f64(oracle.linear_f64(x[lo:hi], codes[e], sc[e])))
        assert np.all((h[:, :I] >= -6) & (h[:, :I] <= -3))
        ref[lo:hi] = oracle.bf16_bits_to_f64(oracle.bf16_from_f64(oracle.gelu_tanh(h[:, :I]) * h[:, I:]))
    rel = np.abs(got - ref) / np.abs(ref)
    same = np.mean(got == ref)
    say("  worst element-wise rel %.2e, bit-identical %.4f" % (rel.max(), same))
    assert rel.max() <= 2.0 ** -8 and same >= 0.98
