"""GPU parity of the FP8 (W8A8, E4M3) comparison path against the oracle
(oracle/fp8.py): the per-row quantization bit for bit (an integer decision
taken from fp32 divisions on both sides), the grouped matmul on the FP8
matrix cores and the whole layer with the normwise tolerance."""

import numpy as np
import pytest
import torch

import gen
import int4_group_quantized_q4_amd as w4
import oracle
from oracle import fp8
from gpu_util import bf16_dev, bits_host, say, to_dev

pytestmark = pytest.mark.gpu


def quantize_on_gpu(x_bits):
    rows, K = x_bits.shape
    xd = bf16_dev(x_bits)
    q = torch.empty(rows, K, dtype=torch.uint8, device=xd.device)
    s = torch.empty(rows, dtype=torch.float32, device=xd.device)
    w4.w8a8_quantize_rows(xd, q, s)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("rows,K", [(1, 32), (37, 96), (64, 2816), (300, 704)])
def test_quantize_rows_bit_exact(rows, K):
    say("[fp8 quant] rows=%d K=%d" % (rows, K))
    rng = gen.rng_for(950, rows + K)
    x = gen.bf16_normal(rng, (rows, K))
    q, s = quantize_on_gpu(x)
    qr, sr = fp8.quantize_rows(x)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(q, qr)


def test_quantize_rows_ties_subnormals_and_zero_rows():
    """Rows whose largest magnitude is 448 have scale 1, so x / s = x exactly
    and the E4M3 rounding itself is exercised: every midpoint between
    neighbouring codes (ties go to the even code), values one bf16 step either
    side of it, the subnormal range, and a row of zeros."""
    vals = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = oracle.bf16_from_f64((vals[:-1] + vals[1:]) / 2.0)     # 5 significant bits: exact in bf16
    lead = oracle.bf16_from_f64(np.array([448.0]))
    rows = []
    for sign in (0, 0x8000):
        for v in (mids, mids - 1, mids + 1):                       # the midpoint, one bf16 step below, above
            row = np.zeros(160, dtype=np.uint16)
            row[0] = lead[0]
            row[1:1 + len(v)] = (v.astype(np.uint16) | sign).astype(np.uint16)
            rows.append(row)
    rows.append(np.zeros(160, dtype=np.uint16))
    bits = np.array(rows, dtype=np.uint16)
    q, s = quantize_on_gpu(bits)
    qr, sr = fp8.quantize_rows(bits)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(q, qr)
    assert not q[-1].any() and s[-1] == 1.0


def fp8_experts(rng, E, N, K):
    return gen.fp8_codes(rng, (E, N, K)), gen.fp8_scales(rng, (E, N))


def run_gmm(xq, xs, row_index, offsets, E, R, K, N, wq, wsc, epi, out_dtype):
    dv = torch.device("cuda:0")
    ncol = N // 2 if epi != w4.W4_EPI_NONE else N
    out = torch.empty(R, ncol, dtype=torch.float32 if out_dtype == w4.W4_OUT_F32 else torch.bfloat16, device=dv)
    w4.w8a8_moe_gmm(to_dev(xq), to_dev(xs), None if row_index is None else to_dev(row_index),
                    None if offsets is None else to_dev(offsets), E, R, K, N, to_dev(wq.reshape(-1)),
                    to_dev(wsc.reshape(-1)), epi, out, out_dtype)
    torch.cuda.synchronize()
    return out


def oracle_gmm(xq, xs, row_index, offsets, wq, wsc, epi):
    """Sorted row i of expert e: fp64 FP8 matmul, then the epilogue's bf16
    rounding points (gated: bf16 h, bf16(act(h_gate) * h_up))."""
    E, N, K = wq.shape
    R = len(row_index) if row_index is not None else xq.shape[0]
    src = row_index if row_index is not None else np.arange(R)
    offs = offsets if offsets is not None else np.array([0, R])
    out = np.zeros((R, N // 2 if epi != w4.W4_EPI_NONE else N), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if lo == hi:
            continue
        y = fp8.linear(xq[src[lo:hi]], xs[src[lo:hi]], wq[e], wsc[e])
        if epi == w4.W4_EPI_NONE:
            out[lo:hi] = y
        else:
            h = oracle.bf16_bits_to_f64(oracle.bf16_from_f64(y))
            act = oracle.gelu_tanh if epi == w4.W4_EPI_GEGLU_TANH else fp8.ACTIVATIONS["silu"]
            out[lo:hi] = oracle.bf16_bits_to_f64(oracle.bf16_from_f64(act(h[:, :N // 2]) * h[:, N // 2:]))
    return out


def check(y_gpu, ref, label):
    y = y_gpu.float().cpu().numpy().astype(np.float64)
    ok, mx, rms = oracle.within_tolerance(y, ref)
    say("[fp8 gmm] %s max_rel=%.3g rms_rel=%.3g" % (label, mx, rms))
    assert ok, (label, mx, rms)


# (E, counts law, K, N): few rows per expert take the streaming kernel, many the tiled one
GMM_CASES = [
    ("stream", 8, 3, 2816, 256),
    ("stream-tailK", 5, 7, 704, 128),
    ("stream-K96", 4, 20, 96, 64),
    ("tiled", 4, 150, 704, 256),
    ("tiled-ragged", 6, 97, 2816, 128),
]


@pytest.mark.parametrize("label,E,mean_rows,K,N", GMM_CASES)
@pytest.mark.parametrize("epi", [w4.W4_EPI_NONE, w4.W4_EPI_GEGLU_TANH])
def test_fp8_gmm_vs_oracle(label, E, mean_rows, K, N, epi):
    if epi != w4.W4_EPI_NONE and (N // 16 // 2) % 2 != 0:
        pytest.skip("gate tiles go in pairs")
    rng = gen.rng_for(951, E * 1000 + K + N + epi)
    counts = rng.integers(0, 2 * mean_rows + 1, E)
    counts[rng.integers(0, E)] = 0                  # an empty expert
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(offsets[-1])
    x_rows = max(1, R // 2 + 3)
    x = gen.bf16_normal(rng, (x_rows, K))
    xq, xs = fp8.quantize_rows(x)
    row_index = rng.integers(0, x_rows, R).astype(np.int32)
    wq, wsc = fp8_experts(rng, E, N, K)
    say("[fp8 gmm] %s E=%d R=%d K=%d N=%d epi=%d" % (label, E, R, K, N, epi))
    out_dtype = w4.W4_OUT_BF16 if epi != w4.W4_EPI_NONE else w4.W4_OUT_F32
    y = run_gmm(xq, xs, row_index, offsets, E, R, K, N, wq, wsc, epi, out_dtype)
    check(y, oracle_gmm(xq, xs, row_index, offsets, wq, wsc, epi), label)


def test_fp8_dense_no_offsets_bf16_out():
    rng = gen.rng_for(952, 1)
    M, K, N = 40, 512, 192
    x = gen.bf16_normal(rng, (M, K))
    xq, xs = fp8.quantize_rows(x)
    wq, wsc = fp8_experts(rng, 1, N, K)
    say("[fp8 gmm] dense M=%d K=%d N=%d" % (M, K, N))
    y = run_gmm(xq, xs, None, None, 1, M, K, N, wq, wsc, w4.W4_EPI_NONE, w4.W4_OUT_BF16)
    ref = fp8.linear(xq, xs, wq[0], wsc[0])
    check(y, ref, "dense")
    # bf16 output: the rounding of the fp32 result
    yf = run_gmm(xq, xs, None, None, 1, M, K, N, wq, wsc, w4.W4_EPI_NONE, w4.W4_OUT_F32)
    assert np.array_equal(bits_host(y), oracle.bf16_from_f32(yf.cpu().numpy()))


def layer_case(T, router, label):
    """The layer stage by stage, each stage against the oracle fed with the
    GPU's own input to that stage: the per-row quantizations are integer
    decisions taken from fp32 divisions on both sides (bit-exact), the
    matmuls and the combine are floating point (normwise tolerance).  The
    oracle's own end-to-end y is compared too, with a looser bound: the gated
    activation a is re-quantized to E4M3 per row, and wherever the GPU's a
    and the oracle's a differ by a bf16 step (fp32 against fp64 sums) at a
    row's largest element, that row's scale and all its codes move, which
    is FP8 quantization noise of about 2^-5 relative on those rows."""
    cfg = gen.MOE_DECODE
    E, k, d, I = cfg["E"], cfg["k"], cfg["d"], cfg["I"]
    R = T * k
    rng = gen.rng_for(953, T)
    x = gen.bf16_normal(rng, (T, d))
    logits = gen.router_logits(rng, T, E, router, 1.1)
    w1q, w1s = fp8_experts(rng, E, 2 * I, d)
    w2q, w2s = fp8_experts(rng, E, d, I)
    say("[fp8 layer] %s T=%d" % (label, T))
    y, views = w4.fp8_moe_layer(bf16_dev(x), to_dev(logits), k, I, to_dev(w1q.reshape(-1)), to_dev(w1s.reshape(-1)),
                                to_dev(w2q.reshape(-1)), to_dev(w2s.reshape(-1)))
    torch.cuda.synchronize()
    ref = fp8.moe_layer(x, logits, w1q, w1s, w2q, w2s, k=k, keep=True)
    plan = ref["plan"]
    assert np.array_equal(views["topk_ids"].cpu().numpy(), plan["ids"])
    assert np.array_equal(views["expert_offsets"].cpu().numpy(), plan["offsets"])
    # quantized x: bit-exact
    assert np.array_equal(views["xq"].cpu().numpy(), ref["xq"])
    assert np.array_equal(views["x_scale"].cpu().numpy().view(np.uint32), ref["x_scale"].view(np.uint32))

    def close(got, want, what):
        ok, mx, rms = oracle.within_tolerance(got, want)
        say("[fp8 layer] %s %s: max_rel=%.3g rms_rel=%.3g" % (label, what, mx, rms))
        assert ok, (what, mx, rms)

    # gate/up with the gated activation, from the (identical) quantized x
    a_bits = bits_host(views["a"])
    close(oracle.bf16_bits_to_f64(a_bits), oracle.bf16_bits_to_f64(ref["a"]), "a")
    # quantized a: bit-exact against the oracle's quantization of the GPU's a
    aq_ref, as_ref = fp8.quantize_rows(a_bits)
    aq = views["aq"].cpu().numpy()
    a_scale = views["a_scale"].cpu().numpy()
    assert np.array_equal(a_scale.view(np.uint32), as_ref.view(np.uint32))
    assert np.array_equal(aq, aq_ref)
    # down matmul from the GPU's quantized a
    o_ref = np.zeros((R, d))
    offs = plan["offsets"]
    for e in range(E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi > lo:
            o_ref[lo:hi] = fp8.linear(aq[lo:hi], a_scale[lo:hi], w2q[e], w2s[e])
    o = views["o"].cpu().numpy().astype(np.float64)
    close(o, o_ref, "o")
    # combine of the GPU's o
    from oracle.moe import combine
    y_ref = combine(o, plan["inv"], plan["weights"])
    yg = oracle.bf16_bits_to_f64(bits_host(y))
    close(yg, y_ref, "y (combine of the GPU's o)")
    # end to end against the oracle's own chain
    ok, mx, rms = oracle.within_tolerance(yg, ref["y64"], 2e-2, 1e-2)
    say("[fp8 layer] %s y end to end: max_rel=%.3g rms_rel=%.3g" % (label, mx, rms))
    assert ok, ("y end to end", mx, rms)


def test_fp8_layer_decode_full_size():
    layer_case(64, "normal", "moe-decode")


def test_fp8_layer_prefill_tiled_path():
    # 1024 tokens x 8 slots over 128 experts: 64 rows per expert on average,
    # past the streaming threshold, so both matmuls take the tiled kernel
    layer_case(1024, "zipf", "prefill-1024")
