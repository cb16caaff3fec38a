"""GPU parity of the MoE path (route, grouped matmul, epilogues, combine, the
whole layer) against the oracle.  Integer plan outputs are compared exactly;
floating-point outputs with the normwise tolerance."""

import numpy as np
import pytest
import torch

import gen
import int4_group_quantized_q4_amd as w4
import oracle
from gpu_util import bf16_dev, bits_host, expert_weights, say, to_dev

pytestmark = pytest.mark.gpu


def check_route(logits, k, label):
    T, E = logits.shape
    say("[route] %s T=%d E=%d k=%d" % (label, T, E, k))
    plan = w4.moe_route(to_dev(logits), k)
    torch.cuda.synchronize()
    ref = oracle.route(logits, k)
    assert np.array_equal(plan["topk_ids"].cpu().numpy(), ref["ids"]), label
    assert np.array_equal(plan["expert_offsets"].cpu().numpy(), ref["offsets"]), label
    assert np.array_equal(plan["sorted_rows"].cpu().numpy(), ref["perm"]), label
    assert np.array_equal(plan["sorted_tokens"].cpu().numpy(), ref["tokens"]), label
    assert np.array_equal(plan["row_to_sorted"].cpu().numpy(), ref["inv"]), label
    assert np.allclose(plan["topk_weights"].cpu().numpy(), ref["weights"], rtol=2e-6, atol=1e-9), label


def test_route_moe_decode():
    cfg = gen.MOE_DECODE
    check_route(gen.router_logits(gen.rng_for(cfg["id"], 3), cfg["T"], cfg["E"]), cfg["k"], "moe-decode")


def test_route_moe_prefill_zipf():
    cfg = gen.MOE_PREFILL
    logits = gen.router_logits(gen.rng_for(cfg["id"], 3), cfg["T"], cfg["E"], "zipf", cfg["zipf_s"])
    check_route(logits, cfg["k"], "moe-prefill")


# R = 4096: the largest one-workgroup plan; R = 33600 and 36900: more than 128
# chunks of 256 rows, where the scan's parts walk their chunks in batches
@pytest.mark.parametrize("T,E,k", [(1, 128, 8), (37, 16, 3), (33, 256, 16), (5, 8, 8), (300, 64, 1), (1000, 128, 8),
                                   (512, 128, 8), (513, 128, 8), (4200, 128, 8), (4100, 256, 9)])
def test_route_shapes_and_ties(T, E, k):
    rng = gen.rng_for(930, T + E + k)
    logits = gen.router_logits(rng, T, E)
    logits[0, :] = 0.5                               # a row of ties: ids 0..k-1
    if T > 3:
        logits[3, E // 2] = logits[3, 1]
        logits[2, :] = np.round(logits[2, :])        # many ties
    check_route(logits, k, "shapes")


def test_route_empty():
    offs = torch.full((129,), -1, dtype=torch.int32, device="cuda")
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    w4.w4a16_moe_route(torch.empty(0, 128, dtype=torch.float32, device="cuda"), 8, e, e.float(), offs, e, e, e,
                       torch.empty(16, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert int(offs.abs().sum()) == 0


def _gmm_case(E, R, K, N, seed, empty_every=3):
    rng = gen.rng_for(931, seed)
    counts = rng.integers(0, 2 * R // E + 1, E)
    counts[::empty_every] = 0                        # some experts get no rows
    if counts.sum() == 0:
        counts[1] = 5
    R = int(counts.sum())
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    x_rows = max(1, R // 2 + 3)
    x = gen.bf16_normal(rng, (x_rows, K))
    row_index = rng.integers(0, x_rows, R).astype(np.int32)
    packed, sct, codes, sc = expert_weights(rng, E, N, K)
    return offsets, R, x, row_index, packed, sct, codes, sc


@pytest.mark.parametrize("E,R,K,N", [(8, 40, 256, 64), (4, 100, 704, 32), (16, 20, 96, 48), (3, 600, 128, 16)])
def test_gmm_plain_f32_with_gather(E, R, K, N):
    offsets, R, x, row_index, packed, sct, codes, sc = _gmm_case(E, R, K, N, E + R + K + N)
    say("[gmm] E=%d R=%d K=%d N=%d" % (E, R, K, N))
    out = torch.full((R, N), float("nan"), dtype=torch.float32, device="cuda")
    w4.moe_gmm(bf16_dev(x), to_dev(row_index), to_dev(offsets), E, R, K, N, to_dev(packed), bf16_dev(sct),
                     w4.W4_EPI_NONE, out, w4.W4_OUT_F32)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = np.zeros((R, N))
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            ref[lo:hi] = oracle.linear_f64(x[row_index[lo:hi]], codes[e], sc[e])
    ok, mx, rms = oracle.within_tolerance(got, ref)
    say("  max_rel %.2e rms_rel %.2e" % (mx, rms))
    assert ok and not np.isnan(got).any()


# Short-K kernel (K <= 1024, plain epilogue, <= 16 rows per expert on
# average): an expert above 16 rows takes several row passes; K at the limit
# (8 full blocks), with 3 tail groups, and below one block; tiles per expert
# not a multiple of the workgroup's 16; both output types.
@pytest.mark.parametrize("K,N,counts,out_dtype", [
    (704, 96, [40, 0, 5, 3], w4.W4_OUT_F32),
    (1024, 64, [17, 1, 0, 16, 2], w4.W4_OUT_F32),
    (992, 272, [3, 33, 0, 9], w4.W4_OUT_BF16),
    (96, 48, [1, 2, 20, 0, 4], w4.W4_OUT_BF16),
])
def test_gmm_short_k(K, N, counts, out_dtype):
    rng = gen.rng_for(932, K + N)
    E = len(counts)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    R = int(offsets[-1])
    x_rows = R // 2 + 3
    x = gen.bf16_normal(rng, (x_rows, K))
    row_index = rng.integers(0, x_rows, R).astype(np.int32)
    packed, sct, codes, sc = expert_weights(rng, E, N, K)
    say("[gmm short-K] K=%d N=%d counts=%s" % (K, N, counts))
    tdt = torch.float32 if out_dtype == w4.W4_OUT_F32 else torch.bfloat16
    out = torch.full((R, N), float("nan"), dtype=tdt, device="cuda")
    w4.moe_gmm(bf16_dev(x), to_dev(row_index), to_dev(offsets), E, R, K, N, to_dev(packed), bf16_dev(sct),
               w4.W4_EPI_NONE, out, out_dtype)
    torch.cuda.synchronize()
    got = (out.cpu().numpy().astype(np.float64) if out_dtype == w4.W4_OUT_F32
           else oracle.bf16_bits_to_f64(bits_host(out)))
    ref = np.zeros((R, N))
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            ref[lo:hi] = oracle.linear_f64(x[row_index[lo:hi]], codes[e], sc[e])
    ok, mx, rms = oracle.within_tolerance(got, ref)
    say("  max_rel %.2e rms_rel %.2e" % (mx, rms))
    assert ok and not np.isnan(got).any()


# Decode shapes (a few rows per expert) with many weight tiles: the streaming
# kernel's ring variants (>= 4096 tiles in all, and fewer) and the short-K
# kernel (K = 736).  Partial last blocks of 1, 2 and 3 groups and whole
# blocks; plain fp32 / bf16 and both gated outputs; experts with 0, 1, 8, 9
# and 17 rows (one and two passes of 16).
@pytest.mark.parametrize("E,N,K,epi,out_dtype", [
    (16, 8192, 1056, w4.W4_EPI_NONE, w4.W4_OUT_F32),
    (32, 4096, 736, w4.W4_EPI_NONE, w4.W4_OUT_BF16),
    (16, 8192, 2848, w4.W4_EPI_SWIGLU, w4.W4_OUT_BF16),
    (16, 8192, 1024, w4.W4_EPI_GEGLU_TANH, w4.W4_OUT_BF16),
    (32, 1024, 3040, w4.W4_EPI_NONE, w4.W4_OUT_BF16),
])
def test_gmm_decode_many_tiles(E, N, K, epi, out_dtype):
    counts = ([1, 0, 0, 8, 9, 0, 17, 0, 3] + [0] * E)[:E - 1] + [2]
    rng = gen.rng_for(933, K + epi + E)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    R = int(offsets[-1])
    x_rows = R + 5
    x = gen.bf16_normal(rng, (x_rows, K))
    row_index = rng.integers(0, x_rows, R).astype(np.int32)
    packed, sct, codes, sc = expert_weights(rng, E, N, K)
    say("[gmm decode] E=%d N=%d K=%d epi=%d out=%d" % (E, N, K, epi, out_dtype))
    gated = epi != w4.W4_EPI_NONE
    NO = N // 2 if gated else N
    tdt = torch.float32 if out_dtype == w4.W4_OUT_F32 else torch.bfloat16
    out = torch.full((R, NO), float("nan"), dtype=tdt, device="cuda")
    w4.moe_gmm(bf16_dev(x), to_dev(row_index), to_dev(offsets), E, R, K, N, to_dev(packed), bf16_dev(sct),
               epi, out, out_dtype)
    torch.cuda.synchronize()
    got = (out.cpu().numpy().astype(np.float64) if out_dtype == w4.W4_OUT_F32
           else oracle.bf16_bits_to_f64(bits_host(out)))
    ref = np.zeros((R, NO))
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            if gated:
                h = oracle.bf16_bits_to_f64(oracle.linear(x[row_index[lo:hi]], codes[e], sc[e]))
                fn = oracle.gelu_tanh if epi == w4.W4_EPI_GEGLU_TANH else oracle.moe.silu
                ref[lo:hi] = fn(h[:, :NO]) * h[:, NO:]
            else:
                ref[lo:hi] = oracle.linear_f64(x[row_index[lo:hi]], codes[e], sc[e])
    ok, mx, rms = oracle.within_tolerance(got, ref)
    say("  max_rel %.2e rms_rel %.2e" % (mx, rms))
    assert ok and not np.isnan(got).any()


@pytest.mark.parametrize("act", [w4.W4_EPI_GEGLU_TANH, w4.W4_EPI_SWIGLU])
def test_gmm_gated_epilogue(act):
    E, R, K, N = 6, 90, 256, 128
    offsets, R, x, row_index, packed, sct, codes, sc = _gmm_case(E, R, K, N, 77 + act)
    say("[gmm gated] act=%d" % act)
    out = torch.empty((R, N // 2), dtype=torch.bfloat16, device="cuda")
    w4.moe_gmm(bf16_dev(x), to_dev(row_index), to_dev(offsets), E, R, K, N, to_dev(packed), bf16_dev(sct),
                     act, out, w4.W4_OUT_BF16)
    torch.cuda.synchronize()
    got = oracle.bf16_bits_to_f64(bits_host(out))
    fn = oracle.gelu_tanh if act == w4.W4_EPI_GEGLU_TANH else oracle.moe.silu
    ref = np.zeros((R, N // 2))
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            h = oracle.bf16_bits_to_f64(oracle.linear(x[row_index[lo:hi]], codes[e], sc[e]))
            ref[lo:hi] = fn(h[:, :N // 2]) * h[:, N // 2:]
    ok, mx, rms = oracle.within_tolerance(got, ref)
    say("  max_rel %.2e rms_rel %.2e" % (mx, rms))
    assert ok


# The weighted combine on its own: fp32 and bf16 expert outputs, k a multiple
# of the kernel's 4-slot chunk (8, 12), below it (1, 3) and between (5).
@pytest.mark.parametrize("T,k,N,o_dtype", [(64, 8, 2816, w4.W4_OUT_F32), (64, 8, 2816, w4.W4_OUT_BF16),
                                           (5, 3, 96, w4.W4_OUT_BF16), (33, 1, 64, w4.W4_OUT_F32),
                                           (7, 5, 16, w4.W4_OUT_F32), (3, 12, 48, w4.W4_OUT_BF16)])
def test_combine(T, k, N, o_dtype):
    rng = gen.rng_for(941, T * k + N + o_dtype)
    R = T * k
    inv = rng.permutation(R).astype(np.int32)
    wts = rng.random((T, k)).astype(np.float32)
    if o_dtype == w4.W4_OUT_F32:
        o = rng.standard_normal((R, N)).astype(np.float32)
        o_dev = torch.from_numpy(o).cuda()
        o64 = o.astype(np.float64)
    else:
        o_bits = gen.bf16_normal(rng, (R, N))
        o_dev = bf16_dev(o_bits)
        o64 = oracle.bf16_bits_to_f64(o_bits)
    say("[combine] T=%d k=%d N=%d o_dtype=%d" % (T, k, N, o_dtype))
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    w4.w4a16_moe_combine(o_dev, o_dtype, to_dev(inv), to_dev(wts), T, k, N, y)
    torch.cuda.synchronize()
    got = oracle.bf16_bits_to_f64(bits_host(y))
    ref = oracle.moe.combine(o64, inv, wts)
    ok, mx, rms = oracle.within_tolerance(got, ref)
    say("  max_rel %.2e rms_rel %.2e" % (mx, rms))
    assert ok


def moe_inputs(cfg, seed_base=0):
    rng = gen.rng_for(cfg["id"], 20 + seed_base)
    T, d, I, E, k = cfg["T"], cfg["d"], cfg["I"], cfg["E"], cfg["k"]
    x = gen.bf16_normal(rng, (T, d))
    logits = gen.router_logits(rng, T, E, cfg["router"], cfg.get("zipf_s", 1.1))
    w1p, w1t, w1c, w1s = expert_weights(rng, E, 2 * I, d)
    w2p, w2t, w2c, w2s = expert_weights(rng, E, d, I)
    return x, logits, (w1p, w1t, w1c, w1s), (w2p, w2t, w2c, w2s)


def check_layer(cfg, label, ties=False, bump=()):
    T, d, I, E, k = cfg["T"], cfg["d"], cfg["I"], cfg["E"], cfg["k"]
    x, logits, (w1p, w1t, w1c, w1s), (w2p, w2t, w2c, w2s) = moe_inputs(cfg)
    for e, t0, t1 in bump:                               # expert e in the top-k of tokens t0 .. t1-1
        logits[t0:t1, e] += 20.0
    if ties:
        logits[0, :] = 0.5                               # a row of ties: ids 0..k-1
        if T > 5:
            logits[3, E // 2] = logits[3, 1]
            logits[2, :] = np.round(logits[2, :])            # many ties
            logits[5:, :] = np.round(logits[5:, :] * 4) / 4  # ties in every row
    say("[moe layer] %s T=%d" % (label, T))
    y, views = w4.moe_layer(bf16_dev(x), to_dev(logits), k, I, to_dev(w1p), bf16_dev(w1t), to_dev(w2p),
                            bf16_dev(w2t), w4.W4_EPI_GEGLU_TANH)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(x, logits, w1c, w1s, w2c, w2s, k=k, keep=True)
    plan = ref["plan"]
    assert np.array_equal(views["topk_ids"].cpu().numpy(), plan["ids"])
    assert np.allclose(views["topk_weights"].cpu().numpy(), plan["weights"], rtol=2e-6, atol=1e-9)
    if views["sorted"]:   # the sort outputs exist on the sorted path only
        assert np.array_equal(views["expert_offsets"].cpu().numpy(), plan["offsets"])
        assert np.array_equal(views["sorted_tokens"].cpu().numpy(), plan["tokens"])
    # o is stored at the routed rows r = t*k + j, a too on the streaming path
    # and in sorted order on the sorted path; the oracle's follow the sort
    a_ref = ref["a"] if views["sorted"] else ref["a"][plan["inv"]]
    a_ok, a_mx, a_rms = oracle.within_tolerance(oracle.bf16_bits_to_f64(bits_host(views["a"])),
                                                oracle.bf16_bits_to_f64(a_ref))
    o_ok, o_mx, o_rms = oracle.within_tolerance(views["o"].cpu().numpy(), ref["o"][plan["inv"]])
    y_ok, y_mx, y_rms = oracle.within_tolerance(oracle.bf16_bits_to_f64(bits_host(y)),
                                                oracle.bf16_bits_to_f64(ref["y"]))
    say("  %s path  a: %.2e/%.2e  o: %.2e/%.2e  y: %.2e/%.2e (max_rel/rms_rel)"
        % ("sorted" if views["sorted"] else "streaming", a_mx, a_rms, o_mx, o_rms, y_mx, y_rms))
    assert a_ok and o_ok and y_ok
    return views["sorted"]


def test_moe_layer_decode_full_size():
    assert not check_layer(gen.MOE_DECODE, "moe-decode")


@pytest.mark.parametrize("kernel", [w4.W4_KERNEL_AUTO, w4.W4_KERNEL_TILED])
def test_moe_layer_decode_both_paths(kernel):
    """The 64-token layer on the streaming path (rows found from the ids, no
    sort) and, forced, on the sorted tiled path."""
    cfg = dict(gen.MOE_DECODE, id=942)
    with w4.gemm_kernel(kernel):
        assert check_layer(cfg, "moe-decode kernel=%d" % kernel) == (kernel == w4.W4_KERNEL_TILED)


def test_moe_layer_decode_popular_experts():
    """The 64-token layer (4 rows per expert on average, so each gate/up
    workgroup takes several unit sets in turn) with three experts far above
    the average: 40 rows (16-row passes of 16, 16 and 8), 20 rows (16 and 4)
    and 21 rows (16 and 5).  Each pass loads the next pass's weight ring and first
    scale span, and here a pass's successor is another pass over the same
    tiles as well as the next unit set's tiles."""
    cfg = dict(gen.MOE_DECODE, id=943)
    assert not check_layer(cfg, "moe-decode, popular experts", bump=((5, 0, 40), (77, 20, 38), (126, 47, 64)))


@pytest.mark.parametrize("T", [1, 40, 64])
def test_moe_layer_rows_from_logits_with_ties(T):
    """Up to 64 tokens on the one-tile streaming kernel (K = d above the
    short kernel's limit, at least 4096 weight tiles) the gate/up workgroups
    rank the logits themselves instead of reading top-k ids, and write the
    ids and weights.  Ties between logits must resolve to the lower expert
    id, as in the routing kernel."""
    cfg = dict(id=949, T=T, d=1536, I=256, E=128, k=8, router="normal")
    assert not check_layer(cfg, "rows from logits, ties", ties=True)


@pytest.mark.parametrize("cfg", [dict(id=940, T=19, d=96, I=64, E=8, k=3, router="normal"),
                                 dict(id=943, T=1, d=2816, I=704, E=128, k=8, router="normal"),
                                 dict(id=944, T=256, d=256, I=96, E=16, k=4, router="normal"),
                                 dict(id=945, T=40, d=64, I=1056, E=8, k=2, router="normal"),
                                 dict(id=946, T=300, d=128, I=64, E=64, k=1, router="normal")])
def test_moe_layer_small_shapes(cfg):
    """Streaming path with a 1-token batch, with many rows per expert
    (multi-pass, 64 per expert), with K above the short kernel's limit (I =
    1056: the down matmul on the long-K kernel), and more than 256 tokens (the
    sorted path)."""
    check_layer(cfg, "small T=%d" % cfg["T"])


@pytest.mark.parametrize("cfg", [dict(id=947, T=256, d=2816, I=704, E=128, k=8, router="normal"),
                                 dict(id=948, T=160, d=256, I=1056, E=64, k=8, router="normal")])
def test_moe_layer_sixteen_rows_per_expert(cfg):
    """About 16 rows per expert on the streaming path, where about half the
    experts take a second 16-row pass: the 256-token batch of the end-to-end
    decode at full size, and a long-K down projection (decode kernel)."""
    assert not check_layer(cfg, "16 rows/expert T=%d" % cfg["T"])


@pytest.mark.parametrize("kernel", [w4.W4_KERNEL_AUTO, w4.W4_KERNEL_STREAM])
def test_moe_layer_prefill_full_size(kernel):
    with w4.gemm_kernel(kernel):
        assert check_layer(gen.MOE_PREFILL, "moe-prefill kernel=%d" % kernel)   # over 256 tokens: sorted


@pytest.mark.parametrize("T,d,I,E,k", [(64, 256, 96, 16, 4), (64, 2816, 704, 128, 8), (3, 64, 32, 8, 8),
                                       (256, 128, 64, 16, 2)])
def test_streaming_calls_topk_gmm_ids(T, d, I, E, k):
    """The streaming path's calls on their own: top-k equals the routing plan's;
    the gate/up and down matmuls over rows found from the ids match the
    oracle's a and o (stored at the routed rows); the combine with the
    identity row map gives the oracle's y."""
    cfg = dict(id=947, T=T, d=d, I=I, E=E, k=k, router="normal")
    x, logits, (w1p, w1t, w1c, w1s), (w2p, w2t, w2c, w2s) = moe_inputs(cfg, T + d)
    say("[streaming calls] T=%d d=%d I=%d E=%d k=%d" % (T, d, I, E, k))
    dev = "cuda"
    R = T * k
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    wts = torch.empty(T, k, dtype=torch.float32, device=dev)
    w4.w4a16_moe_topk(to_dev(logits), k, ids, wts)
    a = torch.full((R, I), float("nan"), dtype=torch.bfloat16, device=dev)
    o = torch.full((R, d), float("nan"), dtype=torch.float32, device=dev)
    y = torch.empty(T, d, dtype=torch.bfloat16, device=dev)
    w1q, w1s_d, w2q, w2s_d = to_dev(w1p), bf16_dev(w1t), to_dev(w2p), bf16_dev(w2t)
    w4.w4a16_moe_gmm_ids(bf16_dev(x), ids, T, k, k, E, d, 2 * I, w1q, w1s_d, w4.W4_EPI_GEGLU_TANH, a, w4.W4_OUT_BF16)
    w4.w4a16_moe_gmm_ids(a, ids, T, k, 1, E, I, d, w2q, w2s_d, w4.W4_EPI_NONE, o, w4.W4_OUT_F32)
    ident = torch.arange(R, dtype=torch.int32, device=dev)
    w4.w4a16_moe_combine(o, w4.W4_OUT_F32, ident, wts, T, k, d, y)
    torch.cuda.synchronize()
    ref = oracle.moe_layer(x, logits, w1c, w1s, w2c, w2s, k=k, keep=True)
    plan = ref["plan"]
    assert np.array_equal(ids.cpu().numpy(), plan["ids"])
    assert np.allclose(wts.cpu().numpy(), plan["weights"], rtol=2e-6, atol=1e-9)
    a_ok, a_mx, a_rms = oracle.within_tolerance(oracle.bf16_bits_to_f64(bits_host(a)),
                                                oracle.bf16_bits_to_f64(ref["a"][plan["inv"]]))
    o_ok, o_mx, o_rms = oracle.within_tolerance(o.cpu().numpy(), ref["o"][plan["inv"]])
    y_ok, y_mx, y_rms = oracle.within_tolerance(oracle.bf16_bits_to_f64(bits_host(y)),
                                                oracle.bf16_bits_to_f64(ref["y"]))
    say("  a %.2e/%.2e  o %.2e/%.2e  y %.2e/%.2e" % (a_mx, a_rms, o_mx, o_rms, y_mx, y_rms))
    assert a_ok and o_ok and y_ok


@pytest.mark.parametrize("T,d,I,E,k", [(64, 2816, 704, 128, 8), (1, 2816, 704, 128, 8), (40, 1536, 256, 128, 8),
                                       (64, 256, 96, 16, 4), (100, 2816, 704, 128, 8)])
def test_gmm_logits_matches_topk_and_gmm_ids(T, d, I, E, k):
    """w4a16_moe_gmm_logits against w4a16_moe_topk + w4a16_moe_gmm_ids (row_div
    k) on the same inputs: the ids agree exactly, the weights to fp32
    rounding (the two sum the softmax in different orders only when one of
    them is the routing kernel), and the gated outputs bit for bit (the same
    matmul over the same rows).  The first three shapes rank the logits in
    the matmul; the others (short K, more than 64 tokens) take the top-k
    launch."""
    cfg = dict(id=950, T=T, d=d, I=I, E=E, k=k, router="normal")
    x, logits, (w1p, w1t, _, _), _ = moe_inputs(cfg, T + d)
    logits[0, :] = 0.5                                   # ties
    if T > 3:
        logits[2, :] = np.round(logits[2, :])
    say("[gmm logits] T=%d d=%d I=%d E=%d k=%d" % (T, d, I, E, k))
    dev = "cuda"
    R = T * k
    xd, lg, w1q, w1s_d = bf16_dev(x), to_dev(logits), to_dev(w1p), bf16_dev(w1t)
    ids0 = torch.empty(T, k, dtype=torch.int32, device=dev)
    wts0 = torch.empty(T, k, dtype=torch.float32, device=dev)
    a0 = torch.full((R, I), float("nan"), dtype=torch.bfloat16, device=dev)
    w4.w4a16_moe_topk(lg, k, ids0, wts0)
    w4.w4a16_moe_gmm_ids(xd, ids0, T, k, k, E, d, 2 * I, w1q, w1s_d, w4.W4_EPI_GEGLU_TANH, a0, w4.W4_OUT_BF16)
    ids1 = torch.full((T, k), -1, dtype=torch.int32, device=dev)
    wts1 = torch.full((T, k), float("nan"), dtype=torch.float32, device=dev)
    a1 = torch.full((R, I), float("nan"), dtype=torch.bfloat16, device=dev)
    w4.w4a16_moe_gmm_logits(xd, lg, k, d, 2 * I, w1q, w1s_d, w4.W4_EPI_GEGLU_TANH, a1, ids1, wts1)
    torch.cuda.synchronize()
    assert np.array_equal(ids1.cpu().numpy(), ids0.cpu().numpy())
    assert np.array_equal(ids1.cpu().numpy(), oracle.moe.route(logits, k)["ids"])
    assert np.allclose(wts1.cpu().numpy(), wts0.cpu().numpy(), rtol=1e-6, atol=0)
    assert np.array_equal(bits_host(a1), bits_host(a0))
