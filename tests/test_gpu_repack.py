"""GPU parity of q4_group_repack, q4_pack_codes and q4_group_dequant_f32
against the oracle: bit-exact codes, scales, status, counters and fp32
dequantized weights."""

import json
import os

import numpy as np
import pytest
import torch

import gen
import int4_group_quantized_q4_amd as w4
import layout
import oracle
from gpu_util import bf16_dev, bits_host, f32_bits_equal, say, to_dev

pytestmark = pytest.mark.gpu


def run_and_check(w_bits, label):
    rows, K = w_bits.shape
    say("[repack] %s rows=%d K=%d" % (label, rows, K))
    w = bf16_dev(w_bits)
    q, s, st, cnt = w4.repack(w)
    deq = w4.dequant(q, s, rows, K)
    torch.cuda.synchronize()
    ref = oracle.repack_matrix(w_bits)
    codes = layout.decode(q.cpu().numpy(), rows, K)
    assert np.array_equal(codes, ref["codes"]), label
    assert np.array_equal(layout.decode_scales(bits_host(s), rows, K), ref["scale"]), label
    assert np.array_equal(st.cpu().numpy(), ref["status"]), label
    c = cnt.cpu().numpy()
    assert int(c[0]) == ref["off_grid"] and int(c[1]) == ref["nonfinite"], label
    assert f32_bits_equal(deq.cpu().numpy(), oracle.dequant_f32(ref["codes"], ref["scale"])), label
    return ref, q


def test_repack_dense_tiny_source():
    cfg = gen.DENSE_TINY
    src = gen.ongrid_source(gen.rng_for(cfg["id"], 10), cfg["N"], cfg["K"], *cfg["peak"])
    ref, _ = run_and_check(src["w_bits"], "dense-tiny on-grid")
    assert ref["off_grid"] == 0
    # closed form: dequant reproduces the source
    assert np.array_equal(oracle.dequant_f32(ref["codes"], ref["scale"]), oracle.bf16_bits_to_f32(src["w_bits"]))


@pytest.mark.parametrize("rows,K", [(16, 32), (32, 96), (48, 704), (16, 4096), (64, 160)])
def test_repack_ragged_groups(rows, K):
    src = gen.ongrid_source(gen.rng_for(910, rows + K), rows, K, 1, 8)
    run_and_check(src["w_bits"], "ragged")


def test_repack_special_and_offgrid_groups():
    rng = gen.rng_for(910, 1)
    rows, K = 32, 256
    w = gen.bf16_normal(rng, (rows, K))                         # off the grid
    src = gen.ongrid_source(rng, rows, K, 1, 8)
    w[::2] = src["w_bits"][::2]                                  # half the rows on the grid
    w[1, 0:32] = 0                                               # all-zero group
    w[3, 32:64] = 0x8000                                         # all -0.0
    w[5, 40] = 0x7FC0                                            # NaN
    w[7, 64] = 0x7F80                                            # +inf
    w[9, 100] = 0xFF80                                           # -inf
    q0 = np.array([(i % 15) - 7 for i in range(32)], dtype=np.int64)
    q0[3] = -8
    # subnormal grid with step 2^-133: the bf16 pattern of q * 2^-133 is sign | |q|
    w[11, 128:160] = np.array([0x8000 | -int(v) if v < 0 else int(v) for v in q0], dtype=np.uint16)
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "textbook_failure_groups.json")))
    s0 = np.float32(oracle.bf16_bits_to_f32(np.array([int(fx["scale_bits_hex"], 16)], dtype=np.uint16))[0])
    for gi, g in enumerate(fx["groups"]):
        w[13 + 2 * gi, 0:32] = oracle.bf16_from_f32(s0 * np.array(g["codes"], dtype=np.float32))
    ref, _ = run_and_check(w, "special")
    assert ref["nonfinite"] == 3
    assert ref["status"][11, 4] == 8
    for gi, g in enumerate(fx["groups"]):
        assert ref["status"][13 + 2 * gi, 0] == g["m_star"]


def test_repack_expert_shape_and_determinism():
    cfg = gen.MOE_E2E
    rows, K = 2 * cfg["I"], cfg["d"]
    src = gen.ongrid_source(gen.rng_for(cfg["id"], 11), rows, K, *cfg["peak"])
    ref, q = run_and_check(src["w_bits"], "expert gate/up shape")
    assert ref["off_grid"] == 0
    q2, s2, _, _ = w4.repack(bf16_dev(src["w_bits"]))
    torch.cuda.synchronize()
    assert torch.equal(q, q2)


def test_repack_realistic_variant_bit_exact():
    rng = gen.rng_for(910, 2)
    G = 16 * 64
    q0 = gen.codes_uniform(rng, (G, 32)).astype(np.float64)
    s = np.exp(rng.uniform(np.log(1e-3), np.log(1e-2), G))
    wb = oracle.bf16_from_f64(s[:, None] * q0).reshape(16 * 8, 256)
    run_and_check(wb, "realistic bf16-rounded source")


@pytest.mark.parametrize("rows,K", [(16, 32), (32, 96), (48, 704), (1408, 2816)])
def test_pack_codes_and_scales_match_layout(rows, K):
    say("[pack] rows=%d K=%d" % (rows, K))
    rng = gen.rng_for(911, rows + K)
    codes = gen.codes_uniform(rng, (rows, K))
    sc = gen.scales_loguniform(rng, (rows, K // 32))
    q = w4.pack_codes(to_dev(codes))
    st = w4.pack_scales(bf16_dev(sc))
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), layout.encode(codes))
    assert np.array_equal(bits_host(st), layout.encode_scales(sc))


def test_dequant_random_weights():
    rng = gen.rng_for(911, 1)
    rows, K = 64, 704
    codes = gen.codes_uniform(rng, (rows, K))
    sc = gen.scales_loguniform(rng, (rows, K // 32))
    say("[dequant] rows=%d K=%d" % (rows, K))
    out = w4.dequant(to_dev(layout.encode(codes)), bf16_dev(layout.encode_scales(sc)), rows, K)
    torch.cuda.synchronize()
    assert f32_bits_equal(out.cpu().numpy(), oracle.dequant_f32(codes, sc))


def test_repack_decision_boundaries():
    """Groups whose quotients sit on the decision boundaries: distances to the
    nearest integer of exactly 3/32 and a bf16 step either side (groups that
    are accepted at the boundary), and exact ties of the m = 8 fallback
    (off-grid groups keep those codes); peaks whose trial steps a/m are
    inexact (a = 7, 5.5, 3 x 2^k, 1e-3-scale) and tiny and huge magnitudes
    (the division-only path).  Bit-exact against the oracle."""
    rng = np.random.default_rng(912)
    near = np.array([0.0, 3 / 32, -3 / 32, 3 / 32 - 2 ** -9, -(3 / 32 - 2 ** -9), 3 / 32 + 2 ** -9])
    far = np.array([0.0, 0.5, -0.5, 1.5, 3 / 32 + 2 ** -7, 0.125])
    groups = []
    for peak in (8.0, 7.0, 5.5, 3.0, 6.0, 7.0 * 2.0 ** -10, 1e-3 * 7, 2.0 ** -120 * 8, 2.0 ** 110 * 5):
        for m in range(1, 9):
            for deltas in (near, near, far):
                s = peak / m
                q = rng.integers(-min(m, 8), min(m, 7) + 1, 32).astype(np.float64)
                q[rng.integers(32)] = m if m < 8 else -8
                d = rng.choice(deltas, 32) * (rng.random(32) < 0.5)
                d[np.abs(q) == m] = 0.0
                groups.append((q + d) * s)
    w = oracle.bf16_from_f64(np.array(groups))
    rows = (len(groups) // 16) * 16
    w = w[:rows].reshape(rows, 32)
    say("[repack] decision boundaries: %d groups" % rows)
    ref, _ = run_and_check(w, "decision boundaries")
    say("  off-grid %d of %d" % (ref["off_grid"], rows))
