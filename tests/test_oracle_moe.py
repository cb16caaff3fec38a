"""Pins of the oracle's routing and MoE layer.

Routing is checked against a brute-force sort per token and torch's float64
softmax; the layer is checked where it reduces to something else: one expert
with weight 1 is a dense gated MLP built from torch float64 ops, and identical
experts make the combine a plain weighted sum of one MLP output."""

import numpy as np
import torch
import torch.nn.functional as F

import gen
import oracle
from exact import f64_to_bf16_bits_intmath


def _bits_to_t64(bits):
    return torch.from_numpy(oracle.bf16_bits_to_f64(bits))


def test_gelu_tanh_and_silu_match_torch():
    # absolute agreement at the ulp level of the input (the negative tail cancels
    # to ~0, where a relative comparison is meaningless)
    x = np.linspace(-12, 12, 20001)
    scale = np.maximum(np.abs(x), 1.0)
    g = oracle.gelu_tanh(x)
    ref = F.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.max(np.abs(g - ref) / scale) < 1e-15
    from oracle.moe import silu
    ref = F.silu(torch.from_numpy(x)).numpy()
    assert np.max(np.abs(silu(x) - ref) / scale) < 1e-15


def test_route_brute_force_and_invariants():
    rng = gen.rng_for(902, 1)
    T, E, k = 50, 16, 4
    logits = gen.router_logits(rng, T, E)
    logits[3, 5] = logits[3, 2]            # ties -> lower id first
    logits[7, :] = 0.25
    plan = oracle.route(logits, k)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        assert list(plan["ids"][t]) == order
    p = torch.softmax(torch.from_numpy(logits.astype(np.float64)), dim=1).numpy()
    assert np.allclose(plan["weights"], np.take_along_axis(p, plan["ids"].astype(np.int64), 1), rtol=1e-14)
    assert list(plan["ids"][7]) == [0, 1, 2, 3]
    offs = plan["offsets"]
    assert offs[0] == 0 and offs[-1] == T * k and np.all(np.diff(offs) >= 0)
    flat = plan["ids"].reshape(-1)
    assert sorted(plan["perm"].tolist()) == list(range(T * k))
    for e in range(E):
        rows = plan["perm"][offs[e]:offs[e + 1]]
        assert np.all(flat[rows] == e)
        assert np.all(np.diff(rows) > 0)                  # stable: original order kept
    assert np.array_equal(plan["perm"][plan["inv"]], np.arange(T * k))
    assert np.array_equal(plan["tokens"], plan["perm"] // k)


def test_route_zipf_imbalance():
    rng = gen.rng_for(902, 2)
    logits = gen.router_logits(rng, 4096, 128, "zipf", 1.1)
    plan = oracle.route(logits, 8)
    c = plan["counts"]
    assert c.sum() == 4096 * 8
    assert c[0] == c.max() and c[0] > 3000 and np.median(c) < 200


def _dense_mlp_torch(x_bits, w1, w2, act):
    x = _bits_to_t64(x_bits)
    h = x @ torch.from_numpy(w1).T
    h_b = f64_to_bf16_bits_intmath(h.numpy())
    h = _bits_to_t64(h_b)
    I = h.shape[1] // 2
    g = F.gelu(h[:, :I], approximate="tanh") if act == "gelu_tanh" else F.silu(h[:, :I])
    a_b = f64_to_bf16_bits_intmath((g * h[:, I:]).numpy())
    o = _bits_to_t64(a_b) @ torch.from_numpy(w2).T
    return o.numpy()


def _expert_weights(rng, E, d, I):
    w1c = gen.codes_uniform(rng, (E, 2 * I, d))
    w1s = gen.scales_loguniform(rng, (E, 2 * I, d // 32))
    w2c = gen.codes_uniform(rng, (E, d, I))
    w2s = gen.scales_loguniform(rng, (E, d, I // 32))
    return w1c, w1s, w2c, w2s


def test_single_expert_is_dense_gated_mlp():
    rng = gen.rng_for(902, 3)
    T, d, I = 24, 128, 64
    x = gen.bf16_normal(rng, (T, d))
    w1c, w1s, w2c, w2s = _expert_weights(rng, 1, d, I)
    for act in ("gelu_tanh", "silu"):
        out = oracle.moe_layer(x, np.zeros((T, 1), np.float32), w1c, w1s, w2c, w2s, k=1, activation=act)
        w1 = oracle.dequant_f32(w1c[0], w1s[0]).astype(np.float64)
        w2 = oracle.dequant_f32(w2c[0], w2s[0]).astype(np.float64)
        o = _dense_mlp_torch(x, w1, w2, act)
        assert np.array_equal(out["y"], f64_to_bf16_bits_intmath(o))


def test_identical_experts_combine_is_weighted_sum():
    rng = gen.rng_for(902, 4)
    T, d, I, E, k = 16, 64, 32, 8, 3
    x = gen.bf16_normal(rng, (T, d))
    w1c, w1s, w2c, w2s = _expert_weights(rng, 1, d, I)
    rep = lambda a: np.repeat(a, E, axis=0)
    logits = gen.router_logits(rng, T, E)
    out = oracle.moe_layer(x, logits, rep(w1c), rep(w1s), rep(w2c), rep(w2s), k=k)
    w1 = oracle.dequant_f32(w1c[0], w1s[0]).astype(np.float64)
    w2 = oracle.dequant_f32(w2c[0], w2s[0]).astype(np.float64)
    o = _dense_mlp_torch(x, w1, w2, "gelu_tanh")
    p = torch.softmax(torch.from_numpy(logits.astype(np.float64)), 1)
    wsum = torch.topk(p, k, dim=1).values.sum(1).numpy()
    ref = o * wsum[:, None]
    assert np.allclose(out["y64"], ref, rtol=1e-12, atol=1e-300)


def test_token_order_invariance():
    rng = gen.rng_for(902, 5)
    T, d, I, E, k = 32, 64, 32, 8, 2
    x = gen.bf16_normal(rng, (T, d))
    logits = gen.router_logits(rng, T, E)
    w = _expert_weights(rng, E, d, I)
    a = oracle.moe_layer(x, logits, *w, k=k)
    pi = rng.permutation(T)
    b = oracle.moe_layer(x[pi], logits[pi], *w, k=k)
    assert np.allclose(a["y64"][pi], b["y64"], rtol=1e-13, atol=1e-300)
    assert np.mean(a["y"][pi] == b["y"]) > 0.999
