"""End to end at the 30-layer MoE weight set: 30 layers of 128 experts (3,840
experts, fused gate/up 2816 -> 2x704 and down 704 -> 2816) generated exactly on
a Q4_0 grid on the device (per-group peak level 4..8, log-uniform scales),
repacked by q4_group_repack, then a batch of 256 tokens decoded through the 30
layers with top-8 routing.

Checked against what the construction and the oracle fix:
  * every group of every layer round-trips exactly (the fp32 dequantization of
    the repacked weights equals the source) and none is reported off the grid
    or non-finite -- on-grid groups must be recovered;
  * sampled source rows repacked by the oracle give the same codes and scales
    bit for bit;
  * at three layers, the routing plan of the whole batch equals the oracle's,
    and the outputs of sampled tokens match the oracle layer run on the same
    layer input (normwise tolerance)."""

import numpy as np
import pytest
import torch

import gen
import int4_group_quantized_q4_amd as w4
import layout
import oracle
from gpu_util import bits_host, say

pytestmark = pytest.mark.gpu


class LazyExperts:
    """Expert codes or scales decoded from the packed device tensors on first
    use: the oracle layer only touches the experts its tokens route to."""

    def __init__(self, packed, E, rows, K, scales):
        self.packed, self.rows, self.K, self.scales = packed, rows, K, scales
        self.shape = (E, rows, K if not scales else K // 32)
        self.cache = {}

    def __getitem__(self, e):
        if e not in self.cache:
            if self.scales:
                n = self.rows * self.K // 32
                bits = bits_host(self.packed[e * n:(e + 1) * n])
                self.cache[e] = layout.decode_scales(bits, self.rows, self.K)
            else:
                n = self.rows * self.K // 2
                self.cache[e] = layout.decode(self.packed[e * n:(e + 1) * n].cpu().numpy(), self.rows, self.K)
        return self.cache[e]


def repack_and_check(w, rows, K, counters, label, sample_rows):
    """Repack one stacked-expert source on the device; check the exact round
    trip of every group there and the oracle's repack of sample_rows."""
    q = torch.empty(rows * K // 2, dtype=torch.uint8, device=w.device)
    s = torch.empty(rows * K // 32, dtype=torch.bfloat16, device=w.device)
    w4.q4_group_repack(w, q, s, None, counters)
    deq = w4.dequant(q, s, rows, K)
    assert torch.equal(deq, w.float()), label + ": dequantized repack differs from the on-grid source"
    del deq
    if sample_rows is not None:
        # rows of one 16-row tile per sampled expert-aligned tile index
        src = w[sample_rows].view(torch.int16).cpu().numpy().view(np.uint16)
        ref = oracle.repack_matrix(src)
        assert ref["off_grid"] == 0 and ref["nonfinite"] == 0
        for n, row in enumerate(sample_rows.tolist()):
            t = row // 16
            tile_q = q[t * 8 * K:(t + 1) * 8 * K].cpu().numpy()
            tile_s = bits_host(s[t * 16 * (K // 32):(t + 1) * 16 * (K // 32)])
            assert np.array_equal(layout.decode(tile_q, 16, K)[row % 16], ref["codes"][n]), label
            assert np.array_equal(layout.decode_scales(tile_s, 16, K)[row % 16], ref["scale"][n]), label
    return q, s


def test_e2e_30_layer_repack_then_decode():
    cfg = gen.MOE_E2E
    L, T, d, I, E, k = cfg["layers"], cfg["T"], cfg["d"], cfg["I"], cfg["E"], cfg["k"]
    dev = torch.device("cuda")
    g = gen.torch_generator(dev, 5)
    check_layers = (0, L // 2, L - 1)
    counters = torch.zeros(2, dtype=torch.int64, device=dev)
    pick = np.random.default_rng(5)
    layers = []
    for l in range(L):
        say("[e2e] layer %d: generate on the grid + repack" % l)
        w1, _, _ = gen.ongrid_source_t(g, E * 2 * I, d, *cfg["peak"], dev)
        w2, _, _ = gen.ongrid_source_t(g, E * d, I, *cfg["peak"], dev)
        s1 = s2 = None
        if l in check_layers:
            s1 = torch.from_numpy(np.sort(pick.choice(E * 2 * I, 24, replace=False))).to(dev)
            s2 = torch.from_numpy(np.sort(pick.choice(E * d, 24, replace=False))).to(dev)
        w1q, w1s = repack_and_check(w1, E * 2 * I, d, counters, "layer %d gate/up" % l, s1)
        w2q, w2s = repack_and_check(w2, E * d, I, counters, "layer %d down" % l, s2)
        del w1, w2
        layers.append((w1q, w1s, w2q, w2s))
    c = counters.cpu().numpy()
    say("[e2e] off-grid %d, non-finite %d" % (c[0], c[1]))
    assert int(c[0]) == 0 and int(c[1]) == 0

    x = gen.bf16_normal_t(g, (T, d), dev)
    logits = [gen.router_logits_t(g, T, E, dev) for _ in range(L)]
    ws = torch.empty(w4.w4a16_moe_layer_workspace(T, E, k, d, I), dtype=torch.uint8, device=dev)
    saved = {}
    for l, (w1q, w1s, w2q, w2s) in enumerate(layers):
        y, views = w4.moe_layer(x, logits[l], k, I, w1q, w1s, w2q, w2s, w4.W4_EPI_GEGLU_TANH, ws)
        if l in check_layers:
            torch.cuda.synchronize()
            saved[l] = dict(x=bits_host(x), y=bits_host(y), logits=logits[l].cpu().numpy(),
                            ids=views["topk_ids"].cpu().numpy(), weights=views["topk_weights"].cpu().numpy())
        x = (x.float() + y.float()).to(torch.bfloat16)   # residual stream, outside the library
    torch.cuda.synchronize()
    assert torch.isfinite(x.float()).all()

    for l in check_layers:
        sv = saved[l]
        plan = oracle.route(sv["logits"], k)
        # (256 tokens take the streaming path: each matmul finds its expert's
        # rows in the ids, so the ids and weights are the whole plan)
        assert np.array_equal(sv["ids"], plan["ids"]), l
        assert np.allclose(sv["weights"], plan["weights"], rtol=2e-6, atol=1e-9), l
        toks = np.sort(pick.choice(T, 4, replace=False))
        w1q, w1s, w2q, w2s = layers[l]
        ref = oracle.moe_layer(sv["x"][toks], sv["logits"][toks],
                               LazyExperts(w1q, E, 2 * I, d, False), LazyExperts(w1s, E, 2 * I, d, True),
                               LazyExperts(w2q, E, d, I, False), LazyExperts(w2s, E, d, I, True), k=k)
        ok, mx, rms = oracle.within_tolerance(oracle.bf16_bits_to_f64(sv["y"][toks]),
                                              oracle.bf16_bits_to_f64(ref["y"]))
        say("[e2e] layer %d tokens %s: max_rel %.2e rms_rel %.2e" % (l, toks.tolist(), mx, rms))
        assert ok, (l, mx, rms)
