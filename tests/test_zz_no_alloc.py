"""w4a16_moe_layer_noalloc (the layer with the library's static device scratch
in place of a workspace) against w4a16_moe_layer on the same inputs: two calls
in a row, the second with fewer tokens, each within the output tolerance of
the workspace call (the array keeps the first call's contents when the second
runs)."""

import numpy as np
import pytest
import torch

import gen
import int4_group_quantized_q4_amd as w4
import oracle
from gpu_util import bits_host, say

pytestmark = pytest.mark.gpu


def test_noalloc_layer_matches_workspace_layer_twice():
    dev = torch.device("cuda:0")
    g = gen.torch_generator(dev, 4321)
    E, k, d, I = 128, 8, 2816, 704
    w1q = gen.bytes_uniform_t(g, E * 2 * I * d // 2, dev)
    w1s = gen.scales_loguniform_t(g, (E, 2 * I, d // 32), dev)
    w2q = gen.bytes_uniform_t(g, E * d * I // 2, dev)
    w2s = gen.scales_loguniform_t(g, (E, d, I // 32), dev)
    for T in (256, 24):
        say("[noalloc] T=%d" % T)
        x = gen.bf16_normal_t(g, (T, d), dev)
        logits = gen.router_logits_t(g, T, E, dev)
        y_ws, _ = w4.moe_layer(x, logits, k, I, w1q, w1s, w2q, w2s)
        y_na = torch.empty(T, d, dtype=torch.bfloat16, device=dev)
        w4.w4a16_moe_layer_noalloc(x, logits, k, I, w1q, w1s, w2q, w2s, w4.W4_EPI_GEGLU_TANH, y_na)
        torch.cuda.synchronize()
        a = oracle.bf16_bits_to_f64(bits_host(y_na))
        b = oracle.bf16_bits_to_f64(bits_host(y_ws))
        ok, mx, rms = oracle.within_tolerance(a, b)
        say("  max_rel %.2e rms_rel %.2e, bit-identical %.4f" % (mx, rms, np.mean(a == b)))
        assert ok and np.all(np.isfinite(a))


def test_noalloc_rejects_a_layer_larger_than_its_scratch():
    with pytest.raises(w4.W4Error) as ei:
        dev = torch.device("cuda:0")
        T, E, k, d, I = 4096, 128, 8, 2816, 704
        x = torch.zeros(T, d, dtype=torch.bfloat16, device=dev)
        logits = torch.zeros(T, E, dtype=torch.float32, device=dev)
        w1q = torch.zeros(E * 2 * I * d // 2, dtype=torch.uint8, device=dev)
        w1s = torch.zeros(E * 2 * I * d // 32, dtype=torch.bfloat16, device=dev)
        w2q = torch.zeros(E * d * I // 2, dtype=torch.uint8, device=dev)
        w2s = torch.zeros(E * d * I // 32, dtype=torch.bfloat16, device=dev)
        y = torch.zeros(T, d, dtype=torch.bfloat16, device=dev)
        w4.w4a16_moe_layer_noalloc(x, logits, k, I, w1q, w1s, w2q, w2s, w4.W4_EPI_GEGLU_TANH, y)
    assert ei.value.status == w4.W4_ERR_WORKSPACE
