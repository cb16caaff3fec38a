"""W4A16 dense linear layer -- oracle side (test infrastructure only).

W4A16 means 4-bit weights and 16-bit activations ([WQ] "What you choose to
shrink"); the weights are dequantized on the fly and the activations stay in
bf16 ([RQ] "What changed in vLLM's TPU backend"; [VG] "2. What you can
quantize").

Definition used: y = x . W^T with W[n, k] = s[n, k//32] * q[n, k], computed
in fp64 from the exact bf16 / dequantized values, then rounded once to bf16.
Every product is exact in fp64; the fp64 summation error (about K * 2^-53
relative) is far below half a bf16 ulp, so the rounded result is the exactly
rounded one except in cases of measure ~0 (the exact-rational pins check it).
"""

import numpy as np

from .bf16 import bf16_bits_to_f64, bf16_from_f64
from .q4 import dequant_f32


def linear_f64(x_bits, codes, scale_bits):
    """Unrounded fp64 product x . W^T.  x_bits uint16 [M, K]; codes int8
    [N, K]; scale_bits uint16 [N, K/32].  Returns float64 [M, N]."""
    x = bf16_bits_to_f64(x_bits)
    w = dequant_f32(codes, scale_bits).astype(np.float64)
    return x @ w.T


def linear(x_bits, codes, scale_bits):
    """bf16 output y = bf16(x . W^T); returns uint16 [M, N]."""
    return bf16_from_f64(linear_f64(x_bits, codes, scale_bits))
