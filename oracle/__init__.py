"""CPU oracle for the W4A16 / Q4_0 group-32 path -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference that the GPU
library is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``int4_group_quantized_q4_amd``) never imports it and shares no code with it.

Everything here is Python + NumPy on host cores, in fp64 where the pages leave
the precision open.  Each function cites the passage it follows.  Pages cited
throughout (key -> page title, with the section named at each use):

  [RQ]  "Repacked QAT Gemma 4 26B-A4B serves on one TPU v6e at 1.9x FP8
        throughput"  (news write-up of the repack build)
  [QP]  "The Quantization Problem I Didn't Know I Had Until I Tried Running
        LLMs Locally"  (blog commentary on the same build)
  [WQ]  "What quantization really is"  (tutorial: the ruler, the teaching
        sketch, the worked example)
  [VG]  "Compression Without Regret: Quantization, QAT, and Shipping Smaller
        Models"  (vLLM field guide, part 5)

Parity status of each function (which pins it, see tests/test_oracle_*.py):
  bf16_from_f64 / bf16_from_f32   pinned (torch CPU conversion; exact rationals)
  repack_groups                   pinned (closed form on exact on-grid groups,
                                  worked example, textbook-failure cases,
                                  brute-force least squares on fallbacks)
  textbook_quantize               pinned (worked example, outlier illustration)
  dequant_f32                     pinned (exact rationals)
  linear                          pinned (exact-rational brute force; unit-scale
                                  case vs torch float64 matmul)
  route                           pinned (brute-force top-k by sorting; softmax
                                  vs torch float64; count/offset invariants)
  moe_layer                       pinned (E=1 reduces to a dense gated MLP
                                  built from torch float64 ops; token-order
                                  invariance)
  gelu_tanh                       pinned (torch.nn.functional.gelu tanh, fp64)
  combine (moe.py)                pinned (one-hot expert rows with distinct
                                  weights: every slot/weight/token pairing is
                                  visible; slot order of the fp64 sum)
  normwise_errors / within_tolerance
                                  pinned (hand-computed exact vectors that
                                  separate the normwise figures from element-wise
                                  or max|y|-based ones; zero and scaled references)
  fp8.e4m3_decode / e4m3_encode   pinned (torch float8_e4m3fn on every code and
                                  on random values; brute-force nearest value;
                                  midpoints to the even code; saturation)
  fp8.quantize_rows               pinned (amax lands on +-448; zero rows; codes
                                  equal torch's conversion of the fp32 quotients)
  fp8.linear                      pinned (exact integer matmul; row/column scales)
  fp8.moe_layer                   pinned (E=1, k=1 equals the dense FP8 MLP
                                  composed from torch fp8 conversion and float64
                                  ops)

The FP8 (W8A8) leg in fp8.py is the comparison path the pages set against
W4A16 ([RQ] "What happened"; [VG] "2. What you can quantize").
"""

from .bf16 import (
    bf16_bits_to_f32,
    bf16_bits_to_f64,
    bf16_from_f32,
    bf16_from_f64,
)
from .q4 import (
    GROUP,
    ACCEPT_TOL,
    STATUS_OFF_GRID,
    STATUS_NONFINITE,
    repack_groups,
    repack_matrix,
    textbook_quantize,
    dequant_f32,
)
from .linear import linear, linear_f64
from .moe import gelu_tanh, route, moe_layer
from .metrics import normwise_errors, within_tolerance, MAX_REL_TOL, RMS_REL_TOL

__all__ = [
    "bf16_bits_to_f32", "bf16_bits_to_f64", "bf16_from_f32", "bf16_from_f64",
    "GROUP", "ACCEPT_TOL", "STATUS_OFF_GRID", "STATUS_NONFINITE",
    "repack_groups", "repack_matrix", "textbook_quantize", "dequant_f32",
    "linear", "linear_f64", "gelu_tanh", "route", "moe_layer",
    "normwise_errors", "within_tolerance", "MAX_REL_TOL", "RMS_REL_TOL",
]
