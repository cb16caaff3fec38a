"""Mixture-of-experts layer over W4A16 experts -- oracle side (test infra only).

The model family has 128 experts per layer with 8 active per token and keeps
every expert resident ([RQ] "The gap at 26B"; [WQ] "Gemma 4 puts numbers on
the tip").  The experts' weights are int4 with one scale per 32-wide group and
are multiplied by a grouped matmul that dequantizes each weight tile on chip,
while activations stay bf16 ([RQ] "What changed in vLLM's TPU backend").

The pages do not spell out the router or the expert MLP.  Readings taken:
  * router: softmax over all experts in fp64, top-k by logit value (ties go to
    the lower expert id), the weights are the softmax probabilities at those
    ids, not renormalised.
  * expert MLP: a fused gate/up projection [d -> 2I] (rows [0, I) gate,
    [I, 2I) up), a gated activation act(gate) * up, then the down projection
    [I -> d].  The default activation is GELU with the tanh approximation
    (the Gemma family's gated GELU); SiLU is the alternative.
  * bf16 rounding happens exactly at the activation tensors: the input x, the
    gate/up output h, the gated activation a and the layer output y.  The down
    projection's per-row output o is kept unrounded, and y[t] sums
    w[t, j] * o[row(t, j)] over the slots j = 0..k-1 in that order, in fp64.
  * the routing plan groups the T*k routed rows by expert; within an expert
    the rows keep their original order r = t*k + j (a stable sort).
"""

import math

import numpy as np

from .bf16 import bf16_bits_to_f64, bf16_from_f64
from .q4 import dequant_f32


def gelu_tanh(x):
    """GELU, tanh approximation, in fp64:
    0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    x = np.asarray(x, dtype=np.float64)
    c = math.sqrt(2.0 / math.pi)
    return 0.5 * x * (1.0 + np.tanh(c * (x + 0.044715 * x * x * x)))


def silu(x):
    """SiLU in fp64: x / (1 + exp(-x))."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


ACTIVATIONS = {"gelu_tanh": gelu_tanh, "silu": silu}


def route(logits, k):
    """Top-k routing plan.  logits float32 [T, E] (finite).

    Returns dict with
      ids      int32 [T, k]   expert ids, by descending logit, ties -> lower id
      weights  f64   [T, k]   softmax(logits)[t, ids]
      counts   int64 [E]
      offsets  int32 [E + 1]  exclusive prefix sum of counts
      perm     int32 [T*k]    sorted position -> routed row r = t*k + j
      inv      int32 [T*k]    routed row r -> sorted position
      tokens   int32 [T*k]    sorted position -> token t
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    order = np.argsort(-logits, axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    z = logits.astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    weights = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    flat = ids.reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size, dtype=np.int32)
    return {
        "ids": ids, "weights": weights, "counts": counts, "offsets": offsets,
        "perm": perm, "inv": inv, "tokens": (perm // k).astype(np.int32),
    }


def combine(o, inv, weights):
    """The weighted combine back into token order: y64[t] = sum over slots j of
    weights[t, j] * o[inv[t*k + j]], in fp64.

    o        float64 [R, d]   expert outputs, indexed by sorted position
    inv      int    [T*k]     sorted position of routed row t*k + j
    weights  float  [T, k]    the top-k softmax weights
    """
    T, k = weights.shape
    inv = np.asarray(inv).reshape(T, k)
    w = np.asarray(weights, dtype=np.float64)
    y64 = np.zeros((T, o.shape[1]), dtype=np.float64)
    for j in range(k):
        y64 = y64 + w[:, j:j + 1] * o[inv[:, j]]
    return y64


def moe_layer(x_bits, logits, w1_codes, w1_scale, w2_codes, w2_scale, k=8,
              activation="gelu_tanh", keep=False):
    """One MoE layer.

    x_bits   uint16 [T, d]          bf16 activations
    logits   float32 [T, E]         router logits
    w1_codes int8  [E, 2I, d]       fused gate/up codes; w1_scale uint16 [E, 2I, d/32]
    w2_codes int8  [E, d, I]        down codes;          w2_scale uint16 [E, d, I/32]

    Returns dict with y (uint16 [T, d]) and y64 (the unrounded fp64 sum), the
    routing plan, and with keep=True the per-sorted-row h (uint16 [R, 2I]),
    a (uint16 [R, I]) and o (float64 [R, d]).
    """
    act = ACTIVATIONS[activation]
    x = bf16_bits_to_f64(x_bits)
    T, d = x.shape
    E, twoI, _ = w1_codes.shape
    I = twoI // 2
    plan = route(logits, k)
    R = T * k
    o = np.zeros((R, d), dtype=np.float64)       # indexed by sorted position
    h_all = np.zeros((R, twoI), dtype=np.uint16) if keep else None
    a_all = np.zeros((R, I), dtype=np.uint16) if keep else None
    offs = plan["offsets"]
    for e in range(E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if lo == hi:
            continue
        xs = x[plan["tokens"][lo:hi]]
        w1 = dequant_f32(w1_codes[e], w1_scale[e]).astype(np.float64)
        h_bits = bf16_from_f64(xs @ w1.T)
        h = bf16_bits_to_f64(h_bits)
        a_bits = bf16_from_f64(act(h[:, :I]) * h[:, I:])
        a = bf16_bits_to_f64(a_bits)
        w2 = dequant_f32(w2_codes[e], w2_scale[e]).astype(np.float64)
        o[lo:hi] = a @ w2.T
        if keep:
            h_all[lo:hi] = h_bits
            a_all[lo:hi] = a_bits
    y64 = combine(o, plan["inv"], plan["weights"])
    out = {"y": bf16_from_f64(y64), "y64": y64, "plan": plan}
    if keep:
        out.update(h=h_all, a=a_all, o=o)
    return out
