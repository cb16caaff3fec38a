"""FP8 (W8A8) comparison path -- oracle side (test infrastructure only).

The pages set the W4A16 build against an FP8 build of the same model on the
same chip ([RQ] "What happened": the FP8 checkpoint serves fewer output
tokens per second and holds far less KV cache).  They class FP8 as a
weights-and-activations format whose matmuls run natively in low precision,
the common first rung on hardware that supports it, provided the scaling is
done properly ([VG] "2. What you can quantize", "3. The precision ladder").
They fix neither the 8-bit encoding nor the scale granularity.  Readings
taken (the plainest ones the rest supports):

  * encoding: OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent bits (bias 7),
    3 fraction bits; exponent field 0 is subnormal (value m/8 * 2^-6), the
    all-ones pattern S.1111.111 is NaN and there is no infinity, so the
    largest finite magnitude is 1.75 * 2^8 = 448.  This is the FP8 format the
    gfx950 matrix cores take natively.
  * weights: an E4M3 code per weight and one fp32 scale per output channel
    (per row of W[N, K]); w = scale[n] * decode(code).
  * activations: quantized per row at run time: amax = max |x| over the row,
    s = fl32(amax / 448) (zero row: s = 1), code = E4M3(clamp(fl32(x / s),
    -448, 448)) rounded to nearest, ties to even.  The divisions are single
    IEEE fp32 operations, so a GPU kernel taking them in fp32 reaches the same
    codes bit for bit.
  * the matmul: y[r, n] = s_x[r] * s_w[n] * sum_k decode(xq[r, k]) *
    decode(wq[n, k]), formed here exactly in fp64.
  * the MoE layer: the routing, gated activation, bf16 rounding points and
    combine of oracle.moe.moe_layer, with the fp8 matmul in place of the W4A16
    one: x is quantized once per token, the gated activation a once per
    routed row.

The E4M3 codec is written from its definition, not from any library; its
pins are in tests/test_oracle_fp8.py (every code's value from the bit
fields, round trips, midpoints, brute-force nearest value, saturation).
"""

import numpy as np

from .bf16 import bf16_bits_to_f32, bf16_bits_to_f64, bf16_from_f64
from .moe import ACTIVATIONS, combine, route

E4M3_MAX = 448.0
E4M3_NAN_CODES = (0x7F, 0xFF)


def _decode_table():
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            t[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


E4M3_VALUES = _decode_table()


def e4m3_decode(codes):
    """uint8 E4M3 codes -> float64 values (NaN for the two NaN codes)."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x):
    """Round finite float values with |x| <= 448 to E4M3 (nearest, ties to
    even) -> uint8 codes.  -0.0 and values that round to zero keep their sign
    bit.  Larger magnitudes saturate to +-448 (the callers clamp first).

    Normal range (|x| >= 2^-6): with 2^e <= |x| < 2^(e+1) the neighbours are
    2^(e-3) apart; subnormal range: 2^-9 apart.  Dividing by that power of
    two is exact in fp64 and np.rint rounds half to even, which on the
    integer step count is ties-to-even on the code's last fraction bit.
    """
    x = np.asarray(x, dtype=np.float64)
    shape = x.shape
    x = x.ravel()
    if np.any(~np.isfinite(x)):
        raise ValueError("e4m3_encode takes finite values")
    sign = np.signbit(x)
    mag = np.minimum(np.abs(x), E4M3_MAX)
    _, E = np.frexp(np.where(mag > 0, mag, 1.0))
    e = np.maximum(E.astype(np.int64) - 1, -6)        # subnormals share 2^-6's spacing
    step = e - 3
    n = np.rint(np.ldexp(mag, -step)).astype(np.int64)  # steps of 2^step
    n = np.where(mag > 0, n, 0)
    # n in [8, 16] for a normal e (16: carried into the next binade);
    # n in [0, 8] for the subnormal range (8: the smallest normal)
    val = np.ldexp(n.astype(np.float64), step)
    val = np.minimum(val, E4M3_MAX)
    # re-derive the fields from the rounded value (exact)
    _, E2 = np.frexp(np.where(val > 0, val, 1.0))
    e2 = E2.astype(np.int64) - 1
    normal = val >= 2.0 ** -6
    field_e = np.where(normal, e2 + 7, 0)
    frac = np.where(normal, np.ldexp(val, -e2) - 1.0, np.ldexp(val, 6))   # [0,1) or [0,1)
    field_m = np.rint(frac * 8.0).astype(np.int64)
    code = (field_e << 3) | field_m
    code = np.where(sign, code | 0x80, code)
    return code.astype(np.uint8).reshape(shape)


def quantize_rows(x_bits):
    """Per-row dynamic E4M3 quantization of bf16 rows.

    x_bits uint16 [rows, K].  Returns (codes uint8 [rows, K], scale float32
    [rows]) with scale = fl32(amax / 448) (1.0 for an all-zero row) and codes
    = E4M3(clamp(fl32(x / scale), -448, 448)).
    """
    x = bf16_bits_to_f32(np.asarray(x_bits, dtype=np.uint16))
    amax = np.max(np.abs(x), axis=1)                               # exact in fp32
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    r = (x / scale[:, None]).astype(np.float32)                    # IEEE fp32 division
    r = np.clip(r, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3_encode(r), scale


def linear(xq, x_scale, wq, w_scale):
    """y[r, n] = x_scale[r] * w_scale[n] * sum_k decode(xq[r,k]) decode(wq[n,k]),
    in fp64.  Every product of two E4M3 values is a multiple of 2^-18 below
    2^17.6 in magnitude, so the sum over K < 2^17 terms is exact in fp64 in
    any order; the two scale multiplications round once each."""
    a = e4m3_decode(xq)
    b = e4m3_decode(wq)
    acc = a @ b.T
    return (np.asarray(x_scale, dtype=np.float64)[:, None] * np.asarray(w_scale, dtype=np.float64)[None, :]) * acc


def moe_layer(x_bits, logits, w1q, w1_scale, w2q, w2_scale, k=8, activation="gelu_tanh", keep=False):
    """One MoE layer over FP8 experts.

    x_bits   uint16 [T, d]       bf16 activations
    logits   float32 [T, E]
    w1q      uint8 [E, 2I, d]    fused gate/up E4M3 codes; w1_scale float32 [E, 2I]
    w2q      uint8 [E, d, I]     down E4M3 codes;          w2_scale float32 [E, d]

    Returns dict with y (uint16 [T, d]), y64, the routing plan, and with
    keep=True the sorted-row h (uint16 [R, 2I]), a (uint16 [R, I]), the
    quantized a (codes, scales) and o (float64 [R, d]).
    """
    act = ACTIVATIONS[activation]
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, d = x_bits.shape
    E, twoI, _ = w1q.shape
    I = twoI // 2
    plan = route(logits, k)
    R = T * k
    xq, xs = quantize_rows(x_bits)
    o = np.zeros((R, d), dtype=np.float64)
    h_all = np.zeros((R, twoI), dtype=np.uint16)
    a_all = np.zeros((R, I), dtype=np.uint16)
    offs = plan["offsets"]
    for e in range(E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if lo == hi:
            continue
        toks = plan["tokens"][lo:hi]
        h_bits = bf16_from_f64(linear(xq[toks], xs[toks], w1q[e], w1_scale[e]))
        h = bf16_bits_to_f64(h_bits)
        a_bits = bf16_from_f64(act(h[:, :I]) * h[:, I:])
        h_all[lo:hi] = h_bits
        a_all[lo:hi] = a_bits
    aq, a_scale = quantize_rows(a_all)
    for e in range(E):
        lo, hi = int(offs[e]), int(offs[e + 1])
        if lo == hi:
            continue
        o[lo:hi] = linear(aq[lo:hi], a_scale[lo:hi], w2q[e], w2_scale[e])
    y64 = combine(o, plan["inv"], plan["weights"])
    out = {"y": bf16_from_f64(y64), "y64": y64, "plan": plan}
    if keep:
        out.update(h=h_all, a=a_all, aq=aq, a_scale=a_scale, o=o, xq=xq, x_scale=xs)
    return out
