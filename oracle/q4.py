"""Q4_0 group-32 number format and the repack (scale recovery) -- oracle side.

Test infrastructure only; see the package docstring for the page keys.

The format ([RQ] "A repack, not a re-quantization"; [QP] "The Real Problem"):
weights are cut into groups of 32 consecutive values along the input
dimension K; each group has one scale s and 32 integer levels q in -8..7; the
weight value is s * q.

The repack ([RQ] "A repack, not a re-quantization"; [QP] "Building the
Missing Piece", steps 2-3) starts from bf16 weights that already lie on such a
grid and recovers, per group, the step: with a = max|w|, try s_m = a/m for
m = 1, 2, ..., 8, keep the first m whose grid reproduces every value of the
group, then refine the scale by least squares over the 32 values, and store
it at bf16.

Readings taken where the pages leave a step open (each is listed in the
design notes):
  * "reproduces the whole group" is read as: every quotient r_i = w_i / s_m
    lies within ACCEPT_TOL = 3/32 of the integer it rounds to.  The source is
    bf16, so exact equality would reject groups that are on the grid up to
    bf16 rounding; a wrong m leaves some quotient at least 1/8 away from an
    integer, a right one at most ~0.055.
  * s_m and r_i are fp32 with correctly rounded division; rounding is to
    nearest, ties to even; codes are clamped to -8..7 (the grid's range).
  * no accepted m  ->  status 0 (off the grid), codes from m = 8 (the
    textbook max/8 rule the page contrasts with), scale still refined.
  * all-zero group -> codes 0, scale +0, status 1.
  * any non-finite value -> codes 0, scale = bf16 quiet NaN, status 0xFF.
  * least squares with the codes held fixed: s = sum(w q) / sum(q^2), both
    sums in fp64 in pairwise order (first half + second half, repeatedly),
    then one round-to-nearest-even to bf16.
"""

import numpy as np

from .bf16 import bf16_bits_to_f32, bf16_from_f64, BF16_QNAN

GROUP = 32
QMIN, QMAX = -8, 7
ACCEPT_TOL = np.float32(3.0 / 32.0)
STATUS_OFF_GRID = np.uint8(0)
STATUS_NONFINITE = np.uint8(0xFF)


def _pairwise_sum(v):
    """Sum along the last axis (length a power of two) by repeated halving:
    v[..., :h] + v[..., h:], then again on the result, down to one value."""
    while v.shape[-1] > 1:
        h = v.shape[-1] // 2
        v = v[..., :h] + v[..., h:]
    return v[..., 0]


def textbook_quantize(w, m, per_tensor=False, clamp_min=None):
    """Symmetric rounding of w onto the grid of step a/m, a = max|w|.

    ``m = 8`` per group is the textbook Q4_0 rule the repack page warns about
    ([RQ] "A repack, not a re-quantization").  ``m = 7`` over the whole tensor
    with ``clamp_min=1e-8`` is the teaching sketch ([WQ] "How you actually do
    it": q_max = 2^(bits-1) - 1 = 7, round, clamp to [-q_max-1, q_max]).

    w: float32 array [..., 32] (per group) or any shape (per tensor).
    Returns (codes int8, step float32).
    """
    w = np.asarray(w, dtype=np.float32)
    if per_tensor:
        a = np.float32(np.max(np.abs(w)))
    else:
        a = np.max(np.abs(w), axis=-1, keepdims=True)
    if clamp_min is not None:
        a = np.maximum(a, np.float32(clamp_min))
    s = (a / np.float32(m)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (w / s).astype(np.float32)
    q = np.clip(np.rint(r), QMIN, QMAX)
    return q.astype(np.int8), s


def repack_groups(w_bits):
    """Repack bf16 groups.  w_bits: uint16 [G, 32] bf16 patterns.

    Returns dict with
      codes   int8   [G, 32]  levels in -8..7
      scale   uint16 [G]      bf16 pattern of the refined scale
      status  uint8  [G]      accepted m (1..8), 0 off-grid, 0xFF non-finite
      off_grid, nonfinite     int counts
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    assert w_bits.ndim == 2 and w_bits.shape[1] == GROUP
    G = w_bits.shape[0]
    w = bf16_bits_to_f32(w_bits)                     # exact fp32 values

    nonfinite = ~np.all(np.isfinite(w), axis=1)
    wf = np.where(nonfinite[:, None], np.float32(0), w)
    a = np.max(np.abs(wf), axis=1)                   # fp32
    zero = a == 0

    codes = np.zeros((G, GROUP), dtype=np.float32)
    status = np.zeros(G, dtype=np.uint8)
    decided = nonfinite | zero
    codes_m8 = None
    for m in range(1, 9):
        s_m = (a / np.float32(m)).astype(np.float32)
        s_safe = np.where(decided, np.float32(1), s_m)
        r = (wf / s_safe[:, None]).astype(np.float32)
        q = np.clip(np.rint(r), QMIN, QMAX).astype(np.float32)
        ok = np.all(np.abs(r - q) <= ACCEPT_TOL, axis=1)
        take = ok & ~decided
        codes[take] = q[take]
        status[take] = m
        decided |= take
        if m == 8:
            codes_m8 = q
    off = ~decided                                   # no m reproduced the group
    codes[off] = codes_m8[off]
    status[off] = STATUS_OFF_GRID

    # least-squares refinement with the codes fixed, fp64, pairwise order
    w64 = wf.astype(np.float64)
    q64 = codes.astype(np.float64)
    num = _pairwise_sum(w64 * q64)
    den = _pairwise_sum(q64 * q64)
    with np.errstate(divide="ignore", invalid="ignore"):
        s_ls = np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)
    scale = bf16_from_f64(s_ls)

    # special groups
    status[zero & ~nonfinite] = 1
    scale[zero & ~nonfinite] = np.uint16(0)
    codes[nonfinite] = 0
    status[nonfinite] = STATUS_NONFINITE
    scale[nonfinite] = BF16_QNAN

    return {
        "codes": codes.astype(np.int8),
        "scale": scale,
        "status": status,
        "off_grid": int(np.count_nonzero(status == STATUS_OFF_GRID)),
        "nonfinite": int(np.count_nonzero(nonfinite)),
    }


def repack_matrix(w_bits, chunk_groups=1 << 20):
    """Repack a bf16 matrix [rows, K] (K % 32 == 0) group by group.

    Returns codes int8 [rows, K], scale uint16 [rows, K/32],
    status uint8 [rows, K/32], and the two counts.
    """
    w_bits = np.asarray(w_bits, dtype=np.uint16)
    rows, K = w_bits.shape
    assert K % GROUP == 0
    flat = w_bits.reshape(-1, GROUP)
    codes = np.empty(flat.shape, dtype=np.int8)
    scale = np.empty(flat.shape[0], dtype=np.uint16)
    status = np.empty(flat.shape[0], dtype=np.uint8)
    off = nonf = 0
    for lo in range(0, flat.shape[0], chunk_groups):
        r = repack_groups(flat[lo:lo + chunk_groups])
        codes[lo:lo + chunk_groups] = r["codes"]
        scale[lo:lo + chunk_groups] = r["scale"]
        status[lo:lo + chunk_groups] = r["status"]
        off += r["off_grid"]
        nonf += r["nonfinite"]
    G = K // GROUP
    return {
        "codes": codes.reshape(rows, K),
        "scale": scale.reshape(rows, G),
        "status": status.reshape(rows, G),
        "off_grid": off,
        "nonfinite": nonf,
    }


def dequant_f32(codes, scale_bits):
    """fp32 weight values s * q per group ([WQ] "How you actually do it":
    dequantize = code times scale).  codes int8 [rows, K], scale_bits uint16
    [rows, K/32].  The product of an 8-bit and a 4-bit significand is exact
    in fp32, so this is the exact value."""
    codes = np.asarray(codes, dtype=np.int8)
    rows, K = codes.shape
    s = bf16_bits_to_f32(scale_bits).reshape(rows, K // GROUP, 1)
    q = codes.astype(np.float32).reshape(rows, K // GROUP, GROUP)
    return (s * q).reshape(rows, K).astype(np.float32)
