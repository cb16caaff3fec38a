"""bfloat16 codec of the oracle (test infrastructure only).

bf16 is the storage type of activations and of the per-group scales on the
W4A16 path ([RQ] "A repack, not a re-quantization": the scale is kept at
bf16, the precision the W4A16 layers load; [RQ] "What changed in vLLM's TPU
backend": activations stay in bf16).  The pages fix no rounding rule; the
oracle rounds to nearest, ties to even (IEEE default), in ONE step from the
exact value.

Rounding is written from the definition: for a finite x != 0 with
2^e <= |x| < 2^(e+1), the bf16 neighbours are spaced 2^(e-7) apart (7 stored
fraction bits), or 2^-133 below the smallest normal exponent -126.  Dividing
by that power of two is exact in fp64, ``np.rint`` rounds half to even, and
multiplying back is exact.  The result has at most 8 significant bits, so it
converts to fp32 exactly and its fp32 bit pattern ends in 16 zero bits.
"""

import numpy as np

BF16_QNAN = np.uint16(0x7FC0)


def bf16_bits_to_f32(bits):
    """uint16 bf16 patterns -> float32 (exact: bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits):
    """uint16 bf16 patterns -> float64 (exact)."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def bf16_from_f64(x):
    """Round float64 values to bf16 (nearest, ties to even) -> uint16 bits.

    NaN maps to the quiet NaN 0x7FC0; values whose rounded magnitude reaches
    2^128 become +-inf; signed zeros keep their sign; subnormal bf16 results
    are kept (no flush to zero).
    """
    x = np.asarray(x, dtype=np.float64)
    shape = x.shape
    x = x.ravel()
    out = np.empty(x.shape, dtype=np.uint16)
    nan = np.isnan(x)
    mag = np.abs(x)
    finite_nonzero = np.isfinite(x) & (mag > 0)

    # exponent e with 2^e <= |x| < 2^(e+1): frexp gives |x| = f * 2^E, f in [0.5, 1)
    _, E = np.frexp(np.where(finite_nonzero, mag, 1.0))
    e = E.astype(np.int64) - 1
    q_exp = np.maximum(e, -126) - 7          # spacing of bf16 values near |x|
    steps = np.rint(np.ldexp(mag, -q_exp))  # exact scaling, then round half-even
    rounded = np.ldexp(steps, q_exp)        # exact
    rounded = np.where(finite_nonzero, rounded, mag)
    rounded = np.where(rounded >= 2.0 ** 128, np.inf, rounded)
    signed = np.copysign(rounded, x)
    with np.errstate(over="ignore"):
        f32 = signed.astype(np.float32)     # exact for every value produced above
    out[:] = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out[nan] = BF16_QNAN
    return out.reshape(shape)


def bf16_from_f32(x):
    """Round float32 values to bf16 (nearest, ties to even) -> uint16 bits.

    float32 -> float64 is exact, so this is the same single rounding.
    """
    with np.errstate(invalid="ignore"):       # signalling NaNs quieten on the cast
        x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    return bf16_from_f64(x64)
