"""Seeded synthetic inputs (no method arithmetic here).

Distributions and shapes of the five workloads:

  dense-tiny     M=4, K=256, N=512, group 32; plus an on-grid bf16 repack
                 source whose per-group peak level is uniform in 1..8.
  dense-decode   M in {1, 8, 16}, K=4096, N=14336.
  dense-prefill  M=4096, K=4096, N=14336 (the same projection over a prompt).
  moe-decode     T=64 tokens, d_model=2816, 128 experts, expert hidden 704
                 (fused gate/up 2816 -> 2x704, down 704 -> 2816), top-8,
                 router logits N(0,1).
  moe-prefill    as moe-decode with T=4096 and routing drawn from a Zipf(1.1)
                 expert-popularity law.
  moe-e2e        30 layers x 128 experts of on-grid bf16 source (per-group
                 peak level uniform in 4..8), repacked, then T=256 decode
                 through all 30 layers.

Common laws: int4 codes uniform in [-8, 7]; bf16 scales log-uniform in
[1e-3, 1e-2]; activations bf16 N(0, 1); router logits fp32 N(0, 1).

Host draws use NumPy's PCG64 ``default_rng(1000 * workload_id + tensor_id)``;
device draws (only for bench-sized weight sets) use a seeded torch generator on
the device.  fp32 -> bf16 conversion of drawn values uses torch's own
conversion.
"""

import numpy as np
import torch

GROUP = 32

DENSE_TINY = dict(id=1, M=4, K=256, N=512, peak=(1, 8))
DENSE_DECODE = dict(id=2, Ms=(1, 8, 16), K=4096, N=14336)
DENSE_PREFILL = dict(id=6, M=4096, K=4096, N=14336)
MOE_DECODE = dict(id=3, T=64, d=2816, I=704, E=128, k=8, router="normal")
MOE_PREFILL = dict(id=4, T=4096, d=2816, I=704, E=128, k=8, router="zipf", zipf_s=1.1)
MOE_E2E = dict(id=5, layers=30, T=256, d=2816, I=704, E=128, k=8, router="normal", peak=(4, 8))

SCALE_LO, SCALE_HI = 1e-3, 1e-2


def rng_for(workload_id, tensor_id):
    return np.random.default_rng(1000 * workload_id + tensor_id)


def to_bf16_bits(f32):
    """fp32 array -> uint16 bf16 patterns using torch's conversion."""
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_normal(rng, shape):
    return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def _loguniform_f32(rng, shape, lo=SCALE_LO, hi=SCALE_HI):
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size=shape)).astype(np.float32)


def truncate_significand(f32, bits):
    """Keep the top ``bits`` significant bits of each fp32 value (round toward
    zero).  With bits=5 a scale times any code in -8..7 fits in bf16."""
    drop = 24 - bits
    mask = np.uint32((0xFFFFFFFF << drop) & 0xFFFFFFFF)
    return (np.asarray(f32, dtype=np.float32).view(np.uint32) & mask).view(np.float32)


def scales_loguniform(rng, shape, significant_bits=None):
    v = _loguniform_f32(rng, shape)
    if significant_bits is not None:
        v = truncate_significand(v, significant_bits)
    return to_bf16_bits(v)


def codes_uniform(rng, shape):
    return rng.integers(-8, 8, size=shape, dtype=np.int8)


def bytes_uniform(rng, nbytes):
    """Uniform random bytes.  Read as packed 4-bit codes (offset-binary
    nibbles) these are int4 codes uniform in [-8, 7], whatever the nibble
    order."""
    return rng.integers(0, 256, size=nbytes, dtype=np.uint8)


def ongrid_source(rng, rows, K, peak_lo, peak_hi):
    """bf16 weights that lie exactly on a Q4_0 grid.

    Per group: a peak level L uniform in [peak_lo, peak_hi]; codes uniform in
    [-L, min(L, 7)] with one element forced to the peak (-8 when L = 8, else
    +L or -L with equal odds); a log-uniform scale cut to 5 significant bits.
    Then w = s0 * q0, which is exact in fp32 and in bf16.

    Returns dict(w_bits uint16 [rows, K], q0 int8 [rows, K],
                 s0_bits uint16 [rows, K/32], L int8 [rows, K/32]).
    """
    assert K % GROUP == 0
    G = K // GROUP
    L = rng.integers(peak_lo, peak_hi + 1, size=(rows, G))
    lo = -L
    hi = np.minimum(L, 7)
    u = rng.random((rows, G, GROUP))
    q = np.floor(lo[..., None] + u * (hi - lo + 1)[..., None]).astype(np.int64)
    q = np.minimum(q, hi[..., None])
    pos = rng.integers(0, GROUP, size=(rows, G))
    sign = rng.integers(0, 2, size=(rows, G))
    peak = np.where(L == 8, -8, np.where(sign == 1, L, -L))
    np.put_along_axis(q, pos[..., None], peak[..., None], axis=2)
    s0 = truncate_significand(_loguniform_f32(rng, (rows, G)), 5)
    w = (s0[..., None] * q.astype(np.float32)).astype(np.float32)
    return {
        "w_bits": to_bf16_bits(w.reshape(rows, K)),
        "q0": q.reshape(rows, K).astype(np.int8),
        "s0_bits": to_bf16_bits(s0),
        "L": L.astype(np.int8),
    }


def router_logits(rng, T, E, law="normal", zipf_s=1.1):
    """fp32 router logits.  'normal': N(0, 1).  'zipf': log p_e + Gumbel(0, 1)
    with p_e proportional to (e + 1)^-s, so the top-k of a row is a draw
    without replacement from the Zipf law (the Gumbel-top-k property)."""
    if law == "normal":
        return rng.standard_normal((T, E), dtype=np.float32)
    if law == "zipf":
        logp = -zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
        logp = logp - np.log(np.exp(logp).sum())
        return (logp[None, :] + rng.gumbel(size=(T, E))).astype(np.float32)
    raise ValueError(law)


# ---------------------------------------------------------------- device draws
# FP8 comparison experts: E4M3 codes and one fp32 scale per output channel
FP8_SCALE_LO, FP8_SCALE_HI = 5e-4, 2e-3


def fp8_codes(rng, shape):
    """E4M3 codes drawn uniformly from the 254 finite patterns: draws 0..126
    are codes 0x00..0x7E, draws 127..253 codes 0x80..0xFE (the NaN patterns
    0x7F and 0xFF are never drawn)."""
    u = rng.integers(0, 254, size=shape)
    return (u + (u >= 127)).astype(np.uint8)


def fp8_scales(rng, shape):
    """fp32 per-channel scales, log-uniform in [FP8_SCALE_LO, FP8_SCALE_HI]."""
    return _loguniform_f32(rng, shape, FP8_SCALE_LO, FP8_SCALE_HI)


def torch_generator(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def bytes_uniform_t(gen, nbytes, device):
    return torch.randint(0, 256, (int(nbytes),), dtype=torch.uint8, device=device, generator=gen)


def scales_loguniform_t(gen, shape, device):
    u = torch.rand(shape, dtype=torch.float32, device=device, generator=gen)
    v = torch.exp(np.log(SCALE_LO) + u * (np.log(SCALE_HI) - np.log(SCALE_LO)))
    return v.to(torch.bfloat16).view(torch.int16)


def bf16_normal_t(gen, shape, device):
    return torch.randn(shape, dtype=torch.float32, device=device, generator=gen).to(torch.bfloat16)


def router_logits_t(gen, T, E, device, law="normal", zipf_s=1.1):
    if law == "normal":
        return torch.randn((T, E), dtype=torch.float32, device=device, generator=gen)
    logp = -zipf_s * torch.log(torch.arange(1, E + 1, dtype=torch.float64, device=device))
    logp = logp - torch.logsumexp(logp, 0)
    u = torch.rand((T, E), dtype=torch.float64, device=device, generator=gen).clamp_min(1e-300)
    gumbel = -torch.log(-torch.log(u))
    return (logp[None, :] + gumbel).to(torch.float32)


def ongrid_source_t(gen, rows, K, peak_lo, peak_hi, device, export=False):
    """Device version of ``ongrid_source`` (same law, torch RNG).  Returns
    (w bf16 tensor [rows, K], q0 int8 [rows, K], s0 bf16-bits int16 [rows, G]).

    export=True: a "realistic export" instead -- the scale keeps its full fp32
    precision and w = bf16(s0 * q0) is rounded, as when a QAT model's fp32
    grid is saved in bf16 (s0 is then returned rounded to bf16)."""
    G = K // GROUP
    L = torch.randint(peak_lo, peak_hi + 1, (rows, G), device=device, generator=gen)
    hi = torch.clamp(L, max=7)
    span = (hi + L + 1).to(torch.float32)
    u = torch.rand((rows, G, GROUP), device=device, generator=gen)
    q = torch.floor(-L[..., None].to(torch.float32) + u * span[..., None]).to(torch.int32)
    q = torch.minimum(q, hi[..., None].to(torch.int32))
    pos = torch.randint(0, GROUP, (rows, G, 1), device=device, generator=gen)
    sign = torch.randint(0, 2, (rows, G), device=device, generator=gen)
    peak = torch.where(L == 8, torch.full_like(L, -8), torch.where(sign == 1, L, -L)).to(torch.int32)
    q.scatter_(2, pos, peak[..., None])
    uu = torch.rand((rows, G), dtype=torch.float32, device=device, generator=gen)
    s0 = torch.exp(np.log(SCALE_LO) + uu * (np.log(SCALE_HI) - np.log(SCALE_LO)))
    if not export:
        s0 = (s0.view(torch.int32) & int(np.int32(np.uint32(0xFFF80000).view(np.int32)))).view(torch.float32)
    w = (s0[..., None] * q.to(torch.float32)).to(torch.bfloat16).reshape(rows, K)
    return w, q.to(torch.int8).reshape(rows, K), s0.to(torch.bfloat16).view(torch.int16)


def fp8_codes_t(gen, shape, device):
    """Device version of ``fp8_codes``."""
    u = torch.randint(0, 254, shape, dtype=torch.int32, device=device, generator=gen)
    return (u + (u >= 127).to(torch.int32)).to(torch.uint8)


def fp8_scales_t(gen, shape, device):
    """Device version of ``fp8_scales``."""
    u = torch.rand(shape, dtype=torch.float32, device=device, generator=gen)
    return torch.exp(np.log(FP8_SCALE_LO) + u * (np.log(FP8_SCALE_HI) - np.log(FP8_SCALE_LO)))
