"""Helpers for the GPU parity tests: host <-> device transfer of bf16 bit
patterns and seeded MoE weight sets (packed bytes for the GPU, decoded
logical codes for the oracle)."""

import sys

import numpy as np
import torch

import gen
import layout


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def bits_host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def linear_weights(rng, N, K):
    """(packed bytes uint8 [N*K/2], tiled scale bits [N*K/32], codes int8 [N, K],
    plain scale bits uint16 [N, K/32]).  The first two feed the GPU, the last
    two the oracle."""
    packed = gen.bytes_uniform(rng, N * K // 2)
    codes = layout.decode(packed, N, K)
    scales = gen.scales_loguniform(rng, (N, K // 32))
    return packed, layout.encode_scales(scales), codes, scales


def expert_weights(rng, E, N, K):
    """Stacked experts: (packed [E*N*K/2], tiled scales [E*N*K/32]) for the GPU,
    (codes int8 [E, N, K], plain scales [E, N, K/32]) for the oracle."""
    packed = gen.bytes_uniform(rng, E * N * K // 2)
    byte, shift = layout._index(N, K)
    per = packed.reshape(E, N * K // 2)
    v = (per[:, byte] >> shift[None]) & 0xF
    codes = (v.astype(np.int16) - 8).astype(np.int8)
    scales = gen.scales_loguniform(rng, (E, N, K // 32))
    tiled = np.empty(E * N * (K // 32), dtype=scales.dtype).reshape(E, -1)
    idx = layout._scale_index(N, K)
    for e in range(E):
        tiled[e, idx] = scales[e]
    return packed, tiled.reshape(-1), codes, scales


def f32_bits_equal(a, b):
    """Bitwise equality of fp32 arrays, with any NaN matching any NaN."""
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    return np.array_equal(na, nb) and np.array_equal(a[~na].view(np.uint32), b[~nb].view(np.uint32))
