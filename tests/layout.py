"""Host-side encoder/decoder of the tile16 packed layout (offset-binary codes), written from its
description in include/w4a16.h (test infrastructure; independent of the HIP
code that reads and writes the layout on the GPU)."""

import functools

import numpy as np


@functools.lru_cache(maxsize=16)
def _index(rows, K):
    """Byte index and nibble shift of every logical code (row, k)."""
    assert rows % 16 == 0 and K % 32 == 0
    G = K // 32
    row = np.arange(rows, dtype=np.int64)[:, None]
    k = np.arange(K, dtype=np.int64)[None, :]
    t, r = row // 16, row % 16
    g = k // 32
    b, j = g // 4, g % 4
    gb = np.minimum(4, G - 4 * b)
    c = (k % 32) // 8
    i = k % 8
    word = t * 8 * K + 1024 * b + 4 * gb * (16 * c + r) + 4 * j
    bit = 4 * (i // 2) + 16 * (i % 2)              # position inside the little-endian word
    byte = word + bit // 8
    shift = bit % 8
    return byte, np.broadcast_to(shift, byte.shape).astype(np.uint8)


def encode(codes):
    """int8 codes [rows, K] (each in -8..7) -> packed uint8 [rows*K/2]."""
    codes = np.asarray(codes)
    rows, K = codes.shape
    byte, shift = _index(rows, K)
    nib = (codes.astype(np.int16) + 8).astype(np.uint8) << shift      # offset binary
    out = np.zeros(rows * K // 2, dtype=np.uint8)
    lo = shift == 0                      # every byte gets one low and one high nibble
    out[byte[lo]] = nib[lo]
    out[byte[~lo]] |= nib[~lo]
    return out


def decode(packed, rows, K):
    """packed uint8 [rows*K/2] -> int8 codes [rows, K]."""
    packed = np.asarray(packed, dtype=np.uint8).reshape(-1)
    assert packed.size == rows * K // 2
    byte, shift = _index(rows, K)
    v = (packed[byte] >> shift) & 0xF
    return (v.astype(np.int16) - 8).astype(np.int8)


def decode_experts(packed, E, rows, K):
    """Stacked experts: packed [E * rows*K/2] -> int8 [E, rows, K]."""
    packed = np.asarray(packed, dtype=np.uint8).reshape(E, rows * K // 2)
    return np.stack([decode(packed[e], rows, K) for e in range(E)])


@functools.lru_cache(maxsize=16)
def _scale_index(rows, K):
    """Position, in the tile16 scale array, of the scale of (row, group)."""
    assert rows % 16 == 0 and K % 32 == 0
    G = K // 32
    row = np.arange(rows, dtype=np.int64)[:, None]
    g = np.arange(G, dtype=np.int64)[None, :]
    t, r = row // 16, row % 16
    b, j = g // 4, g % 4
    gb = np.minimum(4, G - 4 * b)
    return t * 16 * G + 64 * b + r * gb + j


def encode_scales(scales):
    """plain bf16 bits [rows, K/32] -> tile16 scale array [rows*K/32]."""
    scales = np.asarray(scales)
    rows, G = scales.shape
    out = np.empty(rows * G, dtype=scales.dtype)
    out[_scale_index(rows, G * 32)] = scales
    return out


def decode_scales(tiled, rows, K):
    """tile16 scale array [rows*K/32] -> plain [rows, K/32]."""
    tiled = np.asarray(tiled).reshape(-1)
    return tiled[_scale_index(rows, K)]
