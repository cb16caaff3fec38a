"""Host-side encoder/decoder of the tile16 packed layout, written from its
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
    byte = t * 8 * K + 1024 * b + 4 * gb * (16 * c + r) + 4 * j + i // 2
    shift = 4 * (i % 2)
    return byte, shift.astype(np.uint8)


def encode(codes):
    """int8 codes [rows, K] (each in -8..7) -> packed uint8 [rows*K/2]."""
    codes = np.asarray(codes)
    rows, K = codes.shape
    byte, shift = _index(rows, K)
    shift = np.broadcast_to(shift, codes.shape)
    nib = (codes.astype(np.int16) & 0xF).astype(np.uint8) << shift
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
    return ((v.astype(np.int16) ^ 8) - 8).astype(np.int8)


def decode_experts(packed, E, rows, K):
    """Stacked experts: packed [E * rows*K/2] -> int8 [E, rows, K]."""
    packed = np.asarray(packed, dtype=np.uint8).reshape(E, rows * K // 2)
    return np.stack([decode(packed[e], rows, K) for e in range(E)])
