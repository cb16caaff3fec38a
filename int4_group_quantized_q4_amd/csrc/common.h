// Device helpers shared by the W4A16 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kGroup = 32;      // codes per scale group along K
constexpr int kTileRows = 16;   // rows per tile16 tile
constexpr int kBlockGroups = 4; // groups per tile16 block

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Byte offset, inside a tile16 matrix of K columns, of the 4-byte word that
// holds chunk c (codes 8c..8c+7 of the group) of row r within tile t for
// group g.  See the layout description in w4a16.h.
__device__ __forceinline__ int64_t tile16_word_offset(int64_t t, int r, int64_t g, int c, int64_t K) {
  const int64_t G = K / kGroup;
  const int64_t b = g / kBlockGroups;
  const int j = (int)(g - b * kBlockGroups);
  const int64_t rem = G - b * kBlockGroups;
  const int gb = rem < kBlockGroups ? (int)rem : kBlockGroups;
  return t * 8 * K + 1024 * b + 4 * gb * (16 * c + r) + 4 * j;
}

// Element index, inside a tile16 scale array of a matrix with G groups per
// row, of the scale of row r of tile t, group g (see w4a16.h).
__device__ __forceinline__ int64_t tile16_scale_index(int64_t t, int r, int64_t g, int64_t G) {
  const int64_t b = g / kBlockGroups;
  const int j = (int)(g - b * kBlockGroups);
  const int64_t rem = G - b * kBlockGroups;
  const int gb = rem < kBlockGroups ? (int)rem : kBlockGroups;
  return t * 16 * G + 64 * b + r * gb + j;
}

// Bit position, inside a tile16 word, of code i (0..7) of a chunk: even codes
// in the low half-word, odd codes in the high half-word.
__host__ __device__ constexpr int tile16_bit(int i) { return 4 * (i >> 1) + 16 * (i & 1); }

// Offset-binary nibble u of every code in the word -> bf16 pairs (128 + u of
// code 2d | 128 + u of code 2d+1 << 16), d = 0..3.  0x4300 is bf16 128.0, whose
// 7 mantissa bits step by 1, so OR-ing u in gives 128 + u = 136 + q exactly.
// The nibbles are split once into the low and high nibble of every byte
// (lo: codes 0, 4, 1, 5; hi: codes 2, 6, 3, 7 by byte), and each pair is one
// byte permute of those bytes against 0x43 (7 VALU ops per word).
__device__ __forceinline__ u32x4 biased_pairs(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu;
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
  u32x4 p;
  // v_perm_b32(S0, S1, sel): selector bytes 0-3 take S1's bytes, 4-7 S0's
  p[0] = __builtin_amdgcn_perm(0x43434343u, lo, 0x04020400u);   // [lo.b0, 43, lo.b2, 43] = codes 0, 1
  p[1] = __builtin_amdgcn_perm(0x43434343u, hi, 0x04020400u);   // codes 2, 3
  p[2] = __builtin_amdgcn_perm(0x43434343u, lo, 0x04030401u);   // [lo.b1, 43, lo.b3, 43] = codes 4, 5
  p[3] = __builtin_amdgcn_perm(0x43434343u, hi, 0x04030401u);   // codes 6, 7
  return p;
}

// bf16 -136 in every element: the operand that cancels the +136 bias of
// biased_pairs() through the MFMA's accumulator input.
constexpr uint32_t kNeg136Pair = 0xC308C308u;

// v_cvt_off_f32_i4 on byte B of a word: the low nibble of that byte, read as a
// two's-complement 4-bit integer, divided by 16 (exact).  SDWA byte select
// saves the shift.
template <int B>
__device__ __forceinline__ float cvt_i4_byte(uint32_t w) {
  float r;
  if constexpr (B == 0) {
    r = __builtin_amdgcn_cvt_off_f32_i4(w);
  } else if constexpr (B == 1) {
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(w));
  } else if constexpr (B == 2) {
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(w));
  } else {
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(w));
  }
  return r;
}

// The eight codes of a word as exact bf16 values q/16 (element i = code i).
// Flipping bit 3 of every nibble turns offset binary into two's complement;
// v_cvt_off_f32_i4 then gives q/16.  Code i sits in nibble (i/2) + 4*(i%2).
__device__ __forceinline__ bf16x8 unpack8_div16(uint32_t w) {
  const uint32_t t = w ^ 0x88888888u;
  const uint32_t h = t >> 4;
  bf16x8 r;
  r[0] = (__bf16)cvt_i4_byte<0>(t);   // nibble 0
  r[1] = (__bf16)cvt_i4_byte<2>(t);   // nibble 4
  r[2] = (__bf16)cvt_i4_byte<0>(h);   // nibble 1
  r[3] = (__bf16)cvt_i4_byte<2>(h);   // nibble 5
  r[4] = (__bf16)cvt_i4_byte<1>(t);   // nibble 2
  r[5] = (__bf16)cvt_i4_byte<3>(t);   // nibble 6
  r[6] = (__bf16)cvt_i4_byte<1>(h);   // nibble 3
  r[7] = (__bf16)cvt_i4_byte<3>(h);   // nibble 7
  return r;
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Gated activations of the MoE epilogues.  gelu with the tanh approximation,
// tanh(y) = 1 - 2 / (1 + e^(2y)): the absolute error of the hardware exp and
// reciprocal (~1e-7) moves 0.5 x (1 + tanh) by ~1e-7 relative, far below the
// bf16 rounding that follows.
__device__ __forceinline__ float gelu_tanh_f32(float x) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  const float y = c * (x + 0.044715f * x * x * x);
  const float th = 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + __expf(2.0f * y));
  return 0.5f * x * (1.0f + th);
}

__device__ __forceinline__ float silu_f32(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// fp32 -> bf16 bits, round to nearest even, by the hardware conversion.
__device__ __forceinline__ uint16_t bf16_rne(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// Wave-wide reductions (wave64).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace w4
