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

// Eight codes of one word (code i in bits 4i..4i+3, two's complement) ->
// eight bf16 values q/16, exact: one shift, eight conversions, four packs.
// The 1/16 is undone by the caller in fp32 (an exact power-of-two scaling).
__device__ __forceinline__ bf16x8 unpack8_div16(uint32_t w) {
  const uint32_t h = w >> 4;
  bf16x8 r;
  r[0] = (__bf16)cvt_i4_byte<0>(w);
  r[1] = (__bf16)cvt_i4_byte<0>(h);
  r[2] = (__bf16)cvt_i4_byte<1>(w);
  r[3] = (__bf16)cvt_i4_byte<1>(h);
  r[4] = (__bf16)cvt_i4_byte<2>(w);
  r[5] = (__bf16)cvt_i4_byte<2>(h);
  r[6] = (__bf16)cvt_i4_byte<3>(w);
  r[7] = (__bf16)cvt_i4_byte<3>(h);
  return r;
}

// Signed 4-bit code i of a word, as an integer.
__device__ __forceinline__ int code_of(uint32_t w, int i) {
  return ((int)(w << (28 - 4 * i))) >> 28;
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Wave-wide reductions (wave64).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace w4
