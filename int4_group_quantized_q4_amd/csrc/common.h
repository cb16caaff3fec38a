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

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Gated activations of the MoE epilogues.  gelu with the tanh approximation:
// 0.5 x (1 + tanh(y)) = x * sigmoid(2y) = x / (1 + e^(-2y)), y = sqrt(2/pi) (x +
// 0.044715 x^3).  No term cancels, so the hardware exp and reciprocal (about
// 1e-7 relative each) give about 3e-7 relative error for every x, in the
// negative tail too (where 1 + tanh(y) formed by subtraction would lose every
// digit below x = -5); e^(-2y) = inf at large negative x gives -0.
__device__ __forceinline__ float gelu_tanh_f32(float x) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  const float y = c * (x + 0.044715f * x * x * x);
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-2.0f * y));
}

__device__ __forceinline__ float silu_f32(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// fp32 -> bf16 bits, round to nearest even, by the hardware conversion.
__device__ __forceinline__ uint16_t bf16_rne(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// Routed rows of expert e in a top-k id list ids[0 .. R) (routed row r = t*k + j
// holds the j-th expert of token t): the r with ids[r] == e, in increasing
// order, written to rows[0 .. min(count, cap)); returns count.  All NW waves of
// the workgroup take part: in round q, wave w scans ids [512 (q NW + w), +512)
// and a prefix over the waves' counts (s_cnt, NW ints of LDS) places its
// rows, so each round costs one load latency (R <= 512: wave 0 alone).  Round 0's ids
// are loaded by ids_batch() beforehand, so a caller can issue those loads
// ahead of its other loads (vector loads complete in order: loads issued
// before them would be waited for too).  Ends with a workgroup barrier.
__device__ __forceinline__ void ids_batch(const int32_t* __restrict__ ids, int R, int batch, int v[8]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int r = 512 * batch + 64 * q + lane;
    v[q] = r < R ? ids[r] : -1;
  }
}

template <int NW>
__device__ __forceinline__ int expert_rows_from_ids(const int32_t* __restrict__ ids, int R, int e, int* rows,
                                                    int cap, int* s_cnt, int v[8]) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint64_t below = (1ull << lane) - 1ull;
  if (R <= 512) {   // one batch: wave 0 alone, one barrier
    if (wv == 0) {
      int n = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint64_t b = __ballot(v[q] == e);
        const int pos = n + __popcll(b & below);
        if (((b >> lane) & 1ull) && pos < cap) rows[pos] = 64 * q + lane;
        n += __popcll(b);
      }
      if (lane == 0) s_cnt[0] = n;
    }
    __syncthreads();
    return s_cnt[0];
  }
  int total = 0;
  for (int round = 0; 512 * NW * round < R; ++round) {
    if (round > 0) ids_batch(ids, R, NW * round + wv, v);
    uint64_t b[8];
    int n = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      b[q] = __ballot(v[q] == e);
      n += __popcll(b[q]);
    }
    if (lane == 0) s_cnt[wv] = n;
    __syncthreads();
    int base = total, all = total;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int c = s_cnt[w];
      if (w < wv) base += c;
      all += c;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int pos = base + __popcll(b[q] & below);
      if (((b[q] >> lane) & 1ull) && pos < cap) rows[pos] = 512 * (NW * round + wv) + 64 * q + lane;
      base += __popcll(b[q]);
    }
    total = all;
    __syncthreads();   // rows written; s_cnt free for the next round
  }
  return total;
}

// Reductions within each 16-lane row by DPP (every lane gets its row's
// result), and over the wave from the four rows' results.
template <int CTRL>
__device__ __forceinline__ float dpp_row_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_row_f32<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_row_f32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_row_f32<0x141>(v));   // row_half_mirror
  return fmaxf(v, dpp_row_f32<0x140>(v));   // row_mirror
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_row_f32<0xB1>(v);
  v += dpp_row_f32<0x4E>(v);
  v += dpp_row_f32<0x141>(v);
  return v + dpp_row_f32<0x140>(v);
}
__device__ __forceinline__ float lane_f32(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// wave-uniform maximum
__device__ __forceinline__ float wave_max_all(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(lane_f32(v, 0), lane_f32(v, 16)), fmaxf(lane_f32(v, 32), lane_f32(v, 48)));
}
// wave-uniform sum, as (row0 + row1) + (row2 + row3)
__device__ __forceinline__ float wave_sum_all(float v) {
  v = row16_sum(v);
  return (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
}

// Softmax terms of one token whose logits sit S per lane (lane l holds experts
// l, l + 64, ...; live[s] false past E): the token's largest logit mx and
// sum_e exp(l_e - mx), both wave-uniform.  The routing kernel and the
// logits-mode decode matmul both take them from here, so the routing weights
// they write agree bit for bit.
template <int S>
__device__ __forceinline__ void token_softmax_terms(const float v[S], const bool live[S], float& mx, float& sum) {
  float cand = -INFINITY;
#pragma unroll
  for (int s = 0; s < S; ++s)
    if (live[s]) cand = fmaxf(cand, v[s]);
  mx = wave_max_all(cand);
  sum = 0.f;
#pragma unroll
  for (int s = 0; s < S; ++s)
    if (live[s]) sum += expf(v[s] - mx);
  sum = wave_sum_all(sum);
}

// Wave-wide reductions (wave64).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace w4
