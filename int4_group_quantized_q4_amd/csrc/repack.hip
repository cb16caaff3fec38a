// Q4_0 group-32 repack, dequant and code packing kernels (gfx950).
//
// Repack: [RQ] "Repacked QAT Gemma 4 26B-A4B serves on one TPU v6e at 1.9x FP8
// throughput", section "A repack, not a re-quantization"; [QP] "The
// Quantization Problem I Didn't Know I Had ...", section "Building the Missing
// Piece".  The bf16 source already lies on a 16-level grid per group of 32; the
// kernel recovers each group's step by trying max|w|/m for m = 1..8, keeps the
// first m that reproduces the group, refines the step by least squares and
// stores it at bf16.
//
// Work split: 8 lanes per group, 4 consecutive values per lane (one 64-bit
// load), so a wave holds 8 groups.  max|w| is a DPP reduction inside the 8
// lanes; each trial step's verdict for a group is one byte of a ballot.  The
// quotients w / s_m of a trial come from one reciprocal and a multiply per
// value; where that cannot decide (a value whose distance to the nearest
// integer lies within 1e-5 of the tolerance, or, for the m = 8 codes kept by
// off-grid groups, within 1e-5 of a tie), the lane recomputes its values with
// the correctly rounded division -- so every decision and code is the one the
// exact quotients give.  The least-squares sums add lane j + 4, j + 2, j + 1
// and then inside the lane: the pairwise order (first half + second half,
// repeatedly) the scale is defined with, so the fp64 result is unique.

#include "common.h"
#include "internal.h"

namespace w4 {

namespace {

constexpr float kAcceptTol = 0.09375f;  // 3/32 of a grid step

// fp64 -> bf16 bits, one rounding to nearest even (finite input).
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  const uint64_t mag = u & 0x7FFFFFFFFFFFFFFFull;
  const double ax = __longlong_as_double((long long)mag);
  if (ax < 0x1p-126) {
    // bf16 subnormal range: multiples of 2^-133; scaling by 2^133 is exact.
    const double k = rint(ax * 0x1p133);
    return sign | (uint32_t)k;  // k == 128 is the smallest normal, 0x0080
  }
  const uint64_t r = (mag + 0xFFFFFFFFFFFull + ((mag >> 45) & 1ull)) >> 45;
  const int64_t e = (int64_t)(r >> 7) - 1023 + 127;
  if (e >= 255) return sign | 0x7F80u;
  return sign | ((uint32_t)e << 7) | (uint32_t)(r & 0x7F);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// v (fp64) of lane i + N of the 16-lane row (row_shl:N); lanes past the row's
// end read 0 -- only lanes whose partner is in the same 8-lane group are used
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// |quotient error| of the reciprocal path is below 2e-6 (|w/s| <= 8); decisions
// within kUnsure of a boundary take the exact division
constexpr float kUnsure = 1e-5f;

__global__ void __launch_bounds__(256) repack_kernel(
    const uint16_t* __restrict__ src, int64_t rows, int64_t K, uint8_t* __restrict__ qweight,
    uint16_t* __restrict__ scales, uint8_t* __restrict__ status_out,
    unsigned long long* __restrict__ counters) {
#pragma clang fp contract(off)
  const int64_t G = K / kGroup;
  const int64_t total_groups = rows * G;
  const int lane = threadIdx.x & 63;
  const int j = lane & 7;       // this lane's values: 4j .. 4j+3 of its group
  const int gsl = lane >> 3;    // group slot in the wave
  const int64_t waves_per_grid = (int64_t)gridDim.x * (blockDim.x >> 6);
  int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);

  for (; wave * 8 < total_groups; wave += waves_per_grid) {
    const int64_t gid = wave * 8 + gsl;
    const bool live = gid < total_groups;
    float w[4] = {0.f, 0.f, 0.f, 0.f};
    if (live) {
      const uint2 v = *reinterpret_cast<const uint2*>(src + gid * kGroup + 4 * j);
      w[0] = bf16_to_f32(v.x & 0xFFFFu);
      w[1] = bf16_to_f32(v.x >> 16);
      w[2] = bf16_to_f32(v.y & 0xFFFFu);
      w[3] = bf16_to_f32(v.y >> 16);
    }

    // a group with a non-finite value counts as all zeros until the end
    bool bad = false;
#pragma unroll
    for (int k = 0; k < 4; ++k) bad |= !(fabsf(w[k]) <= 3.4028234663852886e38f);
    const bool nonfinite = ((uint32_t)(__ballot(bad) >> (8 * gsl)) & 0xFFu) != 0u;
    if (nonfinite) {
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = 0.f;
    }

    float a = fmaxf(fmaxf(fabsf(w[0]), fabsf(w[1])), fmaxf(fabsf(w[2]), fabsf(w[3])));
    a = fmaxf(a, dpp_f32<0xB1>(a));    // quad_perm [1,0,3,2]
    a = fmaxf(a, dpp_f32<0x4E>(a));    // quad_perm [2,3,0,1]
    a = fmaxf(a, dpp_f32<0x141>(a));   // row_half_mirror: the 8 lanes of the group
    const bool zero = (a == 0.0f);

    bool decided = nonfinite || zero || !live;
    int status = nonfinite ? 255 : (zero ? 1 : 0);
    float qa[4] = {0.f, 0.f, 0.f, 0.f};   // accepted codes
    float q8[4] = {0.f, 0.f, 0.f, 0.f};   // codes of m = 8 (the off-grid fallback)
    // s_m = a / m correctly rounded: a division for m = 3, 5, 7; the others
    // are exact power-of-two scalings of a, a/3 (normal range: a within
    // [2^-100, 2^100]; outside it every step is a division)
    const bool scale_ok = a >= 0x1p-100f && a <= 0x1p100f;
    float a3 = 0.f;
#pragma unroll 1
    for (int m = 1; m <= 8; ++m) {
      float s;
      if (!scale_ok || m == 5 || m == 7) {
        s = a / (float)m;
      } else if (m == 3) {
        a3 = a / 3.0f;
        s = a3;
      } else if (m == 6) {
        s = a3 * 0.5f;
      } else {
        s = a * (m == 1 ? 1.0f : m == 2 ? 0.5f : m == 4 ? 0.25f : 0.125f);
      }
      const float sd = decided ? 1.0f : s;
      const bool fast = sd >= 0x1p-100f && sd <= 0x1p100f;
      const float rc = __builtin_amdgcn_rcpf(sd);
      float q[4];
      bool pass = true, unsure = !fast;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float r = w[k] * rc;
        const float qk = fminf(fmaxf(rintf(r), -8.0f), 7.0f);
        const float d = fabsf(r - qk);
        unsure |= fabsf(d - kAcceptTol) <= kUnsure;
        if (m == 8) unsure |= fabsf(fabsf(r - floorf(r)) - 0.5f) <= kUnsure;
        q[k] = qk;
        pass &= d <= kAcceptTol;
      }
      if (unsure && !decided) {   // the correctly rounded quotients
        pass = true;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float r = w[k] / sd;
          q[k] = fminf(fmaxf(rintf(r), -8.0f), 7.0f);
          pass &= fabsf(r - q[k]) <= kAcceptTol;
        }
      }
      const bool ok = ((uint32_t)(__ballot(!pass) >> (8 * gsl)) & 0xFFu) == 0u;
      if (!decided && ok) {
        decided = true;
        status = m;
#pragma unroll
        for (int k = 0; k < 4; ++k) qa[k] = q[k];
      }
      if (m == 8) {
#pragma unroll
        for (int k = 0; k < 4; ++k) q8[k] = q[k];
      }
      // every group of the wave decided: later steps cannot change anything
      if (__ballot(!decided) == 0ull) break;
    }
    const bool off_grid = !decided;
    if (off_grid) {
#pragma unroll
      for (int k = 0; k < 4; ++k) qa[k] = q8[k];
      status = 0;
    }
    if (nonfinite || zero) {
#pragma unroll
      for (int k = 0; k < 4; ++k) qa[k] = 0.f;
    }

    // least squares with the codes fixed, fp64, pairwise order: values i and
    // i + 16 (lane j + 4), then i + 8 (lane j + 2), i + 4 (lane j + 1), then
    // inside lane j = 0: values k and k + 2, then the last pair
    double nv[4], dv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      nv[k] = (double)w[k] * (double)qa[k];
      dv[k] = (double)qa[k] * (double)qa[k];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      nv[k] = nv[k] + dpp_f64<0x104>(nv[k]);   // row_shl:4: lane j + 4
      dv[k] = dv[k] + dpp_f64<0x104>(dv[k]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      nv[k] = nv[k] + dpp_f64<0x102>(nv[k]);   // row_shl:2
      dv[k] = dv[k] + dpp_f64<0x102>(dv[k]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      nv[k] = nv[k] + dpp_f64<0x101>(nv[k]);   // row_shl:1
      dv[k] = dv[k] + dpp_f64<0x101>(dv[k]);
    }
    const double num = (nv[0] + nv[2]) + (nv[1] + nv[3]);
    const double den = (dv[0] + dv[2]) + (dv[1] + dv[3]);
    uint32_t scale_bits;
    if (nonfinite) scale_bits = 0x7FC0u;
    else if (zero) scale_bits = 0u;
    else scale_bits = f64_to_bf16_rne(den > 0.0 ? num / den : 0.0);

    // pack: lane j holds codes 4j..4j+3, half of chunk j/2; lanes 2c and 2c+1
    // OR their halves into chunk c's 4-byte word (offset binary)
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) word |= ((uint32_t)((int)qa[k] + 8) & 0xFu) << tile16_bit(4 * (j & 1) + k);
    word |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)word, 0xB1, 0xF, 0xF, false);   // lane ^ 1
    if (live) {
      const int64_t row = gid / G;
      const int64_t g = gid - row * G;
      if ((j & 1) == 0) {
        const int64_t off = tile16_word_offset(row / kTileRows, (int)(row % kTileRows), g, j >> 1, K);
        *reinterpret_cast<uint32_t*>(qweight + off) = word;
      }
      if (j == 0) {
        scales[tile16_scale_index(row / kTileRows, (int)(row % kTileRows), g, G)] = (uint16_t)scale_bits;
        if (status_out) status_out[gid] = (uint8_t)status;
      }
    }
    if (counters) {
      const uint64_t offb = __ballot(live && j == 0 && off_grid && !nonfinite);
      const uint64_t nfb = __ballot(live && j == 0 && nonfinite);
      if (lane == 0) {
        if (offb) atomicAdd(&counters[0], (unsigned long long)__popcll(offb));
        if (nfb) atomicAdd(&counters[1], (unsigned long long)__popcll(nfb));
      }
    }
  }
}

// One thread per 4-byte word (8 codes): out[n][32g + 8c + i] = scale * q.  The
// codes go through biased_pairs(), the unpack the weight-streaming matmul
// kernels feed to the matrix cores (bf16 136 + q, two codes per register), so
// a bit-exact check of this output checks that routine's nibble order too.
__global__ void __launch_bounds__(256) dequant_kernel(
    const uint8_t* __restrict__ qweight, const uint16_t* __restrict__ scales, int64_t rows,
    int64_t K, float* __restrict__ out) {
  const int64_t words_per_row = K / 8;
  const int64_t total = rows * words_per_row;
  const int64_t G = K / kGroup;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = idx / words_per_row;
    const int64_t wk = idx - n * words_per_row;
    const int64_t g = wk >> 2;
    const int c = (int)(wk & 3);
    const uint32_t word = *reinterpret_cast<const uint32_t*>(
        qweight + tile16_word_offset(n / kTileRows, (int)(n % kTileRows), g, c, K));
    const float s = bf16_to_f32(scales[tile16_scale_index(n / kTileRows, (int)(n % kTileRows), g, G)]);
    const u32x4 p = biased_pairs(word);   // pair d: codes 2d (low half), 2d + 1 (high half)
    float v[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      v[2 * d] = s * (bf16_to_f32(p[d] & 0xFFFFu) - 136.0f);
      v[2 * d + 1] = s * (bf16_to_f32(p[d] >> 16) - 136.0f);
    }
    float4* dst = reinterpret_cast<float4*>(out + n * K + wk * 8);
    dst[0] = float4{v[0], v[1], v[2], v[3]};
    dst[1] = float4{v[4], v[5], v[6], v[7]};
  }
}

// One thread per word: 8 int8 codes -> 8 offset-binary nibbles at their tile16 place.
__global__ void __launch_bounds__(256) pack_kernel(const int8_t* __restrict__ codes, int64_t rows,
                                                   int64_t K, uint8_t* __restrict__ qweight) {
  const int64_t words_per_row = K / 8;
  const int64_t total = rows * words_per_row;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = idx / words_per_row;
    const int64_t wk = idx - n * words_per_row;
    const uint2 src = *reinterpret_cast<const uint2*>(codes + n * K + wk * 8);
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t byte = ((i < 4 ? src.x : src.y) >> (8 * (i & 3))) & 0xFFu;
      word |= ((byte + 8u) & 0xFu) << tile16_bit(i);   // offset binary of the signed code
    }
    *reinterpret_cast<uint32_t*>(
        qweight + tile16_word_offset(n / kTileRows, (int)(n % kTileRows), wk >> 2, (int)(wk & 3), K)) = word;
  }
}

// One thread per scale: plain [rows][G] -> tile16 scale layout.
__global__ void __launch_bounds__(256) pack_scales_kernel(const uint16_t* __restrict__ src, int64_t rows,
                                                          int64_t G, uint16_t* __restrict__ dst) {
  const int64_t total = rows * G;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = idx / G;
    const int64_t g = idx - n * G;
    dst[tile16_scale_index(n / kTileRows, (int)(n % kTileRows), g, G)] = src[idx];
  }
}

int grid_for(int64_t items, int per_block) {
  int64_t b = (items + per_block - 1) / per_block;
  if (b < 1) b = 1;
  const int64_t cap = 256 * 64;  // enough blocks to fill 256 CUs many times over
  return (int)(b < cap ? b : cap);
}

}  // namespace

void launch_repack(const uint16_t* src, int64_t rows, int64_t K, uint8_t* qweight, uint16_t* scales,
                   uint8_t* status, unsigned long long* counters, hipStream_t stream) {
  const int64_t groups = rows * (K / kGroup);
  const int grid = grid_for(groups, 32);  // 32 groups per 256-thread block
  hipLaunchKernelGGL(repack_kernel, dim3(grid), dim3(256), 0, stream, src, rows, K, qweight, scales,
                     status, counters);
}

void launch_dequant(const uint8_t* qweight, const uint16_t* scales, int64_t rows, int64_t K,
                    float* out, hipStream_t stream) {
  const int grid = grid_for(rows * (K / 8), 256);
  hipLaunchKernelGGL(dequant_kernel, dim3(grid), dim3(256), 0, stream, qweight, scales, rows, K, out);
}

void launch_pack_scales(const uint16_t* src, int64_t rows, int64_t K, uint16_t* dst, hipStream_t stream) {
  const int64_t G = K / kGroup;
  const int grid = grid_for(rows * G, 256);
  hipLaunchKernelGGL(pack_scales_kernel, dim3(grid), dim3(256), 0, stream, src, rows, G, dst);
}

void launch_pack(const int8_t* codes, int64_t rows, int64_t K, uint8_t* qweight, hipStream_t stream) {
  const int grid = grid_for(rows * (K / 8), 256);
  hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(256), 0, stream, codes, rows, K, qweight);
}

}  // namespace w4
