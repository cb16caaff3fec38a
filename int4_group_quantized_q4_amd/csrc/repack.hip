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
// Work split: one lane per weight, a half wave (32 lanes) per group, so a
// wave64 handles two consecutive groups.  All eight trial steps of a group are
// tested with one ballot each; the least-squares sums are xor-butterflies over
// the half wave, which add first half + second half, then halves again -- the
// pairwise order the scale is defined with -- so the fp64 result is unique.

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

__global__ void __launch_bounds__(256) repack_kernel(
    const uint16_t* __restrict__ src, int64_t rows, int64_t K, uint8_t* __restrict__ qweight,
    uint16_t* __restrict__ scales, uint8_t* __restrict__ status_out,
    unsigned long long* __restrict__ counters) {
#pragma clang fp contract(off)
  const int64_t G = K / kGroup;
  const int64_t total_groups = rows * G;
  const int lane = threadIdx.x & 63;
  const int i = lane & 31;                 // element within the group
  const int half = lane >> 5;
  const int64_t waves_per_grid = (int64_t)gridDim.x * (blockDim.x >> 6);
  int64_t wave = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);

  for (; wave * 2 < total_groups; wave += waves_per_grid) {
    const int64_t gid = wave * 2 + half;
    const bool live = gid < total_groups;
    const float w = live ? bf16_to_f32(src[gid * kGroup + i]) : 0.0f;

    // non-finite groups
    const uint64_t bad = __ballot(!(fabsf(w) <= 3.4028234663852886e38f));
    const uint32_t bad_half = (uint32_t)(bad >> (32 * half));
    const bool nonfinite = bad_half != 0u;

    float a = fabsf(w);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
    const bool zero = (a == 0.0f);

    bool decided = nonfinite || zero || !live;
    int status = nonfinite ? 255 : (zero ? 1 : 0);
    float q_acc = 0.0f;   // accepted codes
    float q_m8 = 0.0f;    // codes of m = 8 (fallback)
#pragma unroll 1
    for (int m = 1; m <= 8; ++m) {
      const float s = a / (float)m;
      const float r = w / s;
      const float q = fminf(fmaxf(rintf(r), -8.0f), 7.0f);
      const bool pass = fabsf(r - q) <= kAcceptTol;
      const uint64_t fail = __ballot(!pass);
      const bool ok = ((uint32_t)(fail >> (32 * half))) == 0u;
      if (!decided && ok) {
        decided = true;
        status = m;
        q_acc = q;
      }
      if (m == 8) q_m8 = q;
      // both groups of the wave decided: later steps cannot change anything
      const uint64_t open = __ballot(!decided);
      if (open == 0ull) break;
    }
    const bool off_grid = !decided;
    if (off_grid) {
      q_acc = q_m8;
      status = 0;
    }
    if (nonfinite || zero) q_acc = 0.0f;

    // least squares with the codes fixed, fp64, pairwise (butterfly) order
    double num = (double)w * (double)q_acc;
    double den = (double)q_acc * (double)q_acc;
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) {
      num = num + __shfl_xor(num, o, 64);
      den = den + __shfl_xor(den, o, 64);
    }
    uint32_t scale_bits;
    if (nonfinite) scale_bits = 0x7FC0u;
    else if (zero) scale_bits = 0u;
    else scale_bits = f64_to_bf16_rne(num / den);

    // pack: lanes 8c..8c+7 of a half form chunk c's 4-byte word (offset binary)
    const int qi = (int)q_acc;
    uint32_t word = (uint32_t)(qi + 8) << tile16_bit(i & 7);
    word |= __shfl_xor(word, 1, 64);
    word |= __shfl_xor(word, 2, 64);
    word |= __shfl_xor(word, 4, 64);
    if (live) {
      const int64_t row = gid / G;
      const int64_t g = gid - row * G;
      if ((i & 7) == 0) {
        const int c = i >> 3;
        const int64_t off = tile16_word_offset(row / kTileRows, (int)(row % kTileRows), g, c, K);
        *reinterpret_cast<uint32_t*>(qweight + off) = word;
      }
      if (i == 0) {
        scales[tile16_scale_index(row / kTileRows, (int)(row % kTileRows), g, G)] = (uint16_t)scale_bits;
        if (status_out) status_out[gid] = (uint8_t)status;
      }
    }
    if (counters) {
      const uint64_t offb = __ballot(live && i == 0 && off_grid && !nonfinite);
      const uint64_t nfb = __ballot(live && i == 0 && nonfinite);
      if (lane == 0) {
        if (offb) atomicAdd(&counters[0], (unsigned long long)__popcll(offb));
        if (nfb) atomicAdd(&counters[1], (unsigned long long)__popcll(nfb));
      }
    }
  }
}

// One thread per 4-byte word (8 codes): out[n][32g + 8c + i] = scale * q.
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
    const bf16x8 v = unpack8_div16(word);
    float4 lo, hi;
    lo.x = s * ((float)v[0] * 16.0f);
    lo.y = s * ((float)v[1] * 16.0f);
    lo.z = s * ((float)v[2] * 16.0f);
    lo.w = s * ((float)v[3] * 16.0f);
    hi.x = s * ((float)v[4] * 16.0f);
    hi.y = s * ((float)v[5] * 16.0f);
    hi.z = s * ((float)v[6] * 16.0f);
    hi.w = s * ((float)v[7] * 16.0f);
    float4* dst = reinterpret_cast<float4*>(out + n * K + wk * 8);
    dst[0] = lo;
    dst[1] = hi;
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
  const int grid = grid_for(groups, 8);  // 8 groups per 256-thread block
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
