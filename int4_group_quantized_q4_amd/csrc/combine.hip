// Weighted combine of the experts' outputs back into token order:
// y[t][n] = bf16( sum_{j<k} w[t][j] * o[row_to_sorted[t*k+j]][n] ), summed in
// slot order in fp32 (o[t*k+j] when row_to_sorted is null).  One thread per
// (token, 16 bytes of each o row: 4 fp32 or 8 bf16 columns).  With k = 8 (the
// MoE layers here) all eight rows are loaded before any is summed, so the
// call waits for one memory latency; other k go in chunks of 4 slots.

#include "common.h"
#include "internal.h"
#include "w4a16.h"

namespace w4 {

namespace {

template <int ODT>
constexpr int kCols = ODT == W4_OUT_F32 ? 4 : 8;   // columns per thread: one 16-byte load per slot

// Slots j0 .. j0+NS-1 of token t added into acc, slot order; the NS rows are
// loaded before any is summed.
template <int ODT, int NS>
__device__ __forceinline__ void combine_slots(const void* __restrict__ o, const int32_t* __restrict__ row_to_sorted,
                                              const float* __restrict__ w, int64_t t, int k, int j0, int64_t N,
                                              int64_t n0, float* acc) {
  int64_t row[NS];
  float wj[NS];
#pragma unroll
  for (int c = 0; c < NS; ++c) {
    row[c] = row_to_sorted ? row_to_sorted[t * k + j0 + c] : t * k + j0 + c;
    wj[c] = w[t * k + j0 + c];
  }
  u32x4 v[NS];
#pragma unroll
  for (int c = 0; c < NS; ++c) {
    // (o is read once: non-temporal loads)
    if constexpr (ODT == W4_OUT_F32)
      v[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const float*>(o) + row[c] * N + n0));
    else
      v[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(o) + row[c] * N + n0));
  }
#pragma unroll
  for (int c = 0; c < NS; ++c) {
    if constexpr (ODT == W4_OUT_F32) {
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] += wj[c] * __uint_as_float(v[c][q]);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += wj[c] * bf16_to_f32(v[c][q] & 0xFFFFu);
        acc[2 * q + 1] += wj[c] * bf16_to_f32(v[c][q] >> 16);
      }
    }
  }
}

// KS = 8: exactly eight slots, all in flight together; KS = 0: any k.
template <int ODT, int KS>
__global__ void __launch_bounds__(256) combine_kernel(const void* __restrict__ o, const int32_t* __restrict__ row_to_sorted,
                                                      const float* __restrict__ w, int64_t T, int k, int64_t N,
                                                      uint16_t* __restrict__ y) {
  constexpr int C = kCols<ODT>;
  constexpr int CH = 4;   // slots in flight together for KS = 0
  const int64_t cols = N / C;
  const int64_t total = T * cols;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = idx / cols;
    const int64_t n0 = (idx - t * cols) * C;
    float acc[C];
#pragma unroll
    for (int q = 0; q < C; ++q) acc[q] = 0.f;
    if constexpr (KS > 0) {
      combine_slots<ODT, KS>(o, row_to_sorted, w, t, k, 0, N, n0, acc);
    } else {
      int j0 = 0;
      for (; j0 + CH <= k; j0 += CH) combine_slots<ODT, CH>(o, row_to_sorted, w, t, k, j0, N, n0, acc);
      for (; j0 < k; ++j0) combine_slots<ODT, 1>(o, row_to_sorted, w, t, k, j0, N, n0, acc);
    }
    if constexpr (C == 4) {
      u32x2 out;
#pragma unroll
      for (int q = 0; q < 2; ++q) out[q] = f32_to_bf16(acc[2 * q]) | (f32_to_bf16(acc[2 * q + 1]) << 16);
      *reinterpret_cast<u32x2*>(y + t * N + n0) = out;
    } else {
      u32x4 out;
#pragma unroll
      for (int q = 0; q < 4; ++q) out[q] = f32_to_bf16(acc[2 * q]) | (f32_to_bf16(acc[2 * q + 1]) << 16);
      *reinterpret_cast<u32x4*>(y + t * N + n0) = out;
    }
  }
}

template <int ODT>
void launch_typed(const void* o, const int32_t* row_to_sorted, const float* w, int64_t T, int32_t k, int64_t N,
                  uint16_t* y, hipStream_t stream) {
  const int64_t total = T * (N / kCols<ODT>);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  if (k == 8)
    hipLaunchKernelGGL((combine_kernel<ODT, 8>), dim3((unsigned)blocks), dim3(256), 0, stream, o, row_to_sorted, w, T,
                       k, N, y);
  else
    hipLaunchKernelGGL((combine_kernel<ODT, 0>), dim3((unsigned)blocks), dim3(256), 0, stream, o, row_to_sorted, w, T,
                       k, N, y);
}

}  // namespace

void launch_combine(const void* o, int32_t o_dtype, const int32_t* row_to_sorted, const float* w, int64_t T,
                    int32_t k, int64_t N, uint16_t* y, hipStream_t stream) {
  if (o_dtype == W4_OUT_F32) launch_typed<W4_OUT_F32>(o, row_to_sorted, w, T, k, N, y, stream);
  else launch_typed<W4_OUT_BF16>(o, row_to_sorted, w, T, k, N, y, stream);
}

}  // namespace w4
