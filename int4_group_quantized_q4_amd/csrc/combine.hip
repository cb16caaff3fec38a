// Weighted combine of the experts' outputs back into token order:
// y[t][n] = bf16( sum_{j<k} w[t][j] * o[row_to_sorted[t*k+j]][n] ), summed in
// slot order in fp32 (o[t*k+j] when row_to_sorted is null).  One thread per (token, 8 consecutive columns); the rows
// of 4 slots are loaded before any is summed, so their latencies overlap.

#include "common.h"
#include "internal.h"
#include "w4a16.h"

namespace w4 {

namespace {

// Slots j0 .. j0+NS-1 of token t added into acc, slot order; the NS rows are
// loaded before any is summed.
template <int ODT, int NS>
__device__ __forceinline__ void combine_slots(const void* __restrict__ o, const int32_t* __restrict__ row_to_sorted,
                                              const float* __restrict__ w, int64_t t, int k, int j0, int64_t N,
                                              int64_t n8, float* acc) {
  int64_t row[NS];
  float wj[NS];
#pragma unroll
  for (int c = 0; c < NS; ++c) {
    row[c] = row_to_sorted ? row_to_sorted[t * k + j0 + c] : t * k + j0 + c;
    wj[c] = w[t * k + j0 + c];
  }
  if constexpr (ODT == W4_OUT_F32) {
    float4 a[NS], b[NS];
#pragma unroll
    for (int c = 0; c < NS; ++c) {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(o) + row[c] * N + n8);
      a[c] = p[0];
      b[c] = p[1];
    }
#pragma unroll
    for (int c = 0; c < NS; ++c) {
      acc[0] += wj[c] * a[c].x; acc[1] += wj[c] * a[c].y; acc[2] += wj[c] * a[c].z; acc[3] += wj[c] * a[c].w;
      acc[4] += wj[c] * b[c].x; acc[5] += wj[c] * b[c].y; acc[6] += wj[c] * b[c].z; acc[7] += wj[c] * b[c].w;
    }
  } else {
    u32x4 v[NS];
#pragma unroll
    for (int c = 0; c < NS; ++c) v[c] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(o) + row[c] * N + n8);
#pragma unroll
    for (int c = 0; c < NS; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += wj[c] * bf16_to_f32(v[c][q] & 0xFFFFu);
        acc[2 * q + 1] += wj[c] * bf16_to_f32(v[c][q] >> 16);
      }
  }
}

template <int ODT>
__global__ void __launch_bounds__(256) combine_kernel(const void* __restrict__ o, const int32_t* __restrict__ row_to_sorted,
                                                      const float* __restrict__ w, int64_t T, int k, int64_t N,
                                                      uint16_t* __restrict__ y) {
  constexpr int CH = 4;   // slots whose rows are in flight together
  const int64_t cols8 = N / 8;
  const int64_t total = T * cols8;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = idx / cols8;
    const int64_t n8 = (idx - t * cols8) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int j0 = 0;
    for (; j0 + CH <= k; j0 += CH) combine_slots<ODT, CH>(o, row_to_sorted, w, t, k, j0, N, n8, acc);
    for (; j0 < k; ++j0) combine_slots<ODT, 1>(o, row_to_sorted, w, t, k, j0, N, n8, acc);
    u32x4 out;
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = f32_to_bf16(acc[2 * q]) | (f32_to_bf16(acc[2 * q + 1]) << 16);
    *reinterpret_cast<u32x4*>(y + t * N + n8) = out;
  }
}

}  // namespace

void launch_combine(const void* o, int32_t o_dtype, const int32_t* row_to_sorted, const float* w, int64_t T,
                    int32_t k, int64_t N, uint16_t* y, hipStream_t stream) {
  const int64_t total = T * (N / 8);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  if (o_dtype == W4_OUT_F32)
    hipLaunchKernelGGL(combine_kernel<W4_OUT_F32>, dim3((unsigned)blocks), dim3(256), 0, stream, o, row_to_sorted, w, T,
                       k, N, y);
  else
    hipLaunchKernelGGL(combine_kernel<W4_OUT_BF16>, dim3((unsigned)blocks), dim3(256), 0, stream, o, row_to_sorted, w,
                       T, k, N, y);
}

}  // namespace w4
