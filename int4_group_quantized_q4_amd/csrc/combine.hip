// Weighted combine of the experts' outputs back into token order:
// y[t][n] = bf16( sum_{j<k} w[t][j] * o[row_to_sorted[t*k+j]][n] ), summed in
// slot order in fp32.  One thread per (token, 8 consecutive columns).

#include "common.h"
#include "internal.h"
#include "w4a16.h"

namespace w4 {

namespace {

template <int ODT>
__global__ void __launch_bounds__(256) combine_kernel(const void* __restrict__ o, const int32_t* __restrict__ row_to_sorted,
                                                      const float* __restrict__ w, int64_t T, int k, int64_t N,
                                                      uint16_t* __restrict__ y) {
  const int64_t cols8 = N / 8;
  const int64_t total = T * cols8;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = idx / cols8;
    const int64_t n8 = (idx - t * cols8) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int64_t row = row_to_sorted[t * k + j];
      const float wj = w[t * k + j];
      if constexpr (ODT == W4_OUT_F32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(o) + row * N + n8);
        const float4 a = p[0], b = p[1];
        acc[0] += wj * a.x; acc[1] += wj * a.y; acc[2] += wj * a.z; acc[3] += wj * a.w;
        acc[4] += wj * b.x; acc[5] += wj * b.y; acc[6] += wj * b.z; acc[7] += wj * b.w;
      } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(o) + row * N + n8);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += wj * bf16_to_f32(v[q] & 0xFFFFu);
          acc[2 * q + 1] += wj * bf16_to_f32(v[q] >> 16);
        }
      }
    }
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
