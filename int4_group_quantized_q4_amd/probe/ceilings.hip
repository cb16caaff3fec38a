// Machine ceilings measured beside the matmul kernels (libw4probe.so, used by
// bench.py only): how fast this GPU streams bytes out of HBM with plain
// 16-byte loads, and how fast its matrix cores run fp16 16x16x32 MFMAs with
// every operand already in registers.  The matmul kernels' rates are read
// against these as well as against the published peaks.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Each thread reads 16-byte words at a grid stride (loads of one wave cover
// 1 KiB of consecutive bytes), four in flight, and folds them with XOR; one
// word per block is written so that nothing is optimized away.
__global__ void __launch_bounds__(256) stream_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                     uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= src[i];
  uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int o = 32; o > 0; o >>= 1) v ^= (uint32_t)__shfl_xor((int)v, o, 64);
  if ((threadIdx.x & 63) == 0) atomicXor(out + blockIdx.x, v);
}

// Eight independent accumulator chains per wave, each with its own B operand,
// A and B in registers.
__global__ void __launch_bounds__(256) mfma_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  h8 a, b[8];
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (lane + i));
    for (int j = 0; j < 8; ++j) b[j][i] = (_Float16)(0.002f * (lane - i) + 0.01f * j);
  }
  f32x4 c[8];
  for (int j = 0; j < 8; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[j], c[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[j], a, c[j], 0, 0, 0);
  }
  const f32x4 s4 = ((c[0] + c[1]) + (c[2] + c[3])) + ((c[4] + c[5]) + (c[6] + c[7]));
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16) from src; out holds `blocks` words (zeroed by the caller).
int w4probe_stream(const void* src, int64_t bytes, uint32_t* out, int blocks, hipStream_t stream) {
  if (!src || !out || bytes < 16 || bytes % 16 != 0 || blocks < 1) return -1;
  hipLaunchKernelGGL(stream_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const u32x4*>(src), bytes / 16,
                     out);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// blocks x 4 waves, each running iters x 8 MFMAs of 16x16x32 (16384 flops each);
// out holds blocks * 256 floats.
int w4probe_mfma(float* out, int blocks, int iters, hipStream_t stream) {
  if (!out || blocks < 1 || iters < 1) return -1;
  hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(256), 0, stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
