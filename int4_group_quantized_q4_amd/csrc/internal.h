// Kernel launchers behind the C ABI (host side, namespace w4).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4 {

void launch_repack(const uint16_t* src, int64_t rows, int64_t K, uint8_t* qweight, uint16_t* scales,
                   uint8_t* status, unsigned long long* counters, hipStream_t stream);
void launch_dequant(const uint8_t* qweight, const uint16_t* scales, int64_t rows, int64_t K,
                    float* out, hipStream_t stream);
void launch_pack(const int8_t* codes, int64_t rows, int64_t K, uint8_t* qweight, hipStream_t stream);
void launch_pack_scales(const uint16_t* src, int64_t rows, int64_t K, uint16_t* dst, hipStream_t stream);

// Grouped W4A16 matmul arguments (a dense linear layer is E = 1, no offsets).
struct GemmArgs {
  const uint16_t* x;         // [x_rows][K] bf16
  int64_t x_rows;
  const int32_t* row_index;  // nullable, [R]
  const int32_t* offsets;    // nullable (dense: rows [0, R) belong to expert 0), [E+1]
  int32_t E;
  int64_t R;                 // routed rows
  int64_t K, N;              // weight rows N (before a gated epilogue halves them)
  const uint8_t* qweight;    // E * N*K/2 bytes
  const uint16_t* scales;    // E * N*K/32, tile16 scale layout
  int32_t epilogue;          // W4_EPI_*
  void* out;
  int32_t out_dtype;         // W4_OUT_*
  // set by launch_gemm_tiled: x as fp16 rows scaled by 2^-xexp[row]
  const uint16_t* xh;
  const int32_t* xexp;
};

void launch_gemm_skinny(const GemmArgs& a, hipStream_t stream);
bool gemm_tiled_supported(const GemmArgs& a);
size_t gemm_tiled_workspace(int64_t x_rows, int64_t R, int32_t E, int64_t K, int64_t N);
void launch_gemm_tiled(const GemmArgs& a, void* ws, hipStream_t stream);
bool gemm_short_supported(const GemmArgs& a);
void launch_gemm_short(const GemmArgs& a, hipStream_t stream);
bool gemm_splitk_supported(const GemmArgs& a);
size_t gemm_splitk_workspace(int64_t R, int64_t K, int64_t N);
void launch_gemm_splitk(const GemmArgs& a, void* ws, hipStream_t stream);

size_t route_workspace_bytes(int64_t T, int32_t E, int32_t k);
void launch_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids, float* weights,
                  int32_t* offsets, int32_t* sorted_rows, int32_t* sorted_tokens, int32_t* row_to_sorted,
                  void* ws, hipStream_t stream);

void launch_combine(const void* o, int32_t o_dtype, const int32_t* row_to_sorted, const float* w,
                    int64_t T, int32_t k, int64_t N, uint16_t* y, hipStream_t stream);

}  // namespace w4
