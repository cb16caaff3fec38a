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
  // nullable: output row of sorted row i is out_index[i] (else i)
  const int32_t* out_index;
  // Rows from top-k ids (streaming kernels only; offsets, row_index and
  // out_index are then null): expert e's rows are the routed rows r with
  // ids[r] == e, in increasing r; the activation row of r is x[r / kslots]
  // and its output row is r.  R = T * k routed rows, at most kIdsMaxRows.
  const int32_t* ids;
  int32_t kslots;
  // Rows from the router logits [R / kslots][E] instead (decode workgroups of
  // gated matmuls only, see gemm_skinny_takes_logits): the routed rows are
  // those of the top-k ids, which the call writes to ids_out and the softmax
  // weights to wts_out ([R], slot order), as the routing kernel would.
  const float* logits;
  int32_t* ids_out;
  float* wts_out;
};

// Most routed rows of an ids-mode call (an expert holds at most T of them).
constexpr int kIdsMaxRows = 4096;
constexpr int kIdsMaxExpertRows = 256;

void launch_gemm_skinny(const GemmArgs& a, hipStream_t stream);
// true when launch_gemm_skinny(a) can take its rows from router logits
// [T][E] at `logits` (a gated matmul on the one-tile streaming kernel,
// T <= 64, E <= 128)
bool gemm_skinny_takes_logits(const GemmArgs& a, int64_t T, const float* logits);
bool gemm_tiled_supported(const GemmArgs& a);
size_t gemm_tiled_workspace(int64_t x_rows, int64_t R, int32_t E, int64_t K, int64_t N);
void launch_gemm_tiled(const GemmArgs& a, void* ws, hipStream_t stream);
bool gemm_short_supported(const GemmArgs& a);
void launch_gemm_short(const GemmArgs& a, hipStream_t stream);
bool gemm_splitk_supported(const GemmArgs& a);
size_t gemm_splitk_workspace(int64_t R, int64_t K, int64_t N);
// false when one kernel does the whole call (K <= 4096): no workspace is used
bool gemm_splitk_needs_workspace(const GemmArgs& a);
void launch_gemm_splitk(const GemmArgs& a, void* ws, hipStream_t stream);

size_t route_workspace_bytes(int64_t T, int32_t E, int32_t k);
void launch_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids, float* weights,
                  int32_t* offsets, int32_t* sorted_rows, int32_t* sorted_tokens, int32_t* row_to_sorted,
                  void* ws, hipStream_t stream);
void launch_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids, float* weights,
                 hipStream_t stream);

// row_to_sorted null: the rows of token t are o[t*k + j]
void launch_combine(const void* o, int32_t o_dtype, const int32_t* row_to_sorted, const float* w,
                    int64_t T, int32_t k, int64_t N, uint16_t* y, hipStream_t stream);

// FP8 (W8A8, E4M3) grouped matmul arguments (dense: E = 1, no offsets).
struct Fp8Args {
  const uint8_t* xq;         // [x_rows][K] E4M3 codes
  const float* xs;           // [x_rows] row scales
  int64_t x_rows;
  const int32_t* row_index;  // nullable, [R]
  const int32_t* offsets;    // nullable, [E+1]
  int32_t E;
  int64_t R, K, N;
  const uint8_t* wq;         // [E][N][K] E4M3 codes
  const float* ws;           // [E][N] row scales
  int32_t epilogue;
  void* out;                 // [R][N] (gated: [R][N/2]) at the sorted rows
  int32_t out_dtype;
};

// Rows per expert up to which the FP8 matmul streams weights (else 128-row tiles).
constexpr int kFp8StreamRowsPerExpert = 32;

bool fp8_gemm_supported(const Fp8Args& a);
void launch_fp8_gemm(const Fp8Args& a, hipStream_t stream);
void launch_fp8_quant_rows(const uint16_t* x, int64_t rows, int64_t K, uint8_t* q, float* scale, hipStream_t stream);

}  // namespace w4
