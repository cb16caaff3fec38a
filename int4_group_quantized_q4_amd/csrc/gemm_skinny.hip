// Decode-shaped W4A16 matmul: few activation rows per expert, weight-streaming.
//
// [RQ] "Repacked QAT Gemma 4 26B-A4B serves on one TPU v6e at 1.9x FP8
// throughput", section "What changed in vLLM's TPU backend": the grouped
// matmul takes one scale per 32-wide group and dequantizes each weight tile on
// chip before the multiply; activations stay bf16.  "What quantization really
// is", section "Why the tip exists": generation rereads the weights token by
// token, so this kernel is bound by the weight bytes it streams.
//
// One workgroup = one work item = one 16-row weight tile (two for a gated
// epilogue: the gate tile and the matching up tile) of one expert, against all
// of that expert's activation rows, 16 rows per MFMA tile.  KSPLIT waves split
// the K blocks of the tile round-robin, so together they read the tile's bytes
// front to back; each wave reads one 1 KiB tile16 block per weight tile with a
// single 128-bit load per lane, unpacks the nibbles in registers, runs one
// 16x16x32 bf16 MFMA per group into a zeroed accumulator and adds the group's
// partial sums, scaled by the bf16 group scale, into an fp32 accumulator.
// The codes enter the MFMA as q/16 (exact); the epilogue multiplies by 16.

#include "common.h"
#include "internal.h"
#include "w4a16.h"

namespace w4 {

namespace {

__device__ __forceinline__ float gelu_tanh_f32(float x) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * x * (1.0f + tanhf(c * (x + 0.044715f * x * x * x)));
}

__device__ __forceinline__ float silu_f32(float x) { return x / (1.0f + expf(-x)); }

// blockIdx -> work item so that consecutive items land on the same XCD
// (blocks are dealt to the 8 XCDs round-robin).
__device__ __forceinline__ int xcd_item(int b, int total) {
  const int xcd = b & 7, idx = b >> 3;
  const int per = total >> 3, rem = total & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

template <int KSPLIT, int MAXT, int EPI, int OUT>
__global__ void __launch_bounds__(64 * KSPLIT) skinny_kernel(GemmArgs a, int items_per_expert,
                                                             int total_items) {
  constexpr bool GATED = EPI != W4_EPI_NONE;
  constexpr int NW = GATED ? 2 : 1;
  const int item = xcd_item(blockIdx.x, total_items);
  const int e = item / items_per_expert;
  const int nt = item - e * items_per_expert;
  int64_t row_begin = 0, row_end = a.R;
  if (a.offsets) {
    row_begin = a.offsets[e];
    row_end = a.offsets[e + 1];
  }
  if (row_begin >= row_end) return;

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int r = lane & 15;
  const int c = lane >> 4;
  const int64_t K = a.K, N = a.N;
  const int64_t G = K / kGroup;
  const int64_t NB = (G + kBlockGroups - 1) / kBlockGroups;

  const uint8_t* wbase[NW];
  const uint16_t* sbase[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int64_t tile = GATED ? (nt + w * (N / 32)) : nt;   // up tile sits N/2 rows below
    wbase[w] = a.qweight + (int64_t)e * (N * K / 2) + tile * 8 * K;
    sbase[w] = a.scales + ((int64_t)e * N + tile * kTileRows + r) * G;
  }

  __shared__ f32x4 red[(KSPLIT > 1) ? (KSPLIT - 1) * MAXT * NW * 64 : 1];

  for (int64_t row0 = row_begin; row0 < row_end; row0 += 16 * MAXT) {
    const int64_t rows_here = row_end - row0 < 16 * MAXT ? row_end - row0 : 16 * MAXT;
    const int ntt = (int)((rows_here + 15) / 16);

    const uint16_t* xrow[MAXT];
    bool xvalid[MAXT];
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt) {
      const int64_t rr = row0 + 16 * tt + r;     // A operand row = lane % 16
      xvalid[tt] = rr < row_end;
      const int64_t src = xvalid[tt] ? (a.row_index ? (int64_t)a.row_index[rr] : rr) : 0;
      xrow[tt] = a.x + src * K + 8 * c;
    }

    f32x4 acc[MAXT][NW];
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt)
#pragma unroll
      for (int w = 0; w < NW; ++w) acc[tt][w] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int64_t b = wv; b < NB; b += KSPLIT) {
      const int64_t rem = G - b * kBlockGroups;
      const int gb = rem < kBlockGroups ? (int)rem : kBlockGroups;
      uint32_t cw[NW][4];
      float sc[NW][4];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        if (gb == 4) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(wbase[w] + 1024 * b + 16 * lane);
          cw[w][0] = v[0]; cw[w][1] = v[1]; cw[w][2] = v[2]; cw[w][3] = v[3];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            cw[w][j] = j < gb ? *reinterpret_cast<const uint32_t*>(wbase[w] + 1024 * b + 4 * gb * lane + 4 * j) : 0u;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[w][j] = j < gb ? bf16_to_f32(sbase[w][b * kBlockGroups + j]) : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j < gb) {
          bf16x8 B[NW];
#pragma unroll
          for (int w = 0; w < NW; ++w) B[w] = unpack8_div16(cw[w][j]);
          const int64_t kofs = (b * kBlockGroups + j) * kGroup;
#pragma unroll
          for (int tt = 0; tt < MAXT; ++tt) {
            if (tt < ntt) {
              bf16x8 A;
              if (xvalid[tt]) {
                A = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xrow[tt] + kofs));
              } else {
                A = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
              }
#pragma unroll
              for (int w = 0; w < NW; ++w) {
                const f32x4 p = mfma16x16x32(A, B[w], f32x4{0.f, 0.f, 0.f, 0.f});
                acc[tt][w] += sc[w][j] * p;
              }
            }
          }
        }
      }
    }

    if (KSPLIT > 1) {
      if (wv > 0) {
#pragma unroll
        for (int tt = 0; tt < MAXT; ++tt)
#pragma unroll
          for (int w = 0; w < NW; ++w) red[(((wv - 1) * MAXT + tt) * NW + w) * 64 + lane] = acc[tt][w];
      }
      __syncthreads();
      if (wv == 0) {
        for (int s = 1; s < KSPLIT; ++s)
#pragma unroll
          for (int tt = 0; tt < MAXT; ++tt)
#pragma unroll
            for (int w = 0; w < NW; ++w) acc[tt][w] += red[(((s - 1) * MAXT + tt) * NW + w) * 64 + lane];
      }
      __syncthreads();
    }

    if (wv == 0) {
#pragma unroll
      for (int tt = 0; tt < MAXT; ++tt) {
        if (tt >= ntt) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t row = row0 + 16 * tt + 4 * c + i;   // D rows = 4*(lane/16)+i
          if (row >= row_end) continue;
          if constexpr (GATED) {
            const float g = bf16_to_f32(f32_to_bf16(acc[tt][0][i] * 16.0f));
            const float u = bf16_to_f32(f32_to_bf16(acc[tt][1][i] * 16.0f));
            const float act = (EPI == W4_EPI_GEGLU_TANH) ? gelu_tanh_f32(g) : silu_f32(g);
            const int64_t col = (int64_t)nt * kTileRows + r;
            static_cast<uint16_t*>(a.out)[row * (N / 2) + col] = (uint16_t)f32_to_bf16(act * u);
          } else {
            const float v = acc[tt][0][i] * 16.0f;
            const int64_t col = (int64_t)nt * kTileRows + r;
            if constexpr (OUT == W4_OUT_F32) static_cast<float*>(a.out)[row * N + col] = v;
            else static_cast<uint16_t*>(a.out)[row * N + col] = (uint16_t)f32_to_bf16(v);
          }
        }
      }
    }
  }
}

template <int KSPLIT, int MAXT>
void launch_k(const GemmArgs& a, hipStream_t stream) {
  const bool gated = a.epilogue != W4_EPI_NONE;
  const int items_per_expert = (int)(gated ? a.N / 32 : a.N / 16);
  const int total = items_per_expert * a.E;
  dim3 grid(total), block(64 * KSPLIT);
  if (a.epilogue == W4_EPI_GEGLU_TANH)
    hipLaunchKernelGGL((skinny_kernel<KSPLIT, MAXT, W4_EPI_GEGLU_TANH, W4_OUT_BF16>), grid, block, 0, stream, a, items_per_expert, total);
  else if (a.epilogue == W4_EPI_SWIGLU)
    hipLaunchKernelGGL((skinny_kernel<KSPLIT, MAXT, W4_EPI_SWIGLU, W4_OUT_BF16>), grid, block, 0, stream, a, items_per_expert, total);
  else if (a.out_dtype == W4_OUT_F32)
    hipLaunchKernelGGL((skinny_kernel<KSPLIT, MAXT, W4_EPI_NONE, W4_OUT_F32>), grid, block, 0, stream, a, items_per_expert, total);
  else
    hipLaunchKernelGGL((skinny_kernel<KSPLIT, MAXT, W4_EPI_NONE, W4_OUT_BF16>), grid, block, 0, stream, a, items_per_expert, total);
}

template <int KSPLIT>
void launch_ks(const GemmArgs& a, int maxt, hipStream_t stream) {
  if (maxt <= 1) launch_k<KSPLIT, 1>(a, stream);
  else if (maxt == 2) launch_k<KSPLIT, 2>(a, stream);
  else launch_k<KSPLIT, 4>(a, stream);
}

}  // namespace

void launch_gemm_skinny(const GemmArgs& a, hipStream_t stream) {
  const bool gated = a.epilogue != W4_EPI_NONE;
  const int64_t items = (gated ? a.N / 32 : a.N / 16) * a.E;
  const int64_t G = a.K / kGroup;
  const int64_t NB = (G + kBlockGroups - 1) / kBlockGroups;
  // rows per expert on average decides how many 16-row MFMA tiles stay in registers
  const int64_t avg = (a.R + a.E - 1) / a.E;
  const int maxt = avg <= 12 ? 1 : (avg <= 28 ? 2 : 4);
  // enough waves in flight to cover HBM latency: aim for >= 8192 waves
  int ks = 1;
  while (ks < 8 && items * ks < 8192 && NB >= 2 * ks * 2) ks *= 2;
  switch (ks) {
    case 1: launch_ks<1>(a, maxt, stream); break;
    case 2: launch_ks<2>(a, maxt, stream); break;
    case 4: launch_ks<4>(a, maxt, stream); break;
    default: launch_ks<8>(a, maxt, stream); break;
  }
}

}  // namespace w4
