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
// of that expert's activation rows, 16 rows per MFMA tile.  KSPLIT waves take
// the full 4-group tile16 blocks of the tile round-robin (wave w: blocks w,
// w+KSPLIT, ...), so together they read the tile front to back.
//
// Each wave first issues the loads of ALL its code blocks (one 128-bit load per
// lane per 1 KiB block, at most kMaxBlocksPerWave of them) so that many bytes
// are in flight, while the workgroup stages the tile's bf16 scales in LDS.
// Then, per block: four 16x16x32 bf16 MFMAs per weight tile, one per group,
// each into a zeroed accumulator, whose fp32 partial sums are scaled by the
// group scale and added up.  Codes enter the MFMA as q/16 (exact); the
// epilogue multiplies by 16.  Activation fragments are loaded one block ahead.
// The main loop has no per-lane branches: invalid activation rows are pointed
// at a valid row and their (unused) results are never stored.

#include "common.h"
#include "internal.h"
#include "w4a16.h"

namespace w4 {

namespace {

// Code blocks a wave keeps in registers (1 KiB of codes per weight tile each),
// and the occupancy the register allocation aims for (waves per SIMD).
#ifndef W4_SKINNY_BLOCKS_PER_WAVE
#define W4_SKINNY_BLOCKS_PER_WAVE 6
#endif
#ifndef W4_SKINNY_WAVES_PER_SIMD
#define W4_SKINNY_WAVES_PER_SIMD 3
#endif
constexpr int kMaxBlocksPerWave = W4_SKINNY_BLOCKS_PER_WAVE;

__device__ __forceinline__ float gelu_tanh_f32(float x) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * x * (1.0f + tanhf(c * (x + 0.044715f * x * x * x)));
}

__device__ __forceinline__ float silu_f32(float x) { return x / (1.0f + expf(-x)); }

// blockIdx -> work item so that consecutive items land on the same XCD
// (workgroups are dealt to the 8 XCDs round-robin).
__device__ __forceinline__ int xcd_item(int b, int total) {
  const int xcd = b & 7, idx = b >> 3;
  const int per = total >> 3, rem = total & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int KSPLIT, int MAXT, int EPI, int OUT>
__global__ void __launch_bounds__(64 * KSPLIT) __attribute__((amdgpu_waves_per_eu(W4_SKINNY_WAVES_PER_SIMD)))
skinny_kernel(GemmArgs a, int items_per_expert, int total_items) {
  constexpr bool GATED = EPI != W4_EPI_NONE;
  constexpr int NW = GATED ? 2 : 1;
  constexpr int NBW = kMaxBlocksPerWave;
  extern __shared__ __align__(16) uint8_t smem[];

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
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int c = lane >> 4;
  const int64_t K = a.K, N = a.N;
  const int G = (int)(K / kGroup);
  const int NBF = G / kBlockGroups;          // full 4-group blocks
  const int gtail = G - NBF * kBlockGroups;  // groups in the last, partial block
  const int GP = (G + 3) & ~3;               // LDS row stride of the scales
  const int nbw = wv < NBF ? (NBF - wv + KSPLIT - 1) / KSPLIT : 0;
  const bool tail_here = gtail > 0 && wv == NBF % KSPLIT;

  const uint8_t* wbase[NW];
  const uint16_t* stile[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int64_t tile = GATED ? (nt + w * (N / 32)) : nt;   // the up tile sits N/2 rows below
    wbase[w] = a.qweight + (int64_t)e * (N * K / 2) + tile * 8 * K;
    stile[w] = a.scales + ((int64_t)e * N + tile * kTileRows) * G;
  }

  // Rounds of up to NBW blocks: round q holds this wave's blocks
  // wv + KSPLIT*(q*NBW + i), i < NBW.  Codes of a round live in registers;
  // after block i of a round is used, block i of the next round is loaded into
  // the same registers (a rolling prefetch).
  const int nrounds = (nbw + NBW - 1) / NBW;
  auto round_blocks = [&](int q) { const int left = nbw - q * NBW; return left < NBW ? left : NBW; };
  auto code_ptr = [&](int w, int q, int i) {
    return reinterpret_cast<const u32x4*>(wbase[w] + 1024 * (wv + KSPLIT * (q * NBW + i)) + 16 * lane);
  };

  // 1. the first round's code loads, before anything else
  u32x4 cw[NBW][NW];
  {
    const int nb0 = nrounds > 0 ? round_blocks(0) : 0;
#pragma unroll
    for (int i = 0; i < NBW; ++i)
#pragma unroll
      for (int w = 0; w < NW; ++w)
        if (i < nb0) cw[i][w] = *code_ptr(w, 0, i);
  }
  uint32_t ct[NW][3] = {};
  if (tail_here) {
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (j < gtail)
          ct[w][j] = *reinterpret_cast<const uint32_t*>(wbase[w] + 1024 * NBF + 4 * gtail * lane + 4 * j);
  }

  // 2. the tiles' scales -> LDS, rows padded to a multiple of 4 groups
  uint16_t* ss = reinterpret_cast<uint16_t*>(smem);
  for (int idx = threadIdx.x; idx < NW * 16 * G; idx += 64 * KSPLIT) {
    const int w = idx / (16 * G);
    const int rem = idx - w * 16 * G;
    const int rr = rem / G;
    const int g = rem - rr * G;
    ss[(w * 16 + rr) * GP + g] = stile[w][rem];
  }
  f32x4* red = reinterpret_cast<f32x4*>(smem + ((NW * 16 * GP * 2 + 15) & ~15));
  __syncthreads();

  for (int64_t row0 = row_begin; row0 < row_end; row0 += 16 * MAXT) {
    const int64_t left = row_end - row0;
    const int ntt = left >= 16 * MAXT ? MAXT : (int)((left + 15) / 16);
    const bool more_passes = row0 + 16 * MAXT < row_end;

    const uint16_t* xrow[MAXT];
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt) {
      int64_t rr = row0 + 16 * tt + r;        // A operand row = lane % 16
      if (rr >= row_end) rr = row_begin;      // padding rows read a valid row; never stored
      const int64_t src = a.row_index ? (int64_t)a.row_index[rr] : rr;
      xrow[tt] = a.x + src * K + 8 * c;
    }

    f32x4 acc[MAXT][NW];
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt)
#pragma unroll
      for (int w = 0; w < NW; ++w) acc[tt][w] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int q = 0; q < nrounds; ++q) {
      const int nb = round_blocks(q);
      // the round whose codes go into the registers freed during this one
      const int qn = q + 1 < nrounds ? q + 1 : ((more_passes && nrounds > 1) ? 0 : -1);
      const int nbn = qn >= 0 ? round_blocks(qn) : 0;

      u32x4 A[MAXT][4];
#pragma unroll
      for (int tt = 0; tt < MAXT; ++tt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (tt < ntt) A[tt][j] = *reinterpret_cast<const u32x4*>(xrow[tt] + (int64_t)((wv + KSPLIT * q * NBW) * 4 + j) * kGroup);

#pragma unroll
      for (int i = 0; i < NBW; ++i) {
        if (i < nb) {
          const int b = wv + KSPLIT * (q * NBW + i);
          u32x4 An[MAXT][4];
          if (i + 1 < nb) {
#pragma unroll
            for (int tt = 0; tt < MAXT; ++tt)
#pragma unroll
              for (int j = 0; j < 4; ++j)
                if (tt < ntt)
                  An[tt][j] = *reinterpret_cast<const u32x4*>(xrow[tt] + (int64_t)((b + KSPLIT) * 4 + j) * kGroup);
          }
          float sc[NW][4];
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            const u32x2 sv = *reinterpret_cast<const u32x2*>(ss + (w * 16 + r) * GP + 4 * b);
            sc[w][0] = bf16_to_f32(sv[0] & 0xFFFFu);
            sc[w][1] = bf16_to_f32(sv[0] >> 16);
            sc[w][2] = bf16_to_f32(sv[1] & 0xFFFFu);
            sc[w][3] = bf16_to_f32(sv[1] >> 16);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            bf16x8 B[NW];
#pragma unroll
            for (int w = 0; w < NW; ++w) B[w] = unpack8_div16(cw[i][w][j]);
#pragma unroll
            for (int tt = 0; tt < MAXT; ++tt) {
              if (tt < ntt) {
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                  const f32x4 p = mfma16x16x32(as_bf16x8(A[tt][j]), B[w], f32x4{0.f, 0.f, 0.f, 0.f});
                  acc[tt][w] += sc[w][j] * p;
                }
              }
            }
          }
          if (i < nbn) {
#pragma unroll
            for (int w = 0; w < NW; ++w) cw[i][w] = *code_ptr(w, qn, i);
          }
          if (i + 1 < nb) {
#pragma unroll
            for (int tt = 0; tt < MAXT; ++tt)
#pragma unroll
              for (int j = 0; j < 4; ++j) A[tt][j] = An[tt][j];
          }
        }
      }
    }

    if (tail_here) {
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        if (j < gtail) {
          const int g = NBF * 4 + j;
          float sc[NW];
          bf16x8 B[NW];
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            sc[w] = bf16_to_f32(ss[(w * 16 + r) * GP + g]);
            B[w] = unpack8_div16(ct[w][j]);
          }
#pragma unroll
          for (int tt = 0; tt < MAXT; ++tt) {
            if (tt < ntt) {
              const u32x4 At = *reinterpret_cast<const u32x4*>(xrow[tt] + (int64_t)g * kGroup);
#pragma unroll
              for (int w = 0; w < NW; ++w) {
                const f32x4 p = mfma16x16x32(as_bf16x8(At), B[w], f32x4{0.f, 0.f, 0.f, 0.f});
                acc[tt][w] += sc[w] * p;
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
          const int64_t row = row0 + 16 * tt + 4 * c + i;   // D rows = 4*(lane/16)+i, column = lane%16
          if (row >= row_end) continue;
          const int64_t col = (int64_t)nt * kTileRows + r;
          if constexpr (GATED) {
            const float g = bf16_to_f32(f32_to_bf16(acc[tt][0][i] * 16.0f));
            const float u = bf16_to_f32(f32_to_bf16(acc[tt][1][i] * 16.0f));
            const float act = (EPI == W4_EPI_GEGLU_TANH) ? gelu_tanh_f32(g) : silu_f32(g);
            static_cast<uint16_t*>(a.out)[row * (N / 2) + col] = (uint16_t)f32_to_bf16(act * u);
          } else {
            const float v = acc[tt][0][i] * 16.0f;
            if constexpr (OUT == W4_OUT_F32) static_cast<float*>(a.out)[row * N + col] = v;
            else static_cast<uint16_t*>(a.out)[row * N + col] = (uint16_t)f32_to_bf16(v);
          }
        }
      }
    }
  }
}

size_t smem_bytes(int NW, int G, int KSPLIT, int MAXT) {
  const size_t GP = (size_t)((G + 3) & ~3);
  const size_t scales = ((size_t)NW * 16 * GP * 2 + 15) & ~(size_t)15;
  const size_t red = KSPLIT > 1 ? (size_t)(KSPLIT - 1) * MAXT * NW * 64 * 16 : 0;
  return scales + red;
}

template <int KSPLIT, int MAXT>
void launch_k(const GemmArgs& a, hipStream_t stream) {
  const bool gated = a.epilogue != W4_EPI_NONE;
  const int NW = gated ? 2 : 1;
  const int items_per_expert = (int)(gated ? a.N / 32 : a.N / 16);
  const int total = items_per_expert * a.E;
  const size_t smem = smem_bytes(NW, (int)(a.K / kGroup), KSPLIT, MAXT);
  dim3 grid(total), block(64 * KSPLIT);
  if (a.epilogue == W4_EPI_GEGLU_TANH)
    hipLaunchKernelGGL((skinny_kernel<KSPLIT, MAXT, W4_EPI_GEGLU_TANH, W4_OUT_BF16>), grid, block, smem, stream, a,
                       items_per_expert, total);
  else if (a.epilogue == W4_EPI_SWIGLU)
    hipLaunchKernelGGL((skinny_kernel<KSPLIT, MAXT, W4_EPI_SWIGLU, W4_OUT_BF16>), grid, block, smem, stream, a,
                       items_per_expert, total);
  else if (a.out_dtype == W4_OUT_F32)
    hipLaunchKernelGGL((skinny_kernel<KSPLIT, MAXT, W4_EPI_NONE, W4_OUT_F32>), grid, block, smem, stream, a,
                       items_per_expert, total);
  else
    hipLaunchKernelGGL((skinny_kernel<KSPLIT, MAXT, W4_EPI_NONE, W4_OUT_BF16>), grid, block, smem, stream, a,
                       items_per_expert, total);
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
  const int64_t NBF = (a.K / kGroup) / kBlockGroups;
  // rows per expert on average decides how many 16-row MFMA tiles stay in registers
  const int64_t avg = (a.R + a.E - 1) / a.E;
  const int maxt = avg <= 12 ? 1 : (avg <= 28 ? 2 : 4);
  // each wave holds at most kMaxBlocksPerWave blocks; then add waves while the
  // grid is small and every wave still gets at least two blocks
  int ks = 1;
  while (ks < 8 && (NBF + ks - 1) / ks > kMaxBlocksPerWave) ks *= 2;
  while (ks < 8 && items * ks < 8192 && NBF >= 4 * ks) ks *= 2;
  switch (ks) {
    case 1: launch_ks<1>(a, maxt, stream); break;
    case 2: launch_ks<2>(a, maxt, stream); break;
    case 4: launch_ks<4>(a, maxt, stream); break;
    default: launch_ks<8>(a, maxt, stream); break;
  }
}

}  // namespace w4
