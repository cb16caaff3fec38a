// Decode-shaped W4A16 matmul: few activation rows per expert, weight-streaming.
//
// [RQ] "Repacked QAT Gemma 4 26B-A4B serves on one TPU v6e at 1.9x FP8
// throughput", section "What changed in vLLM's TPU backend": the grouped
// matmul takes one scale per 32-wide group and dequantizes each weight tile on
// chip before the multiply; activations stay bf16.  "What quantization really
// is", section "Why the tip exists": generation rereads the weights token by
// token, so this kernel is bound by the weight bytes it streams.
//
// Work split: a workgroup of 4 waves serves 4 consecutive work items of one
// expert; a work item is one 16-row weight tile (two with a gated epilogue:
// the gate tile and the matching up tile), and its wave streams that tile over
// the whole K.  The expert's activation rows are staged in LDS chunk by chunk
// (shared by the 4 waves); the codes and scales of each wave's blocks come
// straight from global memory through a ring of kPrefetch blocks held in
// registers (one 128-bit load per lane per 1 KiB tile16 block).
//
// Per 4-group block and weight tile: the nibbles become bf16 136+q with one
// shift and one and-or per pair (biased_pairs); a first MFMA against a
// constant -136 operand gives -136*sum(x) per row and group, and is the
// accumulator input of the MFMAs against the biased codes, so each group's
// partial sum sum(x*q) comes out of the matrix core; the VALU then adds
// scale * partial into the fp32 accumulator.  Rows beyond the expert's count
// read a valid row and their results are never stored.

#include "common.h"
#include "internal.h"
#include "w4a16.h"

namespace w4 {

namespace {

// Code/scale blocks in flight per wave, waves (work items) per workgroup, and
// the occupancy (waves per SIMD) the register allocation aims for (0: none).
#ifndef W4_DECODE_PREFETCH
#define W4_DECODE_PREFETCH 4
#endif
#ifndef W4_DECODE_WAVES
#define W4_DECODE_WAVES 4
#endif
#ifndef W4_DECODE_WAVES_PER_SIMD
#define W4_DECODE_WAVES_PER_SIMD 0
#endif
constexpr int kPrefetch = W4_DECODE_PREFETCH;
constexpr int kWaves = W4_DECODE_WAVES;
#if W4_DECODE_WAVES_PER_SIMD > 0
#define W4_DECODE_OCC __attribute__((amdgpu_waves_per_eu(W4_DECODE_WAVES_PER_SIMD)))
#else
#define W4_DECODE_OCC
#endif

__device__ __forceinline__ float gelu_tanh_f32(float x) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * x * (1.0f + tanhf(c * (x + 0.044715f * x * x * x)));
}

__device__ __forceinline__ float silu_f32(float x) { return x / (1.0f + expf(-x)); }

// blockIdx -> workgroup index so that consecutive indices (the same expert)
// land on the same XCD (workgroups are dealt to the 8 XCDs round-robin).
__device__ __forceinline__ int xcd_item(int b, int total) {
  const int xcd = b & 7, idx = b >> 3;
  const int per = total >> 3, rem = total & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int MAXT, int EPI, int OUT>
__global__ void __launch_bounds__(64 * kWaves) W4_DECODE_OCC decode_kernel(GemmArgs a, int wg_per_expert,
                                                                           int total_wg, int items_per_expert) {
  constexpr bool GATED = EPI != W4_EPI_NONE;
  constexpr int NW = GATED ? 2 : 1;
  constexpr int D = kPrefetch;
  constexpr int KCB = (8 / MAXT) > D ? (8 / MAXT) : D;   // blocks per staged activation chunk
  constexpr int KC = KCB * 128;          // columns per chunk
  constexpr int XS = KC * 2 + 16;        // LDS row stride in bytes (padded off the bank period)
  static_assert(KCB % D == 0, "chunk must hold whole prefetch rounds");
  __shared__ __align__(16) uint8_t xs[16 * MAXT * XS];

  const int wg = xcd_item(blockIdx.x, total_wg);
  const int e = wg / wg_per_expert;
  const int wgi = wg - e * wg_per_expert;
  int64_t row_begin = 0, row_end = a.R;
  if (a.offsets) {
    row_begin = a.offsets[e];
    row_end = a.offsets[e + 1];
  }
  if (row_begin >= row_end) return;   // the whole workgroup leaves together

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nt = wgi * kWaves + wv;
  const bool active = nt < items_per_expert;   // idle waves still stage and sync
  const int r = lane & 15;
  const int c = lane >> 4;
  const int64_t K = a.K, N = a.N;
  const int G = (int)(K / kGroup);
  const int NBF = G / kBlockGroups;
  const int gtail = G - NBF * kBlockGroups;
  const int NBall = NBF + (gtail > 0 ? 1 : 0);

  const uint8_t* wb[NW];
  const uint16_t* sb[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int64_t tile = active ? (GATED ? (nt + w * (N / 32)) : nt) : 0;   // up tile: N/2 rows below
    wb[w] = a.qweight + (int64_t)e * (N * K / 2) + tile * 8 * K;
    sb[w] = a.scales + ((int64_t)e * N + tile * kTileRows) * G;            // the tile's tile16 scales
  }

  u32x4 cw[D][NW];
  u32x2 sw[D][NW];
  auto load_block = [&](int slot, int b) __attribute__((always_inline)) {
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      cw[slot][w] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wb[w] + 1024 * (int64_t)b + 16 * lane));
      sw[slot][w] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(sb[w] + 64 * (int64_t)b + 4 * r));
    }
  };

  // the partial last block (1..3 groups), loaded once
  uint32_t ct[NW][3] = {};
  float st[NW][3] = {};
  if (active && gtail > 0) {
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (j < gtail) {
          ct[w][j] = *reinterpret_cast<const uint32_t*>(wb[w] + 1024 * (int64_t)NBF + 4 * gtail * lane + 4 * j);
          st[w][j] = bf16_to_f32(sb[w][64 * (int64_t)NBF + r * gtail + j]);
        }
  }

  const u32x4 neg136 = {kNeg136Pair, kNeg136Pair, kNeg136Pair, kNeg136Pair};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  for (int64_t row0 = row_begin; row0 < row_end; row0 += 16 * MAXT) {
    const int cnt = (int)(row_end - row0 < 16 * MAXT ? row_end - row0 : 16 * MAXT);
    const int ntt = (cnt + 15) >> 4;

    if (active) {
#pragma unroll
      for (int i = 0; i < D; ++i)
        if (i < NBF) load_block(i, i);
    }

    int arow[MAXT];   // LDS row of this lane's A operand (padding rows read row 0)
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt) arow[tt] = (16 * tt + r < cnt) ? 16 * tt + r : 0;

    f32x4 acc[MAXT][NW];
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt)
#pragma unroll
      for (int w = 0; w < NW; ++w) acc[tt][w] = zero4;

    for (int ch = 0; ch * KCB < NBall; ++ch) {
      // stage activation rows [row0, row0+cnt) x columns [ch*KC, ch*KC + ncol) in LDS
      __syncthreads();
      const int col0 = ch * KC;
      const int ncol = (int)(K - col0 < KC ? K - col0 : KC);
      const int ppr = ncol >> 3;   // 16-byte pieces per row
      for (int p = threadIdx.x; p < cnt * ppr; p += 64 * kWaves) {
        const int rr = p / ppr;
        const int pc = p - rr * ppr;
        const int64_t src = a.row_index ? (int64_t)a.row_index[row0 + rr] : row0 + rr;
        *reinterpret_cast<u32x4*>(xs + rr * XS + pc * 16) =
            *reinterpret_cast<const u32x4*>(a.x + src * K + col0 + pc * 8);
      }
      __syncthreads();
      if (!active) continue;

#pragma unroll
      for (int lb = 0; lb < KCB; ++lb) {
        const int b = ch * KCB + lb;
        if (b < NBF) {
          const int slot = lb % D;
          bf16x8 A[MAXT][4];
          f32x4 Cb[MAXT][4];
#pragma unroll
          for (int tt = 0; tt < MAXT; ++tt)
            if (tt < ntt) {
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                A[tt][j] = *reinterpret_cast<const bf16x8*>(xs + arow[tt] * XS + (lb * 4 + j) * 64 + c * 16);
                Cb[tt][j] = mfma16x16x32(A[tt][j], as_bf16x8(neg136), zero4);
              }
            }
          f32x4 P[MAXT][NW][4];
#pragma unroll
          for (int w = 0; w < NW; ++w) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const bf16x8 B = as_bf16x8(biased_pairs(cw[slot][w][j]));
#pragma unroll
              for (int tt = 0; tt < MAXT; ++tt)
                if (tt < ntt) P[tt][w][j] = mfma16x16x32(A[tt][j], B, Cb[tt][j]);
            }
          }
          float sc[NW][4];
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            sc[w][0] = bf16_to_f32(sw[slot][w][0] & 0xFFFFu);
            sc[w][1] = bf16_to_f32(sw[slot][w][0] >> 16);
            sc[w][2] = bf16_to_f32(sw[slot][w][1] & 0xFFFFu);
            sc[w][3] = bf16_to_f32(sw[slot][w][1] >> 16);
          }
          if (b + D < NBF) load_block(slot, b + D);
#pragma unroll
          for (int tt = 0; tt < MAXT; ++tt)
            if (tt < ntt) {
#pragma unroll
              for (int w = 0; w < NW; ++w)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[tt][w] += sc[w][j] * P[tt][w][j];
            }
        }
      }

      if (gtail > 0 && ch == (NBall - 1) / KCB) {
        const int lb = NBF - ch * KCB;   // local index of the partial block
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          if (j < gtail) {
#pragma unroll
            for (int tt = 0; tt < MAXT; ++tt)
              if (tt < ntt) {
                const bf16x8 At = *reinterpret_cast<const bf16x8*>(xs + arow[tt] * XS + (lb * 4 + j) * 64 + c * 16);
                const f32x4 cb = mfma16x16x32(At, as_bf16x8(neg136), zero4);
#pragma unroll
                for (int w = 0; w < NW; ++w) {
                  const f32x4 p = mfma16x16x32(At, as_bf16x8(biased_pairs(ct[w][j])), cb);
                  acc[tt][w] += st[w][j] * p;
                }
              }
          }
        }
      }
    }

    if (active) {
#pragma unroll
      for (int tt = 0; tt < MAXT; ++tt) {
        if (tt >= ntt) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t row = row0 + 16 * tt + 4 * c + i;   // D rows = 4*(lane/16)+i, column = lane%16
          if (row >= row_end) continue;
          const int64_t col = (int64_t)nt * kTileRows + r;
          if constexpr (GATED) {
            const float g = bf16_to_f32(f32_to_bf16(acc[tt][0][i]));
            const float u = bf16_to_f32(f32_to_bf16(acc[tt][1][i]));
            const float act = (EPI == W4_EPI_GEGLU_TANH) ? gelu_tanh_f32(g) : silu_f32(g);
            static_cast<uint16_t*>(a.out)[row * (N / 2) + col] = (uint16_t)f32_to_bf16(act * u);
          } else {
            const float v = acc[tt][0][i];
            if constexpr (OUT == W4_OUT_F32) static_cast<float*>(a.out)[row * N + col] = v;
            else static_cast<uint16_t*>(a.out)[row * N + col] = (uint16_t)f32_to_bf16(v);
          }
        }
      }
    }
  }
}

template <int MAXT>
void launch_m(const GemmArgs& a, hipStream_t stream) {
  const bool gated = a.epilogue != W4_EPI_NONE;
  const int items_per_expert = (int)(gated ? a.N / 32 : a.N / 16);
  const int wg_per_expert = (items_per_expert + kWaves - 1) / kWaves;
  const int total = wg_per_expert * a.E;
  dim3 grid(total), block(64 * kWaves);
  if (a.epilogue == W4_EPI_GEGLU_TANH)
    hipLaunchKernelGGL((decode_kernel<MAXT, W4_EPI_GEGLU_TANH, W4_OUT_BF16>), grid, block, 0, stream, a,
                       wg_per_expert, total, items_per_expert);
  else if (a.epilogue == W4_EPI_SWIGLU)
    hipLaunchKernelGGL((decode_kernel<MAXT, W4_EPI_SWIGLU, W4_OUT_BF16>), grid, block, 0, stream, a,
                       wg_per_expert, total, items_per_expert);
  else if (a.out_dtype == W4_OUT_F32)
    hipLaunchKernelGGL((decode_kernel<MAXT, W4_EPI_NONE, W4_OUT_F32>), grid, block, 0, stream, a,
                       wg_per_expert, total, items_per_expert);
  else
    hipLaunchKernelGGL((decode_kernel<MAXT, W4_EPI_NONE, W4_OUT_BF16>), grid, block, 0, stream, a,
                       wg_per_expert, total, items_per_expert);
}

}  // namespace

void launch_gemm_skinny(const GemmArgs& a, hipStream_t stream) {
  // rows per expert on average decides how many 16-row MFMA tiles one pass covers
  const int64_t avg = (a.R + a.E - 1) / a.E;
  if (avg <= 16) launch_m<1>(a, stream);
  else launch_m<2>(a, stream);
}

}  // namespace w4
