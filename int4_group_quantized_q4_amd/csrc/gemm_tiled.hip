// Prefill-shaped W4A16 grouped matmul: many activation rows per expert, MFMA-bound.
//
// [RQ] "Repacked QAT Gemma 4 26B-A4B serves on one TPU v6e at 1.9x FP8
// throughput", section "What changed in vLLM's TPU backend": the grouped
// matmul takes a scale per 32-wide group and dequantizes each weight tile on
// chip right before the multiply; activations stay bf16, accumulation fp32.
//
// Block tile: BM = 128 activation rows of one expert x 256 weight rows, K in
// stages of 128 (one tile16 block = 4 groups).  4 waves, each owning all 128
// rows x 64 weight rows (4 MFMA column tiles of 16).
//  * Activations: the block's 128 gathered rows x 128 columns are staged in
//    LDS, double-buffered through registers (rows past the expert's count
//    re-read its first row; their results are never stored).
//  * Weights: each lane loads exactly its 16x16x32 MFMA B operand from the
//    tile16 layout (one 16-byte load per column tile per stage, prefetched a
//    stage ahead) and unpacks the codes in registers to exact bf16 q/16.
//  * Per group: one MFMA per (row tile, column tile) into a zero accumulator,
//    then acc += scale(row, group) * partial in fp32.  The exact weight is
//    scale*q, which bf16 cannot hold, so the scale goes onto the fp32 partial
//    sum; the epilogue multiplies by 16.
// Gated epilogue: a wave's 4 column tiles are 2 gate tiles and the matching 2
// up tiles, so act(gate) * up is formed in registers.
// Scheduling: block b takes item (expert, row tile, column block) with the
// column block fastest, dealt so that consecutive items share an XCD and its
// L2: the row tile's activations and the expert's weights are re-read from L2.

#include "common.h"
#include "internal.h"
#include "w4a16.h"

namespace w4 {

namespace {

constexpr int BM = 128;                      // activation rows per block
constexpr int WN_TILES = 4;                  // 16-row weight tiles per wave
constexpr int NWAVES = 4;
constexpr int BN_TILES = NWAVES * WN_TILES;  // weight tiles per block (256 rows)
constexpr int MT = BM / 16;                  // MFMA row tiles per wave
constexpr int XS = 128 * 2 + 16;             // LDS row stride of staged activations, bytes
constexpr int ABUF = BM * XS;
constexpr int APIECES = BM * 16 / (64 * NWAVES);  // 16-byte activation pieces per thread per stage

__device__ __forceinline__ float gelu_tanh_f32(float x) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * x * (1.0f + tanhf(c * (x + 0.044715f * x * x * x)));
}

__device__ __forceinline__ float silu_f32(float x) { return x / (1.0f + expf(-x)); }

// Blocks are dispatched round-robin over the 8 XCDs; give XCD x a contiguous
// range of items so neighbouring items share its L2.
__device__ __forceinline__ int xcd_item(int b, int total) {
  const int xcd = b & 7, idx = b >> 3;
  const int per = total >> 3, rem = total & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// The experts' row tiles (ceil(count/BM) each, in expert order), times
// ncol_blocks column blocks, are the work items.  Returns the item of block
// `blk`: expert (-1 past the end), row tile inside the expert, column block.
// Whole-wave; E <= 256.
struct Item {
  int expert, mtile, nblock;
};

__device__ Item find_item(const int32_t* offsets, int E, int64_t R, int ncol_blocks, int blk) {
  const int lane = threadIdx.x & 63;
  int cnt[4], pre = 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int e = lane * 4 + s;
    int n = 0;
    if (offsets) {
      if (e < E) n = (offsets[e + 1] - offsets[e] + BM - 1) / BM;
    } else if (e == 0) {
      n = (int)((R + BM - 1) / BM);
    }
    cnt[s] = n;
    pre += n;
  }
  int incl = pre;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  Item it{-1, 0, 0};
  const int total_items = __shfl(incl, 63, 64) * ncol_blocks;
  if (blk >= total_items) return it;
  const int item = xcd_item(blk, total_items);
  const int lin = item / ncol_blocks;
  const int excl = incl - pre;
  const uint64_t bal = __ballot(lin >= excl && lin < incl);
  const int owner = __ffsll((unsigned long long)bal) - 1;
  int e = 0, mt = 0;
  if (lane == owner) {
    int base = excl;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (lin >= base && lin < base + cnt[s]) {
        e = lane * 4 + s;
        mt = lin - base;
      }
      base += cnt[s];
    }
  }
  it.expert = __shfl(e, owner, 64);
  it.mtile = __shfl(mt, owner, 64);
  it.nblock = item - lin * ncol_blocks;
  return it;
}

template <int EPI, int OUT>
__global__ void __launch_bounds__(64 * NWAVES) tiled_kernel(GemmArgs a, int ncol_blocks) {
  constexpr bool GATED = EPI != W4_EPI_NONE;
  __shared__ __align__(16) uint8_t As[2 * ABUF];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int c = lane >> 4;
  const int64_t K = a.K, N = a.N;

  const Item it = find_item(a.offsets, a.E, a.R, ncol_blocks, blockIdx.x);
  if (it.expert < 0) return;   // uniform over the block
  const int e = __builtin_amdgcn_readfirstlane(it.expert);
  const int mt = __builtin_amdgcn_readfirstlane(it.mtile);
  const int nb = __builtin_amdgcn_readfirstlane(it.nblock);
  const int64_t e_begin = a.offsets ? a.offsets[e] : 0;
  const int64_t e_end = a.offsets ? a.offsets[e + 1] : a.R;
  const int64_t row_begin = e_begin + (int64_t)mt * BM;
  const int cnt = (int)(e_end - row_begin < BM ? e_end - row_begin : BM);

  // this wave's weight tiles (tile16 tile index inside the expert's matrix)
  const int tiles_total = (int)(N / kTileRows);
  int tile[WN_TILES];
  bool active;
  if constexpr (GATED) {
    const int half = tiles_total / 2;
    const int g0 = nb * (BN_TILES / 2) + wv * 2;   // two gate tiles per wave; half is even
    active = g0 < half;
    tile[0] = g0;
    tile[1] = g0 + 1;
    tile[2] = g0 + half;
    tile[3] = g0 + 1 + half;
  } else {
    const int t0 = nb * BN_TILES + wv * WN_TILES;
    active = t0 < tiles_total;                     // tiles_total is a multiple of 4
#pragma unroll
    for (int t = 0; t < WN_TILES; ++t) tile[t] = t0 + t;
  }
  if (!active) {
    // idle waves still take part in the staging and the barriers
#pragma unroll
    for (int t = 0; t < WN_TILES; ++t) tile[t] = 0;
  }

  const int G = (int)(K / kGroup);
  const int NBF = G / kBlockGroups;   // full 4-group blocks
  const int gtail = G - NBF * kBlockGroups;
  const uint8_t* wb[WN_TILES];
  const uint16_t* sb[WN_TILES];
#pragma unroll
  for (int t = 0; t < WN_TILES; ++t) {
    wb[t] = a.qweight + (int64_t)e * (N * K / 2) + (int64_t)tile[t] * 8 * K;
    sb[t] = a.scales + ((int64_t)e * N + (int64_t)tile[t] * kTileRows) * G;
  }

  // activation staging: piece p = thread + q*256 is row p/16, columns (p%16)*8 .. +8
  const uint16_t* asrc[APIECES];
  int adst[APIECES], acol[APIECES];
#pragma unroll
  for (int q = 0; q < APIECES; ++q) {
    const int p = (int)threadIdx.x + q * 64 * NWAVES;
    const int rr = p >> 4;
    acol[q] = (p & 15) * 8;
    const int64_t row = row_begin + (rr < cnt ? rr : 0);
    const int64_t src = a.row_index ? (int64_t)a.row_index[row] : row;
    asrc[q] = a.x + src * K;
    adst[q] = rr * XS + acol[q] * 2;
  }
  u32x4 ar[APIECES];
  // columns at or past ncol re-read column 0 of the stage: they land in LDS
  // columns that the partial last stage never reads
  auto a_load = [&](int b, int ncol) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < APIECES; ++q) {
      const int col = acol[q] < ncol ? acol[q] : 0;
      ar[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(asrc[q] + (int64_t)b * 128 + col));
    }
  };
  auto a_store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < APIECES; ++q) *reinterpret_cast<u32x4*>(As + buf * ABUF + adst[q]) = ar[q];
  };

  u32x4 bw[WN_TILES];
  u32x2 bs[WN_TILES];
  auto b_load = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < WN_TILES; ++t) {
      bw[t] = *reinterpret_cast<const u32x4*>(wb[t] + 1024 * (int64_t)b + 16 * lane);
      bs[t] = *reinterpret_cast<const u32x2*>(sb[t] + 64 * (int64_t)b + 4 * r);
    }
  };

  f32x4 acc[MT][WN_TILES];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < WN_TILES; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // one group j of a stage: B operands of the 4 tiles, their scales, 8 row tiles
  auto group = [&](const uint8_t* Ab, int j, const uint32_t* words, const float* sc) __attribute__((always_inline)) {
    bf16x8 B[WN_TILES];
#pragma unroll
    for (int t = 0; t < WN_TILES; ++t) B[t] = unpack8_div16(words[t]);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const bf16x8 A = *reinterpret_cast<const bf16x8*>(Ab + (16 * i + r) * XS + j * 64 + c * 16);
#pragma unroll
      for (int t = 0; t < WN_TILES; ++t) {
        const f32x4 p = mfma16x16x32(A, B[t], zero4);
        acc[i][t] += sc[t] * p;
      }
    }
  };
  auto full_stage = [&](int buf, const u32x4* cw, const u32x2* cs) __attribute__((always_inline)) {
    const uint8_t* Ab = As + buf * ABUF;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t words[WN_TILES];
      float sc[WN_TILES];
#pragma unroll
      for (int t = 0; t < WN_TILES; ++t) {
        words[t] = cw[t][j];
        const uint32_t pair = cs[t][j >> 1];
        sc[t] = bf16_to_f32((j & 1) ? (pair >> 16) : (pair & 0xFFFFu));
      }
      group(Ab, j, words, sc);
    }
  };

  // prologue: stage 0
  if (NBF > 0) {
    a_load(0, 128);
    b_load(0);
  } else {
    a_load(0, gtail * kGroup);
  }
  a_store(0);
  __syncthreads();

  for (int s = 0; s + 1 < NBF; ++s) {
    u32x4 cw[WN_TILES];
    u32x2 cs[WN_TILES];
#pragma unroll
    for (int t = 0; t < WN_TILES; ++t) {
      cw[t] = bw[t];
      cs[t] = bs[t];
    }
    a_load(s + 1, 128);
    b_load(s + 1);
    full_stage(s & 1, cw, cs);
    a_store((s + 1) & 1);
    __syncthreads();
  }
  if (NBF > 0) {
    u32x4 cw[WN_TILES];
    u32x2 cs[WN_TILES];
#pragma unroll
    for (int t = 0; t < WN_TILES; ++t) {
      cw[t] = bw[t];
      cs[t] = bs[t];
    }
    if (gtail > 0) a_load(NBF, gtail * kGroup);
    full_stage((NBF - 1) & 1, cw, cs);
    if (gtail > 0) {
      a_store(NBF & 1);
      __syncthreads();
    }
  }
  if (gtail > 0) {
    // the partial last block: gtail (1..3) groups, word stride 4*gtail per lane
    const uint8_t* Ab = As + (NBF & 1) * ABUF;
    for (int j = 0; j < gtail; ++j) {
      uint32_t words[WN_TILES];
      float sc[WN_TILES];
#pragma unroll
      for (int t = 0; t < WN_TILES; ++t) {
        words[t] = *reinterpret_cast<const uint32_t*>(wb[t] + 1024 * (int64_t)NBF + 4 * gtail * lane + 4 * j);
        sc[t] = bf16_to_f32(sb[t][64 * (int64_t)NBF + r * gtail + j]);
      }
      group(Ab, j, words, sc);
    }
  }

  if (!active) return;
  // D element q of row tile i: row 16i + 4*(lane/16) + q, weight row lane%16 of each tile
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = 16 * i + 4 * c + q;
      if (rr >= cnt) continue;
      const int64_t row = row_begin + rr;
      if constexpr (GATED) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float g = bf16_to_f32(f32_to_bf16(acc[i][t][q] * 16.0f));
          const float u = bf16_to_f32(f32_to_bf16(acc[i][t + 2][q] * 16.0f));
          const float act = (EPI == W4_EPI_GEGLU_TANH) ? gelu_tanh_f32(g) : silu_f32(g);
          static_cast<uint16_t*>(a.out)[row * (N / 2) + (int64_t)tile[t] * kTileRows + r] =
              (uint16_t)f32_to_bf16(act * u);
        }
      } else {
#pragma unroll
        for (int t = 0; t < WN_TILES; ++t) {
          const float v = acc[i][t][q] * 16.0f;
          const int64_t o = row * N + (int64_t)tile[t] * kTileRows + r;
          if constexpr (OUT == W4_OUT_F32) static_cast<float*>(a.out)[o] = v;
          else static_cast<uint16_t*>(a.out)[o] = (uint16_t)f32_to_bf16(v);
        }
      }
    }
  }
}

}  // namespace

bool gemm_tiled_supported(const GemmArgs& a) {
  const int64_t tiles = a.N / kTileRows;
  if (a.E > 256 || a.R >= ((int64_t)1 << 31)) return false;
  if (a.epilogue != W4_EPI_NONE) return (tiles / 2) % 2 == 0;   // gate tiles go in pairs
  return tiles % WN_TILES == 0;
}

void launch_gemm_tiled(const GemmArgs& a, hipStream_t stream) {
  const bool gated = a.epilogue != W4_EPI_NONE;
  const int64_t tiles = a.N / kTileRows;
  const int ncol_blocks = (int)(gated ? (tiles / 2 + BN_TILES / 2 - 1) / (BN_TILES / 2)
                                      : (tiles + BN_TILES - 1) / BN_TILES);
  // upper bound on the experts' row tiles: sum ceil(count/BM) <= R/BM + E
  const int64_t mt_bound = a.R / BM + a.E;
  const dim3 grid((unsigned)(mt_bound * ncol_blocks)), block(64 * NWAVES);
  if (a.epilogue == W4_EPI_GEGLU_TANH)
    hipLaunchKernelGGL((tiled_kernel<W4_EPI_GEGLU_TANH, W4_OUT_BF16>), grid, block, 0, stream, a, ncol_blocks);
  else if (a.epilogue == W4_EPI_SWIGLU)
    hipLaunchKernelGGL((tiled_kernel<W4_EPI_SWIGLU, W4_OUT_BF16>), grid, block, 0, stream, a, ncol_blocks);
  else if (a.out_dtype == W4_OUT_F32)
    hipLaunchKernelGGL((tiled_kernel<W4_EPI_NONE, W4_OUT_F32>), grid, block, 0, stream, a, ncol_blocks);
  else
    hipLaunchKernelGGL((tiled_kernel<W4_EPI_NONE, W4_OUT_BF16>), grid, block, 0, stream, a, ncol_blocks);
}

}  // namespace w4
