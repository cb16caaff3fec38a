// Decode-shaped W4A16 matmul for short K (K <= 1024: at most 8 tile16 blocks
// per row), plain epilogue: the MoE down projection (K = 704) at decode.
//
// [RQ] "Repacked QAT Gemma 4 26B-A4B serves on one TPU v6e at 1.9x FP8
// throughput", section "What changed in vLLM's TPU backend": one scale per
// 32-wide group, each weight tile dequantized on chip before the multiply,
// activations in bf16.  "What quantization really is", section "Why the tip
// exists": generation rereads the weights token by token, so the kernel is
// bound by the weight bytes it streams.
//
// With K = 704 a 16-row weight tile is 6 KiB: a wave that streams one tile and
// leaves spends most of its life waiting for its first bytes.  Here a wave
// takes TPW tiles of its expert (tile i*W + wave of the workgroup's range), with
// two whole tiles in registers: the next tile's codes and scales are loaded
// while the current one is multiplied, so only the first tile's latency is
// exposed.  The expert's activation rows (all of K, at most 16 rows per pass)
// are staged in LDS once per workgroup, with a table of -136 x each row's sum
// over each group.  Per group one MFMA takes the bf16 128+u codes with that
// table entry as its accumulator input, which cancels the +136 bias; the fp32
// scale per group is applied on the VALU.  A tile's
// full-block scales (NBF x 128 B, contiguous) are one 128-bit load per lane,
// parked in a per-wave LDS buffer (one per register set) before use.

#include "common.h"
#include "internal.h"
#include "w4a16.h"

namespace w4 {

namespace {

constexpr int kSW = 4;                     // waves per workgroup (each stages the rows once; 3 per CU)
constexpr int kTPW = 4;                    // tiles per wave
constexpr int kMaxCols = 1024;             // K limit (8 tile16 blocks)
constexpr int kRsrcFlags = 0x00020000;     // raw buffer descriptor word 3

__device__ __forceinline__ int short_xcd_item(int b, int total) {
  const int xcd = b & 7, idx = b >> 3;
  const int per = total >> 3, rem = total & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// NBF: full tile16 blocks per row (K / 128); the 0..3 groups past them form
// the partial block.
// IDS: rows from the top-k ids (GemmArgs::ids): activation row r / kslots,
// output row r.
template <int NBF, int OUT, bool IDS>
__global__ void __launch_bounds__(64 * kSW) __attribute__((amdgpu_waves_per_eu(3)))
short_kernel(GemmArgs a, int wg_per_expert, int total_wg, int tiles_per_expert) {
  constexpr int CB = NBF > 0 ? NBF : 1;
  __shared__ __align__(16) uint8_t xs[16 * (2 * kMaxCols + 16)];
  __shared__ __align__(16) uint8_t ssc[kSW * 2 * 1024];
  __shared__ __align__(16) float ctab[(kMaxCols / kGroup) * 16];   // [G][16]: -136 x group sum of each row
  __shared__ int s_rows[IDS ? kIdsMaxExpertRows : 1];              // the expert's routed rows
  __shared__ int s_wcnt[kSW];                              // per-wave counts of the ids scan

  const int wg = short_xcd_item(blockIdx.x, total_wg);
  const int e = wg / wg_per_expert;
  const int wgi = wg - e * wg_per_expert;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, c = lane >> 4;
  const int64_t K = a.K, N = a.N;
  const int G = (int)(K / kGroup);
  const int gtail = G - NBF * kBlockGroups;
  constexpr int XS = 2 * kMaxCols + 16;   // LDS row stride: 16 B off the 256 B bank period

  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.qweight + (int64_t)e * (N * K / 2)), 0, (int)(N * K / 2), kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.scales + (int64_t)e * N * G), 0, (int)(N * G * 2), kRsrcFlags);

  // tile of iteration i; past the expert's last tile the loads re-read it
  // and nothing is computed or stored
  auto tile_of = [&](int i) { return wgi * kSW * kTPW + i * kSW + wv; };
  auto load_tile = [&](u32x4* cw, uint32_t* ct, u32x4& sp, uint32_t* st, int i) __attribute__((always_inline)) {
    int t = tile_of(i);
    t = t < tiles_per_expert ? t : tiles_per_expert - 1;
    const uint32_t wt = (uint32_t)t * (uint32_t)(8 * K), stt = (uint32_t)t * (uint32_t)(32 * G);
#pragma unroll
    for (int b = 0; b < NBF; ++b)
      cw[b] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, wt + 1024u * b + 16u * lane, 0, 0));
    if (NBF > 0)   // lanes past the tile's NBF*128 bytes read the partial block or the next tile: unused
      sp = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, stt + 16u * lane, 0, 0));
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < gtail) {
        ct[j] = __builtin_amdgcn_raw_buffer_load_b32(rw, wt + 1024u * NBF + 4u * gtail * lane + 4u * j, 0, 0);
        st[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, stt + 128u * NBF + 2u * (r * gtail + j), 0, 0);
      }
  };

  // The first pass's first tile does not depend on the expert's rows: its
  // loads go out before the row range is read, so the weight stream starts
  // without waiting for that read.
  u32x4 cwA[CB], cwB[CB], spA = {0u, 0u, 0u, 0u}, spB = {0u, 0u, 0u, 0u};
  uint32_t ctA[3] = {0u, 0u, 0u}, ctB[3] = {0u, 0u, 0u}, stA[3] = {0u, 0u, 0u}, stB[3] = {0u, 0u, 0u};
  // (the ids go out before the tile: the scan must not wait for the tile to land)
  int idv[8];
  if constexpr (IDS) {
    if (a.R > 512 || wv == 0) ids_batch(a.ids, (int)a.R, wv, idv);
  }
  load_tile(cwA, ctA, spA, stA, 0);

  int64_t row_begin = 0, row_end = a.R;
  if constexpr (IDS) {
    row_end = __builtin_amdgcn_readfirstlane(
        expert_rows_from_ids<kSW>(a.ids, (int)a.R, e, s_rows, kIdsMaxExpertRows, s_wcnt, idv));
  } else if (a.offsets) {
    row_begin = a.offsets[e];
    row_end = a.offsets[e + 1];
  }
  if (row_begin >= row_end) {   // the whole workgroup leaves together
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }
  // sorted row i (of this expert's range) -> activation row and output row
  auto xrow = [&](int64_t i) __attribute__((always_inline)) -> int64_t {
    if constexpr (IDS) return (int64_t)(s_rows[i] / a.kslots);
    else return a.row_index ? (int64_t)a.row_index[i] : i;
  };
  auto orow = [&](int64_t i) __attribute__((always_inline)) -> int64_t {
    if constexpr (IDS) return (int64_t)s_rows[i];
    else return a.out_index ? (int64_t)a.out_index[i] : i;
  };
  // the whole output (R * N * ESZ < 2^31, checked on the host); rows past the
  // expert's count get the offset of the range's end, so their stores are dropped
  constexpr int ESZ = OUT == W4_OUT_F32 ? 4 : 2;
  const uint32_t orange = (uint32_t)(a.R * N * ESZ);
  const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(a.out, 0, orange, kRsrcFlags);

  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  for (int64_t row0 = row_begin;;) {
    const int cnt = (int)(row_end - row0 < 16 ? row_end - row0 : 16);
    const int arow = r < cnt ? r : 0;   // rows past the count read row 0; never stored

    // the pass's activation rows, all of K, by DMA to LDS: wave w copies rows
    // w, w + kSW, ..., 1 KiB (64 lanes x 16 B) per instruction; lanes past K
    // re-read the row's last 16 bytes into the row's own padding (the row
    // stride holds 2 KiB), so no VGPRs hold activation data
    {
      const int nrow_dma = (int)((K * 2 + 1023) / 1024);
#pragma unroll
      for (int h = 0; h < 16 / kSW; ++h) {
        const int m = wv + kSW * h;
        if (m < cnt) {   // wave-uniform
          const int64_t row = xrow(row0 + m);
          const uint16_t* src = a.x + row * K;
          for (int d = 0; d < nrow_dma; ++d) {
            int64_t col = (int64_t)d * 512 + 8 * lane;
            col = col < K - 8 ? col : K - 8;
            __builtin_amdgcn_global_load_lds((const void*)(src + col),
                                             (__attribute__((address_space(3))) void*)(xs + m * XS + 1024 * d), 16,
                                             0, 0);
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0);   // vmcnt(0) expcnt(0) lgkmcnt(0): this wave's DMA has landed
      // bias table of the rows this wave staged: -136 x the row's sum over
      // each group, lane g for group g
#pragma unroll
      for (int h = 0; h < 16 / kSW; ++h) {
        const int m = wv + kSW * h;
        if (m < cnt && lane < G) {
          const uint8_t* xr = xs + m * XS + lane * 64;
          float sum = 0.f;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const u32x4 q = *reinterpret_cast<const u32x4*>(xr + 16 * v);
#pragma unroll
            for (int k = 0; k < 4; ++k) sum += bf16_to_f32(q[k] & 0xFFFFu) + bf16_to_f32(q[k] >> 16);
          }
          ctab[lane * 16 + m] = -136.f * sum;
        }
      }
    }
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);

    const uint8_t* xa = xs + arow * XS + c * 16;
    const uint8_t* ca = reinterpret_cast<const uint8_t*>(ctab) + c * 16;   // rows 4c .. 4c+3
    uint32_t obase[4];   // this lane's output rows 4c + q (past the count: dropped)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      obase[q] = 4 * c + q < cnt ? (uint32_t)((orow(row0 + 4 * c + q) * N + r) * ESZ) : orange;
    auto run_tile = [&](const u32x4* cw, const uint32_t* ct, const u32x4& sp, const uint32_t* st, int i,
                        int set) __attribute__((always_inline)) {
      const int t = tile_of(i);
      if (t >= tiles_per_expert) return;   // wave-uniform
      uint8_t* mys = ssc + (wv * 2 + set) * 1024;
      if (NBF > 0) *reinterpret_cast<u32x4*>(mys + 16 * lane) = sp;
      f32x4 acc = zero4;
#pragma unroll
      for (int b = 0; b < NBF; ++b) {
        const u32x2 sv = *reinterpret_cast<const u32x2*>(mys + 128 * b + 8 * r);
        const float sc[4] = {bf16_to_f32(sv[0] & 0xFFFFu), bf16_to_f32(sv[0] >> 16), bf16_to_f32(sv[1] & 0xFFFFu),
                             bf16_to_f32(sv[1] >> 16)};
        constexpr int NP = NBF >= 7 ? 1 : 2;   // independent groups at a time (two sets of 7-8 blocks leave room for 1)
#pragma unroll
        for (int h = 0; h < 4; h += NP) {
          bf16x8 A[NP];
          f32x4 p[NP];
#pragma unroll
          for (int j = 0; j < NP; ++j) {
            A[j] = *reinterpret_cast<const bf16x8*>(xa + (b * 4 + h + j) * 64);
            p[j] = *reinterpret_cast<const f32x4*>(ca + (b * 4 + h + j) * 64);
          }
#pragma unroll
          for (int j = 0; j < NP; ++j) p[j] = mfma16x16x32(A[j], as_bf16x8(biased_pairs(cw[b][h + j])), p[j]);
#pragma unroll
          for (int j = 0; j < NP; ++j) acc += sc[h + j] * p[j];
        }
        __builtin_amdgcn_sched_barrier(0);   // one block's operands live at a time
      }
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (j < gtail) {
          const bf16x8 A = *reinterpret_cast<const bf16x8*>(xa + (NBF * 4 + j) * 64);
          const f32x4 cb = *reinterpret_cast<const f32x4*>(ca + (NBF * 4 + j) * 64);
          const f32x4 p = mfma16x16x32(A, as_bf16x8(biased_pairs(ct[j])), cb);
          acc += bf16_to_f32(st[j]) * p;
        }
      // D rows = 4c + q, column = r; rows past the expert's count have an
      // offset at the end of the output descriptor's range and are dropped
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t off = obase[q] + (uint32_t)(t * kTileRows * ESZ);
        if constexpr (OUT == W4_OUT_F32)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[q]), ors, off, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b16(bf16_rne(acc[q]), ors, off, 0, 0);
      }
    };

    // ping-pong over the two register sets: load tile i+1, multiply tile i
#pragma unroll
    for (int i = 0; i < kTPW; i += 2) {
      if (i + 1 < kTPW) load_tile(cwB, ctB, spB, stB, i + 1);
      run_tile(cwA, ctA, spA, stA, i, 0);
      if (i + 1 < kTPW) {
        if (i + 2 < kTPW) load_tile(cwA, ctA, spA, stA, i + 2);
        run_tile(cwB, ctB, spB, stB, i + 1, 1);
      }
    }
    row0 += 16;
    if (row0 >= row_end) break;
    __syncthreads();   // the pass is done with the staged rows
    load_tile(cwA, ctA, spA, stA, 0);   // the next pass's first tile
  }
}

template <int NBF>
void launch_nbf(const GemmArgs& a, hipStream_t stream) {
  const int tiles = (int)(a.N / kTileRows);
  const int wg_per_expert = (tiles + kSW * kTPW - 1) / (kSW * kTPW);
  const int total = wg_per_expert * a.E;
  if (a.ids) {
    if (a.out_dtype == W4_OUT_F32)
      hipLaunchKernelGGL((short_kernel<NBF, W4_OUT_F32, true>), dim3(total), dim3(64 * kSW), 0, stream, a,
                         wg_per_expert, total, tiles);
    else
      hipLaunchKernelGGL((short_kernel<NBF, W4_OUT_BF16, true>), dim3(total), dim3(64 * kSW), 0, stream, a,
                         wg_per_expert, total, tiles);
  } else if (a.out_dtype == W4_OUT_F32) {
    hipLaunchKernelGGL((short_kernel<NBF, W4_OUT_F32, false>), dim3(total), dim3(64 * kSW), 0, stream, a,
                       wg_per_expert, total, tiles);
  } else {
    hipLaunchKernelGGL((short_kernel<NBF, W4_OUT_BF16, false>), dim3(total), dim3(64 * kSW), 0, stream, a,
                       wg_per_expert, total, tiles);
  }
}

}  // namespace

bool gemm_short_supported(const GemmArgs& a) {
  return a.epilogue == W4_EPI_NONE && a.K >= kGroup && a.K <= kMaxCols && a.R * a.N * 4 < ((int64_t)1 << 31);
}

void launch_gemm_short(const GemmArgs& a, hipStream_t stream) {
  switch ((int)(a.K / kGroup) / kBlockGroups) {
    case 0: launch_nbf<0>(a, stream); break;
    case 1: launch_nbf<1>(a, stream); break;
    case 2: launch_nbf<2>(a, stream); break;
    case 3: launch_nbf<3>(a, stream); break;
    case 4: launch_nbf<4>(a, stream); break;
    case 5: launch_nbf<5>(a, stream); break;
    case 6: launch_nbf<6>(a, stream); break;
    case 7: launch_nbf<7>(a, stream); break;
    default: launch_nbf<8>(a, stream); break;
  }
}

}  // namespace w4
