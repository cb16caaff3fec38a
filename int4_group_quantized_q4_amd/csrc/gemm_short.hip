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
// takes TPW tiles of its expert (tile i*W + wave of the workgroup's range) and
// streams their blocks one after another (NBF full tile16 blocks per tile,
// then the partial one) through a ring of 4 blocks in registers, refilled as
// each block is used, so the weight stream runs on across tile boundaries and
// only the first block's latency is exposed.  The expert's activation rows
// (all of K, at most 16 rows per pass) are staged in LDS once per workgroup,
// with a table of -136 x each row's sum over each group.  Per group one MFMA
// takes the bf16 128+u codes with that table entry as its accumulator input,
// which cancels the +136 bias; the fp32 scale per group is applied on the
// VALU.  A tile's scales (32 G bytes, contiguous) are one 128-bit load per
// lane issued with the tile's first block and parked in a per-wave LDS buffer
// when the tile starts.

#include "common.h"
#include "internal.h"
#include "w4a16.h"

namespace w4 {

namespace {

constexpr int kSW = 4;                     // waves per workgroup (each stages the rows once; 4 per CU)
constexpr int kTPW = 6;                    // tiles per wave
constexpr int kRing = 4;                   // code blocks in flight per wave
constexpr int kWavesPerSimd = 4;
constexpr uint32_t kOOB = 0x80000000u;     // buffer offset past every range: reads zeros, moves no bytes
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
__global__ void __launch_bounds__(64 * kSW) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd)))
short_kernel(GemmArgs a, int wg_per_expert, int total_wg, int tiles_per_expert) {
  // A wave's blocks in order: tile i of its kTPW, block b of the tile's NB
  // (NBF full blocks, then the partial one: gtail groups, or nothing when
  // gtail = 0).  Codes travel through a ring of D 16-byte registers per lane.
  constexpr int NB = NBF + 1;
  constexpr int D = NB < kRing ? NB : kRing;
  constexpr int STEPS = kTPW * NB;
  __shared__ __align__(16) uint8_t xs[16 * (2 * kMaxCols + 16)];
  __shared__ __align__(16) uint8_t ssc[kSW * 1024];
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

  // tile of iteration i; tiles past the expert's last read nothing (offsets
  // outside the buffers) and are neither computed nor stored
  auto tile_of = [&](int i) { return wgi * kSW * kTPW + i * kSW + wv; };
  // codes of step j (tile j / NB, block j % NB) into ring slot j % D, and at
  // a tile's first block the tile's scales (all its groups: NBF x 128 B, then
  // the partial block's 16 x gtail; one 16-byte load per lane, lanes past the
  // tile read the next tile or zeros -- unused) into sp
  u32x4 cw[D];
  u32x4 sp = {0u, 0u, 0u, 0u};
  auto load_step = [&](int j) __attribute__((always_inline)) {
    const int ti = j / NB, b = j - (j / NB) * NB;   // (j is a compile-time constant here)
    const int t = tile_of(ti);
    const bool live = t < tiles_per_expert;
    const uint32_t wt = (uint32_t)t * (uint32_t)(8 * K);
    uint32_t off;
    if (b < NBF) off = wt + 1024u * b + 16u * lane;
    else off = gtail > 0 ? wt + 1024u * NBF + 4u * gtail * lane : kOOB;
    cw[j % D] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, live ? off : kOOB, 0, 0));
    if (b == 0) {
      const uint32_t so = (uint32_t)t * (uint32_t)(32 * G) + 16u * lane;
      sp = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, live ? so : kOOB, 0, 0));
    }
  };

  // The first pass's ring does not depend on the expert's rows: its loads go
  // out before the row range is read, so the weight stream starts without
  // waiting for that read.  (The ids go out before the ring: the scan must not
  // wait for the ring to land.)
  int idv[8];
  if constexpr (IDS) {
    if (a.R > 512 || wv == 0) ids_batch(a.ids, (int)a.R, wv, idv);
  }
#pragma unroll
  for (int j = 0; j < D; ++j) load_step(j);

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
  uint8_t* mys = ssc + wv * 1024;   // this wave's tile scales

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
      __builtin_amdgcn_s_waitcnt(0);   // vmcnt(0) expcnt(0) lgkmcnt(0): this wave's DMA (and the ring) has landed
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

    f32x4 acc = zero4;
#pragma unroll
    for (int j = 0; j < STEPS; ++j) {
      const int ti = j / NB, b = j % NB;
      const int t = tile_of(ti);
      const bool live = t < tiles_per_expert;   // wave-uniform
      // a tile's scales to LDS at its first block (this wave's earlier reads
      // of the buffer complete first: one wave's LDS accesses are in order)
      if (b == 0) *reinterpret_cast<u32x4*>(mys + 16 * lane) = sp;
      const u32x4 w = cw[j % D];
      if (live) {
        if (b < NBF) {
          const u32x2 sv = *reinterpret_cast<const u32x2*>(mys + 128 * b + 8 * r);
          const float sc[4] = {bf16_to_f32(sv[0] & 0xFFFFu), bf16_to_f32(sv[0] >> 16),
                               bf16_to_f32(sv[1] & 0xFFFFu), bf16_to_f32(sv[1] >> 16)};
#pragma unroll
          for (int h = 0; h < 4; h += 2) {
            bf16x8 A[2];
            f32x4 p[2];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
              A[jj] = *reinterpret_cast<const bf16x8*>(xa + (b * 4 + h + jj) * 64);
              p[jj] = *reinterpret_cast<const f32x4*>(ca + (b * 4 + h + jj) * 64);
            }
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) p[jj] = mfma16x16x32(A[jj], as_bf16x8(biased_pairs(w[h + jj])), p[jj]);
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) acc += sc[h + jj] * p[jj];
          }
        } else {
#pragma unroll
          for (int g = 0; g < 3; ++g)
            if (g < gtail) {
              const bf16x8 A = *reinterpret_cast<const bf16x8*>(xa + (NBF * 4 + g) * 64);
              const f32x4 cb = *reinterpret_cast<const f32x4*>(ca + (NBF * 4 + g) * 64);
              const f32x4 p = mfma16x16x32(A, as_bf16x8(biased_pairs(w[g])), cb);
              const uint32_t sb = *reinterpret_cast<const uint16_t*>(mys + 128 * NBF + 2 * (r * gtail + g));
              acc += bf16_to_f32(sb) * p;
            }
        }
      }
      // refill the slot: step j + D
      if (j + D < STEPS) load_step(j + D);
      if (b == NB - 1) {
        // D rows = 4c + q, column = r; rows past the expert's count have an
        // offset at the end of the output descriptor's range and are dropped
        if (live) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t off = obase[q] + (uint32_t)(t * kTileRows * ESZ);
            if constexpr (OUT == W4_OUT_F32)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[q]), ors, off, 0, 0);
            else
              __builtin_amdgcn_raw_buffer_store_b16(bf16_rne(acc[q]), ors, off, 0, 0);
          }
        }
        acc = zero4;
      }
      __builtin_amdgcn_sched_barrier(0);   // one block's operands live at a time
    }
    row0 += 16;
    if (row0 >= row_end) break;
    __syncthreads();   // the pass is done with the staged rows
#pragma unroll
    for (int j = 0; j < D; ++j) load_step(j);   // the next pass's ring
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
