// Decode-shaped W4A16 matmul: few activation rows per expert, weight-streaming.
//
// [RQ] "Repacked QAT Gemma 4 26B-A4B serves on one TPU v6e at 1.9x FP8
// throughput", section "What changed in vLLM's TPU backend": the grouped
// matmul takes one scale per 32-wide group and dequantizes each weight tile on
// chip before the multiply; activations stay bf16.  "What quantization really
// is", section "Why the tip exists": generation rereads the weights token by
// token, so this kernel is bound by the weight bytes it streams.
//
// Work split: one wave per 16-row weight tile, streaming it over the whole K.
// A workgroup of 8 waves serves 8 tiles of one expert; with a gated epilogue
// they are 4 gate/up pairs (wave 2i the gate tile of pair i, wave 2i+1 its up
// tile) and the up wave hands its accumulator to the gate wave through LDS.
// The expert's activation rows are staged in LDS in chunks of KC columns,
// shared by the 8 waves; each wave's codes and scales come straight from global
// memory through a ring of D blocks held in registers (one 128-bit load per
// lane per 1 KiB tile16 block, one 64-bit load per lane for its 128 B of
// scales).
//
// Per 4-group block: the nibbles become bf16 136+q with one shift and one
// and-or per pair (biased_pairs); a first MFMA against a constant -136 operand
// gives -136*sum(x) per row and group and is the accumulator input of the MFMA
// against the biased codes, so each group's partial sum sum(x*q) comes out of
// the matrix core; the VALU adds scale * partial into the fp32 accumulator.
// Rows beyond the expert's count read a valid row; their results are never
// stored.

#include "common.h"
#include "internal.h"
#include "w4a16.h"

namespace w4 {

namespace {

constexpr int kWaves = 8;   // waves (weight tiles) per workgroup
constexpr int kRsrcFlags = 0x00020000;   // raw buffer descriptor word 3 (32-bit data, no swizzle)

// Ring depth of the many-tile (MoE) path and the occupancy its register
// allocation aims for (waves per SIMD; 0 = compiler default).
#ifndef W4_DECODE_RING
#define W4_DECODE_RING 4
#endif
// Short K (at most 8 tile16 blocks) with a plain epilogue goes to the
// several-tiles-per-wave kernel (gemm_short.hip).
#ifndef W4_DECODE_SHORT_K
#define W4_DECODE_SHORT_K 1
#endif
// Occupancy the register allocation aims for (waves per SIMD): 4 for one
// 16-row tile of activation rows (two 8-wave workgroups per CU), 2 for two.
#ifndef W4_DECODE_WAVES_PER_SIMD
#define W4_DECODE_WAVES_PER_SIMD 4
#endif
#define W4_DECODE_OCC __attribute__((amdgpu_waves_per_eu(MAXT == 1 ? W4_DECODE_WAVES_PER_SIMD : 2)))


// blockIdx -> workgroup index so that consecutive indices (the same expert)
// land on the same XCD (workgroups are dealt to the 8 XCDs round-robin).
__device__ __forceinline__ int xcd_item(int b, int total) {
  const int xcd = b & 7, idx = b >> 3;
  const int per = total >> 3, rem = total & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D: code/scale blocks in flight per wave (ring depth); a chunk of staged
// activations spans max(4, D) blocks so that ring slots are compile-time.
template <int MAXT, int EPI, int OUT, int D>
__global__ void __launch_bounds__(64 * kWaves) W4_DECODE_OCC decode_kernel(GemmArgs a, int wg_per_expert,
                                                                           int total_wg, int units_per_expert) {
  constexpr bool GATED = EPI != W4_EPI_NONE;
  constexpr int CB = D > 4 ? D : 4;       // blocks per staged activation chunk
  constexpr int KC = CB * 128;            // columns per chunk
  constexpr int XS = KC * 2 + 16;         // LDS row stride in bytes (padded off the bank period)
  constexpr int XBUF = 16 * MAXT * XS;                       // one staging buffer
  constexpr int EXBYTES = (kWaves / 2) * MAXT * 64 * 16;     // gate/up hand-over
  __shared__ __align__(16) uint8_t xs[2 * XBUF > EXBYTES ? 2 * XBUF : EXBYTES];
  // scale spans: SPB blocks (a whole number of chunks, at least 8), 128 B each
  constexpr int SPB = CB > 8 ? CB : 8;
  constexpr int SPBYTES = SPB * 128;
  constexpr int SPL = SPB / 8;   // 16-byte loads per lane per span
  __shared__ __align__(16) uint8_t ssc[kWaves * SPBYTES];

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
  const int r = lane & 15;
  const int c = lane >> 4;
  const int64_t K = a.K, N = a.N;

  // this wave's weight tile
  int unit, tile;
  if constexpr (GATED) {
    unit = wgi * (kWaves / 2) + (wv >> 1);           // gate/up pair
    tile = unit + ((wv & 1) ? (int)(N / 32) : 0);    // the up tile sits N/2 rows below
  } else {
    unit = wgi * kWaves + wv;
    tile = unit;
  }
  // idle waves (past the expert's last tile) run on tile 0 and store nothing,
  // so every wave executes the same loads and barriers
  const bool active = unit < units_per_expert;
  if (!active) tile = 0;

  const int G = (int)(K / kGroup);
  const int NBF = G / kBlockGroups;
  const int gtail = G - NBF * kBlockGroups;
  const int NBall = NBF + (gtail > 0 ? 1 : 0);
  const uint8_t* wb = a.qweight + (int64_t)e * (N * K / 2) + (int64_t)tile * 8 * K;
  const uint16_t* sb = a.scales + ((int64_t)e * N + (int64_t)tile * kTileRows) * G;

  u32x4 cw[D];
  auto load_block = [&](int slot, int b) __attribute__((always_inline)) {
    cw[slot] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wb + 1024 * (int64_t)b + 16 * lane));
  };

  // Scales of the full blocks travel in spans of SPB blocks (contiguous in the
  // tile's scale layout): 128-bit loads, one per lane per 8 blocks, parked in
  // this wave's LDS span buffer, then 8 bytes per lane per block from there.
  // The next span overwrites the buffer after the wave's last read of the
  // current one (LDS accesses of one wave complete in order).  Per-block
  // 128-byte scale loads would make a second, sparse stream beside the codes.
  // The loads go through a buffer descriptor over the expert's scales: lanes
  // past the tile's last full block read the tail block or the next tile, and
  // past the end of the expert get zeros; those bytes are never used.
  uint8_t* mys = ssc + wv * SPBYTES;
  const int NSP = (NBF + SPB - 1) / SPB;
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.scales + (int64_t)e * N * G), 0, (int)(N * G * 2), kRsrcFlags);
  const uint32_t sv_lane = (uint32_t)tile * (uint32_t)(32 * G) + 16u * (uint32_t)lane;
  auto span_load = [&](u32x4* t, int sp) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SPL; ++i)
      t[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           srs, sv_lane, (uint32_t)(SPBYTES * sp + 1024 * i), 0));
  };
  auto span_store = [&](const u32x4* t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SPL; ++i) *reinterpret_cast<u32x4*>(mys + 1024 * i + 16 * lane) = t[i];
  };

  // the partial last block (1..3 groups), loaded once
  uint32_t ct[3] = {0u, 0u, 0u};
  float st[3] = {0.f, 0.f, 0.f};
  if (gtail > 0) {
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < gtail) {
        ct[j] = *reinterpret_cast<const uint32_t*>(wb + 1024 * (int64_t)NBF + 4 * gtail * lane + 4 * j);
        st[j] = bf16_to_f32(sb[64 * (int64_t)NBF + r * gtail + j]);
      }
  }

  const u32x4 neg136 = {kNeg136Pair, kNeg136Pair, kNeg136Pair, kNeg136Pair};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  // Activation staging: chunk ch (columns [ch*KC, ch*KC+KC)) of the pass's rows
  // goes to LDS buffer ch%2.  The global loads of chunk ch+1 are issued before
  // the code loads of chunk ch's blocks and written to LDS after them, so the
  // (in-order) wait for the activations never drains the code prefetch ring.
  constexpr int PPR = KC / 8;                       // 16-byte pieces per row of a chunk
  constexpr int NP = 16 * MAXT * PPR / (64 * kWaves);   // pieces per thread
  static_assert(NP * 64 * kWaves == 16 * MAXT * PPR, "chunk must split evenly over the threads");

  for (int64_t row0 = row_begin; row0 < row_end; row0 += 16 * MAXT) {
    const int cnt = (int)(row_end - row0 < 16 * MAXT ? row_end - row0 : 16 * MAXT);
    const int ntt = (cnt + 15) >> 4;
    const int nch = (NBall + CB - 1) / CB;

    // this thread's staging pieces: one buffer descriptor per piece row,
    // fixed for the pass.  A row is staged by whole waves (a row's pieces are
    // 64 consecutive threads), so each descriptor is wave-uniform.  Rows
    // beyond the count get an empty range: their loads return zeros without
    // touching memory (those LDS rows are never read as operands: their lanes
    // read row 0).  Columns past K are clamped.
    static_assert(PPR % 64 == 0, "a staged row must cover whole waves");
    __amdgpu_buffer_rsrc_t xrs[NP];
    int xdst[NP];
    uint32_t xoff[NP];
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int p = (int)threadIdx.x + q * 64 * kWaves;
      const int rr = __builtin_amdgcn_readfirstlane(p / PPR);
      const int pc = p - rr * PPR;
      const bool live = rr < cnt;
      const int64_t srow = live ? (a.row_index ? (int64_t)a.row_index[row0 + rr] : row0 + rr)
                                : (a.row_index ? (int64_t)a.row_index[row0] : row0);   // a valid row
      // (readfirstlane returns int: each half goes back through uint32_t so
      // the low half is not sign-extended into the high one)
      const uint64_t base = (uint64_t)(a.x + srow * K);
      const uint32_t bhi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32));
      const uint32_t blo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)base);
      const uint64_t ub = ((uint64_t)bhi << 32) | (uint64_t)blo;
      xrs[q] = __builtin_amdgcn_make_buffer_rsrc((void*)ub, 0, live ? (int)(K * 2) : 0, kRsrcFlags);
      xdst[q] = rr * XS + pc * 16;
      xoff[q] = (uint32_t)(pc * 16);
    }
    u32x4 xr[NP];
    auto stage_load = [&](int ch) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        uint32_t off = (uint32_t)(ch * KC * 2) + xoff[q];
        off = off < (uint32_t)(K * 2 - 16) ? off : (uint32_t)(K * 2 - 16);
        xr[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs[q], off, 0, 0));
      }
    };
    auto stage_store = [&](int ch) __attribute__((always_inline)) {
      uint8_t* buf = xs + (ch & 1) * XBUF;
#pragma unroll
      for (int q = 0; q < NP; ++q) *reinterpret_cast<u32x4*>(buf + xdst[q]) = xr[q];
    };

    // every load of the pass's start is issued before the first wait: the
    // first chunk's activations, the first scale span, the ring's blocks
    __syncthreads();   // the previous pass is done with both buffers
    stage_load(0);
    if (NBF > 0) {
      u32x4 s0[SPL];
      span_load(s0, 0);
#pragma unroll
      for (int i = 0; i < D; ++i) load_block(i, i < NBF ? i : NBF - 1);
      span_store(s0);
    }
    stage_store(0);
    __syncthreads();

    int arow[MAXT];   // LDS row of this lane's A operand (padding rows read row 0)
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt) arow[tt] = (16 * tt + r < cnt) ? 16 * tt + r : 0;

    f32x4 acc[MAXT];
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt) acc[tt] = zero4;

    // one block: MFMAs on the slot's codes, then refill the slot with block bn
    // (after the slot's last use, so no register copies are needed)
    auto do_block = [&](const uint8_t* xb, int b, int lb, int slot, int bn) __attribute__((always_inline)) {
      const u32x2 sv = *reinterpret_cast<const u32x2*>(mys + (b % SPB) * 128 + 8 * r);
      const float sc[4] = {bf16_to_f32(sv[0] & 0xFFFFu), bf16_to_f32(sv[0] >> 16),
                           bf16_to_f32(sv[1] & 0xFFFFu), bf16_to_f32(sv[1] >> 16)};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 B = as_bf16x8(biased_pairs(cw[slot][j]));
#pragma unroll
        for (int tt = 0; tt < MAXT; ++tt)
          if (tt < ntt) {
            const bf16x8 A = *reinterpret_cast<const bf16x8*>(xb + arow[tt] * XS + (lb * 4 + j) * 64 + c * 16);
            const f32x4 cb = mfma16x16x32(A, as_bf16x8(neg136), zero4);
            const f32x4 p = mfma16x16x32(A, B, cb);
            acc[tt] += sc[j] * p;
          }
      }
      load_block(slot, bn);
      __builtin_amdgcn_sched_barrier(0);   // issue the refill here, not later
    };

    // full chunks: straight-line code, every load unconditional (indices clamped)
    // (a span is a whole number of chunks: its next span is loaded at its
    // first chunk and parked after its last)
    static_assert(SPB % CB == 0, "a scale span must cover whole chunks");
    constexpr int CPS = SPB / CB;   // chunks per span
    const int nfull = NBF / CB;
    auto do_chunk = [&](int ch) __attribute__((always_inline)) {
      const int chn = ch + 1 < nch ? ch + 1 : nch - 1;
      stage_load(chn);
      const uint8_t* xb = xs + (ch & 1) * XBUF;
#pragma unroll
      for (int lb = 0; lb < CB; ++lb) {
        const int bn = ch * CB + lb + D;
        do_block(xb, ch * CB + lb, lb, lb % D, bn < NBF ? bn : NBF - 1);
      }
      stage_store(chn);
      __syncthreads();
    };
    // whole spans of full chunks: the next span's scales are loaded at the
    // span's first chunk and parked after its last, unconditionally (past
    // the last span they are junk that no block reads)
    const int nspan_full = nfull / CPS;
    for (int sp = 0; sp < nspan_full; ++sp) {
      u32x4 snext[SPL];
      span_load(snext, sp + 1);
#pragma unroll
      for (int k = 0; k < CPS; ++k) do_chunk(sp * CPS + k);
      span_store(snext);
    }
    // the remaining full chunks, in the span parked last
    for (int ch = nspan_full * CPS; ch < nfull; ++ch) do_chunk(ch);
    // the last, partial chunk: remaining full blocks and the partial block
    if (nfull < nch) {
      const int ch = nfull;
      const uint8_t* xb = xs + (ch & 1) * XBUF;
#pragma unroll
      for (int lb = 0; lb < CB; ++lb)
        if (ch * CB + lb < NBF) do_block(xb, ch * CB + lb, lb, lb % D, NBF - 1);
      if (gtail > 0) {
        const int lb = NBF - ch * CB;   // local index of the partial block
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          if (j < gtail) {
            const bf16x8 B = as_bf16x8(biased_pairs(ct[j]));
#pragma unroll
            for (int tt = 0; tt < MAXT; ++tt)
              if (tt < ntt) {
                const bf16x8 A = *reinterpret_cast<const bf16x8*>(xb + arow[tt] * XS + (lb * 4 + j) * 64 + c * 16);
                const f32x4 cb = mfma16x16x32(A, as_bf16x8(neg136), zero4);
                const f32x4 p = mfma16x16x32(A, B, cb);
                acc[tt] += st[j] * p;
              }
          }
        }
      }
      __syncthreads();
    }

    // D rows = 4*(lane/16)+i, column = lane%16
    if constexpr (GATED) {
      f32x4* ex = reinterpret_cast<f32x4*>(xs);   // the chunk loop ended with a barrier
      if (active && (wv & 1)) {
#pragma unroll
        for (int tt = 0; tt < MAXT; ++tt) ex[((wv >> 1) * MAXT + tt) * 64 + lane] = acc[tt];
      }
      __syncthreads();
      if (active && !(wv & 1)) {
#pragma unroll
        for (int tt = 0; tt < MAXT; ++tt) {
          if (tt >= ntt) continue;
          const f32x4 up = ex[((wv >> 1) * MAXT + tt) * 64 + lane];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t row = row0 + 16 * tt + 4 * c + i;
            if (row >= row_end) continue;
            const float g = (float)(__bf16)acc[tt][i];
            const float u = (float)(__bf16)up[i];
            const float act = (EPI == W4_EPI_GEGLU_TANH) ? gelu_tanh_f32(g) : silu_f32(g);
            static_cast<uint16_t*>(a.out)[row * (N / 2) + (int64_t)unit * kTileRows + r] = bf16_rne(act * u);
          }
        }
      }
    } else {
      if (active) {
#pragma unroll
        for (int tt = 0; tt < MAXT; ++tt) {
          if (tt >= ntt) continue;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t row = row0 + 16 * tt + 4 * c + i;
            if (row >= row_end) continue;
            const int64_t col = (int64_t)tile * kTileRows + r;
            if constexpr (OUT == W4_OUT_F32) static_cast<float*>(a.out)[row * N + col] = acc[tt][i];
            else static_cast<uint16_t*>(a.out)[row * N + col] = bf16_rne(acc[tt][i]);
          }
        }
      }
    }
  }
}

template <int MAXT, int D>
void launch_m(const GemmArgs& a, hipStream_t stream) {
  const bool gated = a.epilogue != W4_EPI_NONE;
  const int units = (int)(gated ? a.N / 32 : a.N / 16);
  const int per_wg = gated ? kWaves / 2 : kWaves;
  const int wg_per_expert = (units + per_wg - 1) / per_wg;
  const int total = wg_per_expert * a.E;
  dim3 grid(total), block(64 * kWaves);
  if (a.epilogue == W4_EPI_GEGLU_TANH)
    hipLaunchKernelGGL((decode_kernel<MAXT, W4_EPI_GEGLU_TANH, W4_OUT_BF16, D>), grid, block, 0, stream, a,
                       wg_per_expert, total, units);
  else if (a.epilogue == W4_EPI_SWIGLU)
    hipLaunchKernelGGL((decode_kernel<MAXT, W4_EPI_SWIGLU, W4_OUT_BF16, D>), grid, block, 0, stream, a,
                       wg_per_expert, total, units);
  else if (a.out_dtype == W4_OUT_F32)
    hipLaunchKernelGGL((decode_kernel<MAXT, W4_EPI_NONE, W4_OUT_F32, D>), grid, block, 0, stream, a,
                       wg_per_expert, total, units);
  else
    hipLaunchKernelGGL((decode_kernel<MAXT, W4_EPI_NONE, W4_OUT_BF16, D>), grid, block, 0, stream, a,
                       wg_per_expert, total, units);
}

}  // namespace

void launch_gemm_skinny(const GemmArgs& a, hipStream_t stream) {
  // Fewer waves than SIMDs need a deeper register ring to keep HBM busy.
  const int64_t tiles = (a.N / 16) * a.E;
  const int64_t avg = (a.R + a.E - 1) / a.E;   // rows per expert: 16-row MFMA tiles per pass
  const bool deep = tiles < 4096;
  if (avg <= 16 && W4_DECODE_SHORT_K && gemm_short_supported(a)) {
    launch_gemm_short(a, stream);   // K <= 1024: several whole tiles per wave
  } else if (avg <= 16) {
    if (deep) launch_m<1, 16>(a, stream);
    else launch_m<1, W4_DECODE_RING>(a, stream);
  } else {
    if (deep) launch_m<2, 8>(a, stream);
    else launch_m<2, W4_DECODE_RING>(a, stream);
  }
}

}  // namespace w4
