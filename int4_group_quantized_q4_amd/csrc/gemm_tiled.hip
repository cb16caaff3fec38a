// Prefill-shaped W4A16 grouped matmul: many activation rows per expert, MFMA-bound.
//
// [RQ] "Repacked QAT Gemma 4 26B-A4B serves on one TPU v6e at 1.9x FP8
// throughput", section "What changed in vLLM's TPU backend": the grouped
// matmul takes a scale per 32-wide group and dequantizes each weight tile on
// chip right before the multiply, with fp32 accumulation.
//
// Number format.  A dequantized weight s*q (bf16 scale: 8 significant bits,
// |q| <= 8: 3 more) needs 11 significant bits.  bf16 holds 8, fp16 holds 11, so
// the weight tile is dequantized to fp16, where s*q is exact for every scale in
// [2^-14, 2^13).  The activations enter as fp16 rows from rows_to_f16(): each
// row was multiplied by a power of two 2^-e that puts its largest magnitude in
// [2^14, 2^15), which converts every bf16 value exactly except magnitudes below
// 2^-32 of the row's largest (rounded to fp16's 2^-24 quantum).  The fp16
// MFMA's products are therefore the exact products of the bf16 operands (up to
// that power of two), accumulated in fp32 straight in the MFMA accumulators;
// the epilogue multiplies by 2^e.  A block whose scales leave the exact range
// (zero, tiny, huge or non-finite) is recomputed by an exact path that scales
// each group's fp32 partial sum instead.
//
// Block tile: BM = 128 activation rows of one expert x 256 weight rows (16
// tile16 tiles), 4 waves each owning all 128 rows x 64 weight rows (4 MFMA
// column tiles); two blocks per CU.  K advances in stages of 64 (2 groups).
//  * Activations: a 4-stage ring of 16 KB LDS buffers filled by global->LDS DMA
//    (each lane's 16 bytes go straight to LDS), three stages ahead.  Inside a
//    buffer, row r's 16-byte chunk h sits at chunk h ^ ((r & 7) ^ ((r >> 3) & 1)),
//    which keeps both the DMA writes and the MFMA operand reads free of bank
//    conflicts.  Rows past the expert's count re-read its first row; their
//    results are never stored.
//  * Weights: each lane loads exactly its 16x16x32 MFMA B operand from the
//    tile16 layout (8 bytes per column tile per stage, one stage ahead) and
//    expands it in registers: the offset-binary nibble u OR-ed into fp16 1024.0
//    gives 1024 + u, minus 1032 gives q, times the fp16 scale gives s*q.
// Gated epilogue: a wave's 4 column tiles are 2 gate tiles and the matching 2
// up tiles, so act(gate) * up is formed in registers; the results leave
// through LDS as 64-byte row pieces.
// Padding: an item holding at most 64 rows (an expert's last row tile) runs a
// copy of the pipeline with MFMAs for 4 row tiles instead of 8, and in a
// matrix's last column block the waves left without weight tiles skip the
// expansion and the MFMAs (they still stage activations and meet the
// barriers).
// Scheduling: block b takes item (expert, row tile, column block), dealt so
// that consecutive items share an XCD and its L2: for grouped experts the
// column block fastest (the row tile's activations and the expert's weights
// are re-read from L2); for one weight matrix, groups of 8 row tiles with the
// column block outer, so the blocks running together share weight panels too.

#include <type_traits>

#include "common.h"
#include "internal.h"
#include "w4a16.h"

namespace w4 {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
template <int V>
using I = std::integral_constant<int, V>;

constexpr int BM = 128;                      // activation rows per block
constexpr int WN_TILES = 4;                  // 16-row weight tiles per wave
constexpr int NWAVES = 4;                    // 2 blocks per CU: 2 waves per SIMD
constexpr int BN_TILES = NWAVES * WN_TILES;  // weight tiles per block
constexpr int MT = BM / 16;                  // MFMA row tiles per wave
constexpr int BK = 64;                       // K per stage: 2 groups
constexpr int NST = 4;                       // LDS ring depth (activation stages)
constexpr int AROW = BK * 2;                 // bytes of one staged activation row
constexpr int ASTAGE = BM * AROW;            // 16 KB per stage
constexpr int AQ = ASTAGE / (1024 * NWAVES); // DMA instructions per wave per stage

// Exact-range test of bf16 scale pairs: |s| in [2^-14, 2^13) <=> the 15 low bits
// minus 0x3880 (2^-14) stay below 0x0D80 (2^13 - 2^-14 in bf16 bit distance).
constexpr unsigned kScaleLo = 0x3880u;
// Fourth word of a raw buffer descriptor (32-bit data format, no swizzle).
constexpr int kRsrcFlags = 0x00020000;
constexpr unsigned kScaleSpan = 0x0D80u;


__device__ __forceinline__ f32x4 mfma_f16(h8 a, h8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// fp16 pairs 1024 + u of a tile16 word's codes (2d, 2d+1), d = 0..3: the low
// nibbles of the word's bytes are codes 0, 4, 1, 5 and the high nibbles codes
// 2, 6, 3, 7; a byte permute places each code below the fp16 exponent byte 0x64.
__device__ __forceinline__ void biased_f16_pairs(uint32_t w, uint32_t out[4]) {
  const uint32_t lo = w & 0x0F0F0F0Fu;
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
  out[0] = __builtin_amdgcn_perm(0x64646464u, lo, 0x04020400u);
  out[1] = __builtin_amdgcn_perm(0x64646464u, hi, 0x04020400u);
  out[2] = __builtin_amdgcn_perm(0x64646464u, lo, 0x04030401u);
  out[3] = __builtin_amdgcn_perm(0x64646464u, hi, 0x04030401u);
}

// Chunk swizzle of a staged activation row (see the file comment).
__device__ __forceinline__ int aswz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// s_waitcnt vmcnt(N) lgkmcnt(0): at most N vector-memory operations of this
// wave still in flight, and every LDS access of this wave complete.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// Workgroup barrier without the memory fence of __syncthreads(): waits are
// explicit here.  The empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

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
// Inside an expert the items run in groups of gm row tiles: a group's items
// take the column blocks in order, and for each column block its gm row
// tiles, so that the blocks running at once on an XCD (consecutive items)
// share both their weight panels and their activation panels.  gm = 1: the
// column block fastest.  Whole-wave; E <= 256.
struct Item {
  int expert, mtile, nblock;
  int begin, end;   // the expert's sorted rows [begin, end)
};

__device__ Item find_item(const int32_t* offsets, int E, int64_t R, int ncol_blocks, int gm, int blk) {
  const int lane = threadIdx.x & 63;
  int cnt[4], lo[4], hi[4], pre = 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int e = lane * 4 + s;
    lo[s] = 0;
    hi[s] = 0;
    if (offsets) {
      if (e < E) {
        lo[s] = offsets[e];
        hi[s] = offsets[e + 1];
      }
    } else if (e == 0) {
      hi[s] = (int)R;
    }
    cnt[s] = (hi[s] - lo[s] + BM - 1) / BM;
    pre += cnt[s];
  }
  int incl = pre;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  Item it{-1, 0, 0, 0, 0};
  const int total_items = __shfl(incl, 63, 64) * ncol_blocks;
  if (blk >= total_items) return it;
  const int item = xcd_item(blk, total_items);
  const int lin = item / ncol_blocks;
  const int excl = incl - pre;
  const uint64_t bal = __ballot(lin >= excl && lin < incl);
  const int owner = __ffsll((unsigned long long)bal) - 1;
  int e = 0, b = 0, en = 0, tb = 0, tc = 0;
  if (lane == owner) {
    int base = excl;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (lin >= base && lin < base + cnt[s]) {
        e = lane * 4 + s;
        tb = base;
        tc = cnt[s];
        b = lo[s];
        en = hi[s];
      }
      base += cnt[s];
    }
  }
  it.expert = __shfl(e, owner, 64);
  it.begin = __shfl(b, owner, 64);
  it.end = __shfl(en, owner, 64);
  // the item's place among its expert's items: group of gm row tiles (the
  // last group may hold fewer), then column block, then row tile
  const int ebase = __shfl(tb, owner, 64), ecnt = __shfl(tc, owner, 64);
  const int li = item - ebase * ncol_blocks;
  const int g = li / (gm * ncol_blocks);
  const int rem = li - g * gm * ncol_blocks;
  const int gsz = ecnt - g * gm < gm ? ecnt - g * gm : gm;
  it.nblock = rem / gsz;
  it.mtile = g * gm + (rem - it.nblock * gsz);
  return it;
}

// The fast path computes the block's tile with B = s*q in fp16.  A block that
// meets a scale outside the exact fp16 range anywhere in its tile then
// recomputes the tile in place with B = q in fp16 and each group's fp32
// partial sum times its fp32 scale (the exact path), before the epilogue.
template <int EPI, int OUT>
__global__ void __launch_bounds__(64 * NWAVES) __attribute__((amdgpu_waves_per_eu(2)))
tiled_kernel(GemmArgs a, int ncol_blocks, int gm) {
  constexpr bool GATED = EPI != W4_EPI_NONE;
  // One array per ring slot, every access naming its slot at compile time: the
  // compiler then tells the slots apart and waits, before an operand read, only
  // for the DMA that filled that slot, not for the DMAs issued after it.
  __shared__ __align__(16) uint8_t As0[ASTAGE];
  __shared__ __align__(16) uint8_t As1[ASTAGE];
  __shared__ __align__(16) uint8_t As2[ASTAGE];
  __shared__ __align__(16) uint8_t As3[ASTAGE];
  // per row of the block: its activation exponent and its output row, read
  // at the start so that the epilogue waits for no global load
  __shared__ int s_xexp[BM];
  __shared__ int s_orow[BM];
  static_assert(NST == 4, "one array per ring slot");
  auto slot_buf = [&](auto J) __attribute__((always_inline)) -> uint8_t* {
    constexpr int j = decltype(J)::value % NST;
    if constexpr (j == 0) return As0;
    else if constexpr (j == 1) return As1;
    else if constexpr (j == 2) return As2;
    else return As3;
  };

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int c = lane >> 4;
  const int64_t K = a.K, N = a.N;

  const Item it = find_item(a.offsets, a.E, a.R, ncol_blocks, gm, blockIdx.x);
  if (it.expert < 0) return;   // uniform over the block
  const int e = __builtin_amdgcn_readfirstlane(it.expert);
  const int mt = __builtin_amdgcn_readfirstlane(it.mtile);
  const int nb = __builtin_amdgcn_readfirstlane(it.nblock);
  const int64_t e_begin = __builtin_amdgcn_readfirstlane(it.begin);
  const int64_t e_end = __builtin_amdgcn_readfirstlane(it.end);
  const int64_t row_begin = e_begin + (int64_t)mt * BM;
  const int cnt = (int)(e_end - row_begin < BM ? e_end - row_begin : BM);

  // this wave's weight tiles (tile16 tile index inside the expert's matrix);
  // in the last column block of a matrix whose tile count is not a multiple of
  // the block's, waves without tiles only take part in the staging and the
  // barriers
  const int tiles_total = (int)(N / kTileRows);
  int tile[WN_TILES];
  bool active;
  {
    const int per_wave = GATED ? 2 : WN_TILES;   // gate tiles (gated) or tiles per wave
    const int left = GATED ? tiles_total / 2 - nb * (BN_TILES / 2) : tiles_total - nb * BN_TILES;
    active = wv < left / per_wave;   // left % per_wave == 0
    if constexpr (GATED) {
      const int half = tiles_total / 2;
      const int g0 = nb * (BN_TILES / 2) + wv * 2;   // two gate tiles per wave; half is even
      tile[0] = g0;
      tile[1] = g0 + 1;
      tile[2] = g0 + half;
      tile[3] = g0 + 1 + half;
    } else {
      const int t0 = nb * BN_TILES + wv * WN_TILES;   // tiles_total is a multiple of 4
#pragma unroll
      for (int t = 0; t < WN_TILES; ++t) tile[t] = t0 + t;
    }
  }
  // row tiles holding rows of the expert (the exact path and the epilogue skip
  // the others)
  const int nmt = __builtin_amdgcn_readfirstlane((cnt + 15) >> 4);
  if (!active) {
#pragma unroll
    for (int t = 0; t < WN_TILES; ++t) tile[t] = 0;
  }

  const int G = (int)(K / kGroup);
  const int NBF = G / kBlockGroups;        // full 4-group tile16 blocks
  const int gtail = G - NBF * kBlockGroups;
  const int S = (G + 1) / 2;               // stages; the last holds one group when G is odd

  // Operands are read through buffer descriptors: a uniform base and size in
  // SGPRs, a 32-bit per-lane offset, a uniform per-tile offset; reads past the
  // size return zeros instead of faulting.
  const uint32_t wbytes = (uint32_t)(N * K / 2), sbytes = (uint32_t)(N * G * 2);
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.qweight + (int64_t)e * (N * K / 2)), 0, wbytes, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.scales + (int64_t)e * N * G), 0, sbytes, kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.xh, 0, (uint32_t)(a.x_rows * K * 2), kRsrcFlags);
  uint32_t wtoff[WN_TILES], stoff[WN_TILES];   // uniform byte offsets of the tiles
#pragma unroll
  for (int t = 0; t < WN_TILES; ++t) {
    wtoff[t] = (uint32_t)tile[t] * (uint32_t)(8 * K);
    stoff[t] = (uint32_t)tile[t] * (uint32_t)(32 * G);
  }

  // ---- activation DMA: wave wv's instruction q fills bytes [1024n, 1024n+1024)
  // of a stage buffer, n = AQ*wv + q: rows 8n .. 8n+7, lane -> row 8n + lane/8,
  // chunk slot lane%8, which holds source chunk slot ^ aswz(row).
  uint32_t aoff[AQ];   // byte offset of the lane's source chunk in stage 0
  uint32_t ahigh = 0;  // bit q: that chunk lies in the second group of a stage
  int xe[AQ], orw[AQ];
#pragma unroll
  for (int q = 0; q < AQ; ++q) {
    const int n = AQ * wv + q;
    const int rr = 8 * n + (lane >> 3);
    const int ch = (lane & 7) ^ aswz(rr);
    const int64_t row = row_begin + (rr < cnt ? rr : 0);
    const int64_t src = a.row_index ? (int64_t)a.row_index[row] : row;
    aoff[q] = (uint32_t)(src * K * 2) + (uint32_t)(ch * 16);
    ahigh |= (ch >= 4 ? 1u : 0u) << q;
    xe[q] = a.xexp[src];
    orw[q] = a.out_index ? a.out_index[row] : (int)row;
  }
  // The first lane of each row's 8 writes the row's entries, once the
  // pipeline's first loads are issued (so that waiting for xe and orw does not
  // hold them back); the pipeline's barriers order these writes before the
  // epilogue's reads.
  auto stash_rows = [&]() __attribute__((always_inline)) {
    if ((lane & 7) == 0) {
#pragma unroll
      for (int q = 0; q < AQ; ++q) {
        const int rr = 8 * (AQ * wv + q) + (lane >> 3);
        s_xexp[rr] = xe[q];
        s_orow[rr] = orw[q];
      }
    }
  };
  // activations of stage `st` into ring slot J
  auto a_issue = [&](int st, auto J) __attribute__((always_inline)) {
    uint8_t* dst = slot_buf(J) + (AQ * wv) * 1024;
    // a one-group last stage re-reads chunks 0..3 in place of 4..7 (unused)
    const bool one = 2 * st + 1 >= G;
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const uint32_t voff = aoff[q] - ((one && ((ahigh >> q) & 1u)) ? 64u : 0u);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(dst + q * 1024), 16,
                                               voff, (uint32_t)st * AROW, 0, 0);
    }
  };

  // ---- weights: per tile16 block b (stages 2b and 2b+1) and tile, the lane's
  // four code words (groups 0..3) and four scales.  A full block holds them at
  // 16*lane and 8*r bytes; the partial last block (gtail groups) at
  // 4*gtail*lane and 2*gtail*r, where the same 16- and 8-byte loads pick up
  // words 0..gtail-1 (the rest is the next rows' data or, past the end of the
  // buffer, zeros -- never used).
  const int NB = NBF + (gtail > 0 ? 1 : 0);
  u32x4 bw[2][WN_TILES];
  u32x2 bs[2][WN_TILES];
  auto bblk_issue = [&](int blk, auto SLOT) __attribute__((always_inline)) {
    constexpr int sl = decltype(SLOT)::value;
    const bool tail = blk >= NBF;
    const uint32_t wv = tail ? (uint32_t)(4 * gtail * lane) : (uint32_t)(16 * lane);
    // scale rows of a partial block start at 2-byte boundaries: load from the
    // dword below and shift the row's first scale down to bit 0
    const uint32_t sv = tail ? (uint32_t)(2 * gtail * r) : (uint32_t)(8 * r);
    const uint32_t sva = sv & ~3u, ssh = (sv & 3u) * 8u;
#pragma unroll
    for (int t = 0; t < WN_TILES; ++t) {
      // whole offsets in the VGPR operand: the buffer's range check covers
      // them, so the partial block's over-reads at the matrix end return zeros
      bw[sl][t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, wv + wtoff[t] + 1024 * blk, 0, 0));
      const uint64_t sc64 =
          __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(rs, sva + stoff[t] + 128 * blk, 0, 0));
      bs[sl][t] = __builtin_bit_cast(u32x2, sc64 >> ssh);
    }
  };

  f32x4 acc[MT][WN_TILES];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < WN_TILES; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // MFMA operand reads: row 16i + r, chunk 4j + c of the stage buffer
  const int apos0 = (r * AROW) + ((c ^ aswz(r)) * 16);
  const int apos1 = (r * AROW) + (((4 + c) ^ aswz(r)) * 16);
  const h2 kOff = {(_Float16)1032.0f, (_Float16)1032.0f};

  u16x2 srange = {0, 0};   // running max of (|scale bits| - kScaleLo), wrapping

  // The block's scales as fp16 pairs (groups 0,1 and 2,3), converted once per
  // block; exact for every scale in the fast path's range.
  h2 sfh[WN_TILES][2];
  auto block_scales = [&](int blk, auto SLOT) __attribute__((always_inline)) {
    constexpr int sl = decltype(SLOT)::value;
    const int ngb = blk < NBF ? kBlockGroups : gtail;   // groups present
#pragma unroll
    for (int t = 0; t < WN_TILES; ++t) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const uint32_t w = bs[sl][t][p];
        sfh[t][p] = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_pkrtz(bf16_to_f32(w & 0xFFFFu), bf16_to_f32(w >> 16)));
        // range test; an absent group counts as scale 1.0
        const uint32_t lo = (2 * p < ngb) ? (w & 0xFFFFu) : 0x3F80u;
        const uint32_t hi = (2 * p + 1 < ngb) ? (w >> 16) : 0x3F80u;
        const u16x2 v = __builtin_bit_cast(u16x2, (lo | (hi << 16)) & 0x7FFF7FFFu) - u16x2{kScaleLo, kScaleLo};
        srange = __builtin_elementwise_max(srange, v);
      }
    }
  };

  // fast path: group g (0..3) of the block in slot SLOT, B = s*q exactly in fp16
  auto fast_group = [&](const uint8_t* Ab, int apos, auto SLOT, auto GRP, auto ROWT) __attribute__((always_inline)) {
    constexpr int sl = decltype(SLOT)::value;
    constexpr int g = decltype(GRP)::value;
    constexpr int mtv = decltype(ROWT)::value;
    h8 B[WN_TILES];
#pragma unroll
    for (int t = 0; t < WN_TILES; ++t) {
      uint32_t pr[4];
      biased_f16_pairs(bw[sl][t][g], pr);
      const _Float16 sh = sfh[t][g >> 1][g & 1];
      const h2 s2 = {sh, sh};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const h2 q2 = (__builtin_bit_cast(h2, pr[d]) - kOff) * s2;
        B[t][2 * d] = q2[0];
        B[t][2 * d + 1] = q2[1];
      }
    }
    // every row tile of the variant, also those past the expert's count
    // (never stored).  The A operands are read two row tiles at a time, one
    // pair ahead of the MFMAs that use them, and scheduling barriers keep the
    // reads there: left to itself the compiler reads each pair right before
    // its MFMAs and waits out the LDS latency every 8 MFMAs.
    const uint8_t* ap = Ab + apos;
    h8 A0 = *reinterpret_cast<const h8*>(ap);
    h8 A1 = *reinterpret_cast<const h8*>(ap + 16 * AROW);
#pragma unroll
    for (int i = 0; i < mtv; i += 2) {
      h8 N0 = A0, N1 = A1;
      if (i + 2 < mtv) {
        N0 = *reinterpret_cast<const h8*>(ap + (i + 2) * 16 * AROW);
        N1 = *reinterpret_cast<const h8*>(ap + (i + 3) * 16 * AROW);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < WN_TILES; ++t) acc[i][t] = mfma_f16(A0, B[t], acc[i][t]);
#pragma unroll
      for (int t = 0; t < WN_TILES; ++t) acc[i + 1][t] = mfma_f16(A1, B[t], acc[i + 1][t]);
      __builtin_amdgcn_sched_barrier(0);
      A0 = N0;
      A1 = N1;
    }
  };

  // Pipeline.  Stage s computes groups 2h, 2h+1 (h = s % 2) of tile16 block
  // s/2 from LDS buffer s % NST.  Issue order: an even stage issues the next
  // block's weights, then every stage the activations of stage s + NST - 1;
  // issues past the end re-read the last block/stage into a free slot, so the
  // number of loads in flight is the same at every stage and the waits are
  // fixed:
  //   end of an even stage: A(s+1) has landed -- after it come A(s+2) ..
  //     A(s+NST-1) and (at most) one block's 8 weight loads;
  //   end of an odd stage: A(s+1) and the next block have landed -- after the
  //     block come A(s+NST-2) and A(s+NST-1).
  // The barrier then makes every wave's DMA visible and frees buffer s % NST,
  // which the next stage's DMA refills.
  const int last_st = S - 1;
  auto stage = [&](int s, auto SLOT, auto HALF, auto RING, auto ROWT) __attribute__((always_inline)) {
    constexpr int sl = decltype(SLOT)::value;
    constexpr int h = decltype(HALF)::value;
    constexpr int j = decltype(RING)::value;   // s % NST
    const int nb = (s >> 1) + 1;
    const int nbc = nb < NB ? nb : NB - 1;
    if constexpr (h == 0) bblk_issue(nbc, std::integral_constant<int, sl ^ 1>{});
    a_issue(s + NST - 1 <= last_st ? s + NST - 1 : last_st, std::integral_constant<int, j + NST - 1>{});
    // keep the loads at the top of the stage: sunk to its end they would be
    // waited for at once
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* Ab = slot_buf(RING);
    // a wave without weight tiles (last column block) only stages and waits
    if (active) {
      if constexpr (h == 0) block_scales(s >> 1, SLOT);
      fast_group(Ab, apos0, SLOT, std::integral_constant<int, 2 * h>{}, ROWT);
      if (2 * s + 1 < G) fast_group(Ab, apos1, SLOT, std::integral_constant<int, 2 * h + 1>{}, ROWT);
    }
    if constexpr (h == 0) wait_vm<(NST - 2) * AQ + 2 * WN_TILES>();
    else wait_vm<2 * AQ>();
    barrier_only();
  };

  {
    // prologue: block 0, then A(0) .. A(NST-2); wait for A(0) and block 0
    bblk_issue(0, std::integral_constant<int, 0>{});
    a_issue(0, std::integral_constant<int, 0>{});
    a_issue(1 <= last_st ? 1 : last_st, std::integral_constant<int, 1>{});
    a_issue(2 <= last_st ? 2 : last_st, std::integral_constant<int, 2>{});
    stash_rows();
    wait_vm<(NST - 2) * AQ>();
    barrier_only();

    // the stages with MFMAs for all MT row tiles, or (an item of at most 64
    // rows: the tail of an expert) for the first MT/2
    auto pipeline = [&](auto ROWT) __attribute__((always_inline)) {
      int s = 0;
#pragma unroll 1
      for (; s + 3 < S; s += 4) {
        stage(s, I<0>{}, I<0>{}, I<0>{}, ROWT);
        stage(s + 1, I<0>{}, I<1>{}, I<1>{}, ROWT);
        stage(s + 2, I<1>{}, I<0>{}, I<2>{}, ROWT);
        stage(s + 3, I<1>{}, I<1>{}, I<3>{}, ROWT);
      }
      if (s < S) stage(s, I<0>{}, I<0>{}, I<0>{}, ROWT);
      if (s + 1 < S) stage(s + 1, I<0>{}, I<1>{}, I<1>{}, ROWT);
      if (s + 2 < S) stage(s + 2, I<1>{}, I<0>{}, I<2>{}, ROWT);
    };
    if (nmt > MT / 2) pipeline(I<MT>{});
    else pipeline(I<MT / 2>{});
    // the loads issued past the end are still in flight: drain before the
    // block's LDS is released
    wait_vm<0>();

  }
  // Any scale outside the exact fp16 range anywhere in the block: the fast
  // path's sums are discarded and the exact path recomputes the tile.  (The
  // row entries stashed in the prologue stay valid; the barrier inside
  // __syncthreads_or comes after every wave's last read of the ring.)
  const bool bad = srange[0] >= kScaleSpan || srange[1] >= kScaleSpan;
  if (__syncthreads_or(bad)) {
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int t = 0; t < WN_TILES; ++t) acc[i][t] = zero4;
    for (int s = 0; s < S; ++s) {
      __syncthreads();
      a_issue(s, std::integral_constant<int, 0>{});
      bblk_issue(s >> 1, std::integral_constant<int, 0>{});
      wait_vm<0>();
      __syncthreads();
      const uint8_t* Ab = As0;
      const int ng = (2 * s + 1 < G) ? 2 : 1;
      for (int jj = 0; jj < ng; ++jj) {
        const int g = 2 * (s & 1) + jj;
        h8 B[WN_TILES];
        float sc[WN_TILES];
#pragma unroll
        for (int t = 0; t < WN_TILES; ++t) {
          const uint32_t w = bw[0][t][g];
          const uint32_t pair = bs[0][t][g >> 1];
          sc[t] = bf16_to_f32((g & 1) ? (pair >> 16) : (pair & 0xFFFFu));
          uint32_t pr[4];
          biased_f16_pairs(w, pr);
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const h2 q2 = __builtin_bit_cast(h2, pr[d]) - kOff;
            B[t][2 * d] = q2[0];
            B[t][2 * d + 1] = q2[1];
          }
        }
        const int apos = jj ? apos1 : apos0;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          if (i >= nmt) continue;
          const h8 A = *reinterpret_cast<const h8*>(Ab + apos + i * 16 * AROW);
#pragma unroll
          for (int t = 0; t < WN_TILES; ++t) {
            const f32x4 p = mfma_f16(A, B[t], zero4);
            acc[i][t] += sc[t] * p;
          }
        }
      }
    }
    __syncthreads();   // every wave is done with the staging buffer before the epilogue reuses LDS
  }

  if (!active) return;
  // D element q of row tile i: row 16i + 4*(lane/16) + q, weight row lane%16 of
  // each tile; the row's activation exponent undoes the fp16 scaling.  bf16
  // results are rounded to nearest even by the hardware conversion.
  auto row_exp = [&](int rr) __attribute__((always_inline)) { return s_xexp[rr]; };
  auto dst_row = [&](int rr) __attribute__((always_inline)) -> int64_t { return (int64_t)s_orow[rr]; };
  // Gated results go out through LDS (each wave its own 16 KiB ring slot,
  // free once the loop is done): written there in the MFMA layout, read back
  // by rows and stored 16 bytes per lane, so a row's 64-byte segment leaves in
  // one piece instead of as 2-byte stores.  Staged rows are padded to 80 B so
  // that the four row groups of a wave's writes fall in different banks.
  uint8_t* eb = wv == 0 ? As0 : (wv == 1 ? As1 : (wv == 2 ? As2 : As3));
  if constexpr (GATED) {
    constexpr int GS = 80;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (i >= nmt) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rr = 16 * i + 4 * c + q;
        const int ex = row_exp(rr);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float g = (float)(__bf16)ldexpf(acc[i][t][q], ex);
          const float u = (float)(__bf16)ldexpf(acc[i][t + 2][q], ex);
          const float act = (EPI == W4_EPI_GEGLU_TANH) ? gelu_tanh_f32(g) : silu_f32(g);
          *reinterpret_cast<uint16_t*>(eb + rr * GS + (16 * t + r) * 2) = __builtin_bit_cast(uint16_t, (__bf16)(act * u));
        }
      }
    }
    // 4 lanes per row (64 bytes: the wave's two gate tiles), 16 rows per store
    uint16_t* obase = static_cast<uint16_t*>(a.out) + tile[0] * kTileRows + 8 * (lane & 3);
#pragma unroll
    for (int k = 0; k < MT; ++k) {
      const int rr = 16 * k + (lane >> 2);
      if (rr < cnt) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(eb + rr * GS + 16 * (lane & 3));
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(obase + dst_row(rr) * (N / 2)));
      }
    }
  } else if constexpr (OUT == W4_OUT_F32) {
    // (staged through LDS like the gated case this measured no faster: the
    // 369 MB of fp32 rows the MoE down matmul writes are bound by their bytes)
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (i >= nmt) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rr = 16 * i + 4 * c + q;
        if (rr >= cnt) continue;
        const int ex = row_exp(rr);
        float* orow = static_cast<float*>(a.out) + dst_row(rr) * N + r;
#pragma unroll
        for (int t = 0; t < WN_TILES; ++t) __builtin_nontemporal_store(ldexpf(acc[i][t][q], ex), orow + tile[t] * kTileRows);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (i >= nmt) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rr = 16 * i + 4 * c + q;
        if (rr >= cnt) continue;
        const int ex = row_exp(rr);
        uint16_t* orow = static_cast<uint16_t*>(a.out) + dst_row(rr) * N + r;
#pragma unroll
        for (int t = 0; t < WN_TILES; ++t)
          __builtin_nontemporal_store(__builtin_bit_cast(uint16_t, (__bf16)ldexpf(acc[i][t][q], ex)),
                                      orow + tile[t] * kTileRows);
      }
    }
  }
}

// One wave per row: e = exponent putting max|x| in [2^14, 2^15), then
// xh = fp16(x * 2^-e) (round to nearest even), xexp = e.  NCH > 0: the row
// (at most NCH 16-byte chunks per lane) is loaded into registers at once and
// converted from there; NCH = 0: any K, the row read twice in a loop.
__device__ __forceinline__ int row_exponent(uint32_t m) {
  int ex = 0;
  if (m != 0 && m < 0x7F80u) {
    int fe;
    frexpf(bf16_to_f32(m), &fe);   // max|x| in [2^(fe-1), 2^fe)
    ex = fe - 15;
  }
  return ex;
}

__device__ __forceinline__ u32x4 chunk_to_f16(u32x4 v, int ex) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const _Float16 lo = (_Float16)ldexpf(bf16_to_f32(v[i] & 0xFFFFu), -ex);
    const _Float16 hi = (_Float16)ldexpf(bf16_to_f32(v[i] >> 16), -ex);
    o[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  return o;
}

template <int NCH>
__global__ void __launch_bounds__(256) rows_to_f16_kernel(const uint16_t* x, int64_t rows, int64_t K, uint16_t* xh,
                                                          int32_t* xexp) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + row * K);
  u32x4* dst = reinterpret_cast<u32x4*>(xh + row * K);
  const int nch = (int)(K / 8);
  uint32_t m = 0;
  if constexpr (NCH > 0) {
    u32x4 v[NCH];
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const int ch = lane + 64 * q;
      v[q] = ch < nch ? src[ch] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int q = 0; q < NCH; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m = max(m, v[q][i] & 0x7FFFu);
        m = max(m, (v[q][i] >> 16) & 0x7FFFu);
      }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
    const int ex = row_exponent(m);
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
      const int ch = lane + 64 * q;
      if (ch < nch) dst[ch] = chunk_to_f16(v[q], ex);
    }
    if (lane == 0) xexp[row] = ex;
  } else {
    for (int ch = lane; ch < nch; ch += 64) {
      const u32x4 v = src[ch];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m = max(m, v[i] & 0x7FFFu);
        m = max(m, (v[i] >> 16) & 0x7FFFu);
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
    const int ex = row_exponent(m);
    for (int ch = lane; ch < nch; ch += 64) dst[ch] = chunk_to_f16(src[ch], ex);
    if (lane == 0) xexp[row] = ex;
  }
}

}  // namespace

bool gemm_tiled_supported(const GemmArgs& a) {
  const int64_t tiles = a.N / kTileRows;
  if (a.E > 256 || a.R >= ((int64_t)1 << 31)) return false;
  // activation byte offsets are 32-bit
  if (a.x_rows * a.K * 2 >= ((int64_t)1 << 32)) return false;
  if (a.epilogue != W4_EPI_NONE) return (tiles / 2) % 2 == 0;   // gate tiles go in pairs
  return tiles % WN_TILES == 0;
}

static int64_t tiled_grid(const GemmArgs& a, int* ncol_blocks) {
  const bool gated = a.epilogue != W4_EPI_NONE;
  const int64_t tiles = a.N / kTileRows;
  *ncol_blocks = (int)(gated ? (tiles / 2 + BN_TILES / 2 - 1) / (BN_TILES / 2) : (tiles + BN_TILES - 1) / BN_TILES);
  // upper bound on the experts' row tiles: sum ceil(count/BM) <= R/BM + E
  return (a.R / BM + a.E) * *ncol_blocks;
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// fp16 activation rows and their exponents
size_t gemm_tiled_workspace(int64_t x_rows, int64_t R, int32_t E, int64_t K, int64_t N) {
  (void)R;
  (void)E;
  (void)N;
  return align256((size_t)x_rows * (size_t)K * 2) + align256((size_t)x_rows * 4);
}

template <int EPI, int OUT>
static void launch_tiled(const GemmArgs& a, int64_t blocks, int ncol_blocks, hipStream_t stream) {
  // one weight matrix (a dense prefill): groups of 8 row tiles; grouped
  // experts: the column block fastest
  const int gm = a.E == 1 ? 8 : 1;
  hipLaunchKernelGGL((tiled_kernel<EPI, OUT>), dim3((unsigned)blocks), dim3(64 * NWAVES), 0, stream, a, ncol_blocks,
                     gm);
}

void launch_gemm_tiled(const GemmArgs& a_in, void* ws, hipStream_t stream) {
  GemmArgs a = a_in;
  uint8_t* base = static_cast<uint8_t*>(ws);
  const size_t xh_bytes = align256((size_t)a.x_rows * (size_t)a.K * 2);
  const size_t xe_bytes = align256((size_t)a.x_rows * 4);
  a.xh = reinterpret_cast<uint16_t*>(base);
  a.xexp = reinterpret_cast<int32_t*>(base + xh_bytes);
  if (a.x_rows > 0) {
    // 16-byte chunks per lane of one row: held in registers up to 8
    const int64_t per_lane = (a.K / 8 + 63) / 64;
    const dim3 grid((unsigned)((a.x_rows + 3) / 4)), block(256);
    uint16_t* xh = const_cast<uint16_t*>(a.xh);
    int32_t* xe = const_cast<int32_t*>(a.xexp);
    if (per_lane <= 2) hipLaunchKernelGGL(rows_to_f16_kernel<2>, grid, block, 0, stream, a.x, a.x_rows, a.K, xh, xe);
    else if (per_lane <= 4) hipLaunchKernelGGL(rows_to_f16_kernel<4>, grid, block, 0, stream, a.x, a.x_rows, a.K, xh, xe);
    else if (per_lane <= 8) hipLaunchKernelGGL(rows_to_f16_kernel<8>, grid, block, 0, stream, a.x, a.x_rows, a.K, xh, xe);
    else hipLaunchKernelGGL(rows_to_f16_kernel<0>, grid, block, 0, stream, a.x, a.x_rows, a.K, xh, xe);
  }
  int nc;
  const int64_t blocks = tiled_grid(a, &nc);
  if (a.epilogue == W4_EPI_GEGLU_TANH) launch_tiled<W4_EPI_GEGLU_TANH, W4_OUT_BF16>(a, blocks, nc, stream);
  else if (a.epilogue == W4_EPI_SWIGLU) launch_tiled<W4_EPI_SWIGLU, W4_OUT_BF16>(a, blocks, nc, stream);
  else if (a.out_dtype == W4_OUT_F32) launch_tiled<W4_EPI_NONE, W4_OUT_F32>(a, blocks, nc, stream);
  else launch_tiled<W4_EPI_NONE, W4_OUT_BF16>(a, blocks, nc, stream);
}

}  // namespace w4
