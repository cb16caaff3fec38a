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
// and-or per pair (biased_pairs).  When a chunk of activations is staged, each
// row's sum over each group is formed from the staged registers and -136 x
// that sum goes to a small LDS table beside the chunk; the table entry is the
// accumulator input of the MFMA against the biased codes, so each group's
// partial sum sum(x*q) comes out of the matrix core in one MFMA; the VALU adds
// scale * partial into the fp32 accumulator.
// Rows beyond the expert's count read a valid row; their results are never
// stored.

#include <cmath>

#include "common.h"
#include "internal.h"
#include "w4a16.h"

namespace w4 {

namespace {

constexpr int kWaves = 8;   // waves (weight tiles) per workgroup
constexpr int kRsrcFlags = 0x00020000;   // raw buffer descriptor word 3 (32-bit data, no swizzle)

// Ring depth (code blocks in flight per wave) of the many-tile (MoE) path.
constexpr int kDecodeRing = 4;
// Occupancy the register allocation aims for (waves per SIMD): 4 for one
// 16-row tile of activation rows (two 8-wave workgroups per CU), 2 for two.
constexpr int kWavesPerSimd1 = 4;
#define W4_DECODE_OCC __attribute__((amdgpu_waves_per_eu(MAXT == 1 ? kWavesPerSimd1 : 2)))

// blockIdx -> workgroup index so that consecutive indices (the same expert)
// land on the same XCD (workgroups are dealt to the 8 XCDs round-robin).
__device__ __forceinline__ int xcd_item(int b, int total) {
  const int xcd = b & 7, idx = b >> 3;
  const int per = total >> 3, rem = total & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
// ---- Rows from the router logits (T <= 64 tokens, E <= 128 experts,
// finite logits).  Token t sends a row to expert e in slot j =
// the number of its logits above l[t][e], equal logits of lower ids counted
// as above, when j < k: the top-k order of the routing kernel (descending
// logit, ties to the lower id), so routed row r = t*k + j is the row that
// kernel's ids would give.
constexpr int kLogitsMaxTokens = 64;
constexpr int kLogitsMaxExperts = 128;
constexpr int kLogitsPerWave = kLogitsMaxTokens / kWaves;   // tokens ranked per wave

// Wave w ranks tokens w, w + 8, ...; lg[i][s] holds the i-th one's logits of
// experts lane + 64 s (-inf past E or T).
__device__ __forceinline__ void logits_batch(const float* __restrict__ logits, int T, int E,
                                             float lg[kLogitsPerWave][2]) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < kLogitsPerWave; ++i) {
    const int t = wv + kWaves * i;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int x = lane + 64 * s;
      lg[i][s] = (t < T && x < E) ? logits[(int64_t)t * E + x] : -INFINITY;
    }
  }
}

// Expert e's routed rows, in increasing r, to rows[0 .. count); returns count.
// The expert's plan entries (ids and softmax weights at t*k + j) are written
// by workgroup part = t % nparts of the expert's nparts workgroups (ids_out
// null: none).  s_rank: 64 ints of LDS.  Ends with a workgroup barrier.
__device__ __forceinline__ int expert_rows_from_logits(const float lg[kLogitsPerWave][2], int T, int E, int k, int e,
                                                       int* rows, int* s_rank, int* s_cnt, int part, int nparts,
                                                       int32_t* __restrict__ ids_out, float* __restrict__ wts_out) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool live[2] = {lane < E, lane + 64 < E};
#pragma unroll
  for (int i = 0; i < kLogitsPerWave; ++i) {
    const int t = wv + kWaves * i;
    if (t >= T) break;   // wave-uniform
    const float held = e >= 64 ? lg[i][1] : lg[i][0];   // (e is uniform)
    const float le = lane_f32(held, e & 63);
    const bool a0 = lg[i][0] > le || (lg[i][0] == le && lane < e);
    const bool a1 = lg[i][1] > le || (lg[i][1] == le && lane + 64 < e);
    const int j = __popcll(__ballot(a0)) + __popcll(__ballot(a1));
    if (lane == 0) s_rank[t] = j;
    if (ids_out && j < k && t % nparts == part) {   // wave-uniform
      float mx, sum;
      token_softmax_terms<2>(lg[i], live, mx, sum);
      if (lane == 0) {
        ids_out[(int64_t)t * k + j] = e;
        wts_out[(int64_t)t * k + j] = expf(le - mx) / sum;
      }
    }
  }
  __syncthreads();
  if (wv == 0) {
    const int j = lane < T ? s_rank[lane] : k;
    const uint64_t b = __ballot(j < k);
    const int pos = __popcll(b & ((1ull << lane) - 1ull));
    if (j < k) rows[pos] = lane * k + j;
    if (lane == 0) s_cnt[0] = __popcll(b);
  }
  __syncthreads();
  return s_cnt[0];
}

// D: code/scale blocks in flight per wave (ring depth); a chunk of staged
// activations spans max(4, D) blocks so that ring slots are compile-time.
// RM (row mode) 0: rows from the expert offsets (optionally gathered);
// 1: routed rows r from the top-k ids (GemmArgs::ids), activation row
// r / kslots, output row r; 2: the same routed rows found from the router
// logits (GemmArgs::logits), the expert's workgroups writing the expert's
// entries of the top-k plan (ids_out, wts_out) between them.
template <int MAXT, int EPI, int OUT, int D, int RM>
__global__ void __launch_bounds__(64 * kWaves) W4_DECODE_OCC decode_kernel(GemmArgs a, int wg_per_expert,
                                                                           int total_wg, int units_per_expert,
                                                                           int tsets) {
  constexpr bool GATED = EPI != W4_EPI_NONE;
  constexpr bool IDS = RM != 0;
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

  // -136 x each staged row's group sums, per staging buffer: [buffer][group of the chunk][row]
  constexpr int TROWS = 16 * MAXT;
  __shared__ __align__(16) float ctab[2 * CB * 4 * TROWS];
  __shared__ int s_rows[IDS ? kIdsMaxExpertRows : 1];   // the expert's routed rows
  __shared__ int s_wcnt[kWaves];                              // per-wave counts of the ids scan

  const int wg = xcd_item(blockIdx.x, total_wg);
  const int e = wg / wg_per_expert;
  const int wgi = wg - e * wg_per_expert;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15;
  const int c = lane >> 4;
  const int64_t K = a.K, N = a.N;

  const int G = (int)(K / kGroup);
  const int NBF = G / kBlockGroups;
  const int gtail = G - NBF * kBlockGroups;
  const int NBall = NBF + (gtail > 0 ? 1 : 0);

  // The workgroup takes tsets sets of units one after another (tsets > 1
  // when the expert's units would otherwise need more than one round of
  // resident workgroups); this wave's weight tile in set ts.  Idle waves
  // (past the expert's last tile) run on tile 0 and store nothing, so every
  // wave executes the same loads and barriers.
  constexpr int PER_WG = GATED ? kWaves / 2 : kWaves;
  int unit, tile;
  bool active;
  const uint8_t* wb;
  const uint16_t* sb;
  auto tiles_for = [&](int ts, int& u, int& t, bool& act) __attribute__((always_inline)) {
    const int u0 = (wgi * tsets + ts) * PER_WG;
    if constexpr (GATED) {
      u = u0 + (wv >> 1);                           // gate/up pair
      t = u + ((wv & 1) ? (int)(N / 32) : 0);       // the up tile sits N/2 rows below
    } else {
      u = u0 + wv;
      t = u;
    }
    act = u < units_per_expert;
    if (!act) t = 0;
  };
  auto set_tiles = [&](int ts) __attribute__((always_inline)) {
    tiles_for(ts, unit, tile, active);
    wb = a.qweight + (int64_t)e * (N * K / 2) + (int64_t)tile * 8 * K;
    sb = a.scales + ((int64_t)e * N + (int64_t)tile * kTileRows) * G;
  };
  set_tiles(0);

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
  uint32_t sv_lane = (uint32_t)tile * (uint32_t)(32 * G) + 16u * (uint32_t)lane;
  auto span_load_at = [&](u32x4* t, uint32_t sv, int sp) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SPL; ++i)
      t[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           srs, sv, (uint32_t)(SPBYTES * sp + 1024 * i), 0));
  };
  auto span_load = [&](u32x4* t, int sp) __attribute__((always_inline)) { span_load_at(t, sv_lane, sp); };
  u32x4 snx[SPL];   // the next pass's first scale span, loaded during this pass
  auto span_store = [&](const u32x4* t) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SPL; ++i) *reinterpret_cast<u32x4*>(mys + 1024 * i + 16 * lane) = t[i];
  };

  int64_t row_begin = 0, row_end = a.R;
  // The first pass's weight ring and first scale span do not depend on the
  // rows: they are issued before the row range is known (ids scan or offsets
  // read) and that wait overlaps the weight stream's first latency.  Every
  // later pass (of the
  // same tile or of the next unit set's) gets its ring and its first scale
  // span from the pass before it: the last D refills of a pass load the next
  // pass's blocks 0 .. D-1 (block b sits in ring slot b % D, so the slots
  // they free are exactly the ones those blocks go to), and the span goes to
  // registers after the pass's span loop.  Only registers are loaded early;
  // the span reaches its LDS buffer in the next pass's prologue, after the
  // barrier, as before.  (The ids go out first: the scan must not wait for
  // the ring to land.)
  int idv[8];
  float lgv[RM == 2 ? kLogitsPerWave : 1][2];
  const int ntok = (int)a.R / a.kslots;   // (logits mode: R <= 64 k)
  if constexpr (RM == 1) {
    if (a.R > 512 || wv == 0) ids_batch(a.ids, (int)a.R, wv, idv);
  } else if constexpr (RM == 2) {
    logits_batch(a.logits, ntok, a.E, lgv);
  }
  if (NBF > 0) {
#pragma unroll
    for (int i = 0; i < D; ++i) load_block(i, i < NBF ? i : NBF - 1);
    span_load(snx, 0);
  }
  if constexpr (RM == 1) {
    row_end = __builtin_amdgcn_readfirstlane(
        expert_rows_from_ids<kWaves>(a.ids, (int)a.R, e, s_rows, kIdsMaxExpertRows, s_wcnt, idv));
  } else if constexpr (RM == 2) {
    // rows at s_rows[0, 64), ranks staged at s_rows[64, 128)
    row_end = __builtin_amdgcn_readfirstlane(expert_rows_from_logits(lgv, ntok, a.E, a.kslots, e, s_rows,
                                                                     s_rows + kLogitsMaxTokens, s_wcnt, wgi,
                                                                     wg_per_expert, a.ids_out, a.wts_out));
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


  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  for (int ts = 0; ts < tsets; ++ts) {
  if (ts > 0) {
    set_tiles(ts);
    // a set with no unit of the expert (the expert's last workgroup) ends the
    // workgroup's work: units grow with the wave index, so wave 0 decides
    const int u0 = (wgi * tsets + ts) * PER_WG;
    if (u0 >= units_per_expert) break;   // uniform over the workgroup
    sv_lane = (uint32_t)tile * (uint32_t)(32 * G) + 16u * (uint32_t)lane;
  }
  // the partial last block (1..3 groups), loaded once per set, in its first
  // pass after the prologue's barrier (used at the pass's end only: loaded
  // earlier, the prologue's waits would include it)
  uint32_t ct[3] = {0u, 0u, 0u};
  float st[3] = {0.f, 0.f, 0.f};

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
      const int64_t srow = xrow(live ? row0 + rr : row0);   // a valid row
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
    // a piece's group inside the chunk and its first lane: a group is 4
    // consecutive pieces of a row, held by 4 consecutive lanes
    int tidx[NP];
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int p = (int)threadIdx.x + q * 64 * kWaves;
      const int rr = p / PPR;
      const int pc = p - rr * PPR;
      tidx[q] = (pc & 3) == 0 ? (pc >> 2) * TROWS + rr : -1;
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
      float* tb = ctab + (ch & 1) * (CB * 4 * TROWS);
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        *reinterpret_cast<u32x4*>(buf + xdst[q]) = xr[q];
        float sum = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) sum += bf16_to_f32(xr[q][k] & 0xFFFFu) + bf16_to_f32(xr[q][k] >> 16);
        // quad sums: lanes 4i .. 4i+3 hold the group's four pieces
        sum += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(sum), 0xB1, 0xF, 0xF, true));   // [1,0,3,2]
        sum += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(sum), 0x4E, 0xF, 0xF, true));   // [2,3,0,1]
        if (tidx[q] >= 0) tb[tidx[q]] = -136.f * sum;
      }
    };

    // The pass after this one, whose ring and first span this pass loads:
    // another pass over the same tile, the next unit set's tile, or none
    // (uniform over the wave).
    const uint8_t* wnx = nullptr;
    uint32_t svnx = 0u;
    if (row0 + 16 * MAXT < row_end) {
      wnx = wb;
      svnx = sv_lane;
    } else if (ts + 1 < tsets && (wgi * tsets + ts + 1) * PER_WG < units_per_expert) {
      int u2, t2;
      bool a2;
      tiles_for(ts + 1, u2, t2, a2);
      wnx = a.qweight + (int64_t)e * (N * K / 2) + (int64_t)t2 * 8 * K;
      svnx = (uint32_t)t2 * (uint32_t)(32 * G) + 16u * (uint32_t)lane;
    }
    // the first chunk's activations are the only load the prologue waits for
    // (the pass's ring and first span were loaded earlier)
    __syncthreads();   // the previous pass is done with both buffers
    stage_load(0);
    if (NBF > 0) span_store(snx);
    stage_store(0);
    __syncthreads();
    if (gtail > 0 && row0 == row_begin) {
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (j < gtail) {
          ct[j] = *reinterpret_cast<const uint32_t*>(wb + 1024 * (int64_t)NBF + 4 * gtail * lane + 4 * j);
          st[j] = bf16_to_f32(sb[64 * (int64_t)NBF + r * gtail + j]);
        }
    }

    int arow[MAXT];   // LDS row of this lane's A operand (padding rows read row 0)
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt) arow[tt] = (16 * tt + r < cnt) ? 16 * tt + r : 0;

    f32x4 acc[MAXT];
#pragma unroll
    for (int tt = 0; tt < MAXT; ++tt) acc[tt] = zero4;

    // one block: MFMAs on the slot's codes, then refill the slot with block bn
    // (after the slot's last use, so no register copies are needed); past
    // the tile's last block, with block `slot` of the next pass (none: the
    // last block again, never used)
    auto do_block = [&](const uint8_t* xb, const float* tb, int b, int lb, int slot, int bn)
                        __attribute__((always_inline)) {
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
            const f32x4 cb = *reinterpret_cast<const f32x4*>(tb + (lb * 4 + j) * TROWS + 16 * tt + 4 * c);
            const f32x4 p = mfma16x16x32(A, B, cb);
            acc[tt] += sc[j] * p;
          }
      }
      // the block's accumulation happens here: left free, the code generator
      // defers these adds past the scheduling barrier below and every
      // block's MFMA results stay live until the end of the chunk
#pragma unroll
      for (int tt = 0; tt < MAXT; ++tt) asm volatile("" : "+v"(acc[tt]));
      const uint8_t* src = bn < NBF ? wb + 1024 * (int64_t)bn
                                    : (wnx ? wnx + 1024 * (int64_t)(slot < NBF ? slot : NBF - 1)
                                           : wb + 1024 * (int64_t)(NBF - 1));
      cw[slot] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + 16 * lane));
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
      const float* tb = ctab + (ch & 1) * (CB * 4 * TROWS);
#pragma unroll
      for (int lb = 0; lb < CB; ++lb) {
        do_block(xb, tb, ch * CB + lb, lb, lb % D, ch * CB + lb + D);
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
    // the next pass's first span (its registers are free from here on; with
    // no next pass, a span that is never used)
    if (NBF > 0) span_load_at(snx, svnx, 0);
    // the remaining full chunks, in the span parked last
    for (int ch = nspan_full * CPS; ch < nfull; ++ch) do_chunk(ch);
    // the last, partial chunk: remaining full blocks and the partial block
    if (nfull < nch) {
      const int ch = nfull;
      const uint8_t* xb = xs + (ch & 1) * XBUF;
      const float* tb = ctab + (ch & 1) * (CB * 4 * TROWS);
#pragma unroll
      for (int lb = 0; lb < CB; ++lb)
        if (ch * CB + lb < NBF) do_block(xb, tb, ch * CB + lb, lb, lb % D, ch * CB + lb + D);
      if (gtail > 0) {
        const int lb = NBF - ch * CB;   // local index of the partial block
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          if (j < gtail) {
            // converted here: hoisted out of the pass loop, the pairs would
            // hold 12 registers through the main loop
            uint32_t w = ct[j];
            asm volatile("" : "+v"(w));
            const bf16x8 B = as_bf16x8(biased_pairs(w));
#pragma unroll
            for (int tt = 0; tt < MAXT; ++tt)
              if (tt < ntt) {
                const bf16x8 A = *reinterpret_cast<const bf16x8*>(xb + arow[tt] * XS + (lb * 4 + j) * 64 + c * 16);
                const f32x4 cb = *reinterpret_cast<const f32x4*>(tb + (lb * 4 + j) * TROWS + 16 * tt + 4 * c);
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
            static_cast<uint16_t*>(a.out)[orow(row) * (N / 2) + (int64_t)unit * kTileRows + r] = bf16_rne(act * u);
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
            const int64_t orw = orow(row);
            if constexpr (OUT == W4_OUT_F32) static_cast<float*>(a.out)[orw * N + col] = acc[tt][i];
            else static_cast<uint16_t*>(a.out)[orw * N + col] = bf16_rne(acc[tt][i]);
          }
        }
      }
    }
  }
  }   // tile sets
}

int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
                                                 hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

// Workgroups per expert and unit sets per workgroup: one set is PER_WG units
// (tiles, or gate/up pairs); a workgroup takes several sets one after another
// when the experts' sets would not fit in one round of resident workgroups
// (wg_per_cu of them per CU), so the launch runs as one round.  Only where
// that pays: the experts that get rows (expected E (1 - (1 - 1/E)^R) of them
// for R routed rows) must fill at least two rounds of one-set workgroups (at
// 8 tokens, 0.6 rounds' worth, three sets per workgroup took 67.6 against
// 57.1 us per layer), and at most 4 rows per expert on average: with more,
// the experts' row counts differ enough (some take a second 16-row pass)
// that the dispatcher's balancing over several rounds does better (128
// tokens: 103.4 against 108.6 us per layer; 256 tokens: 151 against 160 us).
void decode_grid(const GemmArgs& a, int units, int per_wg, int wg_per_cu, int* wg_per_expert, int* tsets) {
  const int sets = (units + per_wg - 1) / per_wg;
  const double slots = (double)wg_per_cu * device_cus();
  const double touched = a.E * (1.0 - std::pow(1.0 - 1.0 / a.E, (double)a.R));
  int ts = (int)std::ceil(sets * touched / slots);
  if (sets * touched < 2.0 * slots || a.R > 4 * (int64_t)a.E) ts = 1;
  ts = ts < 1 ? 1 : (ts > sets ? sets : ts);
  *tsets = ts;
  *wg_per_expert = (sets + ts - 1) / ts;
}

template <int MAXT, int D, int IDS>
void launch_m_ids(const GemmArgs& a, hipStream_t stream) {
  const bool gated = a.epilogue != W4_EPI_NONE;
  const int units = (int)(gated ? a.N / 32 : a.N / 16);
  const int per_wg = gated ? kWaves / 2 : kWaves;
  // resident 8-wave workgroups per CU: two at 4 waves per SIMD (the one-tile
  // kernel with the 4-block ring), one otherwise
  const int wg_per_cu = (MAXT == 1 && D == kDecodeRing) ? 2 : 1;
  int wg_per_expert, tsets;
  decode_grid(a, units, per_wg, wg_per_cu, &wg_per_expert, &tsets);
  const int total = wg_per_expert * a.E;
  dim3 grid(total), block(64 * kWaves);
  if (a.epilogue == W4_EPI_GEGLU_TANH)
    hipLaunchKernelGGL((decode_kernel<MAXT, W4_EPI_GEGLU_TANH, W4_OUT_BF16, D, IDS>), grid, block, 0, stream, a,
                       wg_per_expert, total, units, tsets);
  else if (a.epilogue == W4_EPI_SWIGLU)
    hipLaunchKernelGGL((decode_kernel<MAXT, W4_EPI_SWIGLU, W4_OUT_BF16, D, IDS>), grid, block, 0, stream, a,
                       wg_per_expert, total, units, tsets);
  else if (a.out_dtype == W4_OUT_F32)
    hipLaunchKernelGGL((decode_kernel<MAXT, W4_EPI_NONE, W4_OUT_F32, D, IDS>), grid, block, 0, stream, a,
                       wg_per_expert, total, units, tsets);
  else
    hipLaunchKernelGGL((decode_kernel<MAXT, W4_EPI_NONE, W4_OUT_BF16, D, IDS>), grid, block, 0, stream, a,
                       wg_per_expert, total, units, tsets);
}

template <int MAXT, int D>
void launch_m(const GemmArgs& a, hipStream_t stream) {
  if constexpr (MAXT == 1 && D == kDecodeRing) {
    if (a.logits) {
      // (gated only: gemm_skinny_takes_logits)
      const int units = (int)(a.N / 32);
      int wg_per_expert, tsets;
      decode_grid(a, units, kWaves / 2, 2, &wg_per_expert, &tsets);
      const int total = wg_per_expert * a.E;
      if (a.epilogue == W4_EPI_GEGLU_TANH)
        hipLaunchKernelGGL((decode_kernel<1, W4_EPI_GEGLU_TANH, W4_OUT_BF16, kDecodeRing, 2>), dim3(total),
                           dim3(64 * kWaves), 0, stream, a, wg_per_expert, total, units, tsets);
      else
        hipLaunchKernelGGL((decode_kernel<1, W4_EPI_SWIGLU, W4_OUT_BF16, kDecodeRing, 2>), dim3(total),
                           dim3(64 * kWaves), 0, stream, a, wg_per_expert, total, units, tsets);
      return;
    }
  }
  if (a.ids) launch_m_ids<MAXT, D, 1>(a, stream);
  else launch_m_ids<MAXT, D, 0>(a, stream);
}

// avg rows per expert, short-K eligibility and ring depth -> which kernel
enum class SkinnyPath { kShort, kM1Deep, kM1, kM2Deep, kM2 };
SkinnyPath skinny_path(const GemmArgs& a) {
  const int64_t tiles = (a.N / 16) * a.E;
  const int64_t avg = (a.R + a.E - 1) / a.E;   // rows per expert: 16-row MFMA tiles per pass
  const bool deep = tiles < 4096;              // fewer waves than SIMDs need a deeper register ring
  if (avg <= 16 && gemm_short_supported(a)) return SkinnyPath::kShort;
  if (avg <= 16) return deep ? SkinnyPath::kM1Deep : SkinnyPath::kM1;
  return deep ? SkinnyPath::kM2Deep : SkinnyPath::kM2;
}

}  // namespace

bool gemm_skinny_takes_logits(const GemmArgs& a, int64_t T, const float* logits) {
  return a.epilogue != W4_EPI_NONE && a.offsets == nullptr && a.row_index == nullptr && T >= 1 &&
         T <= kLogitsMaxTokens && a.E >= 1 && a.E <= kLogitsMaxExperts && logits != nullptr &&
         a.kslots >= 1 && a.R == T * a.kslots &&
         skinny_path(a) == SkinnyPath::kM1;
}

void launch_gemm_skinny(const GemmArgs& a, hipStream_t stream) {
  switch (skinny_path(a)) {
    case SkinnyPath::kShort: launch_gemm_short(a, stream); break;   // K <= 1024: several whole tiles per wave
    case SkinnyPath::kM1Deep: launch_m<1, 16>(a, stream); break;
    case SkinnyPath::kM1: launch_m<1, kDecodeRing>(a, stream); break;
    case SkinnyPath::kM2Deep: launch_m<2, 8>(a, stream); break;
    case SkinnyPath::kM2: launch_m<2, kDecodeRing>(a, stream); break;
  }
}

}  // namespace w4
