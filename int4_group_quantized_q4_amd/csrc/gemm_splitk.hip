// Dense decode-shaped W4A16 matmul split along K: one weight matrix, at most
// 16 activation rows.
//
// [RQ] "Repacked QAT Gemma 4 26B-A4B serves on one TPU v6e at 1.9x FP8
// throughput", section "What changed in vLLM's TPU backend": one scale per
// 32-wide group, each weight tile dequantized on chip before the multiply,
// activations in bf16.  "What quantization really is", section "Why the tip
// exists": generation rereads the weights token by token, so the kernel is
// bound by the weight bytes it streams.
//
// One wave per 16-row weight tile streams its whole K in the weight-streaming
// kernel; a matrix of few tiles (14336 rows = 896 tiles) then keeps only a
// third of the chip's SIMDs busy.  Here the K axis is cut into slices of 8
// tile16 blocks (1024 columns): a workgroup of 8 waves takes one slice of 8
// tiles, so the launch has tiles x slices waves.  Each wave issues its 8 code
// blocks (one 128-bit load per lane each) and its 1 KiB scale span before any
// wait, so a workgroup waits for memory once.  The slice of the activation
// rows is staged in LDS once per workgroup.  Per group the partial dot
// products come out of the matrix core as in the streaming kernel (bf16 128+u
// codes, a -136 operand for the bias, fp32 scale per group on the VALU).
// Slices write fp32 partial sums to the workspace; a second kernel adds the
// slices and rounds.
//
// For K <= 4096 (every activation row of the call fits in LDS) one kernel
// does it all: a workgroup holds FT weight tiles x FS K-slices, one wave
// each (4 x 4 for up to 16 rows, 2 x 4 for up to 8 or 4, 1 x 8 for one row),
// the activation rows are staged in LDS once, and after the slices' MFMAs the
// partial sums meet in LDS and are added in slice order and rounded by the
// slice-0 waves.  With 4 slices at K = 4096 each slice is 1024 columns, the
// slicing of the two-kernel path, so both give the same bits; one row is
// summed over 8 slices of 512 columns.  No workspace, no second launch, no
// ordering between workgroups.

#include "common.h"
#include "internal.h"
#include "w4a16.h"

namespace w4 {

namespace {

constexpr int kSKWaves = 8;                         // weight tiles per workgroup
constexpr int kSliceBlocks = 8;                     // tile16 blocks per K-slice
constexpr int kSliceCols = kSliceBlocks * 128;      // 1024
constexpr int kXStride = kSliceCols * 2 + 16;       // LDS row stride: 16 B off the 256 B bank period
constexpr int kMaxRows = 16;
constexpr int kRsrcFlags = 0x00020000;              // raw buffer descriptor word 3

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

int slices_of(int64_t K) {
  const int64_t G = K / kGroup;
  const int64_t nb = (G + kBlockGroups - 1) / kBlockGroups;   // blocks, the partial one included
  return (int)((nb + kSliceBlocks - 1) / kSliceBlocks);
}

// grid: (tile groups) x (slices), slice fastest.  part: [slices][R][N] fp32.
__global__ void __launch_bounds__(64 * kSKWaves) splitk_partial_kernel(GemmArgs a, int nslices, float* part) {
  __shared__ __align__(16) uint8_t xs[kMaxRows * kXStride];
  __shared__ __align__(16) uint8_t ssc[kSKWaves * 1024];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, c = lane >> 4;
  const int s = blockIdx.x % nslices;
  const int tg = blockIdx.x / nslices;
  const int M = (int)a.R;
  const int64_t K = a.K, N = a.N;
  const int G = (int)(K / kGroup);
  const int NBF = G / kBlockGroups;
  const int gtail = G - NBF * kBlockGroups;
  const int tiles = (int)(N / kTileRows);
  int tile = tg * kSKWaves + wv;
  const bool active = tile < tiles;
  if (!active) tile = tiles - 1;   // idle waves re-read a valid tile and store nothing

  const int kb0 = s * kSliceBlocks;
  const int nb = NBF - kb0 < kSliceBlocks ? NBF - kb0 : kSliceBlocks;   // full blocks of the slice (may be 0)
  const bool tail = gtail > 0 && s == nslices - 1;
  const int64_t col0 = (int64_t)s * kSliceCols;
  const int ncols = (int)(K - col0 < kSliceCols ? K - col0 : kSliceCols);

  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)a.qweight, 0, (int)(N * K / 2), kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)a.scales, 0, (int)(N * G * 2), kRsrcFlags);
  const uint32_t wtile = (uint32_t)tile * (uint32_t)(8 * K);
  const uint32_t stile = (uint32_t)tile * (uint32_t)(32 * G);

  // 1. every weight load of the wave: 8 code blocks (past the slice's last
  // full block they re-read it), the slice's 1 KiB scale span (lane l: block
  // l/8, rows 2(l%8) and 2(l%8)+1; past the matrix the descriptor returns
  // zeros), and the partial block's codes and scales
  u32x4 cw[kSliceBlocks];
  u32x4 sv = {0u, 0u, 0u, 0u};
  if (nb > 0) {
#pragma unroll
    for (int i = 0; i < kSliceBlocks; ++i) {
      const int bb = kb0 + (i < nb ? i : nb - 1);
      cw[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, wtile + 1024u * bb + 16u * lane, 0, 0));
    }
    sv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, stile + 128u * kb0 + 16u * lane, 0, 0));
  }
  uint32_t ct[3] = {0u, 0u, 0u};
  float st[3] = {0.f, 0.f, 0.f};
  if (tail) {
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < gtail) {
        ct[j] = __builtin_amdgcn_raw_buffer_load_b32(rw, wtile + 1024u * NBF + 4u * gtail * lane + 4u * j, 0, 0);
        st[j] = bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rs, stile + 128u * NBF + 2u * (r * gtail + j), 0, 0));
      }
  }

  // 2. the slice of the activation rows (rows < M only) into LDS
  const int ppr = ncols / 8;   // 16-byte pieces per row
  for (int p = (int)threadIdx.x; p < M * ppr; p += 64 * kSKWaves) {
    const int m = p / ppr, pc = p - m * ppr;
    const int64_t row = a.row_index ? (int64_t)a.row_index[m] : (int64_t)m;
    const u32x4 v = *reinterpret_cast<const u32x4*>(a.x + row * K + col0 + 8 * pc);
    *reinterpret_cast<u32x4*>(xs + m * kXStride + 16 * pc) = v;
  }
  uint8_t* mys = ssc + wv * 1024;
  *reinterpret_cast<u32x4*>(mys + 16 * lane) = sv;
  __syncthreads();

  // 3. the slice's blocks: D rows = 4c + i, column = r
  const u32x4 neg136 = {kNeg136Pair, kNeg136Pair, kNeg136Pair, kNeg136Pair};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const int arow = r < M ? r : 0;   // rows past M read row 0; their results are never stored
  const uint8_t* xa = xs + arow * kXStride + c * 16;
  f32x4 acc = zero4;
#pragma unroll
  for (int i = 0; i < kSliceBlocks; ++i) {
    if (i >= nb) break;
    const u32x2 sp = *reinterpret_cast<const u32x2*>(mys + 128 * i + 8 * r);
    const float sc[4] = {bf16_to_f32(sp[0] & 0xFFFFu), bf16_to_f32(sp[0] >> 16), bf16_to_f32(sp[1] & 0xFFFFu),
                         bf16_to_f32(sp[1] >> 16)};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 A = *reinterpret_cast<const bf16x8*>(xa + (i * 4 + j) * 64);
      const f32x4 cb = mfma16x16x32(A, as_bf16x8(neg136), zero4);
      const f32x4 p = mfma16x16x32(A, as_bf16x8(biased_pairs(cw[i][j])), cb);
      acc += sc[j] * p;
    }
  }
  if (tail) {
    const int lb = nb > 0 ? nb : 0;   // the partial block follows the slice's full blocks
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < gtail) {
        const bf16x8 A = *reinterpret_cast<const bf16x8*>(xa + (lb * 4 + j) * 64);
        const f32x4 cb = mfma16x16x32(A, as_bf16x8(neg136), zero4);
        const f32x4 p = mfma16x16x32(A, as_bf16x8(biased_pairs(ct[j])), cb);
        acc += st[j] * p;
      }
  }

  if (active) {
    float* dst = part + ((int64_t)s * M) * N + (int64_t)tile * kTileRows + r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * c + i < M) dst[(int64_t)(4 * c + i) * N] = acc[i];
  }
}

constexpr int kFMaxK = 4096;
constexpr int kFXStride = kFMaxK * 2 + 16;          // LDS row stride of the staged activations

// MR: activation rows staged (the call's M <= MR); FT weight tiles x FS
// K-slices per workgroup, one wave each.  grid: tile groups of FT; wave wv:
// tile wv % FT, slice wv / FT; each slice spans sb blocks (the partial block
// counts as one), at most kFMaxK / 128 / FS.
template <int OUT, int MR, int FT, int FS>
__global__ void __launch_bounds__(64 * FT * FS) splitk_fused_kernel(GemmArgs a, int sb) {
  constexpr int kFTiles = FT, kFSlices = FS;
  constexpr int kFMaxBlocks = (kFMaxK / 128 + FS - 1) / FS;   // tile16 blocks per slice, at most
  __shared__ __align__(16) uint8_t xs[MR * kFXStride];
  __shared__ __align__(16) uint8_t ssc[kFTiles * kFSlices * 1024];   // scale spans, then the partial sums

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, c = lane >> 4;
  const int tl = wv % kFTiles, s = wv / kFTiles;
  const int M = (int)a.R;
  const int64_t K = a.K, N = a.N;
  const int G = (int)(K / kGroup);
  const int NBF = G / kBlockGroups;
  const int gtail = G - NBF * kBlockGroups;
  const int tiles = (int)(N / kTileRows);
  int tile = blockIdx.x * kFTiles + tl;
  const bool active = tile < tiles;
  if (!active) tile = tiles - 1;   // idle waves re-read a valid tile and store nothing

  const int kb0 = s * sb;
  int nb = NBF - kb0 < sb ? NBF - kb0 : sb;   // full blocks of the slice
  if (nb < 0) nb = 0;
  const bool tail = gtail > 0 && kb0 <= NBF && NBF < kb0 + sb;   // the partial block is in this slice

  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)a.qweight, 0, (int)(N * K / 2), kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)a.scales, 0, (int)(N * G * 2), kRsrcFlags);
  const uint32_t wtile = (uint32_t)tile * (uint32_t)(8 * K);
  const uint32_t stile = (uint32_t)tile * (uint32_t)(32 * G);

  // 1. every load of the wave, in the order the waits need them (memory
  // counters drain in issue order), all unconditional so that the compiler
  // counts them exactly: its pieces of the activation rows, the slice's scale
  // span, then the code blocks (past the last full block they re-read it)
  // and the partial block.  The LDS stores below wait for the first two
  // only, so the blocks are still arriving when the MFMAs start.  Loads that
  // are not needed get an offset past their descriptor's range and return
  // zeros.
  constexpr int kXP = MR * (kFMaxK / 8) / (64 * kFTiles * kFSlices);   // pieces per thread, at most
  static_assert(kXP * 64 * kFTiles * kFSlices == MR * (kFMaxK / 8), "the rows split evenly over the threads");
  constexpr uint32_t kOff = 0x80000000u;                                     // past every range
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)a.x, 0, (int)(M * K * 2), kRsrcFlags);
  u32x4 xv[kXP];
#pragma unroll
  for (int q = 0; q < kXP; ++q)   // piece p: row p / (K/8), 16 bytes at p*16 (rows are contiguous)
    xv[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                          rx, 16u * ((uint32_t)threadIdx.x + (uint32_t)(q * 64 * kFTiles * kFSlices)), 0, 0));
  const u32x4 sv = __builtin_bit_cast(
      u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, nb > 0 ? stile + 128u * kb0 + 16u * lane : kOff, 0, 0));
  u32x4 cw[kFMaxBlocks];
#pragma unroll
  for (int i = 0; i < kFMaxBlocks; ++i) {
    const int bb = kb0 + (i < nb ? i : nb - 1);
    cw[i] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, nb > 0 ? wtile + 1024u * bb + 16u * lane : kOff, 0, 0));
  }
  uint32_t ct[3], stb[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const bool live = tail && j < gtail;
    ct[j] = __builtin_amdgcn_raw_buffer_load_b32(rw, live ? wtile + 1024u * NBF + 4u * gtail * lane + 4u * j : kOff, 0, 0);
    stb[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, live ? stile + 128u * NBF + 2u * (r * gtail + j) : kOff, 0, 0);
  }

  // 2. the activation rows (rows < M, all of K) and the scale span into LDS
  const int ppr = (int)(K / 8);   // 16-byte pieces per row
#pragma unroll
  for (int q = 0; q < kXP; ++q) {
    const int p = (int)threadIdx.x + q * 64 * kFTiles * kFSlices;
    if (p < M * ppr) {
      const int m = p / ppr, pc = p - m * ppr;
      *reinterpret_cast<u32x4*>(xs + m * kFXStride + 16 * pc) = xv[q];
    }
  }
  uint8_t* mys = ssc + wv * 1024;
  *reinterpret_cast<u32x4*>(mys + 16 * lane) = sv;
  __syncthreads();
  float st[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) st[j] = bf16_to_f32(stb[j]);

  // 3. the slice's blocks: D rows = 4c + i, column = r
  const u32x4 neg136 = {kNeg136Pair, kNeg136Pair, kNeg136Pair, kNeg136Pair};
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const int arow = r < M ? r : 0;   // rows past M read row 0; their results are never stored
  const uint8_t* xa = xs + arow * kFXStride + (int64_t)kb0 * 256 + c * 16;
  f32x4 acc = zero4;
#pragma unroll
  for (int i = 0; i < kFMaxBlocks; ++i) {
    if (i >= nb) break;
    const u32x2 sp = *reinterpret_cast<const u32x2*>(mys + 128 * i + 8 * r);
    const float sc[4] = {bf16_to_f32(sp[0] & 0xFFFFu), bf16_to_f32(sp[0] >> 16), bf16_to_f32(sp[1] & 0xFFFFu),
                         bf16_to_f32(sp[1] >> 16)};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 A = *reinterpret_cast<const bf16x8*>(xa + (i * 4 + j) * 64);
      const f32x4 cb = mfma16x16x32(A, as_bf16x8(neg136), zero4);
      const f32x4 p = mfma16x16x32(A, as_bf16x8(biased_pairs(cw[i][j])), cb);
      acc += sc[j] * p;
    }
  }
  if (tail) {
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < gtail) {
        const bf16x8 A = *reinterpret_cast<const bf16x8*>(xa + (nb * 4 + j) * 64);
        const f32x4 cb = mfma16x16x32(A, as_bf16x8(neg136), zero4);
        const f32x4 p = mfma16x16x32(A, as_bf16x8(biased_pairs(ct[j])), cb);
        acc += st[j] * p;
      }
  }

  // 4. the slices' partial sums meet in LDS (the scale spans are done with
  // once every wave has passed the barrier) and are added in slice order
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(ssc);
  if (s > 0) red[((s - 1) * kFTiles + tl) * 64 + lane] = acc;
  __syncthreads();
  if (s == 0 && active) {
    f32x4 v = acc;
#pragma unroll
    for (int q = 1; q < kFSlices; ++q) v += red[((q - 1) * kFTiles + tl) * 64 + lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 4 * c + i;
      if (m >= M) continue;
      const int64_t o = (int64_t)m * N + (int64_t)tile * kTileRows + r;
      if constexpr (OUT == W4_OUT_F32) static_cast<float*>(a.out)[o] = v[i];
      else static_cast<uint16_t*>(a.out)[o] = bf16_rne(v[i]);
    }
  }
}

// y[m][n] = sum over slices of part[s][m][n], stored as fp32 or bf16.
template <int OUT>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ part, int nslices, int64_t MN,
                                                            void* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= MN) return;
  f32x4 v = *reinterpret_cast<const f32x4*>(part + i);
  for (int s = 1; s < nslices; ++s) v += *reinterpret_cast<const f32x4*>(part + (int64_t)s * MN + i);
  if constexpr (OUT == W4_OUT_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + i) = v;
  } else {
    u32x2 o;
    o[0] = (uint32_t)bf16_rne(v[0]) | ((uint32_t)bf16_rne(v[1]) << 16);
    o[1] = (uint32_t)bf16_rne(v[2]) | ((uint32_t)bf16_rne(v[3]) << 16);
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + i) = o;
  }
}

}  // namespace

bool gemm_splitk_supported(const GemmArgs& a) {
  return a.E == 1 && !a.offsets && a.epilogue == W4_EPI_NONE && a.R >= 1 && a.R <= kMaxRows &&
         slices_of(a.K) >= 2 && (a.N / kTileRows) < 4096;
}

size_t gemm_splitk_workspace(int64_t R, int64_t K, int64_t N) {
  if (R < 1 || R > kMaxRows || K < kGroup) return 0;
  return (size_t)slices_of(K) * (size_t)R * (size_t)N * sizeof(float);
}

static bool fused_fits(const GemmArgs& a);

bool gemm_splitk_needs_workspace(const GemmArgs& a) { return !fused_fits(a); }

static bool fused_fits(const GemmArgs& a) {
  // the fused kernel reads the activation rows as one contiguous block; any
  // K <= kFMaxK fits its slices
  return !a.row_index && a.K <= kFMaxK;
}

template <int MR, int FT, int FS>
void launch_fused(const GemmArgs& a, hipStream_t stream) {
  const int64_t G = a.K / kGroup;
  const int nball = (int)((G + kBlockGroups - 1) / kBlockGroups);
  const int sb = (nball + FS - 1) / FS;
  const int groups = (int)((a.N / kTileRows + FT - 1) / FT);
  const dim3 grid((unsigned)groups), block(64 * FT * FS);
  if (a.out_dtype == W4_OUT_F32)
    hipLaunchKernelGGL((splitk_fused_kernel<W4_OUT_F32, MR, FT, FS>), grid, block, 0, stream, a, sb);
  else
    hipLaunchKernelGGL((splitk_fused_kernel<W4_OUT_BF16, MR, FT, FS>), grid, block, 0, stream, a, sb);
}

void launch_gemm_splitk(const GemmArgs& a, void* ws, hipStream_t stream) {
  if (fused_fits(a)) {
    // LDS holds the rows the call has (1, 4, 8 or 16 of them), so that more
    // workgroups are resident at once; the activations of one row take so
    // little that 1 tile x 8 slices per workgroup fit (a 14336-row matrix:
    // 7168 waves of 4 blocks each).  At K = 4096, N = 14336 (16 rotating
    // weight copies) against 4 x 4 tiles x slices with 16 rows staged for
    // every M: M = 1 12.1 -> 9.5 us, M = 8 12.4 -> 11.8 us.
    if (a.R == 1) launch_fused<1, 1, 8>(a, stream);
    else if (a.R <= 4) launch_fused<4, 2, 4>(a, stream);
    else if (a.R <= 8) launch_fused<8, 2, 4>(a, stream);
    else launch_fused<kMaxRows, 4, 4>(a, stream);
    return;
  }
  const int ns = slices_of(a.K);
  const int tgs = (int)((a.N / kTileRows + kSKWaves - 1) / kSKWaves);
  float* part = static_cast<float*>(ws);
  hipLaunchKernelGGL(splitk_partial_kernel, dim3((unsigned)(tgs * ns)), dim3(64 * kSKWaves), 0, stream, a, ns, part);
  const int64_t MN = a.R * a.N;
  const dim3 rg((unsigned)((MN / 4 + 255) / 256));
  if (a.out_dtype == W4_OUT_F32)
    hipLaunchKernelGGL(splitk_reduce_kernel<W4_OUT_F32>, rg, dim3(256), 0, stream, part, ns, MN, a.out);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<W4_OUT_BF16>, rg, dim3(256), 0, stream, part, ns, MN, a.out);
}

}  // namespace w4
