// FP8 (W8A8, OCP E4M3) comparison path: the format the pages set against
// W4A16 on the same chip.
//
// [RQ] "Repacked QAT Gemma 4 26B-A4B serves on one TPU v6e at 1.9x FP8
// throughput", section "What happened": the W4A16 build is compared with an
// FP8 build of the same model.  [VG] "Compression Without Regret", sections
// "2. What you can quantize" and "3. The precision ladder": FP8 quantizes
// weights and activations and runs the matmul natively in low precision.
// Readings (the pages fix neither): OCP E4M3 codes, one fp32 scale per weight
// row (output channel), activations quantized per row at run time with scale
// amax / 448.
//
// Kernels:
//  * quant_rows_kernel: one wave per row; amax, s = amax / 448 (IEEE fp32
//    division; 1 for a zero row), code = E4M3(clamp(x / s, +-448)) through
//    the hardware conversion (round to nearest even).
//  * The matmuls run on the gfx950 FP8 matrix cores (16x16x128 MFMA, E4M3 x
//    E4M3, fp32 accumulation).  Lane (r, c) supplies row r of the A tile and
//    row r of the B tile (a weight row), both at bytes [32c, 32c+32) of a
//    128-byte K step, so the K elements the MFMA pairs come from the same
//    column whatever order the matrix core takes them in.  Columns past K read
//    as zeros (buffer range checks).  Epilogue: acc * s_x[row] * s_w[col],
//    then the gated activation or the plain store at the sorted row.
//  * fp8_stream_kernel (few rows per expert, bound by the weight bytes): each
//    wave takes units (expert, weight tile, or gate/up tile pair) in turn,
//    streams the unit's weight rows through a register ring D steps deep
//    together with the activation rows (read straight from L2), with no LDS
//    and no barriers.  The unit's first weight loads go out before its rows
//    are read.
//  * fp8_tiled_kernel (many rows per expert): work items (expert, 128-row
//    tile, 256-weight-row column block) as in the W4A16 tiled kernel; 4
//    waves, each owning 4 weight tiles; the block's activation rows go to an
//    LDS ring of 4 steps by DMA, three steps ahead, and the weights come
//    through a two-step register ring.

#include <type_traits>

#include "common.h"
#include "internal.h"
#include "w4a16.h"

namespace w4 {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kNW = 4;                  // waves per block
constexpr int kWT = 4;                  // 16-row weight tiles per wave
constexpr int kBT = kNW * kWT;          // weight tiles per block
constexpr int kKS = 128;                // K bytes per MFMA step
constexpr int kAStride = kKS + 16;      // LDS row stride of a staged activation step
constexpr int kRsrcFlags = 0x00020000;  // raw buffer descriptor word 3 (32-bit data, no swizzle)
// A buffer offset past every range (ranges stay below 2^31), also after the
// +16 of a lane's second 16-byte load: such loads return zeros.
constexpr uint32_t kOOB = 0x80000000u;
constexpr float kE4M3Max = 448.0f;

// E4M3 x E4M3 -> fp32, 16x16x128; unit block scales (E8M0 127 = 2^0).
__device__ __forceinline__ f32x4 mfma_fp8(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ int xcd_item(int b, int total) {
  const int xcd = b & 7, idx = b >> 3;
  const int per = total >> 3, rem = total & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

// ---------------------------------------------------------------- quantize
// 8 bf16 values of a 16-byte chunk -> 8 E4M3 codes (two words), x / s clamped
__device__ __forceinline__ void chunk_to_e4m3(u32x4 v, float s, uint32_t w[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float f[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      f[2 * i] = fminf(fmaxf(bf16_to_f32(v[2 * h + i] & 0xFFFFu) / s, -kE4M3Max), kE4M3Max);
      f[2 * i + 1] = fminf(fmaxf(bf16_to_f32(v[2 * h + i] >> 16) / s, -kE4M3Max), kE4M3Max);
    }
    int p = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    p = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], p, true);
    w[h] = (uint32_t)p;
  }
}

// NCH > 0: the row (at most NCH 16-byte chunks per lane) is loaded into
// registers at once and quantized from there; NCH = 0: any K, read twice.
template <int NCH>
__global__ void __launch_bounds__(256) quant_rows_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t K,
                                                         uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + row * K);
  const int nch = (int)(K / 8);   // 8 values per 16-byte chunk
  uint32_t* dst = reinterpret_cast<uint32_t*>(q + row * K);
  uint32_t m = 0;
  u32x4 v[NCH > 0 ? NCH : 1];
  if constexpr (NCH > 0) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int ch = lane + 64 * k;
      v[k] = ch < nch ? src[ch] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < NCH; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m = max(m, v[k][i] & 0x7FFFu);
        m = max(m, (v[k][i] >> 16) & 0x7FFFu);
      }
  } else {
    for (int ch = lane; ch < nch; ch += 64) {
      const u32x4 c = src[ch];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m = max(m, c[i] & 0x7FFFu);
        m = max(m, (c[i] >> 16) & 0x7FFFu);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
  const float amax = bf16_to_f32(m);
  const float s = amax > 0.f ? amax / kE4M3Max : 1.0f;
  if constexpr (NCH > 0) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int ch = lane + 64 * k;
      if (ch < nch) {
        uint32_t w[2];
        chunk_to_e4m3(v[k], s, w);
        dst[2 * ch] = w[0];
        dst[2 * ch + 1] = w[1];
      }
    }
  } else {
    for (int ch = lane; ch < nch; ch += 64) {
      uint32_t w[2];
      chunk_to_e4m3(src[ch], s, w);
      dst[2 * ch] = w[0];
      dst[2 * ch + 1] = w[1];
    }
  }
  if (lane == 0) scale[row] = s;
}

// ------------------------------------------------------------------ matmul
struct Item {
  int expert, mtile, nblock;
};

// Item of block `blk` over the experts' row tiles (ceil(count / BM) each, in
// expert order) times ncol column blocks; expert -1 past the end.  E <= 256.
template <int BM>
__device__ Item find_item(const int32_t* offsets, int E, int64_t R, int ncol, int blk) {
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
  const int total = __shfl(incl, 63, 64) * ncol;
  if (blk >= total) return it;
  const int item = xcd_item(blk, total);
  const int lin = item / ncol;
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
  it.nblock = item - lin * ncol;
  return it;
}

// s_waitcnt vmcnt(N) lgkmcnt(0): at most N vector-memory operations of this
// wave still in flight, and every LDS access of this wave complete.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// Workgroup barrier without a memory fence: the waits are explicit.
__device__ __forceinline__ void barrier_only() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Chunk swizzle of a staged 128-byte activation row: 16-byte chunk h of row
// r sits at chunk h ^ aswz(r), which keeps the DMA writes and the operand
// reads free of bank conflicts.
__device__ __forceinline__ int aswz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

template <int V>
using IC = std::integral_constant<int, V>;

// Pipeline (one step = 128 bytes of K):
//  * activations: an LDS ring of 4 steps (16 KiB each, BM = 128 rows), filled
//    by buffer_load ... lds three steps ahead; one array per ring slot, named
//    at compile time, so that the compiler's wait before an operand read
//    covers only that slot's DMA;
//  * weights: each lane's 32 bytes of its 4 tiles' rows per step, a register
//    ring D = 2 steps deep;
//  * every step issues the same number of loads (re-reads past the end), so
//    the wait at a step's end is a constant: A(s+1) has landed once at most
//    32 loads are younger (B(s), A(s+2), B(s+1), A(s+3), B(s+2)); the
//    prologue issues A(0), A(1), B(0), A(2), B(1), which makes that count
//    hold from the first step on.
template <int MT, int D, int EPI, int OUT>
__global__ void __launch_bounds__(64 * kNW) __attribute__((amdgpu_waves_per_eu(2)))
fp8_tiled_kernel(Fp8Args a, int ncol) {
  constexpr bool GATED = EPI != W4_EPI_NONE;
  constexpr int BM = 16 * MT;
  constexpr int NST = 4;
  constexpr int ASTAGE = BM * kKS;                   // 16 KiB
  constexpr int AQ = ASTAGE / (1024 * kNW);          // DMA instructions per wave per step
  static_assert(D == 2, "the end-of-step wait assumes a two-step weight ring");
  __shared__ __align__(16) uint8_t As0[ASTAGE];
  __shared__ __align__(16) uint8_t As1[ASTAGE];
  __shared__ __align__(16) uint8_t As2[ASTAGE];
  __shared__ __align__(16) uint8_t As3[ASTAGE];
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

  const Item it = find_item<BM>(a.offsets, a.E, a.R, ncol, blockIdx.x);
  if (it.expert < 0) return;   // uniform over the block
  const int e = __builtin_amdgcn_readfirstlane(it.expert);
  const int mt = __builtin_amdgcn_readfirstlane(it.mtile);
  const int nb = __builtin_amdgcn_readfirstlane(it.nblock);
  const int64_t e_begin = a.offsets ? a.offsets[e] : 0;
  const int64_t e_end = a.offsets ? a.offsets[e + 1] : a.R;
  const int64_t row_begin = e_begin + (int64_t)mt * BM;
  const int cnt = (int)(e_end - row_begin < BM ? e_end - row_begin : BM);

  // this wave's weight tiles; in a last, partial column block the waves
  // without tiles stage activations and meet the barriers only (their
  // weight loads read nothing, so every wave's load count is the same)
  const int tiles_total = (int)(N / kTileRows);
  int tile[kWT];
  bool active;
  {
    const int per_wave = GATED ? 2 : kWT;
    const int left = GATED ? tiles_total / 2 - nb * (kBT / 2) : tiles_total - nb * kBT;
    active = wv < left / per_wave;
    if constexpr (GATED) {
      const int half = tiles_total / 2;
      const int g0 = nb * (kBT / 2) + wv * 2;
      tile[0] = g0;
      tile[1] = g0 + 1;
      tile[2] = g0 + half;
      tile[3] = g0 + 1 + half;
    } else {
      const int t0 = nb * kBT + wv * kWT;
#pragma unroll
      for (int t = 0; t < kWT; ++t) tile[t] = t0 + t;
    }
    if (!active) {
#pragma unroll
      for (int t = 0; t < kWT; ++t) tile[t] = 0;
    }
  }

  const int nks = (int)((K + kKS - 1) / kKS);
  const int last = nks - 1;
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.wq + (int64_t)e * N * K), 0, (int)(N * K), kRsrcFlags);
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.xq, 0, (int)(a.x_rows * K), kRsrcFlags);

  // weights: lane's 32 bytes of each tile's row at step ks (zeros past K)
  uint32_t woff[kWT];
#pragma unroll
  for (int t = 0; t < kWT; ++t) woff[t] = (uint32_t)((int64_t)(tile[t] * kTileRows + r) * K) + 32u * (uint32_t)c;
  i32x8 bw[D][kWT];
  // (offsets of dead lanes get bit 31 set -- past every range, so they read
  // zeros -- by arithmetic, not a select the compiler could turn into
  // branches around the loads)
  auto b_issue = [&](int slot, int ks) __attribute__((always_inline)) {
    const uint32_t dead = (uint32_t)(!active || (int64_t)ks * kKS + 32 * c >= K);
#pragma unroll
    for (int t = 0; t < kWT; ++t) {
      const uint32_t off = (woff[t] + (uint32_t)(ks * kKS)) | (dead << 31);
      const i32x4 lo = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0));
      const i32x4 hi = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, off + 16u, 0, 0));
      bw[slot][t] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };

  // activation DMA: wave wv's instruction q fills bytes [1024n, 1024n + 1024)
  // of a step buffer, n = AQ*wv + q: rows 8n .. 8n+7, lane -> row 8n + lane/8,
  // chunk slot lane % 8, which holds source chunk slot ^ aswz(row); chunks
  // past K read zeros
  uint32_t aoff[AQ];
  int achk[AQ];
#pragma unroll
  for (int q = 0; q < AQ; ++q) {
    const int n = AQ * wv + q;
    const int rr = 8 * n + (lane >> 3);
    const int ch = (lane & 7) ^ aswz(rr);
    const int64_t row = row_begin + (rr < cnt ? rr : 0);
    const int64_t src = a.row_index ? (int64_t)a.row_index[row] : row;
    aoff[q] = (uint32_t)(src * K) + 16u * (uint32_t)ch;
    achk[q] = 16 * ch;
  }
  auto a_issue = [&](int st, auto J) __attribute__((always_inline)) {
    uint8_t* dst = slot_buf(J) + (AQ * wv) * 1024;
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const uint32_t dead = (uint32_t)((int64_t)st * kKS + achk[q] >= K);
      const uint32_t voff = (aoff[q] + (uint32_t)(st * kKS)) | (dead << 31);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(dst + q * 1024), 16,
                                               voff, 0, 0, 0);
    }
  };

  f32x4 acc[MT][kWT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < kWT; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // operand reads: row 16i + r, K bytes 32c .. 32c+31 = chunks 2c, 2c+1
  const int apos_lo = r * kKS + ((2 * c) ^ aswz(r)) * 16;
  const int apos_hi = r * kKS + ((2 * c + 1) ^ aswz(r)) * 16;
  auto read_a = [&](const uint8_t* Ab, int i) __attribute__((always_inline)) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(Ab + apos_lo + i * 16 * kKS);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(Ab + apos_hi + i * 16 * kKS);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  auto step = [&](int s, auto J) __attribute__((always_inline)) {
    constexpr int j = decltype(J)::value;   // s % NST
    constexpr int sl = j % D;               // s % D
    a_issue(s + NST - 1 <= last ? s + NST - 1 : last, IC<j + NST - 1>{});
    __builtin_amdgcn_sched_barrier(0);
    if (active) {
      const uint8_t* Ab = slot_buf(J);
      i32x8 A = read_a(Ab, 0);
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const i32x8 An = i + 1 < MT ? read_a(Ab, i + 1) : A;
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < kWT; ++t) acc[i][t] = mfma_fp8(A, bw[sl][t], acc[i][t]);
        __builtin_amdgcn_sched_barrier(0);
        A = An;
      }
    }
    b_issue(sl, s + D <= last ? s + D : last);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<3 * 2 * kWT + 2 * AQ>();   // A(s+1) has landed (see above)
    barrier_only();
  };

  // prologue, in the order the steps would have issued them: A(0), A(1),
  // B(0), A(2), B(1); then wait for A(0)
  a_issue(0, IC<0>{});
  a_issue(1 <= last ? 1 : last, IC<1>{});
  b_issue(0, 0);
  a_issue(2 <= last ? 2 : last, IC<2>{});
  b_issue(1, 1 <= last ? 1 : last);
  wait_vm<2 * 2 * kWT + 2 * AQ>();
  barrier_only();

  int s = 0;
#pragma unroll 1
  for (; s + 3 < nks; s += 4) {
    step(s, IC<0>{});
    step(s + 1, IC<1>{});
    step(s + 2, IC<2>{});
    step(s + 3, IC<3>{});
  }
  if (s < nks) step(s, IC<0>{});
  if (s + 1 < nks) step(s + 1, IC<1>{});
  if (s + 2 < nks) step(s + 2, IC<2>{});
  wait_vm<0>();   // the re-reads past the end

  if (!active) return;
  // D element q of row tile i: row 16i + 4c + q, weight row r of each tile
  float sw[kWT];
#pragma unroll
  for (int t = 0; t < kWT; ++t) sw[t] = a.ws[(int64_t)e * N + tile[t] * kTileRows + r];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = 16 * i + 4 * c + q;
      if (rr >= cnt) continue;
      const int64_t row = row_begin + rr;
      const int64_t src = a.row_index ? (int64_t)a.row_index[row] : row;
      const float sx = a.xs[src];
      if constexpr (GATED) {
        uint16_t* orow = static_cast<uint16_t*>(a.out) + row * (N / 2) + r;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const float g = bf16_to_f32(f32_to_bf16(acc[i][t][q] * sx * sw[t]));
          const float u = bf16_to_f32(f32_to_bf16(acc[i][t + 2][q] * sx * sw[t + 2]));
          const float act = (EPI == W4_EPI_GEGLU_TANH) ? gelu_tanh_f32(g) : silu_f32(g);
          orow[tile[t] * kTileRows] = (uint16_t)f32_to_bf16(act * u);
        }
      } else if constexpr (OUT == W4_OUT_F32) {
        float* orow = static_cast<float*>(a.out) + row * N + r;
#pragma unroll
        for (int t = 0; t < kWT; ++t) orow[tile[t] * kTileRows] = acc[i][t][q] * sx * sw[t];
      } else {
        uint16_t* orow = static_cast<uint16_t*>(a.out) + row * N + r;
#pragma unroll
        for (int t = 0; t < kWT; ++t) orow[tile[t] * kTileRows] = (uint16_t)f32_to_bf16(acc[i][t][q] * sx * sw[t]);
      }
    }
  }
}

// Few rows per expert.  Unit u of expert e: weight tile u (plain) or gate
// tile u with its up tile u + N/32 (gated).  Wave w of W takes units w, w+W, ...
template <int EPI, int OUT, int D>
__global__ void __launch_bounds__(64 * kNW) __attribute__((amdgpu_waves_per_eu(3)))
fp8_stream_kernel(Fp8Args a, int units_per_expert, int total_units) {
  constexpr bool GATED = EPI != W4_EPI_NONE;
  constexpr int NT = GATED ? 2 : 1;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int c = lane >> 4;
  const int64_t K = a.K, N = a.N;
  const int nks = (int)((K + kKS - 1) / kKS);
  const int W = (int)gridDim.x * kNW;
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.xq, 0, (int)(a.x_rows * K), kRsrcFlags);

  for (int unit = __builtin_amdgcn_readfirstlane((int)blockIdx.x * kNW + (int)(threadIdx.x >> 6)); unit < total_units;
       unit += W) {
    const int e = unit / units_per_expert;
    const int u = unit - e * units_per_expert;
    int tile[NT];
    tile[0] = u;
    if constexpr (GATED) tile[1] = u + (int)(N / 32);
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.wq + (int64_t)e * N * K), 0, (int)(N * K), kRsrcFlags);
    uint32_t woff[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) woff[t] = (uint32_t)((int64_t)(tile[t] * kTileRows + r) * K) + 32u * (uint32_t)c;
    u32x4 bw[D][NT][2];
    u32x4 ax[D][2];
    uint32_t aoff = kOOB;
    auto b_issue = [&](int slot, int ks) __attribute__((always_inline)) {
      const bool live = (int64_t)ks * kKS + 32 * c < K;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t off = live ? woff[t] + (uint32_t)(ks * kKS) : kOOB;
        bw[slot][t][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0));
        bw[slot][t][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, off + 16u, 0, 0));
      }
    };
    auto a_issue = [&](int slot, int ks) __attribute__((always_inline)) {
      const bool live = aoff != kOOB && (int64_t)ks * kKS + 32 * c < K;
      const uint32_t off = live ? aoff + (uint32_t)(ks * kKS) : kOOB;
      ax[slot][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off, 0, 0));
      ax[slot][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16u, 0, 0));
    };
    // the weight ring does not depend on the rows: issue it first
#pragma unroll
    for (int s = 0; s < D; ++s) b_issue(s, s < nks ? s : nks - 1);
    const int64_t e_begin = a.offsets ? a.offsets[e] : 0;
    const int64_t e_end = a.offsets ? a.offsets[e + 1] : a.R;
    for (int64_t row0 = e_begin; row0 < e_end; row0 += 16) {
      const int cnt = (int)(e_end - row0 < 16 ? e_end - row0 : 16);
      {
        const int64_t row = row0 + (r < cnt ? r : 0);
        const int64_t src = a.row_index ? (int64_t)a.row_index[row] : row;
        aoff = (uint32_t)(src * K) + 32u * (uint32_t)c;
      }
      if (row0 != e_begin) {   // a second row tile re-streams the weights
#pragma unroll
        for (int s = 0; s < D; ++s) b_issue(s, s < nks ? s : nks - 1);
      }
#pragma unroll
      for (int s = 0; s < D; ++s) a_issue(s, s < nks ? s : nks - 1);
      f32x4 acc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      auto step = [&](int ks, auto SLOT) __attribute__((always_inline)) {
        constexpr int sl = decltype(SLOT)::value;
        const i32x8 A = {(int)ax[sl][0][0], (int)ax[sl][0][1], (int)ax[sl][0][2], (int)ax[sl][0][3],
                         (int)ax[sl][1][0], (int)ax[sl][1][1], (int)ax[sl][1][2], (int)ax[sl][1][3]};
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const i32x8 B = {(int)bw[sl][t][0][0], (int)bw[sl][t][0][1], (int)bw[sl][t][0][2], (int)bw[sl][t][0][3],
                           (int)bw[sl][t][1][0], (int)bw[sl][t][1][1], (int)bw[sl][t][1][2], (int)bw[sl][t][1][3]};
          acc[t] = mfma_fp8(A, B, acc[t]);
        }
        const int kn = ks + D < nks ? ks + D : nks - 1;
        b_issue(sl, kn);
        a_issue(sl, kn);
      };
      int ks = 0;
#pragma unroll 1
      for (; ks + D <= nks; ks += D) {
        [&]<int... S>(std::integer_sequence<int, S...>) {
          (step(ks + S, std::integral_constant<int, S>{}), ...);
        }(std::make_integer_sequence<int, D>{});
      }
      [&]<int... S>(std::integer_sequence<int, S...>) {
        ((ks + S < nks ? step(ks + S, std::integral_constant<int, S>{}) : void()), ...);
      }(std::make_integer_sequence<int, D>{});
      // D element q: row 4c + q, weight row r of each tile
      float sw[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) sw[t] = a.ws[(int64_t)e * N + tile[t] * kTileRows + r];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rr = 4 * c + q;
        if (rr >= cnt) continue;
        const int64_t row = row0 + rr;
        const int64_t src = a.row_index ? (int64_t)a.row_index[row] : row;
        const float sx = a.xs[src];
        if constexpr (GATED) {
          const float g = bf16_to_f32(f32_to_bf16(acc[0][q] * sx * sw[0]));
          const float up = bf16_to_f32(f32_to_bf16(acc[1][q] * sx * sw[1]));
          const float act = (EPI == W4_EPI_GEGLU_TANH) ? gelu_tanh_f32(g) : silu_f32(g);
          static_cast<uint16_t*>(a.out)[row * (N / 2) + tile[0] * kTileRows + r] = (uint16_t)f32_to_bf16(act * up);
        } else if constexpr (OUT == W4_OUT_F32) {
          static_cast<float*>(a.out)[row * N + tile[0] * kTileRows + r] = acc[0][q] * sx * sw[0];
        } else {
          static_cast<uint16_t*>(a.out)[row * N + tile[0] * kTileRows + r] =
              (uint16_t)f32_to_bf16(acc[0][q] * sx * sw[0]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);   // the clamped refills past the end
  }
}

template <int EPI, int OUT>
void launch_epi(const Fp8Args& a, bool stream_path, hipStream_t st) {
  const bool gated = EPI != W4_EPI_NONE;
  const int64_t tiles = a.N / kTileRows;
  if (stream_path) {
    const int upe = (int)(gated ? tiles / 2 : tiles);
    const int64_t total = (int64_t)upe * a.E;
    // about three resident waves per SIMD; more blocks would only queue
    const int64_t want = (total + kNW - 1) / kNW;
    const int blocks = (int)(want < 256 * 3 ? want : 256 * 3);
    hipLaunchKernelGGL((fp8_stream_kernel<EPI, OUT, 4>), dim3(blocks), dim3(64 * kNW), 0, st, a, upe, (int)total);
  } else {
    const int ncol = (int)(gated ? (tiles / 2 + kBT / 2 - 1) / (kBT / 2) : (tiles + kBT - 1) / kBT);
    const int64_t blocks = (a.R / 128 + a.E) * ncol;
    hipLaunchKernelGGL((fp8_tiled_kernel<8, 2, EPI, OUT>), dim3((unsigned)blocks), dim3(64 * kNW), 0, st, a, ncol);
  }
}

}  // namespace

bool fp8_gemm_supported(const Fp8Args& a) {
  const int64_t tiles = a.N / kTileRows;
  if (a.E > 256 || a.R >= ((int64_t)1 << 31)) return false;
  if (a.x_rows * a.K >= ((int64_t)1 << 31) || a.N * a.K >= ((int64_t)1 << 31)) return false;
  if (a.epilogue != W4_EPI_NONE) return (tiles / 2) % 2 == 0;
  return tiles % kWT == 0;
}

void launch_fp8_gemm(const Fp8Args& a, hipStream_t stream) {
  // few rows per expert: weight streaming; many: 128-row tiles
  const bool sp = a.R <= (int64_t)kFp8StreamRowsPerExpert * a.E;
  if (a.epilogue == W4_EPI_GEGLU_TANH) launch_epi<W4_EPI_GEGLU_TANH, W4_OUT_BF16>(a, sp, stream);
  else if (a.epilogue == W4_EPI_SWIGLU) launch_epi<W4_EPI_SWIGLU, W4_OUT_BF16>(a, sp, stream);
  else if (a.out_dtype == W4_OUT_F32) launch_epi<W4_EPI_NONE, W4_OUT_F32>(a, sp, stream);
  else launch_epi<W4_EPI_NONE, W4_OUT_BF16>(a, sp, stream);
}

void launch_fp8_quant_rows(const uint16_t* x, int64_t rows, int64_t K, uint8_t* q, float* scale, hipStream_t stream) {
  if (rows <= 0) return;
  // 16-byte chunks per lane of one row: held in registers up to 8
  const int64_t per_lane = (K / 8 + 63) / 64;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (per_lane <= 2) hipLaunchKernelGGL(quant_rows_kernel<2>, grid, block, 0, stream, x, rows, K, q, scale);
  else if (per_lane <= 4) hipLaunchKernelGGL(quant_rows_kernel<4>, grid, block, 0, stream, x, rows, K, q, scale);
  else if (per_lane <= 8) hipLaunchKernelGGL(quant_rows_kernel<8>, grid, block, 0, stream, x, rows, K, q, scale);
  else hipLaunchKernelGGL(quant_rows_kernel<0>, grid, block, 0, stream, x, rows, K, q, scale);
}

}  // namespace w4
