// Top-k routing plan: token -> expert ids/weights, expert offsets and the
// stable token sort that feeds the grouped matmul.
//
// [RQ] "Repacked QAT Gemma 4 26B-A4B serves on one TPU v6e at 1.9x FP8
// throughput", section "The gap at 26B" (128 experts per layer, 8 active per
// token) and section "What changed in vLLM's TPU backend" (the experts' rows
// are handed to a grouped-matmul backend).
//
// Top-k: one wave per token, lane l holding logits l, l+64, ...  Slot j is a
// wave-wide argmax over the logits not yet taken: DPP max within each 16-lane
// row, four readlanes across the rows, then ballots pick the lowest id holding
// that maximum (ties go to the lower id).  The first round's maximum is the
// softmax shift; the sum is one butterfly.
//
// Sort: the T*k routed rows r = t*k + j are grouped by expert, keeping r order
// within an expert.  Small plans (R <= kSmallRows) are sorted by one
// workgroup that counts, ranks, scans and scatters.  Larger plans use chunks
// of the rows:
// a kernel ranks each chunk's rows within their expert (ballot-based match
// inside each wave, prefix over the waves), one block scans the chunk counts
// into offsets, and a scatter kernel writes the permutation.

#include "common.h"
#include "internal.h"

namespace w4 {

namespace {

constexpr int kTopkWaves = 2;       // tokens per top-k workgroup (spread over many CUs)
constexpr int kChunkThreads = 256;  // routed rows per ranking chunk
constexpr int kSmallRows = 4096;    // single-workgroup sort up to this many rows
constexpr int kSmallThreads = 1024;

// Token t on one wave: ids[t][0..k) by descending logit (ties: lower id
// first) and their softmax probabilities.  E <= 64*S <= 256, k <= E, finite
// logits.
template <int S>
__device__ __forceinline__ void topk_token(const float* __restrict__ logits, int64_t t, int E, int k, int lane,
                                           int32_t* __restrict__ ids, float* __restrict__ weights) {
  float v[S];
  bool live[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int e = lane + 64 * s;
    live[s] = e < E;
    v[s] = live[s] ? logits[t * E + e] : -INFINITY;
  }
  unsigned taken = 0;
  float mx = 0.f, sum = 0.f;
  for (int j = 0; j < k; ++j) {
    float cand = -INFINITY;
#pragma unroll
    for (int s = 0; s < S; ++s)
      if (live[s] && !((taken >> s) & 1u)) cand = fmaxf(cand, v[s]);
    const float m = wave_max_all(cand);
    if (j == 0) token_softmax_terms<S>(v, live, mx, sum);
    int sel = -1;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint64_t bal = __ballot(live[s] && !((taken >> s) & 1u) && v[s] == m);
      if (sel < 0 && bal != 0ull) sel = 64 * s + __builtin_ctzll(bal);
    }
    if ((sel & 63) == lane) taken |= 1u << (sel >> 6);
    if (lane == 0) {
      ids[t * k + j] = sel;
      weights[t * k + j] = expf(m - mx) / sum;
    }
  }
}

template <int S>
__global__ void __launch_bounds__(64 * kTopkWaves) topk_kernel(const float* __restrict__ logits, int64_t T, int E,
                                                               int k, int32_t* __restrict__ ids,
                                                               float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kTopkWaves + (threadIdx.x >> 6);
  if (t >= T) return;   // wave-uniform; no barriers in this kernel
  topk_token<S>(logits, t, E, k, lane, ids, weights);
}

// rank of each lane's row among the wave's rows with the same expert id
// (ids < 512; dead lanes pass 0x1ff), and the size of its id group
__device__ __forceinline__ void wave_match(int e, int lane, int& rank_in_wave, int& group) {
  uint64_t same = ~0ull;
#pragma unroll
  for (int bit = 0; bit < 9; ++bit) {
    const uint64_t bal = __ballot((e >> bit) & 1);
    same &= ((e >> bit) & 1) ? bal : ~bal;
  }
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  rank_in_wave = __popcll(same & lt);
  group = __popcll(same);
}

// One workgroup for the whole plan (R <= kSmallRows).
__global__ void __launch_bounds__(kSmallThreads) sort_small_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                                  int k, int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ sorted_rows,
                                                                  int32_t* __restrict__ sorted_tokens,
                                                                  int32_t* __restrict__ row_to_sorted) {
  constexpr int NW = kSmallThreads / 64;
  __shared__ int s_ids[kSmallRows];
  __shared__ int s_cnt[NW][256];   // per-wave counts of the current pass
  __shared__ int s_base[256];      // rows of each expert seen in earlier passes
  __shared__ int s_off[257];
  __shared__ int s_wtot[4];
  __shared__ int s_rank[kSmallRows];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int r = tid; r < R; r += kSmallThreads) s_ids[r] = ids[r];
  for (int x = tid; x < 256; x += kSmallThreads) s_base[x] = 0;
  for (int r0 = 0; r0 < R; r0 += kSmallThreads) {
    for (int x = tid; x < NW * 256; x += kSmallThreads) (&s_cnt[0][0])[x] = 0;
    __syncthreads();
    const int r = r0 + tid;
    const bool live = r < R;
    const int e = live ? s_ids[r] : 0x1ff;
    int rw, grp;
    wave_match(e, lane, rw, grp);
    if (live && rw == 0) s_cnt[wv][e] = grp;
    __syncthreads();
    if (live) {
      int before = s_base[e];
      for (int w = 0; w < wv; ++w) before += s_cnt[w][e];
      s_rank[r] = before + rw;
    }
    __syncthreads();
    for (int x = tid; x < E; x += kSmallThreads) {
      int add = 0;
      for (int w = 0; w < NW; ++w) add += s_cnt[w][x];
      s_base[x] += add;
    }
    __syncthreads();   // the next pass clears s_cnt
  }
  // exclusive scan of the E <= 256 counts: waves 0..3 scan 64 each
  int incl = 0, own = 0;
  if (tid < 256) {
    own = tid < E ? s_base[tid] : 0;
    incl = own;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int up = __shfl_up(incl, o, 64);
      if (lane >= o) incl += up;
    }
    if (lane == 63) s_wtot[wv] = incl;
  }
  __syncthreads();
  if (tid < 256) {
    int before = 0;
    for (int w = 0; w < wv; ++w) before += s_wtot[w];
    if (tid < E) s_off[tid] = before + incl - own;
    if (tid == E - 1) s_off[E] = before + incl;
  }
  __syncthreads();
  for (int x = tid; x <= E; x += kSmallThreads) offsets[x] = s_off[x];
  for (int r = tid; r < R; r += kSmallThreads) {
    const int pos = s_off[s_ids[r]] + s_rank[r];
    sorted_rows[pos] = r;
    sorted_tokens[pos] = r / k;
    row_to_sorted[r] = pos;
  }
}

// Large plans, step 1: rank each chunk's rows within their expert.
__global__ void __launch_bounds__(kChunkThreads) rank_chunks_kernel(const int32_t* __restrict__ ids, int64_t R, int E,
                                                                    int32_t* __restrict__ chunk_counts,
                                                                    int32_t* __restrict__ rank) {
  __shared__ int s_cnt[kChunkThreads / 64][256];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int x = tid; x < (kChunkThreads / 64) * 256; x += kChunkThreads) (&s_cnt[0][0])[x] = 0;
  __syncthreads();
  const int64_t r = (int64_t)blockIdx.x * kChunkThreads + tid;
  const bool live = r < R;
  const int e = live ? ids[r] : 0x1ff;
  int rw, grp;
  wave_match(e, lane, rw, grp);
  if (live && rw == 0) s_cnt[wv][e] = grp;
  __syncthreads();
  if (live) {
    int before = 0;
    for (int w = 0; w < wv; ++w) before += s_cnt[w][e];
    rank[r] = before + rw;
  }
  for (int x = tid; x < E; x += kChunkThreads) {
    int total = 0;
#pragma unroll
    for (int w = 0; w < kChunkThreads / 64; ++w) total += s_cnt[w][x];
    chunk_counts[(int64_t)blockIdx.x * E + x] = total;
  }
}

// Large plans, step 2: chunk counts -> chunk bases (in place) and offsets.
__global__ void __launch_bounds__(256) scan_kernel(int32_t* __restrict__ chunk_counts, int nchunks, int E,
                                                   int32_t* __restrict__ offsets) {
  __shared__ int s_tot[256];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    int ch = 0;
    for (; ch + 8 <= nchunks; ch += 8) {   // independent loads in flight, then the running sum
      int c[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) c[q] = chunk_counts[(int64_t)(ch + q) * E + e];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        chunk_counts[(int64_t)(ch + q) * E + e] = run;
        run += c[q];
      }
    }
    for (; ch < nchunks; ++ch) {
      const int cc = chunk_counts[(int64_t)ch * E + e];
      chunk_counts[(int64_t)ch * E + e] = run;
      run += cc;
    }
  }
  s_tot[e] = (e < E) ? run : 0;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {   // inclusive scan over experts (Hillis-Steele)
    const int add = (e >= o) ? s_tot[e - o] : 0;
    __syncthreads();
    s_tot[e] += add;
    __syncthreads();
  }
  if (e < E) offsets[e + 1] = s_tot[e];
  if (e == 0) offsets[0] = 0;
}

// Large plans, step 3: sorted position = offset + chunk base + rank in chunk.
__global__ void __launch_bounds__(256) scatter_kernel(const int32_t* __restrict__ ids, int64_t R, int E, int k,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ chunk_base,
                                                      const int32_t* __restrict__ rank,
                                                      int32_t* __restrict__ sorted_rows,
                                                      int32_t* __restrict__ sorted_tokens,
                                                      int32_t* __restrict__ row_to_sorted) {
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < R; r += (int64_t)gridDim.x * blockDim.x) {
    const int e = ids[r];
    const int64_t ch = r / kChunkThreads;
    const int pos = offsets[e] + chunk_base[ch * E + e] + rank[r];
    sorted_rows[pos] = (int32_t)r;
    sorted_tokens[pos] = (int32_t)(r / k);
    row_to_sorted[r] = pos;
  }
}

__global__ void zero_offsets_kernel(int32_t* offsets, int E) {
  for (int e = threadIdx.x; e <= E; e += blockDim.x) offsets[e] = 0;
}

}  // namespace

size_t route_workspace_bytes(int64_t T, int32_t E, int32_t k) {
  const int64_t R = T * k;
  const int64_t nchunks = (R + kChunkThreads - 1) / kChunkThreads;
  return (size_t)(nchunks * E + R) * sizeof(int32_t);
}

void launch_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids, float* weights,
                 hipStream_t stream) {
  if (T == 0) return;
  const dim3 tg((unsigned)((T + kTopkWaves - 1) / kTopkWaves)), tb(64 * kTopkWaves);
  if (E <= 64) hipLaunchKernelGGL(topk_kernel<1>, tg, tb, 0, stream, logits, T, E, k, ids, weights);
  else if (E <= 128) hipLaunchKernelGGL(topk_kernel<2>, tg, tb, 0, stream, logits, T, E, k, ids, weights);
  else hipLaunchKernelGGL(topk_kernel<4>, tg, tb, 0, stream, logits, T, E, k, ids, weights);
}

void launch_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids, float* weights,
                  int32_t* offsets, int32_t* sorted_rows, int32_t* sorted_tokens, int32_t* row_to_sorted,
                  void* ws, hipStream_t stream) {
  if (T == 0) {
    hipLaunchKernelGGL(zero_offsets_kernel, dim3(1), dim3(256), 0, stream, offsets, E);
    return;
  }
  const int64_t R = T * k;
  launch_topk(logits, T, E, k, ids, weights, stream);
  if (R <= kSmallRows) {
    hipLaunchKernelGGL(sort_small_kernel, dim3(1), dim3(kSmallThreads), 0, stream, ids, (int)R, E, k, offsets,
                       sorted_rows, sorted_tokens, row_to_sorted);
    return;
  }
  const int64_t nchunks = (R + kChunkThreads - 1) / kChunkThreads;
  int32_t* chunk_counts = static_cast<int32_t*>(ws);
  int32_t* rank = chunk_counts + nchunks * E;
  hipLaunchKernelGGL(rank_chunks_kernel, dim3((unsigned)nchunks), dim3(kChunkThreads), 0, stream, ids, R, E,
                     chunk_counts, rank);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(256), 0, stream, chunk_counts, (int)nchunks, E, offsets);
  int64_t blocks = (R + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ids, R, E, k, offsets,
                     chunk_counts, rank, sorted_rows, sorted_tokens, row_to_sorted);
}

}  // namespace w4
