// Top-k routing plan: token -> expert ids/weights, expert offsets and the
// stable token sort that feeds the grouped matmul.
//
// [RQ] "Repacked QAT Gemma 4 26B-A4B serves on one TPU v6e at 1.9x FP8
// throughput", section "The gap at 26B" (128 experts per layer, 8 active per
// token) and section "What changed in vLLM's TPU backend" (the experts' rows
// are handed to a grouped-matmul backend).
//
// Three kernels:
//  1. topk_rank: a block takes TB tokens (TB*k <= 256 routed rows).  One wave
//     per token finds the top k logits (ties -> lower id) and the softmax
//     weights; then the block ranks its TB*k rows within their expert
//     (ballot-based match inside each wave, prefix over the block's waves) and
//     writes the per-expert row count of the chunk.
//  2. scan: one block turns the chunk counts into per-chunk bases and the
//     expert offsets (exclusive prefix sums).
//  3. scatter: sorted position = offsets[e] + chunk base + rank in chunk.
// Rows of one expert keep their original order r = t*k + j (a stable sort).

#include "common.h"
#include "internal.h"

namespace w4 {

namespace {

constexpr int kRouteThreads = 256;

__host__ __device__ inline int tokens_per_block(int k) { return kRouteThreads / k; }

__global__ void __launch_bounds__(kRouteThreads) topk_rank_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k, int32_t* __restrict__ ids,
    float* __restrict__ weights, int32_t* __restrict__ chunk_counts, int32_t* __restrict__ rank) {
  __shared__ int s_ids[kRouteThreads];
  __shared__ int s_cnt[kRouteThreads / 64][256];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int TB = tokens_per_block(k);
  const int64_t t0 = (int64_t)blockIdx.x * TB;
  const int nvals = (E + 63) / 64;

  for (int tl = wv; tl < TB; tl += kRouteThreads / 64) {
    const int64_t t = t0 + tl;
    if (t >= T) break;
    float v[4];
    float mx = -INFINITY;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int e = lane + 64 * s;
      v[s] = (s < nvals && e < E) ? logits[t * E + e] : -INFINITY;
      mx = fmaxf(mx, v[s]);
    }
    mx = wave_max(mx);
    float sum = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int e = lane + 64 * s;
      if (s < nvals && e < E) sum += expf(v[s] - mx);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
    bool taken[4] = {false, false, false, false};
    for (int j = 0; j < k; ++j) {
      // best of this lane
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int e = lane + 64 * s;
        if (s < nvals && e < E && !taken[s] && (v[s] > bv || (v[s] == bv && e < bi))) {
          bv = v[s];
          bi = e;
        }
      }
      // wave argmax, ties -> lower id
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (lane + 64 * s == bi) taken[s] = true;
      if (lane == 0) {
        ids[t * k + j] = bi;
        weights[t * k + j] = expf(bv - mx) / sum;
        s_ids[tl * k + j] = bi;
      }
    }
  }
  for (int x = threadIdx.x; x < (kRouteThreads / 64) * 256; x += kRouteThreads) (&s_cnt[0][0])[x] = 0;
  __syncthreads();

  // rank each routed row of this chunk within its expert
  const int64_t rows_here_i = (T - t0) < TB ? (T - t0) * k : (int64_t)TB * k;
  const int rows_here = (int)rows_here_i;
  const int rl = threadIdx.x;
  const bool live = rl < rows_here;
  const int e = live ? s_ids[rl] : 0x1ff;   // dead lanes use an id no expert has
  uint64_t same = ~0ull;
#pragma unroll
  for (int bit = 0; bit < 9; ++bit) {
    const uint64_t bal = __ballot((e >> bit) & 1);
    same &= ((e >> bit) & 1) ? bal : ~bal;
  }
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank_in_wave = __popcll(same & lt);
  if (live && rank_in_wave == 0) s_cnt[wv][e] = __popcll(same);
  __syncthreads();
  if (live) {
    int before = 0;
    for (int w = 0; w < wv; ++w) before += s_cnt[w][e];
    rank[t0 * k + rl] = before + rank_in_wave;
  }
  for (int ee = threadIdx.x; ee < E; ee += kRouteThreads) {
    int total = 0;
#pragma unroll
    for (int w = 0; w < kRouteThreads / 64; ++w) total += s_cnt[w][ee];
    chunk_counts[(int64_t)blockIdx.x * E + ee] = total;
  }
}

// One block: chunk counts -> chunk bases (in place), expert offsets.
__global__ void __launch_bounds__(256) scan_kernel(int32_t* __restrict__ chunk_counts, int nchunks, int E,
                                                   int32_t* __restrict__ offsets) {
  __shared__ int s_tot[256];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    for (int ch = 0; ch < nchunks; ++ch) {
      const int c = chunk_counts[(int64_t)ch * E + e];
      chunk_counts[(int64_t)ch * E + e] = run;
      run += c;
    }
  }
  s_tot[e] = (e < E) ? run : 0;
  __syncthreads();
  // exclusive scan over experts (Hillis-Steele on 256 entries)
  for (int o = 1; o < 256; o <<= 1) {
    const int add = (e >= o) ? s_tot[e - o] : 0;
    __syncthreads();
    s_tot[e] += add;
    __syncthreads();
  }
  if (e < E) offsets[e + 1] = s_tot[e];
  if (e == 0) offsets[0] = 0;
}

__global__ void __launch_bounds__(256) scatter_kernel(const int32_t* __restrict__ ids, int64_t R, int E, int k,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ chunk_base,
                                                      const int32_t* __restrict__ rank,
                                                      int32_t* __restrict__ sorted_rows,
                                                      int32_t* __restrict__ sorted_tokens,
                                                      int32_t* __restrict__ row_to_sorted) {
  const int64_t chunk_rows = (int64_t)tokens_per_block(k) * k;
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < R; r += (int64_t)gridDim.x * blockDim.x) {
    const int e = ids[r];
    const int64_t ch = r / chunk_rows;
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
  const int64_t TB = tokens_per_block(k);
  const int64_t nchunks = (T + TB - 1) / TB;
  return (size_t)(nchunks * E + T * k) * sizeof(int32_t);
}

void launch_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* ids, float* weights,
                  int32_t* offsets, int32_t* sorted_rows, int32_t* sorted_tokens, int32_t* row_to_sorted,
                  void* ws, hipStream_t stream) {
  if (T == 0) {
    hipLaunchKernelGGL(zero_offsets_kernel, dim3(1), dim3(256), 0, stream, offsets, E);
    return;
  }
  const int64_t TB = tokens_per_block(k);
  const int64_t nchunks = (T + TB - 1) / TB;
  int32_t* chunk_counts = static_cast<int32_t*>(ws);
  int32_t* rank = chunk_counts + nchunks * E;
  hipLaunchKernelGGL(topk_rank_kernel, dim3((unsigned)nchunks), dim3(kRouteThreads), 0, stream, logits, T, E, k,
                     ids, weights, chunk_counts, rank);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(256), 0, stream, chunk_counts, (int)nchunks, E, offsets);
  const int64_t R = T * k;
  int64_t blocks = (R + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, ids, R, E, k, offsets,
                     chunk_counts, rank, sorted_rows, sorted_tokens, row_to_sorted);
}

}  // namespace w4
