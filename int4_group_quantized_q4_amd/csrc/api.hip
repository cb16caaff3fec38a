// extern "C" entry points of libw4a16.so: argument checks on the host, then
// kernel launches on the caller's stream.  No allocation, no synchronisation.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "internal.h"
#include "w4a16.h"

namespace {

constexpr int kAbiVersion = 2;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? W4_OK : W4_ERR_HIP;
}

int check_matrix(int64_t rows, int64_t K) {
  if (rows < 0 || K < 0) return W4_ERR_ARG;
  if (rows % 16 != 0 || K % 32 != 0) return W4_ERR_SHAPE;
  if (rows > 0 && K > 0 && rows > ((int64_t)1 << 40) / K) return W4_ERR_SHAPE;
  return W4_OK;
}

}  // namespace

extern "C" {

const char* w4a16_status_string(int status) {
  switch (status) {
    case W4_OK: return "W4_OK: success";
    case W4_ERR_ARG: return "W4_ERR_ARG: null pointer, negative size, misaligned pointer or bad enum";
    case W4_ERR_SHAPE: return "W4_ERR_SHAPE: rows % 16 != 0, K % 32 != 0 or a size out of range";
    case W4_ERR_WORKSPACE: return "W4_ERR_WORKSPACE: workspace missing or too small";
    case W4_ERR_HIP: return "W4_ERR_HIP: kernel launch failed";
    default: return "unknown w4a16 status";
  }
}

int w4a16_abi_version(void) { return kAbiVersion; }

int q4_group_repack(const uint16_t* w_bf16, int64_t rows, int64_t K, uint8_t* qweight, uint16_t* scales,
                    uint8_t* group_status, unsigned long long* counters, hipStream_t stream) {
  int st = check_matrix(rows, K);
  if (st != W4_OK) return st;
  if (rows == 0 || K == 0) return W4_OK;
  if (!w_bf16 || !qweight || !scales) return W4_ERR_ARG;
  if (!aligned16(w_bf16) || !aligned16(qweight) || !aligned16(scales)) return W4_ERR_ARG;
  if (counters && !aligned8(counters)) return W4_ERR_ARG;
  w4::launch_repack(w_bf16, rows, K, qweight, scales, group_status, counters, stream);
  return launch_status();
}

int q4_group_dequant_f32(const uint8_t* qweight, const uint16_t* scales, int64_t rows, int64_t K, float* out,
                         hipStream_t stream) {
  int st = check_matrix(rows, K);
  if (st != W4_OK) return st;
  if (rows == 0 || K == 0) return W4_OK;
  if (!qweight || !scales || !out) return W4_ERR_ARG;
  if (!aligned16(qweight) || !aligned16(scales) || !aligned16(out)) return W4_ERR_ARG;
  w4::launch_dequant(qweight, scales, rows, K, out, stream);
  return launch_status();
}

int q4_pack_codes(const int8_t* codes, int64_t rows, int64_t K, uint8_t* qweight, hipStream_t stream) {
  int st = check_matrix(rows, K);
  if (st != W4_OK) return st;
  if (rows == 0 || K == 0) return W4_OK;
  if (!codes || !qweight) return W4_ERR_ARG;
  if (!aligned16(codes) || !aligned16(qweight)) return W4_ERR_ARG;
  w4::launch_pack(codes, rows, K, qweight, stream);
  return launch_status();
}

int q4_pack_scales(const uint16_t* scales, int64_t rows, int64_t K, uint16_t* scales_tiled, hipStream_t stream) {
  int st = check_matrix(rows, K);
  if (st != W4_OK) return st;
  if (rows == 0 || K == 0) return W4_OK;
  if (!scales || !scales_tiled) return W4_ERR_ARG;
  if (!aligned16(scales) || !aligned16(scales_tiled)) return W4_ERR_ARG;
  w4::launch_pack_scales(scales, rows, K, scales_tiled, stream);
  return launch_status();
}

static std::atomic<int> g_gemm_kernel{W4_KERNEL_AUTO};

int w4a16_set_gemm_kernel(int kernel) {
  if (kernel != W4_KERNEL_AUTO && kernel != W4_KERNEL_STREAM && kernel != W4_KERNEL_TILED) return W4_ERR_ARG;
  return g_gemm_kernel.exchange(kernel);
}

static int run_gemm(const w4::GemmArgs& a, void* ws, size_t ws_bytes, hipStream_t stream) {
  // Average rows per expert decides the kernel: weight-streaming (decode) or
  // LDS-tiled MFMA (prefill, needs the workspace for the fp16 activations).
  // the kernels address one expert's codes through 32-bit buffer offsets
  if (a.N * a.K / 2 >= ((int64_t)1 << 31)) return W4_ERR_SHAPE;
  const int policy = g_gemm_kernel.load(std::memory_order_relaxed);
  bool tiled = w4::gemm_tiled_supported(a);
  if (policy == W4_KERNEL_STREAM) tiled = false;
  else if (policy == W4_KERNEL_AUTO) tiled = tiled && a.R > (int64_t)W4_TILED_MIN_ROWS * a.E;
  if (tiled) {
    if (!ws || !aligned16(ws) || ws_bytes < w4::gemm_tiled_workspace(a.x_rows, a.R, a.E, a.K, a.N)) {
      return W4_ERR_WORKSPACE;
    }
    w4::launch_gemm_tiled(a, ws, stream);
  } else if (policy != W4_KERNEL_STREAM && w4::gemm_splitk_supported(a) &&
             (!w4::gemm_splitk_needs_workspace(a) ||
              (ws && aligned16(ws) && ws_bytes >= w4::gemm_splitk_workspace(a.R, a.K, a.N)))) {
    w4::launch_gemm_splitk(a, ws, stream);   // few tiles: split K over more waves
  } else {
    w4::launch_gemm_skinny(a, stream);
  }
  return launch_status();
}

size_t w4a16_linear_workspace(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || K < 0 || N < 0) return 0;
  const size_t tiled = w4::gemm_tiled_workspace(M, M, 1, K, N);
  const size_t splitk = w4::gemm_splitk_workspace(M, K, N);
  return tiled > splitk ? tiled : splitk;
}

size_t w4a16_moe_gmm_workspace(int64_t x_rows, int64_t R, int32_t E, int64_t K, int64_t N) {
  if (x_rows < 0 || R < 0 || E < 1 || K < 0 || N < 0) return 0;
  return w4::gemm_tiled_workspace(x_rows, R, E, K, N);
}

int w4a16_linear(const uint16_t* x, int64_t M, int64_t K, const uint8_t* qweight, const uint16_t* scales, int64_t N,
                 uint16_t* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (M < 0) return W4_ERR_ARG;
  int st = check_matrix(N, K);
  if (st != W4_OK) return st;
  if (M == 0 || N == 0) return W4_OK;
  if (K == 0) return W4_ERR_SHAPE;
  if (M > INT32_MAX) return W4_ERR_SHAPE;
  if (!x || !qweight || !scales || !y) return W4_ERR_ARG;
  if (!aligned16(x) || !aligned16(qweight) || !aligned16(scales) || !aligned16(y)) return W4_ERR_ARG;
  w4::GemmArgs a{};
  a.x = x;
  a.x_rows = M;
  a.row_index = nullptr;
  a.offsets = nullptr;
  a.E = 1;
  a.R = M;
  a.K = K;
  a.N = N;
  a.qweight = qweight;
  a.scales = scales;
  a.epilogue = W4_EPI_NONE;
  a.out = y;
  a.out_dtype = W4_OUT_BF16;
  return run_gemm(a, ws, ws_bytes, stream);
}

size_t w4a16_moe_route_workspace(int64_t T, int32_t E, int32_t k) {
  if (T < 0 || E < 1 || k < 1 || k > E) return 0;
  return w4::route_workspace_bytes(T, E, k);
}

int w4a16_moe_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_ids, float* topk_weights,
                    int32_t* expert_offsets, int32_t* sorted_rows, int32_t* sorted_tokens, int32_t* row_to_sorted,
                    void* ws, size_t ws_bytes, hipStream_t stream) {
  if (T < 0 || E < 1 || E > 256 || k < 1 || k > E || k > 16) return W4_ERR_ARG;
  if (T * (int64_t)k >= ((int64_t)1 << 31)) return W4_ERR_SHAPE;
  if (!expert_offsets) return W4_ERR_ARG;
  if (T > 0) {
    if (!logits || !topk_ids || !topk_weights || !sorted_rows || !sorted_tokens || !row_to_sorted) return W4_ERR_ARG;
    if (!ws || ws_bytes < w4::route_workspace_bytes(T, E, k)) return W4_ERR_WORKSPACE;
  }
  w4::launch_route(logits, T, E, k, topk_ids, topk_weights, expert_offsets, sorted_rows, sorted_tokens, row_to_sorted,
                   ws, stream);
  return launch_status();
}

int w4a16_moe_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_ids, float* topk_weights,
                   hipStream_t stream) {
  if (T < 0 || E < 1 || E > 256 || k < 1 || k > E || k > 16) return W4_ERR_ARG;
  if (T * (int64_t)k >= ((int64_t)1 << 31)) return W4_ERR_SHAPE;
  if (T == 0) return W4_OK;
  if (!logits || !topk_ids || !topk_weights) return W4_ERR_ARG;
  w4::launch_topk(logits, T, E, k, topk_ids, topk_weights, stream);
  return launch_status();
}

// Shape and pointer checks shared by the two ids-mode matmuls.
static int check_gmm_ids(const void* x, const int32_t* ids, int64_t T, int32_t k, int32_t E, int64_t K, int64_t N,
                         const uint8_t* qweight, const uint16_t* scales, const void* out) {
  if (T < 0 || k < 1 || k > 16 || E < 1 || E > 256 || k > E) return W4_ERR_ARG;
  int st = check_matrix(N, K);
  if (st != W4_OK) return st;
  if (T > w4::kIdsMaxExpertRows || T * k > w4::kIdsMaxRows) return W4_ERR_SHAPE;
  if (N * K / 2 >= ((int64_t)1 << 31)) return W4_ERR_SHAPE;
  if (T == 0 || N == 0) return W4_OK;
  if (K == 0) return W4_ERR_SHAPE;
  if (!x || !ids || !qweight || !scales || !out) return W4_ERR_ARG;
  if (!aligned16(x) || !aligned16(qweight) || !aligned16(scales) || !aligned16(out)) return W4_ERR_ARG;
  return W4_OK;
}

int w4a16_moe_gmm_ids(const uint16_t* x, const int32_t* topk_ids, int64_t T, int32_t k, int32_t row_div, int32_t E,
                      int64_t K, int64_t N, const uint8_t* qweight, const uint16_t* scales, int32_t epilogue,
                      void* out, int32_t out_dtype, hipStream_t stream) {
  if (row_div != 1 && row_div != k) return W4_ERR_ARG;
  if (epilogue != W4_EPI_NONE && epilogue != W4_EPI_GEGLU_TANH && epilogue != W4_EPI_SWIGLU) return W4_ERR_ARG;
  if (out_dtype != W4_OUT_BF16 && out_dtype != W4_OUT_F32) return W4_ERR_ARG;
  if (epilogue != W4_EPI_NONE && out_dtype != W4_OUT_BF16) return W4_ERR_ARG;
  int st = check_gmm_ids(x, topk_ids, T, k, E, K, N, qweight, scales, out);
  if (st != W4_OK || T == 0 || N == 0) return st;
  if (epilogue != W4_EPI_NONE && N % 32 != 0) return W4_ERR_SHAPE;
  w4::GemmArgs a{};
  a.x = x;
  a.x_rows = T * k / row_div;
  a.E = E;
  a.R = T * k;
  a.K = K;
  a.N = N;
  a.qweight = qweight;
  a.scales = scales;
  a.epilogue = epilogue;
  a.out = out;
  a.out_dtype = out_dtype;
  a.ids = topk_ids;
  a.kslots = row_div;
  w4::launch_gemm_skinny(a, stream);
  return launch_status();
}

// The gate/up matmul of the streaming path from the logits: its workgroups
// rank the logits when the one-tile streaming kernel takes it (up to 64
// tokens), else the top-k launch and the ids-mode matmul.  a: the ids-mode
// arguments without ids (x_rows = T, R = T*k, kslots = k).
static void enqueue_gateup_from_logits(w4::GemmArgs a, const float* logits, int64_t T, int32_t E, int32_t k,
                                       int32_t* ids, float* wts, hipStream_t stream) {
  a.kslots = k;
  if (w4::gemm_skinny_takes_logits(a, T, logits)) {
    a.logits = logits;
    a.ids_out = ids;
    a.wts_out = wts;
  } else {
    w4::launch_topk(logits, T, E, k, ids, wts, stream);
    a.ids = ids;
  }
  w4::launch_gemm_skinny(a, stream);
}

int w4a16_moe_gmm_logits(const uint16_t* x, const float* logits, int64_t T, int32_t E, int32_t k, int64_t K, int64_t N,
                         const uint8_t* qweight, const uint16_t* scales, int32_t epilogue, uint16_t* out,
                         int32_t* topk_ids, float* topk_weights, hipStream_t stream) {
  if (epilogue != W4_EPI_GEGLU_TANH && epilogue != W4_EPI_SWIGLU) return W4_ERR_ARG;
  int st = check_gmm_ids(x, topk_ids, T, k, E, K, N, qweight, scales, out);
  if (st != W4_OK) return st;
  if (N % 32 != 0) return W4_ERR_SHAPE;
  if (T == 0) return W4_OK;
  if (!logits || !topk_ids || !topk_weights) return W4_ERR_ARG;
  if (N == 0) {   // no matmul, but the plan is still an output
    w4::launch_topk(logits, T, E, k, topk_ids, topk_weights, stream);
    return launch_status();
  }
  w4::GemmArgs a{};
  a.x = x;
  a.x_rows = T;
  a.E = E;
  a.R = T * k;
  a.K = K;
  a.N = N;
  a.qweight = qweight;
  a.scales = scales;
  a.epilogue = epilogue;
  a.out = out;
  a.out_dtype = W4_OUT_BF16;
  enqueue_gateup_from_logits(a, logits, T, E, k, topk_ids, topk_weights, stream);
  return launch_status();
}

int w4a16_moe_gmm(const uint16_t* x, int64_t x_rows, const int32_t* row_index, const int32_t* expert_offsets,
                  int32_t E, int64_t R, int64_t K, int64_t N, const uint8_t* qweight, const uint16_t* scales,
                  int32_t epilogue, void* out, int32_t out_dtype, void* ws, size_t ws_bytes,
                  hipStream_t stream) {
  if (x_rows < 0 || E < 1 || R < 0) return W4_ERR_ARG;
  if (epilogue != W4_EPI_NONE && epilogue != W4_EPI_GEGLU_TANH && epilogue != W4_EPI_SWIGLU) return W4_ERR_ARG;
  if (out_dtype != W4_OUT_BF16 && out_dtype != W4_OUT_F32) return W4_ERR_ARG;
  if (epilogue != W4_EPI_NONE && out_dtype != W4_OUT_BF16) return W4_ERR_ARG;
  int st = check_matrix(N, K);
  if (st != W4_OK) return st;
  if (epilogue != W4_EPI_NONE && N % 32 != 0) return W4_ERR_SHAPE;
  if (R >= ((int64_t)1 << 31) || x_rows >= ((int64_t)1 << 31)) return W4_ERR_SHAPE;
  if (R == 0 || N == 0) return W4_OK;
  if (K == 0) return W4_ERR_SHAPE;
  if (!x || !expert_offsets || !qweight || !scales || !out) return W4_ERR_ARG;
  if (!row_index && x_rows < R) return W4_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(qweight) || !aligned16(scales) || !aligned16(out)) return W4_ERR_ARG;
  w4::GemmArgs a{};
  a.x = x;
  a.x_rows = x_rows;
  a.row_index = row_index;
  a.offsets = expert_offsets;
  a.E = E;
  a.R = R;
  a.K = K;
  a.N = N;
  a.qweight = qweight;
  a.scales = scales;
  a.epilogue = epilogue;
  a.out = out;
  a.out_dtype = out_dtype;
  return run_gemm(a, ws, ws_bytes, stream);
}

int w4a16_moe_combine(const void* o, int32_t o_dtype, const int32_t* row_to_sorted, const float* topk_weights,
                      int64_t T, int32_t k, int64_t N, uint16_t* y, hipStream_t stream) {
  if (T < 0 || k < 1 || N < 0) return W4_ERR_ARG;
  if (o_dtype != W4_OUT_BF16 && o_dtype != W4_OUT_F32) return W4_ERR_ARG;
  if (N % 8 != 0) return W4_ERR_SHAPE;
  if (T == 0 || N == 0) return W4_OK;
  if (!o || !row_to_sorted || !topk_weights || !y) return W4_ERR_ARG;
  if (!aligned16(o) || !aligned16(y)) return W4_ERR_ARG;
  w4::launch_combine(o, o_dtype, row_to_sorted, topk_weights, T, k, N, y, stream);
  return launch_status();
}

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int w4a16_moe_layer_plan(int64_t T, int32_t E, int32_t k, int64_t d, int64_t I, size_t out[9]) {
  if (!out || T < 0 || E < 1 || E > 256 || k < 1 || k > E || k > 16 || d < 0 || I < 0) return W4_ERR_ARG;
  const size_t R = (size_t)T * (size_t)k;
  size_t off = 0;
  const size_t sizes[9] = {R * 4, R * 4, (size_t)(E + 1) * 4, R * 4, R * 4, R * 4,
                           w4::route_workspace_bytes(T, E, k), R * (size_t)I * 2, R * (size_t)d * 4};
  for (int i = 0; i < 9; ++i) {
    out[i] = off;
    off = align256(off + sizes[i]);
  }
  return W4_OK;
}

// The GEMM workspace (fp16 activations) follows the plan region; the two GEMMs
// run one after the other and share it.
static size_t layer_gemm_ws_offset(const size_t p[9], int64_t T, int32_t k, int64_t d) {
  const size_t R = (size_t)T * (size_t)k;
  return align256(p[8] + R * (size_t)d * 4);
}

static size_t layer_gemm_ws_bytes(int64_t T, int32_t E, int32_t k, int64_t d, int64_t I) {
  const size_t a = w4::gemm_tiled_workspace(T, T * (int64_t)k, E, d, 2 * I);
  const size_t b = w4::gemm_tiled_workspace(T * (int64_t)k, T * (int64_t)k, E, I, d);
  return a > b ? a : b;
}

size_t w4a16_moe_layer_workspace(int64_t T, int32_t E, int32_t k, int64_t d, int64_t I) {
  size_t p[9];
  if (w4a16_moe_layer_plan(T, E, k, d, I, p) != W4_OK) return 0;
  return layer_gemm_ws_offset(p, T, k, d) + layer_gemm_ws_bytes(T, E, k, d, I);
}

// Which path a layer takes: the streaming kernels with rows found from the
// top-k ids (few rows per expert, at most kIdsMaxExpertRows tokens), else the
// sorted plan.
static bool layer_sorted(const w4::GemmArgs& a1, const w4::GemmArgs& a2, int64_t T) {
  const int policy = g_gemm_kernel.load(std::memory_order_relaxed);
  const bool streaming = policy == W4_KERNEL_STREAM ||
                         (policy == W4_KERNEL_AUTO && a1.R <= (int64_t)W4_TILED_MIN_ROWS * a1.E) ||
                         !w4::gemm_tiled_supported(a1) || !w4::gemm_tiled_supported(a2);
  return !(streaming && T <= w4::kIdsMaxExpertRows && a1.R <= w4::kIdsMaxRows);
}

int w4a16_moe_layer_sorted(int64_t T, int32_t E, int32_t k, int64_t d, int64_t I) {
  if (T < 0 || E < 1 || k < 1 || d < 0 || I < 0) return W4_ERR_ARG;
  w4::GemmArgs a1{}, a2{};
  a1.x_rows = T;
  a1.E = a2.E = E;
  a1.R = a2.R = T * k;
  a2.x_rows = T * k;
  a1.K = d;
  a1.N = 2 * I;
  a1.epilogue = W4_EPI_GEGLU_TANH;
  a2.K = I;
  a2.N = d;
  a2.epilogue = W4_EPI_NONE;
  return layer_sorted(a1, a2, T) ? 1 : 0;
}

// Host checks of a layer call, everything but the workspace: W4_OK to run,
// kLayerEmpty when there is nothing to enqueue, else the error.
static constexpr int kLayerEmpty = 1;
static int check_layer(const uint16_t* x, const float* logits, int64_t T, int32_t E, int32_t k, int64_t d, int64_t I,
                       const uint8_t* w1_q, const uint16_t* w1_s, const uint8_t* w2_q, const uint16_t* w2_s,
                       int32_t activation, const uint16_t* y) {
  if (activation != W4_EPI_GEGLU_TANH && activation != W4_EPI_SWIGLU) return W4_ERR_ARG;
  size_t p[9];
  const int st = w4a16_moe_layer_plan(T, E, k, d, I, p);
  if (st != W4_OK) return st;
  if (d % 32 != 0 || I % 32 != 0) return W4_ERR_SHAPE;
  if (T * (int64_t)k >= ((int64_t)1 << 31)) return W4_ERR_SHAPE;
  if (T == 0 || d == 0) return kLayerEmpty;
  if (I == 0) return W4_ERR_SHAPE;
  if (!x || !logits || !w1_q || !w1_s || !w2_q || !w2_s || !y) return W4_ERR_ARG;
  // everything the later calls check, checked before the first launch so that
  // an error enqueues nothing
  if (!aligned16(x) || !aligned16(w1_q) || !aligned16(w1_s) || !aligned16(w2_q) || !aligned16(w2_s) || !aligned16(y))
    return W4_ERR_ARG;
  if (2 * I * d / 2 >= ((int64_t)1 << 31) || d * I / 2 >= ((int64_t)1 << 31)) return W4_ERR_SHAPE;
  return W4_OK;
}

int w4a16_moe_layer(const uint16_t* x, const float* logits, int64_t T, int32_t E, int32_t k, int64_t d, int64_t I,
                    const uint8_t* w1_q, const uint16_t* w1_s, const uint8_t* w2_q, const uint16_t* w2_s,
                    int32_t activation, uint16_t* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_layer(x, logits, T, E, k, d, I, w1_q, w1_s, w2_q, w2_s, activation, y);
  if (st == kLayerEmpty) return W4_OK;
  if (st != W4_OK) return st;
  if (!ws || !aligned16(ws) || ws_bytes < w4a16_moe_layer_workspace(T, E, k, d, I)) return W4_ERR_WORKSPACE;
  size_t p[9];
  w4a16_moe_layer_plan(T, E, k, d, I, p);
  char* base = static_cast<char*>(ws);
  int32_t* ids = reinterpret_cast<int32_t*>(base + p[0]);
  float* wts = reinterpret_cast<float*>(base + p[1]);
  int32_t* offs = reinterpret_cast<int32_t*>(base + p[2]);
  int32_t* srows = reinterpret_cast<int32_t*>(base + p[3]);
  int32_t* stoks = reinterpret_cast<int32_t*>(base + p[4]);
  int32_t* r2s = reinterpret_cast<int32_t*>(base + p[5]);
  void* rws = base + p[6];
  uint16_t* act = reinterpret_cast<uint16_t*>(base + p[7]);
  float* o = reinterpret_cast<float*>(base + p[8]);
  void* gws = base + layer_gemm_ws_offset(p, T, k, d);
  const size_t gws_bytes = layer_gemm_ws_bytes(T, E, k, d, I);
  const int64_t R = T * k;

  // gate/up: h = x . W1^T with the gated activation -> a (routed-row order)
  w4::GemmArgs a1{};
  a1.x = x;
  a1.x_rows = T;
  a1.E = E;
  a1.R = R;
  a1.K = d;
  a1.N = 2 * I;
  a1.qweight = w1_q;
  a1.scales = w1_s;
  a1.epilogue = activation;
  a1.out = act;
  a1.out_dtype = W4_OUT_BF16;
  // down: o = a . W2^T (fp32, routed-row order), then the weighted combine
  w4::GemmArgs a2{};
  a2.x = act;
  a2.x_rows = R;
  a2.E = E;
  a2.R = R;
  a2.K = I;
  a2.N = d;
  a2.qweight = w2_q;
  a2.scales = w2_s;
  a2.epilogue = W4_EPI_NONE;
  a2.out = o;
  a2.out_dtype = W4_OUT_F32;

  if (!layer_sorted(a1, a2, T)) {
    // Few rows per expert: no sort (w4a16_moe_gmm_logits, w4a16_moe_gmm_ids,
    // w4a16_moe_combine).  Each matmul workgroup finds its expert's rows in
    // the top-k ids, or (gate/up, up to 64 tokens) from the logits, writing
    // the ids and weights for the down matmul and the combine.
    enqueue_gateup_from_logits(a1, logits, T, E, k, ids, wts, stream);
    a2.ids = ids;
    a2.kslots = 1;
    w4::launch_gemm_skinny(a2, stream);
    w4::launch_combine(o, W4_OUT_F32, nullptr, wts, T, k, d, y, stream);
    return launch_status();
  }
  // Many rows per expert: the routing plan sorts the rows by expert.  The
  // gate/up matmul gathers its x rows through it and stores a in sorted
  // order, so the down matmul reads each expert's rows contiguously (its
  // first activation loads wait for no index load) and stores o at the rows'
  // own (routed) positions, where the combine reads them.
  st = w4a16_moe_route(logits, T, E, k, ids, wts, offs, srows, stoks, r2s, rws, p[7] - p[6], stream);
  if (st != W4_OK) return st;
  a1.row_index = stoks;
  a1.offsets = offs;
  a1.out_index = nullptr;
  st = run_gemm(a1, gws, gws_bytes, stream);
  if (st != W4_OK) return st;
  a2.row_index = nullptr;
  a2.offsets = offs;
  a2.out_index = srows;
  st = run_gemm(a2, gws, gws_bytes, stream);
  if (st != W4_OK) return st;
  w4::launch_combine(o, W4_OUT_F32, nullptr, wts, T, k, d, y, stream);
  return launch_status();
}

// ---------------------------------------------------------------------------
// w4a16_moe_layer_noalloc: the layer with its workspace in a static device
// array instead of a caller buffer.  `scratch` below is a host-side stand-in
// for that array: its device address on each GPU comes from
// hipGetSymbolAddress (taken once per device, with that device current) and
// only that address is ever passed to kernels.
static __device__ __align__(256) uint8_t scratch[W4_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up on first use.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return W4_ERR_HIP;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return W4_ERR_HIP;
      }
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return W4_OK;
}
}  // namespace

int w4a16_moe_layer_noalloc(const uint16_t* x, const float* logits, int64_t T, int32_t E, int32_t k, int64_t d,
                            int64_t I, const uint8_t* w1_q, const uint16_t* w1_s, const uint8_t* w2_q,
                            const uint16_t* w2_s, int32_t activation, uint16_t* y, hipStream_t stream) {
  const int st = check_layer(x, logits, T, E, k, d, I, w1_q, w1_s, w2_q, w2_s, activation, y);
  if (st == kLayerEmpty) return W4_OK;
  if (st != W4_OK) return st;
  // nothing in the layer's workspace has to start at zero: every kernel writes
  // what a later one reads, so the array's previous contents never matter
  if (w4a16_moe_layer_workspace(T, E, k, d, I) > (size_t)W4_NOALLOC_SCRATCH_BYTES) return W4_ERR_WORKSPACE;
  void* ws = nullptr;
  const int sa = scratch_address(&ws);
  if (sa != W4_OK) return sa;
  return w4a16_moe_layer(x, logits, T, E, k, d, I, w1_q, w1_s, w2_q, w2_s, activation, y, ws,
                         (size_t)W4_NOALLOC_SCRATCH_BYTES, stream);
}

// ------------------------------------------------------------ FP8 (W8A8)

int w8a8_quantize_rows(const uint16_t* x, int64_t rows, int64_t K, uint8_t* q, float* scale, hipStream_t stream) {
  if (rows < 0 || K < 0) return W4_ERR_ARG;
  if (K % 32 != 0) return W4_ERR_SHAPE;
  if (rows == 0 || K == 0) return W4_OK;
  if (rows * K >= ((int64_t)1 << 40)) return W4_ERR_SHAPE;
  if (!x || !q || !scale) return W4_ERR_ARG;
  if (!aligned16(x) || !aligned16(q) || (reinterpret_cast<uintptr_t>(scale) & 3u)) return W4_ERR_ARG;
  w4::launch_fp8_quant_rows(x, rows, K, q, scale, stream);
  return launch_status();
}

static int check_fp8_gmm(const w4::Fp8Args& a) {
  if (a.x_rows < 0 || a.E < 1 || a.E > 256 || a.R < 0 || a.K < 0 || a.N < 0) return W4_ERR_ARG;
  if (a.epilogue != W4_EPI_NONE && a.epilogue != W4_EPI_GEGLU_TANH && a.epilogue != W4_EPI_SWIGLU) return W4_ERR_ARG;
  if (a.out_dtype != W4_OUT_BF16 && a.out_dtype != W4_OUT_F32) return W4_ERR_ARG;
  if (a.epilogue != W4_EPI_NONE && a.out_dtype != W4_OUT_BF16) return W4_ERR_ARG;
  if (a.K % 32 != 0 || a.N % 16 != 0) return W4_ERR_SHAPE;
  if (a.R == 0 || a.N == 0) return W4_OK;
  if (a.K == 0) return W4_ERR_SHAPE;
  if (!w4::fp8_gemm_supported(a)) return W4_ERR_SHAPE;
  if (!a.xq || !a.xs || !a.wq || !a.ws || !a.out) return W4_ERR_ARG;
  if (!a.offsets && a.E != 1) return W4_ERR_ARG;
  if (!a.row_index && a.x_rows < a.R) return W4_ERR_SHAPE;
  if (!aligned16(a.xq) || !aligned16(a.wq) || !aligned16(a.out)) return W4_ERR_ARG;
  return W4_OK;
}

int w8a8_moe_gmm(const uint8_t* xq, const float* x_scale, int64_t x_rows, const int32_t* row_index,
                 const int32_t* expert_offsets, int32_t E, int64_t R, int64_t K, int64_t N, const uint8_t* wq,
                 const float* w_scale, int32_t epilogue, void* out, int32_t out_dtype, hipStream_t stream) {
  w4::Fp8Args a{};
  a.xq = xq;
  a.xs = x_scale;
  a.x_rows = x_rows;
  a.row_index = row_index;
  a.offsets = expert_offsets;
  a.E = E;
  a.R = R;
  a.K = K;
  a.N = N;
  a.wq = wq;
  a.ws = w_scale;
  a.epilogue = epilogue;
  a.out = out;
  a.out_dtype = out_dtype;
  const int st = check_fp8_gmm(a);
  if (st != W4_OK || R == 0 || N == 0) return st;
  w4::launch_fp8_gemm(a, stream);
  return launch_status();
}

int w8a8_moe_layer_plan(int64_t T, int32_t E, int32_t k, int64_t d, int64_t I, size_t out[13]) {
  if (!out || T < 0 || E < 1 || E > 256 || k < 1 || k > E || k > 16 || d < 0 || I < 0) return W4_ERR_ARG;
  const size_t R = (size_t)T * (size_t)k;
  const size_t sizes[13] = {R * 4, R * 4, (size_t)(E + 1) * 4, R * 4, R * 4, R * 4,
                            w4::route_workspace_bytes(T, E, k),
                            (size_t)T * (size_t)d, (size_t)T * 4,
                            R * (size_t)I * 2, R * (size_t)I, R * 4,
                            R * (size_t)d * 4};
  size_t off = 0;
  for (int i = 0; i < 13; ++i) {
    out[i] = off;
    off = align256(off + sizes[i]);
  }
  return W4_OK;
}

size_t w8a8_moe_layer_workspace(int64_t T, int32_t E, int32_t k, int64_t d, int64_t I) {
  size_t p[13];
  if (w8a8_moe_layer_plan(T, E, k, d, I, p) != W4_OK) return 0;
  const size_t R = (size_t)T * (size_t)k;
  return align256(p[12] + R * (size_t)d * 4);
}

int w8a8_moe_layer(const uint16_t* x, const float* logits, int64_t T, int32_t E, int32_t k, int64_t d, int64_t I,
                   const uint8_t* w1q, const float* w1_scale, const uint8_t* w2q, const float* w2_scale,
                   int32_t activation, uint16_t* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (T < 0 || E < 1 || E > 256 || k < 1 || k > E || k > 16 || d < 0 || I < 0) return W4_ERR_ARG;
  if (activation != W4_EPI_GEGLU_TANH && activation != W4_EPI_SWIGLU) return W4_ERR_ARG;
  if (d % 32 != 0 || I % 32 != 0) return W4_ERR_SHAPE;
  if (T * (int64_t)k >= ((int64_t)1 << 31)) return W4_ERR_SHAPE;
  if (T == 0 || d == 0) return W4_OK;
  if (I == 0) return W4_ERR_SHAPE;
  if (!x || !logits || !w1q || !w1_scale || !w2q || !w2_scale || !y) return W4_ERR_ARG;
  if (!aligned16(x) || !aligned16(y) || !aligned16(w1q) || !aligned16(w2q)) return W4_ERR_ARG;
  const size_t need = w8a8_moe_layer_workspace(T, E, k, d, I);
  if (!ws || !aligned16(ws) || ws_bytes < need) return W4_ERR_WORKSPACE;
  size_t p[13];
  w8a8_moe_layer_plan(T, E, k, d, I, p);
  uint8_t* b = static_cast<uint8_t*>(ws);
  const int64_t R = T * (int64_t)k;
  int32_t* ids = reinterpret_cast<int32_t*>(b + p[0]);
  float* wts = reinterpret_cast<float*>(b + p[1]);
  int32_t* offs = reinterpret_cast<int32_t*>(b + p[2]);
  int32_t* srows = reinterpret_cast<int32_t*>(b + p[3]);
  int32_t* stoks = reinterpret_cast<int32_t*>(b + p[4]);
  int32_t* r2s = reinterpret_cast<int32_t*>(b + p[5]);
  uint8_t* xq = b + p[7];
  float* xs = reinterpret_cast<float*>(b + p[8]);
  uint16_t* act = reinterpret_cast<uint16_t*>(b + p[9]);
  uint8_t* aq = b + p[10];
  float* as = reinterpret_cast<float*>(b + p[11]);
  float* o = reinterpret_cast<float*>(b + p[12]);
  w4::Fp8Args a1{}, a2{};
  a1.xq = xq;
  a1.xs = xs;
  a1.x_rows = T;
  a1.row_index = stoks;
  a1.offsets = offs;
  a1.E = a2.E = E;
  a1.R = a2.R = R;
  a1.K = d;
  a1.N = 2 * I;
  a1.wq = w1q;
  a1.ws = w1_scale;
  a1.epilogue = activation;
  a1.out = act;
  a1.out_dtype = W4_OUT_BF16;
  a2.xq = aq;
  a2.xs = as;
  a2.x_rows = R;
  a2.row_index = nullptr;
  a2.offsets = offs;
  a2.K = I;
  a2.N = d;
  a2.wq = w2q;
  a2.ws = w2_scale;
  a2.epilogue = W4_EPI_NONE;
  a2.out = o;
  a2.out_dtype = W4_OUT_F32;
  if (!w4::fp8_gemm_supported(a1) || !w4::fp8_gemm_supported(a2)) return W4_ERR_SHAPE;
  w4::launch_route(logits, T, E, k, ids, wts, offs, srows, stoks, r2s, b + p[6], stream);
  w4::launch_fp8_quant_rows(x, T, d, xq, xs, stream);
  w4::launch_fp8_gemm(a1, stream);
  w4::launch_fp8_quant_rows(act, R, I, aq, as, stream);
  w4::launch_fp8_gemm(a2, stream);
  w4::launch_combine(o, W4_OUT_F32, r2s, wts, T, k, d, y, stream);
  return launch_status();
}

}  // extern "C"
