/*
 * w4a16.h -- C ABI of libw4a16.so: W4A16 matmuls over Q4_0 group-32 weights on
 * AMD Instinct MI355X (gfx950).
 *
 * Pages cited (key -> page title; the section is named at each use):
 *   [RQ] "Repacked QAT Gemma 4 26B-A4B serves on one TPU v6e at 1.9x FP8 throughput"
 *   [QP] "The Quantization Problem I Didn't Know I Had Until I Tried Running LLMs Locally"
 *   [WQ] "What quantization really is"
 *
 * Number format ([RQ] "A repack, not a re-quantization"): weights are cut into
 * groups of 32 consecutive values along the input dimension K; each group has
 * one bf16 scale s and 32 integer levels q in -8..7; the weight is s*q.
 * Activations stay bf16 and the product accumulates in fp32 ([RQ] "What
 * changed in vLLM's TPU backend").
 *
 * ------------------------------------------------------------------------
 * Conventions shared by every entry point
 * ------------------------------------------------------------------------
 *  - Every tensor pointer is a DEVICE pointer into caller-owned memory on the
 *    current HIP device.  The library never allocates, frees or synchronises;
 *    each call only enqueues kernels on `stream` (0 = the null stream) and
 *    returns.  Calls are stateless and may be made from several host threads.
 *  - bf16 values travel as uint16_t bit patterns.
 *  - Row-major, densely packed unless stated otherwise.
 *  - The return value is a status code (W4_OK or a negative W4_ERR_*).  Shape
 *    and pointer checks happen on the host before anything is enqueued; on an
 *    error nothing is enqueued.  Conditions that depend on the data (non-finite
 *    inputs, groups off the grid) are reported through device-side outputs,
 *    because the call returns before the kernels run.
 *  - Pointers must be 16-byte aligned unless stated otherwise (W4_ERR_ARG).
 *
 * ------------------------------------------------------------------------
 * Packed code layout "tile16" (this library's own layout for gfx950)
 * ------------------------------------------------------------------------
 * A logical code matrix q[rows][K] (rows % 16 == 0, K % 32 == 0) is stored in
 * rows*K/2 bytes.  Each code is stored offset-binary, u = q + 8 in 0..15.
 *   G  = K/32 groups per row; row tile t = row/16, r = row%16.
 *   Tile t occupies bytes [t*8*K, (t+1)*8*K).
 *   Inside a tile, block b holds groups 4b .. 4b+gb-1 with gb = min(4, G-4b);
 *   it starts at byte 1024*b and is 256*gb bytes long.
 *   The code at column k of group g = 4b+j (chunk c = (k%32)/8, i = k%8) sits
 *   in the 32-bit little-endian word at byte
 *       t*8*K + 1024*b + 4*gb*(16*c + r) + 4*j
 *   at bit 4*(i/2) + 16*(i%2): the even codes of the chunk fill the low
 *   half-word, the odd codes the high half-word.
 * So "lane" 16*c+r of a block owns 4*gb contiguous bytes: the 8 codes of chunk
 * c of row r for each of the block's groups, which is exactly the operand one
 * lane feeds to a 16x16x32 bf16 MFMA; a 64-lane wave reads a whole block
 * (1 KiB for gb = 4) with one 128-bit load per lane.  ((word >> 4d) &
 * 0x000F000F) | 0x43004300 is the bf16 pair (128+u of code 2d, 128+u of code
 * 2d+1), exact, in one shift and one and-or.
 * Scales ("tile16" too): the bf16 scale of row n = 16t+r, group g = 4b+j is
 * element  t*16*G + 64*b + r*gb + j  (gb as above) of a rows*G array, i.e.
 * for each tile and block the 16 x gb scales sit together, row by row (128
 * bytes for a full block), so a wave reads one block's scales from one cache
 * line.  q4_pack_scales converts a plain row-major [rows][G] array.
 * MoE weights stack E such matrices: codes [E][rows*K/2] bytes, scales
 * [E][rows*G].
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  W4_OK = 0,
  W4_ERR_ARG = -1,       /* null pointer, negative size, misaligned pointer, bad enum */
  W4_ERR_SHAPE = -2,     /* rows % 16 != 0, K % 32 != 0, or a size out of range */
  W4_ERR_WORKSPACE = -3, /* workspace pointer null or smaller than required */
  W4_ERR_HIP = -4        /* a kernel launch failed (hipGetLastError) */
};

/* Epilogues of w4a16_moe_gmm. */
enum {
  W4_EPI_NONE = 0,       /* out[r][n] = acc[r][n]                              */
  W4_EPI_GEGLU_TANH = 1, /* out[r][n] = bf16(gelu_tanh(bf16(acc[r][n])) * bf16(acc[r][n+N/2])) */
  W4_EPI_SWIGLU = 2      /* out[r][n] = bf16(silu(bf16(acc[r][n])) * bf16(acc[r][n+N/2]))      */
};

/* Output element types. */
enum { W4_OUT_BF16 = 0, W4_OUT_F32 = 1 };

/* Status-code text (static storage). */
const char* w4a16_status_string(int status);

/* Library ABI version (increments when a signature changes). */
int w4a16_abi_version(void);

/*
 * GEMM kernel choice of w4a16_linear, w4a16_moe_gmm and w4a16_moe_layer.
 *   W4_KERNEL_AUTO    (default) by the average rows per expert R/E: up to
 *                     W4_TILED_MIN_ROWS the weight-streaming kernel (every
 *                     weight byte read once per pass of 16 or 32 rows),
 *                     above it the LDS-tiled MFMA kernel; a dense call of at
 *                     most 16 rows splits K over more waves (one kernel for
 *                     K <= 4096, else two and the workspace);
 *   W4_KERNEL_STREAM  always the weight-streaming kernel;
 *   W4_KERNEL_TILED   the tiled kernel wherever its shape conditions hold
 *                     (gated: N/32 even; otherwise N % 64 == 0; E <= 256),
 *                     else the streaming one.
 * Both kernels compute the same exact products; their fp32 sums differ only
 * in order (see below).  Process-wide, not synchronised with launches in flight on other
 * threads.  Returns the previous setting, or W4_ERR_ARG for an unknown value.
 */
enum { W4_KERNEL_AUTO = 0, W4_KERNEL_STREAM = 1, W4_KERNEL_TILED = 2 };
#define W4_TILED_MIN_ROWS 64
int w4a16_set_gemm_kernel(int kernel);

/* Device-side group status values written by q4_group_repack. */
#define W4_GROUP_OFF_GRID 0u    /* no m in 1..8 reproduced the group */
#define W4_GROUP_NONFINITE 255u /* the group holds a NaN or an infinity */

/*
 * q4_group_repack -- recover the Q4_0 grid of bf16 weights and pack them.
 *
 * [RQ] "A repack, not a re-quantization"; [QP] "Building the Missing Piece".
 * For each group of 32 bf16 values w (a = max|w|):
 *   for m = 1..8: s_m = a/m (fp32, correctly rounded), r_i = w_i/s_m (fp32,
 *   correctly rounded), q_i = clamp(round-half-even(r_i), -8, 7); accept the
 *   first m with |r_i - q_i| <= 3/32 for all i.  If none is accepted the codes
 *   of m = 8 are kept and the group counts as off the grid.  The scale is then
 *   refined by least squares with the codes fixed, s = sum(w q)/sum(q^2) in
 *   fp64 (pairwise order: first half plus second half, repeatedly) and rounded
 *   once to bf16 (nearest, ties to even).
 *   All-zero group: codes 0, scale +0, status 1.  Any NaN/Inf: codes 0, scale
 *   0x7FC0 (quiet NaN), status W4_GROUP_NONFINITE.
 *
 *   w_bf16    in   [rows][K] bf16
 *   qweight   out  rows*K/2 bytes, tile16 layout
 *   scales    out  rows*K/32 bf16, tile16 scale layout
 *   group_status  out, nullable  [rows][K/32] uint8 (plain row-major): accepted m (1..8),
 *                 W4_GROUP_OFF_GRID or W4_GROUP_NONFINITE
 *   counters  in/out, nullable, 8-byte aligned: counters[0] += groups off the
 *             grid, counters[1] += non-finite groups (the caller zeroes them)
 * Requires rows % 16 == 0, K % 32 == 0, rows*K < 2^40.
 */
int q4_group_repack(const uint16_t* w_bf16, int64_t rows, int64_t K,
                    uint8_t* qweight, uint16_t* scales, uint8_t* group_status,
                    unsigned long long* counters, hipStream_t stream);

/*
 * q4_group_dequant_f32 -- out[n][k] = fp32(scale[n][k/32]) * q[n][k].
 *
 * [WQ] "How you actually do it" (dequantize = code times scale).  The codes
 * are unpacked by the routine the weight-streaming matmul kernels (decode,
 * short-K, split-K) feed to the matrix cores: bf16 136 + q, two codes per
 * register.  The prefill kernel's fp16 unpack is a different routine, which
 * this call does not run.  The product of an 8-bit and a 4-bit significand is
 * exact in fp32.
 *   qweight in rows*K/2 bytes tile16; scales in rows*K/32 tile16; out [rows][K] f32.
 */
int q4_group_dequant_f32(const uint8_t* qweight, const uint16_t* scales,
                         int64_t rows, int64_t K, float* out, hipStream_t stream);

/*
 * q4_pack_codes -- store logical int8 codes (each in -8..7; other values are
 * masked to their low 4 bits) in the tile16 layout.  For weights that already
 * come as codes plus group scales ([RQ] "A repack, not a re-quantization":
 * the 4-bit container is only a change of storage).
 *   codes in [rows][K] int8; qweight out rows*K/2 bytes.
 */
int q4_pack_codes(const int8_t* codes, int64_t rows, int64_t K, uint8_t* qweight,
                  hipStream_t stream);

/*
 * q4_pack_scales -- reorder plain row-major bf16 group scales [rows][K/32]
 * into the tile16 scale layout (rows*K/32 elements).  Same conditions as
 * q4_pack_codes.
 */
int q4_pack_scales(const uint16_t* scales, int64_t rows, int64_t K, uint16_t* scales_tiled,
                   hipStream_t stream);

/*
 * Products and accumulation of w4a16_linear and w4a16_moe_gmm.  Every product
 * of an activation and a code is formed exactly and accumulated in fp32; the
 * kernels differ in the order of the fp32 additions and in how the scale and
 * the code offset enter:
 *   streaming kernels (decode shapes, including the short-K and split-K ones)
 *                     bf16 MFMA on the codes as 136 + q (exact in bf16), the
 *                     offset removed through the MFMA's accumulator input
 *                     (-136 times the activations' fp32 group sum), each
 *                     32-group's fp32 partial sum times its scale;
 *   tiled kernel      fp16 MFMA on s*q, exact in fp16 for |s| in [2^-14, 2^13),
 *                     with the activation rows converted to fp16 under a
 *                     per-row power of two (exact for every value within 2^32
 *                     of the row's largest magnitude; smaller ones round to
 *                     fp16's finest step).  A block meeting a scale outside that
 *                     range recomputes its tile, in the same launch, with
 *                     per-group fp32 scaling.
 * One (expert's) weight matrix must stay below 2 GiB of codes (N*K/2 < 2^31),
 * else W4_ERR_SHAPE.
 *   split-K kernel    (w4a16_linear with M <= 16 and fewer than 4096 16-row
 *                     tiles) the streaming kernel's products, per slice of K
 *                     (1024 columns; 512 at K <= 4096 with M = 1); the
 *                     slices' fp32 partial sums are added in slice order, in
 *                     LDS at K <= 4096, else through the workspace.
 * The tiled kernel needs a workspace for the fp16 activation rows, the split-K
 * kernel one for its partial sums: w4a16_linear_workspace /
 * w4a16_moe_gmm_workspace bytes, 16-byte aligned.  A call that selects the
 * tiled kernel (w4a16_set_gemm_kernel) without enough workspace returns
 * W4_ERR_WORKSPACE; without enough workspace for the split-K kernel the
 * streaming kernel runs instead (which ignores ws).
 */

/*
 * w4a16_linear -- y = bf16(x . W^T), W[n][k] = s[n][k/32] * q[n][k].
 *
 * The W4A16 linear layer ([RQ] "What changed in vLLM's TPU backend"): int4
 * weights are dequantized on chip, products are exact and accumulate in fp32,
 * the output is rounded once to bf16.
 *   x        in  [M][K] bf16
 *   qweight  in  N*K/2 bytes tile16; scales in N*K/32 bf16, tile16 scale layout
 *   y        out [M][N] bf16
 *   ws       nullable workspace of ws_bytes (see above)
 * Requires N % 16 == 0, K % 32 == 0, M >= 0 (M == 0 enqueues nothing).
 */
size_t w4a16_linear_workspace(int64_t M, int64_t K, int64_t N);
int w4a16_linear(const uint16_t* x, int64_t M, int64_t K,
                 const uint8_t* qweight, const uint16_t* scales, int64_t N,
                 uint16_t* y, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * w4a16_moe_route -- top-k routing plan of a mixture-of-experts layer.
 *
 * The model family routes each token to 8 of 128 experts ([RQ] "The gap at
 * 26B") and hands the experts' rows to a grouped matmul ([RQ] "What changed in
 * vLLM's TPU backend").  Softmax over all E logits (fp32); top-k by logit value,
 * ties to the lower expert id; weights are the softmax probabilities at those
 * ids (not renormalised).  The T*k routed rows r = t*k + j are grouped by expert
 * (stable: within an expert they keep increasing r).
 *   logits         in  [T][E] fp32, finite
 *   topk_ids       out [T][k] int32
 *   topk_weights   out [T][k] fp32
 *   expert_offsets out [E+1] int32, exclusive prefix sum of the per-expert counts
 *   sorted_rows    out [T*k] int32, sorted position -> routed row r
 *   sorted_tokens  out [T*k] int32, sorted position -> token r / k
 *   row_to_sorted  out [T*k] int32, routed row r -> sorted position
 *   ws, ws_bytes   workspace of at least w4a16_moe_route_workspace(T, E, k) bytes
 * Requires 1 <= k <= E <= 256, k <= 16, T*k < 2^31.  T == 0 writes only the offsets.
 */
size_t w4a16_moe_route_workspace(int64_t T, int32_t E, int32_t k);
int w4a16_moe_route(const float* logits, int64_t T, int32_t E, int32_t k,
                    int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                    int32_t* sorted_rows, int32_t* sorted_tokens, int32_t* row_to_sorted,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * w4a16_moe_topk -- the top-k part of w4a16_moe_route alone: topk_ids and
 * topk_weights as defined there, with no sort.  Same limits; T == 0 enqueues
 * nothing.
 */
int w4a16_moe_topk(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* topk_ids, float* topk_weights,
                   hipStream_t stream);

/*
 * w4a16_moe_gmm_ids -- grouped W4A16 matmul whose rows come straight from the
 * top-k ids, with no sorted plan ([RQ] "What changed in vLLM's TPU backend":
 * the grouped matmul over the experts' packed int4 weights and 32-wide
 * scales).  For every routed row r = t*k + j (expert e = topk_ids[r]):
 *     acc[r][n] = sum_c x[r / row_div][c] * s_e[n][c/32] * q_e[n][c]     (fp32)
 * and out[r][.] = epilogue(acc[r][.]) as in w4a16_moe_gmm.  Each workgroup
 * finds its expert's rows by scanning the ids; rows are taken in increasing r.
 *   x          in  [T*k / row_div][K] bf16 (row_div = k: one row per token;
 *                  row_div = 1: one row per routed row)
 *   topk_ids   in  [T][k] int32, each in [0, E), distinct within a token
 *   qweight, scales  as in w4a16_moe_gmm
 *   out        out [T*k][N] (W4_EPI_NONE) or [T*k][N/2] of out_dtype
 * Requires T <= 256 (W4_ERR_SHAPE), k <= 16, E <= 256 and the w4a16_moe_gmm
 * shape rules.  Uses the weight-streaming kernels (decode batches).
 */
int w4a16_moe_gmm_ids(const uint16_t* x, const int32_t* topk_ids, int64_t T, int32_t k, int32_t row_div, int32_t E,
                      int64_t K, int64_t N, const uint8_t* qweight, const uint16_t* scales, int32_t epilogue,
                      void* out, int32_t out_dtype, hipStream_t stream);

/*
 * w4a16_moe_gmm_logits -- the gate/up matmul of a decode batch with its rows
 * taken from the router logits: the routed rows of the top-k plan of
 * w4a16_moe_topk (descending logit, ties to the lower id), each with x row
 * t, through a gated epilogue:
 *     out[t*k + j][.] = epilogue(x[t] . W_e^T),  e = the j-th expert of token t
 * and topk_ids / topk_weights written as w4a16_moe_topk writes them.  Up to
 * 64 tokens and 128 experts, when the matmul runs on the one-tile streaming
 * kernel, its workgroups rank the logits themselves (no top-k launch);
 * otherwise this is w4a16_moe_topk followed by w4a16_moe_gmm_ids (row_div k).
 * This is the first half of the streaming path of w4a16_moe_layer.
 *   x          in  [T][K] bf16;  logits in [T][E] fp32 (finite)
 *   qweight, scales  as in w4a16_moe_gmm (N = 2 x the gated width)
 *   epilogue   W4_EPI_GEGLU_TANH or W4_EPI_SWIGLU
 *   out        out [T*k][N/2] bf16
 *   topk_ids   out [T][k] int32;  topk_weights out [T][k] fp32
 * Limits of w4a16_moe_topk and w4a16_moe_gmm_ids.
 */
int w4a16_moe_gmm_logits(const uint16_t* x, const float* logits, int64_t T, int32_t E, int32_t k, int64_t K, int64_t N,
                         const uint8_t* qweight, const uint16_t* scales, int32_t epilogue, uint16_t* out,
                         int32_t* topk_ids, float* topk_weights, hipStream_t stream);

/*
 * w4a16_moe_gmm -- grouped W4A16 matmul over expert row ranges.
 *
 * The grouped matmul with one scale per 32-wide group that dequantizes each
 * weight tile on chip before the multiply ([RQ] "What changed in vLLM's TPU
 * backend").  For every expert e and every sorted row i in
 * [expert_offsets[e], expert_offsets[e+1]):
 *     acc[i][n] = sum_k x[src(i)][k] * s_e[n][k/32] * q_e[n][k]     (fp32)
 * with src(i) = row_index[i] if row_index is not null, else i.  The epilogue
 * (W4_EPI_*) maps acc to out[i][.]; with GEGLU/SWIGLU the first N/2 weight rows
 * are the gate and the last N/2 the up projection and out has N/2 columns.
 *   x              in  [x_rows][K] bf16
 *   row_index      in, nullable  [R] int32, each in [0, x_rows)
 *   expert_offsets in  [E+1] int32, non-decreasing, offsets[0] = 0, offsets[E] = R
 *   qweight        in  E * N*K/2 bytes (tile16 per expert); scales in E * N*K/32 (tile16 per expert)
 *   out            out [R][N] (EPI_NONE) or [R][N/2], of out_dtype
 *   ws             nullable workspace of ws_bytes (see above)
 * Requires N % 16 == 0 (N % 32 == 0 with a gated epilogue), K % 32 == 0;
 * out_dtype must be W4_OUT_BF16 for gated epilogues.  Rows outside every
 * expert range are left untouched.
 */
size_t w4a16_moe_gmm_workspace(int64_t x_rows, int64_t R, int32_t E, int64_t K, int64_t N);
int w4a16_moe_gmm(const uint16_t* x, int64_t x_rows, const int32_t* row_index,
                  const int32_t* expert_offsets, int32_t E, int64_t R, int64_t K, int64_t N,
                  const uint8_t* qweight, const uint16_t* scales,
                  int32_t epilogue, void* out, int32_t out_dtype, void* ws, size_t ws_bytes,
                  hipStream_t stream);

/*
 * w4a16_moe_combine -- y[t][n] = bf16( sum_{j<k} w[t][j] * o[row_to_sorted[t*k+j]][n] ),
 * summed in slot order j = 0..k-1 in fp32.
 *
 * The end of a mixture-of-experts layer: each token's output is its k active
 * experts' outputs weighted by the router ([RQ] "The gap at 26B": 8 of 128
 * experts run per token).  The weights are used as given (w4a16_moe_route
 * passes the softmax probabilities at the chosen ids, not renormalised); the
 * bf16 rounding happens once, on the sum, since the layer's activations are
 * bf16 ([RQ] "What changed in vLLM's TPU backend").
 *   o              in  [T*k][N] of o_dtype (W4_OUT_F32 or W4_OUT_BF16)
 *   row_to_sorted  in  [T*k] int32; topk_weights in [T][k] fp32
 *   y              out [T][N] bf16
 * Requires N % 8 == 0.
 */
int w4a16_moe_combine(const void* o, int32_t o_dtype, const int32_t* row_to_sorted,
                      const float* topk_weights, int64_t T, int32_t k, int64_t N,
                      uint16_t* y, hipStream_t stream);

/*
 * w4a16_moe_layer -- one whole mixture-of-experts layer over W4A16 experts:
 * top-k routing, the fused gate/up matmul with the gated epilogue, the down
 * matmul (fp32 rows), and the weighted combine, all enqueued on `stream`.
 * This is the experts method of [RQ] "What changed in vLLM's TPU backend":
 * the packed int4 experts and their 32-wide group scales go straight to the
 * grouped matmul.  Two paths, by w4a16_moe_layer_sorted():
 *   streaming  (at most 64 rows per expert on average and T <= 256; the
 *              default for decode batches) w4a16_moe_gmm_logits for the
 *              gate/up matmul (top-k and rows from the logits),
 *              w4a16_moe_gmm_ids for the down matmul (row_div = 1), then
 *              w4a16_moe_combine (row r = t*k + j): no sort;
 *   sorted     the full routing plan of w4a16_moe_route, then the gate/up
 *              matmul gathers its x rows through it, the down matmul reads
 *              a's rows in sorted order, then w4a16_moe_combine.
 * Both store o at the routed rows r = t*k + j.  The streaming path stores a
 * at the routed rows too, the sorted path at the sorted positions (a's row i
 * belongs to routed row sorted_rows[i]).
 *   x       in  [T][d] bf16;  logits in [T][E] fp32
 *   w1_q    in  E * (2I)*d/2 bytes tile16 (rows [0, I) gate, [I, 2I) up);
 *   w1_s    in  E * 2I*d/32 bf16, tile16 scale layout
 *   w2_q    in  E * d*I/2 bytes tile16;  w2_s in E * d*I/32 bf16, tile16
 *   activation  W4_EPI_GEGLU_TANH or W4_EPI_SWIGLU
 *   y       out [T][d] bf16
 *   ws      workspace of at least w4a16_moe_layer_workspace(T, E, k, d, I) bytes,
 *           16-byte aligned; it holds the routing plan (see w4a16_moe_layer_plan)
 *           and the intermediate activations.  Its contents on entry do not matter.
 * Requires d % 32 == 0, I % 32 == 0 and the w4a16_moe_route limits.
 */
size_t w4a16_moe_layer_workspace(int64_t T, int32_t E, int32_t k, int64_t d, int64_t I);
int w4a16_moe_layer(const uint16_t* x, const float* logits, int64_t T, int32_t E, int32_t k, int64_t d, int64_t I,
                    const uint8_t* w1_q, const uint16_t* w1_s, const uint8_t* w2_q, const uint16_t* w2_s,
                    int32_t activation, uint16_t* y, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * w4a16_moe_layer_sorted -- 1 when w4a16_moe_layer takes the sorted path for
 * these sizes under the current kernel choice (w4a16_set_gemm_kernel), 0 when
 * it takes the streaming path, W4_ERR_ARG for bad sizes.
 */
int w4a16_moe_layer_sorted(int64_t T, int32_t E, int32_t k, int64_t d, int64_t I);

/*
 * w4a16_moe_layer_plan -- byte offsets, inside a w4a16_moe_layer workspace, of
 * the routing plan and intermediates it leaves behind (for inspection):
 *   out[0] topk_ids [T][k] i32      out[1] topk_weights [T][k] f32
 *   out[2] expert_offsets [E+1] i32 out[3] sorted_rows [T*k] i32
 *   out[4] sorted_tokens [T*k] i32  out[5] row_to_sorted [T*k] i32
 *          (out[2..5]: sorted path only)
 *   out[6] route scratch (sorted path)
 *   out[7] a: gated activations [T*k][I] bf16, row r = t*k + j
 *   out[8] o: down-projection rows [T*k][d] f32, row r = t*k + j
 * Returns W4_ERR_ARG for out == NULL or bad sizes.
 */
int w4a16_moe_layer_plan(int64_t T, int32_t E, int32_t k, int64_t d, int64_t I, size_t out[9]);

/*
 * w4a16_moe_layer_noalloc -- w4a16_moe_layer without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The workspace is a
 * static device array of W4_NOALLOC_SCRATCH_BYTES inside the library, one
 * per GPU, held from the first call on that GPU until the process ends; the
 * call itself allocates and frees nothing.  Arguments, outputs and errors are
 * those of w4a16_moe_layer, plus:
 *   W4_ERR_WORKSPACE  when w4a16_moe_layer_workspace(T, E, k, d, I) exceeds the
 *                     array (at d = 2816, I = 704, E = 128, k = 8: T up to 290);
 *                     nothing is enqueued.
 *   W4_ERR_HIP        when the array's device address cannot be obtained.
 * Every call on one GPU uses that GPU's one array and it keeps the last call's
 * contents (nothing in it needs to start at zero), so calls that overlap on
 * one GPU -- on two streams, or from two host threads -- race and give wrong
 * results: serialise them.
 */
#define W4_NOALLOC_SCRATCH_BYTES (32u << 20)
int w4a16_moe_layer_noalloc(const uint16_t* x, const float* logits, int64_t T, int32_t E, int32_t k, int64_t d,
                            int64_t I, const uint8_t* w1_q, const uint16_t* w1_s, const uint8_t* w2_q,
                            const uint16_t* w2_s, int32_t activation, uint16_t* y, hipStream_t stream);

/* ---------------------------------------------------------------- FP8 (W8A8)
 * The comparison path: the same MoE layer over FP8 experts, run natively on the
 * FP8 matrix cores.  [RQ] "Repacked QAT Gemma 4 26B-A4B serves on one TPU v6e at
 * 1.9x FP8 throughput", section "What happened" (the W4A16 build against an FP8
 * build of the same model); [VG] "Compression Without Regret", sections "2. What
 * you can quantize" and "3. The precision ladder" (FP8 quantizes weights and
 * activations and multiplies natively in low precision).  The pages fix neither
 * the encoding nor the scales; this library takes OCP E4M3 codes (largest finite
 * magnitude 448, no infinities, 0x7F/0xFF NaN), one fp32 scale per weight row
 * (output channel) and activations quantized per row at run time.
 */

/*
 * w8a8_quantize_rows -- per-row dynamic E4M3 quantization.
 *   x      in  [rows][K] bf16 (finite)
 *   q      out [rows][K] E4M3 codes
 *   scale  out [rows] fp32: amax / 448 (one IEEE fp32 division; 1.0 for a row of
 *          zeros); q = E4M3(clamp(x / scale, -448, 448)), x / scale one IEEE fp32
 *          division, rounded to nearest even.
 * K % 32 == 0.  x and q 16-byte aligned, scale 4-byte aligned.
 */
int w8a8_quantize_rows(const uint16_t* x, int64_t rows, int64_t K, uint8_t* q, float* scale, hipStream_t stream);

/*
 * w8a8_moe_gmm -- grouped FP8 matmul over expert row ranges (the layout of
 * w4a16_moe_gmm with byte codes and fp32 row scales):
 *   out[i][n] = epilogue(x_scale[src(i)] * w_scale[e][n] *
 *                        sum_k E4M3(xq[src(i)][k]) * E4M3(wq[e][n][k]))
 * for sorted row i of expert e (offsets[e] <= i < offsets[e+1]), src(i) =
 * row_index[i] (or i when row_index is NULL), fp32 accumulation.
 *   xq, x_scale      in  [x_rows][K] E4M3 codes, [x_rows] fp32
 *   row_index        in  [R] or NULL
 *   expert_offsets   in  [E+1], or NULL with E == 1 (rows [0, R) are expert 0's)
 *   wq, w_scale      in  [E][N][K] E4M3 codes (row-major), [E][N] fp32
 *   epilogue         W4_EPI_* (gated: first N/2 rows gate, last N/2 up;
 *                    out is [R][N/2] bf16)
 *   out              out [R][N] (W4_EPI_NONE) of out_dtype, at the sorted rows
 * K % 32 == 0; N % 16 == 0 with N/16 a multiple of 4 (plain) or N/32 even
 * (gated); E <= 256; x_rows*K, N*K < 2^31.  Few rows per expert (at most 32 on
 * average) take the weight-streaming kernel, more the 128-row tiled one.
 */
int w8a8_moe_gmm(const uint8_t* xq, const float* x_scale, int64_t x_rows, const int32_t* row_index,
                 const int32_t* expert_offsets, int32_t E, int64_t R, int64_t K, int64_t N, const uint8_t* wq,
                 const float* w_scale, int32_t epilogue, void* out, int32_t out_dtype, hipStream_t stream);

/*
 * w8a8_moe_layer -- the MoE layer over FP8 experts, one call: route (as
 * w4a16_moe_route), quantize x per token, the gate/up grouped matmul with the
 * gated activation (a, bf16, sorted rows), quantize a per routed row, the down
 * grouped matmul (o, fp32, sorted rows), the weighted combine into y.
 *   w1q [E][2I][d], w1_scale [E][2I]; w2q [E][d][I], w2_scale [E][d]
 * The workspace (w8a8_moe_layer_workspace bytes, 16-byte aligned) holds, at the
 * offsets w8a8_moe_layer_plan writes to out[0..12]: ids, weights, offsets,
 * sorted rows, sorted tokens, row-to-sorted, route scratch, xq, x scales, a,
 * a's codes, a's scales, o.  d % 32 == 0, I % 32 == 0, and the two matmuls'
 * N conditions above hold.
 */
int w8a8_moe_layer_plan(int64_t T, int32_t E, int32_t k, int64_t d, int64_t I, size_t out[13]);
size_t w8a8_moe_layer_workspace(int64_t T, int32_t E, int32_t k, int64_t d, int64_t I);
int w8a8_moe_layer(const uint16_t* x, const float* logits, int64_t T, int32_t E, int32_t k, int64_t d, int64_t I,
                   const uint8_t* w1q, const float* w1_scale, const uint8_t* w2q, const float* w2_scale,
                   int32_t activation, uint16_t* y, void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
