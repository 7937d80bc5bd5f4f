/*
 * moeffn.h - C ABI of the MI355X (gfx950) MoE / gated-MLP FFN hot path.
 *
 * One GPU's share of a Pre-Norm transformer FFN sub-block, FFN(RMSNorm(R)),
 * as pages on LLM inference describe it ("推理计算流梳理", Norm&Residual,
 * 实际 MLP 计算策略, 专家并行; "「赤兔」Chitu 框架深度解读（七）：MoE", token
 * dispatchers and experts):
 *
 *   rmsnorm -> moe_route -> moe_permute -> grouped_swiglu -> moe_combine
 *
 * plus the dense tensor-parallel shard of the same gated MLP, tp_shard_mlp.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every tensor argument is caller-owned DEVICE memory on the current HIP
 *    device, row-major and contiguous, 16-byte aligned. Sizes are in elements.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL is
 *    the null stream). They never synchronise the host, never allocate device
 *    memory and keep no mutable global state, so they are re-entrant. Calls
 *    that share an output or workspace buffer must be ordered by the caller.
 *  - Linear-layer weights are given as [out_features, in_features] (each
 *    output feature's weights contiguous), i.e. the transpose of the pages' W
 *    in Y = X W; the router weight W_r is [E, d], as in the pages' z = x W_r^T.
 *    Every weight argument of the GEMM calls (W_r, the experts' W_gate, W_up,
 *    W_down and the TP shards) is passed PACKED by pack_weights, once, ahead
 *    of use: a layout in which each MFMA weight fragment is one contiguous
 *    1 KB block (see pack_weights).
 *  - Return value: MF_OK (0), MF_EINVAL (-1: null pointer, bad size or value),
 *    MF_EUNSUPPORTED (-2: valid but outside what the kernels implement, such
 *    as a dtype combination, an alignment or a dimension that is not a
 *    multiple of the tile), MF_EHIP (-3: the HIP runtime reported an error at
 *    launch). Arguments are validated before anything is enqueued: on
 *    MF_EINVAL or MF_EUNSUPPORTED nothing was enqueued.
 *  - A call with zero tokens/rows is valid; it enqueues only what is needed
 *    to leave the outputs well defined (moe_permute still writes zero counts
 *    and offsets) and returns MF_OK.
 *  - Data-dependent values (token ids, expert ids, offsets, row indices) are
 *    clamped or skipped by the kernels so that no access leaves its buffer,
 *    whatever the device data holds.
 */
#ifndef MOEFFN_H
#define MOEFFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { MF_OK = 0, MF_EINVAL = -1, MF_EUNSUPPORTED = -2, MF_EHIP = -3 };
enum { MF_F32 = 0, MF_BF16 = 1, MF_FP8_E4M3 = 2 };

/* Human-readable name of a status code (static storage). */
const char* mf_status_string(int status);

/* Library version string (static storage). */
const char* mf_version(void);

/*
 * rmsnorm - y[t, j] = gamma[j] * x[t, j] / sqrt(mean_k x[t, k]^2 + eps).
 *
 * "推理计算流梳理", Norm&Residual: the RMSNorm equation (the mean square over
 * the hidden vector, eps = 1e-5 inside the square root) and V = RMSNorm_ffn(R),
 * the input of the FFN.
 *
 * x, y   [T, d]  dtype (MF_BF16 or MF_F32); y may alias x.
 * gamma  [d]     dtype.
 * Math in fp32; y is rounded to nearest-even into dtype.
 * Requires d % 64 == 0 and d <= 8192; eps >= 0 (MF_EUNSUPPORTED beyond 8192).
 */
int rmsnorm(const void* x, const void* gamma, void* y, int64_t T, int32_t d,
            float eps, int32_t dtype, void* stream);

/*
 * rmsnorm_quantize_fp8 - rmsnorm (bf16) and, in the same pass, the per-token
 * fp8 activations of its output for the block-fp8 prefill variant: y as
 * rmsnorm writes it, and q / scales exactly as quantize_fp8_rows(y) would
 * write them (each row of y cut into groups of 128 channels, group scale
 * s = max(amax, 1e-4) / 448, code = the E4M3FN value nearest to y / s, ties
 * to even, fp32 with IEEE division).
 *
 * "推理计算流梳理", Norm&Residual (V = RMSNorm_ffn(R)); "「赤兔」Chitu 框架深度解读
 * （七）：MoE", 专家计算实现 / 量化支持 (FP8 GEMMs for prefill, block fp8).
 *
 * x, y [T, d] bf16 (y may alias x); gamma [d] bf16; q [T, d] E4M3FN codes
 * (8-byte aligned); scales [T, d/128] f32. Requires d % 128 == 0, d <= 8192
 * (MF_EUNSUPPORTED otherwise); eps >= 0.
 */
int rmsnorm_quantize_fp8(const void* x, const void* gamma, void* y, void* q, float* scales,
                         int64_t T, int32_t d, float eps, void* stream);

/*
 * packed_weights_bytes - bytes of pack_weights' output for `groups` weight
 * matrices of N rows and K columns (dtype MF_BF16 or MF_FP8_E4M3). Returns 0
 * for arguments pack_weights would reject.
 */
size_t packed_weights_bytes(int64_t groups, int32_t N, int32_t K, int32_t dtype);

/*
 * pack_weights - rearranges src [groups, N, K] (row-major, [out, in]) into the
 * order the GEMM calls consume, dst (packed_weights_bytes bytes). A pure
 * permutation plus zero padding of the last row block; the values are
 * unchanged. Weights are packed once, when they are loaded, not per call.
 *
 *   MF_BF16: 32-row x 16-column fragments of 1 KB, row block major:
 *     dst[g][nb][kb][l][v] = W[g][32 nb + l % 32][16 kb + 8 (l / 32) + v]
 *     (l = 0..63, v = 0..7; rows >= N read as 0). Requires K % 16 == 0.
 *   MF_FP8_E4M3 (codes; block scales are not packed): 16-row x 128-column
 *     blocks of 2 KB, each two 1 KB halves, 128-column slab major (a packed
 *     tensor is therefore not sliced by group: pack each group set on its own):
 *     dst[kb][g][nb][h][l][b] = W[g][16 nb + l % 16][128 kb + 32 (l / 16) + 16 h + b]
 *     (h = 0..1, l = 0..63, b = 0..15; rows >= N read as 0). Requires K % 128 == 0.
 */
int pack_weights(const void* src, void* dst, int64_t groups, int32_t N, int32_t K,
                 int32_t dtype, void* stream);

/*
 * pack_weights_kn - pack_weights for weights stored [groups, K, N] ([in, out],
 * row-major: the orientation of a linear layer W in R^{d x f} with Y = X W in
 * "推理计算流梳理", 张量并行和通信, used by the gated MLP of 实际 MLP 计算策略,
 * so W_gate and W_up of an expert are [d, f] and W_down [f, d]). dst
 * receives exactly the bytes pack_weights
 * writes for the transposed [groups, N, K] tensor; N, K, dtype, the size of
 * dst and the requirements are the same. The source is read element by
 * element (bf16: src 2-byte aligned; dst 16-byte aligned). Errors: as
 * pack_weights.
 */
int pack_weights_kn(const void* src, void* dst, int64_t groups, int32_t N, int32_t K,
                    int32_t dtype, void* stream);

/*
 * moe_route_workspace_size - bytes of device workspace moe_route needs for
 * T tokens, hidden size d and E experts (fp32 partial logits). Depends on
 * (T, d, E) only. Returns 0 for arguments moe_route would reject.
 */
size_t moe_route_workspace_size(int64_t T, int32_t d, int32_t E);

/*
 * moe_route - sigmoid-with-bias top-k expert router.
 *
 * "推理计算流梳理", 专家并行 / MoE Router 过程, router equation:
 *   z = x W_r^T,  s = sigmoid(z),  I = Top8(s + b),  w_i = s_i / sum_{j in I} s_j.
 * The bias only selects experts; the weights use the unbiased scores.
 *
 * x        [T, d] bf16      router input (RMSNorm output inside the FFN block)
 * w_r      [E, d] bf16      router weight, packed (pack_weights, MF_BF16)
 * bias     [E]    f32
 * topk_idx [T, k] int32     out: the k selected expert ids of each token, in
 *                           ascending order (I is a set)
 * topk_w   [T, k] f32       out: w_i aligned with topk_idx; each row sums to 1
 * workspace                 moe_route_workspace_size(T, d, E) bytes; its
 *                           content on entry does not matter
 * Logits are bf16 x bf16 products accumulated in fp32 on MFMA (the d-long
 * contraction may be split into ranges whose fp32 partial sums are added in a
 * fixed order); s, s + b and w are fp32. The result is the same run to run.
 * Ties in s + b go to the lower id.
 * Requires k == 8, 8 <= E <= 256, d % 64 == 0.
 */
int moe_route(const void* x, const void* w_r, const float* bias, int64_t T,
              int32_t d, int32_t E, int32_t k, int32_t* topk_idx, float* topk_w,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_permute_workspace_size - bytes of device workspace moe_permute needs.
 * Returns 0 for invalid arguments (then moe_permute would return MF_EINVAL).
 */
size_t moe_permute_workspace_size(int64_t T, int32_t k, int32_t e_count);

/*
 * moe_permute - stable counting sort of the routing slots (t, j) by expert,
 * over the local experts [e_begin, e_begin + e_count), and the gather of the
 * token rows into that expert-contiguous order.
 *
 * "「赤兔」Chitu 框架深度解读（七）：MoE": token_permutation of a dispatcher with
 * no communication, and the expert-contiguous token layout its grouped GEMM
 * consumes; "推理计算流梳理", EP 路径: each rank runs its own experts.
 *
 * topk_idx  [T, k] int32   expert ids; ids in a row must be distinct (the
 *                          router's always are); ids outside the local range
 *                          are dropped
 * x         [T, d] or NULL rows to gather (x_dtype MF_BF16 or MF_F32); NULL
 *                          computes the indices only and leaves x_perm untouched
 * x_perm    [T*k, d]       out: row r = x[src_token[r]] for r < offsets[e_count]
 * counts    [e_count] i32  out: slots per local expert
 * offsets   [e_count+1]    out: exclusive prefix sum of counts, offsets[0] = 0
 * src_token [T*k] i32      out: token of each permuted row (first
 *                          offsets[e_count] entries); tokens ascend within an
 *                          expert (stable)
 * inv_pos   [T, k] i32     out: permuted row of slot (t, j), -1 if non-local
 * workspace                moe_permute_workspace_size(T, k, e_count) bytes
 * Integer results are exact and deterministic (no order-dependent atomics).
 * Requires 1 <= k <= 8, 1 <= e_count <= 256, e_begin >= 0, T*k < 2^31, and
 * (when x != NULL) d * sizeof(x_dtype) % 16 == 0.
 */
int moe_permute(const int32_t* topk_idx, int64_t T, int32_t k, int32_t e_begin,
                int32_t e_count, const void* x, int32_t d, int32_t x_dtype,
                void* x_perm, int32_t* counts, int32_t* offsets,
                int32_t* src_token, int32_t* inv_pos, void* workspace,
                size_t workspace_bytes, void* stream);

/*
 * moe_permute_noalloc - moe_permute without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation). Same arguments, outputs,
 * results and errors as moe_permute, minus workspace / workspace_bytes.
 *
 * Its count tables live in a static device array of the library (about
 * 512 KiB, held on every GPU the library runs on until the process ends),
 * whose address is looked up once per device on the first call there. It
 * allocates nothing. Limit: ceil(T / 256) * e_count <= 65536 (for instance
 * T <= 65536 with 256 local experts); larger calls return MF_EUNSUPPORTED
 * with nothing enqueued. Every call on one GPU shares that GPU's array, so
 * calls that may overlap on one GPU (different streams, different host
 * threads) race: order them. Returns MF_EHIP if the array's address cannot be
 * obtained.
 */
int moe_permute_noalloc(const int32_t* topk_idx, int64_t T, int32_t k, int32_t e_begin,
                        int32_t e_count, const void* x, int32_t d, int32_t x_dtype, void* x_perm,
                        int32_t* counts, int32_t* offsets, int32_t* src_token, int32_t* inv_pos,
                        void* stream);

/*
 * moe_dispatch_masked - the masked (fixed-capacity) layout of the routing
 * slots, the decode variant of the permutation ("「赤兔」Chitu 框架深度解读（七）：MoE":
 * the decode experts run as a masked GEMM (deepgemm_masked), the decode
 * dispatcher is the low-latency one). Local expert e owns rows
 * [e*cap, (e+1)*cap); slot (t, j) routed to a local expert e goes to row
 * e*cap + rank, rank = the number of earlier tokens routed to e (stable, token
 * order). There is no prefix over experts. A slot whose rank reaches cap is
 * dropped (pos = -1, it adds nothing in moe_combine); with cap >= T nothing is
 * dropped (a token picks an expert at most once).
 *
 * topk_idx  [T, k] int32 (moe_route's ids); T >= 0, 1 <= k <= 8
 * e_begin, e_count  local experts [e_begin, e_begin + e_count), e_count <= 256
 * cap       rows per expert block, >= 1 (e_count * cap < 2^31)
 * counts    [e_count] int32 out: rows used in each block, min(routed, cap)
 * row_index [e_count * cap] int32 out: token of each used row (rows past
 *           counts[e] are not written); the masked GEMMs gather V[row_index]
 * pos       [T, k] int32 out: row of each slot, or -1
 * workspace moe_permute_workspace_size(T, k, e_count) bytes (16-byte aligned)
 * Deterministic and bit-exact (no order-dependent atomics).
 */
int moe_dispatch_masked(const int32_t* topk_idx, int64_t T, int32_t k, int32_t e_begin,
                        int32_t e_count, int32_t cap, int32_t* counts, int32_t* row_index,
                        int32_t* pos, void* workspace, size_t workspace_bytes, void* stream);

/*
 * grouped_swiglu - every local expert's gated MLP over its contiguous rows:
 *   H[o_e:o_{e+1}]      = SiLU(X_perm W_gate_e) * (X_perm W_up_e)
 *   Y_perm[o_e:o_{e+1}] = H[o_e:o_{e+1}] W_down_e
 *
 * "推理计算流梳理", 实际 MLP 计算策略 (the gated MLP equation) and EP 路径 (one
 * rank runs many experts as one grouped GEMM); "「赤兔」Chitu ... MoE", experts
 * (BatchedExperts; one kernel for all experts; block-fp8 quantised experts).
 *
 * x        the grouped input, in one of two forms:
 *          row_index == NULL: x is X_perm [max_rows, d] bf16, rows grouped by
 *            expert (moe_permute's gathered output);
 *          row_index != NULL: x is the un-permuted [src_rows, d] bf16 tensor and
 *            row r of X_perm is x[row_index[r]] (row_index = moe_permute's
 *            src_token, [max_rows] int32, entries clamped to [0, src_rows)):
 *            the gather is done inside the GEMM's A load and moe_permute can
 *            run with x == NULL (indices only).
 * src_rows rows of x when row_index != NULL (>= 1), else ignored
 * offsets  [e_count+1] int32     device; expert e owns rows [offsets[e], offsets[e+1])
 * w_gate, w_up [e_count, f, d]   w_dtype (MF_BF16, or MF_FP8_E4M3 codes), packed
 * w_down   [e_count, d, f]       w_dtype, packed (pack_weights with groups = e_count)
 * s_gate, s_up [e_count, f/128, d/128] f32, s_down [e_count, d/128, f/128] f32:
 *                                fp8 only (NULL for bf16): one scale per 128x128
 *                                block; weight value = code value * scale
 * h_work   [max_rows, f] bf16    out: H (the bf16 operand of the down GEMM)
 * y_perm   [max_rows, d] bf16    out: expert outputs (rows < offsets[e_count])
 * max_rows bounds the rows (T*k after moe_permute), so no host sync is needed.
 * GEMMs run on MFMA with bf16 operands and fp32 accumulation; SiLU(g)*u is
 * fused into the gate/up epilogue in fp32. fp8 codes are converted to bf16
 * exactly and each 128-deep partial sum is scaled in fp32; with fp8 weights
 * the work is tiled 128 rows at a time when max_rows >= 32 * e_count (and
 * d, f <= 16384), else 16 rows per pass over each expert's weights (decode
 * shapes, where an expert holds a few rows).
 * Requires 1 <= e_count <= 256; bf16: d % 64 == 0 and f % 64 == 0;
 * fp8: d % 128 == 0 and f % 128 == 0.
 */
int grouped_swiglu(const void* x, const int32_t* row_index, int64_t src_rows,
                   const int32_t* offsets, int32_t e_count, int64_t max_rows, int32_t d,
                   int32_t f, const void* w_gate, const void* w_up, const void* w_down,
                   int32_t w_dtype, const float* s_gate, const float* s_up,
                   const float* s_down, void* h_work, void* y_perm, void* stream);

/*
 * grouped_gate_up - the first half of grouped_swiglu on its own:
 *   H[o_e:o_{e+1}] = SiLU(X_perm W_gate_e) * (X_perm W_up_e)
 * Same passages, arguments (x, row_index, src_rows included), layouts and
 * requirements as grouped_swiglu (h_out is its h_work). The SiLU product is
 * fused into the GEMM epilogue.
 */
int grouped_gate_up(const void* x, const int32_t* row_index, int64_t src_rows,
                    const int32_t* offsets, int32_t e_count, int64_t max_rows, int32_t d,
                    int32_t f, const void* w_gate, const void* w_up, int32_t w_dtype,
                    const float* s_gate, const float* s_up, void* h_out, void* stream);

/*
 * grouped_down - the second half of grouped_swiglu on its own:
 *   Y_perm[o_e:o_{e+1}] = H[o_e:o_{e+1}] W_down_e
 * h [max_rows, f] bf16 (grouped_gate_up's output), w_down [e_count, d, f],
 * s_down as in grouped_swiglu, y_perm [max_rows, d] bf16. Same requirements.
 */
int grouped_down(const void* h, const int32_t* offsets, int32_t e_count,
                 int64_t max_rows, int32_t f, int32_t d, const void* w_down,
                 int32_t w_dtype, const float* s_down, void* y_perm, void* stream);

/*
 * grouped_gate_up_masked / grouped_down_masked - grouped_gate_up /
 * grouped_down over the masked layout (moe_dispatch_masked): expert e's rows
 * are the first counts[e] (clamped to cap) rows of its block [e*cap, (e+1)*cap).
 * The passages, weights, dtypes and requirements are grouped_swiglu's, with
 * max_rows = e_count * cap:
 *   x, row_index, src_rows as grouped_swiglu (row_index = moe_dispatch_masked's)
 *   h_out / h  [e_count*cap, f] bf16, y_perm [e_count*cap, d] bf16; rows past
 *   counts[e] in each block are not written. moe_combine takes pos as inv_pos
 *   with max_rows = e_count * cap.
 */
int grouped_gate_up_masked(const void* x, const int32_t* row_index, int64_t src_rows,
                           const int32_t* counts, int32_t cap, int32_t e_count, int32_t d,
                           int32_t f, const void* w_gate, const void* w_up, int32_t w_dtype,
                           const float* s_gate, const float* s_up, void* h_out, void* stream);
int grouped_down_masked(const void* h, const int32_t* counts, int32_t cap, int32_t e_count,
                        int32_t f, int32_t d, const void* w_down, int32_t w_dtype,
                        const float* s_down, void* y_perm, void* stream);

/*
 * quantize_fp8_rows - per-token fp8 activations for the block-fp8 prefill
 * variant ("「赤兔」Chitu 框架深度解读（七）：MoE", 专家计算实现: prefill experts run as
 * FP8 GEMMs on tokens laid out contiguously by expert; 量化支持: block fp8).
 * Each row of x is cut into groups of 128 consecutive channels; a group's
 * scale is s = max(amax, 1e-4) / 448 and each element's code is the E4M3FN
 * value nearest to x / s (ties to even), both in fp32 with IEEE division.
 *
 * x          [rows, K] bf16 (16-byte aligned)
 * row_count  NULL, or a device int32: only rows [0, min(*row_count, rows)) are
 *            quantised and the rest of q / scales is left untouched (e.g.
 *            offsets + e_count for a grouped H, whose live rows are known only
 *            on the device)
 * q          [rows, K] E4M3FN codes (8-byte aligned)     out
 * scales     [rows, K/128] f32                            out
 * Requires K % 128 == 0. rows == 0 is a no-op.
 */
int quantize_fp8_rows(const void* x, int64_t rows, const int32_t* row_count, int32_t K, void* q,
                      float* scales, void* stream);

/*
 * grouped_gate_up_a8 - grouped_gate_up with fp8 activations on the fp8 MFMA:
 *   H[o_e:o_{e+1}] = SiLU(X_perm W_gate_e) * (X_perm W_up_e)
 * with X_perm[t, k] = xq[t, k] * x_scale[t, k/128] (quantize_fp8_rows) and
 * block-fp8 weights (code * scale per 128x128 block). Same passages as
 * grouped_swiglu plus quantize_fp8_rows' ([P5] FP8 GEMMs for prefill).
 *
 * xq, x_scale  row_index == NULL: [max_rows, d] codes and [max_rows, d/128] f32,
 *              rows grouped by expert; row_index != NULL: [src_rows, d] and
 *              [src_rows, d/128] un-permuted, row r of X_perm is row row_index[r]
 *              (entries clamped to [0, src_rows)): the gather is done in the A load
 * offsets, e_count, max_rows  as grouped_swiglu
 * w_gate, w_up [e_count, f, d] E4M3FN codes packed by pack_weights
 * s_gate, s_up [e_count, f/128, d/128] f32
 * h_out        [max_rows, f] bf16      out (rows < offsets[e_count])
 * Each 128-deep block of the contraction is summed exactly on the fp8 MFMA
 * (fp32 accumulation) and added into the fp32 result scaled by its activation
 * and weight scales; SiLU(g)*u in fp32 in the epilogue.
 * Requires 1 <= e_count <= 256, d % 128 == 0, f % 128 == 0, d <= 16384
 * (MF_EUNSUPPORTED otherwise).
 */
int grouped_gate_up_a8(const void* xq, const float* x_scale, const int32_t* row_index,
                       int64_t src_rows, const int32_t* offsets, int32_t e_count,
                       int64_t max_rows, int32_t d, int32_t f, const void* w_gate,
                       const void* w_up, const float* s_gate, const float* s_up, void* h_out,
                       void* stream);

/*
 * grouped_down_a8 - grouped_down with fp8 activations on the fp8 MFMA:
 *   Y_perm[o_e:o_{e+1}] = H W_down_e, H[t, k] = hq[t, k] * h_scale[t, k/128]
 * hq [max_rows, f] codes and h_scale [max_rows, f/128] f32 (quantize_fp8_rows
 * of grouped_gate_up_a8's bf16 H), w_down [e_count, d, f] packed E4M3FN codes,
 * s_down [e_count, d/128, f/128] f32, y_perm [max_rows, d] bf16 out.
 * Same requirements as grouped_gate_up_a8, with f <= 16384 (the contraction).
 */
int grouped_down_a8(const void* hq, const float* h_scale, const int32_t* offsets,
                    int32_t e_count, int64_t max_rows, int32_t f, int32_t d, const void* w_down,
                    const float* s_down, void* y_perm, void* stream);

/*
 * moe_combine - out[t] = sum_{j : inv_pos[t,j] >= 0} topk_w[t,j] * y_perm[inv_pos[t,j]]
 *                        (+ residual[t]).
 * The optional residual is the Pre-Norm block's skip connection ("推理计算流梳理",
 * Norm&Residual: the layer output is the residual stream plus the FFN of its
 * normalised copy); with expert parallelism it is passed on one rank only.
 *
 * "推理计算流梳理", EP 路径: the expert outputs are summed with the router
 * weights back at the token's source ("「赤兔」Chitu ... MoE":
 * token_unpermutation). The global weights are used as they are (no
 * renormalisation over local experts): a token with no local expert gets 0,
 * and the outputs of disjoint expert ranges add up to the full FFN output.
 *
 * y_perm  [max_rows, d] bf16; inv_pos [T, k] int32 (entries < 0 or >= max_rows
 * are skipped); topk_w [T, k] f32; residual [T, d] out_dtype or NULL; out
 * [T, d] out_dtype (MF_BF16 or MF_F32; may alias residual).
 * fp32 accumulation in slot order j = 0..k-1, then the residual is added.
 * Requires 1 <= k <= 8, d % 64 == 0.
 */
int moe_combine(const void* y_perm, const int32_t* inv_pos, const float* topk_w,
                int64_t T, int32_t k, int32_t d, int64_t max_rows, const void* residual,
                void* out, int32_t out_dtype, void* stream);

/*
 * tp_shard_mlp - one tensor-parallel shard of the dense gated MLP:
 *   H_i = SiLU(X W_gate[:, F_i]) * (X W_up[:, F_i]),   P_i = H_i W_down[F_i, :]
 *
 * "推理计算流梳理", 实际 MLP 计算策略 (W_gate / W_up column-parallel, the pointwise
 * part needs no communication, W_down row-parallel) and 行并行 (each rank's
 * output has the full shape but is only part of the sum); "tensor_parallelism",
 * Outer Dim / Inner Dim; "LLM推理并行优化的必备知识" §1.4.
 *
 * x        [T, d]    dtype
 * w_gate_s, w_up_s [f_s, d] dtype: rows F_i of the [f, d] weight
 * w_down_s [d, f_s]  dtype: columns F_i of the [d, f] weight
 *                    (MF_BF16: packed by pack_weights; MF_F32: row-major as shown)
 * h_work   [T, f_s]  dtype, out: H_i
 * partial  [T, d]    f32, out: P_i, the full-shape partial sum
 * dtype MF_BF16 (MFMA, fp32 accumulation; H_i rounded to bf16; requires
 * d % 64 == 0, f_s % 64 == 0) or MF_F32 (fp32 FMA throughout; any sizes).
 */
int tp_shard_mlp(const void* x, const void* w_gate_s, const void* w_up_s,
                 const void* w_down_s, int64_t T, int32_t d, int32_t f_s,
                 int32_t dtype, void* h_work, float* partial, void* stream);

/*
 * Measurement probes. Not part of the FFN path: they state what this GPU
 * sustains, so that a benchmark can report its kernels' fractions of the
 * attainable rates beside the published peaks.
 *
 * mf_probe_mfma_bf16 - `workgroups` workgroups of four waves; every wave
 *   issues iters * 16 back-to-back v_mfma_f32_32x32x16_bf16 on 16 independent
 *   accumulators (no memory traffic in the loop). FLOPs =
 *   workgroups * 4 * iters * 16 * 32768. out [workgroups * 256] f32 receives
 *   one folded value per thread.
 * mf_probe_hbm_read - reads bytes (a multiple of 16) of src once, with
 *   grid-strided 16-byte loads from `workgroups` 256-thread workgroups; out
 *   [workgroups * 256] u32 receives one folded word per thread.
 * mf_probe_hbm_copy - copies bytes (a multiple of 16) from src to dst with
 *   grid-strided 16-byte accesses from `workgroups` 256-thread workgroups:
 *   HBM traffic = 2 * bytes, the read + write pattern of a streaming kernel.
 * All are asynchronous on `stream`; time them with events. MF_EINVAL on bad
 * arguments.
 */
int mf_probe_mfma_bf16(int32_t workgroups, int32_t iters, float* out, void* stream);
int mf_probe_hbm_read(const void* src, int64_t bytes, int32_t workgroups, uint32_t* out,
                      void* stream);
int mf_probe_hbm_copy(const void* src, void* dst, int64_t bytes, int32_t workgroups,
                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEFFN_H */
