/*
 * libmoe -- the routed mixture-of-experts feed-forward layer on one AMD
 * Instinct MI355X (CDNA4, gfx950), as a C ABI.
 *
 * The layer is the one described in "Mixture of Experts (MoEs) in
 * Transformers" (Hugging Face blog).  Section "From Dense to Sparse": a
 * bank of small trainable feed-forward networks (experts) stands in for a
 * dense feed-forward block, and for each token a router picks a few of them
 * from that token's activations.  Section "Expert Backend": an execution
 * strategy has to route tokens to their chosen experts' weights, run the
 * projections, scale by the routing weights and return the results in
 * token order; its "grouped_mm" strategy orders tokens by expert, makes
 * each expert's tokens contiguous and runs one grouped matrix product.
 * The calls below are those steps, in order:
 *
 *   moe_route                        router logits, top-k, routing weights
 *   moe_topk                         top-k + weights from given logits
 *   moe_permute                      sort by expert ID (histogram, scan,
 *                                    stable scatter) + gather of the rows
 *   moe_permute_noalloc              the same with the library's own scratch
 *                                    (for callers that cannot allocate)
 *   moe_grouped_gemm_gateup_swiglu   per-expert gate/up projection + SwiGLU
 *   moe_grouped_gemm_gateup_swiglu_gather  the same, reading the rows
 *                                    through the sort instead of x_perm
 *   moe_grouped_gemm_down            per-expert down projection
 *   moe_unpermute_combine            weighted combine back to token order
 *   moe_localize_ids                 expert-parallel share: global ids to
 *   moe_localize_ids_strided         local ones, other experts masked
 *   moe_localize_ids_mapped          (a block, every N-th expert, or any set)
 *   moe_decode_gateup_swiglu         small-batch variants that stream only
 *   moe_decode_gateup_swiglu_gather  the active experts' weights (the
 *   moe_decode_down                  _gather form reads the rows through
 *                                    the sort instead of x_perm)
 *   moe_decode_gateup_swiglu_mxfp4   decode calls for MXFP4 expert weights
 *   moe_decode_down_mxfp4            (OCP MX: E2M1 codes, E8M0 block scales)
 *   moe_batched_gateup_swiglu        the small-batch "batched_mm" strategy:
 *   moe_batched_down_combine         per (token, slot) pair, no sort; the
 *                                    down call also applies the weights
 *   moe_batched_gateup_swiglu_mxfp4  the same with MXFP4 expert weights
 *   moe_batched_down_combine_mxfp4
 *   moe_batched_gateup_swiglu_select        batched gate/up that also selects
 *   moe_batched_gateup_swiglu_mxfp4_select  the experts from the logits
 *
 * All experts of a layer share one packed buffer per projection, the layout
 * the article's "Dynamic Weight Loading with WeightConverter" subsection
 * produces: per-expert gate (w1) and up (w3) matrices of shape [f, d] are
 * stacked over experts and concatenated along dim 1, giving
 * w_gate_up[E][2f][d] (rows [0, f) gate, rows [f, 2f) up); the down
 * projection is w_down[E][d][f].  All matrices are row-major.
 *
 * Conventions shared by every call
 *   - Every data pointer is DEVICE memory owned by the caller.  The library
 *     never allocates, frees, retains pointers past the return, or
 *     synchronises; work is enqueued on `stream` (a hipStream_t; NULL is the
 *     null stream) and the call returns after validation and launch.
 *   - Host-side validation runs before any launch; on any error nothing is
 *     launched and outputs are untouched.  Calls never abort and no C++
 *     exception crosses the ABI.  Faults inside kernels are asynchronous and
 *     surface at the caller's next synchronisation.
 *   - T == 0 (or rows == 0) is valid and launches nothing (moe_permute still
 *     zero-fills counts / offsets).
 *   - d and f must be multiples of 64; 1 <= k <= min(E, 16); 1 <= E <= 256;
 *     T * k < 2^31.  Data pointers must be 16-byte aligned.
 *   - Outputs must not alias inputs.
 *   - Index tensors are int32; routing weights and logits are fp32; the
 *     activation / weight element type is given by `dtype` (bf16 or fp32).
 *     bf16 paths accumulate in fp32 and round results to bf16 (RNE).
 *   - The library keeps no state, apart from the per-GPU scratch of
 *     moe_permute_noalloc: concurrent calls on different streams with
 *     disjoint buffers are allowed (moe_permute_noalloc excepted).
 */
#ifndef LIBMOE_H
#define LIBMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

#if defined(__GNUC__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null pointer, negative size, k/E out of range   */
  MOE_ERR_UNSUPPORTED = 2,  /* valid but outside what the kernels handle       */
  MOE_ERR_ALIGNMENT = 3,    /* pointer not 16-byte aligned, d or f not % 64    */
  MOE_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required      */
  MOE_ERR_HIP = 5           /* a HIP launch reported an error                  */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score;

/* ABI version (MOE_ABI_VERSION of the built library). */
MOE_API int moe_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
MOE_API const char* moe_status_string(moe_status s);

/*
 * Router (article, "From Dense to Sparse": per token, a few experts are
 * chosen from scores computed on the token's activations).
 *
 *   logits[t][e]  = sum_i x[t][i] * w_router[e][i] + bias[e]      (fp32)
 *   topk_ids[t][j] = expert with the j-th largest logit of token t; equal
 *                    logits go to the lower expert index
 *   topk_w[t][j]   = softmax over the k selected logits, or for
 *                    MOE_SCORE_SIGMOID sigmoid(logit) / sum of the k selected
 *                    sigmoids (both sum to 1 over j)
 *
 *   x        [T][d]  dtype          w_router [E][d] dtype
 *   bias     [E] fp32, may be NULL  logits   [T][E] fp32 (output)
 *   topk_ids [T][k] int32 (output)  topk_w   [T][k] fp32 (output)
 *   With topk_ids and topk_w both NULL only the logits are computed (the
 *   batched_mm "_select" calls then choose the experts); one of them NULL
 *   alone is MOE_ERR_INVALID_ARG.
 */
MOE_API moe_status moe_route(const void* x, const void* w_router, const float* bias,
                     int64_t T, int64_t d, int32_t E, int32_t k, moe_dtype dtype,
                     moe_score score, float* logits, int32_t* topk_ids,
                     float* topk_w, void* stream);

/*
 * The selection half of moe_route on caller-supplied fp32 logits [T][E]
 * (same outputs and tie rule).  No alignment requirement on `logits`.
 */
MOE_API moe_status moe_topk(const float* logits, int64_t T, int32_t E, int32_t k,
                    moe_score score, int32_t* topk_ids, float* topk_w,
                    void* stream);

/* Bytes of device workspace moe_permute needs for these sizes. */
MOE_API size_t moe_permute_workspace_size(int64_t T, int32_t k, int32_t E);

/*
 * Order the routed (token, slot) pairs by expert ID, each expert's pairs
 * contiguous ("grouped_mm" strategy, article section "Expert Backend").
 * With p = t*k + j:
 *
 *   counts[e]    = #{p : topk_ids[p] == e}
 *   offsets[0]   = 0, offsets[e+1] = offsets[e] + counts[e]  (offsets[E] = T*k)
 *   perm[r]      = the p placed at row r; rows of expert e are
 *                  [offsets[e], offsets[e+1]) in ascending p (stable)
 *   inv_perm[p]  = row of p
 *   x_perm[r][:] = x[perm[r] / k][:]     (skipped when x_perm is NULL)
 *
 *   topk_ids [T*k] int32             x [T][d] dtype (may be NULL iff x_perm is)
 *   counts [E], offsets [E+1], perm [T*k], inv_perm [T*k]  int32 outputs
 *   x_perm [T*k][d] dtype output
 *   ws / ws_bytes: device scratch of at least moe_permute_workspace_size()
 * Ids outside [0, E) mark pairs routed to experts this call does not hold
 * (an expert-parallel share, see moe_localize_ids): they get no row, are
 * counted nowhere and get inv_perm[p] = -1, so offsets[E] is the number of
 * pairs held here; perm and x_perm rows past offsets[E] are not written.
 * 1 <= k <= 16 (k may exceed E for such a share).
 */
MOE_API moe_status moe_permute(const int32_t* topk_ids, const void* x, int64_t T, int64_t d,
                       int32_t E, int32_t k, moe_dtype dtype, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                       void* x_perm, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_permute for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same outputs, but the per-chunk counts live in a scratch
 * array the library holds on each GPU (MOE_PERMUTE_SCRATCH_BYTES bytes,
 * held until the process ends) instead of a caller workspace.  The call
 * allocates nothing; its first call on a device looks up that device's
 * scratch address, with the device current (the current device must be the
 * one `stream` belongs to).  Sizes whose moe_permute_workspace_size()
 * exceeds MOE_PERMUTE_SCRATCH_BYTES (with E = 256 experts: more than
 * 1 048 576 pairs) return MOE_ERR_WORKSPACE, launching nothing.  Every call
 * on one GPU uses the same scratch, which keeps the last call's contents
 * (each call writes all of the part it reads first): calls that overlap on
 * one GPU (different streams, or other threads) race and must be
 * serialised by the caller.
 */
#define MOE_PERMUTE_SCRATCH_BYTES (1u << 20)

MOE_API moe_status moe_permute_noalloc(const int32_t* topk_ids, const void* x, int64_t T, int64_t d,
                                       int32_t E, int32_t k, moe_dtype dtype, int32_t* counts,
                                       int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                                       void* x_perm, void* stream);

/*
 * Grouped gate/up projection with SwiGLU, one group per expert:
 *
 *   for e, for r in [offsets[e], offsets[e+1]):
 *     g = x_perm[r] . w_gate_up[e][n]      (n < f, gate)
 *     u = x_perm[r] . w_gate_up[e][f + n]  (up)
 *     h[r][n] = silu(g) * u,  silu(g) = g / (1 + exp(-g))
 *
 *   x_perm [rows][d], w_gate_up [E][2f][d], h [rows][f]  (dtype)
 *   offsets [E+1] int32 (device), non-decreasing, offsets[0] = 0,
 *   offsets[E] <= rows.  Rows past offsets[E] are not written.  Offsets are
 *   clamped to [0, rows] on the device, so malformed offsets give wrong
 *   results but no out-of-bounds access.
 * bf16 tile loads address memory through 32-bit byte offsets from the
 * tile's base: one expert's w_gate_up[e] (2f * d * 2 bytes) must stay under
 * 2 GiB, else MOE_ERR_UNSUPPORTED (a Mixtral-shaped expert's is 235 MB).
 * The whole packed tensor and x_perm may be larger.
 */
MOE_API moe_status moe_grouped_gemm_gateup_swiglu(const void* x_perm, const void* w_gate_up,
                                          const int32_t* offsets, int64_t rows,
                                          int64_t d, int64_t f, int32_t E,
                                          moe_dtype dtype, void* h, void* stream);

/*
 * Grouped down projection, one group per expert:
 *   y_perm[r][c] = h[r] . w_down[e][c]   for r in expert e's rows, c < d
 *
 *   h [rows][f], w_down [E][d][f], y_perm [rows][d]  (dtype); offsets as above.
 * bf16: one expert's w_down[e] (d * f * 2 bytes) must stay under 2 GiB, else
 * MOE_ERR_UNSUPPORTED (32-bit tile offsets, as for the gate/up call).
 */
MOE_API moe_status moe_grouped_gemm_down(const void* h, const void* w_down,
                                 const int32_t* offsets, int64_t rows, int64_t d,
                                 int64_t f, int32_t E, moe_dtype dtype,
                                 void* y_perm, void* stream);

/*
 * Apply the routing weights and collect the rows back in token order
 * (article section "Expert Backend"):
 *   y[t][c] = sum_{j<k} topk_w[t][j] * y_perm[inv_perm[t*k + j]][c]
 *             (+ y_shared[t][c] when y_shared is not NULL)
 * summed in fp32 in increasing j, then the shared row, then rounded once.
 * Deterministic: no atomics.
 *
 *   y_perm [T*k][d], y_shared [T][d] or NULL, y [T][d]  (dtype)
 *   inv_perm [T*k] int32, topk_w [T][k] fp32
 * A negative inv_perm entry (a pair handled by another expert-parallel
 * share) adds nothing and no y_perm row is read for it, so rows that no
 * call wrote may hold anything; the others are clamped to [0, T*k).
 */
MOE_API moe_status moe_unpermute_combine(const void* y_perm, const int32_t* inv_perm,
                                 const float* topk_w, const void* y_shared,
                                 int64_t T, int64_t d, int32_t k, moe_dtype dtype,
                                 void* y, void* stream);

/*
 * Expert-parallel share (article, section "Expert Parallelism"): a device
 * that holds the experts [e_begin, e_begin + e_count) maps the router's
 * global ids to its local ones and masks the pairs of experts held
 * elsewhere:
 *   local_ids[i] = topk_ids[i] - e_begin   if e_begin <= topk_ids[i] < e_begin + e_count
 *                = -1                      otherwise
 * local_ids then feeds moe_permute with E = e_count and the share's slice
 * of the packed expert weights; moe_unpermute_combine gives the share's
 * partial output, and the partial outputs of all shares sum to the layer's
 * output (the exchange between devices is not part of this library).
 *   topk_ids, local_ids [n] int32 (device); 0 <= e_begin, 1 <= e_count <= 256.
 */
MOE_API moe_status moe_localize_ids(const int32_t* topk_ids, int64_t n, int32_t e_begin,
                                    int32_t e_count, int32_t* local_ids, void* stream);

/*
 * moe_localize_ids for a share that holds every e_stride-th expert:
 * e_begin, e_begin + e_stride, ..., e_begin + (e_count - 1) * e_stride (an
 * interleaved assignment, share i of N taking e_begin = i, e_stride = N,
 * spreads popular experts over the shares; the article's section "Expert
 * Parallelism" gives each device E/N experts without fixing which):
 *   local_ids[i] = (topk_ids[i] - e_begin) / e_stride
 *                    if topk_ids[i] is one of those experts
 *                = -1 otherwise
 * The share's packed expert weights hold its experts in that order.
 * e_stride = 1 is moe_localize_ids.  topk_ids, local_ids [n] int32
 * (device); 0 <= e_begin, 1 <= e_stride, 1 <= e_count <= 256, else
 * MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED.
 */
MOE_API moe_status moe_localize_ids_strided(const int32_t* topk_ids, int64_t n, int32_t e_begin,
                                            int32_t e_stride, int32_t e_count, int32_t* local_ids,
                                            void* stream);

/*
 * moe_localize_ids for a share that holds any set of e_count experts, in
 * an order of the caller's choice (for instance an assignment that spreads
 * the most loaded experts over the shares first; the article's section
 * "Expert Parallelism" gives each device E/N experts without fixing which):
 *   local_ids[i] = expert_map[topk_ids[i]]   if 0 <= topk_ids[i] < num_experts
 *                                            and 0 <= that entry < e_count
 *                = -1                        otherwise
 * expert_map [num_experts] int32 (device, read only) gives each global
 * expert's local id, or -1 for an expert held elsewhere; the share's packed
 * expert weights hold its experts in local-id order, and no two experts
 * should share a local id (the pairs of both would run on one expert's
 * weights).  topk_ids, local_ids [n] int32 (device).  1 <= num_experts <=
 * 256 and 1 <= e_count <= 256, else MOE_ERR_INVALID_ARG /
 * MOE_ERR_UNSUPPORTED; n = 0 launches nothing.
 */
MOE_API moe_status moe_localize_ids_mapped(const int32_t* topk_ids, int64_t n, const int32_t* expert_map,
                                           int32_t num_experts, int32_t e_count, int32_t* local_ids,
                                           void* stream);

/*
 * moe_grouped_gemm_gateup_swiglu with the row gather of moe_permute folded
 * into the tile loads: input row r is x[perm[r] / k] for the token
 * activations x [rows/k][d] and perm as written by moe_permute (same sort),
 * so moe_permute can be called with x_perm = NULL and the x_perm copy is
 * neither written nor read.  rows = T*k must be a multiple of k (1 <= k <=
 * 16, else MOE_ERR_INVALID_ARG); perm entries are clamped to [0, rows).
 * bf16 only (MOE_ERR_UNSUPPORTED for fp32, and when x exceeds 2 GiB).
 */
MOE_API moe_status moe_grouped_gemm_gateup_swiglu_gather(const void* x, const int32_t* perm,
                                                 int32_t k, const void* w_gate_up,
                                                 const int32_t* offsets, int64_t rows,
                                                 int64_t d, int64_t f, int32_t E,
                                                 moe_dtype dtype, void* h, void* stream);

/*
 * Small-batch (decode) variants of the two grouped projections, for rows
 * <= 1024: same arguments and results as the grouped calls, but the work is
 * split along the weight rows of the experts that have rows, so each active
 * expert's weights are streamed from HBM once and experts with no rows are
 * never read (article, "From Dense to Sparse": decode speed follows the
 * active parameters; section "Expert Backend": the small-batch strategy).
 * The form follows the rows per expert: vector-ALU dot products up to 2,
 * a split-K MFMA kernel above, and from 3 (gate/up) or 6 (down) the tile
 * kernel of the grouped calls, which then streams the weights fastest.
 * rows > 1024 returns MOE_ERR_UNSUPPORTED.
 */
MOE_API moe_status moe_decode_gateup_swiglu(const void* x_perm, const void* w_gate_up,
                                    const int32_t* offsets, int64_t rows, int64_t d,
                                    int64_t f, int32_t E, moe_dtype dtype, void* h,
                                    void* stream);

MOE_API moe_status moe_decode_down(const void* h, const void* w_down, const int32_t* offsets,
                           int64_t rows, int64_t d, int64_t f, int32_t E,
                           moe_dtype dtype, void* y_perm, void* stream);

/*
 * moe_decode_gateup_swiglu with the row gather of moe_permute folded into
 * its loads: input row r is x[perm[r] / k] for the token activations
 * x [rows/k][d] and perm as written by moe_permute, so moe_permute can be
 * called with x_perm = NULL.  rows = T*k must be a multiple of k (1 <= k <=
 * 16, else MOE_ERR_INVALID_ARG); perm entries are clamped to [0, rows).
 * bf16 only (MOE_ERR_UNSUPPORTED for fp32); rows <= 1024.
 */
MOE_API moe_status moe_decode_gateup_swiglu_gather(const void* x, const int32_t* perm, int32_t k,
                                           const void* w_gate_up, const int32_t* offsets,
                                           int64_t rows, int64_t d, int64_t f, int32_t E,
                                           moe_dtype dtype, void* h, void* stream);

/*
 * Decode calls with MXFP4 expert weights and bf16 activations (article,
 * section "From Dense to Sparse": decoding would be faster still with
 * kernels for the native mxfp4 format of the model's experts; section
 * "Where Quantization Fits In": weights quantised per expert).  MXFP4 is
 * the OCP Microscaling (MX) v1.0 format: blocks of 32 consecutive elements
 * along a weight row share one E8M0 scale code s (value 2^(s - 127), 255 =
 * NaN); each element is an FP4 E2M1 code (sign, 2 exponent bits with bias
 * 1, 1 mantissa bit), two per byte with element 2i in the low nibble.
 * Weight w[r][i] = 2^(s[r][i/32] - 127) * E2M1(code of element i of row r).
 *
 *   moe_decode_gateup_swiglu_mxfp4: as moe_decode_gateup_swiglu with
 *     wq_gate_up [E][2f][d/2] uint8 codes, ws_gate_up [E][2f][d/32] uint8
 *     scale codes (gate rows [0, f), up rows [f, 2f)); input row r is
 *     x[perm[r] / k] (x [rows/k][d], perm from moe_permute, 1 <= k <= 16,
 *     rows % k == 0), or x[r] when perm is NULL (x = x_perm [rows][d]);
 *     h [rows][f] bf16.
 *   moe_decode_down_mxfp4: as moe_decode_down with wq_down [E][d][f/2],
 *     ws_down [E][d][f/32]; h [rows][f], y_perm [rows][d] bf16.
 * Activations are bf16; products accumulate in fp32 (each block's sum is
 * scaled by its power of two, exact for scale codes 1..254 unless the
 * result overflows).  rows <= 1024, K (d for gate/up, f for down) <= 8192
 * and d * f <= 2^30, else MOE_ERR_UNSUPPORTED; codes, scales, activations
 * and outputs 16-byte aligned, else MOE_ERR_ALIGNMENT.  Experts with no
 * rows are never read.
 */
MOE_API moe_status moe_decode_gateup_swiglu_mxfp4(const void* x, const int32_t* perm, int32_t k,
                                                  const void* wq_gate_up, const void* ws_gate_up,
                                                  const int32_t* offsets, int64_t rows, int64_t d,
                                                  int64_t f, int32_t E, void* h, void* stream);

MOE_API moe_status moe_decode_down_mxfp4(const void* h, const void* wq_down, const void* ws_down,
                                         const int32_t* offsets, int64_t rows, int64_t d, int64_t f,
                                         int32_t E, void* y_perm, void* stream);

/*
 * The "batched_mm" strategy (article, section "Expert Backend": for small
 * batches, each token is multiplied with the weights of the experts it
 * selected, in one batched product, without sorting the tokens by expert).
 * The pairs p = t*k + j are taken in token order; each reads its expert's
 * weights in place (nothing is copied), so an expert chosen by several
 * pairs is read once per pair.  No moe_permute is needed.
 *
 * moe_batched_gateup_swiglu:
 *   h[p][n] = silu(x[t] . w_gate_up[e][n]) * (x[t] . w_gate_up[e][f + n]),
 *   e = topk_ids[p], t = p / k
 *   x [T][d], w_gate_up [E][2f][d], h [T*k][f]  (bf16); topk_ids [T][k] int32
 * moe_batched_down_combine:
 *   y[t][c] = sum_{j<k} topk_w[t][j] * (h[t*k+j] . w_down[e_tj][c])
 *             (+ y_shared[t][c] when y_shared is not NULL)
 *   summed in fp32 in increasing j, then the shared row, rounded once (the
 *   down products are not rounded to bf16 before the sum, unlike the
 *   grouped path's y_perm).  Deterministic: no atomics.
 *   h [T*k][f], w_down [E][d][f], y_shared [T][d] or NULL, y [T][d] (bf16);
 *   topk_w [T][k] fp32.
 * Pairs whose id is outside [0, E) (another expert-parallel share's, see
 * moe_localize_ids) get no h row and add nothing to y.  bf16 only
 * (MOE_ERR_UNSUPPORTED for fp32); T*k <= 1024 (else MOE_ERR_UNSUPPORTED).
 */
MOE_API moe_status moe_batched_gateup_swiglu(const void* x, const int32_t* topk_ids, const void* w_gate_up,
                                             int64_t T, int64_t d, int64_t f, int32_t E, int32_t k,
                                             moe_dtype dtype, void* h, void* stream);

MOE_API moe_status moe_batched_down_combine(const void* h, const int32_t* topk_ids, const float* topk_w,
                                            const void* w_down, const void* y_shared, int64_t T, int64_t d,
                                            int64_t f, int32_t E, int32_t k, moe_dtype dtype, void* y,
                                            void* stream);

/*
 * "batched_mm" with MXFP4 expert weights (the two sections above together:
 * the article's small-batch strategy on the MXFP4 layout of the
 * moe_decode_*_mxfp4 calls), bf16 activations and outputs, fp32
 * accumulation:
 *   moe_batched_gateup_swiglu_mxfp4: h[p] as moe_batched_gateup_swiglu with
 *     wq_gate_up [E][2f][d/2], ws_gate_up [E][2f][d/32].
 *   moe_batched_down_combine_mxfp4: y as moe_batched_down_combine with
 *     wq_down [E][d][f/2], ws_down [E][d][f/32] (y_shared may be NULL).
 * Pairs whose id is outside [0, E) get no h row and add nothing to y.
 * T*k <= 1024 and d, f <= 8192, else MOE_ERR_UNSUPPORTED; x, h, codes
 * 16-byte aligned.
 */
MOE_API moe_status moe_batched_gateup_swiglu_mxfp4(const void* x, const int32_t* topk_ids,
                                                   const void* wq_gate_up, const void* ws_gate_up, int64_t T,
                                                   int64_t d, int64_t f, int32_t E, int32_t k, void* h,
                                                   void* stream);

/*
 * The batched_mm gate/up calls with the expert selection folded in, for a
 * router whose logits were computed by moe_route with NULL ids and weights:
 * every workgroup selects its token's experts from logits [T][E] (fp32)
 * with the selection and weights of moe_topk (ids and weights bit for bit
 * the same), writes topk_ids [T][k] and topk_w [T][k] (for the down call),
 * and computes h as moe_batched_gateup_swiglu / _mxfp4 do (k <= E, else
 * MOE_ERR_INVALID_ARG, as for moe_topk).  The saving is
 * the top-k launch, which at one token costs about as much as the
 * selection itself.
 */
MOE_API moe_status moe_batched_gateup_swiglu_select(const void* x, const float* logits, const void* w_gate_up,
                                                    int64_t T, int64_t d, int64_t f, int32_t E, int32_t k,
                                                    moe_score score, moe_dtype dtype, int32_t* topk_ids,
                                                    float* topk_w, void* h, void* stream);

MOE_API moe_status moe_batched_gateup_swiglu_mxfp4_select(const void* x, const float* logits,
                                                          const void* wq_gate_up, const void* ws_gate_up,
                                                          int64_t T, int64_t d, int64_t f, int32_t E, int32_t k,
                                                          moe_score score, int32_t* topk_ids, float* topk_w,
                                                          void* h, void* stream);

MOE_API moe_status moe_batched_down_combine_mxfp4(const void* h, const int32_t* topk_ids, const float* topk_w,
                                                  const void* wq_down, const void* ws_down, const void* y_shared,
                                                  int64_t T, int64_t d, int64_t f, int32_t E, int32_t k, void* y,
                                                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBMOE_H */
