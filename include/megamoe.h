/*
 * megamoe.h - C ABI of libmegamoe.so, an NVFP4 routed-expert ("MegaMoE") layer for gfx950.
 *
 * The layer (nvfp4-megamoe-kernel, CURRENT_BUG.md@2e65594, "Architecture: DeepSeek-V4
 * MegaMoE" and "Test Plan" Phases 1-2) takes top-k routing over many experts, permutes
 * tokens by expert, quantizes activations to NVFP4, runs the L1 gate+up grouped GEMM,
 * applies SiLU(gate)*up, requantizes, runs the L2 down grouped GEMM and combines the
 * expert outputs with the routing weights.  One layer forward is the sequence
 *
 *   moe_route_permute -> nvfp4_quantize_act(x) -> moe_grouped_gemm_l1_silu
 *   -> nvfp4_quantize_act(h, amax from L1) -> moe_grouped_gemm_l2 -> moe_combine
 *
 * Starting from router logits instead of top-k ids, moe_route_logits (moe_router_topk, then
 * moe_route_permute on its ids) takes the place of moe_route_permute.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument is a DEVICE pointer owned by the caller.  The library never
 *   allocates or frees memory and keeps no state between calls; calls are reentrant.
 * - Every call only enqueues kernels on `stream` (a hipStream_t; NULL = the null stream).
 *   No call synchronises the device or copies device memory to the host.
 * - Argument checks run on the host before any HIP call.  Return values:
 *     MEGAMOE_OK              success (work enqueued)
 *     MEGAMOE_ERR_NULL        a required pointer is NULL
 *     MEGAMOE_ERR_SHAPE       a size is out of range (limits stated per function)
 *     MEGAMOE_ERR_WORKSPACE   workspace_bytes is smaller than the matching *_workspace_bytes()
 *     MEGAMOE_ERR_LAUNCH      a kernel launch failed (hipGetLastError after the launch)
 *     MEGAMOE_ERR_DEVICE      the current device is not gfx950
 * - Data errors on the device are defined away: a top-k id outside
 *   [expert_begin, expert_begin + num_experts) is "not local" and is dropped.
 * - Layouts are row-major.  NVFP4 tensors are three parts:
 *     codes  uint8 [rows, K/2]  two E2M1 codes per byte, the even element in the LOW nibble;
 *                               E2M1 = sign.exp(2).mantissa(1), magnitudes {0,.5,1,1.5,2,3,4,6};
 *     scales uint8 [rows, K/16] one OCP E4M3FN block scale per 16 consecutive K elements;
 *     gs     float             one FP32 global scale per tensor (per expert and matrix for
 *                               weights); the real value of element i is
 *                               e2m1(code_i) * e4m3(scale_block(i)) / gs.
 * - Expert weights: W13 codes [E, 2I, H/2], scales [E, 2I, H/16], gs [E]; rows 0..I-1 are the
 *   gate projection and rows I..2I-1 the up projection.  W2 codes [E, H, I/2], scales
 *   [E, H, I/16], gs [E].  bf16 tensors are passed as raw 16-bit storage.
 */
#ifndef MEGAMOE_H
#define MEGAMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MEGAMOE_OK 0
#define MEGAMOE_ERR_NULL (-1)
#define MEGAMOE_ERR_SHAPE (-2)
#define MEGAMOE_ERR_WORKSPACE (-3)
#define MEGAMOE_ERR_LAUNCH (-4)
#define MEGAMOE_ERR_DEVICE (-5)

/* Largest number of local experts one call handles. */
#define MEGAMOE_MAX_EXPERTS 1024

/* Largest number of global experts the router takes. */
#define MEGAMOE_ROUTER_MAX_EXPERTS 1024

/* Slots of the per-workgroup h amax written by moe_grouped_gemm_l1_silu (every slot, every call). */
#define MEGAMOE_L1_AMAX_PARTS 1280

/* Index of the error word in the sync workspace of moe_grouped_ffn_fused (uint32 words). */
#define MEGAMOE_FFN_SYNC_ERROR_WORD 352

/* ------------------------------------------------------------------------------------------
 * Host-side size helpers (no HIP calls; usable without a GPU).
 * ---------------------------------------------------------------------------------------- */

/* Rows of the permuted activation buffers: T*k + E*(P-1), enough for every local assignment
 * with each expert's rows padded to a multiple of P.  Returns -1 for invalid sizes. */
int64_t megamoe_row_capacity(int32_t T, int32_t k, int32_t num_experts, int32_t pad_multiple);

/* int32 entries of the `sched` table written by moe_route_permute for num_experts experts. */
int64_t megamoe_sched_len(int32_t num_experts);

/* Scratch bytes moe_route_permute needs for T tokens, top-k and num_experts experts. */
size_t megamoe_route_workspace_bytes(int32_t T, int32_t k, int32_t num_experts);

/* Scratch bytes nvfp4_quantize_act needs for a [rows, cols] tensor. */
size_t megamoe_quant_workspace_bytes(int64_t rows, int64_t cols);

/* Scratch bytes nvfp4_linear and nvfp4_linear_gate_up_silu need for M rows (0 if M is out of
 * range). */
size_t megamoe_dense_workspace_bytes(int64_t M);

/* Bytes of the sync workspace of moe_grouped_ffn_fused for num_experts experts (0 if out of
 * range). */
size_t megamoe_ffn_sync_bytes(int32_t num_experts);

/* ------------------------------------------------------------------------------------------
 * moe_router_topk - router logits -> top-k expert ids and weights.
 *
 * The routed experts receive topk_ids and topk_weights from the router (CURRENT_BUG.md@2e65594,
 * "Test Plan" Phase 1); the router of the workloads is a softmax over all global experts
 * followed by the k largest probabilities.
 *
 * logits             float32 [T, num_experts_global], finite.
 * topk_ids           int32 [T, k]   global expert ids by descending probability; equal
 *                    probabilities go to the lower id.
 * topk_weights       float32 [T, k] softmax probabilities over all num_experts_global experts
 *                    (float64 arithmetic, max-subtracted, rounded to float32), NOT renormalised
 *                    over the k chosen.
 * Limits: 0 <= T, 1 <= num_experts_global <= MEGAMOE_ROUTER_MAX_EXPERTS,
 * 1 <= k <= min(64, num_experts_global), T*k < 2^31.  Non-finite logits are outside the contract
 * (the outputs are then unspecified; no error is reported).
 * ---------------------------------------------------------------------------------------- */
int32_t moe_router_topk(const float* logits, int32_t T, int32_t num_experts_global, int32_t k,
                        int32_t* topk_ids, float* topk_weights, void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_route_logits - moe_router_topk, then moe_route_permute on the ids it wrote, in one call.
 *
 * Arguments as in those two functions; topk_ids and topk_weights are outputs (the ids feed the
 * permutation, the weights are for moe_combine).  Checks are those of both functions, all made
 * before any launch.
 * ---------------------------------------------------------------------------------------- */
int32_t moe_route_logits(const float* logits, int32_t T, int32_t num_experts_global, int32_t k,
                         int32_t expert_begin, int32_t num_experts, int32_t pad_multiple,
                         int32_t block_m_override, int32_t* topk_ids, float* topk_weights,
                         int32_t* counts, int32_t* expert_offsets, int32_t* padded_offsets,
                         int32_t* row_token, int32_t* token_rows, int32_t* sched, void* workspace,
                         size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_route_permute - local filter, per-expert counts, offsets, stable permutation, tile table.
 *
 * Defined by CURRENT_BUG.md@2e65594, "Test Plan" Phase 1 (the runner receives topk_ids and
 * variable token counts per expert, padded to 128 in vLLM) and Phase 2 (48-expert EP share of
 * 384, zero-token experts, expert_offsets and padded_expert_offsets).
 *
 * topk_ids        int32 [T, k]  global expert id of each (token, slot).  A token may list the
 *                 same expert in several slots; each (token, slot) is then an assignment of its own
 *                 (its own row), in ascending slot order.
 * expert_begin    first global expert held here; local expert e = id - expert_begin.
 * num_experts     E, local experts (1..MEGAMOE_MAX_EXPERTS).
 * pad_multiple    P >= 1: each expert's row block is padded to a multiple of P (zero stays 0).
 * block_m_override 0 = per-expert tile height chosen from the token count (16 for up to 16
 *                 tokens, 256 above); 16 or 256 forces that height for every expert.  The
 *                 choice changes speed only; results agree to FP32 summation order.
 * counts          int32 [E]     local assignments per expert.
 * expert_offsets  int32 [E+1]   exclusive prefix sum of counts.
 * padded_offsets  int32 [E+1]   exclusive prefix sum of round_up(counts, P).
 * row_token       int32 [M_cap] token of each permuted row, -1 for padding and unused rows;
 *                 M_cap = megamoe_row_capacity(T, k, E, P).  Expert e's rows start at
 *                 padded_offsets[e] and hold its tokens in ascending token order.
 * token_rows      int32 [T*k]   permuted row of each (token, slot), -1 if not local.
 * sched           int32 [megamoe_sched_len(E)]  tile table read by the GEMM entry points.
 * workspace       >= megamoe_route_workspace_bytes(T, k, E) bytes of scratch.
 * Limits: 0 <= T, 1 <= k <= 64, T*k < 2^31, P >= 1, M_cap < 2^31.
 * ---------------------------------------------------------------------------------------- */
int32_t moe_route_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t expert_begin,
                          int32_t num_experts, int32_t pad_multiple, int32_t block_m_override,
                          int32_t* counts, int32_t* expert_offsets, int32_t* padded_offsets,
                          int32_t* row_token, int32_t* token_rows, int32_t* sched,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the static per-GPU scratch of moe_route_permute_noalloc (1 MiB). */
#define MEGAMOE_ROUTE_NOALLOC_SCRATCH_BYTES (1 << 20)

/* ------------------------------------------------------------------------------------------
 * moe_route_permute_noalloc - moe_route_permute without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).
 *
 * Arguments and results as moe_route_permute, bit for bit, minus workspace / workspace_bytes.
 * The scratch moe_route_permute keeps in its workspace (the per-chunk expert histograms) lives in
 * a static array of MEGAMOE_ROUTE_NOALLOC_SCRATCH_BYTES bytes in device memory, one per GPU the
 * library runs on, held until the process ends; the call allocates nothing.  Sizes whose
 * megamoe_route_workspace_bytes(T, k, num_experts) exceeds that return MEGAMOE_ERR_WORKSPACE
 * before any launch (with 384 experts: up to 698,368 assignments, e.g. T = 116,394 at k = 6).
 * Every call on one GPU uses that GPU's one array: calls that overlap in time on the same GPU
 * (other streams, other host threads) race and must be ordered by the caller.  The first call on a
 * device looks up the array's device address (MEGAMOE_ERR_LAUNCH if that fails).
 * ---------------------------------------------------------------------------------------- */
int32_t moe_route_permute_noalloc(const int32_t* topk_ids, int32_t T, int32_t k, int32_t expert_begin,
                                  int32_t num_experts, int32_t pad_multiple, int32_t block_m_override,
                                  int32_t* counts, int32_t* expert_offsets, int32_t* padded_offsets,
                                  int32_t* row_token, int32_t* token_rows, int32_t* sched, void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_route_quantize - moe_route_permute and nvfp4_quantize_act of x in one call.
 *
 * The first two steps of the layer (route/permute, then quantize x: CURRENT_BUG.md@2e65594,
 * "Test Plan" Phase 1) do not depend on each other.  At decode sizes (T*k <= 1024 and
 * T*H <= 65536) they run as one launch, routing in one workgroup beside the quantization;
 * otherwise as the two calls would.  Results are those of the two calls, bit for bit.
 *
 * Routing arguments as in moe_route_permute (route_workspace = its workspace).  x_bf16 bf16
 * [T, H] with H > 0 a multiple of 32; x_codes [T, H/2], x_scales [T, H/16].
 * x_gs_in      NULL: the global scale comes from the amax of x, as in nvfp4_quantize_act, and is
 *              written to x_global_scale [1]; quant_workspace >= megamoe_quant_workspace_bytes(T,
 *              H) bytes.  Non-NULL (float [1] on the device): a calibrated scale, as in
 *              nvfp4_quantize_act_gs; x_global_scale and quant_workspace are then not used and
 *              may be NULL.
 * Checks are those of both functions, all made before any launch.
 * ---------------------------------------------------------------------------------------- */
int32_t moe_route_quantize(const int32_t* topk_ids, int32_t T, int32_t k, int32_t expert_begin,
                           int32_t num_experts, int32_t pad_multiple, int32_t block_m_override,
                           int32_t* counts, int32_t* expert_offsets, int32_t* padded_offsets,
                           int32_t* row_token, int32_t* token_rows, int32_t* sched,
                           void* route_workspace, size_t route_workspace_bytes, const void* x_bf16,
                           int64_t H, const float* x_gs_in, uint8_t* x_codes, uint8_t* x_scales,
                           float* x_global_scale, void* quant_workspace, size_t quant_workspace_bytes,
                           void* stream);

/* ------------------------------------------------------------------------------------------
 * nvfp4_quantize_act - NVFP4 quantization with a global scale derived from amax.
 *
 * The FP4 quantizer multiplies the input by a global scale before forming E4M3 block scales
 * (CURRENT_BUG.md@2fc81cc, "Root Cause" and "Key evidence": a global scale taken from a
 * checkpoint, 1/input_scale = 3977.6, overflows E4M3 on activations with amax 2-8).  Here
 * gs = fl32(2688 / amax) (2688 = 448 * 6, so no block scale can exceed E4M3's 448; gs = 1
 * when amax = 0).  Per 16-element block: scale = E4M3 round-to-nearest-even of the exact
 * value block_amax * gs / 6 (saturating at 448); each element's code is the E2M1 point
 * nearest to the exact value x * gs / scale, ties to the even code, sign copied from x.
 * Results are bit-exact with that definition.
 *
 * x_bf16       bf16 [rows, cols]; finite values.
 * rows, cols   rows >= 0, cols > 0 and a multiple of 32.
 * row_valid    nullable int32 [rows]: rows with row_valid[r] < 0 are excluded from amax and
 *              get zero codes and scales (pass row_token to quantize permuted rows).
 * amax_in      nullable float [amax_in_count]: partial maxima whose max is the amax of the valid
 *              rows, when already known (moe_grouped_gemm_l1_silu writes MEGAMOE_L1_AMAX_PARTS of
 *              them for h); NULL = computed here.
 * amax_in_count number of floats at amax_in (1..65536; ignored when amax_in is NULL).
 * codes        uint8 [rows, cols/2];  scales uint8 [rows, cols/16];  global_scale float [1].
 * workspace    >= megamoe_quant_workspace_bytes(rows, cols) bytes (may be NULL if that is 0).
 * ---------------------------------------------------------------------------------------- */
int32_t nvfp4_quantize_act(const void* x_bf16, int64_t rows, int64_t cols, const int32_t* row_valid,
                           const float* amax_in, int32_t amax_in_count, uint8_t* codes, uint8_t* scales,
                           float* global_scale,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * nvfp4_quantize_act_gs - NVFP4 quantization with a global scale given by the caller.
 *
 * The calibrated form of the quantizer above: the global scale is not derived from this
 * tensor's amax but supplied (e.g. measured on warm-up inputs), so no amax pass runs.  The
 * quantizer multiplies by the global scale before forming the E4M3 block scales
 * (CURRENT_BUG.md@2fc81cc, "Root Cause"); a global scale too large for the data (the
 * checkpoint's 3977.6 on amax 2-8 in "Key evidence") makes block_amax * gs / 6 exceed 448:
 * such a block gets the largest finite scale, 448 (0x7E), never NaN, and its elements saturate
 * at +-6.  Otherwise the block scale and element rules are those of nvfp4_quantize_act, with
 * the same bit-exact results for the same gs.
 *
 * global_scale_in float [1] on the device, finite and > 0 (other values are outside the
 *              contract; no error is reported).
 * Other arguments as in nvfp4_quantize_act; rows with row_valid[r] < 0 get zero codes and
 * scales.  No workspace.
 * ---------------------------------------------------------------------------------------- */
int32_t nvfp4_quantize_act_gs(const void* x_bf16, int64_t rows, int64_t cols, const int32_t* row_valid,
                              const float* global_scale_in, uint8_t* codes, uint8_t* scales,
                              void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_grouped_gemm_l1_silu - L1 gate+up grouped GEMM over experts with SiLU(gate)*up.
 *
 * CURRENT_BUG.md@2e65594, "Architecture: DeepSeek-V4 MegaMoE" (persistent grouped GEMM, tile
 * height 16-192 from the tokens per expert, per-expert shapes) and "Test Plan" Phase 1
 * (L1 gate+up GEMM, then SiLU).  For each expert e with counts[e] > 0 and each of its rows r
 * (padded_offsets[e] <= r < padded_offsets[e] + counts[e]):
 *   acc[n] = sum_k dec(x[row_token[r], k]) * dec(W13[e, n, k]),  n in [0, 2I)
 *   h[r, i] = bf16( SiLU(acc[i] / (gs_x * gs13[e])) * acc[I+i] / (gs_x * gs13[e]) )
 * with exact E2M1*E4M3 decode, FP16 MFMA products and FP32 accumulation.  Rows of h that hold
 * no assignment are not written.  Every workgroup writes the max |h| of the rows it wrote (0 if
 * none) into its own slot of h_amax_parts, and every slot is written on every call, so the max
 * over the MEGAMOE_L1_AMAX_PARTS slots is max |h| over the valid rows (no reset, no atomics).
 * Experts with no tokens are never read.
 *
 * x_codes/x_scales/x_gs   NVFP4 x per token: [T, H/2], [T, H/16], [1].
 * row_token, padded_offsets, counts, sched   as written by moe_route_permute.
 * w13_codes/w13_scales/w13_gs   [E, 2I, H/2], [E, 2I, H/16], [E].
 * E, H, I      E as given to moe_route_permute; H a multiple of 256, I a multiple of 128.
 * M_cap        rows of h: megamoe_row_capacity(T, k, E, P).
 * block_m_override  the value given to moe_route_permute (0, 16 or 256).
 * max_rows_per_expert  a bound on counts[e] the caller expects, or 0 if none (e.g. T when no
 *              token lists an expert twice).  It changes which kernels launch, never the results:
 *              with block_m_override 0 and a bound of at most 16 only the 16-row tile kernel is
 *              launched (one launch fewer at decode), and it then also computes, in 16-row tiles,
 *              any expert whose count turns out to exceed the bound.  A bound that is too low
 *              costs time only.
 * h_bf16       bf16 [M_cap, I].   h_amax_parts float [MEGAMOE_L1_AMAX_PARTS].
 * With M_cap == 0 (e.g. T == 0) there are no rows: x_codes, x_scales, row_token and h_bf16 may
 * be NULL, no table is read, and the call only sets every slot of h_amax_parts to 0.
 * ---------------------------------------------------------------------------------------- */
int32_t moe_grouped_gemm_l1_silu(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs,
                                 const int32_t* row_token, const int32_t* padded_offsets,
                                 const int32_t* counts, const int32_t* sched,
                                 const uint8_t* w13_codes, const uint8_t* w13_scales, const float* w13_gs,
                                 int32_t E, int32_t H, int32_t I, int64_t M_cap,
                                 int32_t block_m_override, int32_t max_rows_per_expert,
                                 void* h_bf16, float* h_amax_parts, void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_grouped_gemm_l1_silu_nvfp4 - moe_grouped_gemm_l1_silu with h written as NVFP4 under a
 * calibrated global scale, in the GEMM's epilogue.
 *
 * The L1 of the layer followed by the requantization of h (CURRENT_BUG.md@2e65594, "Test Plan"
 * Phase 1: L1 gate+up, SiLU, requantize, L2) when the global scale of h is known beforehand
 * (CURRENT_BUG.md@2fc81cc, "Root Cause": the checkpoint carries per-layer input scales): each
 * 16-column block of a row of h is quantized as soon as the tile that holds it is done, so h
 * never goes through memory in bf16 and no separate quantization launch runs.  For every row
 * holding an assignment, h_codes and h_scales equal bit for bit those nvfp4_quantize_act_gs
 * writes for the bf16 h of moe_grouped_gemm_l1_silu with the same h_gs; other rows are not
 * written.  h_amax_parts is written as by moe_grouped_gemm_l1_silu (max |h| of the bf16 h), so
 * a caller can watch the calibration.
 *
 * Arguments as for moe_grouped_gemm_l1_silu, with h_bf16 replaced by
 * h_gs         float [1] on the device: the global scale of h (e.g. from a warm-up pass).
 * h_codes      uint8 [M_cap, I/2];   h_scales  uint8 [M_cap, I/16].
 * With M_cap == 0, x_codes, x_scales, row_token, h_codes and h_scales may be NULL and the call
 * only sets every slot of h_amax_parts to 0.
 * ---------------------------------------------------------------------------------------- */
int32_t moe_grouped_gemm_l1_silu_nvfp4(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs,
                                       const int32_t* row_token, const int32_t* padded_offsets,
                                       const int32_t* counts, const int32_t* sched,
                                       const uint8_t* w13_codes, const uint8_t* w13_scales,
                                       const float* w13_gs, int32_t E, int32_t H, int32_t I,
                                       int64_t M_cap, int32_t block_m_override,
                                       int32_t max_rows_per_expert, const float* h_gs,
                                       uint8_t* h_codes, uint8_t* h_scales, float* h_amax_parts,
                                       void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_grouped_gemm_l2 - L2 down grouped GEMM over experts.
 *
 * CURRENT_BUG.md@2e65594, "Test Plan" Phase 1 (L2 GEMM after SiLU) and "What's Been Verified"
 * (NVFP4 MoE, L1 gate+up and L2 down).  For each expert e with counts[e] > 0 and each row r:
 *   y[r, n] = bf16( sum_k dec(h[r, k]) * dec(W2[e, n, k]) / (gs_h * gs2[e]) ),  n in [0, H)
 * Rows of y that hold no assignment are not written.
 *
 * h_codes/h_scales/h_gs   NVFP4 h [M_cap, I/2], [M_cap, I/16], [1] (from nvfp4_quantize_act).
 * padded_offsets, counts, sched   as written by moe_route_permute.
 * w2_codes/w2_scales/w2_gs   [E, H, I/2], [E, H, I/16], [E].
 * block_m_override, max_rows_per_expert   as for moe_grouped_gemm_l1_silu.
 * y_bf16       bf16 [M_cap, H].
 * With M_cap == 0, h_codes, h_scales and y_bf16 may be NULL and the call enqueues nothing.
 * ---------------------------------------------------------------------------------------- */
int32_t moe_grouped_gemm_l2(const uint8_t* h_codes, const uint8_t* h_scales, const float* h_gs,
                            const int32_t* padded_offsets, const int32_t* counts, const int32_t* sched,
                            const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_gs,
                            int32_t E, int32_t H, int32_t I, int64_t M_cap, int32_t block_m_override,
                            int32_t max_rows_per_expert, void* y_bf16, void* stream);

/* ------------------------------------------------------------------------------------------
 * nvfp4_pack_weight_codes - a second copy of NVFP4 weight codes in the layout the 16-row GEMM
 * kernels stream fastest (the *_packed GEMMs below).
 *
 * Same codes, permuted; no arithmetic (the weights are those of CURRENT_BUG.md@2e65594, "Test
 * Plan" Phase 1: E2M1 codes, two per byte).  codes [rows, K/2] row-major (e.g. W13 with rows =
 * E * 2I and K = H, or W2 with rows = E * H and K = I) -> packed [rows * K/2] bytes: for 16-row
 * block b (rows 16b .. 16b+15), 256-element chunk c of K and half q (0, 1) of the chunk's
 * 2 KB, the 1 KB at byte ((b * (K/256) + c) * 2 + q) * 1024 holds, for L = 16g + r (r < 16,
 * g < 4), the 16 code bytes 32g + 16q .. 32g + 16q + 15 of chunk c of row 16b + r at 16L.  The
 * scales keep their row-major layout.  Caller-owned device buffers; the call only enqueues on
 * `stream`.  Errors: rows not a positive multiple of 16 or K not a positive multiple of 256 ->
 * -2; NULL pointer -> -1.
 * ---------------------------------------------------------------------------------------- */
int32_t nvfp4_pack_weight_codes(const uint8_t* codes, int64_t rows, int64_t K, uint8_t* packed, void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_grouped_gemm_l1_silu_packed, moe_grouped_gemm_l1_silu_nvfp4_packed,
 * moe_grouped_gemm_l2_packed - the three grouped GEMMs above, with one more argument after the
 * weights' global scales: w13_packed / w2_packed, the same weight codes as packed by
 * nvfp4_pack_weight_codes (W13 as [E * 2I] rows of K = H, W2 as [E * H] rows of K = I).
 *
 * Same operation and the same results, bit for bit.  The 16-row kernels read the packed copy
 * (each load instruction 1 KB contiguous, non-temporal); the 256-row kernels read the row-major
 * codes, which stay required.  Errors as for the unpacked calls, and: packed NULL -> -1;
 * L2 with I not a multiple of 256 -> -2.
 * ---------------------------------------------------------------------------------------- */
int32_t moe_grouped_gemm_l1_silu_packed(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs,
                                        const int32_t* row_token, const int32_t* padded_offsets,
                                        const int32_t* counts, const int32_t* sched, const uint8_t* w13_codes,
                                        const uint8_t* w13_scales, const float* w13_gs, const uint8_t* w13_packed,
                                        int32_t E, int32_t H, int32_t I, int64_t M_cap, int32_t block_m_override,
                                        int32_t max_rows_per_expert, void* h_bf16, float* h_amax_parts,
                                        void* stream);
int32_t moe_grouped_gemm_l1_silu_nvfp4_packed(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs,
                                              const int32_t* row_token, const int32_t* padded_offsets,
                                              const int32_t* counts, const int32_t* sched, const uint8_t* w13_codes,
                                              const uint8_t* w13_scales, const float* w13_gs,
                                              const uint8_t* w13_packed, int32_t E, int32_t H, int32_t I,
                                              int64_t M_cap, int32_t block_m_override, int32_t max_rows_per_expert,
                                              const float* h_gs, uint8_t* h_codes, uint8_t* h_scales,
                                              float* h_amax_parts, void* stream);
int32_t moe_grouped_gemm_l2_packed(const uint8_t* h_codes, const uint8_t* h_scales, const float* h_gs,
                                   const int32_t* padded_offsets, const int32_t* counts, const int32_t* sched,
                                   const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_gs,
                                   const uint8_t* w2_packed, int32_t E, int32_t H, int32_t I, int64_t M_cap,
                                   int32_t block_m_override, int32_t max_rows_per_expert, void* y_bf16,
                                   void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_grouped_ffn_fused - L1 gate+up with SiLU(gate)*up, the requantization of h and L2 down in
 * one persistent launch (experts taken in 16-row m-tiles: decode sizes).
 *
 * The layer's L1, requantize and L2 steps (CURRENT_BUG.md@2e65594, "Test Plan" Phase 1), with
 * persistent scheduling across expert groups ("Architecture: DeepSeek-V4 MegaMoE"), as one
 * launch instead of two or three, to cut the kernel boundaries of a decode step.  The global scale
 * of h is either calibrated (CURRENT_BUG.md@2fc81cc, "What we've tried": a scale from a warm-up
 * pass; h is then quantized in the L1 epilogue and an expert's L2 starts as soon as its own L1 is
 * done) or the per-tensor amax scale of nvfp4_quantize_act (every L1 group must finish before h
 * is quantized: a wait across the whole launch).  Work is claimed in order from a counter per XCD,
 * so the launch never depends on all workgroups being resident at once.
 *
 * Results, bit for bit, are those of moe_grouped_gemm_l1_silu (or _nvfp4 with h_gs_in), then
 * nvfp4_quantize_act of h with row_valid = row_token and amax_in = h_amax_parts (not with
 * h_gs_in), then moe_grouped_gemm_l2, when those run every expert in 16-row m-tiles (as they do
 * when every expert has at most 16 rows, or with block_m_override 16).  Any routing is accepted;
 * experts with more rows are covered in 16-row m-tiles too (correct, but slow beyond decode).
 *
 * x_codes, x_scales, x_gs, row_token, padded_offsets, counts, sched, w13_*   as for
 *              moe_grouped_gemm_l1_silu.      w2_*   as for moe_grouped_gemm_l2.
 * E, H, I, M_cap   as for the grouped GEMMs.
 * h_gs_in      NULL: the global scale of h is derived from its amax and written to h_gs_out [1];
 *              h_bf16 (bf16 [M_cap, I]) receives the unquantized h.  Non-NULL (float [1] on the
 *              device): a calibrated scale; h_gs_out and h_bf16 are then not used and may be NULL.
 * h_amax_parts float [MEGAMOE_L1_AMAX_PARTS]: as written by moe_grouped_gemm_l1_silu (every slot,
 *              max over them = max |h| over the valid rows).
 * h_codes, h_scales   uint8 [M_cap, I/2], [M_cap, I/16]: NVFP4 h.  Without h_gs_in, rows holding
 *              no assignment are set to zero; with h_gs_in they are not written.
 * y_bf16       bf16 [M_cap, H]; rows holding no assignment are not written.
 * sync         device memory of at least megamoe_ffn_sync_bytes(E) bytes, all zero before the
 *              first call (e.g. from a zeroing allocation).  Every call leaves its counters at zero
 *              again.  Word MEGAMOE_FFN_SYNC_ERROR_WORD becomes non-zero, and stays so, if a wait
 *              inside the launch ever expired (about 0.25 s): results of that call are undefined.
 *              Calls that share one sync buffer must not overlap in time (one stream).
 * With M_cap == 0 nothing is computed: the call only sets every slot of h_amax_parts to 0 and,
 * without h_gs_in, writes 1.0 to h_gs_out.
 * Errors: MEGAMOE_ERR_SHAPE as for the grouped GEMMs; MEGAMOE_ERR_NULL for a missing pointer;
 * MEGAMOE_ERR_WORKSPACE if sync_bytes is too small.
 * ---------------------------------------------------------------------------------------- */
int32_t moe_grouped_ffn_fused(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs,
                              const int32_t* row_token, const int32_t* padded_offsets,
                              const int32_t* counts, const int32_t* sched, const uint8_t* w13_codes,
                              const uint8_t* w13_scales, const float* w13_gs, const uint8_t* w2_codes,
                              const uint8_t* w2_scales, const float* w2_gs, int32_t E, int32_t H,
                              int32_t I, int64_t M_cap, const float* h_gs_in, void* h_bf16,
                              float* h_amax_parts, uint8_t* h_codes, uint8_t* h_scales,
                              float* h_gs_out, void* y_bf16, void* sync, size_t sync_bytes,
                              void* stream);

/* moe_grouped_ffn_fused_packed - moe_grouped_ffn_fused with the packed copies of both weights'
 * codes (nvfp4_pack_weight_codes; w13_packed, w2_packed after w2_gs), read by its 16-row passes.
 * Same results, bit for bit.  Errors as for moe_grouped_ffn_fused, and: a packed copy NULL -> -1;
 * I not a multiple of 256 -> -2.  (For the callers of the *_packed grouped GEMMs above.) */
int32_t moe_grouped_ffn_fused_packed(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs,
                                     const int32_t* row_token, const int32_t* padded_offsets, const int32_t* counts,
                                     const int32_t* sched, const uint8_t* w13_codes, const uint8_t* w13_scales,
                                     const float* w13_gs, const uint8_t* w2_codes, const uint8_t* w2_scales,
                                     const float* w2_gs, const uint8_t* w13_packed, const uint8_t* w2_packed,
                                     int32_t E, int32_t H, int32_t I, int64_t M_cap, const float* h_gs_in,
                                     void* h_bf16, float* h_amax_parts, uint8_t* h_codes, uint8_t* h_scales,
                                     float* h_gs_out, void* y_bf16, void* sync, size_t sync_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * nvfp4_linear - dense NVFP4 linear layer: the L2 GEMM with one group holding every row.
 *
 * The expert GEMM of moe_grouped_gemm_l2 (CURRENT_BUG.md@2e65594, "What's Been Verified": NVFP4
 * L1/L2) for a single expert applied to all M rows, as for a dense projection:
 *   out[m, n] = bf16( sum_k dec(a[m, k]) * dec(W[n, k]) / (gs_a * gs_w) )
 * a_codes/a_scales/a_gs   NVFP4 A [M, K/2], [M, K/16], [1] (e.g. from nvfp4_quantize_act).
 * w_codes/w_scales/w_gs   NVFP4 W [N, K/2], [N, K/16], [1].
 * out_bf16     bf16 [M, N].
 * workspace    >= megamoe_dense_workspace_bytes(0) bytes (64; the group's tables are written
 *              there before the GEMM runs).
 * Limits: 0 <= M < 2^31, K >= 128 and a multiple of 128, N >= 256 and a multiple of 256.
 * ---------------------------------------------------------------------------------------- */
int32_t nvfp4_linear(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs, int64_t M,
                     int32_t K, const uint8_t* w_codes, const uint8_t* w_scales, const float* w_gs,
                     int32_t N, void* out_bf16, void* workspace, size_t workspace_bytes,
                     void* stream);

/* ------------------------------------------------------------------------------------------
 * nvfp4_linear_gate_up_silu - dense gate+up projection with SiLU(gate)*up: the L1 GEMM with one
 * group holding every row.
 *
 * As moe_grouped_gemm_l1_silu (CURRENT_BUG.md@2e65594, "Test Plan" Phase 1: L1 gate+up, then
 * SiLU) for a single expert applied to all M rows, e.g. a shared expert:
 *   h[m, i] = bf16( SiLU(g) * u ),  g / u = sum_k dec(a[m, k]) * dec(W13[i or I+i, k]) / (gs_a * gs_w)
 * a_codes/a_scales/a_gs   NVFP4 A [M, K/2], [M, K/16], [1].
 * w13_codes/w13_scales/w13_gs   [2I, K/2], [2I, K/16], [1]; rows 0..I-1 gate, I..2I-1 up.
 * h_bf16       bf16 [M, I].  h_amax_parts float [MEGAMOE_L1_AMAX_PARTS]: as for
 *              moe_grouped_gemm_l1_silu (max |h| = max over the slots; every slot written).
 * workspace    >= megamoe_dense_workspace_bytes(M) bytes (the group's tables and an identity
 *              row map).
 * Limits: 0 <= M < 2^31, K >= 256 and a multiple of 256, I >= 128 and a multiple of 128.
 * ---------------------------------------------------------------------------------------- */
int32_t nvfp4_linear_gate_up_silu(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                                  int64_t M, int32_t K, const uint8_t* w13_codes,
                                  const uint8_t* w13_scales, const float* w13_gs, int32_t I,
                                  void* h_bf16, float* h_amax_parts, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * nvfp4_linear_gate_up_silu_nvfp4 - nvfp4_linear_gate_up_silu with h written as NVFP4 under a
 * calibrated global scale, in the GEMM's epilogue (as moe_grouped_gemm_l1_silu_nvfp4 for the
 * single group: CURRENT_BUG.md@2e65594, "Test Plan" Phase 1; CURRENT_BUG.md@2fc81cc, "Root
 * Cause").  h_codes/h_scales equal bit for bit those nvfp4_quantize_act_gs writes for the bf16 h
 * of nvfp4_linear_gate_up_silu with the same h_gs, on every row.
 * h_gs         float [1] on the device.   h_codes uint8 [M, I/2];   h_scales uint8 [M, I/16].
 * Other arguments, workspace and limits as for nvfp4_linear_gate_up_silu.
 * ---------------------------------------------------------------------------------------- */
int32_t nvfp4_linear_gate_up_silu_nvfp4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_gs,
                                        int64_t M, int32_t K, const uint8_t* w13_codes,
                                        const uint8_t* w13_scales, const float* w13_gs, int32_t I,
                                        const float* h_gs, uint8_t* h_codes, uint8_t* h_scales,
                                        float* h_amax_parts, void* workspace, size_t workspace_bytes,
                                        void* stream);

/* ------------------------------------------------------------------------------------------
 * moe_combine - routing-weighted combine of the expert outputs back into token order.
 *
 * The last step of the layer: the runner receives topk_weights with the top-k ids
 * (CURRENT_BUG.md@2e65594, "Test Plan" Phase 1) and the routed experts' outputs are summed back
 * per token, each weighted by its routing weight, with the tokens that have no local expert in
 * the 48-of-384 expert-parallel share giving zero ("Test Plan" Phase 2).  The routing weight of
 * each (token, expert) is applied exactly once, here:
 *   out[t, :] = bf16( sum over j = 0..k-1 ascending, token_rows[t*k+j] >= 0, of
 *                     topk_weights[t, j] * y[token_rows[t*k+j], :] )    (FP32 accumulation)
 * Tokens with no local assignment get +0.
 *
 * y_bf16 [M_cap, H] bf16;  token_rows int32 [T*k];  topk_weights float [T, k];
 * out_bf16 bf16 [T, H];  T >= 0, 1 <= k <= 64, H a multiple of 8.
 *
 * moe_combine_shared adds a shared expert's output (weight 1, one row per token, bf16 [T, H],
 * e.g. from nvfp4_linear) to the routed sum before the rounding:
 *   out[t, :] = bf16( (sum over j as above) + y_shared[t, :] )
 * ---------------------------------------------------------------------------------------- */
int32_t moe_combine_shared(const void* y_bf16, const int32_t* token_rows, const float* topk_weights,
                           int32_t T, int32_t k, int32_t H, const void* y_shared_bf16, void* out_bf16,
                           void* stream);

int32_t moe_combine(const void* y_bf16, const int32_t* token_rows, const float* topk_weights,
                    int32_t T, int32_t k, int32_t H, void* out_bf16, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MEGAMOE_H */
