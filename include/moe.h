/*
 * moe.h -- C ABI of libmoe, the MI355X (gfx950) DeepSeekMoE layer forward with
 * auxiliary-loss-free load balancing.
 *
 * The layer (DeepSeek-V3 report, as summarised on mpbf.cn "DeepSeek-V3技术报告",
 * section 2.2 "DeepSeekMoE 与无辅助损失"):
 *   - the FFN is one always-on shared expert plus E fine-grained routed experts;
 *   - token-expert affinity s = sigmoid(x . w_router[e]);
 *   - each expert carries a bias b[e] that is added to s only to choose experts;
 *   - the choice is limited to M of G expert groups (the single-GPU form of
 *     node-limited routing: groups ranked by the summed affinity of their experts);
 *   - the gate of a chosen expert is its unbiased s divided by the sum of s over the
 *     K chosen experts;
 *   - no token is dropped; per-expert loads over the whole batch drive the bias
 *     update after each step: overloaded experts lose gamma, underloaded gain gamma.
 * The output is the shared expert's output plus the gate-weighted routed outputs
 * (blog.resmic.cn "DeepSeek-V3架构深度解析", section 核心架构二).
 *
 * One forward step is five calls on one stream:
 *   moe_route -> moe_permute -> moe_expert_ffn -> moe_combine, then moe_bias_update.
 * The same step without the permuted copy of x: moe_permute with x_sorted = NULL
 * (index maps only), [FP8: moe_quantize_act_fp8], moe_expert_ffn_up_gather,
 * moe_expert_ffn_down, moe_combine, moe_bias_update -- identical results.
 *
 * Conventions for every call
 *   - All tensor pointers are DEVICE pointers, row-major, contiguous, 16-byte aligned.
 *     The caller owns and allocates every buffer, including the workspace; the library
 *     never allocates or frees device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Calls only
 *     enqueue work; none synchronises the host.
 *   - Arguments are validated before anything is launched.  On a negative status
 *     nothing was enqueued and no output was written; moe_last_error() gives the reason
 *     (a per-thread string).
 *   - Outputs are overwritten entirely; the only in/out argument is `bias`.
 *   - Calls that share no output buffers may run concurrently on different streams; the
 *     library keeps no mutable global state apart from the per-thread error string and
 *     the scratch array of moe_permute_noalloc (see there).
 *
 * Problem limits (checked): 1 <= T, T*(K+1) < 2^31; H % 128 == 0, 128 <= H <= 65536;
 * I % 128 == 0, 128 <= I <= 32768, H*I <= 2^28 (one expert's weights addressed with
 * 32-bit byte offsets); 1 <= E <= 512, E % G == 0, 1 <= G <= 64,
 * 1 <= M <= G, 1 <= J <= min(E/G, 8), 1 <= K <= min(M*E/G, 16); S in {0, 1}.
 * Dtypes: act_dtype F32 with expert_dtype F32, or act_dtype BF16 with expert_dtype
 * BF16 or FP8_E4M3.  Inputs must be finite.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* a size, pointer or dtype violates the limits above */
  MOE_ERR_UNSUPPORTED = -2, /* no kernel for this combination (e.g. no gfx950 device) */
  MOE_ERR_WORKSPACE = -3,   /* ws is NULL or smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

typedef struct moe_problem {
  int64_t T;            /* tokens in the batch (one step)                              */
  int32_t H;            /* hidden width                                                */
  int32_t E;            /* routed experts                                              */
  int32_t G;            /* expert groups (experts g*E/G .. (g+1)*E/G-1 form group g)    */
  int32_t M;            /* groups a token may use                                      */
  int32_t K;            /* routed experts per token                                    */
  int32_t J;            /* keys summed into a group's score                            */
  int32_t I;            /* FFN (SwiGLU) width of every expert                          */
  int32_t S;            /* shared experts: 0 or 1                                      */
  int32_t act_dtype;    /* moe_dtype of x, y_sorted and y: MOE_F32 | MOE_BF16           */
  int32_t expert_dtype; /* moe_dtype of the GEMM operands: MOE_F32 | MOE_BF16 | FP8     */
} moe_problem;

/* Rows of the permuted buffers: R = T*K + S*T (routed rows, then T shared rows). */

enum { MOE_CALL_ROUTE = 0, MOE_CALL_PERMUTE = 1, MOE_CALL_EXPERT_FFN = 2 };

/* Workspace bytes a call needs for problem p (0 if none).  Returns 0 and sets the
 * last error for an invalid problem or call id. */
size_t moe_workspace_bytes(const moe_problem* p, int32_t which_call);

/* Routing (mpbf.cn section 2.2; node-limited routing in the same section).
 *   x         [T,H]  act_dtype   token activations
 *   w_router  [E,H]  fp32        router weight
 *   bias      [E]    fp32        per-expert routing bias
 *   topk_idx  [T,K]  int32  out  chosen experts, in rank order (largest key first)
 *   topk_gate [T,K]  fp32   out  s / sum of s over the K chosen (unbiased)
 *   expert_counts [E] int32 out  tokens routed to each expert in this batch
 *   logits_out [T,E] fp32   out  router logits z, or NULL to keep them in ws
 *   ws        >= moe_workspace_bytes(p, MOE_CALL_ROUTE) bytes (T*E*4 when logits_out
 *             is NULL; the same size is reported either way)
 * Numerics: z[t,e] is a sequential fused multiply-add chain over h = 0..H-1 from +0;
 * s = 1/(1+exp(-clamp(z,-80,80))) with a Cody-Waite/Taylor-7 exp; key = s + bias;
 * group score = fp32 sum, from 0, of the group's J largest keys; groups and experts
 * are ranked by (value descending, index ascending); gate = s / sum (IEEE division).
 * The result is bit-for-bit reproducible. */
moe_status moe_route(const moe_problem* p, const void* x, const float* w_router,
                     const float* bias, int32_t* topk_idx, float* topk_gate,
                     int32_t* expert_counts, float* logits_out, void* ws, size_t ws_bytes,
                     void* stream);

/* Permute: the single-GPU form of the dispatch step (mpbf.cn section 3.2: a block is
 * attention / dispatch / expert MLP / combine).  Rows are grouped by expert in index
 * order; within an expert, tokens ascend; the shared expert (S = 1) is the last group
 * and holds every token in order.
 *   x            [T,H] act_dtype
 *   topk_idx     [T,K] int32   from moe_route; every value must lie in [0,E) (moe_route
 *                              only writes such values; moe_count_invalid_ids checks
 *                              indices of other origin).  A pair outside it is skipped
 *                              and its inv_perm entry is -1 (writes stay in bounds);
 *                              offsets[E] is then T*K less the skipped pairs, and the
 *                              calls that read the shared rows at T*K + t (the FFN's
 *                              dense shared launch, the combine, the backward) are not
 *                              defined for such input
 *   offsets      [E+S+1] int32 out  first row of each group; offsets[E] = T*K (for
 *                                   topk_idx within [0,E), the precondition above)
 *   sorted_token [R]     int32 out  token of each row
 *   inv_perm     [T,K]   int32 out  row holding (t, topk_idx[t,k])
 *   x_sorted     [R,H]   out  act_dtype rows, or FP8 E4M3 codes when expert_dtype is
 *                             FP8 (each token quantised once per 128-column tile:
 *                             scale = amax/448, code = RNE-saturating E4M3 of x/scale)
 *   x_sorted_scale [R,H/128] fp32 out (FP8 only, else NULL)
 *   ws           >= moe_workspace_bytes(p, MOE_CALL_PERMUTE) bytes
 * x_sorted = NULL: only offsets, sorted_token and inv_perm are written (x and
 * x_sorted_scale are then not used), for moe_expert_ffn_up_gather.
 * Deterministic: every output is a pure function of the inputs. */
moe_status moe_permute(const moe_problem* p, const void* x, const int32_t* topk_idx,
                       int32_t* offsets, int32_t* sorted_token, int32_t* inv_perm,
                       void* x_sorted, float* x_sorted_scale, void* ws, size_t ws_bytes,
                       void* stream);

/* Index check before moe_permute, for callers that build topk_idx themselves
 * (moe_route only writes values in [0,E)).  Counts the pairs of topk_idx [T,K] (int32,
 * device) that lie outside [0,E) into n_invalid (one int32 in device memory, owned by
 * the caller, overwritten; 0 means every pair meets moe_permute's precondition).  Only
 * enqueues work on `stream`; read the count once the stream has reached it.  With a
 * nonzero count the caller should not run moe_permute and the calls after it: the
 * permute skips such pairs and the calls that read the shared rows at T*K + t are then
 * not defined. */
moe_status moe_count_invalid_ids(const moe_problem* p, const int32_t* topk_idx,
                                 int32_t* n_invalid, void* stream);

/* moe_permute without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, outputs and results as moe_permute, bit for bit; the
 * scratch lives in a fixed 8 MiB device array inside the library, one per GPU, held
 * until the process ends.  The call allocates nothing.
 * Limit (checked, else MOE_ERR_WORKSPACE): T*K + 2*ceil(T/256)*E <= 2,097,088.
 * Calls that overlap in time on one GPU (different streams, host threads) share that
 * array and race: serialise them.  Nothing in the array needs clearing between calls. */
moe_status moe_permute_noalloc(const moe_problem* p, const void* x, const int32_t* topk_idx,
                               int32_t* offsets, int32_t* sorted_token, int32_t* inv_perm,
                               void* x_sorted, float* x_sorted_scale, void* stream);

/* Expert FFNs (SwiGLU) of every group as one grouped GEMM pair:
 *   h = silu(x W13[g][0:I]^T) * (x W13[g][I:2I]^T),  Y = h W2[g]^T,
 * fp32 accumulation (FP8: per-128-deep block partial sums scaled by the two block
 * scales and accumulated in fp32 -- mpbf.cn section 3.1, tile-wise scaling and
 * higher-precision accumulation; joto.ai item 3, FP8 inputs and weights, FP32
 * accumulation).  h is stored at the activation precision (FP8: quantised per
 * (row, 128 columns) like x); Y is rounded to act_dtype.
 *   x_sorted, x_sorted_scale, offsets   from moe_permute
 *   w13  [E+S, 2I, H]  expert_dtype (rows 0..I-1 gate, I..2I-1 up; shared expert last)
 *   w13_scale [E+S, 2I/128, H/128] fp32 (FP8 only, else NULL)
 *   w2   [E+S, H, I]   expert_dtype
 *   w2_scale  [E+S, H/128, I/128]  fp32 (FP8 only, else NULL)
 *   y_sorted  [R,H] act_dtype out
 *   ws   >= moe_workspace_bytes(p, MOE_CALL_EXPERT_FFN) bytes (holds h: [R,I] of the
 *        activation dtype, or [R,I] E4M3 codes followed by [R,I/128] fp32 scales for
 *        FP8, the scales starting at the next 256-byte boundary)
 * offsets must be the values moe_permute wrote (they are read on the device).
 * Equivalent to moe_expert_ffn_up followed by moe_expert_ffn_down on ws. */
moe_status moe_expert_ffn(const moe_problem* p, const void* x_sorted,
                          const float* x_sorted_scale, const int32_t* offsets,
                          const void* w13, const float* w13_scale, const void* w2,
                          const float* w2_scale, void* y_sorted, void* ws, size_t ws_bytes,
                          void* stream);

/* First half of moe_expert_ffn (same passages): the gate/up grouped GEMM with SwiGLU.
 *   h       [R,I] out: act_dtype, or E4M3 codes for FP8 (scale = amax/448 per
 *           (row, 128 columns), code = RNE-saturating E4M3 of h/scale)
 *   h_scale [R,I/128] fp32 out (FP8 only, else NULL)
 * Other arguments as moe_expert_ffn.  Rows of h outside every group are not written. */
moe_status moe_expert_ffn_up(const moe_problem* p, const void* x_sorted,
                             const float* x_sorted_scale, const int32_t* offsets,
                             const void* w13, const float* w13_scale, void* h, float* h_scale,
                             void* stream);

/* moe_expert_ffn_up reading its rows from the unpermuted input: row r of the permuted
 * order is row sorted_token[r] of x (the row copy of the dispatch step, fused into the
 * GEMM's loads).  h and h_scale are identical to moe_expert_ffn_up on the x_sorted that
 * moe_permute would have written.
 *   x        [T,H] act_dtype, or E4M3 codes from moe_quantize_act_fp8 (FP8)
 *   x_scale  [T,H/128] fp32 from moe_quantize_act_fp8 (FP8 only, else NULL)
 *   sorted_token, offsets  from moe_permute
 * Extra limit (checked): T*H*(bytes per x element) < 2^31 - 16. */
moe_status moe_expert_ffn_up_gather(const moe_problem* p, const void* x, const float* x_scale,
                                    const int32_t* sorted_token, const int32_t* offsets,
                                    const void* w13, const float* w13_scale, void* h,
                                    float* h_scale, void* stream);

/* Per-token FP8 quantisation of x for moe_expert_ffn_up_gather (the quantisation
 * moe_permute applies to each row of x_sorted, done once per token; mpbf.cn section
 * 3.1, activations scaled per 1x128 tile): scale = amax/448 per (token, 128 columns),
 * 1 for an all-zero tile; code = RNE-saturating E4M3 of x/scale.
 *   x [T,H] bf16; x_q [T,H] E4M3 codes out; x_scale [T,H/128] fp32 out.
 * Requires act_dtype BF16 and expert_dtype FP8_E4M3. */
moe_status moe_quantize_act_fp8(const moe_problem* p, const void* x, void* x_q, float* x_scale,
                                void* stream);

/* Second half of moe_expert_ffn: Y = h W2[g]^T per group, rounded to act_dtype.
 *   h, h_scale from moe_expert_ffn_up; w2, w2_scale, offsets as moe_expert_ffn;
 *   y_sorted [R,H] act_dtype out. */
moe_status moe_expert_ffn_down(const moe_problem* p, const void* h, const float* h_scale,
                               const int32_t* offsets, const void* w2, const float* w2_scale,
                               void* y_sorted, void* stream);

/* The expert FFN of moe_expert_ffn_up(_gather, _save) and moe_expert_ffn_down (same
 * passages, same arithmetic) over expert weights in a pre-arranged layout that lets the
 * GEMMs stream each weight byte straight into the matrix-core operands.  act dtype BF16
 * with expert dtype BF16 or FP8_E4M3 (else MOE_ERR_UNSUPPORTED).  BF16 results equal the
 * natural-layout calls bit for bit; FP8 results follow the same block-scaled promotion.
 *
 * moe_pack_expert_weights: w13 [E+S, 2I, H] and w2 [E+S, H, I] in the expert dtype
 * (natural layout as above; FP8: the E4M3 codes of moe_quantize_weights_fp8) ->
 * w13_packed and w2_packed, each the same number of bytes as its input.  The packed
 * layout (per group, blocks of 64 weight rows, 64-deep (BF16) or 128-deep (FP8) k steps
 * per block, 8 x 64 chunks of 16 bytes per step) is private to this library: its only
 * consumers are the two calls below.  The FP8 weight scales are not packed.  Either pair
 * may be NULL (that matrix is not packed); the call must not be in place.  Offline
 * preparation, like moe_quantize_weights_fp8. */
moe_status moe_pack_expert_weights(const moe_problem* p, const void* w13, const void* w2,
                                   void* w13_packed, void* w2_packed, void* stream);

/* Gate/up GEMM + SwiGLU over packed weights.
 *   x            sorted_token == NULL: x_sorted [R,H] (moe_permute); else x [T,H] and row r
 *                of the permuted order is x[sorted_token[r]] (limit as
 *                moe_expert_ffn_up_gather); FP8: E4M3 codes
 *   x_scale      FP8: [R,H/128] or [T,H/128] fp32 (as x), else NULL
 *   offsets      from moe_permute
 *   w13          natural layout (the shared expert's rows are multiplied by a dense
 *                kernel that reads it when T >= 2048)
 *   w13_packed   from moe_pack_expert_weights;  w13_scale  FP8 only, as moe_expert_ffn
 *   h  [R,I] out (bf16, or E4M3 codes with h_scale [R,I/128] fp32 out, as
 *   moe_expert_ffn_up);  au [R,2I] bf16 out or NULL (the pre-activations, as
 *   moe_expert_ffn_up_save; bf16 only). */
moe_status moe_expert_ffn_up_packed(const moe_problem* p, const void* x, const float* x_scale,
                                    const int32_t* sorted_token, const int32_t* offsets,
                                    const void* w13, const void* w13_packed,
                                    const float* w13_scale, void* h, float* h_scale, void* au,
                                    void* stream);

/* Down GEMM over packed weights: y_sorted [R,H] bf16 out = h W2[g]^T per group
 * (h, h_scale from moe_expert_ffn_up_packed or moe_expert_ffn_up; w2_packed from
 * moe_pack_expert_weights; w2_scale FP8 only, as moe_expert_ffn). */
moe_status moe_expert_ffn_down_packed(const moe_problem* p, const void* h, const float* h_scale,
                                      const int32_t* offsets, const void* w2_packed,
                                      const float* w2_scale, void* y_sorted, void* stream);

/* Combine (blog.resmic.cn section 核心架构二: shared output + gate-weighted routed
 * outputs):  acc = 0; for k = 0..K-1: acc = fma(gate[t,k], Y[inv_perm[t,k]], acc);
 * if S: acc = Y[T*K + t] + acc;  y[t] = acc rounded (RNE) to act_dtype.
 *   y_sorted [R,H] act_dtype, inv_perm [T,K] int32, topk_gate [T,K] fp32,
 *   y [T,H] act_dtype out.  Bit-for-bit reproducible for given inputs. */
moe_status moe_combine(const moe_problem* p, const void* y_sorted, const int32_t* inv_perm,
                       const float* topk_gate, void* y, void* stream);

/* Bias update after a step (mpbf.cn sections 2.2 and 6.2; joto.ai item 1):
 * for each expert, compare its load with the uniform share exactly in integers,
 *   counts[e]*E > T*K  ->  bias[e] -= gamma;   counts[e]*E < T*K  ->  bias[e] += gamma;
 *   equal -> unchanged   (fp32 arithmetic; the bias never takes a gradient).
 *   expert_counts [E] int32 (from moe_route), bias [E] fp32 in/out. */
moe_status moe_bias_update(const moe_problem* p, const int32_t* expert_counts, float gamma,
                           float* bias, void* stream);

/* Sequence-wise load statistic (mpbf.cn section 2.2: next to the bias rule, a
 * sequence-level balance term with a very small weight keeps any single sequence from
 * extreme imbalance; the pages give that term no formula, so this reports the loads
 * it is built from).  Sequence s holds tokens seq_offsets[s] .. seq_offsets[s+1]-1.
 *   topk_idx    [T,K] int32 from moe_route
 *   seq_offsets [n_seq+1] int32: 0 = seq_offsets[0] <= ... <= seq_offsets[n_seq] = T
 *               (empty sequences allowed)
 *   seq_counts  [n_seq,E] int32 out: tokens of sequence s routed to expert e
 *   seq_stats   [n_seq,3] int32 out: max count, min count, experts with no token
 *   seq_ratio   [n_seq]   fp32  out: max / (L*K/E) for the sequence's L tokens, as
 *               (float)(max*E) / (float)(L*K) with one IEEE division; 0 if L = 0.
 * Limits (checked): 1 <= n_seq <= 2^24, n_seq*E < 2^31.  Offsets that break the
 * ordering above, or indices outside [0,E), give unspecified counts but every write
 * stays inside the outputs.  Bit-for-bit reproducible (integer atomics). */
moe_status moe_seq_load_stats(const moe_problem* p, const int32_t* topk_idx,
                              const int32_t* seq_offsets, int32_t n_seq, int32_t* seq_counts,
                              int32_t* seq_stats, float* seq_ratio, void* stream);

/* ---------------- backward of the layer (bf16 and fp32 paths) ----------------
 * The derivative of the forward above.  The pages fix only that the routing bias
 * takes no part in back-propagation (blog.resmic.cn section 核心架构三) and that
 * gradients accumulate at high precision (joto.ai item 3, FP32 accumulation): all
 * reductions are fp32, weight gradients are stored in fp32, the bias has no gradient.
 * One backward step, after a forward whose gate/up GEMM ran as moe_expert_ffn_up_save:
 *   moe_combine_backward -> moe_router_backward -> moe_expert_ffn_backward_input
 *   -> moe_expert_ffn_backward_weight -> moe_unpermute_sum.
 * The expert backward comes in two calls, input gradient and weight gradient, as the
 * pages' pipeline schedule splits a backward block (mpbf.cn section 3.2, DualPipe):
 * the weight part has no consumer inside the layer and may run later or elsewhere.
 * FP8 expert dtype: MOE_ERR_UNSUPPORTED. */

/* moe_expert_ffn_up (or _gather) that also keeps the gate and up pre-activations for
 * the backward:  au [R, 2I] act_dtype out, au[r][n] = a = x W13[g][n],
 * au[r][I + n] = u = x W13[g][I + n] (fp32 sums rounded to act_dtype).  h as
 * moe_expert_ffn_up.  sorted_token == NULL: x is x_sorted [R,H]; else x is [T,H] and
 * row r is x[sorted_token[r]] (limit as moe_expert_ffn_up_gather). */
moe_status moe_expert_ffn_up_save(const moe_problem* p, const void* x,
                                  const int32_t* sorted_token, const int32_t* offsets,
                                  const void* w13, void* h, void* au, void* stream);

/* Combine backward (of moe_combine):
 *   dy_sorted[inv_perm[t,k]] = topk_gate[t,k] * dy[t]  (rounded to act_dtype),
 *   dy_sorted[T*K + t]       = dy[t]                   (shared expert, S = 1),
 *   dgate[t,k]               = sum_h dy[t,h] * y_sorted[inv_perm[t,k], h]  (fp32).
 *   dy [T,H] act; y_sorted [R,H] act (the forward's); inv_perm, topk_gate [T,K];
 *   dy_sorted [R,H] act out; dgate [T,K] fp32 out. */
moe_status moe_combine_backward(const moe_problem* p, const void* dy, const void* y_sorted,
                                const int32_t* inv_perm, const float* topk_gate,
                                void* dy_sorted, float* dgate, void* stream);

/* Gate and router backward (mpbf.cn section 2.2: gates are the chosen sigmoid
 * affinities renormalised; the bias only chose them):  with s = sigmoid(clamp(z,+-80))
 * of the chosen experts and S their sum,
 *   dz[t,j] = (dgate[t,j] - sum_k gate[t,k] dgate[t,k]) / S * s_j (1 - s_j)
 *             (0 where |z| > 80),
 *   dx_router[t] = sum_j dz[t,j] W_r[e_j]            [T,H] fp32 out,
 *   dw_router[e] = sum over the rows of expert e, tokens ascending, of dz x[token]
 *                                                      [E,H] fp32 out.
 *   logits [T,E] fp32 from moe_route (logits_out); offsets, sorted_token from
 *   moe_permute; dz [T,K] fp32 out. */
moe_status moe_router_backward(const moe_problem* p, const void* x, const float* w_router,
                               const float* logits, const int32_t* topk_idx,
                               const float* topk_gate, const float* dgate,
                               const int32_t* offsets, const int32_t* sorted_token, float* dz,
                               float* dx_router, float* dw_router, void* stream);

/* Expert FFN backward, input part, per group g over its rows (grouped GEMMs, fp32
 * accumulation):
 *   dh = dY W2[g];  da = dh u silu'(a), du = dh silu(a)  -> dau [R,2I] act out;
 *   dx_sorted = dau W13[g]                               -> [R,H] act out.
 *   au from moe_expert_ffn_up_save; dy_sorted [R,H] act from moe_combine_backward.
 * Extra limit (checked): R*max(H,2I)*(bytes per element) < 2^31 - 16. */
moe_status moe_expert_ffn_backward_input(const moe_problem* p, const int32_t* offsets,
                                         const void* w13, const void* w2, const void* au,
                                         const void* dy_sorted, void* dau, void* dx_sorted,
                                         void* stream);

/* Weights for the backward input part over packed weights (bf16 only): the transposes
 * W2[g]^T [I,H] and W13[g]^T [H,2I], each in the down-GEMM packed layout of
 * moe_pack_expert_weights (rows in blocks of 64, k steps of 64), so the two backward
 * GEMMs stream their weights like the forward ones.
 *   w13 [E+S,2I,H] bf16 -> w13t_packed (same size);  w2 [E+S,H,I] bf16 -> w2t_packed
 *   (same size).  Either pair may be NULL.  Outputs are owned by the caller; packing is
 *   not in place.  Errors: MOE_ERR_UNSUPPORTED unless act and expert dtypes are BF16. */
moe_status moe_pack_expert_weights_transposed(const moe_problem* p, const void* w13,
                                              const void* w2, void* w13t_packed,
                                              void* w2t_packed, void* stream);

/* Expert FFN backward, input part, over the packed transposed weights: the same results
 * as moe_expert_ffn_backward_input bit for bit (the same 16-deep products, in the same
 * order, with the same epilogue arithmetic), bf16 only.
 *   w13t_packed, w2t_packed from moe_pack_expert_weights_transposed; the other arguments
 *   as moe_expert_ffn_backward_input. */
moe_status moe_expert_ffn_backward_input_packed(const moe_problem* p, const int32_t* offsets,
                                                const void* w13t_packed,
                                                const void* w2t_packed, const void* au,
                                                const void* dy_sorted, void* dau,
                                                void* dx_sorted, void* stream);

/* Expert FFN backward, weight part, per group g over its rows (fp32 accumulation):
 *   dw2[g]  = dY^T h    [E+S,H,I]  fp32 out,
 *   dw13[g] = dau^T x   [E+S,2I,H] fp32 out   (groups without rows get zeros).
 *   x: x_sorted [R,H] (sorted_token NULL) or x [T,H] with sorted_token; h from
 *   moe_expert_ffn_up_save; dy_sorted from moe_combine_backward; dau from
 *   moe_expert_ffn_backward_input.  Same extra limit as the input part. */
moe_status moe_expert_ffn_backward_weight(const moe_problem* p, const void* x,
                                          const int32_t* sorted_token, const int32_t* offsets,
                                          const void* h, const void* dy_sorted, const void* dau,
                                          float* dw13, float* dw2, void* stream);

/* Input gradient: dx[t] = dx_router[t] + sum_k dx_sorted[inv_perm[t,k]] + dx_sorted[T*K+t]
 * (last term if S = 1), summed in fp32 in that order, rounded to act_dtype.
 * dx_router may be NULL (then omitted). */
moe_status moe_unpermute_sum(const moe_problem* p, const void* dx_sorted,
                             const int32_t* inv_perm, const float* dx_router, void* dx,
                             void* stream);

/* Offline FP8 preparation of expert weights (mpbf.cn section 4.3: block-wise scaling
 * instead of one global scale): for `batch` bf16 matrices [rows, cols] (rows and cols
 * multiples of 128) write E4M3 codes [batch, rows, cols] and fp32 scales
 * [batch, rows/128, cols/128], one per 128x128 block: scale = amax/448 (1 if amax is 0),
 * code = RNE-saturating E4M3 of w/scale. */
moe_status moe_quantize_weights_fp8(const void* w_bf16, void* w_fp8, float* scale,
                                    int64_t batch, int32_t rows, int32_t cols, void* stream);

/* Text of a status code, and the last error message of the calling thread. */
const char* moe_status_str(moe_status s);
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
