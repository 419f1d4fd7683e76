/*
 * moe.h - C ABI of a single-GPU DeepSeekMoE layer forward with auxiliary-loss-free
 * (bias-based) load balancing, for AMD Instinct MI355X (gfx950).
 *
 * One batch runs as five calls on one HIP stream:
 *   moe_route -> moe_dispatch -> moe_expert_ffn -> moe_combine -> moe_update_bias
 *
 * Conventions shared by every entry point
 *  - Every tensor argument is a DEVICE pointer owned by the caller; `cfg` and
 *    `w` are HOST pointers read during the call only.  The library never
 *    allocates or frees memory on these paths and keeps no state between calls.
 *  - Tensors are dense, row-major, contiguous.  Weights are [out, in] (K is the
 *    contiguous dimension of both GEMM operands).  Indices are int32.
 *  - bf16 tensors are raw 16-bit bfloat16 values; fp8 tensors are raw OCP E4M3FN
 *    bytes (bias 7, no infinities, largest finite 448).
 *  - Every call validates all sizes and pointers on the host BEFORE touching the
 *    device and returns a negative moe_status on error (nothing is launched).  A
 *    failed launch returns MOE_ERR_LAUNCH.  Work is asynchronous on `stream`
 *    (a hipStream_t; NULL means the default stream); device faults surface at
 *    the caller's next synchronisation.  The library never synchronises.
 *  - Calls are re-entrant; calls on one stream are ordered by that stream.
 *    Two calls that share an output or workspace buffer on different streams
 *    race.
 *
 * Results: expert indices, counts, the permutation and the bias update are
 * deterministic bit for bit (no atomics anywhere on the path).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = -2,       /* sizes inconsistent or outside the supported range */
  MOE_ERR_UNSUPPORTED = -3, /* dtype combination or option not implemented */
  MOE_ERR_WORKSPACE = -4,   /* workspace smaller than moe_workspace_bytes() */
  MOE_ERR_LAUNCH = -5,      /* a kernel launch failed (hipGetLastError) */
  MOE_ERR_SCRATCH = -6      /* sizes exceed the fixed scratch of a no-allocation entry point */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/*
 * Layer configuration.
 *  T tokens, H hidden, E routed experts in G contiguous groups of E/G experts,
 *  at most M groups per token, k routed experts per token, S shared experts,
 *  I intermediate size of each expert.
 *  group_topr: a group's score is the fp32 sum of its group_topr largest biased
 *              scores, added from the largest down (1 <= group_topr <= E/G, <= 8).
 *  route_scale: gates are route_scale * s_j / sum(s) over the selected experts.
 *  act / wgt (moe_dtype): (F32, F32) | (BF16, BF16) | (BF16, FP8_E4M3).  The
 *              router always runs in `act` precision; FP8_E4M3 applies to the
 *              expert GEMMs only.
 *  bias_eq_mode: 0 - an expert whose load equals T*k/E counts as underloaded
 *              (+gamma), so every bias moves each step; 1 - it is left unchanged.
 * Supported ranges (every call checks them first and returns MOE_ERR_SHAPE
 *  outside them; MOE_ERR_UNSUPPORTED for another act/wgt pair or bias_eq_mode):
 *  1 <= G <= 64, E % G == 0, E <= 512, 1 <= M <= G, 1 <= k <= min(32, M*E/G),
 *  1 <= group_topr <= min(8, E/G), route_scale not NaN, T >= 0, S >= 0,
 *  T*k < 2^31, T*k*H < 2^40, H, I and S*I at most 2^20, one routed expert's
 *  gate/up weights (all shared experts' together) under 2^31 bytes in bf16,
 *  E*H*2 < 2^31, and (T*(k+S)/32 + E + 2) * (max(H, S*I)/64 + 2) < 2^30 (the
 *  grouped GEMMs count their tiles in 32 bits).  F32: H % 4 == 0, I % 4 == 0;
 *  BF16 experts: H % 64 == 0, I % 128 == 0; FP8 experts: H % 128 == 0,
 *  I % 128 == 0, H <= 8192 and max(S, 1)*I <= 8192 (64 scale blocks of K).
 */
typedef struct {
  int32_t T, H, E, G, M, k, S, I;
  int32_t group_topr;
  float route_scale;
  int32_t act;
  int32_t wgt;
  int32_t bias_eq_mode;
} moe_cfg;

/* moe_route flags */
#define MOE_SCORES_IN 1u /* `scores` is an input: route on these fp32 affinities, skip the router GEMM */

/*
 * moe_route - affinity and biased, group-limited top-k with gates.
 *
 * Follows: each expert's bias enters only the ranking used for top-K selection
 * while the gating value comes from the original affinity (DeepSeek-V3
 * Technical Report reading notes, Method §1 "Auxiliary-loss-free 负载均衡";
 * DeepSeek-V3 Technical Report：中英对照解读, §3; DeepSeek V3 product page,
 * "公式解密" box: ranking score = affinity + bias); a token goes to at most M
 * nodes (reading notes, Method §1), here M of G expert groups.
 *
 *  x            [T, H] act dtype                 (unused with MOE_SCORES_IN)
 *  w_router     [E, H] act dtype                 (unused with MOE_SCORES_IN)
 *  logit_offset [E] fp32 added to the logits before the sigmoid, or NULL
 *  bias         [E] fp32 routing bias b
 *  scores       [T, E] fp32: output s = sigmoid(x w_router^T + o), or the input
 *               affinities with MOE_SCORES_IN; may be NULL without MOE_SCORES_IN
 *               (the affinities are then not written: a forward pass that needs
 *               no router gradient)
 *  topk_idx     [T, k] int32 out: selected experts, ordered by s + b descending,
 *               ties to the lower expert index (-0.0 ranks as +0.0)
 *  topk_w       [T, k] fp32 out: route_scale * s_j / sum_j s_j
 *  ws, ws_bytes workspace of at least moe_workspace_bytes(cfg, MOE_WS_ROUTE)
 *               bytes, required when scores is NULL (it stages the affinities
 *               where no kernel keeps them on chip); ignored otherwise (may be NULL)
 * Groups are chosen first (the M largest group scores, ties to the lower group),
 * then the k largest s + b among the experts of the chosen groups.
 * NaN scores give unspecified indices.
 * For mid-size bf16 batches (too large for the split-K router, too small for
 * router tiles of 128 tokens to fill the chip; E = 256: 2049 <= T < 16384) with
 * E = 16, 32, 64, 128 or 256 in groups of a power-of-two number of 16-lane
 * slices, k <= 16 and group_topr <= 4, one kernel runs the router GEMM and the
 * whole selection (the affinities stay in LDS, and are also written when scores
 * is given); it selects with the same code as the MOE_SCORES_IN path, so
 * routing its own affinities again with MOE_SCORES_IN gives the same indices
 * and gates.
 * The router GEMM sums in a fixed order per batch size (repeated calls give
 * identical bits); small and large batches use different kernels, so the last
 * bits of a token's affinities can depend on T.
 * MOE_ERR_WORKSPACE: scores is NULL and ws is NULL or too small.
 */
moe_status moe_route(const moe_cfg* cfg, const void* x, const void* w_router,
                     const float* logit_offset, const float* bias, float* scores,
                     uint32_t flags, int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * moe_dispatch - per-expert loads and the expert-sorted permutation of the
 * (token, slot) pairs, plus the permuted activations.
 *
 * Follows: tokens are dispatched to their experts and combined back
 * (DeepSeek-V3 Technical Report：中英对照解读, §2.2); each expert's load is
 * counted over the whole batch (qwbw.cn essay on the DeepSeek-V3 report,
 * load-balancing section).
 *
 *  topk_idx  [T, k] int32 in, values in [0, E) (a pair whose value lies outside is
 *            not counted, and perm, inv and x_perm are then undefined)
 *  x         [T, H] act dtype in
 *  counts    [E] int32 out: pairs routed to each expert
 *  offsets   [E+1] int32 out: exclusive prefix sum of counts
 *  perm      [T*k] int32 out: flat pair ids f = t*k + j, stably sorted by expert
 *  inv       [T, k] int32 out: row of pair (t, j) in the permuted order
 *  x_perm    [T*k, H] out: row p = x[perm[p] / k]; act dtype, or E4M3 bytes when
 *            wgt == FP8_E4M3 (quantised per 1x128 tile: sc = amax/448, q = e4m3(v/sc)).
 *            NULL: only counts, offsets, perm and inv are written (x and
 *            x_perm_scale may then be NULL too), for moe_expert_ffn_gather.
 *  x_perm_scale [T*k, H/128] fp32 out (FP8 only, else NULL)
 *  ws, ws_bytes  workspace of at least moe_workspace_bytes(cfg, MOE_WS_DISPATCH)
 */
moe_status moe_dispatch(const moe_cfg* cfg, const int32_t* topk_idx, const void* x,
                        int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                        void* x_perm, float* x_perm_scale, void* ws, size_t ws_bytes,
                        void* stream);

/*
 * moe_dispatch_noalloc - moe_dispatch without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments, results
 * and errors as moe_dispatch, bit for bit.
 *
 * Its per-segment counts live in a fixed 4 MiB array of device memory owned by
 * the library: one copy per GPU, held until the process ends; the first call
 * on a device looks up that copy's address (hipGetSymbolAddress).  Nothing is
 * allocated, by the library or anything it calls.  Limit: ceil(T*k / 1024) * E
 * * 4 bytes <= 4 MiB (E = 256: T*k up to 4M pairs), else MOE_ERR_SCRATCH
 * (checked before any device call).  Every call on a GPU shares that GPU's
 * array and nothing in it needs to start at zero; calls that overlap on one
 * GPU (different streams, or threads without ordering) race and give
 * undefined results.  MOE_ERR_LAUNCH also when the array's address cannot be
 * obtained on the current device.
 */
moe_status moe_dispatch_noalloc(const moe_cfg* cfg, const int32_t* topk_idx, const void* x,
                                int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                                void* x_perm, float* x_perm_scale, void* stream);

/* Expert weights.  Scales are only read when wgt == FP8_E4M3 (then the weight
 * tensors hold E4M3 bytes, one fp32 scale per 128 x 128 block). */
typedef struct {
  const void* w_gate_up;         /* [E, 2I, H]: gate rows [0, I), up rows [I, 2I) */
  const void* w_down;            /* [E, H, I] */
  const float* w_gate_up_scale;  /* [E, 2I/128, H/128] */
  const float* w_down_scale;     /* [E, H/128, I/128] */
  const void* ws_gate_up;        /* [S, 2I, H] shared experts */
  const void* ws_down;           /* [S, H, I] */
  const float* ws_gate_up_scale; /* [S, 2I/128, H/128] */
  const float* ws_down_scale;    /* [S, H/128, I/128] */
} moe_expert_weights;

/* moe_expert_ffn phases: the two GEMM launches may be issued by separate calls
 * (GATE_UP then DOWN, same workspace), e.g. to time them apart. */
#define MOE_FFN_ALL 0
#define MOE_FFN_GATE_UP 1
#define MOE_FFN_DOWN 2

/*
 * moe_expert_ffn - routed experts on their segments of x_perm and the shared
 * experts on every token, each a SwiGLU FFN: FFN(v) = W_d (silu(W_g v) * W_u v).
 *
 * Follows: shared experts that every token passes through plus routed experts
 * picked by top-k (DeepSeek-V3 Technical Report：中英对照解读, §2); FP8 with
 * 1x128 activation tiles and 128x128 weight blocks, E4M3 everywhere and
 * full-precision accumulation (qwbw.cn essay, FP8 part of the infrastructure
 * section; same notes, §6).
 *
 *  x_perm, x_perm_scale, offsets  as written by moe_dispatch
 *  w            host pointer to the weight table
 *  x            [T, H] act dtype (input of the shared experts)
 *  y_perm       [T*k, H] out, act dtype: routed expert outputs, ungated
 *  y_shared     [T, H] out, act dtype: sum of the shared experts' outputs (S > 0)
 *  ws, ws_bytes at least moe_workspace_bytes(cfg, MOE_WS_FFN); holds the
 *               SwiGLU intermediates between the two phases
 *  phase        MOE_FFN_ALL | MOE_FFN_GATE_UP | MOE_FFN_DOWN
 * Intermediates are rounded to the activation dtype (bf16) or, for FP8, to E4M3
 * per 1x128 tile of each row; accumulation is fp32.
 */
moe_status moe_expert_ffn(const moe_cfg* cfg, const void* x_perm, const float* x_perm_scale,
                          const int32_t* offsets, const moe_expert_weights* w, const void* x,
                          void* y_perm, void* y_shared, void* ws, size_t ws_bytes, int phase,
                          void* stream);

/*
 * moe_expert_ffn_gather - moe_expert_ffn with dispatch's row copy folded into
 * the routed gate/up GEMM: its operand row p is read straight from
 * x[perm[p] / k] (same arithmetic, same order: y_perm and y_shared equal
 * moe_expert_ffn's bit for bit).  For FP8 the kernel quantises x once per
 * 1x128 tile into the workspace and gathers codes and scales from there (the
 * same codes moe_dispatch would write into x_perm).
 *
 * Follows: the per-expert token rows of dispatch (DeepSeek-V3 Technical
 * Report：中英对照解读, §2.2) read in place instead of copied.
 *
 *  x         [T, H] act dtype in (bf16 for FP8 weights)
 *  perm, offsets  as written by moe_dispatch (which may then skip x_perm)
 *  w, y_perm, y_shared, ws, ws_bytes, phase  as for moe_expert_ffn
 * MOE_ERR_UNSUPPORTED when (T+1) * H * (bytes per element) exceeds 2^31 - 1
 * (the gathered rows are addressed by 32-bit byte offsets; bf16/FP8 only).
 */
moe_status moe_expert_ffn_gather(const moe_cfg* cfg, const void* x, const int32_t* perm,
                                 const int32_t* offsets, const moe_expert_weights* w,
                                 void* y_perm, void* y_shared, void* ws, size_t ws_bytes,
                                 int phase, void* stream);

/* The SwiGLU inputs of the experts (bf16, caller-owned): g = X W_g^T and
 * u = X W_u^T, [T*k, I] in the expert-sorted row order of x_perm, and the
 * shared experts' gs, us [T, S*I] (S > 0; expert s in columns [s*I, (s+1)*I)). */
typedef struct {
  void* g;
  void* u;
  void* gs;
  void* us;
} moe_ffn_saved;

/*
 * moe_expert_ffn_save - moe_expert_ffn (x_perm != NULL) or moe_expert_ffn_gather
 * (x_perm == NULL: rows gathered from x through perm) that also stores the
 * gate and up outputs g, u of the gate/up GEMM in `saved`, for a training step
 * whose backward pass then starts from them (moe_expert_ffn_backward_saved)
 * instead of recomputing the gate/up GEMM.  Same arithmetic and order: y_perm
 * and y_shared equal the other entry points' bit for bit, and g, u equal the
 * backward pass's recomputation bit for bit.  bf16 only (MOE_ERR_UNSUPPORTED
 * otherwise).  The phase MOE_FFN_DOWN leaves `saved` untouched.
 *
 * Follows: the experts are SwiGLU FFNs (DeepSeek-V3 Technical Report：中英对照
 * 解读, §2); which activations a training step keeps and which it recomputes
 * is the memory/compute trade-off the pages make for RMSNorm and the MLA
 * up-projection (qwbw.cn essay, infrastructure section, memory optimisations): keeping g and u costs
 * 2 * (T*k + T*S) * I * 2 bytes and saves the backward pass one gate/up GEMM.
 *
 *  x_perm, perm, offsets, w, x, y_perm, y_shared, ws, ws_bytes, phase  as for
 *  moe_expert_ffn / moe_expert_ffn_gather; saved: every member non-NULL (gs, us
 *  when S > 0).
 */
moe_status moe_expert_ffn_save(const moe_cfg* cfg, const void* x_perm, const int32_t* perm,
                               const int32_t* offsets, const moe_expert_weights* w, const void* x,
                               void* y_perm, void* y_shared, const moe_ffn_saved* saved, void* ws,
                               size_t ws_bytes, int phase, void* stream);

/*
 * moe_combine - y[t] = y_shared[t] + sum_j topk_w[t, j] * y_perm[inv[t, j]]
 * accumulated in fp32 over j ascending; y in the activation dtype.
 * Follows: combine of the expert outputs weighted by gating values taken from
 * the raw affinities (DeepSeek-V3 Technical Report：中英对照解读, §2.2 and §3).
 * y_shared may be NULL when S == 0.  No residual is added.
 */
moe_status moe_combine(const moe_cfg* cfg, const void* y_perm, const void* y_shared,
                       const int32_t* inv, const float* topk_w, void* y, void* stream);

/*
 * moe_update_bias - the per-step balancing rule: for each expert,
 * bias -= gamma if counts*E > T*k (overloaded), bias += gamma if underloaded
 * (counts*E < T*k, or == with bias_eq_mode 0), in fp32 with round-to-nearest-even.
 * Follows: reading notes, Method §1 "Auxiliary-loss-free 负载均衡"; qwbw.cn
 * essay, load-balancing section (loads counted over the whole batch after each
 * step).  bias is updated in place; counts as written by moe_dispatch.
 */
moe_status moe_update_bias(const moe_cfg* cfg, const int32_t* counts, float* bias, float gamma,
                           void* stream);

/*
 * moe_quantize_fp8 - offline weight preparation for the FP8 expert GEMMs:
 * a bf16 matrix [n_mat, rows, cols] becomes E4M3 bytes [n_mat, rows, cols]
 * and one fp32 scale per 128 x 128 block [n_mat, rows/128, cols/128]
 * (sc = amax/448, or 1 for an all-zero block; q = e4m3(v/sc), nearest-even,
 * saturating).  Follows the 128x128 weight blocks of the pages' FP8 recipe
 * (qwbw.cn essay, FP8 part of the infrastructure section).  With block_rows = 1
 * it quantises per 1 x 128 tile instead (scales [n_mat, rows, cols/128]).
 * rows must be a multiple of block_rows (1 or 128), cols of 128.
 */
moe_status moe_quantize_fp8(const void* src_bf16, int32_t n_mat, int32_t rows, int32_t cols,
                            int32_t block_rows, uint8_t* dst, float* scales, void* stream);

/* ------------------------------------------------------------------ backward
 * The gradient of one layer pass (the training step the bias rule lives in),
 * for act = wgt = BF16 (other dtypes: MOE_ERR_UNSUPPORTED).  With the expert
 * choice of the forward pass fixed, the loss sum(dy * y) + L_bal is
 * differentiated exactly: the expert choice and the bias carry no gradient
 * (the bias only ranks experts; the gates come from the raw affinities:
 * reading notes on the DeepSeek-V3 report, Method §1).  Order of the calls:
 *   moe_combine_backward -> moe_expert_ffn_backward -> moe_route_backward ->
 *   moe_dispatch_backward
 * Gradients of activations are bf16 with fp32 accumulation inside every
 * kernel; weight gradients are fp32 (the pages keep gradients in high
 * precision: qwbw.cn essay, FP8 part of the infrastructure section).
 */

/*
 * moe_combine_backward - gradients of y[t] = y_shared[t] + sum_j w[t,j] y_perm[inv[t,j]]:
 *   d_topk_w[t,j]       = sum_h dy[t,h] * y_perm[inv[t,j],h]   (fp32)
 *   dy_perm[inv[t,j],:] = topk_w[t,j] * dy[t,:]                 (bf16)
 * (the shared experts' output gradient is dy itself).
 *  dy [T, H], y_perm [T*k, H] (as written by moe_expert_ffn), inv, topk_w [T, k];
 *  dy_perm [T*k, H] out; d_topk_w [T, k] fp32 out.
 */
moe_status moe_combine_backward(const moe_cfg* cfg, const void* dy, const void* y_perm, const int32_t* inv,
                                const float* topk_w, void* dy_perm, float* d_topk_w, void* stream);

/* Weight gradients (fp32, the weights' shapes). */
typedef struct {
  float* w_gate_up;   /* [E, 2I, H] */
  float* w_down;      /* [E, H, I] */
  float* ws_gate_up;  /* [S, 2I, H] (S > 0) */
  float* ws_down;     /* [S, H, I] (S > 0) */
} moe_expert_grads;

/*
 * moe_expert_ffn_backward - gradients of the routed experts on their segments
 * and of the shared experts on every token.  Recomputes the gate and up
 * outputs g, u (the forward pass keeps only h), then per expert
 *   dh = dY W_d;  dg = dh * u * silu'(g);  du = dh * silu(g);  h = silu(g) * u
 *   dX = [dg du] W_gu;  dW_gu = [dg du]^T X;  dW_d = dY^T h
 * with dY = dy_perm (routed rows) or dy (shared), X = x_perm or x
 * (SwiGLU experts: DeepSeek-V3 Technical Report：中英对照解读, §2).
 *  x_perm [T*k, H] (moe_dispatch's permuted rows), x [T, H], offsets as written
 *  by moe_dispatch; w the forward weights; dy_perm [T*k, H] from
 *  moe_combine_backward; dy [T, H];
 *  dx_perm [T*k, H] out (routed rows' input gradient, permuted order);
 *  dx_shared [T, H] out (S > 0); grads out (every member non-NULL; the shared
 *  ones when S > 0); ws of at least moe_workspace_bytes(cfg, MOE_WS_FFN_BWD).
 * MOE_ERR_UNSUPPORTED when T * max(H, 2 * max(S, 1) * I) * 2 bytes exceeds
 * 2^31 - 1 (operand rows are addressed by 32-bit offsets within a segment).
 */
moe_status moe_expert_ffn_backward(const moe_cfg* cfg, const void* x_perm, const void* x,
                                   const int32_t* offsets, const moe_expert_weights* w, const void* dy_perm,
                                   const void* dy, void* dx_perm, void* dx_shared, const moe_expert_grads* grads,
                                   void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn_backward_saved - moe_expert_ffn_backward starting from the
 * gate and up outputs kept by moe_expert_ffn_save (`saved`, every member
 * non-NULL; gs, us when S > 0) instead of recomputing them: the same outputs,
 * bit for bit, without the gate/up GEMM.  Arguments otherwise as for
 * moe_expert_ffn_backward (x_perm is still read, by dW_gu = [dg du]^T X).
 */
moe_status moe_expert_ffn_backward_saved(const moe_cfg* cfg, const void* x_perm, const void* x,
                                         const int32_t* offsets, const moe_expert_weights* w,
                                         const moe_ffn_saved* saved, const void* dy_perm, const void* dy,
                                         void* dx_perm, void* dx_shared, const moe_expert_grads* grads, void* ws,
                                         size_t ws_bytes, void* stream);

/*
 * moe_route_backward - gradients through the gates and the router, plus the
 * sequence-wise balance loss.
 *   gates   w_j = scale * s_j / sum_j' s_j' over the selected experts:
 *           ds_j = (scale / S) (dw_j - sum_j' dw_j' s_j' / S),  S = sum_j s_j
 *   balance (reading; the pages keep a sequence-wise balance loss with a very
 *           small weight alpha but print no formula: reading notes, Method §1):
 *           sequences of seq_len consecutive tokens; per sequence
 *           f_e = E / (k L) * (selections of e), P_e = mean_t s_te / sum_e' s_te',
 *           L_bal = alpha * mean over sequences of sum_e f_e P_e
 *   router  dlogit = ds * s (1 - s);  dx_router = dlogit W_r;  dw_router = dlogit^T x
 *  x [T, H], w_router [E, H] bf16; scores [T, E] fp32 affinities (moe_route's
 *  output); topk_idx [T, k]; d_topk_w [T, k] from moe_combine_backward;
 *  alpha >= 0 (0: no balance loss); seq_len 0 (= T) or a divisor of T;
 *  dx_router [T, H] fp32 out (may be NULL); dw_router [E, H] fp32 out;
 *  loss: one fp32 out (L_bal); ws of at least moe_workspace_bytes(cfg, MOE_WS_ROUTE_BWD).
 */
moe_status moe_route_backward(const moe_cfg* cfg, const void* x, const void* w_router, const float* scores,
                              const int32_t* topk_idx, const float* d_topk_w, float alpha, int32_t seq_len,
                              float* dx_router, float* dw_router, float* loss, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * moe_dispatch_backward - the input gradient of the layer:
 *   dx[t] = sum_j dx_perm[inv[t,j]] + dx_shared[t] + dx_router[t]
 * accumulated in fp32 (slots in order, then the shared and router terms), dx
 * bf16.  dx_shared may be NULL when S == 0, dx_router may be NULL.
 */
moe_status moe_dispatch_backward(const moe_cfg* cfg, const void* dx_perm, const void* dx_shared,
                                 const float* dx_router, const int32_t* inv, void* dx, void* stream);

/* Workspace kinds for moe_workspace_bytes */
#define MOE_WS_ROUTE 5
#define MOE_WS_DISPATCH 1
#define MOE_WS_FFN 2
#define MOE_WS_FFN_BWD 3
#define MOE_WS_ROUTE_BWD 4

/* Bytes of workspace a call needs for this configuration (0 on an invalid cfg). */
size_t moe_workspace_bytes(const moe_cfg* cfg, int which);

/*
 * moe_ffn_workspace_part - where moe_expert_ffn keeps the SwiGLU intermediate h
 * inside its workspace, so that a caller can read it after MOE_FFN_GATE_UP (or
 * supply it before MOE_FFN_DOWN).  Parts:
 *   MOE_WSP_H               h of the routed rows [T*k, I], act dtype or E4M3
 *   MOE_WSP_H_SCALE         their 1x128 tile scales [T*k, I/128] fp32 (FP8 only)
 *   MOE_WSP_H_SHARED        h of the shared experts [T, S*I]
 *   MOE_WSP_H_SHARED_SCALE  their scales [T, S*I/128] fp32 (FP8 only)
 * Writes the byte offset from the start of the workspace and the byte size
 * (0 for a part this configuration does not hold).  Host only; no device call.
 */
#define MOE_WSP_H 0
#define MOE_WSP_H_SCALE 1
#define MOE_WSP_H_SHARED 2
#define MOE_WSP_H_SHARED_SCALE 3
moe_status moe_ffn_workspace_part(const moe_cfg* cfg, int part, size_t* offset, size_t* bytes);

/* Static description of a status code. */
const char* moe_status_string(moe_status s);

/* MOE_ABI_VERSION of the loaded library. */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
