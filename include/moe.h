/*
 * moe.h -- C ABI of libmoe_mi355x.so: forward pass of a data-sparse
 * token-choice Mixture-of-Experts layer with zero-compute (null) experts, for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (paper review "Improving MoE Compute Efficiency by Composing Weight
 * and Data Sparsity", section 3 "Technical architecture"):
 *   y = E_shared(x) + sum over the chosen real experts i of g_i(x) E_i(x)
 * The router scores N real experts plus one null expert whose output is zero;
 * the null logit is copied M times into the pool before top-K, so a real expert
 * is used only when its logit is strictly larger than the null logit, and at
 * most K are used. Weights are renormalised over the chosen real experts only.
 * Null slots are sorted past the end of the expert-ordered slot list and cut
 * off before the grouped GEMM ("implementation" paragraph), so they cost no
 * compute. The layer also reports the load-balance statistics f_i, P_i, L_bal
 * and the router z-loss over the N+M pool ("load-balance loss", "Z-loss").
 *
 * Conventions shared by every entry point
 *   - Every tensor argument is a DEVICE pointer to a dense row-major buffer,
 *     16-byte aligned. Structs (moe_dims, moe_layer_params, moe_aux_out) live
 *     in host memory and are read during the call only.
 *   - Element type of activations, expert weights and outputs: dims->dtype
 *     (MOE_BF16 = bf16 bit patterns, MOE_F32 = float). The router weight, logits
 *     and routing weights are always float32. The SwiGLU intermediate h is IEEE
 *     half in a bf16 layer (float in a float32 one): every bf16 activation and
 *     weight of magnitude in [2^-17, 65504] converts to half exactly, and h's 11
 *     significant bits keep the error its storage adds to the output well below
 *     bf16's; h or down-projection weights of magnitude above 65504 are outside
 *     the supported range (h overflows to infinity, such a weight is clamped).
 *   - Weight layout follows the linear-layer convention [out, in] with the
 *     reduction dimension contiguous: w_gate, w_up [N][d_ff][d_model];
 *     w_down [N][d_model][d_ff]; the router [N+1][d_model], row N = null.
 *   - Ownership: the caller allocates and frees all memory. The library never
 *     allocates, frees or synchronises (moe_validate_inputs, a checking call,
 *     synchronises); it keeps no state between calls
 *     except a per-device cache of the compute-unit count. Calls on distinct
 *     buffers may run concurrently.
 *   - Execution: every kernel is enqueued on `stream` (a hipStream_t; NULL is
 *     the default stream). MOE_OK means validated and enqueued. A launch
 *     failure returns MOE_ERR_HIP. Nothing is launched when validation fails.
 *     A HIP error already pending on the calling thread when an entry point is
 *     called (hipPeekAtLastError, left by earlier work) is not cleared: the call
 *     returns MOE_ERR_HIP before launching anything and the error stays for its
 *     owner to read.
 *   - Validation: N >= 1, M >= 0, 1 <= K <= N + M, K <= N when M = 0,
 *     N <= MOE_MAX_EXPERTS, K <= MOE_MAX_TOPK, N + M <= MOE_MAX_POOL,
 *     0 <= T and T * K < 2^31, d_model and d_ff multiples of 8. T = 0 is a no-op.
 *   - Pool ids: 0..N-1 are real experts, N..N+M-1 are the null copies.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_MAX_EXPERTS 255
#define MOE_MAX_TOPK 32
#define MOE_MAX_POOL 4096

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,         /* bad dimension or NULL required pointer */
  MOE_ERR_ALIGN = 2,       /* a device pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  MOE_ERR_UNSUPPORTED = 4, /* valid but outside this library's limits */
  MOE_ERR_HIP = 5,         /* a HIP launch or runtime call failed */
  MOE_ERR_NONFINITE = 6    /* moe_validate_inputs found a NaN or an infinity */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* What a null slot outputs (paper review section 3 compares null and copy
 * experts; the MoE++ page lists zero, copy and constant zero-compute experts).
 * MOE_NULL_ZERO: 0, and the weights are renormalised over the chosen reals.
 * MOE_NULL_COPY: the token x. MOE_NULL_CONSTANT: a vector v [d_model].
 * For copy and constant the weights are a softmax over all K chosen pool
 * entries, null slots taking the effective null logit. */
typedef enum { MOE_NULL_ZERO = 0, MOE_NULL_COPY = 1, MOE_NULL_CONSTANT = 2 } moe_null_kind;

typedef struct {
  int64_t T;           /* tokens */
  int32_t d_model;
  int32_t n_experts;   /* N real experts */
  int32_t n_null;      /* M copies of the null logit in the pool */
  int32_t top_k;       /* K slots per token */
  int32_t d_ff;        /* routed expert hidden size */
  int32_t d_ff_shared; /* shared expert hidden size, 0 = no shared expert */
  int32_t dtype;       /* moe_dtype */
  int32_t null_kind;   /* moe_null_kind */
} moe_dims;

/* Which workspace size moe_workspace_bytes() returns. */
enum { MOE_WS_LAYER = 0, MOE_WS_ROUTE = 1, MOE_WS_PERMUTE = 2, MOE_WS_AUX = 3, MOE_WS_BACKWARD = 4 };

typedef void* moe_stream; /* hipStream_t */

/*
 * moe_route -- router GEMM + null-threshold top-K + renormalisation.
 * Paper review section 3, "Null Expert mechanism" and "threshold
 * interpretation"; quant67 MoE primer section 3 (router softmax, top-k,
 * renormalise among the chosen).
 *   logits s = x W^T (float32; column N gets + null_bias + null_bias_tok[t]).
 *   c = #{j < N : s_j > s_N};  r = min(K, max(c, K - M))   (r = K when M = 0)
 *   topk_idx[t, 0..r-1] = the r largest real logits, by (value desc, index asc)
 *   topk_idx[t, r..K-1] = null copies N, N+1, ... (lowest copy ids first)
 *   topk_w = softmax over the chosen real logits (computed in float64 from the
 *            float32 logits, rounded once); 0 on null slots. With null_kind
 *            MOE_NULL_COPY or MOE_NULL_CONSTANT: softmax over all K chosen
 *            entries, null slots at the effective null logit.
 *   n_real[t] = r.
 * x: [T][d_model] dtype; w_router: [N+1][d_model] float32.
 * logits_in: optional [T][N+1] float32 whose column N is already the effective
 *   null logit; when given, x, w_router and the biases are ignored (may be NULL)
 *   and no GEMM runs (routing from identical logits is bit-exact).
 * logits_out: optional [T][N+1] float32 output (column N effective).
 * null_bias_tok: optional [T] float32 per-token null bias.
 * topk_idx [T][K] int32, topk_w [T][K] float32 required; n_real [T] optional.
 * ws: MOE_WS_ROUTE bytes (float32 partial logits, up to 4 planes of [T][N+1],
 *   16 when the batch is one 64-token tile, written when the d_model sum is split
 *   over workgroups: few 64-token tiles or N > 64; at least 256 bytes); may be
 *   NULL when logits_in is given or dtype is MOE_F32. Calls that share a
 *   workspace must not overlap.
 */
moe_status moe_route(const moe_dims* dims, const void* x, const float* w_router,
                     float null_bias, const float* null_bias_tok, const float* logits_in,
                     float* logits_out, int32_t* topk_idx, float* topk_w, int32_t* n_real,
                     void* ws, size_t ws_bytes, moe_stream stream);

/*
 * moe_permute -- counting-sort dispatch of the token slots into expert order.
 * Paper review section 3 "implementation": an argsort sends the null indices
 * (>= N) to the end and the sorted list is truncated before the grouped GEMM.
 * Equivalent to a stable argsort of the flat slot ids f = t*K + k by expert id,
 * null slots removed. Any topk_idx value outside [0, N) counts as null. A token
 * should name each real expert at most once (moe_route guarantees it); if
 * not, R can exceed T*min(K,N) and the slots past that capacity are dropped
 * (their slot_pos still holds the position, which moe_combine then skips).
 *   counts[e]   = number of slots routed to real expert e              [N]
 *   offsets[e]  = exclusive prefix sum of counts; offsets[N] = R        [N+1]
 *   perm_token[p] = token of the p-th slot in expert order, p < R      [T*min(K,N)]
 *                 (entries from R on are left unwritten)
 *   slot_pos[t][k] = position p of slot (t,k) or -1 for a null slot   [T][K]
 *   x_perm[p] = x[perm_token[p]] when x and x_perm are both non-NULL   [T*min(K,N)][d]
 * ws: MOE_WS_PERMUTE bytes (per-chunk expert histograms).
 * R stays on the device; nothing is copied to the host.
 */
moe_status moe_permute(const moe_dims* dims, const int32_t* topk_idx, const void* x,
                       int32_t* counts, int32_t* offsets, int32_t* perm_token,
                       int32_t* slot_pos, void* x_perm, void* ws, size_t ws_bytes,
                       moe_stream stream);

/*
 * moe_expert_ffn -- grouped SwiGLU expert FFN over variable-length segments
 * (the grouped GEMM of the paper review's "implementation" paragraph; the
 * per-token FFN of the quant67 primer section 2, in SwiGLU form):
 *   for each group e and row p in [offsets[e], offsets[e+1]):
 *     h = silu(W_gate[e] a_p) * (W_up[e] a_p),  silu(z) = z / (1 + exp(-z))
 *     out_p = W_down[e] h
 * a: [max_rows][d_model] dtype; out: [max_rows][d_model] FLOAT32 (expert outputs
 * stay float32 so the combine rounds the layer output once);
 * w_gate, w_up: [n_groups][d_ff][d_model];
 * w_down: [n_groups][d_model][d_ff]. offsets: DEVICE [n_groups+1] int32,
 * read on the device only. Segment e is [a, b) with a = clamp(offsets[e], 0,
 * max_rows) and b = clamp(offsets[e+1], a, max_rows), so any offsets stay in
 * bounds; overlapping segments (decreasing offsets) are not meaningful.
 * offsets may be NULL when n_groups == 1 (one segment of max_rows rows).
 * Rows outside the segments are not written.
 * bf16: MFMA with float32 accumulation; h stored as IEEE half, and the down
 * projection multiplies it by W_down converted to half (exact for magnitudes in
 * [2^-17, 65504]; smaller ones truncated toward zero to a multiple of 2^-24) on
 * the half-precision MFMA; float32: float FMA throughout.
 * bf16 limit: (d_ff + 1) * d_model * 2 bytes (one group's weight matrix plus a
 * row) must fit in 4 GB, else MOE_ERR_UNSUPPORTED.
 * ws: moe_expert_ffn_workspace_bytes() bytes (holds h).
 */
moe_status moe_expert_ffn(const moe_dims* dims, int32_t n_groups, int32_t d_ff, int64_t max_rows,
                          const void* a, const int32_t* offsets, const void* w_gate,
                          const void* w_up, const void* w_down, void* out, void* ws,
                          size_t ws_bytes, moe_stream stream);

size_t moe_expert_ffn_workspace_bytes(const moe_dims* dims, int32_t d_ff, int64_t max_rows);

/*
 * moe_grouped_gemm -- one of the two GEMMs of moe_expert_ffn on its own (same
 * passage and segment rules as moe_expert_ffn; offsets NULL = one segment):
 *   op = MOE_GEMM_GATE_UP: out[p] = silu(b0[e] a_p) * (b1[e] a_p)   out h, [rows][n_out]
 *                          a: [rows][k_dim] dtype; b0, b1: [n_groups][n_out][k_dim]
 *   op = MOE_GEMM_DOWN:    out[p] = b0[e] a_p                        out float32, [rows][n_out]
 *                          a: [rows][k_dim] h; b0: [n_groups][n_out][k_dim]; b1 unused
 * where h is the layer's intermediate type (bf16 dtype: IEEE half bit patterns,
 * as GATE_UP writes them; float32 dtype: float); b0, b1 are dtype.
 * n_out and k_dim multiples of 8. No workspace.
 * bf16 limit: (n_out + 1) * k_dim * 2 bytes must fit in 4 GB, else
 * MOE_ERR_UNSUPPORTED.
 */
enum { MOE_GEMM_GATE_UP = 0, MOE_GEMM_DOWN = 1 };
moe_status moe_grouped_gemm(const moe_dims* dims, int32_t op, int32_t n_groups, int32_t n_out,
                            int32_t k_dim, int64_t rows, const void* a, const int32_t* offsets,
                            const void* b0, const void* b1, void* out, moe_stream stream);

/*
 * moe_expert_gate_up -- the layer's gate/up launch on its own (the grouped GEMM
 * of the paper review's "implementation" paragraph over the truncated slot list,
 * with the shared expert of the core formula in the same launch):
 *   h[p]  = silu(W_gate[e] x_{perm_token[p]}) * (W_up[e] x_{perm_token[p]})
 *           for p in [offsets[e], offsets[e+1]), the rows of expert e
 *   hs[t] = silu(Ws_gate x_t) * (Ws_up x_t) for every token (d_ff_shared > 0)
 * x: [T][d_model] dtype; perm_token [T*min(K,N)] and offsets [N+1] as written by
 * moe_permute (device; read on the device only, segments clamped as in
 * moe_expert_ffn, perm_token entries clamped to [0, T)); w_gate, w_up as in the
 * layer; ws_gate, ws_up: [d_ff_shared][d_model] (ignored when d_ff_shared = 0).
 * h: [T*min(K,N)][d_ff] and hs: [T][d_ff_shared] in the layer's intermediate
 * type (bf16 dtype: IEEE half; float32 dtype: float32). No workspace. bf16 limits
 * as for moe_layer_forward.
 */
moe_status moe_expert_gate_up(const moe_dims* dims, const void* x, const int32_t* perm_token,
                              const int32_t* offsets, const void* w_gate, const void* w_up,
                              const void* ws_gate, const void* ws_up, void* h, void* hs,
                              moe_stream stream);

/*
 * moe_combine -- y_t = y_shared_t + sum_k topk_w[t,k] * y_perm[slot_pos[t,k]]
 * (paper review section 3, core formula). A null slot (slot_pos = -1) adds
 * nothing with null_kind MOE_NULL_ZERO, topk_w[t,k] * null_src[t] with
 * MOE_NULL_COPY (null_src = x, [T][d] dtype) and topk_w[t,k] * null_src with
 * MOE_NULL_CONSTANT (null_src = v, [d] dtype); null_src is required for those
 * two and ignored otherwise. Summed in slot order in float32 with one rounding
 * to dtype; no atomics, so the result is bitwise reproducible. Other slots with
 * slot_pos outside [0, T*min(K,N)) are skipped. y_shared [T][d] float32, may be
 * NULL (no shared expert). y_perm: [T*min(K,N)][d] float32; y: [T][d] dtype.
 */
moe_status moe_combine(const moe_dims* dims, const void* y_perm, const int32_t* slot_pos,
                       const float* topk_w, const void* y_shared, const void* null_src, void* y,
                       moe_stream stream);

/*
 * moe_aux_stats -- load-balance and z-loss statistics over the N+M pool
 * (paper review section 3, "load-balance loss" and "Z-loss"):
 *   p_t = softmax over [s_0..s_{N-1}, s_null repeated M times]
 *   P[i] = mean_t p_t,i;  counts[i] = #slots with topk_idx == i;  f[i] = counts[i] / T
 *   scalars[0] = L_bal = N * sum_{i < N+M} f[i] P[i]
 *   scalars[1] = L_z   = mean_t (log sum_i exp v_t,i)^2
 *   scalars[2] = mean_t n_real[t]  (mean number of chosen real experts)
 * With M = 0 the pool is the N reals (column N ignored). A null logit of +inf
 * (an infinite per-token null bias) takes the limit: 1/M per null copy, 0 per
 * real, lse = +inf, so L_z = +inf. Reductions run in float64 in a fixed order
 * (bitwise reproducible), rounded once to float32.
 * logits: [T][N+1] float32 (column N effective); topk_idx: [T][K] int32.
 * f, P: [N+M] float32; counts: [N+M] int32 or NULL; scalars: [3] float32.
 * ws: MOE_WS_AUX bytes.
 */
moe_status moe_aux_stats(const moe_dims* dims, const float* logits, const int32_t* topk_idx,
                         float* f, float* P, int32_t* counts, float* scalars, void* ws,
                         size_t ws_bytes, moe_stream stream);

/* Device pointers of the layer's inputs. */
typedef struct {
  const void* x;               /* [T][d_model] dtype */
  const float* w_router;       /* [N+1][d_model] float32, row N = null */
  float null_bias;             /* added to the null logit */
  const float* null_bias_tok;  /* [T] float32 or NULL */
  const void* w_gate;          /* [N][d_ff][d_model] */
  const void* w_up;            /* [N][d_ff][d_model] */
  const void* w_down;          /* [N][d_model][d_ff] */
  const void* ws_gate;         /* [d_ff_shared][d_model] or NULL when d_ff_shared = 0 */
  const void* ws_up;           /* [d_ff_shared][d_model] */
  const void* ws_down;         /* [d_model][d_ff_shared] */
  const void* null_value;      /* [d_model] dtype, the constant expert's vector
                                  (null_kind MOE_NULL_CONSTANT), else unused */
} moe_layer_params;

/* Optional device outputs of moe_layer_forward; any member may be NULL. */
typedef struct {
  float* logits;      /* [T][N+1] */
  int32_t* topk_idx;  /* [T][K] */
  float* topk_w;      /* [T][K] */
  int32_t* n_real;    /* [T] */
  int32_t* offsets;   /* [N+1] expert segment offsets, offsets[N] = R */
  int32_t* counts;    /* [N+M] pool slot counts */
  float* f;           /* [N+M] */
  float* P;           /* [N+M] */
  float* scalars;     /* [3] L_bal, L_z, mean n_real */
} moe_aux_out;

/*
 * moe_layer_forward -- the whole layer: route -> permute -> gather ->
 * grouped SwiGLU GEMMs -> shared expert -> combine -> statistics, all enqueued
 * on `stream` with no host synchronisation. y: [T][d_model] dtype.
 * aux may be NULL; the statistics kernels run only when aux requests
 * counts, f, P or scalars. ws: moe_workspace_bytes(dims, MOE_WS_LAYER) bytes,
 * sized for the worst case of T*min(K,N) real slots. With a shared expert,
 * zero-output null slots and enough rows per expert for the large GEMM tiles
 * (T*min(K,N)/N and T both at least 512), the combine is done in the epilogue of
 * the shared expert's down projection (same arithmetic: float32 fmaf in slot order,
 * one rounding) and no float32 shared-expert output is kept in the workspace.
 * bf16 limit: (T + 1), (d_ff + 1) and (d_ff_shared + 1) rows of d_model bf16
 * each fit in 4 GB (x is gathered through 32-bit offsets), else
 * MOE_ERR_UNSUPPORTED.
 */
moe_status moe_layer_forward(const moe_dims* dims, const moe_layer_params* params, void* y,
                             const moe_aux_out* aux, void* ws, size_t ws_bytes,
                             moe_stream stream);

/*
 * moe_layer_forward_noalloc -- moe_layer_forward for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): same arguments and results, but no workspace argument. The
 * workspace is a static device array of MOE_NOALLOC_MAX_WS_BYTES bytes that the
 * library holds on every GPU it runs on until the process ends (its address is
 * looked up once per device, on the first call with that device current). Layers
 * whose moe_workspace_bytes(dims, MOE_WS_LAYER) exceeds that size return
 * MOE_ERR_UNSUPPORTED with nothing launched. The calling thread's current device
 * (hipGetDevice) must be the one `stream` belongs to. Every call on a GPU shares
 * that GPU's array: calls that overlap on one GPU (other streams, other threads)
 * race and give undefined results; calls ordered on one stream are safe. The
 * forward writes every workspace byte it reads, so nothing needs clearing between
 * calls. Calls no hipMalloc, hipFree or other allocating routine.
 */
#define MOE_NOALLOC_MAX_WS_BYTES (64u << 20)
moe_status moe_layer_forward_noalloc(const moe_dims* dims, const moe_layer_params* params, void* y,
                                     const moe_aux_out* aux, moe_stream stream);

/* Gradients written by moe_layer_backward (float32, device, 16-byte aligned). */
typedef struct {
  float* dx;        /* [T][d_model] */
  float* dw_router; /* [N+1][d_model]; row N (the null logit's row) is 0 when n_null = 0 */
  float* dw_gate;   /* [N][d_ff][d_model] */
  float* dw_up;     /* [N][d_ff][d_model] */
  float* dw_down;   /* [N][d_model][d_ff] */
  float* dws_gate;  /* [d_ff_shared][d_model]; required when d_ff_shared > 0 */
  float* dws_up;    /* [d_ff_shared][d_model] */
  float* dws_down;  /* [d_model][d_ff_shared] */
} moe_layer_grads;

/*
 * moe_layer_backward -- gradients of the training objective
 *   L = <dy, y> + alpha * L_bal + beta * L_z
 * with y the output of moe_layer_forward on the same inputs, dy [T][d_model] dtype
 * the upstream gradient, and L_bal, L_z the statistics of moe_aux_stats (paper
 * review section 3: load-balance loss and z-loss are added to the task loss; the
 * pages train with alpha = 2e-2, beta = 1e-3). The routing decision is held fixed
 * (top-K is piecewise constant): gradients reach the router through the
 * renormalised weights of the chosen reals and through the pool softmax of L_bal
 * and L_z (the null logit's M copies summed into row N). Expert gradients follow
 * the SwiGLU chain rule per segment; the shared expert's when present.
 * The routing, permutation and expert pre-activations are recomputed from x
 * (nothing is kept from the forward call). All enqueued on `stream`, no host
 * synchronisation; deterministic.
 * bf16 and MOE_NULL_ZERO only (MOE_ERR_UNSUPPORTED otherwise); 32-bit offset
 * limits as for moe_layer_forward, on the transposed activations too.
 * ws: moe_workspace_bytes(dims, MOE_WS_BACKWARD) bytes.
 */
moe_status moe_layer_backward(const moe_dims* dims, const moe_layer_params* params, const void* dy,
                              float alpha, float beta, const moe_layer_grads* grads, void* ws,
                              size_t ws_bytes, moe_stream stream);

/*
 * moe_layer_forward_train / moe_layer_backward_saved -- the same forward and backward
 * for a training step that keeps the forward's state instead of recomputing it (the
 * paper review, section 4 "training configuration", trains the layer; which state a
 * step keeps is not fixed by the pages).
 * moe_layer_forward_train computes y exactly as moe_layer_forward does (bit for bit)
 * and leaves in ws -- moe_workspace_bytes(dims, MOE_WS_BACKWARD) bytes, the backward's
 * workspace -- the routing (logits, selection, weights), the permutation, the pool
 * counts f and the expert pre-activations g, u (float32) and h = silu(g) u (bf16), routed
 * and shared. aux may ask for P, counts and scalars only (its other pointers must be
 * NULL: MOE_ERR_ARG; the routing outputs stay in ws). Same limits as moe_layer_backward
 * (bf16, MOE_NULL_ZERO).
 * moe_layer_backward_saved then returns what moe_layer_backward returns for the same
 * inputs and dy (bit for bit), reading that state from ws instead of recomputing it: ws
 * must be the workspace of a moe_layer_forward_train call with the same dims, params
 * and x, with nothing written to it in between (not checked; the ws memory of the pair
 * is the caller's). Saves the recompute (routing, permutation and one gate/up GEMM);
 * the forward instead stores g and u (8 bytes per row and column) next to h.
 * All enqueued on `stream`; no host synchronisation.
 */
moe_status moe_layer_forward_train(const moe_dims* dims, const moe_layer_params* params, void* y,
                                   const moe_aux_out* aux, void* ws, size_t ws_bytes, moe_stream stream);
moe_status moe_layer_backward_saved(const moe_dims* dims, const moe_layer_params* params, const void* dy,
                                    float alpha, float beta, const moe_layer_grads* grads, void* ws,
                                    size_t ws_bytes, moe_stream stream);

/*
 * moe_validate_inputs -- optional check of the layer's inputs, not part of the
 * forward: NaN or +-inf anywhere in x, the router, the expert and shared-expert
 * weights or the constant vector, and NaN in null_bias / null_bias_tok (an
 * infinite null bias is a valid input: it sends every slot of a token to the
 * null copies, or none). The layer's outputs are undefined for such inputs; the
 * pages fix nothing for them. Same dims and params as moe_layer_forward (and the
 * same pointer checks). Unlike every other entry point this one synchronises
 * `stream`, to read one count back. ws: at least 16 bytes of device memory.
 * Returns MOE_ERR_NONFINITE if anything is found, MOE_OK otherwise.
 */
moe_status moe_validate_inputs(const moe_dims* dims, const moe_layer_params* params, void* ws,
                               size_t ws_bytes, moe_stream stream);

/* Workspace bytes for MOE_WS_LAYER / ROUTE / PERMUTE / AUX / BACKWARD (bf16 only);
 * 0 on invalid dims. */
size_t moe_workspace_bytes(const moe_dims* dims, int32_t which);

/* Static, NUL-terminated description of a status code. */
const char* moe_status_str(moe_status status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
