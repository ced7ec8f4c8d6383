// Launch interfaces between the C-ABI layer (api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// Fixed-point scales of the fused statistics accumulators (probability sums, lse^2 sums).
constexpr double kAuxPScale = 4294967296.0;  // 2^32
constexpr double kAuxZScale = 1048576.0;     // 2^20

struct RouteArgs {
  int64_t T;
  int d, N, M, K;
  bool bf16;
  bool fused;         // also emit per-tile histograms and statistic sums
  const void* x;
  const float* w_router;
  float null_bias;
  const float* null_bias_tok;
  const float* logits_in;
  float* logits_out;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* n_real;
  void* ws;            // bf16 scoring scratch of route_ws_bytes(T, N, d) bytes
  int32_t* chunk_hist; // fused: [tiles][N] real slots per expert and 64-token tile
  int32_t* rhist;      // fused: [tiles][K + 1] tokens per number of chosen reals r
  double* tstats;      // fused: [tiles][N + 3] sums of p_t,j (j <= N), lse_t^2 and r_t
  int null_kind;       // moe_null_kind: 0 weights over the chosen reals, else over all K slots
};
int route_tokens_per_block();
size_t route_ws_bytes(int64_t T, int N, int d);
hipError_t launch_route(const RouteArgs& a, hipStream_t stream);

// Statistics accumulated in fixed point by the standalone statistics kernels.
struct AuxFinal {
  const uint64_t* acc;   // [N + 4]: P sums (N reals, null), lse^2, n_real, tokens with lse = +inf
  const int32_t* cnt;    // [N + M]
  float* f;
  float* P;
  int32_t* counts;
  float* scalars;
};

// Statistics finalised by the permutation's scan kernel in the fused layer path,
// from the router's per-tile sums (added in tile order, so the result does not
// depend on scheduling).
struct AuxTiles {
  const double* tstats;  // [tiles][N + 3]
  const int32_t* rhist;  // [tiles][K + 1]
  float* f;
  float* P;
  int32_t* counts;
  float* scalars;
};

struct PermuteArgs {
  int64_t T;
  int K, N, M, d, elt_bytes;
  const int32_t* topk_idx;
  const void* x;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm_token;
  int32_t* slot_pos;
  void* x_perm;
  int32_t* ws;                    // chunk_hist [nchunks][N]
  bool hist_ready;                // chunk_hist already written (by the fused router)
  const AuxTiles* aux;            // optional statistics finalisation (fused path)
  int32_t* row_dst;               // optional: row_dst[p] = t min(K, N) + k for the slot (t, k) at p
                                  // (the token's reals come first, so k < min(K, N))
};
int permute_nchunks(int64_t T);
size_t permute_ws_bytes(int64_t T, int N);
hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream);
// A few bf16 tokens: the routing step in one workgroup (launch_route uses it by
// itself); with pa (fused routing only) that launch also does what launch_permute(*pa)
// would (permutation and statistics; x_perm is not written).
bool route_small_ok(const RouteArgs& r);
hipError_t launch_route_small(const RouteArgs& r, const PermuteArgs* pa, hipStream_t stream);

struct FfnArgs {
  bool bf16;
  int groups;          // segments (experts)
  int d_model, d_ff;
  int64_t max_rows;
  const void* a;       // [max_rows][d_model]
  const int32_t* offsets;  // [groups+1] device, or NULL: one segment of max_rows rows
  const void* w_gate;  // [groups][d_ff][d_model]
  const void* w_up;
  const void* w_down;  // [groups][d_model][d_ff]
  void* h;             // [max_rows][d_ff] scratch
  void* out;           // [max_rows][d_model]
  int num_cus;
};
hipError_t launch_expert_ffn(const FfnArgs& a, hipStream_t stream);

// One GEMM problem of a grouped launch: rows of segment g (from offsets, or one
// segment of max_rows rows) times weight group g. a_rows optionally redirects
// row p of A to a[a_rows[p]] (the permutation's gather, fused into the loads).
struct GemmProblem {
  const uint16_t* a;        // [a_nrows][k_dim] (bf16 bits, or float for the f32 path)
  const int32_t* a_rows;    // [max_rows] or NULL
  int64_t a_nrows;
  const int32_t* offsets;   // [groups+1] device, or NULL
  int groups;               // 0 = absent
  int64_t max_rows;
  const uint16_t* b0;       // [groups][n_out][k_dim]
  const uint16_t* b1;       // gate/up: the up weights
  int n_out, k_dim;
  void* out;                // [max_rows][n_out]: bf16 h (op 0) or float32 (op 1)
  // Weight-gradient form (bf16 op 1 only; all zero otherwise):
  const int32_t* k_offsets;  // [groups+1] device or NULL: group e reduces over the K
                             // columns [k_offsets[e], k_offsets[e+1]) (multiples of 8) of A
                             // and of b0, which is then one [n_out][ldb] matrix for all groups
  int64_t lda, ldb;          // row strides of a and b0/b1 in elements (0 = k_dim)
  int rows_per_group;        // > 0: group e owns output rows [e*rpg, (e+1)*rpg) and reads
                             // rows [0, rpg) of a (offsets unused)
  // Layer forward, 256 x 256 tiles only (all zero otherwise):
  const int32_t* out_rows;   // op 2, role 2: row p is stored at output row out_rows[p] (token-major slots)
  // op 3, the shared expert's down projection with the combine in its epilogue: output
  // row t (bf16) = acc_t + sum over k < comb_n[t] of comb_w[t][k] * comb_z[t * comb_kr + k],
  // float32 fmaf in slot order, rounded once.
  const float* comb_z;       // [rows * comb_kr][n_out] float32 routed expert outputs, token-major
  const int32_t* comb_n;     // [rows] routed slots of each token (its first slots)
  const float* comb_w;       // [rows][comb_k] slot weights
  int comb_k, comb_kr;
  // K-major weights (op 1 on 256 x 256 tiles only): group e's weights are b0's matrix
  // e of [k_split][n_out] for K rows [0, k_split) and, when k_split < k_dim, b1's matrix
  // e of [k_dim - k_split][n_out] for the rest: B[n][k] = b0[e][k][n] (b1[e][k -
  // k_split][n]). A row-major weight [n_out][k_dim] of the other modes is the transpose
  // of this layout; the backward's data gradients read the forward's weights this way.
  // n_out a multiple of 8, k_split and k_dim multiples of 32.
  // With a_kmajor too (the weight-gradient form, k_offsets and rows_per_group set): group
  // e reduces over rows [k_offsets[e], k_offsets[e+1]) of two row-major sources, A[m][k]
  // = a[k][m0 + m] (row stride lda, m0 the group-relative output row) and B[n][k] =
  // b0[k][n] (row stride ldb); k_dim bounds the rows of either.
  int b_kmajor, k_split;
  int a_kmajor;
  // op 4 (the backward's recompute of op 0, 256 x 256 tiles only): g = a b0^T and u =
  // a b1^T stored as float32 [max_rows][n_out] here, and out = bf16 silu(g) u.
  void* keep_g;  // IEEE half [max_rows][n_out]
  void* keep_u;
  // op 4, optional: h also stored as IEEE half here (the forward's down-projection input,
  // bit for bit what op 0 writes), for a forward that keeps its pre-activations
  void* keep_h16;
};
// op 0: out = silu(a b0^T) * (a b1^T) (bf16 a, half out); op 1: out = a b0^T (bf16 a,
// float32 out; with b_kmajor set in both problems, B read from K-major b0 / b1, 256 x 256
// tiles only); op 2: out = a b0^T with a in half (the layer's h), float32 out; op 3: op 2
// with the combine epilogue (comb_* fields), bf16 out, on the 256 x 256 tiles only (the
// launch is refused where gemm_pair_uses_pp is false); op 4: op 0 keeping g and u
// (keep_g / keep_u, IEEE half) with h in bf16 (256 x 256 tiles, roles 2 and 3). Both problems in one
// launch.
// (float32 layers: op 2 is op 1.)
// role names the launch in profiles: 0 standalone grouped, 1 standalone single
// segment, 2 the layer's fused launch, 3 the layer backward.
hipError_t launch_gemm_pair(bool bf16, int op, const GemmProblem& p0, const GemmProblem& p1,
                            int num_cus, hipStream_t stream, int role);
// bf16 operands are read through buffer resources with 32-bit byte offsets that may
// point one row past the end: one group's weight matrix, and a gathered activation
// matrix (a_rows), each plus one row, must fit in 4 GB. False means the launch is
// refused.
bool gemm_operands_fit(const GemmProblem& p);
// Whether a bf16 launch of these problems (plain forms) runs on the 256 x 256 tiles.
bool gemm_pair_uses_pp(const GemmProblem& p0, const GemmProblem& p1);
// Whether an op 1 launch of these K-major weight problems is taken (else it is refused).
bool gemm_kmajor_ok(const GemmProblem& p0, const GemmProblem& p1);

// Input check (validate.hip): count[0] = 0; count[0] += non-finite elements of data
// (bf16 or float32; nan_only: NaN alone, infinities allowed).
hipError_t launch_zero_count(int32_t* count, hipStream_t s);
hipError_t launch_count_nonfinite(const void* data, int64_t n, bool bf16, bool nan_only, int32_t* count,
                                  hipStream_t s);

// Backward-pass helpers (backward.hip); all enqueue on `s`, bf16 tensors as bits.
// out[b][c][c_out + r] (row stride ldo, batch stride out_batch) = in[b][r][c], in [b][R][C].
hipError_t launch_transpose(const void* in, int64_t batches, int64_t R, int64_t C, void* out, int64_t ldo,
                            int64_t c_out, int64_t out_batch, hipStream_t s);
// kofs[e] = segment starts padded to multiples of 8 (segments as the GEMM clamps them).
hipError_t launch_pad_offsets(const int32_t* offsets, int G, int64_t rows, int32_t* kofs, hipStream_t s);
// dst [C][ld]: each segment's rows (read through src_rows when given) as columns from
// kofs[e], zero up to the next padded start; offsets NULL = one segment of `rows`.
hipError_t launch_transpose_segments(const void* src, const int32_t* src_rows, int64_t src_nrows,
                                     const int32_t* offsets, const int32_t* kofs, int G, int64_t rows,
                                     int64_t C, void* dst, int64_t ld, hipStream_t s);
// out[p] = x[perm_token[p]] (bf16 rows of d, d a multiple of 8) for p < offsets[G] (at most R).
hipError_t launch_gather_slots(const void* x, const int32_t* perm_token, int64_t T, const int32_t* offsets, int G,
                               int64_t R, int d, void* out, hipStream_t s);
hipError_t launch_swiglu_h(const float* g, const float* u, const int32_t* offsets, int G, int64_t rows, int F,
                           void* h, hipStream_t s);
// g and u: float32, or IEEE half when g16 (the keep-mode GEMM's).
hipError_t launch_swiglu_bwd(const void* g, const void* u, bool g16, const float* dh, const int32_t* offsets, int G,
                             int64_t rows, int F, void* dgu, hipStream_t s);
// Real slot (t, k) at row p: dy_perm[p] = topk_w dy_t (bf16), w_perm[p] = topk_w,
// row_slot[p] = t K + k; null slots: dw[t][k] = 0.
hipError_t launch_slot_rows(const void* dy, const int32_t* slot_pos, const float* topk_w, int64_t T, int K,
                            int d, int64_t R, void* dy_perm, float* w_perm, int32_t* row_slot, float* dw,
                            hipStream_t s);
// Routed rows from U = dy W_d: dw[row_slot[p]] = <U_p, h_p>, and the SwiGLU backward
// of dh = w_perm U into dgu (as launch_swiglu_bwd).
hipError_t launch_swiglu_bwd_routed(const void* g, const void* u, bool g16, const float* U, const void* h,
                                    const float* w_perm, const int32_t* row_slot, const int32_t* offsets, int G,
                                    int64_t rows, int F, void* dgu, float* dw, hipStream_t s);
hipError_t launch_router_bwd(const float* logits, const int32_t* topk_idx, const float* topk_w, const float* dw,
                             const float* f, int64_t T, int N, int M, int K, float alpha, float beta, float* ds,
                             hipStream_t s);
size_t router_wgrad_ws_bytes(int64_t T, int N1, int d);
hipError_t launch_router_wgrad(const float* ds, const void* x, int64_t T, int N1, int d, float* part, float* dw,
                               hipStream_t s);
hipError_t launch_scatter_dx(const float* dx_perm, const int32_t* slot_pos, int K, int64_t R, const float* dx_shared,
                             const float* ds, const float* w_router, int N1, int d, int64_t T, float* dx,
                             hipStream_t s);
// kofs[0..S]: S uniform K chunks (multiples of 8) of `rows` rows, for a split weight gradient.
hipError_t launch_split_offsets(int64_t rows, int S, int32_t* kofs, hipStream_t s);
// out = sum over s < S of part[s] (n floats each), in order.
hipError_t launch_sum_partials(const float* part, int S, int64_t n, float* out, hipStream_t s);

struct CombineArgs {
  bool bf16;
  int64_t T;
  int K, d;
  int64_t max_rows;
  const void* y_perm;
  const int32_t* slot_pos;
  const float* topk_w;
  const void* y_shared;
  const void* null_src;    // rows a null slot adds (dtype), or NULL
  int64_t null_stride;     // elements between the rows of consecutive tokens (0: one row)
  void* y;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

struct AuxArgs {
  int64_t T;
  int N, M, K;
  const float* logits;
  const int32_t* topk_idx;
  float* f;
  float* P;
  int32_t* counts;
  float* scalars;
  void* ws;
};
size_t aux_ws_bytes(int N, int M);
hipError_t launch_aux(const AuxArgs& a, hipStream_t stream);

}  // namespace moe
