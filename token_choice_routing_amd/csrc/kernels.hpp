// Launch interfaces between the C-ABI layer (api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

struct RouteArgs {
  int64_t T;
  int d, N, M, K;
  bool bf16;
  const void* x;
  const float* w_router;
  float null_bias;
  const float* null_bias_tok;
  const float* logits_in;
  float* logits_out;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* n_real;
  uint16_t* w_split;  // [3][Np][d] bf16 scratch, bf16 path only
};
size_t route_split_bytes(int N, int d);
hipError_t launch_route(const RouteArgs& a, hipStream_t stream);

struct PermuteArgs {
  int64_t T;
  int K, N, d, elt_bytes;
  const int32_t* topk_idx;
  const void* x;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm_token;
  int32_t* slot_pos;
  void* x_perm;
  int32_t* ws;
};
int permute_nchunks(int64_t TK);
size_t permute_ws_bytes(int64_t TK, int N);
hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream);

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

struct GemmArgs {
  bool bf16;
  int op;              // 0: h = silu(a b0^T) * (a b1^T) -> dtype; 1: out = a b0^T -> float32
  int groups;
  int n_out, k_dim;
  int64_t max_rows;
  const void* a;       // [max_rows][k_dim]
  const int32_t* offsets;  // [groups+1] device, or NULL: one segment of max_rows rows
  const void* b0;      // [groups][n_out][k_dim]
  const void* b1;
  void* out;           // [max_rows][n_out]
  int num_cus;
};
hipError_t launch_grouped_gemm(const GemmArgs& g, hipStream_t stream);

struct CombineArgs {
  bool bf16;
  int64_t T;
  int K, d;
  int64_t max_rows;
  const void* y_perm;
  const int32_t* slot_pos;
  const float* topk_w;
  const void* y_shared;
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
size_t aux_ws_bytes(int64_t T, int N, int M);
hipError_t launch_aux(const AuxArgs& a, hipStream_t stream);

}  // namespace moe
