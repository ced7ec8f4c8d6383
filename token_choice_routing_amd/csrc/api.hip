// C ABI of libmoe_mi355x.so: argument validation, workspace carving and kernel
// launches for the null-expert token-choice MoE layer forward. The entry points
// and their contracts are documented in include/moe.h.
#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "kernels.hpp"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// bf16 GEMM operands are addressed with 32-bit byte offsets that may run one row
// past the end: one group's weight matrix and a gathered activation matrix, plus a
// row, must each fit in 4 GB.
inline bool fits_4g(int64_t rows, int64_t cols) { return (rows + 1) * cols * 2 <= 0xFFFFFFFFll; }

moe_status check_dims(const moe_dims* d) {
  if (!d) return MOE_ERR_ARG;
  if (d->T < 0 || d->n_experts < 1 || d->n_null < 0 || d->top_k < 1) return MOE_ERR_ARG;
  if ((int64_t)d->top_k > (int64_t)d->n_experts + d->n_null) return MOE_ERR_ARG;
  if (d->n_null == 0 && d->top_k > d->n_experts) return MOE_ERR_ARG;
  if (d->d_model < 8 || d->d_model % 8 || d->d_ff < 8 || d->d_ff % 8) return MOE_ERR_ARG;
  if (d->d_ff_shared < 0 || d->d_ff_shared % 8) return MOE_ERR_ARG;
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_ERR_ARG;
  if (d->null_kind < MOE_NULL_ZERO || d->null_kind > MOE_NULL_CONSTANT) return MOE_ERR_ARG;
  if (d->n_experts > MOE_MAX_EXPERTS || d->top_k > MOE_MAX_TOPK ||
      (int64_t)d->n_experts + d->n_null > MOE_MAX_POOL)
    return MOE_ERR_UNSUPPORTED;
  if (d->T * (int64_t)d->top_k >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

inline size_t elt_bytes(const moe_dims* d) { return d->dtype == MOE_BF16 ? 2 : 4; }
inline int64_t max_rows(const moe_dims* d) { return d->T * (int64_t)std::min(d->top_k, d->n_experts); }

// Device pointers that must be present and 16-byte aligned.
moe_status need(const void* p) {
  if (!p) return MOE_ERR_ARG;
  return aligned16(p) ? MOE_OK : MOE_ERR_ALIGN;
}
moe_status maybe(const void* p) { return (!p || aligned16(p)) ? MOE_OK : MOE_ERR_ALIGN; }

#define MOE_TRY(expr)                  \
  do {                                 \
    const moe_status s_ = (expr);      \
    if (s_ != MOE_OK) return s_;       \
  } while (0)

#define HIP_TRY(expr)                              \
  do {                                             \
    if ((expr) != hipSuccess) return MOE_ERR_HIP;  \
  } while (0)

std::atomic<int> g_cu_count[64];

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = g_cu_count[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  g_cu_count[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Layer workspace layout (byte offsets, 256-byte aligned pieces).
struct LayerWs {
  size_t logits, topk_idx, topk_w, n_real, counts, offsets, perm_token, slot_pos, route, permute,
      h, hs, yp, ys, tstats, rhist, total;
};

LayerWs layer_ws(const moe_dims* d) {
  LayerWs w{};
  const int64_t T = d->T, TK = T * d->top_k, R = max_rows(d);
  const int N = d->n_experts, M = d->n_null;
  const size_t e = elt_bytes(d);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  w.logits = take((size_t)T * (N + 1) * 4);
  w.topk_idx = take((size_t)TK * 4);
  w.topk_w = take((size_t)TK * 4);
  w.n_real = take((size_t)T * 4);
  w.counts = take((size_t)N * 4);
  w.offsets = take((size_t)(N + 1) * 4);
  w.perm_token = take((size_t)R * 4);
  w.slot_pos = take((size_t)TK * 4);
  w.route = take(d->dtype == MOE_BF16 ? route_ws_bytes(T, N, d->d_model) : 0);
  w.permute = take(permute_ws_bytes(T, N));
  w.h = take((size_t)R * d->d_ff * e);
  w.hs = take((size_t)T * d->d_ff_shared * e);
  w.yp = take((size_t)R * d->d_model * 4);
  w.ys = take(d->d_ff_shared ? (size_t)T * d->d_model * 4 : 0);
  const int64_t tiles = permute_nchunks(T);  // 64-token tiles of the router and the sort
  w.tstats = take((size_t)tiles * (N + 3) * 8);
  w.rhist = take((size_t)tiles * (d->top_k + 1) * 4);
  w.total = o;
  return w;
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument (dimension or NULL pointer)";
    case MOE_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_UNSUPPORTED: return "dimensions outside this build's limits";
    case MOE_ERR_HIP: return "HIP launch or runtime error";
  }
  return "unknown status";
}

int32_t moe_version(void) { return 100; }

size_t moe_workspace_bytes(const moe_dims* d, int32_t which) {
  if (check_dims(d) != MOE_OK) return 0;
  switch (which) {
    case MOE_WS_LAYER: return layer_ws(d).total;
    case MOE_WS_ROUTE:
      return d->dtype == MOE_BF16 ? route_ws_bytes(d->T, d->n_experts, d->d_model) : 0;
    case MOE_WS_PERMUTE: return permute_ws_bytes(d->T, d->n_experts);
    case MOE_WS_AUX: return aux_ws_bytes(d->n_experts, d->n_null);
  }
  return 0;
}

size_t moe_expert_ffn_workspace_bytes(const moe_dims* d, int32_t d_ff, int64_t rows) {
  if (check_dims(d) != MOE_OK || d_ff < 8 || d_ff % 8 || rows < 0) return 0;
  return (size_t)rows * d_ff * elt_bytes(d);
}

moe_status moe_route(const moe_dims* d, const void* x, const float* w_router, float null_bias,
                     const float* null_bias_tok, const float* logits_in, float* logits_out,
                     int32_t* topk_idx, float* topk_w, int32_t* n_real, void* ws,
                     size_t ws_bytes, moe_stream stream) {
  MOE_TRY(check_dims(d));
  MOE_TRY(need(topk_idx));
  MOE_TRY(need(topk_w));
  MOE_TRY(maybe(n_real));
  MOE_TRY(maybe(logits_out));
  const bool bf16 = d->dtype == MOE_BF16;
  if (logits_in) {
    MOE_TRY(need(logits_in));
  } else {
    MOE_TRY(need(x));
    MOE_TRY(need(w_router));
    MOE_TRY(maybe(null_bias_tok));
    if (bf16) {
      if (!ws || ws_bytes < route_ws_bytes(d->T, d->n_experts, d->d_model)) return MOE_ERR_WORKSPACE;
      MOE_TRY(maybe(ws));
    }
  }
  if (d->T == 0) return MOE_OK;
  (void)hipGetLastError();
  RouteArgs a{d->T, d->d_model, d->n_experts, d->n_null, d->top_k, bf16, false, x, w_router,
              null_bias, null_bias_tok, logits_in, logits_out, topk_idx, topk_w, n_real,
              ws, nullptr, nullptr, nullptr, d->null_kind};
  HIP_TRY(launch_route(a, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_permute(const moe_dims* d, const int32_t* topk_idx, const void* x, int32_t* counts,
                       int32_t* offsets, int32_t* perm_token, int32_t* slot_pos, void* x_perm,
                       void* ws, size_t ws_bytes, moe_stream stream) {
  MOE_TRY(check_dims(d));
  MOE_TRY(need(topk_idx));
  MOE_TRY(need(counts));
  MOE_TRY(need(offsets));
  MOE_TRY(need(perm_token));
  MOE_TRY(need(slot_pos));
  MOE_TRY(maybe(x));
  MOE_TRY(maybe(x_perm));
  const size_t need_ws = permute_ws_bytes(d->T, d->n_experts);
  if (need_ws && (!ws || ws_bytes < need_ws)) return MOE_ERR_WORKSPACE;
  MOE_TRY(maybe(ws));
  if (d->T == 0) return MOE_OK;
  (void)hipGetLastError();
  PermuteArgs a{d->T, d->top_k, d->n_experts, d->n_null, d->d_model, (int)elt_bytes(d), topk_idx,
                x, counts, offsets, perm_token, slot_pos, x_perm, static_cast<int32_t*>(ws),
                false, nullptr};
  HIP_TRY(launch_permute(a, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_dims* d, int32_t n_groups, int32_t d_ff, int64_t rows,
                          const void* a, const int32_t* offsets, const void* w_gate,
                          const void* w_up, const void* w_down, void* out, void* ws,
                          size_t ws_bytes, moe_stream stream) {
  MOE_TRY(check_dims(d));
  if (n_groups < 1 || n_groups > MOE_MAX_EXPERTS + 1 || d_ff < 8 || d_ff % 8 || rows < 0)
    return MOE_ERR_ARG;
  if (!offsets && n_groups != 1) return MOE_ERR_ARG;
  if (rows * (int64_t)std::max(d->d_model, d_ff) >= (int64_t(1) << 40)) return MOE_ERR_UNSUPPORTED;
  if (d->dtype == MOE_BF16 && !fits_4g(d_ff, d->d_model)) return MOE_ERR_UNSUPPORTED;
  MOE_TRY(need(a));
  MOE_TRY(maybe(offsets));
  MOE_TRY(need(w_gate));
  MOE_TRY(need(w_up));
  MOE_TRY(need(w_down));
  MOE_TRY(need(out));
  const size_t need_ws = (size_t)rows * d_ff * elt_bytes(d);
  if (need_ws && (!ws || ws_bytes < need_ws)) return MOE_ERR_WORKSPACE;
  MOE_TRY(maybe(ws));
  if (rows == 0) return MOE_OK;
  (void)hipGetLastError();
  FfnArgs f{d->dtype == MOE_BF16, n_groups, d->d_model, d_ff, rows, a, offsets, w_gate, w_up,
            w_down, ws, out, cu_count()};
  HIP_TRY(launch_expert_ffn(f, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_grouped_gemm(const moe_dims* d, int32_t op, int32_t n_groups, int32_t n_out,
                            int32_t k_dim, int64_t rows, const void* a, const int32_t* offsets,
                            const void* b0, const void* b1, void* out, moe_stream stream) {
  MOE_TRY(check_dims(d));
  if (op != MOE_GEMM_GATE_UP && op != MOE_GEMM_DOWN) return MOE_ERR_ARG;
  if (n_groups < 1 || n_groups > MOE_MAX_EXPERTS + 1 || n_out < 8 || n_out % 8 || k_dim < 8 ||
      k_dim % 8 || rows < 0)
    return MOE_ERR_ARG;
  if (!offsets && n_groups != 1) return MOE_ERR_ARG;
  if (d->dtype == MOE_BF16 && !fits_4g(n_out, k_dim)) return MOE_ERR_UNSUPPORTED;
  MOE_TRY(need(a));
  MOE_TRY(maybe(offsets));
  MOE_TRY(need(b0));
  if (op == MOE_GEMM_GATE_UP) MOE_TRY(need(b1));
  MOE_TRY(need(out));
  if (rows == 0) return MOE_OK;
  (void)hipGetLastError();
  GemmProblem g{static_cast<const uint16_t*>(a), nullptr, rows, offsets, n_groups, rows,
                static_cast<const uint16_t*>(b0),
                op == MOE_GEMM_GATE_UP ? static_cast<const uint16_t*>(b1) : nullptr, n_out, k_dim,
                out};
  HIP_TRY(launch_gemm_pair(d->dtype == MOE_BF16, op, g, GemmProblem{}, cu_count(),
                           static_cast<hipStream_t>(stream), offsets ? 0 : 1));
  return MOE_OK;
}

// Per-token stride (elements) of the rows a null slot adds: x for copy experts,
// the one vector v for constant experts.
inline int64_t null_stride(const moe_dims* d) { return d->null_kind == MOE_NULL_COPY ? d->d_model : 0; }

moe_status moe_combine(const moe_dims* d, const void* y_perm, const int32_t* slot_pos,
                       const float* topk_w, const void* y_shared, const void* null_src, void* y,
                       moe_stream stream) {
  MOE_TRY(check_dims(d));
  MOE_TRY(need(y_perm));
  MOE_TRY(need(slot_pos));
  MOE_TRY(need(topk_w));
  MOE_TRY(maybe(y_shared));
  if (d->null_kind != MOE_NULL_ZERO) MOE_TRY(need(null_src));
  MOE_TRY(need(y));
  if (d->T == 0) return MOE_OK;
  (void)hipGetLastError();
  CombineArgs c{d->dtype == MOE_BF16, d->T, d->top_k, d->d_model, max_rows(d), y_perm, slot_pos,
                topk_w, y_shared, d->null_kind != MOE_NULL_ZERO ? null_src : nullptr, null_stride(d), y};
  HIP_TRY(launch_combine(c, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_aux_stats(const moe_dims* d, const float* logits, const int32_t* topk_idx, float* f,
                         float* P, int32_t* counts, float* scalars, void* ws, size_t ws_bytes,
                         moe_stream stream) {
  MOE_TRY(check_dims(d));
  MOE_TRY(need(logits));
  MOE_TRY(need(topk_idx));
  MOE_TRY(need(f));
  MOE_TRY(need(P));
  MOE_TRY(maybe(counts));
  MOE_TRY(need(scalars));
  const size_t need_ws = aux_ws_bytes(d->n_experts, d->n_null);
  if (!ws || ws_bytes < need_ws) return MOE_ERR_WORKSPACE;
  MOE_TRY(maybe(ws));
  if (d->T == 0) return MOE_OK;
  (void)hipGetLastError();
  AuxArgs a{d->T, d->n_experts, d->n_null, d->top_k, logits, topk_idx, f, P, counts, scalars, ws};
  HIP_TRY(launch_aux(a, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_layer_forward(const moe_dims* d, const moe_layer_params* p, void* y,
                             const moe_aux_out* aux, void* ws, size_t ws_bytes,
                             moe_stream stream) {
  MOE_TRY(check_dims(d));
  if (!p) return MOE_ERR_ARG;
  if (d->dtype == MOE_BF16 && (!fits_4g(d->T, d->d_model) || !fits_4g(d->d_ff, d->d_model) ||
                               !fits_4g(d->d_ff_shared, d->d_model)))
    return MOE_ERR_UNSUPPORTED;
  MOE_TRY(need(p->x));
  MOE_TRY(need(p->w_router));
  MOE_TRY(maybe(p->null_bias_tok));
  MOE_TRY(need(p->w_gate));
  MOE_TRY(need(p->w_up));
  MOE_TRY(need(p->w_down));
  if (d->d_ff_shared) {
    MOE_TRY(need(p->ws_gate));
    MOE_TRY(need(p->ws_up));
    MOE_TRY(need(p->ws_down));
  }
  if (d->null_kind == MOE_NULL_CONSTANT) MOE_TRY(need(p->null_value));
  MOE_TRY(need(y));
  moe_aux_out ao{};
  if (aux) ao = *aux;
  MOE_TRY(maybe(ao.logits));
  MOE_TRY(maybe(ao.topk_idx));
  MOE_TRY(maybe(ao.topk_w));
  MOE_TRY(maybe(ao.n_real));
  MOE_TRY(maybe(ao.offsets));
  MOE_TRY(maybe(ao.counts));
  MOE_TRY(maybe(ao.f));
  MOE_TRY(maybe(ao.P));
  MOE_TRY(maybe(ao.scalars));
  const LayerWs L = layer_ws(d);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  MOE_TRY(maybe(ws));
  if (d->T == 0) return MOE_OK;

  uint8_t* base = static_cast<uint8_t*>(ws);
  auto at = [&](size_t off) { return static_cast<void*>(base + off); };
  float* logits = ao.logits ? ao.logits : static_cast<float*>(at(L.logits));
  int32_t* topk_idx = ao.topk_idx ? ao.topk_idx : static_cast<int32_t*>(at(L.topk_idx));
  float* topk_w = ao.topk_w ? ao.topk_w : static_cast<float*>(at(L.topk_w));
  int32_t* n_real = ao.n_real ? ao.n_real : static_cast<int32_t*>(at(L.n_real));
  int32_t* offsets = ao.offsets ? ao.offsets : static_cast<int32_t*>(at(L.offsets));
  double* tstats = static_cast<double*>(at(L.tstats));
  int32_t* rhist = static_cast<int32_t*>(at(L.rhist));
  int32_t* perm_token = static_cast<int32_t*>(at(L.perm_token));
  int32_t* slot_pos = static_cast<int32_t*>(at(L.slot_pos));
  int32_t* permute_ws = static_cast<int32_t*>(at(L.permute));
  const bool want_stats = ao.counts || ao.f || ao.P || ao.scalars;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = d->dtype == MOE_BF16;
  const int64_t R = max_rows(d);
  const int N = d->n_experts;
  (void)hipGetLastError();

  // 1. scores, selection, weights; per-chunk expert histogram; statistics sums
  RouteArgs ra{d->T, d->d_model, N, d->n_null, d->top_k, bf16, true, p->x, p->w_router,
               p->null_bias, p->null_bias_tok, nullptr, logits, topk_idx, topk_w, n_real,
               at(L.route), permute_ws, rhist, tstats, d->null_kind};
  HIP_TRY(launch_route(ra, s));

  // 2. counting sort (histograms already written) + statistics finalisation
  AuxTiles af{tstats, rhist, ao.f, ao.P, ao.counts, ao.scalars};
  PermuteArgs pa{d->T, d->top_k, N, d->n_null, d->d_model, (int)elt_bytes(d), topk_idx, nullptr,
                 static_cast<int32_t*>(at(L.counts)), offsets, perm_token, slot_pos, nullptr,
                 permute_ws, true, want_stats ? &af : nullptr};
  HIP_TRY(launch_permute(pa, s));

  // 3. gate/up + SwiGLU: routed experts read x through perm_token (the gather), and the
  //    shared expert runs in the same launch
  const int cus = cu_count();
  const uint16_t* x16 = static_cast<const uint16_t*>(p->x);
  GemmProblem r1{x16, perm_token, d->T, offsets, N, R, static_cast<const uint16_t*>(p->w_gate),
                 static_cast<const uint16_t*>(p->w_up), d->d_ff, d->d_model, at(L.h)};
  GemmProblem s1{};
  if (d->d_ff_shared)
    s1 = GemmProblem{x16, nullptr, d->T, nullptr, 1, d->T, static_cast<const uint16_t*>(p->ws_gate),
                     static_cast<const uint16_t*>(p->ws_up), d->d_ff_shared, d->d_model, at(L.hs)};
  HIP_TRY(launch_gemm_pair(bf16, 0, r1, s1, cus, s, 2));

  // 4. down projection, routed and shared, float32 outputs
  GemmProblem r2{static_cast<const uint16_t*>(at(L.h)), nullptr, R, offsets, N, R,
                 static_cast<const uint16_t*>(p->w_down), nullptr, d->d_model, d->d_ff, at(L.yp)};
  GemmProblem s2{};
  if (d->d_ff_shared)
    s2 = GemmProblem{static_cast<const uint16_t*>(at(L.hs)), nullptr, d->T, nullptr, 1, d->T,
                     static_cast<const uint16_t*>(p->ws_down), nullptr, d->d_model,
                     d->d_ff_shared, at(L.ys)};
  HIP_TRY(launch_gemm_pair(bf16, 1, r2, s2, cus, s, 2));

  // 5. weighted combine in slot order, one rounding
  const void* nsrc = d->null_kind == MOE_NULL_COPY       ? p->x
                     : d->null_kind == MOE_NULL_CONSTANT ? p->null_value
                                                         : nullptr;
  CombineArgs ca{bf16, d->T, d->top_k, d->d_model, R, at(L.yp), slot_pos, topk_w,
                 d->d_ff_shared ? at(L.ys) : nullptr, nsrc, null_stride(d), y};
  HIP_TRY(launch_combine(ca, s));
  return MOE_OK;
}

}  // extern "C"
