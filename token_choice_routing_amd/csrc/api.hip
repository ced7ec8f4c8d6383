// C ABI of libmoe_mi355x.so: argument validation, workspace carving and kernel
// launches for the null-expert token-choice MoE layer forward. The entry points
// and their contracts are documented in include/moe.h.
#include <algorithm>
#include <cmath>
#include <atomic>
#include <mutex>

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

// A HIP error left pending on this thread by earlier work (hipPeekAtLastError) is
// reported before anything is launched and left in place for its owner to read:
// the status after a launch then names this call's own launches only.
inline moe_status no_pending_error() { return hipPeekAtLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

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
      h, hs, yp, ys, row_dst, tstats, rhist, total;
};

// Down projection and combine of the layer. With a shared expert, zero-output null
// slots and 256 x 256 tiles for both down projections (bf16), the routed outputs are
// stored token-major (slot k of token t at row t min(K, N) + k) and the shared expert's
// down projection adds them to its own output in its epilogue: no float32 shared
// output round trip and no combine launch. Otherwise the two down projections share
// one launch and the combine kernel follows. The choice depends on the dims alone, so
// the workspace size does too.
bool fused_combine(const moe_dims* d) {
  if (d->dtype != MOE_BF16 || !d->d_ff_shared || d->null_kind != MOE_NULL_ZERO) return false;
  const int64_t R = max_rows(d);
  if ((uint64_t)R * (uint64_t)d->d_model * 4u + (1u << 20) >= (1ull << 32)) return false;
  GemmProblem r2{}, s2{};
  r2.groups = d->n_experts;
  r2.max_rows = R;
  s2.groups = 1;
  s2.max_rows = d->T;
  return gemm_pair_uses_pp(r2, GemmProblem{}) && gemm_pair_uses_pp(s2, GemmProblem{});
}

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
  const bool fused = fused_combine(d);
  w.yp = take((size_t)R * d->d_model * 4);
  w.ys = take(d->d_ff_shared && !fused ? (size_t)T * d->d_model * 4 : 0);
  w.row_dst = take(fused ? (size_t)R * 4 : 0);
  const int64_t tiles = permute_nchunks(T);  // 64-token tiles of the router and the sort
  w.tstats = take((size_t)tiles * (N + 3) * 8);
  w.rhist = take((size_t)tiles * (d->top_k + 1) * 4);
  w.total = o;
  return w;
}

// Backward workspace: the forward's routing state (recomputed), the expert
// pre-activations and gradients of the routed slots, bf16 transposed weights, and the
// activations transposed per segment for the weight gradients (segments padded to 8
// columns: Rp = R + 8 N columns at most).
struct BwdWs {
  bool km;   // the data gradients read the weights K-major (no transposed copies)
  bool km2;  // the weight gradients read both operands K-major (no transposed segments)
  LayerWs fwd;
  size_t f, g, u, h, dyp, wperm, rslot, dw, ds, wdT, wguT, dh, dgu, dxp, kofs, xpT, dypT, hT, dguT, rpart, xp;
  size_t gs, us, hs, dhs, dgus, dxs, wsdT, wsguT, xT, dyT, hsT, dgusT, kofs_s, part_sd, part_sg, part_su, total;
  int64_t Rp, Tp;
  int S;  // K chunks of the shared expert's weight gradients (its K is all T tokens)
};

// The shared expert's weight gradients reduce over all T tokens: split into chunks
// (groups of one GEMM launch, summed in order afterwards), so they spread over the
// chip like the routed experts' segments. Chunks of about 1024 tokens; from 8192
// tokens on, of about 2048 (8 chunks of 16384 tokens already give 3 rounds of 256
// tiles at d = 2048, and every chunk costs a float32 partial of the whole gradient).
inline int shared_splits(int64_t T) {
  const int64_t chunk = T >= 8192 ? 2048 : 1024;
  return (int)std::max<int64_t>(1, std::min<int64_t>(T >= 8192 ? 16 : 32, (T + chunk - 1) / chunk));
}

// The backward's data-gradient products U = dy W_d and da = [dg | du] [W_g ; W_u] (and
// the shared expert's) as K-major weight problems: W_d [N][d][F] is K-major for U (K =
// d), W_g and W_u [N][F][d] are the two K halves of [W_g ; W_u] (K = 2F).
struct DgradKm {
  GemmProblem h3, hs3, a4, as4;
};
static DgradKm dgrad_kmajor(const moe_dims* d, const moe_layer_params* p, const void* dy, const int32_t* perm_token,
                            const int32_t* offsets, const void* dgu, const void* dgus, void* dh, void* dhs,
                            void* dxp, void* dxs) {
  const int64_t T = d->T, R = max_rows(d);
  const int dm = d->d_model, F = d->d_ff, Fs = d->d_ff_shared, N = d->n_experts;
  auto bf = [](const void* q) { return static_cast<const uint16_t*>(q); };
  DgradKm k{};
  k.h3 = GemmProblem{bf(dy), perm_token, T, offsets, N, R, bf(p->w_down), nullptr, F, dm, dh};
  k.h3.b_kmajor = 1;
  k.h3.k_split = dm;
  k.a4 = GemmProblem{bf(dgu), nullptr, R, offsets, N, R, bf(p->w_gate), bf(p->w_up), dm, 2 * F, dxp};
  k.a4.b_kmajor = 1;
  k.a4.k_split = F;
  if (Fs) {
    k.hs3 = GemmProblem{bf(dy), nullptr, T, nullptr, 1, T, bf(p->ws_down), nullptr, Fs, dm, dhs};
    k.hs3.b_kmajor = 1;
    k.hs3.k_split = dm;
    k.as4 = GemmProblem{bf(dgus), nullptr, T, nullptr, 1, T, bf(p->ws_gate), bf(p->ws_up), dm, 2 * Fs, dxs};
    k.as4.b_kmajor = 1;
    k.as4.k_split = Fs;
  }
  return k;
}
// Whether both data-gradient launches of a layer of these dimensions take the K-major
// form (the launcher's conditions, checked on stand-in pointers).
static bool dgrad_kmajor_ok(const moe_dims* d) {
  static const uint16_t stand_in[8] = {};
  const void* q = stand_in;
  void* o = const_cast<uint16_t*>(stand_in);
  moe_layer_params p{};
  p.w_down = p.w_gate = p.w_up = q;
  p.ws_down = p.ws_gate = p.ws_up = q;
  const int32_t* i = reinterpret_cast<const int32_t*>(stand_in);
  const DgradKm k = dgrad_kmajor(d, &p, q, i, i, q, q, o, o, o, o);
  return gemm_kmajor_ok(k.h3, k.hs3) && gemm_kmajor_ok(k.a4, k.as4);
}

// The weight gradients dW_d = dY^T h, [dW_g ; dW_u] = [dg | du]^T x_perm (and the
// shared expert's, per token chunk) with both operands K-major: K = the rows of a
// segment (chunk) of the row-major sources, which are then read in place (x_perm:
// the routed rows of x gathered in expert order).
struct WgradKm {
  GemmProblem wd, wsd, wg, wu, wsg, wsu;
};
static WgradKm wgrad_kmajor(const moe_dims* d, int S, const int32_t* offsets, const int32_t* kofs_s, const void* dyp,
                            const void* h, const void* dgu, const void* xp, const void* dy, const void* hs,
                            const void* dgus, const void* x, float* dw_down, float* dw_gate, float* dw_up,
                            float* part_sd, float* part_sg, float* part_su) {
  const int64_t T = d->T, R = max_rows(d);
  const int dm = d->d_model, F = d->d_ff, Fs = d->d_ff_shared, N = d->n_experts;
  auto bf = [](const void* q) { return static_cast<const uint16_t*>(q); };
  auto km = [](GemmProblem g) {
    g.a_kmajor = 1;
    g.b_kmajor = 1;
    return g;
  };
  WgradKm k{};
  // fields: a, a_rows, a_nrows, offsets, groups, max_rows, b0, b1, n_out, k_dim, out, k_offsets, lda, ldb, rows_per_group
  k.wd = km(GemmProblem{bf(dyp), nullptr, R, nullptr, N, (int64_t)N * dm, bf(h), nullptr, F, (int)R, dw_down,
                        offsets, dm, F, dm});
  k.wg = km(GemmProblem{bf(dgu), nullptr, R, nullptr, N, (int64_t)N * F, bf(xp), nullptr, dm, (int)R, dw_gate,
                        offsets, 2 * F, dm, F});
  k.wu = km(GemmProblem{bf(dgu) + F, nullptr, R, nullptr, N, (int64_t)N * F, bf(xp), nullptr, dm, (int)R, dw_up,
                        offsets, 2 * F, dm, F});
  if (Fs) {
    k.wsd = km(GemmProblem{bf(dy), nullptr, T, nullptr, S, (int64_t)S * dm, bf(hs), nullptr, Fs, (int)T, part_sd,
                           kofs_s, dm, Fs, dm});
    k.wsg = km(GemmProblem{bf(dgus), nullptr, T, nullptr, S, (int64_t)S * Fs, bf(x), nullptr, dm, (int)T, part_sg,
                           kofs_s, 2 * Fs, dm, Fs});
    k.wsu = km(GemmProblem{bf(dgus) + Fs, nullptr, T, nullptr, S, (int64_t)S * Fs, bf(x), nullptr, dm, (int)T,
                           part_su, kofs_s, 2 * Fs, dm, Fs});
  }
  return k;
}
static bool wgrad_kmajor_ok(const moe_dims* d) {
  static const uint16_t stand_in[8] = {};
  const void* q = stand_in;
  float* o = reinterpret_cast<float*>(const_cast<uint16_t*>(stand_in));
  const int32_t* i = reinterpret_cast<const int32_t*>(stand_in);
  const WgradKm k = wgrad_kmajor(d, shared_splits(d->T), i, i, q, q, q, q, q, q, q, q, o, o, o, o, o, o);
  return gemm_kmajor_ok(k.wd, k.wsd) && gemm_kmajor_ok(k.wg, k.wu) && gemm_kmajor_ok(k.wsg, k.wsu);
}

BwdWs bwd_ws(const moe_dims* d) {
  BwdWs w{};
  w.km = dgrad_kmajor_ok(d);
  w.km2 = wgrad_kmajor_ok(d);
  w.fwd = layer_ws(d);
  const int64_t T = d->T, R = max_rows(d), dm = d->d_model, F = d->d_ff, Fs = d->d_ff_shared;
  const int N = d->n_experts, M = d->n_null;
  w.Rp = R + 8 * (int64_t)N;
  w.Tp = (T + 7) & ~int64_t(7);
  size_t o = w.fwd.total;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  w.f = take((size_t)(N + M) * 4);
  w.g = take((size_t)R * F * 4);
  w.u = take((size_t)R * F * 4);
  w.h = take((size_t)R * F * 2);
  w.dyp = take((size_t)R * dm * 2);
  w.wperm = take((size_t)R * 4);
  w.rslot = take((size_t)R * 4);
  w.dw = take((size_t)T * d->top_k * 4);
  w.ds = take((size_t)T * (N + 1) * 4);
  w.wdT = w.km ? 0 : take((size_t)N * F * dm * 2);
  w.wguT = w.km ? 0 : take((size_t)N * dm * 2 * F * 2);
  w.dh = take((size_t)R * F * 4);
  w.dgu = take((size_t)R * 2 * F * 2);
  w.dxp = take((size_t)R * dm * 4);
  w.kofs = take((size_t)(N + 1) * 4);
  w.xpT = w.km2 ? 0 : take((size_t)dm * w.Rp * 2);
  w.dypT = w.km2 ? 0 : take((size_t)dm * w.Rp * 2);
  w.hT = w.km2 ? 0 : take((size_t)F * w.Rp * 2);
  w.dguT = w.km2 ? 0 : take((size_t)2 * F * w.Rp * 2);
  w.xp = w.km2 ? take((size_t)R * dm * 2) : 0;
  w.rpart = take(router_wgrad_ws_bytes(T, N + 1, (int)dm));
  if (Fs) {
    w.gs = take((size_t)T * Fs * 4);
    w.us = take((size_t)T * Fs * 4);
    w.hs = take((size_t)T * Fs * 2);
    w.dhs = take((size_t)T * Fs * 4);
    w.dgus = take((size_t)T * 2 * Fs * 2);
    w.dxs = take((size_t)T * dm * 4);
    w.wsdT = w.km ? 0 : take((size_t)Fs * dm * 2);
    w.wsguT = w.km ? 0 : take((size_t)dm * 2 * Fs * 2);
    w.xT = w.km2 ? 0 : take((size_t)dm * w.Tp * 2);
    w.dyT = w.km2 ? 0 : take((size_t)dm * w.Tp * 2);
    w.hsT = w.km2 ? 0 : take((size_t)Fs * w.Tp * 2);
    w.dgusT = w.km2 ? 0 : take((size_t)2 * Fs * w.Tp * 2);
    w.S = shared_splits(T);
    w.kofs_s = take((size_t)(w.S + 1) * 4);
    w.part_sd = take((size_t)w.S * dm * Fs * 4);
    w.part_sg = take((size_t)w.S * Fs * dm * 4);
    w.part_su = take((size_t)w.S * Fs * dm * 4);
  }
  w.total = o;
  return w;
}

}  // namespace

// Workspace of moe_layer_forward_noalloc: one static array per device, held until the
// process ends. Host code never uses this name as an address (on the host it is a
// stand-in symbol); the device address comes from hipGetSymbolAddress, once per
// device, and only that address reaches kernels.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_MAX_WS_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array (looked up on first use).
moe_status noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument (dimension or NULL pointer)";
    case MOE_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_UNSUPPORTED: return "dimensions outside this library's limits";
    case MOE_ERR_HIP: return "HIP launch or runtime error";
    case MOE_ERR_NONFINITE: return "non-finite input (NaN or infinity)";
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
    case MOE_WS_BACKWARD: return d->dtype == MOE_BF16 ? bwd_ws(d).total : 0;
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
  MOE_TRY(no_pending_error());
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
  MOE_TRY(no_pending_error());
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
  MOE_TRY(no_pending_error());
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
  MOE_TRY(no_pending_error());
  GemmProblem g{static_cast<const uint16_t*>(a), nullptr, rows, offsets, n_groups, rows,
                static_cast<const uint16_t*>(b0),
                op == MOE_GEMM_GATE_UP ? static_cast<const uint16_t*>(b1) : nullptr, n_out, k_dim,
                out};
  HIP_TRY(launch_gemm_pair(d->dtype == MOE_BF16, op == MOE_GEMM_DOWN ? 2 : 0, g, GemmProblem{}, cu_count(),
                           static_cast<hipStream_t>(stream), offsets ? 0 : 1));
  return MOE_OK;
}

// The layer's gate/up + SwiGLU launch: routed rows of x read through perm_token and,
// with a shared expert, every token through the shared expert, as one launch.
static hipError_t launch_layer_gate_up(const moe_dims* d, const void* x, const int32_t* perm_token,
                                       const int32_t* offsets, const void* w_gate, const void* w_up,
                                       const void* ws_gate, const void* ws_up, void* h, void* hs,
                                       hipStream_t s) {
  const uint16_t* x16 = static_cast<const uint16_t*>(x);
  GemmProblem r1{x16, perm_token, d->T, offsets, d->n_experts, max_rows(d), static_cast<const uint16_t*>(w_gate),
                 static_cast<const uint16_t*>(w_up), d->d_ff, d->d_model, h};
  GemmProblem s1{};
  if (d->d_ff_shared)
    s1 = GemmProblem{x16, nullptr, d->T, nullptr, 1, d->T, static_cast<const uint16_t*>(ws_gate),
                     static_cast<const uint16_t*>(ws_up), d->d_ff_shared, d->d_model, hs};
  return launch_gemm_pair(d->dtype == MOE_BF16, 0, r1, s1, cu_count(), s, 2);
}

// Per-token stride (elements) of the rows a null slot adds: x for copy experts,
// the one vector v for constant experts.
inline int64_t null_stride(const moe_dims* d) { return d->null_kind == MOE_NULL_COPY ? d->d_model : 0; }

moe_status moe_expert_gate_up(const moe_dims* d, const void* x, const int32_t* perm_token,
                              const int32_t* offsets, const void* w_gate, const void* w_up,
                              const void* ws_gate, const void* ws_up, void* h, void* hs,
                              moe_stream stream) {
  MOE_TRY(check_dims(d));
  if (d->dtype == MOE_BF16 && (!fits_4g(d->T, d->d_model) || !fits_4g(d->d_ff, d->d_model) ||
                               !fits_4g(d->d_ff_shared, d->d_model)))
    return MOE_ERR_UNSUPPORTED;
  MOE_TRY(need(x));
  MOE_TRY(need(perm_token));
  MOE_TRY(need(offsets));
  MOE_TRY(need(w_gate));
  MOE_TRY(need(w_up));
  MOE_TRY(need(h));
  if (d->d_ff_shared) {
    MOE_TRY(need(ws_gate));
    MOE_TRY(need(ws_up));
    MOE_TRY(need(hs));
  }
  if (d->T == 0) return MOE_OK;
  MOE_TRY(no_pending_error());
  HIP_TRY(launch_layer_gate_up(d, x, perm_token, offsets, w_gate, w_up, ws_gate, ws_up, h, hs,
                               static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

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
  MOE_TRY(no_pending_error());
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
  MOE_TRY(no_pending_error());
  AuxArgs a{d->T, d->n_experts, d->n_null, d->top_k, logits, topk_idx, f, P, counts, scalars, ws};
  HIP_TRY(launch_aux(a, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

static moe_status layer_down_combine(const moe_dims* d, const moe_layer_params* p, void* y, const LayerWs& L,
                                     uint8_t* base, const int32_t* offsets, const int32_t* slot_pos,
                                     const float* topk_w, const int32_t* n_real, const int32_t* row_dst,
                                     hipStream_t s);

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
  const int N = d->n_experts;
  MOE_TRY(no_pending_error());

  // 1. scores, selection, weights; per-chunk expert histogram; statistics sums
  RouteArgs ra{d->T, d->d_model, N, d->n_null, d->top_k, bf16, true, p->x, p->w_router,
               p->null_bias, p->null_bias_tok, nullptr, logits, topk_idx, topk_w, n_real,
               at(L.route), permute_ws, rhist, tstats, d->null_kind};
  // 2. counting sort (histograms already written) + statistics finalisation; a few
  //    tokens take both steps in one workgroup
  AuxTiles af{tstats, rhist, ao.f, ao.P, ao.counts, ao.scalars};
  const bool fused = fused_combine(d);
  int32_t* row_dst = fused ? static_cast<int32_t*>(at(L.row_dst)) : nullptr;
  PermuteArgs pa{d->T, d->top_k, N, d->n_null, d->d_model, (int)elt_bytes(d), topk_idx, nullptr,
                 static_cast<int32_t*>(at(L.counts)), offsets, perm_token, slot_pos, nullptr,
                 permute_ws, true, want_stats ? &af : nullptr, row_dst};
  if (route_small_ok(ra)) {
    HIP_TRY(launch_route_small(ra, &pa, s));
  } else {
    HIP_TRY(launch_route(ra, s));
    HIP_TRY(launch_permute(pa, s));
  }

  // 3. gate/up + SwiGLU: routed experts read x through perm_token (the gather), and the
  //    shared expert runs in the same launch
  HIP_TRY(launch_layer_gate_up(d, p->x, perm_token, offsets, p->w_gate, p->w_up, p->ws_gate, p->ws_up,
                               at(L.h), at(L.hs), s));

  return layer_down_combine(d, p, y, L, base, offsets, slot_pos, topk_w, n_real, row_dst, s);
}

// Steps 4-5 of the layer forward: the down projections (routed and shared, from h and
// hs in L: IEEE half in bf16 layers, float32 in float32 ones) and the weighted combine
// into y, or, given a row_dst (the fused combine), the routed outputs token-major and
// the combine in the shared expert's down projection.
static moe_status layer_down_combine(const moe_dims* d, const moe_layer_params* p, void* y, const LayerWs& L,
                                     uint8_t* base, const int32_t* offsets, const int32_t* slot_pos,
                                     const float* topk_w, const int32_t* n_real, const int32_t* row_dst,
                                     hipStream_t s) {
  auto at = [&](size_t off) { return static_cast<void*>(base + off); };
  const bool bf16 = d->dtype == MOE_BF16, fused = row_dst != nullptr;
  const int64_t R = max_rows(d);
  const int N = d->n_experts;
  const int cus = cu_count();
  // 4. down projection, routed and shared, float32 outputs
  GemmProblem r2{static_cast<const uint16_t*>(at(L.h)), nullptr, R, offsets, N, R,
                 static_cast<const uint16_t*>(p->w_down), nullptr, d->d_model, d->d_ff, at(L.yp)};
  GemmProblem s2{};
  if (d->d_ff_shared)
    s2 = GemmProblem{static_cast<const uint16_t*>(at(L.hs)), nullptr, d->T, nullptr, 1, d->T,
                     static_cast<const uint16_t*>(p->ws_down), nullptr, d->d_model,
                     d->d_ff_shared, at(L.ys)};
  if (fused) {
    // routed outputs token-major, then the shared expert's down projection with the
    // combine in its epilogue (y_t = Ys_t + sum over the token's reals of w yp, in slot
    // order, rounded once)
    r2.out_rows = row_dst;
    HIP_TRY(launch_gemm_pair(bf16, 2, r2, GemmProblem{}, cus, s, 2));
    s2.out = y;
    s2.comb_z = static_cast<const float*>(at(L.yp));
    s2.comb_n = n_real;
    s2.comb_w = topk_w;
    s2.comb_k = d->top_k;
    s2.comb_kr = std::min(d->top_k, N);
    HIP_TRY(launch_gemm_pair(bf16, 3, s2, GemmProblem{}, cus, s, 2));
    return MOE_OK;
  }
  HIP_TRY(launch_gemm_pair(bf16, 2, r2, s2, cus, s, 2));

  // 5. weighted combine in slot order, one rounding
  const void* nsrc = d->null_kind == MOE_NULL_COPY       ? p->x
                     : d->null_kind == MOE_NULL_CONSTANT ? p->null_value
                                                         : nullptr;
  CombineArgs ca{bf16, d->T, d->top_k, d->d_model, R, at(L.yp), slot_pos, topk_w,
                 d->d_ff_shared ? at(L.ys) : nullptr, nsrc, null_stride(d), y};
  HIP_TRY(launch_combine(ca, s));
  return MOE_OK;
}

moe_status moe_layer_forward_noalloc(const moe_dims* d, const moe_layer_params* p, void* y,
                                     const moe_aux_out* aux, moe_stream stream) {
  MOE_TRY(check_dims(d));
  if (!p) return MOE_ERR_ARG;
  if (layer_ws(d).total > MOE_NOALLOC_MAX_WS_BYTES) return MOE_ERR_UNSUPPORTED;
  if (d->T == 0) return moe_layer_forward(d, p, y, aux, nullptr, 0, stream);
  void* ws = nullptr;
  MOE_TRY(noalloc_scratch(&ws));
  return moe_layer_forward(d, p, y, aux, ws, MOE_NOALLOC_MAX_WS_BYTES, stream);
}

moe_status moe_validate_inputs(const moe_dims* d, const moe_layer_params* p, void* ws, size_t ws_bytes,
                               moe_stream stream) {
  MOE_TRY(check_dims(d));
  if (!p) return MOE_ERR_ARG;
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
  if (!ws || ws_bytes < 16) return MOE_ERR_WORKSPACE;
  MOE_TRY(need(ws));
  if (std::isnan(p->null_bias)) return MOE_ERR_NONFINITE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = d->dtype == MOE_BF16;
  const int64_t T = d->T, dm = d->d_model, N = d->n_experts, F = d->d_ff, Fs = d->d_ff_shared;
  int32_t* count = static_cast<int32_t*>(ws);
  MOE_TRY(no_pending_error());
  HIP_TRY(launch_zero_count(count, s));
  HIP_TRY(launch_count_nonfinite(p->x, T * dm, bf16, false, count, s));
  HIP_TRY(launch_count_nonfinite(p->w_router, (N + 1) * dm, false, false, count, s));
  HIP_TRY(launch_count_nonfinite(p->null_bias_tok, T, false, true, count, s));
  HIP_TRY(launch_count_nonfinite(p->w_gate, N * F * dm, bf16, false, count, s));
  HIP_TRY(launch_count_nonfinite(p->w_up, N * F * dm, bf16, false, count, s));
  HIP_TRY(launch_count_nonfinite(p->w_down, N * dm * F, bf16, false, count, s));
  if (Fs) {
    HIP_TRY(launch_count_nonfinite(p->ws_gate, Fs * dm, bf16, false, count, s));
    HIP_TRY(launch_count_nonfinite(p->ws_up, Fs * dm, bf16, false, count, s));
    HIP_TRY(launch_count_nonfinite(p->ws_down, dm * Fs, bf16, false, count, s));
  }
  if (d->null_kind == MOE_NULL_CONSTANT) HIP_TRY(launch_count_nonfinite(p->null_value, dm, bf16, false, count, s));
  int32_t host = 0;
  HIP_TRY(hipMemcpyAsync(&host, count, sizeof(host), hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  return host ? MOE_ERR_NONFINITE : MOE_OK;
}

// Checks shared by the backward entry points and the training forward: dims, the
// layer's parameters and the backward workspace.
static moe_status check_backward_args(const moe_dims* d, const moe_layer_params* p, const BwdWs& W, void* ws,
                                      size_t ws_bytes) {
  if (!p) return MOE_ERR_ARG;
  if (d->dtype != MOE_BF16 || d->null_kind != MOE_NULL_ZERO) return MOE_ERR_UNSUPPORTED;
  const int64_t T = d->T, dm = d->d_model, F = d->d_ff, Fs = d->d_ff_shared;
  // bf16 operands at 32-bit byte offsets (transposed activations: rows of Rp columns)
  if (!fits_4g(T, dm) || !fits_4g(2 * F, dm) || !fits_4g(2 * std::max<int64_t>(F, Fs), W.Rp) ||
      !fits_4g(dm, W.Rp) || !fits_4g(Fs, W.Tp) || !fits_4g(dm, 2 * F) || !fits_4g(dm, W.Tp))
    return MOE_ERR_UNSUPPORTED;
  MOE_TRY(need(p->x));
  MOE_TRY(need(p->w_router));
  MOE_TRY(maybe(p->null_bias_tok));
  MOE_TRY(need(p->w_gate));
  MOE_TRY(need(p->w_up));
  MOE_TRY(need(p->w_down));
  if (Fs) {
    MOE_TRY(need(p->ws_gate));
    MOE_TRY(need(p->ws_up));
    MOE_TRY(need(p->ws_down));
  }
  if (!ws || ws_bytes < W.total) return MOE_ERR_WORKSPACE;
  MOE_TRY(need(ws));
  return MOE_OK;
}

// Whether the expert pre-activations come from the keep-mode launch (g and u stored in
// IEEE half) rather than plain GEMMs (float32): the 256 x 256 tiles take the routed and
// the shared gate/up problems (a function of the dims).
static bool keep_preacts(const moe_dims* d) {
  static const int32_t one = 1;  // a non-null row index and offsets pointer for the shape test
  GemmProblem r{}, sh{};
  r.a_rows = &one;
  r.a_nrows = d->T;
  r.offsets = &one;
  r.groups = d->n_experts;
  r.max_rows = max_rows(d);
  r.n_out = d->d_ff;
  r.k_dim = d->d_model;
  if (d->d_ff_shared) {
    sh.groups = 1;
    sh.max_rows = d->T;
    sh.n_out = d->d_ff_shared;
    sh.k_dim = d->d_model;
  }
  return gemm_pair_uses_pp(r, sh);
}

// The layer state the backward works from, written into the backward workspace:
// routing (logits, selection, weights), the permutation, the pool counts f, and the
// expert pre-activations g, u (float32) and h (bf16), routed and shared. With fwd set
// (the training forward) also the half-precision h and hs of the layer forward's
// layout, the row redirect of the fused combine, and the caller's statistics outputs
// (P, counts, scalars).
static moe_status backward_state(const moe_dims* d, const moe_layer_params* p, const BwdWs& W, uint8_t* base,
                                 hipStream_t s, const moe_aux_out* fwd) {
  auto at = [&](size_t off) { return static_cast<void*>(base + off); };
  auto fp = [&](size_t off) { return static_cast<float*>(at(off)); };
  auto ip = [&](size_t off) { return static_cast<int32_t*>(at(off)); };
  const LayerWs& L = W.fwd;
  const int64_t T = d->T, dm = d->d_model, F = d->d_ff, Fs = d->d_ff_shared;
  const int64_t R = max_rows(d);
  const int N = d->n_experts, M = d->n_null, K = d->top_k;
  const int cus = cu_count();
  const uint16_t* x16 = static_cast<const uint16_t*>(p->x);
  int32_t* offsets = ip(L.offsets);
  int32_t* perm_token = ip(L.perm_token);
  int32_t* permute_ws = ip(L.permute);
  // 1-2. routing, permutation and pool counts f
  RouteArgs ra{T, d->d_model, N, M, K, true, true, p->x, p->w_router, p->null_bias, p->null_bias_tok,
               nullptr, fp(L.logits), ip(L.topk_idx), fp(L.topk_w), ip(L.n_real), at(L.route), permute_ws,
               ip(L.rhist), static_cast<double*>(at(L.tstats)), d->null_kind};
  HIP_TRY(launch_route(ra, s));
  AuxTiles af{static_cast<double*>(at(L.tstats)), ip(L.rhist), fp(W.f), fwd ? fwd->P : nullptr,
              fwd ? fwd->counts : nullptr, fwd ? fwd->scalars : nullptr};
  int32_t* row_dst = fwd && fused_combine(d) ? ip(L.row_dst) : nullptr;
  PermuteArgs pa{T, K, N, M, d->d_model, 2, ip(L.topk_idx), nullptr, ip(L.counts), offsets, perm_token,
                 ip(L.slot_pos), nullptr, permute_ws, true, &af, row_dst};
  HIP_TRY(launch_permute(pa, s));
  // 3. expert pre-activations g = x W_g^T, u = x W_u^T (float32) and h = silu(g) u (bf16):
  // routed and shared in one launch whose epilogue keeps g and u and writes h, when the
  // 256 x 256 tiles take both; else g and u by plain GEMMs and h by its own kernel
  GemmProblem gk{x16, perm_token, T, offsets, N, R, static_cast<const uint16_t*>(p->w_gate),
                 static_cast<const uint16_t*>(p->w_up), (int)F, (int)dm, at(W.h)};
  gk.keep_g = at(W.g);
  gk.keep_u = at(W.u);
  GemmProblem gsk{};
  if (Fs) {
    gsk = GemmProblem{x16, nullptr, T, nullptr, 1, T, static_cast<const uint16_t*>(p->ws_gate),
                      static_cast<const uint16_t*>(p->ws_up), (int)Fs, (int)dm, at(W.hs)};
    gsk.keep_g = at(W.gs);
    gsk.keep_u = at(W.us);
  }
  // (the same test as gemm_pair_uses_pp(gk, gsk); the gradient step reads g and u by it)
  const bool keep = keep_preacts(d);
  if (keep && fwd) {
    // the forward's half-precision h (and hs) from the same epilogue: bit for bit what the
    // layer forward's gate/up launch writes
    gk.keep_h16 = at(L.h);
    if (Fs) gsk.keep_h16 = at(L.hs);
  }
  if (keep) HIP_TRY(launch_gemm_pair(true, 4, gk, gsk, cus, s, fwd ? 2 : 3));
  if (!keep && fwd)
    HIP_TRY(launch_layer_gate_up(d, p->x, perm_token, offsets, p->w_gate, p->w_up, p->ws_gate, p->ws_up, at(L.h),
                                 at(L.hs), s));
  GemmProblem g1{x16, perm_token, T, offsets, N, R, static_cast<const uint16_t*>(p->w_gate), nullptr,
                 (int)F, (int)dm, at(W.g)};
  GemmProblem u1{x16, perm_token, T, offsets, N, R, static_cast<const uint16_t*>(p->w_up), nullptr,
                 (int)F, (int)dm, at(W.u)};
  if (!keep) {
    HIP_TRY(launch_gemm_pair(true, 1, g1, u1, cus, s, 3));
    HIP_TRY(launch_swiglu_h(fp(W.g), fp(W.u), offsets, N, R, (int)F, at(W.h), s));
  }
  if (Fs && !keep) {
    GemmProblem gs{x16, nullptr, T, nullptr, 1, T, static_cast<const uint16_t*>(p->ws_gate), nullptr, (int)Fs,
                   (int)dm, at(W.gs)};
    GemmProblem us{x16, nullptr, T, nullptr, 1, T, static_cast<const uint16_t*>(p->ws_up), nullptr, (int)Fs,
                   (int)dm, at(W.us)};
    HIP_TRY(launch_gemm_pair(true, 1, gs, us, cus, s, 3));
    HIP_TRY(launch_swiglu_h(fp(W.gs), fp(W.us), nullptr, 1, T, (int)Fs, at(W.hs), s));
  }
  return MOE_OK;
}

// The backward from the state in the workspace: recomputed first (recompute), or left
// there by moe_layer_forward_train.
static moe_status layer_backward(const moe_dims* d, const moe_layer_params* p, const void* dy, float alpha,
                                 float beta, const moe_layer_grads* gr, void* ws, size_t ws_bytes, moe_stream stream,
                                 bool recompute) {
  MOE_TRY(check_dims(d));
  if (!p || !gr) return MOE_ERR_ARG;
  const BwdWs W = bwd_ws(d);
  MOE_TRY(check_backward_args(d, p, W, ws, ws_bytes));
  const int64_t T = d->T, dm = d->d_model, F = d->d_ff, Fs = d->d_ff_shared;
  if (Fs) {
    MOE_TRY(need(gr->dws_gate));
    MOE_TRY(need(gr->dws_up));
    MOE_TRY(need(gr->dws_down));
  }
  MOE_TRY(need(dy));
  MOE_TRY(need(gr->dx));
  MOE_TRY(need(gr->dw_router));
  MOE_TRY(need(gr->dw_gate));
  MOE_TRY(need(gr->dw_up));
  MOE_TRY(need(gr->dw_down));
  if (T == 0) return MOE_OK;

  uint8_t* base = static_cast<uint8_t*>(ws);
  auto at = [&](size_t off) { return static_cast<void*>(base + off); };
  auto fp = [&](size_t off) { return static_cast<float*>(at(off)); };
  auto ip = [&](size_t off) { return static_cast<int32_t*>(at(off)); };
  const LayerWs& L = W.fwd;
  float* logits = fp(L.logits);
  int32_t* topk_idx = ip(L.topk_idx);
  float* topk_w = fp(L.topk_w);
  int32_t* offsets = ip(L.offsets);
  int32_t* perm_token = ip(L.perm_token);
  int32_t* slot_pos = ip(L.slot_pos);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t R = max_rows(d);
  const int N = d->n_experts, M = d->n_null, K = d->top_k;
  const int cus = cu_count();
  auto bf = [&](size_t off) { return static_cast<const uint16_t*>(at(off)); };
  MOE_TRY(no_pending_error());

  // 1-3. routing, permutation, pool counts and expert pre-activations
  if (recompute) MOE_TRY(backward_state(d, p, W, base, s, nullptr));

  // 4. per real slot: its expert row's dY = g dy (bf16, for dW_down), g and slot index
  HIP_TRY(launch_slot_rows(dy, slot_pos, topk_w, T, K, (int)dm, R, at(W.dyp), fp(W.wperm), ip(W.rslot), fp(W.dw),
                           s));

  // 5. the data gradients' weights: read K-major in place when the launches allow it
  // (W.km), else transposed copies: W_d^T [N][F][d]; [W_g ; W_u]^T [N][d][2F]
  const DgradKm km = dgrad_kmajor(d, p, dy, perm_token, offsets, at(W.dgu), Fs ? at(W.dgus) : nullptr, at(W.dh),
                                  Fs ? at(W.dhs) : nullptr, at(W.dxp), Fs ? at(W.dxs) : nullptr);
  if (!W.km) {
    HIP_TRY(launch_transpose(p->w_down, N, dm, F, at(W.wdT), dm, 0, F * dm, s));
    HIP_TRY(launch_transpose(p->w_gate, N, F, dm, at(W.wguT), 2 * F, 0, dm * 2 * F, s));
    HIP_TRY(launch_transpose(p->w_up, N, F, dm, at(W.wguT), 2 * F, F, dm * 2 * F, s));
    if (Fs) {
      HIP_TRY(launch_transpose(p->ws_down, 1, dm, Fs, at(W.wsdT), dm, 0, 0, s));
      HIP_TRY(launch_transpose(p->ws_gate, 1, Fs, dm, at(W.wsguT), 2 * Fs, 0, 0, s));
      HIP_TRY(launch_transpose(p->ws_up, 1, Fs, dm, at(W.wsguT), 2 * Fs, Fs, 0, s));
    }
  }

  // 6. U = dy W_d on the routed rows (dy read through perm_token) and dh_s = dy W_sd;
  // then per routed row dg = <U, h> (the slot's weight gradient, so the expert output
  // Y is never recomputed) and the SwiGLU backward of dh = g U; the shared expert's
  // SwiGLU backward; then the router backward (ds), which needs every dg
  GemmProblem h3{static_cast<const uint16_t*>(dy), perm_token, T, offsets, N, R, bf(W.wdT), nullptr, (int)F,
                 (int)dm, at(W.dh)};
  GemmProblem hs3{};
  if (Fs)
    hs3 = GemmProblem{static_cast<const uint16_t*>(dy), nullptr, T, nullptr, 1, T, bf(W.wsdT), nullptr, (int)Fs,
                      (int)dm, at(W.dhs)};
  if (W.km) {
    h3 = km.h3;
    hs3 = km.hs3;
  }
  HIP_TRY(launch_gemm_pair(true, 1, h3, hs3, cus, s, 3));
  const bool g16 = keep_preacts(d);
  HIP_TRY(launch_swiglu_bwd_routed(at(W.g), at(W.u), g16, fp(W.dh), at(W.h), fp(W.wperm), ip(W.rslot), offsets, N, R,
                                    (int)F, at(W.dgu), fp(W.dw), s));
  if (Fs) HIP_TRY(launch_swiglu_bwd(at(W.gs), at(W.us), g16, fp(W.dhs), nullptr, 1, T, (int)Fs, at(W.dgus), s));
  HIP_TRY(launch_router_bwd(logits, topk_idx, topk_w, fp(W.dw), fp(W.f), T, N, M, K, alpha, beta, fp(W.ds), s));

  // 7. da = [dg | du] [W_g ; W_u]: routed rows and shared rows (float32)
  GemmProblem a4{bf(W.dgu), nullptr, R, offsets, N, R, bf(W.wguT), nullptr, (int)dm, (int)(2 * F), at(W.dxp)};
  GemmProblem as4{};
  if (Fs)
    as4 = GemmProblem{bf(W.dgus), nullptr, T, nullptr, 1, T, bf(W.wsguT), nullptr, (int)dm, (int)(2 * Fs),
                      at(W.dxs)};
  if (W.km) {
    a4 = km.a4;
    as4 = km.as4;
  }
  HIP_TRY(launch_gemm_pair(true, 1, a4, as4, cus, s, 3));

  // 8. dx = sum over the token's slots of da + shared da + ds W_r; dW_r = ds^T x
  HIP_TRY(launch_scatter_dx(fp(W.dxp), slot_pos, K, R, Fs ? fp(W.dxs) : nullptr, fp(W.ds), p->w_router, N + 1,
                            (int)dm, T, gr->dx, s));
  HIP_TRY(launch_router_wgrad(fp(W.ds), p->x, T, N + 1, (int)dm, fp(W.rpart), gr->dw_router, s));

  // 9. weight gradients, K = the rows of a segment: both operands read K-major in place
  // when the launches allow it (W.km2), else transposed per segment
  if (W.km2) {
    const int S = W.S;
    int32_t* kofs_s = Fs ? ip(W.kofs_s) : nullptr;
    HIP_TRY(launch_gather_slots(p->x, perm_token, T, offsets, N, R, (int)dm, at(W.xp), s));
    if (Fs) HIP_TRY(launch_split_offsets(T, S, kofs_s, s));
    const WgradKm k = wgrad_kmajor(d, S, offsets, kofs_s, at(W.dyp), at(W.h), at(W.dgu), at(W.xp), dy,
                                   Fs ? at(W.hs) : nullptr, Fs ? at(W.dgus) : nullptr, p->x, gr->dw_down,
                                   gr->dw_gate, gr->dw_up, Fs ? fp(W.part_sd) : nullptr,
                                   Fs ? fp(W.part_sg) : nullptr, Fs ? fp(W.part_su) : nullptr);
    HIP_TRY(launch_gemm_pair(true, 1, k.wd, k.wsd, cus, s, 3));
    if (Fs) HIP_TRY(launch_sum_partials(fp(W.part_sd), S, dm * Fs, gr->dws_down, s));
    HIP_TRY(launch_gemm_pair(true, 1, k.wg, k.wu, cus, s, 3));
    if (Fs) {
      HIP_TRY(launch_gemm_pair(true, 1, k.wsg, k.wsu, cus, s, 3));
      HIP_TRY(launch_sum_partials(fp(W.part_sg), S, Fs * dm, gr->dws_gate, s));
      HIP_TRY(launch_sum_partials(fp(W.part_su), S, Fs * dm, gr->dws_up, s));
    }
    return MOE_OK;
  }
  int32_t* kofs = ip(W.kofs);
  HIP_TRY(launch_pad_offsets(offsets, N, R, kofs, s));
  HIP_TRY(launch_transpose_segments(p->x, perm_token, T, offsets, kofs, N, R, dm, at(W.xpT), W.Rp, s));
  HIP_TRY(launch_transpose_segments(at(W.dyp), nullptr, R, offsets, kofs, N, R, dm, at(W.dypT), W.Rp, s));
  HIP_TRY(launch_transpose_segments(at(W.h), nullptr, R, offsets, kofs, N, R, F, at(W.hT), W.Rp, s));
  HIP_TRY(launch_transpose_segments(at(W.dgu), nullptr, R, offsets, kofs, N, R, 2 * F, at(W.dguT), W.Rp, s));
  // dW_d[e] = dY_e^T h_e: rows d of dY^T, columns F of h^T
  GemmProblem wd{bf(W.dypT), nullptr, dm, nullptr, N, N * dm, bf(W.hT), nullptr, (int)F, (int)W.Rp, gr->dw_down,
                 kofs, W.Rp, W.Rp, (int)dm};
  GemmProblem wsd{};
  const int S = W.S;
  int32_t* kofs_s = Fs ? ip(W.kofs_s) : nullptr;
  if (Fs) {
    HIP_TRY(launch_transpose_segments(p->x, nullptr, T, nullptr, nullptr, 1, T, dm, at(W.xT), W.Tp, s));
    HIP_TRY(launch_transpose_segments(dy, nullptr, T, nullptr, nullptr, 1, T, dm, at(W.dyT), W.Tp, s));
    HIP_TRY(launch_transpose_segments(at(W.hs), nullptr, T, nullptr, nullptr, 1, T, Fs, at(W.hsT), W.Tp, s));
    HIP_TRY(launch_transpose_segments(at(W.dgus), nullptr, T, nullptr, nullptr, 1, T, 2 * Fs, at(W.dgusT), W.Tp, s));
    HIP_TRY(launch_split_offsets(T, S, kofs_s, s));
    // partial dW_sd per token chunk (groups = chunks, each [d][Fs])
    wsd = GemmProblem{bf(W.dyT), nullptr, dm, nullptr, S, S * dm, bf(W.hsT), nullptr, (int)Fs, (int)W.Tp,
                      at(W.part_sd), kofs_s, W.Tp, W.Tp, (int)dm};
  }
  HIP_TRY(launch_gemm_pair(true, 1, wd, wsd, cus, s, 3));
  if (Fs) HIP_TRY(launch_sum_partials(fp(W.part_sd), S, dm * Fs, gr->dws_down, s));
  // dW_g[e] = dg_e^T x_e, dW_u[e] = du_e^T x_e (rows F and F..2F of [dg | du]^T)
  GemmProblem wg{bf(W.dguT), nullptr, F, nullptr, N, N * F, bf(W.xpT), nullptr, (int)dm, (int)W.Rp, gr->dw_gate,
                 kofs, W.Rp, W.Rp, (int)F};
  GemmProblem wu{bf(W.dguT) + F * W.Rp, nullptr, F, nullptr, N, N * F, bf(W.xpT), nullptr, (int)dm, (int)W.Rp,
                 gr->dw_up, kofs, W.Rp, W.Rp, (int)F};
  HIP_TRY(launch_gemm_pair(true, 1, wg, wu, cus, s, 3));
  if (Fs) {
    GemmProblem wsg{bf(W.dgusT), nullptr, Fs, nullptr, S, S * Fs, bf(W.xT), nullptr, (int)dm, (int)W.Tp,
                    at(W.part_sg), kofs_s, W.Tp, W.Tp, (int)Fs};
    GemmProblem wsu{bf(W.dgusT) + Fs * W.Tp, nullptr, Fs, nullptr, S, S * Fs, bf(W.xT), nullptr, (int)dm,
                    (int)W.Tp, at(W.part_su), kofs_s, W.Tp, W.Tp, (int)Fs};
    HIP_TRY(launch_gemm_pair(true, 1, wsg, wsu, cus, s, 3));
    HIP_TRY(launch_sum_partials(fp(W.part_sg), S, Fs * dm, gr->dws_gate, s));
    HIP_TRY(launch_sum_partials(fp(W.part_su), S, Fs * dm, gr->dws_up, s));
  }
  return MOE_OK;
}

moe_status moe_layer_backward(const moe_dims* d, const moe_layer_params* p, const void* dy, float alpha,
                              float beta, const moe_layer_grads* gr, void* ws, size_t ws_bytes,
                              moe_stream stream) {
  return layer_backward(d, p, dy, alpha, beta, gr, ws, ws_bytes, stream, true);
}

moe_status moe_layer_backward_saved(const moe_dims* d, const moe_layer_params* p, const void* dy, float alpha,
                                    float beta, const moe_layer_grads* gr, void* ws, size_t ws_bytes,
                                    moe_stream stream) {
  return layer_backward(d, p, dy, alpha, beta, gr, ws, ws_bytes, stream, false);
}

moe_status moe_layer_forward_train(const moe_dims* d, const moe_layer_params* p, void* y, const moe_aux_out* aux,
                                   void* ws, size_t ws_bytes, moe_stream stream) {
  MOE_TRY(check_dims(d));
  if (!p) return MOE_ERR_ARG;
  const BwdWs W = bwd_ws(d);
  MOE_TRY(check_backward_args(d, p, W, ws, ws_bytes));
  MOE_TRY(need(y));
  moe_aux_out ao{};
  if (aux) ao = *aux;
  // the routing outputs and f stay in the workspace (the backward reads them there)
  if (ao.logits || ao.topk_idx || ao.topk_w || ao.n_real || ao.offsets || ao.f) return MOE_ERR_ARG;
  MOE_TRY(maybe(ao.P));
  MOE_TRY(maybe(ao.counts));
  MOE_TRY(maybe(ao.scalars));
  if (d->T == 0) return MOE_OK;
  MOE_TRY(no_pending_error());
  uint8_t* base = static_cast<uint8_t*>(ws);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY(backward_state(d, p, W, base, s, &ao));
  const LayerWs& L = W.fwd;
  auto at = [&](size_t off) { return static_cast<void*>(base + off); };
  return layer_down_combine(d, p, y, L, base, static_cast<const int32_t*>(at(L.offsets)),
                            static_cast<const int32_t*>(at(L.slot_pos)), static_cast<const float*>(at(L.topk_w)),
                            static_cast<const int32_t*>(at(L.n_real)),
                            fused_combine(d) ? static_cast<const int32_t*>(at(L.row_dst)) : nullptr, s);
}

}  // extern "C"
