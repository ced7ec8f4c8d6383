// Router GEMM with a fused null-threshold top-K / renormalisation epilogue.
//
// Scoring (paper review "Improving MoE Compute Efficiency by Composing Weight
// and Data Sparsity", section 3, "Null Expert mechanism"): the router maps a
// token to N+1 float32 logits, the last one being the null expert's. The null
// logit takes the scalar and per-token null bias.
//
// Selection ("threshold interpretation" paragraph of the same section): the
// null logit is copied M times into the pool and top-K is taken; a real expert
// is chosen only when its logit is strictly larger than the null logit, at
// most K of them, and when M < K the remaining K - M slots must be reals:
//     c = #{j < N : s_j > s_null},  r = min(K, max(c, K - M))   (r = K if M = 0)
// The chosen reals are the r largest by (value desc, index asc). Their weights
// are a softmax over their own logits, i.e. the pool softmax renormalised over
// the chosen reals only; null slots get weight 0.
//
// MI355X design.
//  * x is bf16 and the router weight float32. Every bf16 x bf16 product is
//    exact in float32, and an fp32 weight splits exactly into three bf16 parts
//    (hi + mid + lo, each the bf16 rounding of what is left), so three bf16
//    MFMAs give the products exactly at MFMA rate instead of the slower fp32
//    path. Each wavefront's float32 MFMA sums over 32 K columns (its half of
//    a 64-wide K tile) are accumulated in fp64, which keeps the logits within
//    a few 1e-7 of the exact value (plain fp32
//    accumulation over d = 2048 terms drifts by a few 1e-6, too close to the
//    1e-5 near-tie margin of routing parity). The null row is an fp64 dot
//    product on the vector ALUs.
//  * A workgroup scores 64 tokens against one or two 32-expert tiles (all of
//    them when N <= 64). K tiles of x, of the float32 weight rows and of the
//    null row stream through 5-7 swizzled LDS stages filled by global->LDS loads,
//    so several tiles are in flight while one feeds the MFMAs; the weight is
//    split into its three bf16 parts in registers. With few tokens (or N > 64)
//    K, and the expert tiles, are spread over several workgroups that write
//    float32 partial logits, and a selection kernel adds them in a fixed order.
//  * Epilogue: 4 lanes per token in the scoring kernel, 16 in the 1024-thread
//    selection kernel. Each lane walks its share of the token's logits row in
//    LDS and keeps the best K reals in registers with a branch-free insertion
//    network over 64-bit keys (order-preserving bits of the logit, then the
//    complemented expert index, so ties go to the lower index); DPP exchanges
//    within the row merge the lists. One lane per token then does the per-token
//    fp64 work (weights, log-sum-exp) once.
//  * Fused layer mode additionally writes, per 64-token tile, the real slots
//    per expert (the first pass of the permutation's counting sort), the
//    histogram of r and the load-balance / z-loss sums; the permutation's scan
//    adds them over tiles in tile order, so the totals do not depend on the
//    order in which workgroups finish and no accumulator needs clearing.
#include <algorithm>
#include <type_traits>

#include "aux_final.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kRouteBT = 64;       // tokens per workgroup
constexpr int kRouteThreads = 256;

int route_tokens_per_block() { return kRouteBT; }

// total order of float32 values as unsigned keys (-0.0 and +0.0 equal)
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

struct RouteKernelArgs {
  const bf16_t* x;
  const float* w;          // [N + 1][d] float32, row N = null
  const float* w_null;
  float null_bias;
  const float* null_bias_tok;
  int64_t T;
  int d, N, Np, M, K;
  float* logits_out;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* n_real;
  int32_t* chunk_hist;     // fused: [tiles][N]
  int32_t* rhist;          // fused: [tiles][K + 1]
  double* tstats;          // fused: [tiles][N + 3]
  int KS;                  // bf16 scoring: K splits (partials path)
  int partials;            // bf16 scoring: 1 = write partial logits for route_select_kernel
  float* lpart;            // bf16 scoring, partials path: [KS][T][N + 1] partial logits
  int null_kind;           // 0: weights over the chosen reals; else over all K slots
};

// fp64 LDS scratch of the fused epilogue: block sums [N + 3], per-token lse^2 and r
// [2][64], column parts [P][N + 1] (P = 4 or 16; sized for 16)
__host__ __device__ constexpr int epi_doubles(int N) { return (N + 3) + 2 * 64 + 16 * (N + 1); }

// threads of a selection-only workgroup: 16 lanes per token while the key lists
// are short, else 4 (register budget of 1024-thread workgroups)
template <int KMAX>
constexpr int select_threads() { return KMAX <= 8 ? 1024 : 256; }

// LDS of the selection epilogue: the logits tile [64][N + 1] float32, a per-token
// hand-off of kTokSlots 8-byte slots (the top-KMAX keys at 0 .., then vmax and the
// pool max at 32, r at 33, z at 34, 1/z at 35), and in fused mode the fp64
// statistics scratch and the histogram counters [N + K + 1].
constexpr int kTokSlots = 36;
struct EpiLds {
  float* sl;
  uint64_t* tok;
  double* wacc;
  int* cnt;
};
__device__ __forceinline__ EpiLds epi_lds(unsigned char* smem, int N) {
  EpiLds e;
  e.sl = reinterpret_cast<float*>(smem);
  e.tok = reinterpret_cast<uint64_t*>(e.sl + ((kRouteBT * (N + 1) + 1) & ~1));
  e.wacc = reinterpret_cast<double*>(e.tok + kRouteBT * kTokSlots);
  e.cnt = reinterpret_cast<int*>(e.wacc + epi_doubles(N));
  return e;
}
static size_t epi_lds_bytes(int N, int K, bool fused) {
  size_t b = (size_t)((kRouteBT * (N + 1) + 1) & ~1) * sizeof(float) +
             (size_t)kRouteBT * kTokSlots * sizeof(uint64_t);
  if (fused) b += (size_t)epi_doubles(N) * sizeof(double) + (size_t)(N + K + 1) * sizeof(int);
  return b;
}

// Selection for the (up to 64) tokens of one workgroup, in two phases.
// Phase 1: LPT consecutive lanes (4 or 16) own a token, lane q walking experts
// q, q + LPT, ... of its logits row. Each lane keeps the best KMAX reals it has
// seen in a register list sorted by 64-bit keys (the order-preserving bits of the
// logit, then the complemented index: a larger key is a larger logit, or the lower
// index at equal logits); an insertion is a fixed compare-and-swap chain, so no
// lane diverges. The LPT lists are merged with log2(LPT) rounds of shuffles. In
// fused mode the lanes also overwrite the row with the pool-softmax numerators and
// add them up (z). Lane 0 hands the token's keys, maxima, r and z over in LDS.
// Phase 2: one lane per token (wavefront 0) does the per-token fp64 work once:
// the renormalised weights, the outputs, the histogram counts and, in fused mode,
// 1/z (for the column sums), lse^2 and r in tok_acc[0][t] and tok_acc[1][t].
template <int KMAX>
__device__ __forceinline__ void insert_key(uint64_t (&lk)[KMAX], uint64_t key) {
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    const bool gt = key > lk[i];
    const uint64_t old = lk[i];
    lk[i] = gt ? key : old;
    key = gt ? old : key;
  }
}

// Partner exchange of round R of an all-reduce over the 4 (R < 2) or 16 lanes of a
// DPP row: swap within pairs, swap pairs, mirror within halves of 8, mirror the
// row. Each round combines two disjoint groups that already agree, so after
// log2(lanes) rounds every lane holds the combination of all of them; for a
// commutative combination every lane computes the same value.
template <int R>
__device__ __forceinline__ uint32_t dpp_xchg(uint32_t v) {
  constexpr int kCtl[4] = {0xB1, 0x4E, 0x141, 0x140};  // quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror, row_mirror
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kCtl[R], 0xF, 0xF, false);
}
template <int R>
__device__ __forceinline__ uint64_t dpp_xchg64(uint64_t v) {
  return ((uint64_t)dpp_xchg<R>((uint32_t)(v >> 32)) << 32) | dpp_xchg<R>((uint32_t)v);
}
template <int R>
__device__ __forceinline__ double dpp_xchg_f64(double v) {
  return __longlong_as_double((long long)dpp_xchg64<R>((uint64_t)__double_as_longlong(v)));
}

template <int KMAX, bool FUSED, int LPT>
__device__ void select_tokens(const RouteKernelArgs& a, const EpiLds& L, int ld, int nt, int64_t t0,
                              double* tok_acc) {
  static_assert(LPT == 4 || LPT == 8 || LPT == 16, "lanes per token");
  static_assert(KMAX <= 32, "key slots of the hand-off");
  const int tl = threadIdx.x / LPT, q = threadIdx.x % LPT;
  const int N = a.N, M = a.M, K = a.K;
  const bool live = tl < nt;
  float* s = L.sl + (live ? tl : 0) * ld;
  const float snull = s[N];
  uint64_t lk[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) lk[i] = 0ull;
  int c = 0;
  float vmax = -INFINITY;
#pragma unroll 4
  for (int j = q; j < N; j += LPT) {
    const float v = s[j];
    c += v > snull;
    vmax = fmaxf(vmax, v);
    insert_key(lk, ((uint64_t)ordered_bits(v) << 32) | (0xffffffffu - (uint32_t)j));
  }
  auto merge = [&](auto round) {
    constexpr int R = decltype(round)::value;
    uint64_t other[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) other[i] = dpp_xchg64<R>(lk[i]);
#pragma unroll
    for (int i = 0; i < KMAX; ++i) insert_key(lk, other[i]);
    c += (int)dpp_xchg<R>((uint32_t)c);
    vmax = fmaxf(vmax, __uint_as_float(dpp_xchg<R>(__float_as_uint(vmax))));
  };
  merge(std::integral_constant<int, 0>{});
  merge(std::integral_constant<int, 1>{});
  if constexpr (LPT >= 8) merge(std::integral_constant<int, 2>{});
  if constexpr (LPT == 16) merge(std::integral_constant<int, 3>{});
  const int r = (M == 0) ? K : min(K, max(c, K - M));
  const float mp = M > 0 ? fmaxf(vmax, snull) : vmax;  // pool maximum
  uint64_t* tk = L.tok + tl * kTokSlots;
  if (q == 0) {
#pragma unroll
    for (int i = 0; i < KMAX; ++i) tk[i] = lk[i];
    tk[32] = ((uint64_t)__float_as_uint(mp) << 32) | __float_as_uint(vmax);
    tk[33] = ((uint64_t)__float_as_uint(snull) << 32) | (uint32_t)r;
  }
  if (FUSED) {
    // pool softmax [reals, null x M] numerators written over the logits row
    double zq = 0.0;
#pragma unroll 4
    for (int j = q; j < N; j += LPT) {
      const float ej = expf(s[j] - mp);
      if (live) s[j] = ej;
      zq += (double)ej;
    }
    // every lane adds the same operands in the same tree
    zq += dpp_xchg_f64<0>(zq);
    zq += dpp_xchg_f64<1>(zq);
    if constexpr (LPT >= 8) zq += dpp_xchg_f64<2>(zq);
    if constexpr (LPT == 16) zq += dpp_xchg_f64<3>(zq);
    // a null logit at +inf is the pool maximum itself: its numerator is 1 (the limit;
    // exp(inf - inf) would be NaN), every real one 0, z = M and lse = +inf
    const float en = M > 0 ? (snull == mp ? 1.0f : expf(snull - mp)) : 0.0f;
    if (q == 0) {
      tk[34] = (uint64_t)__double_as_longlong(zq + (double)M * (double)en);
      if (live) s[N] = en;
    }
  }
  __syncthreads();
  if (threadIdx.x >= kRouteBT) return;
  // phase 2: lane t of wavefront 0 finishes token t
  const int t = threadIdx.x;
  uint64_t* tt = L.tok + t * kTokSlots;
  if (t >= nt) {
    if (FUSED) {
      tok_acc[t] = 0.0;
      tok_acc[kRouteBT + t] = 0.0;
    }
    return;
  }
  const int rr = (int)(uint32_t)tt[33];
  const float sn = __uint_as_float((uint32_t)(tt[33] >> 32));
  const float vm = __uint_as_float((uint32_t)tt[32]), pm = __uint_as_float((uint32_t)(tt[32] >> 32));
  // weights in fp64, summed in rank order: a softmax over the chosen reals (null
  // slots 0), or for copy / constant null slots over all K chosen entries, the
  // null slots at the null logit (shifted by the pool maximum)
  const bool all_k = a.null_kind != 0;
  double e[KMAX];
  double tot = 0.0;
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    const double v = i < rr ? (double)from_ordered_bits((uint32_t)(tt[i] >> 32)) : (double)sn;
    const double sh = (double)(all_k ? pm : vm);  // at v == sh the numerator is 1, also at +inf
    e[i] = (i < rr || (all_k && i < K)) ? (v == sh ? 1.0 : exp(v - sh)) : 0.0;
    tot += e[i];
  }
  const int64_t tg = t0 + t;
  int32_t* idx_row = a.topk_idx + tg * K;
  float* w_row = a.topk_w + tg * K;
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    if (i < K) {
      const int id = i < rr ? (int)(0xffffffffu - (uint32_t)tt[i]) : N + (i - rr);
      idx_row[i] = id;
      w_row[i] = (i < rr || all_k) ? (float)(e[i] / tot) : 0.0f;
      if (FUSED && i < rr) atomicAdd(&L.cnt[id], 1);
    }
  }
  if (a.n_real) a.n_real[tg] = rr;
  if (FUSED) {
    atomicAdd(&L.cnt[N + rr], 1);
    const double z = __longlong_as_double((long long)tt[34]);
    reinterpret_cast<float*>(tt + 35)[0] = (float)(1.0 / z);
    const double lse = (double)pm + log(z);
    tok_acc[t] = lse * lse;
    tok_acc[kRouteBT + t] = (double)rr;
  }
}

template <bool FUSED, int KMAX, int NT>
__device__ void route_epilogue(const RouteKernelArgs& a, const EpiLds& L, int ld, int nt, int64_t t0,
                               int64_t tile, bool copy_logits) {
  constexpr int P = NT / kRouteBT;  // lanes per token, and column parts
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int N = a.N;
  float* sl = L.sl;
  double* wacc = L.wacc;
  int* cnt_lds = L.cnt;
  if (copy_logits) {
    // the tile's rows are contiguous in both (ld = N + 1), 16-byte aligned (t0 % 64 == 0)
    const int n = nt * ld;
    float* dst = a.logits_out + t0 * ld;
    for (int i = 4 * threadIdx.x; i < n; i += 4 * NT) {
      if (i + 4 <= n) {
        *reinterpret_cast<f32x4_t*>(dst + i) = *reinterpret_cast<const f32x4_t*>(sl + i);
      } else {
        for (int j = i; j < n; ++j) dst[j] = sl[j];
      }
    }
    __syncthreads();  // the fused selection overwrites the rows
  }
  double* tok_acc = wacc + N + 3;  // [2][64]
  select_tokens<KMAX, FUSED, P>(a, L, ld, nt, t0, tok_acc);
  if (!FUSED) return;
  __syncthreads();
  // per-block sums in a fixed order: lse^2 / n_real over the block's tokens, and
  // the probability columns (numerator x 1/z, rounded to float32) in P
  // interleaved parts added pairwise
  if (wave == 0) {
    const double lz = wave_sum_double(tok_acc[lane]);
    const double nr = wave_sum_double(tok_acc[kRouteBT + lane]);
    if (lane == 0) {
      wacc[N + 1] = lz;
      wacc[N + 2] = nr;
    }
  }
  double* colq = tok_acc + 2 * kRouteBT;  // [P][N + 1]
  for (int i = threadIdx.x; i < P * (N + 1); i += NT) {
    const int j = i % (N + 1), qq = i / (N + 1);
    double sum = 0.0;
#pragma unroll 4
    for (int tl = qq; tl < nt; tl += P)
      sum += (double)(sl[tl * ld + j] * reinterpret_cast<const float*>(L.tok + tl * kTokSlots + 35)[0]);
    colq[qq * (N + 1) + j] = sum;
  }
  __syncthreads();
  for (int j = threadIdx.x; j <= N; j += NT) {
    double v[P];
#pragma unroll
    for (int u = 0; u < P; ++u) v[u] = colq[u * (N + 1) + j];
#pragma unroll
    for (int w = P / 2; w >= 1; w /= 2)
#pragma unroll
      for (int u = 0; u < w; ++u) v[u] += v[u + w];
    wacc[j] = v[0];
  }
  __syncthreads();
  // this tile's sums, real-slot histogram and r histogram; the permutation's scan
  // adds them over tiles in order
  double* ts = a.tstats + tile * (N + 3);
  for (int i = threadIdx.x; i < N + 3; i += NT) ts[i] = wacc[i];
  for (int i = threadIdx.x; i < N; i += NT) a.chunk_hist[tile * N + i] = cnt_lds[i];
  for (int i = threadIdx.x; i <= a.K; i += NT) a.rhist[tile * (a.K + 1) + i] = cnt_lds[N + i];
}

// bf16 x: three-way split MFMA scoring. Workgroup (token tile tt, expert group eg,
// K split ks) scores 64 tokens against ETW 32-expert tiles over its share of the
// K tiles; the workgroups of a token tile are dispatched to one XCD, where they
// share the x tile in L2. K tiles of 64 columns (x rows, the group's float32
// weight rows and the null row) stream through S LDS stages filled by
// global->LDS loads, S-1 of them in flight. Each weight fragment is split into its
// bf16 (hi, mid, lo) parts in registers right before its three MFMAs (hardware
// round-to-nearest-even; the two subtractions are exact), so the float32 weight is
// read as it is. Each wavefront covers one K half (16-wide K steps 2 kp and
// 2 kp + 1 of each tile): with two expert tiles wavefront w takes tile w >> 1 and
// K half w & 1 for both token halves, so each weight fragment is split once per
// workgroup; with one expert tile it takes token half w & 1 and K half w >> 1. The
// two K halves are added in a fixed order at the end. Group 0 also computes the null row as an fp64 dot
// product. With one workgroup per token tile (many tokens, N <= 64) the logits go
// straight to LDS for the selection epilogue. Otherwise each workgroup writes its
// partial logits and route_select_kernel adds the K splits in order and selects:
// with few tokens, splitting K spreads the latency-bound K loop over the CUs (up to
// 16 splits of one K tile each when the batch is a single token tile).
constexpr int kRouteRedOff = 84 * 1024;  // LDS byte offset of the K-half exchange buffer

template <int ETW>
struct RouteTile {
  // stage: x [64][64] bf16 (128-byte rows), weights [32 ETW][64] float32 (256-byte
  // rows), null row slot (1 KB: four copies of 64 floats); in bf16 elements
  static constexpr int x_elems = kRouteBT * 64;
  static constexpr int w_rows = 32 * ETW;
  static constexpr int w_elems = w_rows * 128;
  static constexpr int stage = x_elems + w_elems + 512;
  static constexpr int loads = kRouteBT / 32 + w_rows / 16 + 1;  // per stage per wavefront
  static constexpr int stages = ETW == 1 ? 7 : 5;
  static constexpr size_t lds = (size_t)stages * stage * sizeof(bf16_t);
  static_assert(lds <= 160 * 1024 - 256, "LDS budget of one CU");
  static_assert(kRouteRedOff + 2 * ETW * 16 * kWave * sizeof(double) <= lds, "exchange buffer");
  static_assert(loads * (stages - 2) < 64, "stages in flight must fit the vmcnt counter");
};

__device__ __forceinline__ int rt_off(int row, int chunk) {  // x: 16-byte chunks, 8 per row
  return row * 64 + ((chunk ^ (row & 7)) << 3);
}
__device__ __forceinline__ int wt_off(int row, int unit) {   // weights: floats, 16 units per row
  return row * 64 + ((unit ^ (row & 15)) << 2);
}

typedef float f32x8_t __attribute__((ext_vector_type(8)));

// float32 values of eight packed bf16 (element 2 i is the low half of word i)
__device__ __forceinline__ f32x8_t bf16x8_to_f32(bf16x8_t b) {
  const u32x4_t w = __builtin_bit_cast(u32x4_t, b);
  f32x8_t r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[2 * i] = __uint_as_float(w[i] << 16);
    r[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
  return r;
}

template <bool FUSED, int KMAX, int ETW>
__global__ void __launch_bounds__(kRouteThreads)
route_tile_kernel(RouteKernelArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  using TL = RouteTile<ETW>;
  constexpr int S = TL::stages, JN = TL::loads;
  static_assert(kRouteBT == 64 && kRouteThreads == 256, "tile shape");
  const int N = a.N, d = a.d, Np = a.Np, n_et = Np / 32, EG = (n_et + ETW - 1) / ETW;
  const int KS = a.KS;
  const int ld = N + 1;
  bf16_t* stages = reinterpret_cast<bf16_t*>(smem_raw);

  const int b = blockIdx.x, xcd = b & 7, q = b >> 3;
  const int64_t tt = (int64_t)(q / (EG * KS)) * 8 + xcd;
  const int eg = (q % (EG * KS)) % EG, ks = (q % (EG * KS)) / EG;
  const int64_t T = a.T;
  if (tt * kRouteBT >= T) return;  // padding of the grid to whole XCD rounds
  const int64_t t0 = tt * kRouteBT;
  const int nt = (int)min<int64_t>(kRouteBT, T - t0);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int half = lane >> 5, l32 = lane & 31;
  constexpr int NTH = ETW;  // token halves per wavefront
  const int kp = ETW == 2 ? (wave & 1) : (wave >> 1);
  const int et = ETW == 2 ? (wave >> 1) : 0;     // expert tile of the group
  const int th0 = ETW == 2 ? 0 : (wave & 1);     // first token half
  const int nk_all = (d + 63) / 64;
  const int per = (nk_all + KS - 1) / KS;       // the host makes every split non-empty
  const int kt0 = ks * per;
  const int nk = min(nk_all, kt0 + per) - kt0;  // this workgroup's K tiles kt0 .. kt0 + nk - 1

  // x rows 8 (wave + 4 j) + lane / 8 (j < 2; clamped to T - 1, never stored), logical
  // chunk (lane % 8) ^ (row % 8)
  const int xr = lane >> 3, xc = (lane & 7) ^ xr;
  const bf16_t* xsrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) xsrc[j] = a.x + min<int64_t>(t0 + 8 * (wave + 4 * j) + xr, T - 1) * d;
  // weight rows 4 (wave + 4 j) + lane / 16 of the group (expert 32 (ETW eg + u) + i;
  // rows past N read row 0 and are never stored), logical unit (lane % 16) ^ (row % 16)
  constexpr int JW = TL::w_rows / 16;
  const float* wsrc[JW];
  int wu[JW];
#pragma unroll
  for (int j = 0; j < JW; ++j) {
    const int wr = 4 * (wave + 4 * j) + (lane >> 4);
    const int e = (ETW * eg + wr / 32) * 32 + wr % 32;
    wsrc[j] = a.w + (int64_t)(e < N ? e : 0) * d;
    wu[j] = (lane & 15) ^ (wr & 15);
  }
  // null slot: lane l loads floats [4 (l % 16), 4 (l % 16) + 4) of the tile (four copies)
  const int nl_col = 4 * (lane & 15);
  // Loads of K tile kt into stage st; chunks past d read column 0 and are zeroed at use.
  auto issue = [&](int kl, int st) {
    const int kt = kt0 + kl;
    bf16_t* stage = stages + st * TL::stage;
    const int k = kt * 64 + xc * 8;
    const int kc = k < d ? k : 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) load_lds16(xsrc[j] + kc, stage + 8 * (wave + 4 * j) * 64);
#pragma unroll
    for (int j = 0; j < JW; ++j) {
      const int kw = kt * 64 + 4 * wu[j];
      load_lds16(reinterpret_cast<const bf16_t*>(wsrc[j] + (kw < d ? kw : 0)),
                 stage + TL::x_elems + 4 * (wave + 4 * j) * 128);
    }
    const int kn = kt * 64 + nl_col;
    load_lds16(reinterpret_cast<const bf16_t*>(a.w_null + (kn + 4 <= d ? kn : 0)),
               stage + TL::x_elems + TL::w_elems);
  };

  double acc[NTH][16];
#pragma unroll
  for (int h = 0; h < NTH; ++h)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[h][i] = 0.0;
  const bool do_null = eg == 0;
  const int nl_tok = tid >> 2, nl_part = tid & 3;
  double nacc = 0.0;
  // per-token null bias, loaded before the K loop so its latency is hidden
  const float nbias_tok =
      (do_null && a.null_bias_tok && nl_part == 0 && nl_tok < nt) ? a.null_bias_tok[t0 + nl_tok] : 0.0f;

  auto compute = [&](auto tail, int st, int kvalid) {
    const bf16_t* xs = stages + st * TL::stage;
    const float* ws = reinterpret_cast<const float*>(xs + TL::x_elems);
    const float* wn = reinterpret_cast<const float*>(xs + TL::x_elems + TL::w_elems);
    f32x16_t part[NTH];
#pragma unroll
    for (int h = 0; h < NTH; ++h) part[h] = f32x16_t{};
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int ch = (2 * kp + s2) * 2 + half;
      const bool dead = decltype(tail)::value && ch * 8 >= kvalid;
      const int wr = 32 * et + l32;
      const f32x4_t v0 = *reinterpret_cast<const f32x4_t*>(&ws[wt_off(wr, 2 * ch)]);
      const f32x4_t v1 = *reinterpret_cast<const f32x4_t*>(&ws[wt_off(wr, 2 * ch + 1)]);
      f32x8_t v = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
      if (dead) v = f32x8_t{};
      const bf16x8_t b0 = __builtin_convertvector(v, bf16x8_t);
      const f32x8_t r1 = v - bf16x8_to_f32(b0);
      const bf16x8_t b1 = __builtin_convertvector(r1, bf16x8_t);
      const f32x8_t r2 = r1 - bf16x8_to_f32(b1);
      const bf16x8_t b2 = __builtin_convertvector(r2, bf16x8_t);
#pragma unroll
      for (int h = 0; h < NTH; ++h) {
        bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(&xs[rt_off((th0 + h) * 32 + l32, ch)]);
        if (dead) af = bf16x8_t{};
        part[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, b2, part[h], 0, 0, 0);
        part[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, b1, part[h], 0, 0, 0);
        part[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, b0, part[h], 0, 0, 0);
      }
    }
    if (do_null) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int c = nl_part + 4 * cc;
        if (decltype(tail)::value && c * 8 >= kvalid) continue;
        const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(&xs[rt_off(nl_tok, c)]);
        const f32x4_t w0 = *reinterpret_cast<const f32x4_t*>(wn + c * 8);
        const f32x4_t w1 = *reinterpret_cast<const f32x4_t*>(wn + c * 8 + 4);
        const float wv[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          nacc = fma((double)__uint_as_float(xv[h] << 16), (double)wv[2 * h], nacc);
          nacc = fma((double)__uint_as_float(xv[h] & 0xffff0000u), (double)wv[2 * h + 1], nacc);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < NTH; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[h][i] += (double)part[h][i];
  };

#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nk) issue(s, s);
  for (int kt = 0; kt < nk; ++kt) {
    const int ahead = min(S - 2, nk - 1 - kt);  // K tiles issued after kt
    switch (ahead) {
      case 5: wait_vmcnt<(S > 6 ? 5 : 0) * JN>(); break;
      case 4: wait_vmcnt<(S > 5 ? 4 : 0) * JN>(); break;
      case 3: wait_vmcnt<(S > 4 ? 3 : 0) * JN>(); break;
      case 2: wait_vmcnt<2 * JN>(); break;
      case 1: wait_vmcnt<JN>(); break;
      default: wait_vmcnt<0>(); break;
    }
    stage_barrier();
    if (kt + S - 1 < nk) issue(kt + S - 1, (kt + S - 1) % S);
    const int kvalid = d - (kt0 + kt) * 64;
    if (kvalid < 64) compute(std::true_type{}, kt % S, kvalid);
    else compute(std::false_type{}, kt % S, kvalid);
  }

  // LDS after the K loop: selection tile [64][ld] floats at 0, then the epilogue's
  // statistics scratch, and the K-half exchange buffer at kRouteRedOff.
  stage_barrier();
  const EpiLds L = epi_lds(smem_raw, N);
  float* sl = L.sl;
  double* red = reinterpret_cast<double*>(smem_raw + kRouteRedOff);  // [2][ETW][16][64]
  if (kp == 1) {
#pragma unroll
    for (int h = 0; h < NTH; ++h)
#pragma unroll
      for (int i = 0; i < 16; ++i) red[(((th0 + h) * ETW + et) * 16 + i) * kWave + lane] = acc[h][i];
  }
  const bool direct = !a.partials;  // then EG == 1 and KS == 1
  if (FUSED && direct)
    for (int i = tid; i < N + a.K + 1; i += kRouteThreads) L.cnt[i] = 0;
  __syncthreads();
  if (direct) {
    // the tile's logits go to LDS, then the selection epilogue
    if (kp == 0) {
      const int e = et * 32 + l32;
#pragma unroll
      for (int h = 0; h < NTH; ++h) {
        const int th = th0 + h;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const double v = acc[h][i] + red[((th * ETW + et) * 16 + i) * kWave + lane];
          const int tr = th * 32 + 8 * (i / 4) + 4 * half + (i % 4);
          if (e < N && tr < nt) sl[tr * ld + e] = (float)v;
        }
      }
    }
    if (do_null) {
      const double a01 = nacc + __shfl_xor(nacc, 1, kWave);
      const double sum = a01 + __shfl_xor(a01, 2, kWave);
      if (nl_part == 0 && nl_tok < nt) {
        double vv = sum + (double)a.null_bias;
        if (a.null_bias_tok) vv += (double)nbias_tok;
        sl[nl_tok * ld + N] = (float)vv;
      }
    }
    __syncthreads();
    route_epilogue<FUSED, KMAX, kRouteThreads>(a, L, ld, nt, t0, tt, a.logits_out != nullptr);
    return;
  }
  // partials path: this split's fp64 sums rounded once to float32 (the null column
  // without its biases); split planes are padded to a multiple of 4 floats
  const int64_t plane = (T * ld + 3) & ~int64_t(3);
  float* lp = a.lpart + ks * plane + t0 * ld;
  if (kp == 0) {
    const int e = (ETW * eg + et) * 32 + l32;
#pragma unroll
    for (int h = 0; h < NTH; ++h) {
      const int th = th0 + h;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const double v = acc[h][i] + red[((th * ETW + et) * 16 + i) * kWave + lane];
        const int tr = th * 32 + 8 * (i / 4) + 4 * half + (i % 4);
        if (e < N && tr < nt) lp[tr * ld + e] = (float)v;
      }
    }
  }
  if (do_null) {
    const double a01 = nacc + __shfl_xor(nacc, 1, kWave);
    const double sum = a01 + __shfl_xor(a01, 2, kWave);
    if (nl_part == 0 && nl_tok < nt) lp[nl_tok * ld + N] = (float)sum;
  }
}

// Partials path, second kernel: one workgroup per 64-token tile adds the K splits
// of every logit in split order (fp64), adds the null biases, rounds to float32
// and runs the selection epilogue. Each split is an fp64 sum over its K range
// rounded once to float32: at most 16 splits, so the logit moves by a few float32
// ulps of the split sums (about 1e-7 of their size), far inside the 1e-5 near-tie
// margin, while the workgroup reads half the bytes. MAXKS (4 or 16) bounds the
// splits a launch may have.
template <bool FUSED, int KMAX, int MAXKS>
__global__ void __launch_bounds__(select_threads<KMAX>())
route_select_kernel(RouteKernelArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  constexpr int NT = select_threads<KMAX>();
  constexpr int kMaxSplits = MAXKS;
  const int N = a.N, ld = N + 1, KS = a.KS;
  const EpiLds L = epi_lds(smem_raw, N);
  float* sl = L.sl;
  if (FUSED)
    for (int i = threadIdx.x; i < N + a.K + 1; i += blockDim.x) L.cnt[i] = 0;
  const int64_t T = a.T, t0 = (int64_t)blockIdx.x * kRouteBT;
  const int nt = (int)min<int64_t>(kRouteBT, T - t0);
  const int n = nt * ld;
  const int64_t plane = (T * ld + 3) & ~int64_t(3);
  const float* lp = a.lpart + t0 * ld;  // t0 * ld is a multiple of 4: 16-byte aligned quads
  // element quads (4 i .. 4 i + 3), kQuads per thread at a time, every split's loads in
  // flight together; the splits are added in order
  constexpr int kQuads = std::max(1, 8 * kRouteThreads / NT * 4 / MAXKS);
  const int nquad = (n + 3) / 4;
  for (int p0 = threadIdx.x; p0 < nquad; p0 += kQuads * NT) {
    f32x4_t v[kQuads][kMaxSplits];
#pragma unroll
    for (int u = 0; u < kQuads; ++u)
#pragma unroll
      for (int k = 0; k < kMaxSplits; ++k) {
        const int pi = p0 + u * NT;
        v[u][k] = (pi < nquad && k < KS)
                      ? *reinterpret_cast<const f32x4_t*>(lp + k * plane + 4 * (int64_t)pi)
                      : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      }
#pragma unroll
    for (int u = 0; u < kQuads; ++u) {
      const int pi = p0 + u * NT;
      if (pi >= nquad) continue;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int i = 4 * pi + h;
        if (i >= n) continue;
        double sum = 0.0;
#pragma unroll
        for (int k = 0; k < kMaxSplits; ++k)
          if (k < KS) sum += (double)v[u][k][h];
        if (i % ld == N) {
          sum += (double)a.null_bias;
          if (a.null_bias_tok) sum += (double)a.null_bias_tok[t0 + i / ld];
        }
        sl[i] = (float)sum;
      }
    }
  }
  __syncthreads();
  route_epilogue<FUSED, KMAX, NT>(a, L, ld, nt, t0, blockIdx.x, a.logits_out != nullptr);
}

// float32 x: plain dot products (small workloads), then the same epilogue.
template <bool FUSED, int KMAX>
__global__ void __launch_bounds__(kRouteThreads)
route_simt_kernel(RouteKernelArgs a, const float* __restrict__ xf, const float* __restrict__ w) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const int N = a.N, d = a.d, ld = N + 1;
  const EpiLds L = epi_lds(smem_raw, N);
  float* sl = L.sl;
  if (FUSED)
    for (int i = threadIdx.x; i < N + a.K + 1; i += blockDim.x) L.cnt[i] = 0;
  const int64_t t0 = (int64_t)blockIdx.x * kRouteBT;
  const int nt = (int)min<int64_t>(kRouteBT, a.T - t0);
  for (int i = threadIdx.x; i < nt * ld; i += blockDim.x) {
    const int tl = i / ld, j = i % ld;
    const int64_t t = t0 + tl;
    double acc = 0.0;
    for (int k = 0; k < d; ++k) acc = fma((double)xf[t * d + k], (double)w[(int64_t)j * d + k], acc);
    if (j == N) {
      acc += (double)a.null_bias;
      if (a.null_bias_tok) acc += (double)a.null_bias_tok[t];
    }
    sl[tl * ld + j] = (float)acc;
  }
  __syncthreads();
  route_epilogue<FUSED, KMAX, kRouteThreads>(a, L, ld, nt, t0, blockIdx.x, a.logits_out != nullptr);
}

template <bool FUSED, int KMAX>
__global__ void __launch_bounds__(select_threads<KMAX>())
route_from_logits_kernel(RouteKernelArgs a, const float* __restrict__ logits) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const int N = a.N, ld = N + 1;
  const EpiLds L = epi_lds(smem_raw, N);
  float* sl = L.sl;
  if (FUSED)
    for (int i = threadIdx.x; i < N + a.K + 1; i += blockDim.x) L.cnt[i] = 0;
  const int64_t t0 = (int64_t)blockIdx.x * kRouteBT;
  const int nt = (int)min<int64_t>(kRouteBT, a.T - t0);
  for (int i = threadIdx.x; i < nt * ld; i += blockDim.x) sl[i] = logits[t0 * ld + i];
  __syncthreads();
  route_epilogue<FUSED, KMAX, select_threads<KMAX>()>(a, L, ld, nt, t0, blockIdx.x, a.logits_out != nullptr);
}

// A few tokens (decode-size batches): one workgroup does the whole routing step,
// which would otherwise be a split-K scoring launch, a selection launch and, in the
// layer, the permutation's launch, each a few microseconds of latency for little
// work. Each logit is a float64 dot product of 16 lanes (one DPP row): lane q takes
// the 8-element chunks q, q + 16, ... of the bf16 token row and the float32 router
// row (products exact in float64), and the 16 partial sums are added in a fixed
// tree; the null logit then gets its biases in float64 and every logit is rounded
// once to float32 (within 1e-6 of the exact value, as the MFMA path). The selection
// epilogue is the one of the other routing kernels. In the layer (pm.perm_token set)
// the same workgroup then sorts the tile's slots (per-expert counts, offsets, a
// stable scatter: thread e walks the slots in order and places expert e's) and
// finalises the statistics from the single tile's sums.
// The dot products run on the vector ALUs of one CU in float64, so this pays only
// for a handful of tokens (measured at the Qwen3-0.6B shape: T = 16 took 125 us
// against 67 us for the split-K scoring launches).
constexpr int kSmallT = 4;               // at most this many tokens
constexpr int64_t kSmallMacs = 1 << 19;  // and T (N + 1) d at most this

struct SmallPermute {
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm_token;
  int32_t* slot_pos;
  AuxTiles aux;  // tstats NULL: no statistics wanted
};

template <bool FUSED, int KMAX>
__global__ void __launch_bounds__(select_threads<KMAX>())
route_small_kernel(RouteKernelArgs a, SmallPermute pm) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  constexpr int NT = select_threads<KMAX>();
  constexpr int NG = NT / 16;  // dot products in flight
  const int N = a.N, d = a.d, ld = N + 1, K = a.K;
  const int nt = (int)a.T;
  const EpiLds L = epi_lds(smem_raw, N);
  float* sl = L.sl;
  if (FUSED)
    for (int i = threadIdx.x; i < N + K + 1; i += NT) L.cnt[i] = 0;
  const int q = threadIdx.x & 15, grp = threadIdx.x >> 4;
  const int nchunk = d / 8;
  for (int item = grp; item < nt * ld; item += NG) {  // uniform over the 16 lanes
    const int t = item / ld, j = item - t * ld;
    const bf16_t* xr = a.x + (int64_t)t * d;
    const float* wr = a.w + (int64_t)j * d;  // row N: the null row
    double acc = 0.0;
    // batches of 8 chunks per lane, every load of a batch in flight before its FMAs
    // (chunks past d are zero)
    for (int c0 = q; c0 < nchunk; c0 += 16 * 8) {
      u32x4_t xv[8];
      f32x4_t w0[8], w1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + 16 * u;
        const bool in = c < nchunk;
        xv[u] = in ? *reinterpret_cast<const u32x4_t*>(xr + 8 * c) : u32x4_t{0, 0, 0, 0};
        w0[u] = in ? *reinterpret_cast<const f32x4_t*>(wr + 8 * c) : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        w1[u] = in ? *reinterpret_cast<const f32x4_t*>(wr + 8 * c + 4) : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wv[8] = {w0[u][0], w0[u][1], w0[u][2], w0[u][3], w1[u][0], w1[u][1], w1[u][2], w1[u][3]};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          acc = fma((double)__uint_as_float(xv[u][h] << 16), (double)wv[2 * h], acc);
          acc = fma((double)__uint_as_float(xv[u][h] & 0xffff0000u), (double)wv[2 * h + 1], acc);
        }
      }
    }
    acc += dpp_xchg_f64<0>(acc);
    acc += dpp_xchg_f64<1>(acc);
    acc += dpp_xchg_f64<2>(acc);
    acc += dpp_xchg_f64<3>(acc);
    if (q == 0) {
      if (j == N) {
        acc += (double)a.null_bias;
        if (a.null_bias_tok) acc += (double)a.null_bias_tok[t];
      }
      sl[t * ld + j] = (float)acc;
    }
  }
  __syncthreads();
  route_epilogue<FUSED, KMAX, NT>(a, L, ld, nt, 0, 0, a.logits_out != nullptr);
  if (!FUSED || !pm.perm_token) return;
  // the tile's slots in expert order (LDS: slot keys [T K], counts [N], offsets [N + 1])
  __syncthreads();
  const int TK = nt * K;
  int* skey = reinterpret_cast<int*>(smem_raw);
  int* cnt = skey + TK;
  int* off = cnt + N;
  for (int e = threadIdx.x; e < N; e += NT) cnt[e] = 0;
  __syncthreads();
  for (int f = threadIdx.x; f < TK; f += NT) {
    const int v = a.topk_idx[f];
    const int e = (v >= 0 && v < N) ? v : N;
    skey[f] = e;
    if (e < N) atomicAdd(&cnt[e], 1);
    else pm.slot_pos[f] = -1;
  }
  __syncthreads();
  if (threadIdx.x < kWave) {  // exclusive scan, 4 experts per lane (N <= 256)
    const int lane = threadIdx.x;
    int c4[4], local = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = 4 * lane + u;
      c4[u] = e < N ? cnt[e] : 0;
      local += c4[u];
    }
    int incl = local;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    int run = incl - local;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = 4 * lane + u;
      if (e < N) off[e] = run;
      run += c4[u];
    }
    if (lane == kWave - 1) off[N] = incl;
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= N; e += NT) pm.offsets[e] = off[e];
  for (int e = threadIdx.x; e < N; e += NT) {
    pm.counts[e] = cnt[e];
    int pos = off[e];
    for (int f = 0; f < TK; ++f)
      if (skey[f] == e) {
        pm.perm_token[pos] = f / K;
        pm.slot_pos[f] = pos;
        ++pos;
      }
  }
  if (!pm.aux.tstats) return;
  __syncthreads();  // the LDS is the statistics' scratch from here
  finalize_tiles<16>(pm.aux, a.chunk_hist, 1, a.T, N, a.M, K, smem_raw);
}

// 32-expert tiles per scoring workgroup: all of them when N <= 64, else pairs.
static int route_etw(int N) { return N <= 32 ? 1 : 2; }

// bf16 scoring plan. Many tokens and N <= 64: one workgroup per token tile scores
// and selects (no second kernel). Otherwise K is split so that the scoring grid
// covers about 256 workgroups (at most 4 splits, each non-empty), partial logits go
// to the workspace and route_select_kernel adds and selects.
struct RoutePlan {
  int etw, eg, ks;
  bool partials;
};
static RoutePlan route_plan(int64_t T, int N, int d) {
  const int etw = route_etw(N);
  const int Np = (N + 31) / 32 * 32;
  const int eg = (Np / 32 + etw - 1) / etw;
  const int64_t ntt = std::max<int64_t>(1, (T + kRouteBT - 1) / kRouteBT);
  if (eg == 1 && ntt >= 128) return {etw, 1, 1, false};
  const int nk = (d + 63) / 64;
  // one token tile: up to 16 splits (one K tile each at d = 1024); else up to 4,
  // which keeps the selection's partial-logit reads at twice the logits
  const int64_t cap = ntt == 1 ? 16 : 4;
  int ks = (int)std::min<int64_t>(cap, std::max<int64_t>(1, (256 + ntt * eg - 1) / (ntt * eg)));
  ks = std::min(ks, nk);
  const int per = (nk + ks - 1) / ks;
  ks = (nk + per - 1) / per;
  return {etw, eg, ks, true};
}

// bf16 scoring workspace: the partial logits of the partials path (at least 256
// bytes, so a bf16 call always passes one).
size_t route_ws_bytes(int64_t T, int N, int d) {
  const RoutePlan pl = route_plan(T, N, d);
  const size_t part =
      pl.partials ? (size_t)pl.ks * (size_t)((T * (N + 1) + 3) & ~int64_t(3)) * sizeof(float) : 0;
  return std::max<size_t>(256, (part + 255) / 256 * 256);
}

// LDS of the selection epilogue, and of the scoring kernel (stages) when mfma
static size_t route_lds_bytes(const RouteArgs& r, bool mfma) {
  size_t b = epi_lds_bytes(r.N, r.K, r.fused);
  if (mfma) b = std::max(b, route_etw(r.N) == 1 ? RouteTile<1>::lds : RouteTile<2>::lds);
  return b;
}

template <typename F>
static void allow_lds(F* kernel, size_t lds) {
  if (lds > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

hipError_t launch_route(const RouteArgs& r, hipStream_t stream) {
  if (route_small_ok(r)) return launch_route_small(r, nullptr, stream);
  const int64_t ntt = (r.T + kRouteBT - 1) / kRouteBT;
  const unsigned nblk = (unsigned)ntt;
  const int Np = (r.N + 31) / 32 * 32;
  const bool mfma = !r.logits_in && r.bf16;
  const RoutePlan pl = route_plan(r.T, r.N, r.d);
  RouteKernelArgs a{static_cast<const bf16_t*>(r.x), r.w_router,
                    r.w_router ? r.w_router + (int64_t)r.N * r.d : nullptr, r.null_bias,
                    r.null_bias_tok, r.T, r.d, r.N, Np, r.M, r.K, r.logits_out,
                    r.topk_idx, r.topk_w, r.n_real, r.chunk_hist, r.rhist, r.tstats,
                    pl.ks, pl.partials ? 1 : 0, mfma ? static_cast<float*>(r.ws) : nullptr,
                    r.null_kind};
  const size_t lds = route_lds_bytes(r, mfma && !pl.partials);
  const size_t lds_score = route_etw(r.N) == 1 ? RouteTile<1>::lds : RouteTile<2>::lds;
  const size_t lds_select = route_lds_bytes(r, false);
  const int kmax = r.K <= 2 ? 2 : (r.K <= 8 ? 8 : 32);
#define MOE_KMAX_SWITCH(MACRO, ...)                 \
  do {                                              \
    if (kmax == 2) MACRO(__VA_ARGS__, 2);           \
    else if (kmax == 8) MACRO(__VA_ARGS__, 8);      \
    else MACRO(__VA_ARGS__, 32);                    \
  } while (0)
#define MOE_LOGITS_LAUNCH(F_, KM_)                                                        \
  do {                                                                                    \
    allow_lds(route_from_logits_kernel<F_, KM_>, lds);                                    \
    route_from_logits_kernel<F_, KM_><<<nblk, select_threads<KM_>(), lds, stream>>>(a, r.logits_in); \
  } while (0)
#define MOE_SIMT_LAUNCH(F_, KM_)                                                          \
  do {                                                                                    \
    allow_lds(route_simt_kernel<F_, KM_>, lds);                                           \
    route_simt_kernel<F_, KM_><<<nblk, kRouteThreads, lds, stream>>>(                     \
        a, static_cast<const float*>(r.x), r.w_router);                                   \
  } while (0)
#define MOE_ROUTE_LAUNCH(F_, KM_)                                                         \
  do {                                                                                    \
    if (!pl.partials) {                                                                   \
      if (pl.etw == 1) {                                                                  \
        allow_lds(route_tile_kernel<F_, KM_, 1>, lds);                                    \
        route_tile_kernel<F_, KM_, 1><<<grid, kRouteThreads, lds, stream>>>(a);           \
      } else {                                                                            \
        allow_lds(route_tile_kernel<F_, KM_, 2>, lds);                                    \
        route_tile_kernel<F_, KM_, 2><<<grid, kRouteThreads, lds, stream>>>(a);           \
      }                                                                                   \
    } else {                                                                              \
      if (pl.etw == 1) {                                                                  \
        allow_lds(route_tile_kernel<false, 2, 1>, lds_score);                             \
        route_tile_kernel<false, 2, 1><<<grid, kRouteThreads, lds_score, stream>>>(a);    \
      } else {                                                                            \
        allow_lds(route_tile_kernel<false, 2, 2>, lds_score);                             \
        route_tile_kernel<false, 2, 2><<<grid, kRouteThreads, lds_score, stream>>>(a);    \
      }                                                                                   \
      if (pl.ks <= 4) {                                                                   \
        allow_lds(route_select_kernel<F_, KM_, 4>, lds_select);                           \
        route_select_kernel<F_, KM_, 4><<<nblk, select_threads<KM_>(), lds_select, stream>>>(a); \
      } else {                                                                            \
        allow_lds(route_select_kernel<F_, KM_, 16>, lds_select);                          \
        route_select_kernel<F_, KM_, 16><<<nblk, select_threads<KM_>(), lds_select, stream>>>(a); \
      }                                                                                   \
    }                                                                                     \
  } while (0)
  if (r.logits_in) {
    if (r.fused) MOE_KMAX_SWITCH(MOE_LOGITS_LAUNCH, true);
    else MOE_KMAX_SWITCH(MOE_LOGITS_LAUNCH, false);
  } else if (r.bf16) {
    // token tiles padded to whole rounds of the 8 XCDs, times the groups and splits
    const unsigned grid = (unsigned)((ntt + 7) / 8 * 8 * pl.eg * pl.ks);
    if (r.fused) MOE_KMAX_SWITCH(MOE_ROUTE_LAUNCH, true);
    else MOE_KMAX_SWITCH(MOE_ROUTE_LAUNCH, false);
  } else {
    if (r.fused) MOE_KMAX_SWITCH(MOE_SIMT_LAUNCH, true);
    else MOE_KMAX_SWITCH(MOE_SIMT_LAUNCH, false);
  }
#undef MOE_ROUTE_LAUNCH
#undef MOE_SIMT_LAUNCH
#undef MOE_LOGITS_LAUNCH
#undef MOE_KMAX_SWITCH
  return hipGetLastError();
}

bool route_small_ok(const RouteArgs& r) {
  return r.bf16 && !r.logits_in && r.T >= 1 && r.T <= kSmallT &&
         r.T * (int64_t)(r.N + 1) * r.d <= kSmallMacs;
}

// One launch of route_small_kernel: the routing step, and with pa (fused layer
// path) also the permutation and the statistics.
hipError_t launch_route_small(const RouteArgs& r, const PermuteArgs* pa, hipStream_t stream) {
  if (!route_small_ok(r) || (pa && !r.fused)) return hipErrorInvalidValue;
  const int Np = (r.N + 31) / 32 * 32;
  RouteKernelArgs a{static_cast<const bf16_t*>(r.x), r.w_router, r.w_router + (int64_t)r.N * r.d,
                    r.null_bias, r.null_bias_tok, r.T, r.d, r.N, Np, r.M, r.K, r.logits_out,
                    r.topk_idx, r.topk_w, r.n_real, r.chunk_hist, r.rhist, r.tstats, 1, 0, nullptr,
                    r.null_kind};
  SmallPermute pm{};
  if (pa) {
    pm.counts = pa->counts;
    pm.offsets = pa->offsets;
    pm.perm_token = pa->perm_token;
    pm.slot_pos = pa->slot_pos;
    if (pa->aux) pm.aux = *pa->aux;
  }
  const int kmax = r.K <= 2 ? 2 : (r.K <= 8 ? 8 : 32);
  const int nt_threads = kmax <= 8 ? select_threads<8>() : select_threads<32>();
  size_t lds = epi_lds_bytes(r.N, r.K, r.fused);
  if (pa) {
    lds = std::max(lds, (size_t)(r.T * r.K + 2 * r.N + 1) * sizeof(int));
    if (pm.aux.tstats) {
      const int C = r.N + 3, G = finalize_groups(r.N, r.K, nt_threads);
      lds = std::max(lds, ((size_t)G * C + C + (size_t)(r.N + r.M)) * sizeof(double) +
                              (size_t)(r.N + r.K + 1) * sizeof(int));
    }
  }
#define MOE_SMALL_LAUNCH(F_, KM_)                                                          \
  do {                                                                                     \
    allow_lds(route_small_kernel<F_, KM_>, lds);                                           \
    route_small_kernel<F_, KM_><<<1, select_threads<KM_>(), lds, stream>>>(a, pm);         \
  } while (0)
  if (r.fused) {
    if (kmax == 2) MOE_SMALL_LAUNCH(true, 2);
    else if (kmax == 8) MOE_SMALL_LAUNCH(true, 8);
    else MOE_SMALL_LAUNCH(true, 32);
  } else {
    if (kmax == 2) MOE_SMALL_LAUNCH(false, 2);
    else if (kmax == 8) MOE_SMALL_LAUNCH(false, 8);
    else MOE_SMALL_LAUNCH(false, 32);
  }
#undef MOE_SMALL_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
