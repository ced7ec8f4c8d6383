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
//    path. MFMA partial sums over 32-wide K blocks are accumulated in fp64,
//    which keeps the logits within a few 1e-7 of the exact value (plain fp32
//    accumulation over d = 2048 terms drifts by a few 1e-6, too close to the
//    1e-5 near-tie margin of routing parity). The null row is an fp64 dot
//    product on the vector ALUs.
//  * A workgroup scores 64 tokens. K tiles of x and of the three weight planes
//    are staged through two swizzled LDS buffers by all 256 threads (the next
//    tile is fetched into registers while the current one feeds the MFMAs);
//    wavefront w takes token half w & 1 against every other 32-expert tile.
//  * Epilogue: one lane per token. Each lane walks its token's logits row in
//    LDS once and keeps the best K reals in registers with a branch-free
//    insertion network over 64-bit keys (order-preserving bits of the logit,
//    then the complemented expert index, so ties go to the lower index). This
//    costs a few instructions per (token, expert) instead of wavefront-wide
//    reductions per token.
//  * Fused layer mode additionally writes the per-workgroup expert histogram
//    (the first pass of the permutation's counting sort) and accumulates the
//    load-balance / z-loss sums of its 64 tokens into fixed-point integer
//    accumulators; integer addition is associative, so the totals do not
//    depend on the order in which workgroups finish.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kRouteBT = 64;       // tokens per workgroup
constexpr int kRouteThreads = 256;
// 16-byte loads per thread per K tile of the MFMA router: ((64 + 3 Np) BK / 8 + BK / 4)
// chunks over 256 threads, at most 9 for every (Np, BK) pair route_bk() picks.
constexpr int kRouteMaxLoads = 9;
constexpr int kQ = (MOE_MAX_EXPERTS + kWave - 1) / kWave;

int route_tokens_per_block() { return kRouteBT; }

// Prep: split W into bf16 (hi, mid, lo) planes [3][Np][d] (rows >= N zero) and
// clear the fused-statistics accumulators.
__global__ void route_prep_kernel(const float* __restrict__ w, bf16_t* __restrict__ w3, int N,
                                  int Np, int d, uint64_t* __restrict__ acc, int nacc,
                                  int32_t* __restrict__ cnt, int ncnt) {
  const int64_t total = w3 ? (int64_t)Np * d : 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  for (int64_t i = i0; i < total; i += stride) {
    const int row = (int)(i / d);
    const float v = row < N ? w[i] : 0.0f;
    const bf16_t hi = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(hi);
    const bf16_t mid = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(mid);
    w3[i] = hi;
    w3[total + i] = mid;
    w3[2 * total + i] = f32_to_bf16(r2);
  }
  for (int64_t i = i0; i < nacc; i += stride) acc[i] = 0;
  for (int64_t i = i0; i < ncnt; i += stride) cnt[i] = 0;
}

// total order of float32 values as unsigned keys (-0.0 and +0.0 equal)
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, kWave);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, kWave);
    const uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

struct RouteKernelArgs {
  const bf16_t* x;
  const bf16_t* w3;
  const float* w_null;
  float null_bias;
  const float* null_bias_tok;
  int64_t T;
  int d, N, Np, M, K, ks;  // ks: unused (1)
  float* logits_out;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* n_real;
  int32_t* chunk_hist;     // fused: [blocks][N]
  uint64_t* acc;           // fused: [N + 3] fixed-point sums
  int32_t* counts;         // fused: [N + M] pool slot counts
};

// Lane-per-token selection for the (up to 64) tokens of one workgroup, run by
// wavefront 0 with lane t owning token t. Each lane walks its logits row once,
// keeping the best KMAX reals in a register list sorted by 64-bit keys (the
// order-preserving bits of the logit, then the complemented index: a larger key
// is a larger logit, or the lower index at equal logits). An insertion is a
// fixed compare-and-swap chain, so no lane diverges. In fused mode the row is
// then overwritten with its pool-softmax probabilities for the column sums.
template <int KMAX, bool FUSED>
__device__ void select_lanes(const RouteKernelArgs& a, float* sl, int ld, int nt, int64_t t0,
                             int* cnt_lds, double* lane_acc) {
  const int lane = threadIdx.x & (kWave - 1);
  const int N = a.N, M = a.M, K = a.K;
  const bool live = lane < nt;
  float* s = sl + (live ? lane : 0) * ld;
  const float snull = s[N];
  uint64_t lk[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i) lk[i] = 0ull;
  int c = 0;
  float vmax = -INFINITY;
#pragma unroll 2
  for (int j = 0; j < N; ++j) {
    const float v = s[j];
    c += v > snull;
    vmax = fmaxf(vmax, v);
    uint64_t key = ((uint64_t)ordered_bits(v) << 32) | (0xffffffffu - (uint32_t)j);
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      const bool gt = key > lk[i];
      const uint64_t old = lk[i];
      lk[i] = gt ? key : old;
      key = gt ? old : key;
    }
  }
  const int r = (M == 0) ? K : min(K, max(c, K - M));
  // weights: softmax over the chosen reals in fp64, summed in rank order
  double e[KMAX];
  double tot = 0.0;
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    e[i] = i < r ? exp((double)from_ordered_bits((uint32_t)(lk[i] >> 32)) - (double)vmax) : 0.0;
    tot += e[i];
  }
  if (live) {
    const int64_t t = t0 + lane;
    int32_t* idx_row = a.topk_idx + t * K;
    float* w_row = a.topk_w + t * K;
#pragma unroll
    for (int i = 0; i < KMAX; ++i) {
      if (i < K) {
        const int id = i < r ? (int)(0xffffffffu - (uint32_t)lk[i]) : N + (i - r);
        idx_row[i] = id;
        w_row[i] = i < r ? (float)(e[i] / tot) : 0.0f;
        if (FUSED) atomicAdd(&cnt_lds[id], 1);
      }
    }
    if (a.n_real) a.n_real[t] = r;
  }
  if (FUSED) {
    // pool softmax [reals, null x M]: p_j written over the logits row
    const float mp = M > 0 ? fmaxf(vmax, snull) : vmax;
    double z = 0.0;
#pragma unroll 4
    for (int j = 0; j < N; ++j) z += (double)expf(s[j] - mp);
    const float en = M > 0 ? expf(snull - mp) : 0.0f;
    z += (double)M * (double)en;
    const float iz = (float)(1.0 / z);
    if (live) {
#pragma unroll 4
      for (int j = 0; j < N; ++j) s[j] = expf(s[j] - mp) * iz;
      s[N] = en * iz;
      const double lse = (double)mp + log(z);
      lane_acc[0] = lse * lse;
      lane_acc[1] = (double)r;
    } else {
      lane_acc[0] = lane_acc[1] = 0.0;
    }
  }
}

template <bool FUSED, int KMAX>
__device__ void route_epilogue(const RouteKernelArgs& a, float* sl, int ld, int nt, int64_t t0,
                               int* cnt_lds, double* wacc) {
  const int wave = threadIdx.x / kWave;
  const int N = a.N, M = a.M, P = N + M;
  if (a.logits_out) {
    const int w = N + 1;
    for (int i = threadIdx.x; i < nt * w; i += blockDim.x)
      a.logits_out[(t0 + i / w) * w + i % w] = sl[(i / w) * ld + i % w];
    if (FUSED) __syncthreads();  // the fused selection overwrites the rows
  }
  double lane_acc[2];
  if (wave == 0) select_lanes<KMAX, FUSED>(a, sl, ld, nt, t0, cnt_lds, lane_acc);
  if (!FUSED) return;
  // per-block sums in a fixed order: probability columns over the block's tokens,
  // and lse^2 / n_real over wavefront 0's lanes
  const int rd = N + 3;
  if (wave == 0) {
    const double lz = wave_sum_double(lane_acc[0]);
    const double nr = wave_sum_double(lane_acc[1]);
    if ((threadIdx.x & (kWave - 1)) == 0) {
      wacc[N + 1] = lz;
      wacc[N + 2] = nr;
    }
  }
  __syncthreads();
  for (int j = threadIdx.x; j <= N; j += blockDim.x) {
    double sum = 0.0;
    for (int tl = 0; tl < nt; ++tl) sum += (double)sl[tl * ld + j];
    wacc[j] = sum;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < rd; i += blockDim.x) {
    const double scale = (i == N + 1) ? kAuxZScale : (i == N + 2 ? 1.0 : kAuxPScale);
    const uint64_t q = (uint64_t)(wacc[i] * scale + 0.5);
    if (q) atomicAdd(reinterpret_cast<unsigned long long*>(&a.acc[i]), (unsigned long long)q);
  }
  for (int i = threadIdx.x; i < P; i += blockDim.x) {
    const int cval = cnt_lds[i];
    if (i < N) a.chunk_hist[(int64_t)blockIdx.x * N + i] = cval;
    if (cval) atomicAdd(&a.counts[i], cval);
  }
}

// bf16 x: three-way split MFMA scoring of the N real rows + fp64 null row.
// K tiles of BK columns of x (64 tokens) and of the three weight planes (Np rows)
// are staged through two LDS buffers by all 256 threads; wavefront w computes
// token half (w & 1) against expert tiles (w >> 1), (w >> 1) + 2, ...
template <int BK>
__device__ __forceinline__ int rt_off(int row, int chunk) {
  constexpr int CPR = BK / 8;  // 16-byte chunks per row
  return row * BK + ((chunk ^ (row & (CPR - 1))) << 3);
}

template <bool FUSED, int BK, int TPW, int KMAX>  // TPW: 32-expert tiles per wavefront
__global__ void __launch_bounds__(kRouteThreads)
route_mfma_kernel(RouteKernelArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  constexpr int CPR = BK / 8;
  const int N = a.N, d = a.d, Np = a.Np;
  const int ld = N + 1;
  const int n_et = Np / 32;
  // LDS: 2 x { x tile [64][BK], weight tile [3][Np][BK] bf16, null-row tile [BK] float },
  // logits [64][ld] float, fused: [N+3] doubles and pool counts [N+M] ints
  const int xt_elems = kRouteBT * BK, wt_elems = 3 * Np * BK;
  const int buf_elems = xt_elems + wt_elems + 2 * BK;  // bf16 units; the null tile is BK floats
  bf16_t* tiles = reinterpret_cast<bf16_t*>(smem_raw);
  float* sl = reinterpret_cast<float*>(tiles + 2 * buf_elems);
  double* wacc = reinterpret_cast<double*>(sl + ((kRouteBT * ld + 1) & ~1));
  int* cnt_lds = reinterpret_cast<int*>(wacc + (FUSED ? N + 3 : 0));
  if (FUSED)
    for (int i = threadIdx.x; i < N + a.M; i += blockDim.x) cnt_lds[i] = 0;

  const int64_t T = a.T;
  const int64_t t0 = (int64_t)blockIdx.x * kRouteBT;
  const int nt = (int)min<int64_t>(kRouteBT, T - t0);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int half = lane >> 5, l32 = lane & 31;
  const int th = wave & 1, eg = wave >> 1;
  const int nk = (d + BK - 1) / BK;
  const int64_t plane = (int64_t)Np * d;

  // loader assignment: x chunks [64 rows][CPR], weight chunks [3*Np rows][CPR]
  const int x_chunks = kRouteBT * CPR, w_chunks = 3 * Np * CPR, n_chunks = BK / 4;
  constexpr int kMaxLoads = kRouteMaxLoads;
  const int n_loads = (x_chunks + w_chunks + n_chunks + kRouteThreads - 1) / kRouteThreads;
  u32x4_t rbuf[kMaxLoads];
  // Every load is issued unconditionally from a clamped, valid address, with no
  // branch or select between it and the MFMAs, so the whole next tile stays in
  // flight while the current one is used. Rows past T read row T-1 and padded
  // expert rows are zero in the split weight; neither reaches a stored logit. Only
  // columns past d (the last tile when BK does not divide d) are zeroed, at stash.
  (void)n_loads;
  auto fetch = [&](int kt) {
#pragma unroll
    for (int u = 0; u < kMaxLoads; ++u) {
      const int id = tid + u * kRouteThreads;
      const bool is_x = id < x_chunks;
      const bool is_w = !is_x && id < x_chunks + w_chunks;
      const bool is_n = !is_x && !is_w && id < x_chunks + w_chunks + n_chunks;
      const int wid = is_w ? id - x_chunks : 0;
      const int nid = is_n ? id - x_chunks - w_chunks : 0;
      const int ch = is_x ? id % CPR : wid % CPR;
      const int k = kt * BK + (is_n ? nid * 4 : ch * 8);
      const int kc = k < d ? k : 0;
      const bf16_t* src;
      if (is_x) {
        src = a.x + min<int64_t>(t0 + id / CPR, T - 1) * d + kc;
      } else if (is_w) {
        const int row = wid / CPR;
        src = a.w3 + (row / Np) * plane + (int64_t)(row % Np) * d + kc;
      } else {
        src = reinterpret_cast<const bf16_t*>(a.w_null + kc);
      }
      rbuf[u] = *reinterpret_cast<const u32x4_t*>(src);
    }
  };
  auto stash = [&](int buf, int kt) {
    bf16_t* xt = tiles + buf * buf_elems;
    bf16_t* wt = xt + xt_elems;
    float* nt_ = reinterpret_cast<float*>(wt + wt_elems);
    const bool tail = (kt + 1) * BK > d;  // uniform
#pragma unroll
    for (int u = 0; u < kMaxLoads; ++u) {
      const int id = tid + u * kRouteThreads;
      u32x4_t v = rbuf[u];
      if (id < x_chunks) {
        if (tail && kt * BK + (id % CPR) * 8 >= d) v = u32x4_t{0, 0, 0, 0};
        *reinterpret_cast<u32x4_t*>(&xt[rt_off<BK>(id / CPR, id % CPR)]) = v;
      } else if (id < x_chunks + w_chunks) {
        const int wid = id - x_chunks;
        if (tail && kt * BK + (wid % CPR) * 8 >= d) v = u32x4_t{0, 0, 0, 0};
        *reinterpret_cast<u32x4_t*>(&wt[rt_off<BK>(wid / CPR, wid % CPR)]) = v;
      } else if (id < x_chunks + w_chunks + n_chunks) {
        const int nid = id - x_chunks - w_chunks;
        if (tail && kt * BK + nid * 4 >= d) v = u32x4_t{0, 0, 0, 0};
        *reinterpret_cast<u32x4_t*>(&nt_[nid * 4]) = v;
      }
    }
  };

  constexpr int kMaxTilesPerWave = TPW;
  double acc[kMaxTilesPerWave][16];
#pragma unroll
  for (int e = 0; e < kMaxTilesPerWave; ++e)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[e][i] = 0.0;
  // null row: thread (token tid/4, part tid%4), fp64
  const int nl_tok = tid >> 2, nl_part = tid & 3;
  double nacc = 0.0;

  fetch(0);
  stash(0, 0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) fetch(kt + 1);
    const bf16_t* xt = tiles + buf * buf_elems;
    const bf16_t* wt = xt + xt_elems;
    const float* wn = reinterpret_cast<const float*>(wt + wt_elems);
#pragma unroll
    for (int ti = 0; ti < kMaxTilesPerWave; ++ti) {
      const int et = eg + 2 * ti;
      if (et >= n_et) break;
      f32x16_t part = {};
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int ch = ks * 2 + half;
        const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(&xt[rt_off<BK>(th * 32 + l32, ch)]);
        const int er = et * 32 + l32;
        const bf16x8_t b2 = *reinterpret_cast<const bf16x8_t*>(&wt[rt_off<BK>(2 * Np + er, ch)]);
        const bf16x8_t b1 = *reinterpret_cast<const bf16x8_t*>(&wt[rt_off<BK>(Np + er, ch)]);
        const bf16x8_t b0 = *reinterpret_cast<const bf16x8_t*>(&wt[rt_off<BK>(er, ch)]);
        part = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, b2, part, 0, 0, 0);
        part = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, b1, part, 0, 0, 0);
        part = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, b0, part, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[ti][i] += (double)part[i];
    }
    // null row over this K tile (zero-padded past d): 16 columns per thread for BK = 64
    {
#pragma unroll
      for (int c = nl_part; c < CPR; c += 4) {
        const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(&xt[rt_off<BK>(nl_tok, c)]);
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
    if (kt + 1 < nk) stash(buf ^ 1, kt + 1);
    __syncthreads();
  }
  // logits to LDS: lane holds expert column et*32 + l32, token rows 8*(i/4) + 4*half + i%4
#pragma unroll
  for (int ti = 0; ti < kMaxTilesPerWave; ++ti) {
    const int et = eg + 2 * ti;
    if (et >= n_et) break;
    const int er = et * 32 + l32;
    if (er < N) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tr = th * 32 + 8 * (i / 4) + 4 * half + (i % 4);
        sl[tr * ld + er] = (float)acc[ti][i];
      }
    }
  }
  {
    const double a01 = nacc + __shfl_xor(nacc, 1, kWave);
    const double sum = a01 + __shfl_xor(a01, 2, kWave);
    if (nl_part == 0 && nl_tok < nt) {
      double vv = sum + (double)a.null_bias;
      if (a.null_bias_tok) vv += (double)a.null_bias_tok[t0 + nl_tok];
      sl[nl_tok * ld + N] = (float)vv;
    }
  }
  __syncthreads();
  route_epilogue<FUSED, KMAX>(a, sl, ld, nt, t0, cnt_lds, wacc);
}

// float32 x: plain dot products (small workloads), then the same epilogue.
template <bool FUSED, int KMAX>
__global__ void __launch_bounds__(kRouteThreads)
route_simt_kernel(RouteKernelArgs a, const float* __restrict__ xf, const float* __restrict__ w) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const int N = a.N, d = a.d, ld = N + 1;
  float* sl = reinterpret_cast<float*>(smem_raw);
  double* wacc = reinterpret_cast<double*>(sl + ((kRouteBT * ld + 1) & ~1));
  int* cnt_lds = reinterpret_cast<int*>(wacc + (FUSED ? N + 3 : 0));
  if (FUSED)
    for (int i = threadIdx.x; i < N + a.M; i += blockDim.x) cnt_lds[i] = 0;
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
  route_epilogue<FUSED, KMAX>(a, sl, ld, nt, t0, cnt_lds, wacc);
}

template <bool FUSED, int KMAX>
__global__ void __launch_bounds__(kRouteThreads)
route_from_logits_kernel(RouteKernelArgs a, const float* __restrict__ logits) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const int N = a.N, ld = N + 1;
  float* sl = reinterpret_cast<float*>(smem_raw);
  double* wacc = reinterpret_cast<double*>(sl + ((kRouteBT * ld + 1) & ~1));
  int* cnt_lds = reinterpret_cast<int*>(wacc + (FUSED ? N + 3 : 0));
  if (FUSED)
    for (int i = threadIdx.x; i < N + a.M; i += blockDim.x) cnt_lds[i] = 0;
  const int64_t t0 = (int64_t)blockIdx.x * kRouteBT;
  const int nt = (int)min<int64_t>(kRouteBT, a.T - t0);
  for (int i = threadIdx.x; i < nt * ld; i += blockDim.x) sl[i] = logits[t0 * ld + i];
  __syncthreads();
  route_epilogue<FUSED, KMAX>(a, sl, ld, nt, t0, cnt_lds, wacc);
}

size_t route_split_bytes(int N, int d) {
  const int Np = (N + 31) / 32 * 32;
  return (size_t)3 * Np * d * sizeof(bf16_t);
}

// K tile width of the MFMA router: keeps two buffers of the weight tile in LDS.
static int route_bk(int Np) { return Np <= 64 ? 64 : (Np <= 128 ? 32 : 16); }

static size_t route_lds_bytes(const RouteArgs& r, bool mfma) {
  const int Np = (r.N + 31) / 32 * 32;
  const int ld = r.N + 1;
  size_t b = 0;
  if (mfma) b += (size_t)2 * ((kRouteBT + 3 * Np) * route_bk(Np) + 2 * route_bk(Np)) * sizeof(bf16_t);
  b += (size_t)((kRouteBT * ld + 1) & ~1) * sizeof(float);
  if (r.fused) b += (size_t)(r.N + 3) * sizeof(double) + (size_t)(r.N + r.M) * sizeof(int);
  return b;
}

template <typename F>
static void allow_lds(F* kernel, size_t lds) {
  if (lds > 65536)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

hipError_t launch_route(const RouteArgs& r, hipStream_t stream) {
  const unsigned nblk = (unsigned)((r.T + kRouteBT - 1) / kRouteBT);
  const int Np = (r.N + 31) / 32 * 32;
  const bool mfma = !r.logits_in && r.bf16;
  RouteKernelArgs a{static_cast<const bf16_t*>(r.x), r.w_split,
                    r.w_router ? r.w_router + (int64_t)r.N * r.d : nullptr, r.null_bias,
                    r.null_bias_tok, r.T, r.d, r.N, Np, r.M, r.K, 1, r.logits_out,
                    r.topk_idx, r.topk_w, r.n_real, r.chunk_hist, r.acc, r.counts};
  const size_t lds = route_lds_bytes(r, mfma);
  // prep: split the router weight (bf16 scoring) and clear the fused accumulators
  const int nacc = r.fused ? r.N + 3 : 0, ncnt = r.fused ? r.N + r.M : 0;
  if (mfma || r.fused) {
    const int64_t n = mfma ? (int64_t)Np * r.d : std::max(nacc, ncnt);
    const unsigned sblk = (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 1024));
    route_prep_kernel<<<sblk, 256, 0, stream>>>(r.w_router, mfma ? r.w_split : nullptr, r.N, Np,
                                                r.d, r.acc, nacc, r.counts, ncnt);
  }
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
    route_from_logits_kernel<F_, KM_><<<nblk, kRouteThreads, lds, stream>>>(a, r.logits_in); \
  } while (0)
#define MOE_SIMT_LAUNCH(F_, KM_)                                                          \
  do {                                                                                    \
    allow_lds(route_simt_kernel<F_, KM_>, lds);                                           \
    route_simt_kernel<F_, KM_><<<nblk, kRouteThreads, lds, stream>>>(                     \
        a, static_cast<const float*>(r.x), r.w_router);                                   \
  } while (0)
#define MOE_ROUTE_LAUNCH(F_, BK_, TPW_, KM_)                                              \
  do {                                                                                    \
    allow_lds(route_mfma_kernel<F_, BK_, TPW_, KM_>, lds);                                \
    route_mfma_kernel<F_, BK_, TPW_, KM_><<<nblk, kRouteThreads, lds, stream>>>(a);       \
  } while (0)
  if (r.logits_in) {
    if (r.fused) MOE_KMAX_SWITCH(MOE_LOGITS_LAUNCH, true);
    else MOE_KMAX_SWITCH(MOE_LOGITS_LAUNCH, false);
  } else if (r.bf16) {
    const int bk = route_bk(Np);
    const int chunks = (kRouteBT + 3 * Np) * bk / 8 + bk / 4;
    if (chunks > kRouteMaxLoads * kRouteThreads) return hipErrorInvalidValue;
    if (r.fused) {
      if (bk == 64) MOE_KMAX_SWITCH(MOE_ROUTE_LAUNCH, true, 64, 1);
      else if (bk == 32) MOE_KMAX_SWITCH(MOE_ROUTE_LAUNCH, true, 32, 2);
      else MOE_KMAX_SWITCH(MOE_ROUTE_LAUNCH, true, 16, 4);
    } else {
      if (bk == 64) MOE_KMAX_SWITCH(MOE_ROUTE_LAUNCH, false, 64, 1);
      else if (bk == 32) MOE_KMAX_SWITCH(MOE_ROUTE_LAUNCH, false, 32, 2);
      else MOE_KMAX_SWITCH(MOE_ROUTE_LAUNCH, false, 16, 4);
    }
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

}  // namespace moe
