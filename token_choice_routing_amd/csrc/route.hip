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
//  * A workgroup scores 64 tokens. Its four wavefronts split the work into
//    (32-expert tile, K slice) pairs; the K slices are added in a fixed order
//    through LDS. Fragment loads for the next K block are issued before the
//    MFMAs of the current one.
//  * Epilogue: one wavefront per token. The chosen reals are found by r rounds
//    of a wavefront arg-max over 64-bit keys (order-preserving bits of the
//    logit, then the complemented expert index, so ties go to the lower index);
//    no sort and no O(N) loop per lane.
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

struct AuxPartial {  // per-lane running sums of one wavefront (fused mode)
  double psum[kQ];
  double pnull, lz;
  int nreal;
};

// One wavefront selects one token from its logits row s[0..N] (LDS).
template <bool FUSED>
__device__ void select_token(const float* s, int N, int M, int K, int64_t t,
                             int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                             int32_t* __restrict__ n_real, AuxPartial& ap, int* cnt_lds) {
  const int lane = threadIdx.x & (kWave - 1);
  const float snull = s[N];
  float v[kQ];
  uint64_t key[kQ];
  int c = 0;
  float vmax = -INFINITY;
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int j = lane + q * kWave;
    const bool valid = j < N;
    v[q] = valid ? s[j] : -INFINITY;
    key[q] = valid ? (((uint64_t)ordered_bits(v[q]) << 32) | (0xffffffffu - (uint32_t)j)) : 0ull;
    if (q * kWave < N) {
      c += __popcll(ballot(valid && v[q] > snull));
      vmax = fmaxf(vmax, v[q]);
    }
  }
  vmax = wave_max(vmax);
  const int r = (M == 0) ? K : min(K, max(c, K - M));
  int my_idx = 0;
  float my_v = 0.0f;
  for (int i = 0; i < r; ++i) {
    uint64_t best = 0;
#pragma unroll
    for (int q = 0; q < kQ; ++q) best = key[q] > best ? key[q] : best;
    best = wave_max_u64(best);
#pragma unroll
    for (int q = 0; q < kQ; ++q)
      if (key[q] == best) key[q] = 0;
    if (lane == i) {
      my_idx = (int)(0xffffffffu - (uint32_t)best);
      my_v = from_ordered_bits((uint32_t)(best >> 32));
    }
  }
  // weights: softmax over the chosen reals in fp64 from the fp32 logits (max = vmax)
  const double e = lane < r ? exp((double)my_v - (double)vmax) : 0.0;
  const double tot = wave_sum_double(e);
  int32_t* idx_row = topk_idx + t * K;
  float* w_row = topk_w + t * K;
  if (lane < r) {
    idx_row[lane] = my_idx;
    w_row[lane] = (float)(e / tot);
  } else if (lane < K) {
    idx_row[lane] = N + (lane - r);
    w_row[lane] = 0.0f;
  }
  if (lane == 0 && n_real) n_real[t] = r;
  if (FUSED) {
    // pool softmax over [reals, null x M] in fp32, accumulated per lane in fp64
    const float mp = M > 0 ? fmaxf(vmax, snull) : vmax;
    float ex[kQ];
    double part = 0.0;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      ex[q] = (lane + q * kWave < N) ? expf(v[q] - mp) : 0.0f;
      part += (double)ex[q];
    }
    const float en = M > 0 ? expf(snull - mp) : 0.0f;
    const double z = wave_sum_double(part) + (double)M * (double)en;
    const double iz = 1.0 / z;
#pragma unroll
    for (int q = 0; q < kQ; ++q) ap.psum[q] += (double)ex[q] * iz;
    if (lane == 0) {
      ap.pnull += (double)en * iz;
      const double lse = (double)mp + log(z);
      ap.lz += lse * lse;
      ap.nreal += r;
    }
    if (lane < r)
      atomicAdd(&cnt_lds[my_idx], 1);
    else if (lane < K)
      atomicAdd(&cnt_lds[N + (lane - r)], 1);
  }
}

struct RouteKernelArgs {
  const bf16_t* x;
  const bf16_t* w3;
  const float* w_null;
  float null_bias;
  const float* null_bias_tok;
  int64_t T;
  int d, N, Np, M, K, ks;  // ks: K slices per expert tile
  float* logits_out;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* n_real;
  int32_t* chunk_hist;     // fused: [blocks][N]
  uint64_t* acc;           // fused: [N + 3] fixed-point sums
  int32_t* counts;         // fused: [N + M] pool slot counts
};

template <bool FUSED>
__device__ void route_epilogue(const RouteKernelArgs& a, float* sl, int ld, int nt, int64_t t0,
                               int* cnt_lds, double* wacc) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int N = a.N, M = a.M, P = N + M;
  if (a.logits_out) {
    const int w = N + 1;
    for (int i = threadIdx.x; i < nt * w; i += blockDim.x)
      a.logits_out[(t0 + i / w) * w + i % w] = sl[(i / w) * ld + i % w];
  }
  AuxPartial ap;
#pragma unroll
  for (int q = 0; q < kQ; ++q) ap.psum[q] = 0.0;
  ap.pnull = ap.lz = 0.0;
  ap.nreal = 0;
  for (int tl = wave; tl < nt; tl += kRouteThreads / kWave)
    select_token<FUSED>(sl + tl * ld, N, M, a.K, t0 + tl, a.topk_idx, a.topk_w, a.n_real, ap,
                        cnt_lds);
  if (!FUSED) return;
  const int rd = N + 3;
#pragma unroll
  for (int q = 0; q < kQ; ++q)
    if (lane + q * kWave < N) wacc[wave * rd + lane + q * kWave] = ap.psum[q];
  if (lane == 0) {
    wacc[wave * rd + N] = ap.pnull;
    wacc[wave * rd + N + 1] = ap.lz;
    wacc[wave * rd + N + 2] = (double)ap.nreal;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < rd; i += blockDim.x) {
    double s = 0.0;
    for (int w = 0; w < kRouteThreads / kWave; ++w) s += wacc[w * rd + i];
    const double scale = (i == N + 1) ? kAuxZScale : (i == N + 2 ? 1.0 : kAuxPScale);
    const uint64_t q = (uint64_t)(s * scale + 0.5);
    if (q) atomicAdd(reinterpret_cast<unsigned long long*>(&a.acc[i]), (unsigned long long)q);
  }
  for (int i = threadIdx.x; i < P; i += blockDim.x) {
    const int cval = cnt_lds[i];
    if (i < N) a.chunk_hist[(int64_t)blockIdx.x * N + i] = cval;
    if (cval) atomicAdd(&a.counts[i], cval);
  }
}

// bf16 x: three-way split MFMA scoring of the N real rows + fp64 null row.
template <bool FUSED>
__global__ void __launch_bounds__(kRouteThreads)
route_mfma_kernel(RouteKernelArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const int N = a.N, d = a.d, Np = a.Np, ks = a.ks;
  const int ld = N + 1;
  const int n_et = Np / 32;
  // LDS: partial K-slice sums [ks-1][64][Np] doubles, logits [64][ld] floats,
  // fused: wave partials [4][N+3] doubles and pool counts [N+M] ints
  double* part = reinterpret_cast<double*>(smem_raw);
  float* sl = reinterpret_cast<float*>(part + (size_t)(ks - 1) * kRouteBT * Np);
  double* wacc = reinterpret_cast<double*>(sl + ((kRouteBT * ld + 1) & ~1));
  int* cnt_lds = reinterpret_cast<int*>(wacc + (FUSED ? 4 * (N + 3) : 0));
  if (FUSED)
    for (int i = threadIdx.x; i < N + a.M; i += blockDim.x) cnt_lds[i] = 0;

  const int64_t T = a.T;
  const int64_t t0 = (int64_t)blockIdx.x * kRouteBT;
  const int nt = (int)min<int64_t>(kRouteBT, T - t0);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int half = lane >> 5, l32 = lane & 31;
  const int nch = d / 8;               // 16-byte chunks per row
  const int nsteps = (nch + 1) / 2;    // 16-wide K steps
  const int steps_per_slice = (nsteps + ks - 1) / ks;
  const bf16x8_t* ap0 = reinterpret_cast<const bf16x8_t*>(a.x + min<int64_t>(t0 + l32, T - 1) * d);
  const bf16x8_t* ap1 =
      reinterpret_cast<const bf16x8_t*>(a.x + min<int64_t>(t0 + 32 + l32, T - 1) * d);
  const int64_t plane = (int64_t)Np * d;

  // With ks > 1 there are exactly four (tile, slice) items, one per wavefront, and
  // every wavefront passes the one barrier below; with ks == 1 there is none.
  for (int item = wave; item < n_et * ks; item += kRouteThreads / kWave) {
    const int et = item % n_et, kq = item / n_et;
    const int erow = et * 32 + l32;
    const bf16x8_t* b0 = reinterpret_cast<const bf16x8_t*>(a.w3 + (int64_t)erow * d);
    const bf16x8_t* b1 = reinterpret_cast<const bf16x8_t*>(a.w3 + plane + (int64_t)erow * d);
    const bf16x8_t* b2 = reinterpret_cast<const bf16x8_t*>(a.w3 + 2 * plane + (int64_t)erow * d);
    const int s_begin = kq * steps_per_slice, s_end = min(nsteps, s_begin + steps_per_slice);
    double acc0[16], acc1[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc0[i] = acc1[i] = 0.0;
    // fragments of 2 K steps, double-buffered in registers
    bf16x8_t fa0[2], fa1[2], fb0[2], fb1[2], fb2[2];
    auto fetch = [&](int s, bf16x8_t* xa0, bf16x8_t* xa1, bf16x8_t* xb0, bf16x8_t* xb1,
                     bf16x8_t* xb2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int cidx = 2 * (s + u) + half;
        if (s + u < s_end && cidx < nch) {
          xa0[u] = ap0[cidx];
          xa1[u] = ap1[cidx];
          xb0[u] = b0[cidx];
          xb1[u] = b1[cidx];
          xb2[u] = b2[cidx];
        } else {
          xa0[u] = xa1[u] = xb0[u] = xb1[u] = xb2[u] = bf16x8_t{};
        }
      }
    };
    if (s_begin < s_end) fetch(s_begin, fa0, fa1, fb0, fb1, fb2);
    for (int s = s_begin; s < s_end; s += 2) {
      bf16x8_t na0[2], na1[2], nb0[2], nb1[2], nb2[2];
      if (s + 2 < s_end) fetch(s + 2, na0, na1, nb0, nb1, nb2);
      f32x16_t p0 = {}, p1 = {};
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0[u], fb2[u], p0, 0, 0, 0);
        p1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1[u], fb2[u], p1, 0, 0, 0);
        p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0[u], fb1[u], p0, 0, 0, 0);
        p1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1[u], fb1[u], p1, 0, 0, 0);
        p0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0[u], fb0[u], p0, 0, 0, 0);
        p1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1[u], fb0[u], p1, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        acc0[i] += (double)p0[i];
        acc1[i] += (double)p1[i];
      }
      if (s + 2 < s_end) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          fa0[u] = na0[u];
          fa1[u] = na1[u];
          fb0[u] = nb0[u];
          fb1[u] = nb1[u];
          fb2[u] = nb2[u];
        }
      }
    }
    // lane holds expert column erow, token rows 8*(i/4) + 4*half + i%4 (+32 for acc1)
    if (kq > 0) {
      double* pp = part + (size_t)(kq - 1) * kRouteBT * Np;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tr = 8 * (i / 4) + 4 * half + (i % 4);
        pp[tr * Np + erow] = acc0[i];
        pp[(tr + 32) * Np + erow] = acc1[i];
      }
      __syncthreads();
    } else {
      if (ks > 1) __syncthreads();  // the other slices of this tile are in LDS
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tr = 8 * (i / 4) + 4 * half + (i % 4);
        double s0 = acc0[i], s1 = acc1[i];
        for (int k2 = 1; k2 < ks; ++k2) {
          const double* pp = part + (size_t)(k2 - 1) * kRouteBT * Np;
          s0 += pp[tr * Np + erow];
          s1 += pp[(tr + 32) * Np + erow];
        }
        if (erow < N) {
          sl[tr * ld + erow] = (float)s0;
          sl[(tr + 32) * ld + erow] = (float)s1;
        }
      }
    }
  }
  // Null row: x (bf16) times the float32 row, each product exact in fp64, summed
  // in fp64 by 4 threads per token and combined in a fixed order.
  {
    const int tl = threadIdx.x >> 2, prt = threadIdx.x & 3;
    const int64_t t = min<int64_t>(t0 + tl, T - 1);
    const bf16_t* xr = a.x + t * d;
    double acc = 0.0;
    for (int c = prt; c < nch; c += 4) {
      const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xr + c * 8);
      const f32x4_t w0 = *reinterpret_cast<const f32x4_t*>(a.w_null + c * 8);
      const f32x4_t w1 = *reinterpret_cast<const f32x4_t*>(a.w_null + c * 8 + 4);
      const float wv[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        acc = fma((double)__uint_as_float(xv[h] << 16), (double)wv[2 * h], acc);
        acc = fma((double)__uint_as_float(xv[h] & 0xffff0000u), (double)wv[2 * h + 1], acc);
      }
    }
    const double a01 = acc + __shfl_xor(acc, 1, kWave);
    const double sum = a01 + __shfl_xor(a01, 2, kWave);
    if (prt == 0 && tl < nt) {
      double vv = sum + (double)a.null_bias;
      if (a.null_bias_tok) vv += (double)a.null_bias_tok[t0 + tl];
      sl[tl * ld + N] = (float)vv;
    }
  }
  __syncthreads();
  route_epilogue<FUSED>(a, sl, ld, nt, t0, cnt_lds, wacc);
}

// float32 x: plain dot products (small workloads), then the same epilogue.
template <bool FUSED>
__global__ void __launch_bounds__(kRouteThreads)
route_simt_kernel(RouteKernelArgs a, const float* __restrict__ xf, const float* __restrict__ w) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const int N = a.N, d = a.d, ld = N + 1;
  float* sl = reinterpret_cast<float*>(smem_raw);
  double* wacc = reinterpret_cast<double*>(sl + ((kRouteBT * ld + 1) & ~1));
  int* cnt_lds = reinterpret_cast<int*>(wacc + (FUSED ? 4 * (N + 3) : 0));
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
  route_epilogue<FUSED>(a, sl, ld, nt, t0, cnt_lds, wacc);
}

template <bool FUSED>
__global__ void __launch_bounds__(kRouteThreads)
route_from_logits_kernel(RouteKernelArgs a, const float* __restrict__ logits) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const int N = a.N, ld = N + 1;
  float* sl = reinterpret_cast<float*>(smem_raw);
  double* wacc = reinterpret_cast<double*>(sl + ((kRouteBT * ld + 1) & ~1));
  int* cnt_lds = reinterpret_cast<int*>(wacc + (FUSED ? 4 * (N + 3) : 0));
  if (FUSED)
    for (int i = threadIdx.x; i < N + a.M; i += blockDim.x) cnt_lds[i] = 0;
  const int64_t t0 = (int64_t)blockIdx.x * kRouteBT;
  const int nt = (int)min<int64_t>(kRouteBT, a.T - t0);
  for (int i = threadIdx.x; i < nt * ld; i += blockDim.x) sl[i] = logits[t0 * ld + i];
  __syncthreads();
  route_epilogue<FUSED>(a, sl, ld, nt, t0, cnt_lds, wacc);
}

size_t route_split_bytes(int N, int d) {
  const int Np = (N + 31) / 32 * 32;
  return (size_t)3 * Np * d * sizeof(bf16_t);
}

static int route_ks(int Np) {
  const int n_et = Np / 32;
  return n_et >= 3 ? 1 : 4 / n_et;
}

static size_t route_lds_bytes(const RouteArgs& r, bool mfma) {
  const int Np = (r.N + 31) / 32 * 32;
  const int ld = r.N + 1;
  size_t b = 0;
  if (mfma) b += (size_t)(route_ks(Np) - 1) * kRouteBT * Np * sizeof(double);
  b += (size_t)((kRouteBT * ld + 1) & ~1) * sizeof(float);
  if (r.fused) b += (size_t)4 * (r.N + 3) * sizeof(double) + (size_t)(r.N + r.M) * sizeof(int);
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
                    r.null_bias_tok, r.T, r.d, r.N, Np, r.M, r.K, route_ks(Np), r.logits_out,
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
  if (r.logits_in) {
    if (r.fused) {
      allow_lds(route_from_logits_kernel<true>, lds);
      route_from_logits_kernel<true><<<nblk, kRouteThreads, lds, stream>>>(a, r.logits_in);
    } else {
      allow_lds(route_from_logits_kernel<false>, lds);
      route_from_logits_kernel<false><<<nblk, kRouteThreads, lds, stream>>>(a, r.logits_in);
    }
  } else if (r.bf16) {
    if (r.fused) {
      allow_lds(route_mfma_kernel<true>, lds);
      route_mfma_kernel<true><<<nblk, kRouteThreads, lds, stream>>>(a);
    } else {
      allow_lds(route_mfma_kernel<false>, lds);
      route_mfma_kernel<false><<<nblk, kRouteThreads, lds, stream>>>(a);
    }
  } else {
    const float* xf = static_cast<const float*>(r.x);
    if (r.fused) {
      allow_lds(route_simt_kernel<true>, lds);
      route_simt_kernel<true><<<nblk, kRouteThreads, lds, stream>>>(a, xf, r.w_router);
    } else {
      allow_lds(route_simt_kernel<false>, lds);
      route_simt_kernel<false><<<nblk, kRouteThreads, lds, stream>>>(a, xf, r.w_router);
    }
  }
  return hipGetLastError();
}

}  // namespace moe
