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
// MI355X design. x is bf16 and the router weight float32. Every bf16 x bf16
// product is exact in float32, and an fp32 weight splits exactly into three
// bf16 parts (hi + mid + lo, each the bf16 rounding of what is left), so three
// bf16 MFMAs give the products exactly at MFMA rate instead of the slower
// float32 path. MFMA partial sums over 64-wide K blocks are accumulated across
// blocks in fp64, which keeps the logits within a few 1e-7 of the exact value
// (fp32 accumulation over d = 2048 terms drifts by a few 1e-6, too close to the
// 1e-5 near-tie margin of the routing parity rule). The null row is an fp64
// dot product on the vector ALUs. Each workgroup scores 64 tokens; the logits go through LDS to
// the epilogue, where one wavefront handles one token with a lane per expert.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kRouteBT = 64;       // tokens per workgroup
constexpr int kRouteThreads = 256;

// W [N+1][d] float32 -> W3 [3][Np][d] bf16 (hi, mid, lo), rows >= N zero.
__global__ void split_router_kernel(const float* __restrict__ w, bf16_t* __restrict__ w3,
                                    int N, int Np, int d) {
  const int64_t total = (int64_t)Np * d;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int row = (int)(i / d);
    const float v = row < N ? w[i] : 0.0f;
    const bf16_t hi = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(hi);
    const bf16_t mid = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(mid);
    const bf16_t lo = f32_to_bf16(r2);
    w3[i] = hi;
    w3[total + i] = mid;
    w3[2 * total + i] = lo;
  }
}

// One wavefront selects one token from its logits row s[0..N] in LDS.
__device__ void select_token(const float* s, int N, int M, int K, int64_t t,
                             int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                             int32_t* __restrict__ n_real) {
  const int lane = threadIdx.x & (kWave - 1);
  const float snull = s[N];
  constexpr int QMAX = (MOE_MAX_EXPERTS + kWave - 1) / kWave;
  int rank[QMAX];
  float val[QMAX];
  int c = 0;
  float vmax = -INFINITY;
#pragma unroll
  for (int q = 0; q < QMAX; ++q) {
    rank[q] = 0x7fffffff;
    val[q] = 0.0f;
    if (q * kWave < N) {
      const int j = lane + q * kWave;
      const bool valid = j < N;
      const float v = valid ? s[j] : 0.0f;
      int rk = 0;
      for (int i = 0; i < N; ++i) {
        const float u = s[i];
        rk += (u > v) | ((u == v) & (i < j));
      }
      if (valid) {
        rank[q] = rk;
        val[q] = v;
        vmax = fmaxf(vmax, v);
      }
      c += __popcll(ballot(valid && v > snull));
    }
  }
  const int r = (M == 0) ? K : min(K, max(c, K - M));
  const float m = wave_max(vmax);
  double e[QMAX];
  double part = 0.0;
#pragma unroll
  for (int q = 0; q < QMAX; ++q) {
    e[q] = (rank[q] < r) ? exp((double)val[q] - (double)m) : 0.0;
    part += e[q];
  }
  const double tot = wave_sum_double(part);
  int32_t* idx_row = topk_idx + t * K;
  float* w_row = topk_w + t * K;
#pragma unroll
  for (int q = 0; q < QMAX; ++q) {
    if (rank[q] < r) {
      idx_row[rank[q]] = lane + q * kWave;
      w_row[rank[q]] = (float)(e[q] / tot);
    }
  }
  if (lane < K - r) {
    idx_row[r + lane] = N + lane;
    w_row[r + lane] = 0.0f;
  }
  if (lane == 0 && n_real) n_real[t] = r;
}

// Epilogue shared by every scoring path: logits of `nt` tokens sit in sl[nt][ld].
__device__ void route_epilogue(const float* sl, int ld, int nt, int64_t t0, int N, int M, int K,
                               float* __restrict__ logits_out, int32_t* __restrict__ topk_idx,
                               float* __restrict__ topk_w, int32_t* __restrict__ n_real) {
  if (logits_out) {
    const int w = N + 1;
    for (int i = threadIdx.x; i < nt * w; i += blockDim.x)
      logits_out[(t0 + i / w) * w + i % w] = sl[(i / w) * ld + i % w];
  }
  const int wave = threadIdx.x / kWave;
  const int nwaves = blockDim.x / kWave;
  for (int tl = wave; tl < nt; tl += nwaves)
    select_token(sl + tl * ld, N, M, K, t0 + tl, topk_idx, topk_w, n_real);
}

// bf16 x: three-way split MFMA scoring of the N real rows + fp32 null row.
__global__ void __launch_bounds__(kRouteThreads)
route_mfma_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ w3,
                  const float* __restrict__ w_null, float null_bias,
                  const float* __restrict__ null_bias_tok, int64_t T, int d, int N, int Np,
                  int M, int K, float* __restrict__ logits_out, int32_t* __restrict__ topk_idx,
                  float* __restrict__ topk_w, int32_t* __restrict__ n_real) {
  extern __shared__ float sl[];
  const int ld = N + 1;
  const int64_t t0 = (int64_t)blockIdx.x * kRouteBT;
  const int nt = (int)min<int64_t>(kRouteBT, T - t0);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int wt = wave & 1, we = wave >> 1;
  const int nch = d / 8;          // 16-byte chunks per row
  const int nsteps = (nch + 1) / 2;
  const int64_t trow = min<int64_t>(t0 + wt * 32 + (lane & 31), T - 1);
  const bf16x8_t* ap = reinterpret_cast<const bf16x8_t*>(x + trow * d);
  const int half = lane >> 5;
  const int64_t plane = (int64_t)Np * d;
  for (int et = we; et * 32 < Np; et += 2) {
    const int erow = et * 32 + (lane & 31);
    const bf16x8_t* b0 = reinterpret_cast<const bf16x8_t*>(w3 + (int64_t)erow * d);
    const bf16x8_t* b1 = reinterpret_cast<const bf16x8_t*>(w3 + plane + (int64_t)erow * d);
    const bf16x8_t* b2 = reinterpret_cast<const bf16x8_t*>(w3 + 2 * plane + (int64_t)erow * d);
    // fp32 MFMA partial sums over 64-wide K blocks, accumulated across blocks in fp64
    double acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0;
    for (int kb = 0; kb < nsteps; kb += 4) {
      f32x16_t part = {};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int cidx = 2 * (kb + u) + half;
        bf16x8_t a = {}, v0 = {}, v1 = {}, v2 = {};
        if (kb + u < nsteps && cidx < nch) {
          a = ap[cidx];
          v0 = b0[cidx];
          v1 = b1[cidx];
          v2 = b2[cidx];
        }
        part = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, v2, part, 0, 0, 0);
        part = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, v1, part, 0, 0, 0);
        part = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, v0, part, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] += (double)part[i];
    }
    const int e = et * 32 + (lane & 31);
    if (e < N) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tl = wt * 32 + 8 * (i / 4) + 4 * half + (i % 4);
        sl[tl * ld + e] = (float)acc[i];
      }
    }
  }
  // Null row: x (bf16) times the float32 row, each product exact in fp64, summed in
  // fp64 by 4 threads per token and combined in a fixed order.
  {
    const int tl = threadIdx.x >> 2, part = threadIdx.x & 3;
    const int64_t t = min<int64_t>(t0 + tl, T - 1);
    const bf16_t* xr = x + t * d;
    double acc = 0.0;
    for (int c = part; c < nch; c += 4) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(xr + c * 8);
      const f32x4_t w0 = *reinterpret_cast<const f32x4_t*>(w_null + c * 8);
      const f32x4_t w1 = *reinterpret_cast<const f32x4_t*>(w_null + c * 8 + 4);
      const float wv[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        acc = fma((double)__uint_as_float(v[h] << 16), (double)wv[2 * h], acc);
        acc = fma((double)__uint_as_float(v[h] & 0xffff0000u), (double)wv[2 * h + 1], acc);
      }
    }
    const double a01 = acc + __shfl_xor(acc, 1, kWave);
    const double sum = a01 + __shfl_xor(a01, 2, kWave);
    if (part == 0 && tl < nt) {
      double v = sum + (double)null_bias;
      if (null_bias_tok) v += (double)null_bias_tok[t0 + tl];
      sl[tl * ld + N] = (float)v;
    }
  }
  __syncthreads();
  route_epilogue(sl, ld, nt, t0, N, M, K, logits_out, topk_idx, topk_w, n_real);
}

// float32 (or any element type) x: plain dot products; meant for small workloads.
template <typename XT>
__global__ void __launch_bounds__(kRouteThreads)
route_simt_kernel(const XT* __restrict__ x, const float* __restrict__ w, float null_bias,
                  const float* __restrict__ null_bias_tok, int64_t T, int d, int N, int M, int K,
                  float* __restrict__ logits_out, int32_t* __restrict__ topk_idx,
                  float* __restrict__ topk_w, int32_t* __restrict__ n_real) {
  extern __shared__ float sl[];
  const int ld = N + 1;
  const int64_t t0 = (int64_t)blockIdx.x * kRouteBT;
  const int nt = (int)min<int64_t>(kRouteBT, T - t0);
  for (int i = threadIdx.x; i < nt * ld; i += blockDim.x) {
    const int tl = i / ld, j = i % ld;
    const int64_t t = t0 + tl;
    float acc = 0.0f;
    for (int k = 0; k < d; ++k) acc = fmaf(Elem<XT>::load(x, t * d + k), w[(int64_t)j * d + k], acc);
    if (j == N) {
      acc += null_bias;
      if (null_bias_tok) acc += null_bias_tok[t];
    }
    sl[tl * ld + j] = acc;
  }
  __syncthreads();
  route_epilogue(sl, ld, nt, t0, N, M, K, logits_out, topk_idx, topk_w, n_real);
}

__global__ void __launch_bounds__(kRouteThreads)
route_from_logits_kernel(const float* __restrict__ logits, int64_t T, int N, int M, int K,
                         float* __restrict__ logits_out, int32_t* __restrict__ topk_idx,
                         float* __restrict__ topk_w, int32_t* __restrict__ n_real) {
  extern __shared__ float sl[];
  const int ld = N + 1;
  const int64_t t0 = (int64_t)blockIdx.x * kRouteBT;
  const int nt = (int)min<int64_t>(kRouteBT, T - t0);
  for (int i = threadIdx.x; i < nt * ld; i += blockDim.x) sl[i] = logits[t0 * ld + i];
  __syncthreads();
  route_epilogue(sl, ld, nt, t0, N, M, K, logits_out, topk_idx, topk_w, n_real);
}

size_t route_split_bytes(int N, int d) {
  const int Np = (N + 31) / 32 * 32;
  return (size_t)3 * Np * d * sizeof(bf16_t);
}

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  const unsigned nblk = (unsigned)((a.T + kRouteBT - 1) / kRouteBT);
  const size_t lds = (size_t)kRouteBT * (a.N + 1) * sizeof(float);
  if (a.logits_in) {
    route_from_logits_kernel<<<nblk, kRouteThreads, lds, stream>>>(
        a.logits_in, a.T, a.N, a.M, a.K, a.logits_out, a.topk_idx, a.topk_w, a.n_real);
  } else if (a.bf16) {
    const int Np = (a.N + 31) / 32 * 32;
    const int64_t n = (int64_t)Np * a.d;
    const unsigned sblk = (unsigned)std::min<int64_t>((n + 255) / 256, 1024);
    split_router_kernel<<<sblk, 256, 0, stream>>>(a.w_router, a.w_split, a.N, Np, a.d);
    route_mfma_kernel<<<nblk, kRouteThreads, lds, stream>>>(
        static_cast<const bf16_t*>(a.x), a.w_split, a.w_router + (int64_t)a.N * a.d, a.null_bias,
        a.null_bias_tok, a.T, a.d, a.N, Np, a.M, a.K, a.logits_out, a.topk_idx, a.topk_w,
        a.n_real);
  } else {
    route_simt_kernel<float><<<nblk, kRouteThreads, lds, stream>>>(
        static_cast<const float*>(a.x), a.w_router, a.null_bias, a.null_bias_tok, a.T, a.d, a.N,
        a.M, a.K, a.logits_out, a.topk_idx, a.topk_w, a.n_real);
  }
  return hipGetLastError();
}

}  // namespace moe
