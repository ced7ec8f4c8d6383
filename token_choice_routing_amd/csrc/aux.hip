// Load-balance and z-loss statistics over the N+M pool.
//
// Paper review "Improving MoE Compute Efficiency by Composing Weight and Data
// Sparsity", section 3, "load-balance loss" and "Z-loss":
//   L_bal = N * sum_{i < N+M} f_i P_i,   L_z = mean_t (log sum_{i < N+M} e^{v_t,i})^2
// where v_t is the pool [s_0..s_{N-1}, s_null repeated M times], P_i the mean
// pool-softmax probability and f_i the fraction of tokens routed to slot i.
// The M null copies share one probability, so the pool softmax needs N+1
// exponentials per token.
//
// Two kernels: each workgroup reduces a contiguous token range in float64 (one
// wavefront per token, lanes over experts, tokens in order), then one
// workgroup adds the per-workgroup partials in workgroup order. Pool-slot counts
// use LDS integer atomics (order-free). Everything is bitwise reproducible.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kAuxThreads = 256;
constexpr int kAuxMaxBlocks = 512;
constexpr int kQ = (MOE_MAX_EXPERTS + kWave - 1) / kWave;

static int aux_blocks(int64_t T) { return (int)std::max<int64_t>(1, std::min<int64_t>((T + 63) / 64, kAuxMaxBlocks)); }

// per-block record: [N] real P sums, null P sum, sum lse^2, sum n_real (doubles), then counts
__host__ __device__ inline size_t aux_rec_doubles(int N) { return (size_t)N + 3; }

size_t aux_ws_bytes(int64_t T, int N, int M) {
  const int nb = aux_blocks(T);
  return (size_t)nb * aux_rec_doubles(N) * sizeof(double) + (size_t)nb * (N + M) * sizeof(int32_t);
}

__global__ void __launch_bounds__(kAuxThreads)
aux_partial_kernel(const float* __restrict__ logits, const int32_t* __restrict__ topk_idx,
                   int64_t T, int N, int M, int K, double* __restrict__ rec,
                   int32_t* __restrict__ rec_counts) {
  extern __shared__ double smd[];
  const int nw = kAuxThreads / kWave;
  double* wacc = smd;                                           // [nw][N+3]
  int* cnt = reinterpret_cast<int*>(smd + nw * aux_rec_doubles(N));  // [N+M]
  const int P = N + M;
  for (int i = threadIdx.x; i < P; i += blockDim.x) cnt[i] = 0;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int64_t per = (T + gridDim.x - 1) / gridDim.x;
  const int64_t tb = blockIdx.x * per, te = min<int64_t>(T, tb + per);
  double psum[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) psum[q] = 0.0;
  double pnull = 0.0, lz = 0.0;
  int nreal = 0;
  __syncthreads();
  for (int64_t t = tb + wave; t < te; t += nw) {
    const float* s = logits + t * (N + 1);
    float v[kQ];
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int j = lane + q * kWave;
      v[q] = (j < N) ? s[j] : -INFINITY;
      m = fmaxf(m, v[q]);
    }
    const float sn = s[N];
    m = wave_max(m);
    if (M > 0) m = fmaxf(m, sn);
    double ex[kQ], part = 0.0;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int j = lane + q * kWave;
      ex[q] = (j < N) ? exp((double)v[q] - (double)m) : 0.0;
      part += ex[q];
    }
    const double en = M > 0 ? exp((double)sn - (double)m) : 0.0;
    const double z = wave_sum_double(part) + (double)M * en;
#pragma unroll
    for (int q = 0; q < kQ; ++q) psum[q] += ex[q] / z;
    pnull += en / z;
    const double lse = (double)m + log(z);
    lz += lse * lse;
    if (lane < K) {
      const int id = topk_idx[t * K + lane];
      if (id >= 0 && id < P) atomicAdd(&cnt[id], 1);
      nreal += (id >= 0 && id < N);
    }
  }
  // per-wave totals into LDS, then the block record in wave order
  const int rd = (int)aux_rec_doubles(N);
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int j = lane + q * kWave;
    if (j < N) wacc[wave * rd + j] = psum[q];
  }
  const double nr = (double)wave_sum_int(nreal);
  if (lane == 0) {
    wacc[wave * rd + N] = pnull;
    wacc[wave * rd + N + 1] = lz;
    wacc[wave * rd + N + 2] = nr;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < rd; i += blockDim.x) {
    double acc = 0.0;
    for (int w = 0; w < nw; ++w) acc += wacc[w * rd + i];
    rec[(int64_t)blockIdx.x * rd + i] = acc;
  }
  for (int i = threadIdx.x; i < P; i += blockDim.x) rec_counts[(int64_t)blockIdx.x * P + i] = cnt[i];
}

__global__ void __launch_bounds__(kAuxThreads)
aux_final_kernel(const double* __restrict__ rec, const int32_t* __restrict__ rec_counts, int nb,
                 int64_t T, int N, int M, float* __restrict__ f, float* __restrict__ Pout,
                 int32_t* __restrict__ counts, float* __restrict__ scalars) {
  extern __shared__ double sfin[];
  const int rd = (int)aux_rec_doubles(N);
  const int P = N + M;
  double* tot = sfin;            // [rd]
  double* term = sfin + rd;      // [P]
  for (int i = threadIdx.x; i < rd; i += blockDim.x) {
    double acc = 0.0;
    for (int b = 0; b < nb; ++b) acc += rec[(int64_t)b * rd + i];
    tot[i] = acc;
  }
  __syncthreads();
  const double invT = 1.0 / (double)T;
  for (int i = threadIdx.x; i < P; i += blockDim.x) {
    long long c = 0;
    for (int b = 0; b < nb; ++b) c += rec_counts[(int64_t)b * P + i];
    const double Pi = (i < N ? tot[i] : tot[N]) * invT;
    const double fi = (double)c * invT;
    term[i] = fi * Pi;
    if (f) f[i] = (float)fi;
    if (Pout) Pout[i] = (float)Pi;
    if (counts) counts[i] = (int32_t)c;
  }
  __syncthreads();
  if (threadIdx.x == 0 && scalars) {
    double lb = 0.0;
    for (int i = 0; i < P; ++i) lb += term[i];
    scalars[0] = (float)((double)N * lb);
    scalars[1] = (float)(tot[N + 1] * invT);
    scalars[2] = (float)(tot[N + 2] * invT);
  }
}

hipError_t launch_aux(const AuxArgs& a, hipStream_t stream) {
  if (a.T <= 0) return hipSuccess;
  const int nb = aux_blocks(a.T);
  const int rd = (int)aux_rec_doubles(a.N);
  double* rec = static_cast<double*>(a.ws);
  int32_t* rec_counts = reinterpret_cast<int32_t*>(rec + (size_t)nb * rd);
  const size_t lds1 = (size_t)(kAuxThreads / kWave) * rd * sizeof(double) + (size_t)(a.N + a.M) * sizeof(int);
  aux_partial_kernel<<<nb, kAuxThreads, lds1, stream>>>(a.logits, a.topk_idx, a.T, a.N, a.M, a.K,
                                                        rec, rec_counts);
  const size_t lds2 = ((size_t)rd + a.N + a.M) * sizeof(double);
  aux_final_kernel<<<1, kAuxThreads, lds2, stream>>>(rec, rec_counts, nb, a.T, a.N, a.M, a.f, a.P,
                                                     a.counts, a.scalars);
  return hipGetLastError();
}

}  // namespace moe
