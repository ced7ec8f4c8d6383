// Load-balance and z-loss statistics over the N+M pool (standalone entry point;
// the fused layer path computes the same sums in the router's epilogue).
//
// Paper review "Improving MoE Compute Efficiency by Composing Weight and Data
// Sparsity", section 3, "load-balance loss" and "Z-loss":
//   L_bal = N * sum_{i < N+M} f_i P_i,   L_z = mean_t (log sum_{i < N+M} e^{v_t,i})^2
// where v_t is the pool [s_0..s_{N-1}, s_null repeated M times], P_i the mean
// pool-softmax probability and f_i the fraction of tokens routed to slot i.
// The M null copies share one probability, so the pool softmax needs N+1
// exponentials per token.
//
// Three small kernels: clear the accumulators; one wavefront per token, lanes
// over experts, each workgroup summing its 16 or 32 tokens and adding them into
// fixed-point integer accumulators (order-free, so bitwise reproducible); one
// workgroup turns the sums into f, P, counts and the scalars.
#include <algorithm>

#include "aux_final.hpp"
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kAuxThreads = 256;
// tokens per workgroup: few tokens spread over more workgroups (each wavefront walks
// its tokens one after another); many over fewer, so that the fixed-point atomics of
// the workgroups do not queue on the same addresses (measured at N = 64: T = 2048
// 26 -> 14 us with 16; T = 16384 best with 32)
static int aux_tokens_per_block(int64_t T) { return T <= 4096 ? 16 : 32; }
constexpr int kQa = (MOE_MAX_EXPERTS + kWave - 1) / kWave;

// Accumulators: [N + 4] uint64 (probability sums of the N reals and the null, lse^2,
// n_real, tokens whose lse is +inf), then the slot counts [N + M] int32.
constexpr int kAuxAcc = 4;
size_t aux_ws_bytes(int N, int M) {
  return (size_t)(N + kAuxAcc) * sizeof(uint64_t) + (size_t)(N + M) * sizeof(int32_t);
}

__global__ void aux_clear_kernel(uint64_t* __restrict__ acc, int nacc, int32_t* __restrict__ cnt,
                                 int ncnt) {
  for (int i = threadIdx.x; i < nacc; i += blockDim.x) acc[i] = 0;
  for (int i = threadIdx.x; i < ncnt; i += blockDim.x) cnt[i] = 0;
}

__global__ void __launch_bounds__(kAuxThreads)
aux_partial_kernel(const float* __restrict__ logits, const int32_t* __restrict__ topk_idx,
                   int64_t T, int N, int M, int K, int bt, uint64_t* __restrict__ acc,
                   int32_t* __restrict__ cnt) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const int nw = kAuxThreads / kWave;
  const int rd = N + kAuxAcc, P = N + M;
  double* wacc = reinterpret_cast<double*>(smem_raw);          // [nw][N+3]
  int* cnt_lds = reinterpret_cast<int*>(wacc + nw * rd);       // [N+M]
  for (int i = threadIdx.x; i < P; i += blockDim.x) cnt_lds[i] = 0;
  __syncthreads();
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int64_t tb = (int64_t)blockIdx.x * bt, te = min<int64_t>(T, tb + bt);
  double psum[kQa];
#pragma unroll
  for (int q = 0; q < kQa; ++q) psum[q] = 0.0;
  double pnull = 0.0, lz = 0.0;
  int nreal = 0, ninf = 0;
  for (int64_t t = tb + wave; t < te; t += nw) {
    const float* s = logits + t * (N + 1);
    float v[kQa];
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < kQa; ++q) {
      const int j = lane + q * kWave;
      v[q] = (j < N) ? s[j] : -INFINITY;
      m = fmaxf(m, v[q]);
    }
    const float sn = s[N];
    m = wave_max(m);
    if (M > 0) m = fmaxf(m, sn);
    float ex[kQa];
    double part = 0.0;
#pragma unroll
    for (int q = 0; q < kQa; ++q) {
      ex[q] = (lane + q * kWave < N) ? expf(v[q] - m) : 0.0f;
      part += (double)ex[q];
    }
    // a null logit at +inf is the pool maximum: numerator 1 (the limit), reals 0
    const float en = M > 0 ? (sn == m ? 1.0f : expf(sn - m)) : 0.0f;
    const double z = wave_sum_double(part) + (double)M * (double)en;
    const double iz = 1.0 / z;
#pragma unroll
    for (int q = 0; q < kQa; ++q) psum[q] += (double)ex[q] * iz;
    if (lane == 0) {
      pnull += (double)en * iz;
      const double lse = (double)m + log(z);
      // +inf (null logit at +inf) is counted apart: the sums are fixed point
      if (isinf(lse)) ++ninf;
      else lz += lse * lse;
    }
    if (lane < K) {
      const int id = topk_idx[t * K + lane];
      if (id >= 0 && id < P) atomicAdd(&cnt_lds[id], 1);
      nreal += (id >= 0 && id < N);
    }
  }
  nreal = wave_sum_int(nreal);
#pragma unroll
  for (int q = 0; q < kQa; ++q)
    if (lane + q * kWave < N) wacc[wave * rd + lane + q * kWave] = psum[q];
  if (lane == 0) {
    wacc[wave * rd + N] = pnull;
    wacc[wave * rd + N + 1] = lz;
    wacc[wave * rd + N + 2] = (double)nreal;
    wacc[wave * rd + N + 3] = (double)ninf;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < rd; i += blockDim.x) {
    double s = 0.0;
    for (int w = 0; w < nw; ++w) s += wacc[w * rd + i];
    const double scale = (i == N + 1) ? kAuxZScale : (i >= N + 2 ? 1.0 : kAuxPScale);
    const uint64_t q = (uint64_t)(s * scale + 0.5);
    if (q) atomicAdd(reinterpret_cast<unsigned long long*>(&acc[i]), (unsigned long long)q);
  }
  for (int i = threadIdx.x; i < P; i += blockDim.x)
    if (cnt_lds[i]) atomicAdd(&cnt[i], cnt_lds[i]);
}

__global__ void __launch_bounds__(kAuxThreads)
aux_final_kernel(AuxFinal a, int64_t T, int N, int M) {
  extern __shared__ double terms[];
  aux_finalize(a, T, N, M, terms);
}

hipError_t launch_aux(const AuxArgs& a, hipStream_t stream) {
  if (a.T <= 0) return hipSuccess;
  uint64_t* acc = static_cast<uint64_t*>(a.ws);
  int32_t* cnt = reinterpret_cast<int32_t*>(acc + (a.N + kAuxAcc));
  const int P = a.N + a.M;
  aux_clear_kernel<<<1, 256, 0, stream>>>(acc, a.N + kAuxAcc, cnt, P);
  const int bt = aux_tokens_per_block(a.T);
  const unsigned nb = (unsigned)((a.T + bt - 1) / bt);
  const size_t lds1 = (size_t)(kAuxThreads / kWave) * (a.N + kAuxAcc) * sizeof(double) + (size_t)P * sizeof(int);
  aux_partial_kernel<<<nb, kAuxThreads, lds1, stream>>>(a.logits, a.topk_idx, a.T, a.N, a.M, a.K, bt,
                                                        acc, cnt);
  AuxFinal f{acc, cnt, a.f, a.P, a.counts, a.scalars};
  aux_final_kernel<<<1, kAuxThreads, (size_t)P * sizeof(double), stream>>>(f, a.T, a.N, a.M);
  return hipGetLastError();
}

}  // namespace moe
