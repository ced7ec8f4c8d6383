// Finalisation of the load-balance / z-loss statistics from the fixed-point
// accumulators (shared by the statistics kernels and the permutation's scan
// kernel, which finalises them in the fused layer path).
//
// Paper review "Improving MoE Compute Efficiency by Composing Weight and Data
// Sparsity", section 3, "load-balance loss" and "Z-loss":
//   P_i = mean_t p_t,i (the M null copies share P_null), f_i = counts_i / T,
//   L_bal = N * sum_{i < N+M} f_i P_i,  L_z = mean_t lse_t^2,  plus mean n_real.
#pragma once
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// Called by every thread of one workgroup; lds_terms holds N + M doubles.
__device__ inline void aux_finalize(const AuxFinal& a, int64_t T, int N, int M, double* lds_terms) {
  const int P = N + M;
  const double invT = 1.0 / (double)T;
  for (int i = threadIdx.x; i < P; i += blockDim.x) {
    const int c = a.cnt[i];
    const double Pi = (double)a.acc[i < N ? i : N] / kAuxPScale * invT;
    const double fi = (double)c * invT;
    lds_terms[i] = fi * Pi;
    if (a.f) a.f[i] = (float)fi;
    if (a.P) a.P[i] = (float)Pi;
    if (a.counts) a.counts[i] = c;
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    double s = 0.0;
    for (int i = threadIdx.x; i < P; i += kWave) s += lds_terms[i];
    s = wave_sum_double(s);
    if (threadIdx.x == 0 && a.scalars) {
      a.scalars[0] = (float)((double)N * s);
      a.scalars[1] = a.acc[N + 3] ? INFINITY : (float)((double)a.acc[N + 1] / kAuxZScale * invT);
      a.scalars[2] = (float)((double)a.acc[N + 2] * invT);
    }
  }
}

}  // namespace moe
