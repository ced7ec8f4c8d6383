// Finalisation of the load-balance / z-loss statistics: from the fixed-point
// accumulators of the statistics kernels (aux_finalize), and from the router's
// per-tile sums in the fused layer path (finalize_tiles: the permutation's extra
// workgroup, or the one-workgroup router of a few tokens).
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

// Statistics of the fused layer path from the router's per-tile sums, added in
// tile order (fixed, so the result does not depend on scheduling). Paper review
// "Improving MoE Compute Efficiency by Composing Weight and Data Sparsity",
// section 3, "load-balance loss" and "Z-loss": P_i = mean_t p_t,i (the M null
// copies share P_null), f_i = counts_i / T, L_bal = N sum_{i < N+M} f_i P_i,
// L_z = mean_t lse_t^2, plus mean r. A token with r chosen reals fills null copies
// N .. N + K - r - 1, so copy N + j is used by the tokens with r < K - j.
// Called by every thread of one workgroup. All three per-tile tables (sums, expert
// histograms, r histograms) are added column by column in one pass, so their loads
// are in flight together. LDS: part [G][N + 3], tot [N + 3], terms [N + M] (doubles),
// then cnt [N] and rsum [K + 1] (ints). BATCH: tiles of one column loaded at a time
// (32 for the permutation's workgroup, whose columns are long; the one-workgroup
// router has a single tile and a tight register budget).
template <int BATCH = 64>
__device__ inline void finalize_tiles(const AuxTiles& a, const int32_t* __restrict__ chunk_hist, int tiles,
                               int64_t T, int N, int M, int K, unsigned char* lds) {
  const int C = N + 3, R = K + 1, Q = C + N + R;
  const int G = max(1, (int)blockDim.x / Q);
  const int per = (tiles + G - 1) / G;
  double* part = reinterpret_cast<double*>(lds);
  double* tot = part + G * C;
  double* terms = tot + C;
  int* cnt = reinterpret_cast<int*>(terms + N + M);
  int* rsum = cnt + N;
  for (int i = threadIdx.x; i < N + R; i += blockDim.x) cnt[i] = 0;  // cnt, then rsum
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * Q; idx += blockDim.x) {
    // item (column q, group g) adds tiles [g per, (g + 1) per) of its column, BATCH
    // loads in flight at a time (the fp64 sums stay in tile order)
    const int q = idx % Q, g = idx / Q;
    const int ta = g * per, tb = min(tiles, (g + 1) * per);
    if (q < C) {
      double sum = 0.0;
      for (int t = ta; t < tb; t += BATCH) {
        double v[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) v[u] = t + u < tb ? a.tstats[(int64_t)(t + u) * C + q] : 0.0;
#pragma unroll
        for (int u = 0; u < BATCH; ++u) sum += v[u];
      }
      part[g * C + q] = sum;
    } else {
      // integer sums: any order
      const bool hist = q < C + N;
      const int col = hist ? q - C : q - C - N, width = hist ? N : R;
      const int32_t* src = hist ? chunk_hist : a.rhist;
      int sum = 0;
      for (int t = ta; t < tb; t += BATCH) {
        int v[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) v[u] = t + u < tb ? src[(int64_t)(t + u) * width + col] : 0;
#pragma unroll
        for (int u = 0; u < BATCH; ++u) sum += v[u];
      }
      if (sum) atomicAdd(&cnt[q - C], sum);  // cnt[col] or rsum[col]
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    double sum = 0.0;
    for (int g = 0; g < G; ++g) sum += part[g * C + c];
    tot[c] = sum;
  }
  __syncthreads();
  const int P = N + M;
  const double invT = 1.0 / (double)T;
  for (int i = threadIdx.x; i < P; i += blockDim.x) {
    int c = 0;
    if (i < N) {
      c = cnt[i];
    } else {
      const int j = i - N;
      for (int r = 0; r < K - j; ++r) c += rsum[r];
    }
    const double Pi = tot[i < N ? i : N] * invT;
    const double fi = (double)c * invT;
    terms[i] = fi * Pi;
    if (a.f) a.f[i] = (float)fi;
    if (a.P) a.P[i] = (float)Pi;
    if (a.counts) a.counts[i] = c;
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    double sum = 0.0;
    for (int i = threadIdx.x; i < P; i += kWave) sum += terms[i];
    sum = wave_sum_double(sum);
    if (threadIdx.x == 0 && a.scalars) {
      a.scalars[0] = (float)((double)N * sum);
      a.scalars[1] = (float)(tot[N + 1] * invT);
      a.scalars[2] = (float)(tot[N + 2] * invT);
    }
  }
}

__host__ __device__ constexpr int finalize_groups(int N, int K, int threads) {
  return (threads / ((N + 3) + N + (K + 1))) > 1 ? threads / ((N + 3) + N + (K + 1)) : 1;
}

}  // namespace moe
