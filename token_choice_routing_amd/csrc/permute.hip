// Counting-sort dispatch of the token slots into expert order, null slots dropped.
//
// Paper review "Improving MoE Compute Efficiency by Composing Weight and Data
// Sparsity", section 3 "implementation": the slot list is argsorted so that
// null ids (>= N) land at the end, and it is truncated there before the grouped
// GEMM. The result here equals a stable argsort of the flat slot ids
// f = t*K + k by expert id with the null slots removed:
//   counts[e], offsets[e] (exclusive prefix sum, offsets[N] = R),
//   perm_token[p] (token of the p-th slot in expert order),
//   slot_pos[t][k] (position of the slot, -1 for a null slot).
//
// The slots are cut into chunks of 64 tokens (64*K slots), the same chunks the
// router's workgroups score, so in the fused layer path the router has already
// written each chunk's expert histogram. Kernels: (a) per-chunk histogram
// (standalone path only), (b) one workgroup turns the histograms into counts,
// offsets and per-chunk bases (and, in the fused path, finalises the
// statistics), (c) each chunk ranks its slots stably -- wavefront ballots find
// the lanes holding the same expert -- and scatters. Counts use LDS integer
// atomics, whose result does not depend on their order, so the permutation is
// deterministic. A fourth kernel gathers x_perm[p] = x[perm_token[p]].
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kTokChunk = 64;         // tokens per chunk (= router tokens per workgroup)
constexpr int kPermThreads = 256;     // 4 wavefronts
constexpr int kMaxGroupsPerWave = (MOE_MAX_TOPK * kTokChunk / kWave + 3) / 4;

__device__ __forceinline__ int slot_key(int32_t v, int N) { return (v >= 0 && v < N) ? v : N; }

__global__ void __launch_bounds__(kPermThreads)
permute_hist_kernel(const int32_t* __restrict__ topk_idx, int64_t TK, int K, int N,
                    int32_t* __restrict__ chunk_hist) {
  extern __shared__ int hist[];
  for (int e = threadIdx.x; e < N; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int64_t f0 = (int64_t)blockIdx.x * kTokChunk * K;
  const int64_t f1 = min<int64_t>(f0 + (int64_t)kTokChunk * K, TK);
  for (int64_t f = f0 + threadIdx.x; f < f1; f += blockDim.x) {
    const int k = slot_key(topk_idx[f], N);
    if (k < N) atomicAdd(&hist[k], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += blockDim.x) chunk_hist[(int64_t)blockIdx.x * N + e] = hist[e];
}

// Statistics of the fused layer path from the router's per-tile sums, added in
// tile order (fixed, so the result does not depend on scheduling). Paper review
// "Improving MoE Compute Efficiency by Composing Weight and Data Sparsity",
// section 3, "load-balance loss" and "Z-loss": P_i = mean_t p_t,i (the M null
// copies share P_null), f_i = counts_i / T, L_bal = N sum_{i < N+M} f_i P_i,
// L_z = mean_t lse_t^2, plus mean r. A token with r chosen reals fills null copies
// N .. N + K - r - 1, so copy N + j is used by the tokens with r < K - j.
// Called by every thread of one workgroup; off[0..N] holds the expert offsets.
__device__ void finalize_tiles(const AuxTiles& a, int tiles, int64_t T, int N, int M, int K,
                               const int* off, double* part, double* tot, int* rsum,
                               double* terms) {
  const int C = N + 3;
  const int G = max(1, (int)blockDim.x / C);
  const int per = (tiles + G - 1) / G;
  for (int r = threadIdx.x; r <= K; r += blockDim.x) rsum[r] = 0;
  __syncthreads();
  {
    // thread (c, g) adds tiles [g per, (g + 1) per) of column c, eight loads at a time
    const int c = threadIdx.x % C, g = threadIdx.x / C;
    if (g < G) {
      double s = 0.0;
      const int t1 = min(tiles, (g + 1) * per);
      for (int tb = g * per; tb < t1; tb += 8) {
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = tb + u < t1 ? a.tstats[(int64_t)(tb + u) * C + c] : 0.0;
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
      }
      part[g * C + c] = s;
    }
  }
  {
    // r histogram: integer sums, any order
    const int R = K + 1, GR = max(1, (int)blockDim.x / R), pr = (tiles + GR - 1) / GR;
    const int r = threadIdx.x % R, g = threadIdx.x / R;
    if (g < GR) {
      int s = 0;
      const int t1 = min(tiles, (g + 1) * pr);
      for (int tb = g * pr; tb < t1; tb += 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = tb + u < t1 ? a.rhist[(int64_t)(tb + u) * R + r] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
      }
      if (s) atomicAdd(&rsum[r], s);
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    double s = 0.0;
    for (int g = 0; g < G; ++g) s += part[g * C + c];
    tot[c] = s;
  }
  __syncthreads();
  const int P = N + M;
  const double invT = 1.0 / (double)T;
  for (int i = threadIdx.x; i < P; i += blockDim.x) {
    int cnt = 0;
    if (i < N) {
      cnt = off[i + 1] - off[i];
    } else {
      const int j = i - N;
      for (int r = 0; r < K - j; ++r) cnt += rsum[r];
    }
    const double Pi = tot[i < N ? i : N] * invT;
    const double fi = (double)cnt * invT;
    terms[i] = fi * Pi;
    if (a.f) a.f[i] = (float)fi;
    if (a.P) a.P[i] = (float)Pi;
    if (a.counts) a.counts[i] = cnt;
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    double s = 0.0;
    for (int i = threadIdx.x; i < P; i += kWave) s += terms[i];
    s = wave_sum_double(s);
    if (threadIdx.x == 0 && a.scalars) {
      a.scalars[0] = (float)((double)N * s);
      a.scalars[1] = (float)(tot[N + 1] * invT);
      a.scalars[2] = (float)(tot[N + 2] * invT);
    }
  }
}

// One workgroup of 1024 threads: counts[e] = sum over chunks, offsets = exclusive
// scan over e, chunk_base[c][e] = offsets[e] + sum_{c' < c} hist[c'][e].
// Thread (e, g) owns expert e for the g-th contiguous group of chunks (N <= 255,
// so there are at least 4 groups). In the fused path it also finalises the
// statistics from the router's per-tile sums.
__global__ void __launch_bounds__(1024)
permute_scan_kernel(const int32_t* __restrict__ chunk_hist, int nchunks, int N,
                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                    int32_t* __restrict__ chunk_base, AuxTiles aux, int64_t T, int M, int K) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  const int groups = blockDim.x / N;
  const bool stats = aux.tstats != nullptr;
  // fused: terms [N + M], tile-group partials [G][N + 3], totals [N + 3] (doubles)
  const int C = N + 3, G = max(1, (int)blockDim.x / C);
  double* terms = reinterpret_cast<double*>(smem_raw);
  double* spart = terms + (stats ? N + M : 0);
  double* stot = spart + (stats ? G * C : 0);
  int* part = reinterpret_cast<int*>(stot + (stats ? C : 0));        // [groups][N]
  int* off = part + groups * N;                                      // [N + 1]
  int* rsum = off + N + 1;                                           // [K + 1]
  const int per = (nchunks + groups - 1) / groups;
  const int e = threadIdx.x % N, g = threadIdx.x / N;
  const bool active = g < groups;
  const int c0 = g * per, c1 = min(nchunks, c0 + per);
  if (active) {
    int s = 0;
    for (int cb = c0; cb < c1; cb += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = cb + u < c1 ? chunk_hist[(int64_t)(cb + u) * N + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    part[g * N + e] = s;
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    // wave 0: exclusive scan of the per-expert totals, 4 experts per lane
    const int lane = threadIdx.x;
    int tot[4], local = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ee = lane * 4 + q;
      int t = 0;
      if (ee < N)
        for (int gg = 0; gg < groups; ++gg) t += part[gg * N + ee];
      tot[q] = t;
      local += t;
    }
    int incl = local;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    int run = incl - local;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ee = lane * 4 + q;
      if (ee < N) {
        off[ee] = run;
        offsets[ee] = run;
        counts[ee] = tot[q];
      }
      run += tot[q];
    }
    if (lane == kWave - 1) {
      off[N] = incl;
      offsets[N] = incl;
    }
  }
  __syncthreads();
  if (active) {
    int base = off[e];
    for (int g2 = 0; g2 < g; ++g2) base += part[g2 * N + e];
    for (int c = c0; c < c1; ++c) {
      chunk_base[(int64_t)c * N + e] = base;
      base += chunk_hist[(int64_t)c * N + e];
    }
  }
  if (stats) finalize_tiles(aux, nchunks, T, N, M, K, off, spart, stot, rsum, terms);
}

// One workgroup per chunk of 64 tokens: 64*K slots in K groups of 64; each
// wavefront takes a contiguous run of groups, in order.
__global__ void __launch_bounds__(kPermThreads)
permute_scatter_kernel(const int32_t* __restrict__ topk_idx, int64_t TK, int K, int N,
                       const int32_t* __restrict__ chunk_base, int64_t max_rows,
                       int32_t* __restrict__ perm_token, int32_t* __restrict__ slot_pos) {
  extern __shared__ int sm[];
  const int nkeys = N + 1;
  constexpr int nw = kPermThreads / kWave;
  int* wcnt = sm;                  // [4][N+1] running count per wave
  int* wbase = sm + nw * nkeys;    // [4][N]
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  for (int i = threadIdx.x; i < nw * nkeys; i += blockDim.x) wcnt[i] = 0;
  __syncthreads();
  int nbits = 1;
  while ((1 << nbits) <= N) ++nbits;  // enough bits for keys 0..N
  const int gpw = (K + nw - 1) / nw;  // groups (of 64 slots) per wave
  const int64_t fc = (int64_t)blockIdx.x * kTokChunk * K;
  int key[kMaxGroupsPerWave], lrank[kMaxGroupsPerWave];
  int* mycnt = wcnt + wave * nkeys;
#pragma unroll
  for (int gi = 0; gi < kMaxGroupsPerWave; ++gi) {
    key[gi] = N;
    lrank[gi] = 0;
    const int grp = wave * gpw + gi;
    if (gi >= gpw || grp >= K) continue;  // uniform across the wave
    const int64_t f = fc + (int64_t)grp * kWave + lane;
    const int k = f < TK ? slot_key(topk_idx[f], N) : N;
    uint64_t peers = ~0ull;
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (k >> b) & 1;
      const uint64_t bal = ballot(bit);
      peers &= bit ? bal : ~bal;
    }
    const int before = __popcll(peers & lanemask_lt());
    const int prev = mycnt[k];
    key[gi] = k;
    lrank[gi] = prev + before;
    if (before == 0) mycnt[k] = prev + __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nw * N; i += blockDim.x) {
    const int w = i / N, e = i % N;
    int b = chunk_base[(int64_t)blockIdx.x * N + e];
    for (int w2 = 0; w2 < w; ++w2) b += wcnt[w2 * nkeys + e];
    wbase[w * N + e] = b;
  }
  __syncthreads();
#pragma unroll
  for (int gi = 0; gi < kMaxGroupsPerWave; ++gi) {
    const int grp = wave * gpw + gi;
    if (gi >= gpw || grp >= K) continue;
    const int64_t f = fc + (int64_t)grp * kWave + lane;
    if (f < TK) {
      const int k = key[gi];
      if (k < N) {
        const int p = wbase[wave * N + k] + lrank[gi];
        slot_pos[f] = p;
        if (p < max_rows) perm_token[p] = (int32_t)(f / K);  // past capacity: dropped
      } else {
        slot_pos[f] = -1;
      }
    }
  }
}

// x_perm[p] = x[perm_token[p]] for p < R = offsets[N]: 16-byte vectors, grid-stride.
__global__ void __launch_bounds__(256)
gather_rows_kernel(const uint8_t* __restrict__ x, const int32_t* __restrict__ perm_token,
                   const int32_t* __restrict__ offsets, int N, int64_t T, int64_t max_rows,
                   int row_bytes, uint8_t* __restrict__ x_perm) {
  const int64_t R = min<int64_t>(max<int32_t>(offsets[N], 0), max_rows);
  const int vpr = row_bytes / 16;
  const int64_t total = R * vpr;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  for (; i + 3 * stride < total; i += 4 * stride) {
    u32x4_t v[4];
    int64_t dst[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t ii = i + u * stride;
      const int64_t p = ii / vpr;
      const int c = (int)(ii - p * vpr);
      const int64_t t = min<int64_t>(max(perm_token[p], 0), T - 1);
      v[u] = *reinterpret_cast<const u32x4_t*>(x + t * row_bytes + c * 16);
      dst[u] = p * row_bytes + c * 16;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<u32x4_t*>(x_perm + dst[u]) = v[u];
  }
  for (; i < total; i += stride) {
    const int64_t p = i / vpr;
    const int c = (int)(i - p * vpr);
    const int64_t t = min<int64_t>(max(perm_token[p], 0), T - 1);
    *reinterpret_cast<u32x4_t*>(x_perm + p * row_bytes + c * 16) =
        *reinterpret_cast<const u32x4_t*>(x + t * row_bytes + c * 16);
  }
}

int permute_nchunks(int64_t T) { return (int)((T + kTokChunk - 1) / kTokChunk); }

size_t permute_ws_bytes(int64_t T, int N) {
  return (size_t)2 * permute_nchunks(T) * N * sizeof(int32_t);
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream) {
  const int64_t TK = a.T * a.K;
  const int nchunks = permute_nchunks(a.T);
  int32_t* chunk_hist = a.ws;
  int32_t* chunk_base = a.ws + (int64_t)nchunks * a.N;
  if (!a.hist_ready)
    permute_hist_kernel<<<nchunks, kPermThreads, a.N * sizeof(int), stream>>>(a.topk_idx, TK, a.K,
                                                                             a.N, chunk_hist);
  AuxTiles at{};
  if (a.aux) at = *a.aux;
  const int groups = 1024 / a.N;
  const int C = a.N + 3, G = std::max(1, 1024 / C);
  const size_t scan_lds =
      (at.tstats ? ((size_t)(a.N + a.M) + (size_t)G * C + C) * sizeof(double) : 0) +
      ((size_t)groups * a.N + a.N + 1 + a.K + 1) * sizeof(int);
  permute_scan_kernel<<<1, 1024, scan_lds, stream>>>(chunk_hist, nchunks, a.N, a.counts, a.offsets,
                                                     chunk_base, at, a.T, a.M, a.K);
  const size_t sc_lds = ((size_t)(kPermThreads / kWave) * (a.N + 1) +
                         (size_t)(kPermThreads / kWave) * a.N) * sizeof(int);
  const int64_t max_rows = a.T * (int64_t)std::min(a.K, a.N);
  permute_scatter_kernel<<<nchunks, kPermThreads, sc_lds, stream>>>(
      a.topk_idx, TK, a.K, a.N, chunk_base, max_rows, a.perm_token, a.slot_pos);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.x && a.x_perm) {
    const int row_bytes = a.d * a.elt_bytes;
    const int64_t vecs = max_rows * (row_bytes / 16);
    const unsigned gblk = (unsigned)std::max<int64_t>(1, std::min<int64_t>((vecs + 255) / 256, 4096));
    gather_rows_kernel<<<gblk, 256, 0, stream>>>(static_cast<const uint8_t*>(a.x), a.perm_token,
                                                 a.offsets, a.N, a.T, max_rows, row_bytes,
                                                 static_cast<uint8_t*>(a.x_perm));
    err = hipGetLastError();
  }
  return err;
}

}  // namespace moe
