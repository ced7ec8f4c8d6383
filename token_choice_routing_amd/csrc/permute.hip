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
// Three kernels: (a) per-chunk expert histogram, (b) one workgroup turns the
// histograms into counts, offsets and per-chunk bases, (c) each chunk ranks
// its slots stably (wavefront ballots find the lanes holding the same expert)
// and scatters. Histogram counts use LDS integer atomics, whose result does
// not depend on their order, so the permutation is deterministic.
// A fourth kernel gathers x_perm[p] = x[perm_token[p]].
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kChunk = 2048;          // flat slots per chunk
constexpr int kPermThreads = 256;     // 4 wavefronts, 512 slots each
constexpr int kPerWave = kChunk / (kPermThreads / kWave);

__device__ __forceinline__ int slot_key(int32_t v, int N) { return (v >= 0 && v < N) ? v : N; }

__global__ void __launch_bounds__(kPermThreads)
permute_hist_kernel(const int32_t* __restrict__ topk_idx, int64_t TK, int N,
                    int32_t* __restrict__ chunk_hist) {
  extern __shared__ int hist[];
  for (int e = threadIdx.x; e < N; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int64_t f0 = (int64_t)blockIdx.x * kChunk;
  const int64_t f1 = min<int64_t>(f0 + kChunk, TK);
  for (int64_t f = f0 + threadIdx.x; f < f1; f += blockDim.x) {
    const int k = slot_key(topk_idx[f], N);
    if (k < N) atomicAdd(&hist[k], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += blockDim.x) chunk_hist[(int64_t)blockIdx.x * N + e] = hist[e];
}

// One workgroup of 1024 threads: counts[e] = sum over chunks, offsets = exclusive
// scan over e, chunk_base[c][e] = offsets[e] + sum_{c' < c} hist[c'][e].
// Thread (e, g) owns expert e for the g-th contiguous group of chunks (N <= 255,
// so there are at least 4 groups).
__global__ void __launch_bounds__(1024)
permute_scan_kernel(const int32_t* __restrict__ chunk_hist, int nchunks, int N,
                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                    int32_t* __restrict__ chunk_base) {
  extern __shared__ int sm[];
  const int groups = blockDim.x / N;
  int* part = sm;                    // [groups][N]
  int* off = sm + groups * N;        // [N + 1]
  const int per = (nchunks + groups - 1) / groups;
  const int e = threadIdx.x % N, g = threadIdx.x / N;
  const bool active = g < groups;
  const int c0 = g * per, c1 = min(nchunks, c0 + per);
  if (active) {
    int s = 0;
    for (int c = c0; c < c1; ++c) s += chunk_hist[(int64_t)c * N + e];
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
}

__global__ void __launch_bounds__(kPermThreads)
permute_scatter_kernel(const int32_t* __restrict__ topk_idx, int64_t TK, int K, int N,
                       const int32_t* __restrict__ chunk_base, int64_t max_rows,
                       int32_t* __restrict__ perm_token, int32_t* __restrict__ slot_pos) {
  extern __shared__ int sm[];
  const int nkeys = N + 1;
  int* wcnt = sm;                                   // [4][N+1] running count per wave
  int* wbase = sm + (kPermThreads / kWave) * nkeys; // [4][N]
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  for (int i = threadIdx.x; i < (kPermThreads / kWave) * nkeys; i += blockDim.x) wcnt[i] = 0;
  __syncthreads();
  int nbits = 1;
  while ((1 << nbits) <= N) ++nbits;  // enough bits for keys 0..N
  const int64_t fw = (int64_t)blockIdx.x * kChunk + (int64_t)wave * kPerWave;
  constexpr int G = kPerWave / kWave;
  int key[G], lrank[G];
  int* mycnt = wcnt + wave * nkeys;
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int64_t f = fw + gi * kWave + lane;
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
  const int nw = kPermThreads / kWave;
  for (int i = threadIdx.x; i < nw * N; i += blockDim.x) {
    const int w = i / N, e = i % N;
    int b = chunk_base[(int64_t)blockIdx.x * N + e];
    for (int w2 = 0; w2 < w; ++w2) b += wcnt[w2 * nkeys + e];
    wbase[w * N + e] = b;
  }
  __syncthreads();
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int64_t f = fw + gi * kWave + lane;
    if (f < TK) {
      const int k = key[gi];
      if (k < N) {
        const int p = wbase[wave * N + k] + lrank[gi];
        slot_pos[f] = p;
        if (p < max_rows) perm_token[p] = (int32_t)(f / K);  // rows past capacity: dropped
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

int permute_nchunks(int64_t TK) { return (int)((TK + kChunk - 1) / kChunk); }

size_t permute_ws_bytes(int64_t TK, int N) {
  return (size_t)2 * permute_nchunks(TK) * N * sizeof(int32_t);
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream) {
  const int64_t TK = a.T * a.K;
  const int nchunks = permute_nchunks(TK);
  int32_t* chunk_hist = a.ws;
  int32_t* chunk_base = a.ws + (int64_t)nchunks * a.N;
  permute_hist_kernel<<<nchunks, kPermThreads, a.N * sizeof(int), stream>>>(a.topk_idx, TK, a.N,
                                                                           chunk_hist);
  const size_t scan_lds = ((size_t)(1024 / a.N) * a.N + a.N + 1) * sizeof(int);
  permute_scan_kernel<<<1, 1024, scan_lds, stream>>>(chunk_hist, nchunks, a.N, a.counts,
                                                     a.offsets, chunk_base);
  const size_t sc_lds = ((size_t)(kPermThreads / kWave) * (a.N + 1) +
                         (size_t)(kPermThreads / kWave) * a.N) * sizeof(int);
  permute_scatter_kernel<<<nchunks, kPermThreads, sc_lds, stream>>>(
      a.topk_idx, TK, a.K, a.N, chunk_base, a.T * (int64_t)std::min(a.K, a.N), a.perm_token,
      a.slot_pos);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (a.x && a.x_perm) {
    const int64_t max_rows = a.T * (int64_t)std::min(a.K, a.N);
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
