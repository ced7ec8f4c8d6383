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
// (standalone path only); (b) one launch in which every chunk's workgroup adds the
// histograms itself (all chunks for the expert totals and offsets, earlier chunks
// for its base), ranks its slots stably -- wavefront ballots find the lanes
// holding the same expert -- and scatters, while one more workgroup finalises the
// statistics in the fused path. Counts use integer additions, whose result does
// not depend on their order, so the permutation is deterministic. A further
// kernel gathers x_perm[p] = x[perm_token[p]] (standalone path; the layer's
// gate/up GEMM reads x through perm_token instead).
#include <algorithm>

#include "aux_final.hpp"
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

// Counting sort of the token slots, one launch. Workgroup c < nchunks owns the
// 64 tokens of chunk c: it adds the per-chunk expert histograms (all chunks for
// the totals, chunks before c for its prefix), scans the totals into the expert
// offsets, and scatters its 64 K slots at offsets[e] + prefix[e] + (rank within
// the chunk), so the order is stable (token-major, then k). Workgroup nchunks,
// when statistics are requested, finalises them from the router's per-tile sums.
// K groups of 64 slots per chunk; each wavefront takes a contiguous run of groups.
// With statistics the launch has kStatsThreads per workgroup, for the finalising
// workgroup (more tile groups summed in parallel, each a shorter chain of loads); the
// chunk workgroups use their first kPermThreads and end the other wavefronts at once
// (a workgroup barrier waits only for the wavefronts that have not ended).
constexpr int kStatsThreads = 1024;

template <bool STATS>
__global__ void __launch_bounds__(STATS ? kStatsThreads : kPermThreads)
permute_kernel(const int32_t* __restrict__ topk_idx, int64_t TK, int K, int N,
               const int32_t* __restrict__ chunk_hist, int nchunks, int64_t max_rows,
               int32_t* __restrict__ perm_token, int32_t* __restrict__ slot_pos,
               int32_t* __restrict__ counts, int32_t* __restrict__ offsets, AuxTiles aux,
               int64_t T, int M, int32_t* __restrict__ row_dst) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  constexpr int nw = kPermThreads / kWave;
  const int nkeys = N + 1;
  const int c = blockIdx.x;
  if (STATS && c == nchunks) {
    finalize_tiles<32>(aux, chunk_hist, nchunks, T, N, M, K, smem_raw);
    return;
  }
  if (STATS && threadIdx.x >= kPermThreads) return;  // whole wavefronts
  const int wave = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int gpw = (K + nw - 1) / nw;  // groups (of 64 slots) per wave
  const int64_t fc = (int64_t)c * kTokChunk * K;
  // Loads first: this chunk's slots, then the first rows of the chunk histograms
  // (thread (column quad q4, row phase r) adds rows r, r + RP, ...), so both
  // latencies overlap and the ranking below waits only for the slots.
  int kraw[kMaxGroupsPerWave];
#pragma unroll
  for (int gi = 0; gi < kMaxGroupsPerWave; ++gi) {
    const int grp = wave * gpw + gi;
    const int64_t f = fc + (int64_t)grp * kWave + lane;
    kraw[gi] = (gi < gpw && grp < K && f < TK) ? topk_idx[f] : -1;
  }
  const int N4 = (N + 3) / 4, RP = max(1, kPermThreads / N4);
  const int q4 = threadIdx.x % N4, r = threadIdx.x / N4;
  int v0[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = r + u * RP, e = 4 * q4 + j;
      v0[u][j] = (r < RP && row < nchunks && e < N) ? chunk_hist[(int64_t)row * N + e] : 0;
    }
  // LDS: off [N + 1], base [N], per-wave counts [nw][N + 1], per-wave bases [nw][N],
  // the histogram partials [2][RP][N] (ints)
  int* off = reinterpret_cast<int*>(smem_raw);
  int* cbase = off + (N + 1);
  int* wcnt = cbase + N;
  int* wbase = wcnt + nw * nkeys;
  int* ptot = wbase + nw * N;
  int* ppre = ptot + RP * N;
  for (int i = threadIdx.x; i < nw * nkeys; i += kPermThreads) wcnt[i] = 0;
  __syncthreads();
  // rank the slots: the lanes of a wavefront holding the same expert are found with
  // ballots over the key bits; a slot's rank counts the equal keys in lower lanes and
  // in the wavefront's earlier groups
  int nbits = 1;
  while ((1 << nbits) <= N) ++nbits;  // enough bits for keys 0..N
  int key[kMaxGroupsPerWave], lrank[kMaxGroupsPerWave];
  int* mycnt = wcnt + wave * nkeys;
#pragma unroll
  for (int gi = 0; gi < kMaxGroupsPerWave; ++gi) {
    key[gi] = N;
    lrank[gi] = 0;
    const int grp = wave * gpw + gi;
    if (gi >= gpw || grp >= K) continue;  // uniform across the wave
    const int64_t f = fc + (int64_t)grp * kWave + lane;
    const int k = f < TK ? slot_key(kraw[gi], N) : N;
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
  // expert totals over all chunks and this chunk's prefix (chunks before c)
  if (r < RP) {
    int tot[4] = {0, 0, 0, 0}, pre[4] = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        tot[j] += v0[u][j];
        if (r + u * RP < c) pre[j] += v0[u][j];
      }
    for (int rb = r + 4 * RP; rb < nchunks; rb += 4 * RP) {
      int v[4][4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = rb + u * RP, e = 4 * q4 + j;
          v[u][j] = (row < nchunks && e < N) ? chunk_hist[(int64_t)row * N + e] : 0;
        }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          tot[j] += v[u][j];
          if (rb + u * RP < c) pre[j] += v[u][j];
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * q4 + j;
      if (e < N) {
        ptot[r * N + e] = tot[j];
        ppre[r * N + e] = pre[j];
      }
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += kPermThreads) {
    int t = 0, p = 0;
    for (int rr = 0; rr < RP; ++rr) {
      t += ptot[rr * N + e];
      p += ppre[rr * N + e];
    }
    off[e] = t;  // totals for now
    cbase[e] = p;
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    // wave 0: exclusive scan of the per-expert totals, 4 experts per lane
    int tot[4], local = 0;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int ee = lane * 4 + qq;
      tot[qq] = ee < N ? off[ee] : 0;
      local += tot[qq];
    }
    int incl = local;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    int run = incl - local;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int ee = lane * 4 + qq;
      if (ee < N) {
        off[ee] = run;
        if (c == 0) {
          offsets[ee] = run;
          counts[ee] = tot[qq];
        }
        cbase[ee] += run;
      }
      run += tot[qq];
    }
    if (lane == kWave - 1) {
      off[N] = incl;
      if (c == 0) offsets[N] = incl;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nw * N; i += kPermThreads) {
    const int w = i / N, e = i % N;
    int b = cbase[e];
    for (int w2 = 0; w2 < w; ++w2) b += wcnt[w2 * nkeys + e];
    wbase[w * N + e] = b;
  }
  __syncthreads();
  const int t0 = c * kTokChunk;
#pragma unroll
  for (int gi = 0; gi < kMaxGroupsPerWave; ++gi) {
    const int grp = wave * gpw + gi;
    if (gi >= gpw || grp >= K) continue;
    const int local = grp * kWave + lane;  // slot within the chunk
    const int64_t f = fc + local;
    if (f < TK) {
      const int k = key[gi];
      if (k < N) {
        const int p = wbase[wave * N + k] + lrank[gi];
        slot_pos[f] = p;
        if (p < max_rows) {  // (past capacity: dropped)
          const int tk = (int)((unsigned)local / (unsigned)K);
          perm_token[p] = t0 + tk;
          // token-major destination of the slot's expert output: slot k of token t is
          // one of its reals, which come first, so k < min(K, N)
          if (row_dst) row_dst[p] = (t0 + tk) * min(K, N) + (local - tk * K);
        }
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
  return (size_t)permute_nchunks(T) * N * sizeof(int32_t);
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t stream) {
  const int64_t TK = a.T * a.K;
  const int nchunks = permute_nchunks(a.T);
  int32_t* chunk_hist = a.ws;
  if (!a.hist_ready)
    permute_hist_kernel<<<nchunks, kPermThreads, a.N * sizeof(int), stream>>>(a.topk_idx, TK, a.K,
                                                                             a.N, chunk_hist);
  AuxTiles at{};
  if (a.aux) at = *a.aux;
  const bool stats = at.tstats != nullptr;
  constexpr int nw = kPermThreads / kWave;
  const int N4 = (a.N + 3) / 4, RP = std::max(1, kPermThreads / N4);
  size_t lds = ((size_t)(2 * a.N + 1) + (size_t)nw * (a.N + 1) + (size_t)nw * a.N + (size_t)2 * RP * a.N) *
               sizeof(int);
  if (stats) {
    const int C = a.N + 3, G = finalize_groups(a.N, a.K, kStatsThreads);
    const size_t st = ((size_t)G * C + C + (size_t)(a.N + a.M)) * sizeof(double) +
                      (size_t)(a.N + a.K + 1) * sizeof(int);
    lds = std::max(lds, st);
  }
  const int64_t max_rows = a.T * (int64_t)std::min(a.K, a.N);
  const unsigned grid = (unsigned)(nchunks + (stats ? 1 : 0));
  if (stats)
    permute_kernel<true><<<grid, kStatsThreads, lds, stream>>>(
        a.topk_idx, TK, a.K, a.N, chunk_hist, nchunks, max_rows, a.perm_token, a.slot_pos, a.counts,
        a.offsets, at, a.T, a.M, a.row_dst);
  else
    permute_kernel<false><<<grid, kPermThreads, lds, stream>>>(
        a.topk_idx, TK, a.K, a.N, chunk_hist, nchunks, max_rows, a.perm_token, a.slot_pos, a.counts,
        a.offsets, at, a.T, a.M, a.row_dst);
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
