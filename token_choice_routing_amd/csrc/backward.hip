// Backward pass of the null-expert MoE layer (bf16, null experts that output zero).
//
// Role: the gradients that training the layer needs ([Review] section 3 trains the
// layer with the load-balance and z-loss terms added to the task loss; [Primer]
// sections 4.2 and 4.3). The objective is L = <dy, y> + alpha L_bal + beta L_z for an
// upstream gradient dy, the routing decision held fixed (top-K is piecewise constant).
// The backward recomputes what the forward produced (routing, permutation, expert
// pre-activations) instead of keeping it, then:
//
//   combine      dY_p = g dy_t (bf16) and dg = <dy_t, Y_p> per real slot
//   router       ds = renormalised-softmax backward of dg + the pool-softmax terms of
//                L_bal and L_z; dW_r = ds^T x, and dx gets ds W_r
//   experts      dh = dY W_d, (dg, du) = SwiGLU backward, da = [dg | du] [W_g ; W_u],
//                dW_d = dY^T h, dW_g = dg^T a, dW_u = du^T a
//
// Every contraction of the experts runs on the MFMA grouped GEMM of the forward: the
// data gradients on the weights transposed per expert (bf16 copies made here), the
// weight gradients on the activations transposed per segment (segments padded to 8
// columns, so every group's K range starts 16-byte aligned), with K the segment's
// rows. This file holds the data-movement and element-wise kernels around them.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kTile = 64;

// 64 x 64 bf16 tile through LDS: rows of 66 elements (33 four-byte words), so the
// 8 consecutive rows one lane reads at a column fall in distinct banks.
struct TTile {
  bf16_t v[kTile][kTile + 2];
};

// Thread i of 256 moves 16 bytes: row i / 8 (and row 32 + i / 8) of the tile, 8
// elements from column 8 (i % 8). All widths here are multiples of 8 elements, so
// every global access is one aligned 16-byte load or store; edge tiles are masked
// per 8-element chunk.
__device__ __forceinline__ void tile_to_lds(TTile& t, int r, int c8, const bf16_t* src_row, bool valid) {
  u32x4_t v = valid ? *reinterpret_cast<const u32x4_t*>(src_row) : u32x4_t{0, 0, 0, 0};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    t.v[r][c8 + 2 * e] = (bf16_t)(v[e] & 0xFFFF);
    t.v[r][c8 + 2 * e + 1] = (bf16_t)(v[e] >> 16);
  }
}

// Column c of the tile, rows r8 .. r8 + 7, as one 16-byte word.
__device__ __forceinline__ u32x4_t tile_column(const TTile& t, int c, int r8) {
  u32x4_t v;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    v[e] = (uint32_t)t.v[r8 + 2 * e][c] | ((uint32_t)t.v[r8 + 2 * e + 1][c] << 16);
  return v;
}

// out[b][c][c_out + r] = in[b][r][c] (bf16 bits) for an [R][C] matrix per batch b;
// out rows have stride ldo. R, C, ldo and c_out multiples of 8.
__global__ void __launch_bounds__(256)
transpose_kernel(const bf16_t* __restrict__ in, int64_t R, int64_t C, int64_t in_batch,
                 bf16_t* __restrict__ out, int64_t ldo, int64_t c_out, int64_t out_batch) {
  __shared__ TTile t;
  const int64_t r0 = (int64_t)blockIdx.y * kTile, c0 = (int64_t)blockIdx.x * kTile;
  const bf16_t* src = in + (int64_t)blockIdx.z * in_batch;
  bf16_t* dst = out + (int64_t)blockIdx.z * out_batch;
  const int i = threadIdx.x, c8 = (i & 7) * 8;
  for (int r = i >> 3; r < kTile; r += 32) {
    const bool ok = r0 + r < R && c0 + c8 < C;
    tile_to_lds(t, r, c8, src + (ok ? (r0 + r) * C + c0 + c8 : 0), ok);
  }
  __syncthreads();
  for (int c = i >> 3; c < kTile; c += 32) {
    const int64_t r = r0 + c8;  // this thread's 8 output elements: rows r .. r + 7
    if (c0 + c < C && r < R)
      *reinterpret_cast<u32x4_t*>(dst + (c0 + c) * ldo + c_out + r) = tile_column(t, c, c8);
  }
}

// Segment starts padded to multiples of 8: kofs[e] = sum_{i<e} round_up(len_i, 8),
// kofs[G] the total. One wavefront; segments read from offsets exactly as the GEMM
// clamps them.
__global__ void __launch_bounds__(64) pad_offsets_kernel(const int32_t* __restrict__ offsets, int G,
                                                         int64_t rows, int32_t* __restrict__ kofs) {
  if (threadIdx.x != 0) return;
  int run = 0;
  for (int e = 0; e < G; ++e) {
    int64_t a = offsets[e], b = offsets[e + 1];
    a = min<int64_t>(max<int64_t>(a, 0), rows);
    b = min<int64_t>(max<int64_t>(b, a), rows);
    kofs[e] = run;
    run += (int)((b - a + 7) & ~int64_t(7));
  }
  kofs[G] = run;
}

// dst[c][q] for padded positions q of the segments: row p = offsets[e] + (q - kofs[e])
// of src (read through src_rows[p] when given) while q - kofs[e] < len_e, else 0.
// offsets == NULL means one segment [0, rows) padded to ld. Columns c < C; dst rows
// have stride ld (>= kofs[G]); positions at or past kofs[G] are not written.
__global__ void __launch_bounds__(256)
transpose_segments_kernel(const bf16_t* __restrict__ src, const int32_t* __restrict__ src_rows,
                          int64_t src_nrows, const int32_t* __restrict__ offsets,
                          const int32_t* __restrict__ kofs, int G, int64_t rows, int64_t C,
                          bf16_t* __restrict__ dst, int64_t ld) {
  __shared__ TTile t;
  __shared__ int64_t srow[kTile];
  const int64_t q0 = (int64_t)blockIdx.y * kTile, c0 = (int64_t)blockIdx.x * kTile;
  const int64_t total = offsets ? kofs[G] : (rows + 7) & ~int64_t(7);
  if (q0 >= total) return;
  if (threadIdx.x < kTile) {
    const int64_t q = q0 + threadIdx.x;
    int64_t p = -1;
    if (q < total) {
      if (offsets) {
        int lo = 0, hi = G;  // kofs[lo] <= q < kofs[hi]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (kofs[mid] <= q) lo = mid; else hi = mid;
        }
        int64_t a = offsets[lo], b = offsets[lo + 1];
        a = min<int64_t>(max<int64_t>(a, 0), rows);
        b = min<int64_t>(max<int64_t>(b, a), rows);
        const int64_t local = q - kofs[lo];
        if (local < b - a) p = a + local;
      } else if (q < rows) {
        p = q;
      }
      if (p >= 0 && src_rows) p = min<int64_t>(max<int64_t>(src_rows[p], 0), src_nrows - 1);
    }
    srow[threadIdx.x] = p;
  }
  __syncthreads();
  const int i = threadIdx.x, c8 = (i & 7) * 8;
  for (int r = i >> 3; r < kTile; r += 32) {
    const int64_t p = srow[r];
    const bool ok = p >= 0 && c0 + c8 < C;
    tile_to_lds(t, r, c8, src + (ok ? p * C + c0 + c8 : 0), ok);
  }
  __syncthreads();
  for (int c = i >> 3; c < kTile; c += 32) {
    const int64_t q = q0 + c8;  // positions q .. q + 7 (total is a multiple of 8)
    if (c0 + c < C && q < total)
      *reinterpret_cast<u32x4_t*>(dst + (c0 + c) * ld + q) = tile_column(t, c, c8);
  }
}

// Rows below the real-row count (offsets[G], or rows when offsets is NULL).
__device__ __forceinline__ int64_t live_rows(const int32_t* offsets, int G, int64_t rows) {
  return offsets ? min<int64_t>(max<int64_t>(offsets[G], 0), rows) : rows;
}

// h = silu(g) * u, rounded to bf16 (the forward's expert activation, recomputed).
__global__ void __launch_bounds__(256)
swiglu_h_kernel(const float* __restrict__ g, const float* __restrict__ u, const int32_t* offsets, int G,
                int64_t rows, int F, bf16_t* __restrict__ h) {
  const int64_t n = live_rows(offsets, G, rows) * F;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    h[i] = f32_to_bf16(silu(g[i]) * u[i]);
}

// SwiGLU backward: dgu[p][j] = dh u silu'(g), dgu[p][F + j] = dh silu(g), bf16, with
// silu'(z) = sigma(z) (1 + z (1 - sigma(z))).
// (GT: float, or _Float16 for the keep-mode GEMM's g and u)
template <typename GT>
__global__ void __launch_bounds__(256)
swiglu_bwd_kernel(const GT* __restrict__ g, const GT* __restrict__ u, const float* __restrict__ dh,
                  const int32_t* offsets, int G, int64_t rows, int F, bf16_t* __restrict__ dgu) {
  const int64_t n = live_rows(offsets, G, rows) * F;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = i / F, j = i - p * F;
    const float z = (float)g[i], sg = 1.0f / (1.0f + __expf(-z));
    const float d = dh[i];
    dgu[p * 2 * F + j] = f32_to_bf16(d * (float)u[i] * (sg * (1.0f + z * (1.0f - sg))));
    dgu[p * 2 * F + F + j] = f32_to_bf16(d * z * sg);
  }
}

// Slots to expert-ordered rows, one wavefront per (token, slot): for a real slot
// (slot_pos >= 0) row p gets dy_perm[p] = topk_w dy_t (bf16, the output gradient of
// the expert row, for dW_down), w_perm[p] = topk_w and row_slot[p] = the slot's flat
// index; a null slot's weight gradient dw[t][k] is 0 (nothing flows through it). 8
// elements per lane and step (d is a multiple of 8).
__global__ void __launch_bounds__(256)
slot_rows_kernel(const bf16_t* __restrict__ dy, const int32_t* __restrict__ slot_pos,
                 const float* __restrict__ topk_w, int64_t T, int K, int d, int64_t R,
                 bf16_t* __restrict__ dy_perm, float* __restrict__ w_perm, int32_t* __restrict__ row_slot,
                 float* __restrict__ dw) {
  const int64_t ts = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (ts >= T * K) return;
  const int64_t t = ts / K;
  const int32_t p = slot_pos[ts];
  if (p < 0 || p >= R) {
    if (lane == 0) dw[ts] = 0.0f;
    return;
  }
  const float w = topk_w[ts];
  if (lane == 0) {
    w_perm[p] = w;
    row_slot[p] = (int32_t)ts;
  }
  const bf16_t* dyt = dy + t * d;
  bf16_t* o = dy_perm + (int64_t)p * d;
  for (int c = lane * 8; c < d; c += kWave * 8) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(dyt + c);
    u32x4_t ov;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      ov[e] = pack_bf16x2(w * bf16_to_f32((bf16_t)(v[e] & 0xFFFF)), w * bf16_to_f32((bf16_t)(v[e] >> 16)));
    *reinterpret_cast<u32x4_t*>(o + c) = ov;
  }
}

// SwiGLU and combine backward of the routed rows, one wavefront per row p, from
// U_p = dy_t W_d (the unweighted output gradient pulled back through W_d; the GEMM
// reads dy_t through perm_token): the slot's weight gradient is
//   dg_tk = <dy_t, Y_p> = <dy_t, h_p W_d^T> = <U_p, h_p>
// (so Y_p is never recomputed), written to dw[row_slot[p]] (float32, lanes add in a
// fixed order), and with dh = topk_w U_p the SwiGLU backward as in swiglu_bwd_kernel.
// 4 elements per lane and step (F is a multiple of 8).
// four consecutive g or u values as float32 (GT float, or _Float16)
template <typename GT>
__device__ __forceinline__ f32x4_t load4(const GT* p) {
  if constexpr (sizeof(GT) == 4) {
    return *reinterpret_cast<const f32x4_t*>(p);
  } else {
    typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
    const f16x4_t v = *reinterpret_cast<const f16x4_t*>(p);
    return f32x4_t{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  }
}

template <typename GT>
__global__ void __launch_bounds__(256)
swiglu_bwd_routed_kernel(const GT* __restrict__ g, const GT* __restrict__ u, const float* __restrict__ U,
                         const bf16_t* __restrict__ h, const float* __restrict__ w_perm,
                         const int32_t* __restrict__ row_slot, const int32_t* offsets, int G, int64_t rows,
                         int F, bf16_t* __restrict__ dgu, float* __restrict__ dw) {
  const int64_t p = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (p >= live_rows(offsets, G, rows)) return;
  const float w = w_perm[p];
  const int64_t o = p * F;
  float acc = 0.0f;
  for (int j = lane * 4; j < F; j += kWave * 4) {
    const f32x4_t uu = *reinterpret_cast<const f32x4_t*>(U + o + j);
    const f32x4_t gg = load4(g + o + j);
    const f32x4_t vv = load4(u + o + j);
    const u32x2_t hh = *reinterpret_cast<const u32x2_t*>(h + o + j);
    float dg[4], du[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t hw = hh[e >> 1];
      acc += uu[e] * bf16_to_f32((bf16_t)(e & 1 ? hw >> 16 : hw & 0xFFFF));
      const float z = gg[e], sg = 1.0f / (1.0f + __expf(-z)), d = w * uu[e];
      dg[e] = d * vv[e] * (sg * (1.0f + z * (1.0f - sg)));
      du[e] = d * z * sg;
    }
    bf16_t* row = dgu + p * 2 * F;
    *reinterpret_cast<u32x2_t*>(row + j) = u32x2_t{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])};
    *reinterpret_cast<u32x2_t*>(row + F + j) = u32x2_t{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])};
  }
#pragma unroll
  for (int o2 = 32; o2 > 0; o2 >>= 1) acc += __shfl_xor(acc, o2, kWave);
  if (lane == 0) dw[row_slot[p]] = acc;
}

// Router backward, one wavefront per token, in float64: ds[t][j] for the N real logits
// and the null logit (column N) from
//   the renormalised weights: ds_j += g_j (dg_j - sum_i g_i dg_i) over the chosen reals;
//   L_bal:  ds_c += alpha (N / T) p_c (f_c - sum_i f_i p_i) over the N + M pool;
//   L_z:    ds_c += beta (2 / T) lse p_c;
// the M null copies share one logit, so the null column gets their sum (none if M = 0).
__global__ void __launch_bounds__(256)
router_bwd_kernel(const float* __restrict__ logits, const int32_t* __restrict__ topk_idx,
                  const float* __restrict__ topk_w, const float* __restrict__ dw,
                  const float* __restrict__ f, int64_t T, int N, int M, int K, float alpha, float beta,
                  float* __restrict__ ds) {
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  if (t >= T) return;
  const float* s = logits + t * (N + 1);
  const double sn = s[N];
  // pool max and partition function
  double mx = M > 0 ? sn : -INFINITY;
  for (int j = lane; j < N; j += kWave) mx = fmax(mx, (double)s[j]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, kWave));
  double z = 0.0, fz = 0.0;  // sum e^{v - m}, sum f e^{v - m}
  for (int j = lane; j < N; j += kWave) {
    const double e = exp((double)s[j] - mx);
    z += e;
    fz += (double)f[j] * e;
  }
  double fnull = 0.0;  // sum of f over the null copies
  for (int c = lane; c < M; c += kWave) fnull += (double)f[N + c];
  z = wave_sum_double(z);
  fz = wave_sum_double(fz);
  fnull = wave_sum_double(fnull);
  // a null logit at +inf is the pool maximum: numerator 1 (the limit), reals 0
  const double en = M > 0 ? (sn == mx ? 1.0 : exp(sn - mx)) : 0.0;
  z += M * en;
  fz += fnull * en;
  const double lse = mx + log(z), fbar = fz / z;
  // the z-loss term of a token whose lse is +inf (null logit at +inf) has no finite
  // value and is taken as 0; its balance term is 0 by itself (p is saturated)
  const double ka = (double)alpha * N / (double)T, kb = isinf(lse) ? 0.0 : (double)beta * 2.0 / (double)T;
  // weight term: sum over the chosen reals of g dg
  double gdg = 0.0;
  for (int k = 0; k < K; ++k)
    if (topk_idx[t * K + k] < N) gdg += (double)topk_w[t * K + k] * dw[t * K + k];
  float* o = ds + t * (N + 1);
  for (int j = lane; j < N; j += kWave) {
    const double p = exp((double)s[j] - mx) / z;
    double v = ka * p * ((double)f[j] - fbar) + (kb ? kb * lse * p : 0.0);
    for (int k = 0; k < K; ++k)
      if (topk_idx[t * K + k] == j) v += (double)topk_w[t * K + k] * ((double)dw[t * K + k] - gdg);
    o[j] = (float)v;
  }
  if (lane == 0) {
    const double pn = en / z;
    o[N] = M > 0 ? (float)(ka * pn * (fnull - M * fbar) + (kb ? kb * lse * M * pn : 0.0)) : 0.0f;
  }
}

// dW_r partial sums: part[c][j][col] = sum over tokens t of chunk c of ds[t][j] x[t][col]
// (float32); 16 router rows x 512 columns per workgroup, two adjacent columns per
// thread (one 4-byte load of x per token).
constexpr int kRouterRows = 16;
__global__ void __launch_bounds__(256)
router_wgrad_partial_kernel(const float* __restrict__ ds, const bf16_t* __restrict__ x, int64_t T, int N1,
                            int d, int64_t chunk, float* __restrict__ part) {
  const int j0 = blockIdx.y * kRouterRows, col = (blockIdx.x * 256 + threadIdx.x) * 2;
  const int64_t t0 = (int64_t)blockIdx.z * chunk, t1 = min<int64_t>(T, t0 + chunk);
  float a0[kRouterRows] = {}, a1[kRouterRows] = {};
  __shared__ __attribute__((aligned(16))) float sds[64][kRouterRows];
  for (int64_t tb = t0; tb < t1; tb += 64) {
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * kRouterRows; i += 256) {
      const int64_t t = tb + i / kRouterRows;
      const int j = j0 + i % kRouterRows;
      sds[i / kRouterRows][i % kRouterRows] = t < t1 && j < N1 ? ds[t * N1 + j] : 0.0f;
    }
    __syncthreads();
    if (col < d) {
      const int n = (int)min<int64_t>(64, t1 - tb);
      for (int i = 0; i < n; ++i) {
        const uint32_t xv = *reinterpret_cast<const uint32_t*>(x + (tb + i) * d + col);
        const float x0 = bf16_to_f32((bf16_t)(xv & 0xFFFF)), x1 = bf16_to_f32((bf16_t)(xv >> 16));
#pragma unroll
        for (int r = 0; r < kRouterRows; ++r) {
          a0[r] += sds[i][r] * x0;
          a1[r] += sds[i][r] * x1;
        }
      }
    }
  }
  if (col < d)
#pragma unroll
    for (int r = 0; r < kRouterRows; ++r)
      if (j0 + r < N1) {
        float* o = part + ((int64_t)blockIdx.z * N1 + j0 + r) * d + col;
        o[0] = a0[r];
        o[1] = a1[r];
      }
}

// dW_r = sum of the chunk partials in chunk order (deterministic).
__global__ void __launch_bounds__(256)
router_wgrad_reduce_kernel(const float* __restrict__ part, int chunks, int64_t n, float* __restrict__ dw) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    float s = 0.0f;
    for (int c = 0; c < chunks; ++c) s += part[c * n + i];
    dw[i] = s;
  }
}

// dx[t] = sum over real slots of dx_perm[p] (slot order) + dx_shared[t] + ds[t] W_r,
// float32. A workgroup takes 16 tokens x 256 columns, one column per thread: each
// router row element is read once per 16 tokens, the tokens' ds from LDS four router
// rows at a time (one 16-byte read per token; the rows past N1 are zero).
constexpr int kScatterTok = 16;
__global__ void __launch_bounds__(256)
scatter_dx_kernel(const float* __restrict__ dx_perm, const int32_t* __restrict__ slot_pos, int K, int64_t R,
                  const float* __restrict__ dx_shared, const float* __restrict__ ds,
                  const float* __restrict__ w_router, int N1, int d, int64_t T, float* __restrict__ dx) {
  const int64_t t0 = (int64_t)blockIdx.x * kScatterTok;
  const int nt = (int)min<int64_t>(kScatterTok, T - t0);
  __shared__ __attribute__((aligned(16))) float sds[kScatterTok][260];
  __shared__ int32_t sp[kScatterTok][MOE_MAX_TOPK];
  const int N4 = (N1 + 3) & ~3;  // <= 260
  for (int i = threadIdx.x; i < kScatterTok * N4; i += 256) {
    const int tt = i / N4, j = i - tt * N4;
    sds[tt][j] = tt < nt && j < N1 ? ds[(t0 + tt) * N1 + j] : 0.0f;
  }
  for (int i = threadIdx.x; i < kScatterTok * K; i += 256) {
    const int tt = i / K, k = i - tt * K;
    sp[tt][k] = tt < nt ? slot_pos[(t0 + tt) * K + k] : -1;
  }
  __syncthreads();
  for (int c = blockIdx.y * 256 + threadIdx.x; c < d; c += gridDim.y * 256) {
    float acc[kScatterTok];
#pragma unroll
    for (int tt = 0; tt < kScatterTok; ++tt) acc[tt] = 0.0f;
    for (int j = 0; j < N4; j += 4) {
      float w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = j + q < N1 ? w_router[(int64_t)(j + q) * d + c] : 0.0f;
#pragma unroll
      for (int tt = 0; tt < kScatterTok; ++tt) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(&sds[tt][j]);
        acc[tt] += v[0] * w[0];
        acc[tt] += v[1] * w[1];
        acc[tt] += v[2] * w[2];
        acc[tt] += v[3] * w[3];
      }
    }
    // the slots' rows: four tokens and eight slots at a time, every load issued before
    // the first add (a load per slot, added in slot order, was a chain of round trips)
#pragma unroll
    for (int tg = 0; tg < kScatterTok; tg += 4) {
      if (tg >= nt) break;
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        v[u] = (tg + u < nt && dx_shared) ? dx_shared[(t0 + tg + u) * d + c] : 0.0f;
      for (int k0 = 0; k0 < K; k0 += 8) {
        float g[4][8];
        bool on[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int32_t p = (tg + u < nt && k0 + j < K) ? sp[tg + u][k0 + j] : -1;
            on[u][j] = p >= 0 && p < R;
            g[u][j] = on[u][j] ? dx_perm[(int64_t)p * d + c] : 0.0f;
          }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (on[u][j]) v[u] += g[u][j];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (tg + u < nt) dx[(t0 + tg + u) * d + c] = v[u] + acc[tg + u];
    }
  }
}

// Uniform K chunks for a split weight gradient: kofs[s] = min(s * chunk, rows) with
// chunk a multiple of 8, kofs[S] = rows rounded up to 8 (the padded column count).
__global__ void __launch_bounds__(64) split_offsets_kernel(int64_t rows, int S, int32_t* __restrict__ kofs) {
  const int64_t padded = (rows + 7) & ~int64_t(7);
  const int64_t chunk = ((padded + S - 1) / S + 7) & ~int64_t(7);
  for (int s = threadIdx.x; s <= S; s += 64) kofs[s] = (int32_t)min<int64_t>((int64_t)s * chunk, padded);
}

// out[i] = sum over the S partial matrices in order (deterministic), four elements
// per thread (n is a multiple of 4).
__global__ void __launch_bounds__(256)
sum_partials_kernel(const float* __restrict__ part, int S, int64_t n, float* __restrict__ out) {
  const int64_t n4 = n / 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    f32x4_t v = reinterpret_cast<const f32x4_t*>(part)[i];
    for (int s = 1; s < S; ++s) v += reinterpret_cast<const f32x4_t*>(part + s * n)[i];
    reinterpret_cast<f32x4_t*>(out)[i] = v;
  }
}

unsigned grid_for(int64_t n, int per = 256) {
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + per - 1) / per, 8192));
}

// out[p] = x[perm_token[p]] (rows of d bf16) for the real slots p < offsets[G] (at
// most R): the routed token rows in expert order.
__global__ void __launch_bounds__(256)
gather_slots_kernel(const bf16_t* __restrict__ x, const int32_t* __restrict__ perm_token, int64_t T,
                    const int32_t* __restrict__ offsets, int G, int64_t R, int d, bf16_t* __restrict__ out) {
  const int64_t cpr = d / 8;
  const int64_t n = min<int64_t>(max<int64_t>((int64_t)offsets[G], 0), R) * cpr;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t p = i / cpr, c = i - p * cpr;
    const int64_t t = min<int64_t>(max<int64_t>((int64_t)perm_token[p], 0), T - 1);
    *reinterpret_cast<u32x4_t*>(out + p * d + 8 * c) = *reinterpret_cast<const u32x4_t*>(x + t * d + 8 * c);
  }
}

}  // namespace

hipError_t launch_transpose(const void* in, int64_t batches, int64_t R, int64_t C, void* out, int64_t ldo,
                            int64_t c_out, int64_t out_batch, hipStream_t s) {
  if (batches <= 0 || R <= 0 || C <= 0) return hipSuccess;
  const dim3 grid((unsigned)((C + kTile - 1) / kTile), (unsigned)((R + kTile - 1) / kTile), (unsigned)batches);
  transpose_kernel<<<grid, 256, 0, s>>>(static_cast<const bf16_t*>(in), R, C, R * C,
                                        static_cast<bf16_t*>(out), ldo, c_out, out_batch);
  return hipGetLastError();
}

hipError_t launch_pad_offsets(const int32_t* offsets, int G, int64_t rows, int32_t* kofs, hipStream_t s) {
  pad_offsets_kernel<<<1, 64, 0, s>>>(offsets, G, rows, kofs);
  return hipGetLastError();
}

hipError_t launch_transpose_segments(const void* src, const int32_t* src_rows, int64_t src_nrows,
                                     const int32_t* offsets, const int32_t* kofs, int G, int64_t rows,
                                     int64_t C, void* dst, int64_t ld, hipStream_t s) {
  if (rows <= 0 || C <= 0 || ld <= 0) return hipSuccess;
  const dim3 grid((unsigned)((C + kTile - 1) / kTile), (unsigned)((ld + kTile - 1) / kTile));
  transpose_segments_kernel<<<grid, 256, 0, s>>>(static_cast<const bf16_t*>(src), src_rows, src_nrows,
                                                 offsets, kofs, G, rows, C, static_cast<bf16_t*>(dst), ld);
  return hipGetLastError();
}

hipError_t launch_gather_slots(const void* x, const int32_t* perm_token, int64_t T, const int32_t* offsets, int G,
                               int64_t R, int d, void* out, hipStream_t s) {
  if (R <= 0 || T <= 0) return hipSuccess;
  gather_slots_kernel<<<grid_for(R * (d / 8)), 256, 0, s>>>(static_cast<const bf16_t*>(x), perm_token, T, offsets, G,
                                                             R, d, static_cast<bf16_t*>(out));
  return hipGetLastError();
}

hipError_t launch_swiglu_h(const float* g, const float* u, const int32_t* offsets, int G, int64_t rows, int F,
                           void* h, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  swiglu_h_kernel<<<grid_for(rows * F), 256, 0, s>>>(g, u, offsets, G, rows, F, static_cast<bf16_t*>(h));
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const void* g, const void* u, bool g16, const float* dh, const int32_t* offsets, int G,
                             int64_t rows, int F, void* dgu, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (g16)
    swiglu_bwd_kernel<_Float16><<<grid_for(rows * F), 256, 0, s>>>(
        static_cast<const _Float16*>(g), static_cast<const _Float16*>(u), dh, offsets, G, rows, F,
        static_cast<bf16_t*>(dgu));
  else
    swiglu_bwd_kernel<float><<<grid_for(rows * F), 256, 0, s>>>(
        static_cast<const float*>(g), static_cast<const float*>(u), dh, offsets, G, rows, F, static_cast<bf16_t*>(dgu));
  return hipGetLastError();
}

hipError_t launch_slot_rows(const void* dy, const int32_t* slot_pos, const float* topk_w, int64_t T, int K,
                            int d, int64_t R, void* dy_perm, float* w_perm, int32_t* row_slot, float* dw,
                            hipStream_t s) {
  if (T <= 0) return hipSuccess;
  slot_rows_kernel<<<(unsigned)((T * K + 3) / 4), 256, 0, s>>>(static_cast<const bf16_t*>(dy), slot_pos, topk_w,
                                                                T, K, d, R, static_cast<bf16_t*>(dy_perm), w_perm,
                                                                row_slot, dw);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd_routed(const void* g, const void* u, bool g16, const float* U, const void* h,
                                    const float* w_perm, const int32_t* row_slot, const int32_t* offsets, int G,
                                    int64_t rows, int F, void* dgu, float* dw, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (g16)
    swiglu_bwd_routed_kernel<_Float16><<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(
        static_cast<const _Float16*>(g), static_cast<const _Float16*>(u), U, static_cast<const bf16_t*>(h), w_perm,
        row_slot, offsets, G, rows, F, static_cast<bf16_t*>(dgu), dw);
  else
    swiglu_bwd_routed_kernel<float><<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(
        static_cast<const float*>(g), static_cast<const float*>(u), U, static_cast<const bf16_t*>(h), w_perm,
        row_slot, offsets, G, rows, F, static_cast<bf16_t*>(dgu), dw);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const float* logits, const int32_t* topk_idx, const float* topk_w, const float* dw,
                             const float* f, int64_t T, int N, int M, int K, float alpha, float beta, float* ds,
                             hipStream_t s) {
  if (T <= 0) return hipSuccess;
  router_bwd_kernel<<<(unsigned)((T + 3) / 4), 256, 0, s>>>(logits, topk_idx, topk_w, dw, f, T, N, M, K, alpha,
                                                           beta, ds);
  return hipGetLastError();
}

// Token chunks of the router weight gradient: 64 tokens each, at most 256 chunks.
// Token chunks of the router weight gradient: 64 tokens each, but no more than keep
// the grid near 1024 workgroups, so the float32 partials (chunks x (N+1) x d) stay
// small next to x.
static int64_t router_chunks(int64_t T, int N1, int d) {
  const int64_t tiles = (int64_t)((d + 511) / 512) * ((N1 + kRouterRows - 1) / kRouterRows);
  return std::max<int64_t>(1, std::min<int64_t>(std::max<int64_t>(1, 1024 / tiles), (T + 63) / 64));
}

size_t router_wgrad_ws_bytes(int64_t T, int N1, int d) {
  return (size_t)router_chunks(T, N1, d) * N1 * d * sizeof(float);
}

hipError_t launch_router_wgrad(const float* ds, const void* x, int64_t T, int N1, int d, float* part, float* dw,
                               hipStream_t s) {
  const int64_t chunks = router_chunks(T, N1, d);
  const int64_t chunk = (T + chunks - 1) / chunks;
  const dim3 grid((unsigned)((d + 511) / 512), (unsigned)((N1 + kRouterRows - 1) / kRouterRows), (unsigned)chunks);
  router_wgrad_partial_kernel<<<grid, 256, 0, s>>>(ds, static_cast<const bf16_t*>(x), T, N1, d, chunk, part);
  const int64_t n = (int64_t)N1 * d;
  router_wgrad_reduce_kernel<<<grid_for(n), 256, 0, s>>>(part, (int)chunks, n, dw);
  return hipGetLastError();
}

hipError_t launch_scatter_dx(const float* dx_perm, const int32_t* slot_pos, int K, int64_t R, const float* dx_shared,
                             const float* ds, const float* w_router, int N1, int d, int64_t T, float* dx,
                             hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const dim3 grid((unsigned)((T + kScatterTok - 1) / kScatterTok), (unsigned)((d + 255) / 256));
  scatter_dx_kernel<<<grid, 256, 0, s>>>(
      dx_perm, slot_pos, K, R, dx_shared, ds, w_router, N1, d, T, dx);
  return hipGetLastError();
}

hipError_t launch_split_offsets(int64_t rows, int S, int32_t* kofs, hipStream_t s) {
  split_offsets_kernel<<<1, 64, 0, s>>>(rows, S, kofs);
  return hipGetLastError();
}

hipError_t launch_sum_partials(const float* part, int S, int64_t n, float* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n % 4) return hipErrorInvalidValue;
  sum_partials_kernel<<<grid_for(n / 4), 256, 0, s>>>(part, S, n, out);
  return hipGetLastError();
}

}  // namespace moe
