// Deterministic weighted combine of the expert outputs back into token order.
//
// Paper review "Improving MoE Compute Efficiency by Composing Weight and Data
// Sparsity", section 3, core formula of the token-choice layer with a shared
// expert: y = E_shared(x) + sum_k g_k E_{i_k}(x). A null slot (slot_pos = -1)
// contributes E_null(x) = 0, or with copy / constant zero-compute experts g_k x
// or g_k v (its row of null_src, in the same slot order).
//
// One wavefront per token row: the K (position, weight) pairs are loaded once
// by lanes 0..K-1 and broadcast with shuffles; each lane owns 8-element
// vectors of the row and accumulates the float32 expert outputs in float32 in
// slot order, then rounds once to the output type. No atomics, so repeated
// runs are bitwise identical.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

template <typename ET>
struct Vec8;
template <>
struct Vec8<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float* v) {
    const u32x4_t u = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      v[2 * h] = __uint_as_float(u[h] << 16);
      v[2 * h + 1] = __uint_as_float(u[h] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float* v) {
    *reinterpret_cast<u32x4_t*>(p) = u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                             pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
  }
};
template <>
struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float* v) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      v[h] = a[h];
      v[4 + h] = b[h];
    }
  }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    *reinterpret_cast<f32x4_t*>(p) = f32x4_t{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4_t*>(p + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
  }
};

// y_perm and y_shared are float32; y is ET (bf16 or float32).
template <typename ET, int VPL>  // VPL: 8-element vectors per lane per pass
__global__ void __launch_bounds__(256)
combine_kernel(const float* __restrict__ y_perm, const int32_t* __restrict__ slot_pos,
               const float* __restrict__ topk_w, const float* __restrict__ y_shared,
               const ET* __restrict__ null_src, int64_t null_stride,
               ET* __restrict__ y, int64_t T, int K, int d, int64_t max_rows) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * blockDim.x / kWave;
  const int vpr = d / 8;
  for (int64_t t = wave; t < T; t += nwaves) {
    int my_p = -1;
    float my_w = 0.0f;
    if (lane < K) {
      my_p = slot_pos[t * K + lane];
      my_w = topk_w[t * K + lane];
      // -1: a null slot; -2: nothing to add (a slot past capacity, or no null source)
      if (my_p == -1 ? !null_src : (my_p < 0 || my_p >= max_rows)) my_p = -2;
    }
    for (int v0 = 0; v0 < vpr; v0 += kWave * VPL) {
      float acc[VPL][8];
#pragma unroll
      for (int u = 0; u < VPL; ++u) {
        const int v = v0 + u * kWave + lane;
        if (y_shared && v < vpr) {
          Vec8<float>::load(y_shared + t * d + v * 8, acc[u]);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[u][j] = 0.0f;
        }
      }
      for (int k = 0; k < K; ++k) {
        const int p = __shfl(my_p, k, kWave);
        const float w = __shfl(my_w, k, kWave);
        if (p == -2) continue;
#pragma unroll
        for (int u = 0; u < VPL; ++u) {
          const int v = v0 + u * kWave + lane;
          if (v < vpr) {
            float r[8];
            if (p >= 0) Vec8<float>::load(y_perm + (int64_t)p * d + v * 8, r);
            else Vec8<ET>::load(null_src + t * null_stride + v * 8, r);
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[u][j] = fmaf(w, r[j], acc[u][j]);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < VPL; ++u) {
        const int v = v0 + u * kWave + lane;
        if (v < vpr) Vec8<ET>::store(y + t * d + v * 8, acc[u]);
      }
    }
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.T <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((a.T + 3) / 4, 65536);
  const int vpr = a.d / 8;
  const float* yp = static_cast<const float*>(a.y_perm);
  const float* ys = static_cast<const float*>(a.y_shared);
  if (a.bf16) {
    if (vpr >= 4 * kWave)
      combine_kernel<bf16_t, 4><<<(unsigned)blocks, 256, 0, stream>>>(
          yp, a.slot_pos, a.topk_w, ys, static_cast<const bf16_t*>(a.null_src), a.null_stride,
          static_cast<bf16_t*>(a.y), a.T, a.K, a.d, a.max_rows);
    else
      combine_kernel<bf16_t, 2><<<(unsigned)blocks, 256, 0, stream>>>(
          yp, a.slot_pos, a.topk_w, ys, static_cast<const bf16_t*>(a.null_src), a.null_stride,
          static_cast<bf16_t*>(a.y), a.T, a.K, a.d, a.max_rows);
  } else {
    combine_kernel<float, 1><<<(unsigned)blocks, 256, 0, stream>>>(
        yp, a.slot_pos, a.topk_w, ys, static_cast<const float*>(a.null_src), a.null_stride,
        static_cast<float*>(a.y), a.T, a.K, a.d, a.max_rows);
  }
  return hipGetLastError();
}

}  // namespace moe
