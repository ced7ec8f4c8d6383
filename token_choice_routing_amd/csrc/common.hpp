// Shared device helpers for the gfx950 kernels of libmoe_mi355x.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bf16 bit pattern
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Two float32 values as IEEE half, round to nearest even (beyond +-65504: infinity).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f16x2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Eight bf16 values as IEEE half: exact for every bf16 value of magnitude in
// [2^-17, 65504] (bf16's 8 significant bits fit half's 11, and half subnormals
// reach down to 2^-24 in steps of 2^-24); smaller magnitudes are truncated toward
// zero to a multiple of 2^-24. Each bf16 pair is widened to float32 by a shift or a
// mask and packed by one v_cvt_pkrtz_f16_f32.
__device__ __forceinline__ f16x8_t bf16x8_to_f16x8(bf16x8_t v) {
  const u32x4_t u = __builtin_bit_cast(u32x4_t, v);
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(u[i] << 16),
                                                                  __uint_as_float(u[i] & 0xffff0000u)));
  return __builtin_bit_cast(f16x8_t, o);
}

// Element access for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ double wave_sum_double(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// s_waitcnt immediate that waits until at most n vector-memory operations of this
// wavefront are outstanding (lgkmcnt and expcnt left alone).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
}

// Waits until at most n (wave-uniform, clamped to [0, MAX]) vector memory
// operations of this wavefront are outstanding.
template <int MAX>
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  if constexpr (MAX > 0) {
    if (n >= MAX) {
      wait_vmcnt<MAX>();
      return;
    }
    wait_vmcnt_upto<MAX - 1>(n);
  } else {
    wait_vmcnt<0>();
  }
}

// 16-byte global -> LDS load (global_load_lds_dwordx4). The LDS address must be
// uniform across the wavefront; lane l writes bytes [16 l, 16 l + 16) after it. The
// builtin only exists in the device compilation pass, where it is kept.
__device__ __forceinline__ void load_lds16(const bf16_t* g, bf16_t* l) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
#else
  (void)g;
  (void)l;
#endif
}

// Raw buffer resource over [base, base + bytes) (stride 0, 32-bit data format
// word as for every CDNA raw buffer access). Reads at offsets past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// v unchanged, but opaque to the optimiser: values computed from the result cannot
// be computed earlier than this point (keeps them out of long loops' live ranges).
__device__ __forceinline__ int opaque_v(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// A pointer the caller knows to be the same in every lane, as the compiler's
// uniform (scalar) value: buffer resources built from it stay in SGPRs.
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
}

// 16-byte buffer -> LDS load (buffer_load_dwordx4 ... lds), same LDS placement as
// load_lds16. Unlike the global form, the compiler's wait-count tracking does not
// count it as an LDS-side (lgkm) event, so LDS reads after it keep exact waits.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voffset, bf16_t* l) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(l),
                                           16, voffset, 0, 0, 0);
#else
  (void)r;
  (void)voffset;
  (void)l;
#endif
}

// LDS-only workgroup barrier for tiles written by global->LDS loads: each wavefront
// first retires its own LDS reads; the caller has already waited (vmcnt) for the
// loads that filled the stage about to be read. The asm statement is also a
// compiler memory barrier, so no LDS access moves across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // The same wait again through the builtin, which the compiler's counter tracking
  // sees (it does not read the asm): the LDS reads after the barrier then get exact
  // lgkmcnt waits instead of lgkmcnt(0).
  __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4));
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

}  // namespace moe
