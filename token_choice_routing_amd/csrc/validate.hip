// Input check behind moe_validate_inputs: counts non-finite values in a device
// array (not part of the forward; NaN inputs leave the layer's outputs undefined).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// count[0] += the number of elements whose exponent bits are all ones: NaN or
// +-inf, or with nan_only NaN alone (all-ones exponent and a nonzero mantissa).
// Elements are bf16 (16-bit patterns) or float32.
__global__ void __launch_bounds__(256)
count_nonfinite_kernel(const void* __restrict__ data, int64_t n, int bf16, int nan_only, int32_t* count) {
  int local = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    uint32_t exp_bits, man_bits;
    if (bf16) {
      const uint32_t v = static_cast<const uint16_t*>(data)[i];
      exp_bits = (v >> 7) & 0xFF;
      man_bits = v & 0x7F;
    } else {
      const uint32_t v = static_cast<const uint32_t*>(data)[i];
      exp_bits = (v >> 23) & 0xFF;
      man_bits = v & 0x7FFFFF;
    }
    local += exp_bits == 0xFF && (!nan_only || man_bits != 0);
  }
  if (local) atomicAdd(count, local);
}

__global__ void zero_count_kernel(int32_t* count) {
  if (threadIdx.x == 0) count[0] = 0;
}

}  // namespace

hipError_t launch_zero_count(int32_t* count, hipStream_t s) {
  zero_count_kernel<<<1, 64, 0, s>>>(count);
  return hipGetLastError();
}

hipError_t launch_count_nonfinite(const void* data, int64_t n, bool bf16, bool nan_only, int32_t* count,
                                  hipStream_t s) {
  if (!data || n <= 0) return hipSuccess;
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 4096));
  count_nonfinite_kernel<<<grid, 256, 0, s>>>(data, n, bf16 ? 1 : 0, nan_only ? 1 : 0, count);
  return hipGetLastError();
}

}  // namespace moe
