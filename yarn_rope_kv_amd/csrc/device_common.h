// Device helpers shared by the gfx950 kernels of libyrk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace yrk {

template <typename T>
struct same_type { using type = T; };

// Enqueue a kernel and return the launch's own status.  (Reading the sticky
// hipGetLastError() state instead would also report an error some earlier,
// unrelated call left behind.)
template <typename... KArgs>
inline hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                         hipStream_t stream, typename same_type<KArgs>::type... args) {
  void* ptrs[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, shmem, stream);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp64 -> bf16 bits with a single rounding to nearest even: first to fp32
// rounding toward zero with a sticky bit ("round to odd", which keeps every
// bit the second rounding needs because fp32 carries 16 more significant bits
// than bf16 at every exponent bf16 has), then fp32 -> bf16 RNE.
__device__ __forceinline__ uint16_t f64_to_bf16(double d) {
  float f = __double2float_rz(d);
  uint32_t u = __float_as_uint(f);
  if ((double)f != d) u |= 1u;
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void set_error(uint32_t* err, uint32_t bit) {
  if (err) atomicOr(err, bit);
}

}  // namespace yrk
