// Seeded synthetic inputs, device side.
//
// Same definition as synth_host.c (counter-form SplitMix64 from Steele, Lea
// and Flood, OOPSLA 2014; N(0,1) via a 65,536-entry bf16 quantile table that
// the caller uploads).  It fills the large caches in place on the GPU so that
// a 64 GiB KV cache does not have to cross PCIe.  Holds none of the
// attention, rope or quantisation arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9e3779b97f4a7c15ULL;
constexpr uint64_t kOdd = 0xd1342543de82ef95ULL;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

__host__ __device__ inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64((seed * kGamma) ^ (stream * kOdd));
}

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Each thread writes 8 consecutive elements (one 16-byte store).
__global__ void fill_bf16_kernel(uint64_t key, uint64_t okey, uint64_t first_index, int64_t n8,
                                 int32_t row, const uint16_t* __restrict__ table,
                                 const float* __restrict__ chan_mul, uint32_t thresh, float omul,
                                 uint16_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    uint16_t v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      int64_t e = i * 8 + k;
      uint64_t idx = first_index + (uint64_t)e;
      uint16_t x = table[mix64(key + (idx + 1) * kGamma) >> 48];
      if (chan_mul) x = f32_to_bf16_rne(bf16_to_f32(x) * chan_mul[e % row]);
      if (thresh && (uint32_t)(mix64(okey + (idx + 1) * kGamma) >> 40) < thresh)
        x = f32_to_bf16_rne(bf16_to_f32(x) * omul);
      v[k] = x;
    }
    uint4 w;
    w.x = v[0] | ((uint32_t)v[1] << 16);
    w.y = v[2] | ((uint32_t)v[3] << 16);
    w.z = v[4] | ((uint32_t)v[5] << 16);
    w.w = v[6] | ((uint32_t)v[7] << 16);
    reinterpret_cast<uint4*>(out)[i] = w;
  }
}

}  // namespace

// Device twin of synth_fill_bf16 (host).  out must hold ntok*nheads*dim bf16
// and be 16-byte aligned; nheads*dim must be a multiple of 8.  Returns 0, or
// -1 on bad arguments / launch failure.
extern "C" int synth_dev_fill_bf16(uint64_t seed, uint64_t stream, int64_t token0, int64_t ntok,
                                   int32_t nheads, int32_t dim, const uint16_t* table,
                                   const float* chan_mul, uint64_t outlier_stream,
                                   uint32_t outlier_thresh, float outlier_mul, uint16_t* out,
                                   hipStream_t stream_h) {
  if (!table || !out || ntok < 0 || nheads <= 0 || dim <= 0) return -1;
  int64_t row = (int64_t)nheads * dim;
  if (row % 8 != 0 || ((uintptr_t)out & 15u) != 0) return -1;
  if (ntok == 0) return 0;
  int64_t n8 = ntok * row / 8;
  int64_t blocks = (n8 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  // The launch's own status (not the sticky last-error state).
  uint64_t key = stream_key(seed, stream), okey = stream_key(seed, outlier_stream);
  uint64_t first = (uint64_t)token0 * (uint64_t)row;
  int32_t row32 = (int32_t)row;
  void* args[] = {&key, &okey, &first, &n8, &row32, &table, &chan_mul, &outlier_thresh,
                  &outlier_mul, &out};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(fill_bf16_kernel),
                                       dim3((unsigned)blocks), dim3(256), args, 0, stream_h);
  return e == hipSuccess ? 0 : -(int)e;
}
