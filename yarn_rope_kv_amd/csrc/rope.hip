// YaRN rotary embedding, applied in place to bf16 heads.
//
// [P1] "YaRN, and matching what vLLM actually does": the rotary table is
// stretched by YaRN and the attention temperature mscale is applied to cos
// and sin inside the rope, on the rotary dimensions only.  [P3] "YaRN
// reference and drift guard": 64 rotary dimensions of each 256-element head.
//
// One thread owns one (token, rotation pair) and walks the heads of that
// token, so the fp64 angle and its sin/cos are computed once per pair and
// reused by every head.  fp64 is needed for the angle: at positions near
// 2^20 an fp32 product p * inv_freq is off by up to ~0.06 rad.  The rotation
// itself is also done in fp64 and rounded once to bf16, so the result is the
// correctly rounded value of the exact rotation up to fp64 noise.
//
// Memory: each pair touches 2 x 2 bytes per head (read) and the same again
// (write); the pass-through dimensions are never read.  Lanes of a wave take
// consecutive pairs of one token, so the two 64-byte halves of the rotary
// slice are each read by 32 adjacent lanes.
#include "rope_common.h"
#include "yrk_internal.h"

namespace yrk {
namespace {

struct RopeKernelArgs {
  uint16_t* x;
  int64_t total;          // num_tokens * half
  int64_t token_stride;
  int32_t num_heads;
  int32_t head_dim;
  int32_t half;
  const int32_t* positions;
  uint32_t* err;
  double mscale;
  double inv_freq[kMaxRotaryHalf];
};

__global__ __launch_bounds__(256) void rope_kernel(RopeKernelArgs a) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < a.total; gid += stride) {
    const int64_t t = gid / a.half;
    const int i = (int)(gid - t * a.half);
    const int32_t pos = a.positions[t];
    if (pos < 0) {                  // the token is left as it is and reported
      if (i == 0) set_error(a.err, kErrPosition);
      continue;
    }
    double c, s;
    rope_cos_sin(pos, a.inv_freq[i], a.mscale, &c, &s);
    uint16_t* row = a.x + t * a.token_stride + i;
    for (int h = 0; h < a.num_heads; ++h) {
      uint16_t* p = row + (int64_t)h * a.head_dim;
      const double x1 = (double)bf16_to_f32(p[0]);
      const double x2 = (double)bf16_to_f32(p[a.half]);
      p[0] = rope_first(x1, x2, c, s);
      p[a.half] = rope_second(x1, x2, c, s);
    }
  }
}

// The same rotation with 16-byte accesses: one thread owns 8 consecutive
// pairs (8j .. 8j + 7) of one token and walks its heads, loading the 8
// first-half and the 8 second-half elements of a head with one 16-byte load
// each (4 threads cover a 64-dim rotary slice: 64 contiguous bytes per half).
// The element arithmetic is rope_first / rope_second, so the results are the
// same bits.  Used when the rotary half is a multiple of 8 and every row
// start is 16-byte aligned; the 2-byte accesses of rope_kernel took 8 times
// the memory instructions.
__global__ __launch_bounds__(256) void rope_kernel_x8(RopeKernelArgs a) {
  const int groups = a.half / 8;
  const int64_t total = a.total / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < total; gid += stride) {
    const int64_t t = gid / groups;
    const int j = (int)(gid - t * groups);
    const int32_t pos = a.positions[t];
    if (pos < 0) {                  // the token is left as it is and reported
      if (j == 0) set_error(a.err, kErrPosition);
      continue;
    }
    double c[8], sn[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) rope_cos_sin(pos, a.inv_freq[8 * j + k], a.mscale, &c[k], &sn[k]);
    uint16_t* row = a.x + t * a.token_stride + 8 * j;
    for (int h = 0; h < a.num_heads; ++h) {
      uint4* p1 = reinterpret_cast<uint4*>(row + (int64_t)h * a.head_dim);
      uint4* p2 = reinterpret_cast<uint4*>(row + (int64_t)h * a.head_dim + a.half);
      const uint4 u1 = *p1, u2 = *p2;
      const uint32_t w1[4] = {u1.x, u1.y, u1.z, u1.w}, w2[4] = {u2.x, u2.y, u2.z, u2.w};
      uint32_t r1[4], r2[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint16_t lo1, hi1, lo2, hi2;
        {
          const double x1 = (double)bf16_to_f32((uint16_t)(w1[q] & 0xffffu));
          const double x2 = (double)bf16_to_f32((uint16_t)(w2[q] & 0xffffu));
          lo1 = rope_first(x1, x2, c[2 * q], sn[2 * q]);
          lo2 = rope_second(x1, x2, c[2 * q], sn[2 * q]);
        }
        {
          const double x1 = (double)bf16_to_f32((uint16_t)(w1[q] >> 16));
          const double x2 = (double)bf16_to_f32((uint16_t)(w2[q] >> 16));
          hi1 = rope_first(x1, x2, c[2 * q + 1], sn[2 * q + 1]);
          hi2 = rope_second(x1, x2, c[2 * q + 1], sn[2 * q + 1]);
        }
        r1[q] = (uint32_t)lo1 | ((uint32_t)hi1 << 16);
        r2[q] = (uint32_t)lo2 | ((uint32_t)hi2 << 16);
      }
      *p1 = make_uint4(r1[0], r1[1], r1[2], r1[3]);
      *p2 = make_uint4(r2[0], r2[1], r2[2], r2[3]);
    }
  }
}

}  // namespace

hipError_t launch_rope(const RopeArgs& a, hipStream_t s) {
  RopeKernelArgs k;
  k.x = a.x;
  k.total = a.num_tokens * a.half;
  k.token_stride = a.token_stride;
  k.num_heads = a.num_heads;
  k.head_dim = a.head_dim;
  k.half = a.half;
  k.positions = a.positions;
  k.err = a.err;
  k.mscale = a.mscale;
  for (int i = 0; i < kMaxRotaryHalf; ++i) k.inv_freq[i] = i < a.half ? a.inv_freq[i] : 0.0;
  if (k.total == 0) return hipSuccess;
  const bool x8 = a.half % 8 == 0 && ((uintptr_t)a.x & 15u) == 0 && a.token_stride % 8 == 0 &&
                  a.head_dim % 8 == 0;
  const int64_t threads = x8 ? k.total / 8 : k.total;
  int64_t blocks = (threads + 255) / 256;
  if (blocks > 1 << 20) blocks = 1 << 20;
  if (x8) return launch(rope_kernel_x8, dim3((unsigned)blocks), dim3(256), 0, s, k);
  return launch(rope_kernel, dim3((unsigned)blocks), dim3(256), 0, s, k);
}

}  // namespace yrk
