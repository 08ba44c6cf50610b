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
  int64_t blocks = (k.total + 255) / 256;
  if (blocks > 1 << 20) blocks = 1 << 20;
  return launch(rope_kernel, dim3((unsigned)blocks), dim3(256), 0, s, k);
}

}  // namespace yrk
