// KV append into the paged cache: an exact bf16 copy, or NVFP4 or INT8
// group-64 quantisation on the way in; plus the per-tensor NVFP4 scale.
//
// Paging follows [P1] "Things that bit me" (per-sequence page lists), [P3]
// "Current limits" (one shared pool fixed at start-up) and the HND page
// layout of [P5] "Validation before vibes": a page holds, per KV head, 16
// consecutive token rows.  The NVFP4 format is the one of [P5] "Why NVFP4 KV
// changes the math": e2m1 element codes, one e4m3 scale per 16 contiguous
// head-dim elements, one fp32 tensor scale S = amax / (6 * 448).  The INT8
// cache is the deployed 1M-token format of [P3] (memory table) and [P1] "And
// the memory picture": groups of 64 with 2-byte scales, 16.5 KiB per token
// per device; its rounding rules are readings (symmetric absmax groups,
// binary16 scale RNE(amax / 127), codes clamp(RNE(x / s), +-127)).
#include "rope_common.h"
#include "yrk_internal.h"

namespace yrk {
namespace {

constexpr int kChunksPerRow = kHeadDim * 2 / 16;  // 16-byte chunks of a bf16 row
constexpr int kQBlocks = kHeadDim / 16;           // NVFP4 scale blocks per row

// Row index (in units of one head row) of logical position `pos` for KV head
// h, or -1 after flagging the error.
__device__ __forceinline__ int64_t cache_row(const KvGeometry& g, const int32_t* table,
                                             int64_t table_len, int32_t pos, int h,
                                             uint32_t* err, bool report) {
  if (g.paged) {
    const int64_t b = pos / kBlockSize;
    if (pos < 0 || b >= table_len) {
      if (report) set_error(err, kErrPosition);
      return -1;
    }
    const int64_t blk = table[b];
    if (blk < 0 || blk >= g.num_blocks) {
      if (report) set_error(err, kErrBlockId);
      return -1;
    }
    return (blk * g.num_kv_heads + h) * kBlockSize + pos % kBlockSize;
  }
  if (pos < 0 || (int64_t)pos >= g.num_blocks * kBlockSize) {
    if (report) set_error(err, kErrPosition);
    return -1;
  }
  return (int64_t)pos * g.num_kv_heads + h;
}

// One thread copies one 16-byte chunk of K and the matching chunk of V.
__global__ __launch_bounds__(256) void append_bf16_kernel(AppendArgs a) {
  const int H = a.geo.num_kv_heads;
  const int64_t total = a.num_tokens * H * kChunksPerRow;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < total; gid += stride) {
    const int64_t t = gid / (H * kChunksPerRow);
    const int rem = (int)(gid - t * H * kChunksPerRow);
    const int h = rem / kChunksPerRow;
    const int c = rem % kChunksPerRow;
    // the source loads go out before the destination lookup (position, then
    // page table), whose latency they then overlap
    const int64_t src = (t * H + h) * kChunksPerRow + c;
    const uint4 kx = reinterpret_cast<const uint4*>(a.k_src)[src];
    const uint4 vx = reinterpret_cast<const uint4*>(a.v_src)[src];
    const int64_t row = cache_row(a.geo, a.block_table, a.block_table_len, a.positions[t], h,
                                  a.err, c == 0);
    if (row < 0) continue;
    const int64_t dst = row * kChunksPerRow + c;
    reinterpret_cast<uint4*>(a.k_dst)[dst] = kx;
    reinterpret_cast<uint4*>(a.v_dst)[dst] = vx;
  }
}

// ---- NVFP4 -----------------------------------------------------------------

// e4m3 (OCP E4M3FN) value of a non-negative code 0x00..0x7E, exact.
__device__ __forceinline__ double e4m3_value(int code) {
  const int e = code >> 3, m = code & 7;
  return e == 0 ? (double)m * 0x1p-9 : ldexp((double)(8 + m), e - 10);
}

// Nearest e4m3 code to q >= 0, ties to even mantissa, saturating at 448.
// Works on the IEEE-754 binary64 fields of q: keep 3 fraction bits (or the
// subnormal multiple of 2^-9) and round the dropped bits half-to-even.
__device__ __forceinline__ int e4m3_encode(double q) {
  if (!(q < 448.0)) return 0x7E;
  if (q == 0.0) return 0;
  const uint64_t u = (uint64_t)__double_as_longlong(q);
  const int E = (int)(u >> 52) - 1023;           // q is a normal fp64 here
  const uint64_t sig = (u & 0xFFFFFFFFFFFFFull) | (1ull << 52);
  if (E >= -6) {
    // keep the leading 1 + 3 bits: drop 49 bits
    uint64_t keep = sig >> 49;
    const uint64_t rest = sig & ((1ull << 49) - 1);
    const uint64_t half = 1ull << 48;
    if (rest > half || (rest == half && (keep & 1))) ++keep;   // may carry to 16
    int code = ((E + 7) << 3) + (int)(keep - 8);               // carry bumps the exponent
    return code > 0x7E ? 0x7E : code;
  }
  // subnormal target: k = RNE(q * 2^9) = RNE(sig * 2^(E - 43))
  const int shift = 43 - E;  // >= 50
  if (shift >= 64) return 0;
  uint64_t keep = sig >> shift;
  const uint64_t rest = sig & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rest > half || (rest == half && (keep & 1))) ++keep;
  return (int)keep;  // 0..8; 8 is the smallest normal, code 0x08
}

// The scale of one 16-element block from its largest magnitude (bf16 bits;
// |x| orders like the low 15 bits): the e4m3 code and what the element codes
// are decided with: the effective scale e4m3 * S (exact in fp64) and, for the
// fp32 path, e4m3 (exact in fp32) and S as fp32.
struct Fp4Block {
  int qs;
  double eff;
  float e4, s32;
};
__device__ __forceinline__ Fp4Block nvfp4_block(uint32_t bmax_bits, double S) {
  const double b = (double)bf16_to_f32((uint16_t)bmax_bits);
  Fp4Block B;
  B.qs = e4m3_encode(b / (6.0 * S));
  const double e4 = e4m3_value(B.qs);
  B.eff = e4 * S;
  B.e4 = (float)e4;
  B.s32 = (float)S;
  return B;
}

// Whether the fp32 decisions below are exact for tensor scale S (an fp32
// value): 2^-109 <= S <= 2^100.  Outside that range (tensor maxima below
// ~2^-97 or a caller's own extreme scale) the fp64 decisions are taken.
__device__ __forceinline__ bool nvfp4_f32_exact(double S) {
  return S >= 0x1p-109 && S <= 0x1p100;
}

// Code of one bf16 element: sign bit | nearest e2m1 magnitude of |x| / eff.
// Decision points between neighbouring e2m1 magnitudes, scaled by eff: at a
// point exactly between two codes the even code wins (>= where the upper
// code is even, > where the lower one is).
__device__ __forceinline__ uint32_t nvfp4_code(uint32_t bits, const Fp4Block& B) {
  const double a = (double)bf16_to_f32((uint16_t)(bits & 0x7fffu));
  const double e = B.eff;
  uint32_t mag = 0;
  if (e > 0.0)
    mag = (uint32_t)(a > 0.25 * e) + (uint32_t)(a >= 0.75 * e) + (uint32_t)(a > 1.25 * e) +
          (uint32_t)(a >= 1.75 * e) + (uint32_t)(a > 2.5 * e) + (uint32_t)(a >= 3.5 * e) +
          (uint32_t)(a > 5.0 * e);
  return (((bits >> 15) & 1u) << 3) | mag;
}

// The same code from fp32 arithmetic, exact when nvfp4_f32_exact(S).  Each
// decision compares a = |x| with t e4 S for a decision point t: P = t e4 is
// exact in fp32 (t has at most 3 significant bits, e4 at most 4), and the
// fused multiply-add rounds a - P S once, so its sign is the sign of the
// exact difference unless that difference rounds to zero without being zero.
// It cannot: a is a multiple of 2^-133 (bf16), P of 2^-11 and S (normal, at
// least 2^-109) of 2^(e_S - 23) >= 2^-132, so a nonzero difference is at
// least 2^-143 in magnitude; and with S <= 2^100 nothing overflows.  The
// 7 monotone decisions are taken as a binary search: 1.75 (>=), then 0.75 or
// 3.5 (>=), then 0.25, 1.25, 2.5 or 5 (>).
__device__ __forceinline__ uint32_t nvfp4_code_f32(uint32_t bits, const Fp4Block& B) {
  const float a = bf16_to_f32((uint16_t)(bits & 0x7fffu));
  const float e4 = B.e4, S = B.s32;
  const bool c1 = __builtin_fmaf(-1.75f * e4, S, a) >= 0.0f;
  const bool c2 = __builtin_fmaf(-(c1 ? 3.5f : 0.75f) * e4, S, a) >= 0.0f;
  const float t3 = c1 ? (c2 ? 5.0f : 2.5f) : (c2 ? 1.25f : 0.25f);
  const bool c3 = __builtin_fmaf(-t3 * e4, S, a) > 0.0f;
  const uint32_t mag = B.qs == 0 ? 0u : (uint32_t)c1 * 4u + (uint32_t)c2 * 2u + (uint32_t)c3;
  return (((bits >> 15) & 1u) << 3) | mag;
}

// Quantise 16 bf16 values: returns the scale code and writes 8 packed bytes
// (element 2j in the low nibble of byte j).
__device__ __forceinline__ uint32_t quantize16(const uint4 lo, const uint4 hi, double S,
                                               uint2* packed) {
  uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  uint32_t bmax = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    bmax = max(bmax, w[i] & 0x7fffu);
    bmax = max(bmax, (w[i] >> 16) & 0x7fffu);
  }
  const Fp4Block B = nvfp4_block(bmax, S);
  uint32_t out[2] = {0u, 0u};
  if (nvfp4_f32_exact(S)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t bits = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xffffu);
      out[i >> 3] |= nvfp4_code_f32(bits, B) << (4 * (i & 7));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t bits = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xffffu);
      out[i >> 3] |= nvfp4_code(bits, B) << (4 * (i & 7));
    }
  }
  packed->x = out[0];
  packed->y = out[1];
  return (uint32_t)B.qs;
}

// One wave per token: lane l quantises block l % 16 (16 elements) of K and
// of V of head h0 + l / 16, four heads per pass; the source loads go out
// ahead of the token's one destination lookup (position, then page table),
// and head h's row follows head 0's at a fixed stride.
__global__ __launch_bounds__(256) void append_nvfp4_kernel(AppendArgs a) {
  const int H = a.geo.num_kv_heads;
  const int lane = threadIdx.x & 63;
  const int hl = lane >> 4, qb = lane & 15;
  const double kS = (double)*a.k_tensor_scale;
  const double vS = (double)*a.v_tensor_scale;
  const int64_t wstride = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t hstride = a.geo.paged ? kBlockSize : 1;
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
       t < a.num_tokens; t += wstride) {
    const int32_t pos = a.positions[t];
    for (int h0 = 0; h0 < H; h0 += 4) {
      const int h = h0 + hl;
      uint4 k0 = make_uint4(0, 0, 0, 0), k1 = k0, v0 = k0, v1 = k0;
      if (h < H) {
        const int64_t src = ((t * H + h) * kHeadDim + qb * 16) / 8;   // in uint4 units
        const uint4* ks = reinterpret_cast<const uint4*>(a.k_src) + src;
        const uint4* vs = reinterpret_cast<const uint4*>(a.v_src) + src;
        k0 = ks[0], k1 = ks[1], v0 = vs[0], v1 = vs[1];
      }
      const int64_t row0 = cache_row(a.geo, a.block_table, a.block_table_len, pos, 0, a.err,
                                     lane == 0 && h0 == 0);
      if (row0 < 0) break;
      if (h < H) {
        const int64_t row = row0 + (int64_t)h * hstride;
        uint2 kp, vp;
        const uint32_t kq = quantize16(k0, k1, kS, &kp);
        const uint32_t vq = quantize16(v0, v1, vS, &vp);
        reinterpret_cast<uint2*>(a.k_dst)[row * kQBlocks + qb] = kp;
        reinterpret_cast<uint2*>(a.v_dst)[row * kQBlocks + qb] = vp;
        a.k_scale_dst[row * kQBlocks + qb] = (uint8_t)kq;
        a.v_scale_dst[row * kQBlocks + qb] = (uint8_t)vq;
      }
    }
  }
}

// ---- INT8 group-64 ---------------------------------------------------------

constexpr int kI8Groups = kHeadDim / 64;   // scale groups per row

// The group scale RNE_binary16(m / 127), saturating at 65504, for a group
// maximum m (bf16 bits), and its value.  Computed as m times the fp32
// nearest 1/127 (no division) and the conversion to binary16 (nearest even;
// the compiler may fuse the two into one mixed-precision multiply-add, which
// rounds the exact product once), which gives the rounding of the exact
// quotient: m = a 2^i with a < 2^8, a normal binary16 rounding midpoint is
// c 2^k with c odd and at least 2^11 + 1, so m / 127 is never one (the odd
// part of a 2^i would be 127 c) and lies at least 2^-19 (relative) from
// every one, while the product is within 2^-23 of it, rounded or not.  The
// one subnormal midpoint m / 127 reaches, 2^-25 from m = 127 2^-25, is
// approached from below (the fp32 1/127 is below 1/127) and rounds to 0 as
// the quotient does.  A host test checks every bf16 magnitude both ways.
// Every binary16 value is an fp32 value.
__device__ __forceinline__ uint32_t i8_group_scale(uint32_t mbits, float* value) {
  constexpr float kInv127 = 1.0f / 127.0f;   // the fp32 nearest 1/127
  const float q = bf16_to_f32((uint16_t)mbits) * kInv127;
  const uint32_t h =
      q < 65504.0f ? (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)q) : 0x7BFFu;
  *value = (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  return h;
}

// Largest of x over the 16 lanes of a DPP row (every lane gets it).
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x124, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4e, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xb1, 0xf, 0xf, false));
  return x;
}

// Four bf16 values (one lane's share of a group) -> four packed int8 codes
// and, in every lane, the group's binary16 scale bits.  The lanes of one DPP
// row (16 lanes x 4 = 64 elements) hold one group.  The scale is
// i8_group_scale of the group maximum.  Each code is RNE(x / s) clamped to
// +-127, decided without a division: with x = a 2^i (a < 2^8) and s = b 2^j
// (b < 2^11), x / s is either a half-integer exactly or at least 2^-12 away
// from every half-integer up to 127.5, while q = x * rcp(s) (the hardware
// reciprocal, within 1 ulp) is within 2^-17 of it; so rint(q) is the code
// unless x / s is a half-integer, which the exact test x - h s == 0 finds
// (h = floor(q) + 1/2 has 9 significant bits and s 11, so h s is exact in
// fp32 and the fused multiply-add rounds only a zero or non-zero result);
// then rint(h) is the even neighbour.  (Subnormal x only meet scales that
// make the quotient round to 0 either way.)
__device__ __forceinline__ uint32_t quantize_i8x4(uint2 w, uint32_t* scale_bits) {
  const uint32_t e[4] = {w.x & 0xffffu, w.x >> 16, w.y & 0xffffu, w.y >> 16};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, e[i] & 0x7fffu);   // |x| orders like its bits
  m = row16_max_u32(m);
  float sv;
  *scale_bits = i8_group_scale(m, &sv);
  // branch-free: a zero scale (an all-zero group) computes with s = 1; its
  // elements are all +-0, whose codes are then 0
  const bool zero = !(sv > 0.0f);
  const float s1 = zero ? 1.0f : sv;
  const float r = __builtin_amdgcn_rcpf(s1);
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float x = bf16_to_f32((uint16_t)e[i]);
    const float q = x * r;
    const float h = floorf(q) + 0.5f;
    const float k = fmaf(-h, s1, x) == 0.0f ? rintf(h) : rintf(q);
    const float kc = __builtin_amdgcn_fmed3f(k, -127.0f, 127.0f);
    const int c = (int)kc;
    packed |= ((uint32_t)c & 0xffu) << (8 * i);
  }
  return packed;
}

// One wave per token: lane l quantises elements 4l .. 4l+3 of K and of V of
// each of the token's head rows (group l / 16).  The source loads of up to
// kI8RowsInFlight heads go out together, ahead of the one destination
// lookup per token (position, then page table); head h's row follows head
// 0's at a fixed stride.
constexpr int kI8RowsInFlight = 4;

__global__ __launch_bounds__(256) void append_int8_kernel(AppendArgs a) {
  const int H = a.geo.num_kv_heads;
  const int lane = threadIdx.x & 63;
  const int64_t wstride = (int64_t)gridDim.x * (blockDim.x >> 6);
  const int64_t hstride = a.geo.paged ? kBlockSize : 1;
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
       t < a.num_tokens; t += wstride) {
    for (int h0 = 0; h0 < H; h0 += kI8RowsInFlight) {
      uint2 kw[kI8RowsInFlight], vw[kI8RowsInFlight];
#pragma unroll
      for (int i = 0; i < kI8RowsInFlight; ++i) {
        kw[i] = vw[i] = make_uint2(0u, 0u);
        if (h0 + i < H) {
          const int64_t r = t * H + h0 + i;
          kw[i] = reinterpret_cast<const uint2*>(a.k_src)[r * (kHeadDim / 4) + lane];
          vw[i] = reinterpret_cast<const uint2*>(a.v_src)[r * (kHeadDim / 4) + lane];
        }
      }
      const int64_t row0 = cache_row(a.geo, a.block_table, a.block_table_len, a.positions[t], 0,
                                     a.err, lane == 0 && h0 == 0);
      if (row0 < 0) break;
#pragma unroll
      for (int i = 0; i < kI8RowsInFlight; ++i) {
        if (h0 + i >= H) break;
        const int64_t row = row0 + (int64_t)(h0 + i) * hstride;
        uint32_t ksb, vsb;
        const uint32_t kc = quantize_i8x4(kw[i], &ksb);
        const uint32_t vc = quantize_i8x4(vw[i], &vsb);
        reinterpret_cast<uint32_t*>(a.k_dst)[row * (kHeadDim / 4) + lane] = kc;
        reinterpret_cast<uint32_t*>(a.v_dst)[row * (kHeadDim / 4) + lane] = vc;
        if ((lane & 15) == 0) {
          reinterpret_cast<uint16_t*>(a.k_scale_dst)[row * kI8Groups + (lane >> 4)] =
              (uint16_t)ksb;
          reinterpret_cast<uint16_t*>(a.v_scale_dst)[row * kI8Groups + (lane >> 4)] =
              (uint16_t)vsb;
        }
      }
    }
  }
}

// ---- rope fused with append ------------------------------------------------
//
// One wave per new token.  Work comes in 64-element groups of a head row,
// one group per 16 lanes (lane l owns elements 4 (l % 16) .. +3 of it), so a
// 16-lane DPP row is an INT8 scale group and a 4-lane quad an NVFP4 block.
// The rotary span is group 0; its element i < 32 pairs with i + 32, held by
// lane l ^ 8.  Groups are taken group-major (all heads' group 0 first), so a
// pass of 4 groups is all rotary or all pass-through (with up to 4 heads)
// and the fp64 rotation runs only where it is needed.  Lane l computes the
// cos and sin of pair l % 32 once per token (fp64) and fetches those of its
// pairs 4 (l & 7) .. +3 from their lanes; they serve the token's query heads
// (4 heads at a time, all rotary) and its key heads.  The rotation is the
// rope kernel's, through the same inline functions, so the roped values are
// bit-identical to rope followed by append; keys then take the format's own
// path (copy, NVFP4 or INT8 group-64 quantisation, with the quantisers of the
// plain append) and values are stored or quantised unroped.

// Rotates this lane's 4 elements given its partner's (lane ^ 8) 4 elements.
__device__ __forceinline__ uint2 rotate4(uint2 own, uint2 partner, bool second_half,
                                         const double (&c)[4], const double (&sn)[4]) {
  const uint32_t o[4] = {own.x & 0xffffu, own.x >> 16, own.y & 0xffffu, own.y >> 16};
  const uint32_t p[4] = {partner.x & 0xffffu, partner.x >> 16, partner.y & 0xffffu,
                         partner.y >> 16};
  uint32_t r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const double x = (double)bf16_to_f32((uint16_t)o[j]);
    const double y = (double)bf16_to_f32((uint16_t)p[j]);
    r[j] = second_half ? rope_second(y, x, c[j], sn[j]) : rope_first(x, y, c[j], sn[j]);
  }
  return make_uint2(r[0] | (r[1] << 16), r[2] | (r[3] << 16));
}

// The double held by lane src (byte address 4 src) of the wave.
__device__ __forceinline__ double bpermute_f64(int src, double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * src, (int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * src, (int)(uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ uint2 shfl_xor8(uint2 w) {
  return make_uint2((uint32_t)__shfl_xor((int)w.x, 8), (uint32_t)__shfl_xor((int)w.y, 8));
}

// Largest of x over the 4 lanes of a DPP quad (every lane gets it).
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xb1, 0xf, 0xf, false));
  x = max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4e, 0xf, 0xf, false));
  return x;
}

// Stores this lane's 4 elements (elements 4 c .. 4 c + 3 of a cache row) in
// the layer's format.  The 16 lanes that share a DPP row hold one 64-element
// group, the 4 lanes of a quad one 16-element block.
template <int FMT>
__device__ __forceinline__ void store_row4(const AppendArgs& a, bool is_k, int64_t row, int c,
                                           uint2 w, double S) {
  void* dst = is_k ? a.k_dst : a.v_dst;
  if constexpr (FMT == 0) {
    reinterpret_cast<uint2*>(dst)[row * (kHeadDim / 4) + c] = w;
  } else if constexpr (FMT == 2) {
    uint32_t sb;
    const uint32_t codes = quantize_i8x4(w, &sb);
    reinterpret_cast<uint32_t*>(dst)[row * (kHeadDim / 4) + c] = codes;
    if ((c & 15) == 0)
      reinterpret_cast<uint16_t*>(is_k ? a.k_scale_dst : a.v_scale_dst)[row * kI8Groups +
                                                                        (c >> 4)] =
          (uint16_t)sb;
  } else {
    // a 16-element block is the 4 lanes of a DPP quad
    const uint32_t e[4] = {w.x & 0xffffu, w.x >> 16, w.y & 0xffffu, w.y >> 16};
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, e[i] & 0x7fffu);
    const Fp4Block B = nvfp4_block(quad_max_u32(m), S);
    uint32_t packed = 0;
    if (nvfp4_f32_exact(S)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) packed |= nvfp4_code_f32(e[i], B) << (4 * i);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) packed |= nvfp4_code(e[i], B) << (4 * i);
    }
    reinterpret_cast<uint16_t*>(dst)[row * (kHeadDim / 4) + c] = (uint16_t)packed;
    if ((c & 3) == 0)
      (is_k ? a.k_scale_dst : a.v_scale_dst)[row * kQBlocks + (c >> 2)] = (uint8_t)B.qs;
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void rope_append_kernel(RopeAppendArgs ra) {
  const AppendArgs& a = ra.ap;
  const int H = a.geo.num_kv_heads;
  const int lane = threadIdx.x & 63;
  const bool second = (lane & 8) != 0;
  double kS = 1.0, vS = 1.0;
  if constexpr (FMT == 1) {
    kS = (double)*a.k_tensor_scale;
    vS = (double)*a.v_tensor_scale;
  }
  // W waves share a token (W divides the workgroup's 4 waves): wave share
  // takes every W-th pass of the token's query heads and of its cache items
  const int W = ra.waves_per_token;
  const int wave = threadIdx.x >> 6;
  const int share = wave % W;
  const int64_t wstride = (int64_t)gridDim.x * (blockDim.x >> 6) / W;
  for (int64_t t = ((int64_t)blockIdx.x * (blockDim.x >> 6) + wave) / W; t < a.num_tokens;
       t += wstride) {
    const int32_t pos = a.positions[t];
    double cl, sl;
    rope_cos_sin(pos, ra.inv_freq[lane & 31], ra.mscale, &cl, &sl);
    double c[4], sn[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = bpermute_f64(4 * (lane & 7) + j, cl);
      sn[j] = bpermute_f64(4 * (lane & 7) + j, sl);
    }
    if (ra.q && pos >= 0) {         // a negative position is flagged below, q left as it is
      for (int h0 = 4 * share; h0 < ra.num_q_heads; h0 += 4 * W) {
        const int h = h0 + (lane >> 4);
        const int hl = h < ra.num_q_heads ? h : ra.num_q_heads - 1;   // every lane shuffles
        uint2* p = reinterpret_cast<uint2*>(ra.q + t * ra.q_token_stride +
                                            (int64_t)hl * kHeadDim) + (lane & 15);
        const uint2 w = *p;
        const uint2 r = rotate4(w, shfl_xor8(w), second, c, sn);
        if (h < ra.num_q_heads) *p = r;
      }
    }
    // the token's row for head 0; head h's row follows at a fixed stride
    const int64_t row0 = cache_row(a.geo, a.block_table, a.block_table_len, pos, 0, a.err,
                                   lane == 0 && share == 0);
    if (row0 < 0) continue;
    const int64_t hstride = a.geo.paged ? kBlockSize : 1;
    const int items = H * (kHeadDim / 64);          // (group, head), group-major
    const int sub = lane >> 4, el = lane & 15;      // this lane's item in a pass, element quad
    for (int i0 = 4 * share; i0 < items; i0 += 4 * W) {
      const int it = i0 + sub < items ? i0 + sub : items - 1;   // every lane shuffles
      const int grp = it / H, h = it % H;
      const int e = grp * 16 + el;                  // uint2 index within the row
      const int64_t src = (t * H + h) * (kHeadDim / 4) + e;
      const uint2 kw = reinterpret_cast<const uint2*>(a.k_src)[src];
      const uint2 vw = reinterpret_cast<const uint2*>(a.v_src)[src];
      uint2 kr = kw;
      if (i0 < H) {                                 // the pass holds group-0 (rotary) items
        const uint2 r = rotate4(kw, shfl_xor8(kw), second, c, sn);
        kr = grp == 0 ? r : kw;
      }
      if (i0 + sub < items) {
        const int64_t row = row0 + h * hstride;
        store_row4<FMT>(a, true, row, e, kr, kS);
        store_row4<FMT>(a, false, row, e, vw, vS);
      }
    }
  }
}

// ---- tensor scale ----------------------------------------------------------

__global__ void store_word_kernel(uint32_t* p, uint32_t v) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *p = v;
}

// Largest |x| as bf16 magnitude bits (for finite bf16, |x| orders like the
// low 15 bits); NaN patterns are ignored.
__global__ __launch_bounds__(256) void amax_bits_kernel(const uint16_t* x, int64_t n,
                                                        uint32_t* out) {
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  auto take = [&m](uint32_t bits) {
    const uint32_t a = bits & 0x7fffu;
    if (a <= 0x7f80u) m = max(m, a);
  };
  if (((uintptr_t)x & 15u) == 0) {
    const int64_t n8 = n / 8;
    const uint4* x8 = reinterpret_cast<const uint4*>(x);
    auto take8 = [&](const uint4& w) {
      take(w.x); take(w.x >> 16); take(w.y); take(w.y >> 16);
      take(w.z); take(w.z >> 16); take(w.w); take(w.w >> 16);
    };
    // eight 16-byte loads in flight per thread
    int64_t i = tid;
    for (; i + 7 * stride < n8; i += 8 * stride) {
      uint4 w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = x8[i + u * stride];
#pragma unroll
      for (int u = 0; u < 8; ++u) take8(w[u]);
    }
    for (; i < n8; i += stride) take8(x8[i]);
    for (int64_t j = n8 * 8 + tid; j < n; j += stride) take(x[j]);
  } else {
    for (int64_t i = tid; i < n; i += stride) take(x[i]);
  }
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  // one atomic per workgroup (atomics on one word serialise)
  __shared__ uint32_t wave_max[4];
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
    if (m) atomicMax(out, m);
  }
}

__global__ void finalize_scale_kernel(float* out) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    const uint32_t bits = *reinterpret_cast<uint32_t*>(out);
    const float amax = bf16_to_f32((uint16_t)bits);
    *out = amax == 0.0f ? 1.0f : amax / 2688.0f;
  }
}

unsigned grid_for(int64_t work, int64_t cap) {
  int64_t b = (work + 255) / 256;
  if (b < 1) b = 1;
  return (unsigned)(b > cap ? cap : b);
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  if (a.dtype == 0) {
    const int64_t work = a.num_tokens * a.geo.num_kv_heads * kChunksPerRow;
    return launch(append_bf16_kernel, dim3(grid_for(work, 1 << 20)), dim3(256), 0, s, a);
  }
  if (a.dtype == 2)   // one wave per token
    return launch(append_int8_kernel, dim3(grid_for(a.num_tokens * 64, 1 << 18)), dim3(256), 0,
                  s, a);
  // one wave per token
  return launch(append_nvfp4_kernel, dim3(grid_for(a.num_tokens * 64, 1 << 18)), dim3(256), 0, s,
                a);
}

hipError_t launch_rope_append(const RopeAppendArgs& a, hipStream_t s) {
  if (a.ap.num_tokens == 0) return hipSuccess;
  // One wave per token; a launch of few tokens (a decode step appends one per
  // sequence) gives each token a workgroup of 4 waves instead, each taking a
  // quarter of its passes, so that their load-rotate-store chains overlap:
  // one token with 24 query and 4 KV heads went from 6 query and 4 cache
  // passes in one wave to at most 2 and 1 per wave.
  RopeAppendArgs k = a;
  k.waves_per_token = a.ap.num_tokens <= 512 ? 4 : 1;
  const dim3 grid(grid_for(a.ap.num_tokens * 64 * k.waves_per_token, 1 << 18));
  if (a.ap.dtype == 0) return launch(rope_append_kernel<0>, grid, dim3(256), 0, s, k);
  if (a.ap.dtype == 2) return launch(rope_append_kernel<2>, grid, dim3(256), 0, s, k);
  return launch(rope_append_kernel<1>, grid, dim3(256), 0, s, k);
}

hipError_t launch_tensor_scale(const uint16_t* x, int64_t n, float* out, hipStream_t s) {
  uint32_t* word = reinterpret_cast<uint32_t*>(out);
  hipError_t e = launch(store_word_kernel, dim3(1), dim3(64), 0, s, word, 0u);
  if (e == hipSuccess && n > 0)
    // up to 16,384 workgroups with eight loads in flight per lane: over one
    // 1M-token layer's K (2 GiB) 5.7 TB/s, against 5.1 with 2,048 and four
    // (32,768 workgroups were slower, 4.5 TB/s: one atomic each on one word)
    e = launch(amax_bits_kernel, dim3(grid_for(n / 8 + 1, 16384)), dim3(256), 0, s, x, n, word);
  if (e == hipSuccess) e = launch(finalize_scale_kernel, dim3(1), dim3(64), 0, s, out);
  return e;
}

}  // namespace yrk
