// Device pieces shared by the split-K attention kernels over the KV cache
// (single-query decode and multi-query verify): workgroup shape, page lookup,
// MFMA operand types, the cross-row maximum of an MFMA accumulator and the
// swizzled V staging layout with its transposing read.
#pragma once

#include "device_common.h"
#include "yrk_internal.h"

namespace yrk {
namespace {

constexpr int kWaves = kAttnWaves;
constexpr int kThreads = 64 * kWaves;
constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima
constexpr int kRowBytesF16 = kHeadDim * 2;   // one staged 16-bit V row

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));   // (HIP's uint4 copies as a struct)
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t err_flag(uint32_t* err, uint32_t bit) {
  set_error(err, bit);
  return bit;
}

// Logical page -> element offset of its first row for KV head g, and the
// element stride between consecutive token rows of the page.  Returns false
// (page masked) for a table entry outside the pool.
__device__ __forceinline__ bool page_base(const DecodeArgs& a, int s, int g, int64_t page,
                                          int64_t row_elems, int64_t* base, int64_t* tstride) {
  if (a.geo.paged) {
    // one table entry for the whole wave, read through the constant address
    // space so that it is a scalar load: a vector load here would be waited
    // for with the vector-load counter, which retires in order, so every K/V
    // load still in flight (the pages prefetched for later steps) would be
    // waited for too.  The table is not written while a kernel runs.
    typedef const __attribute__((address_space(4))) int32_t const_i32;
    const const_i32* table = (const const_i32*)(const void*)a.block_tables;
    const int64_t blk = __builtin_amdgcn_readfirstlane(
        table[(int64_t)s * a.block_table_stride + page]);
    if (blk < 0 || blk >= a.geo.num_blocks) return false;
    *base = ((blk * a.geo.num_kv_heads + g) * kBlockSize) * row_elems;
    *tstride = row_elems;
  } else {
    *base = (page * kBlockSize * a.geo.num_kv_heads + g) * row_elems;
    *tstride = (int64_t)a.geo.num_kv_heads * row_elems;
  }
  return true;
}

// Maximum over lanes l, l^16, l^32, l^48 (the four row groups of an MFMA
// accumulator) with the gfx950 cross-row lane swaps.
__device__ __forceinline__ float max_over_row_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Staged V row t keeps 16-byte chunk c at position c ^ vswz(t).  vswz is a
// permutation of 0..7 on rows 0..7 and on rows 8..15 (so the 8 lanes of a
// 128-byte write phase, rows t..t+7 with one chunk index, hit distinct banks)
// and gives rows 4r..4r+3 distinct bits 1-2 (so the transposing reads, 4 rows
// x 32 bytes per 16 lanes, fall into 4 distinct 32-byte bank groups).
__device__ __forceinline__ int vswz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

// The V^T operand of a 16-token staged page (16 rows of kRowBytesF16 bytes,
// swizzled as above) for head dims 16 i .. 16 i + 15: ds_read_b64_tr_b16
// gives lane (lo, hi) dim 16 i + lo at tokens 4 hi .. 4 hi + 3.
__device__ __forceinline__ uint2 vt_operand(const uint8_t* page_stage, int i, int lo, int hi) {
  const int trow = 4 * hi + (lo >> 2);
  const int chunk = 2 * i + ((lo & 3) >> 1);
  const int off = trow * kRowBytesF16 + ((chunk ^ vswz(trow)) * 16) + 8 * (lo & 1);
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_short4_t*)(void*)(page_stage + off));
  return __builtin_bit_cast(uint2, v);
}

// ---- fp16 matrix-core pieces of the quantised-cache kernels ----------------

typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

// The running maximum m is raised only when a step's maximum exceeds it by
// more than kRescaleF4, so s - m <= kRescaleF4 and p = 2^(s - m + kPShiftF4)
// <= 2^15 fits fp16.  The shift keeps probabilities down to 2^-28 of m at
// full fp16 precision (2^-38 as subnormals); it cancels in O / l and is taken
// off the log-sum-exp.  (A threshold of 6 with a shift of 9 ran at the same
// speed and lost 13x in accuracy on the 1M-token outlier workload.)
constexpr float kRescaleF4 = 1.0f;
constexpr float kPShiftF4 = 14.0f;

__device__ __forceinline__ floatx4_t mfma_f16(const uint4& a, const uint4& b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ floatx4_t mfma_f16_k16(const uint2& a, const uint2& b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                               __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
}

// Two floats -> packed fp16, rounded to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pk_f16(float lo, float hi) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){lo, hi}, f16x2_t));
}

// Eight int8 codes (two dwords, element i in byte i) -> eight fp16 integers:
// a byte c becomes fp16 1152 + c exactly (0x64 placed above c ^ 0x80 by a
// byte permute), and one packed subtraction gives c.  This is the published
// exponent-bias conversion (an integer written into the mantissa of a float
// whose exponent makes one mantissa unit equal 1, then the bias subtracted),
// used for int8 weights by Kim et al., "Who Says Elephants Can't Run:
// Bringing Large Scale MoE Models into Cloud Scale Production", 2022; the
// unsigned offset 0x80 keeps the whole int8 range on one exponent (1024 +
// 128 + c).
__device__ __forceinline__ uint4 i8x8_to_f16(uint32_t w0, uint32_t w1) {
  const f16x2_t off = {(_Float16)1152.0f, (_Float16)1152.0f};
  const uint32_t t0 = w0 ^ 0x80808080u, t1 = w1 ^ 0x80808080u;
  auto two = [&](uint32_t t, uint32_t sel) {
    const f16x2_t h = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(0x64646464u, t, sel));
    return __builtin_bit_cast(uint32_t, h - off);
  };
  return make_uint4(two(t0, 0x04010400u), two(t0, 0x04030402u), two(t1, 0x04010400u),
                    two(t1, 0x04030402u));
}

// The largest binary16 V group scale among the 4 token rows of u (two
// scale dwords per row, 4 groups), maxed over the wave's row groups: the
// extra log2 units a page counts as in the running maximum so that p times
// any of its scales stays below 2^15 (s < 2^(b - 14) for exponent field b).
__device__ __forceinline__ float vscale_shift(const u32x2_t (&rows)[4]) {
  uint32_t sb = 0;   // non-negative binary16 bits order like their values
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t w0 = rows[e].x, w1 = rows[e].y;
    sb = max(sb, max(max(w0 & 0xffffu, w0 >> 16), max(w1 & 0xffffu, w1 >> 16)));
  }
  sb = (uint32_t)max_over_row_groups((float)sb);
  return (float)max(0, (int)((sb >> 10) & 31u) - 14);
}

// Orders one wave's LDS writes before its later reads of the same buffer
// (the staging buffers are private to a wave).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Issue priority to the waves of a workgroup that are behind.  Two waves
// share each SIMD, and with equal priority the older one is served first:
// given equal shares, it finished its share well before the other, and the
// SIMD then ran the rest with one wave.  After each step a wave publishes in
// LDS how many steps it has done and takes priority 2 while no wave of the
// workgroup has done fewer, else priority 0.  The steps each wave computes
// are fixed, so only the speed depends on this (a stale count read here only
// delays a change of priority).  progress: NW words, 16-byte aligned.
template <int NW>
__device__ __forceinline__ void balance_issue(uint32_t* progress, uint32_t done, int wave,
                                              int lane) {
  static_assert(NW % 4 == 0, "progress words are read four at a time");
  if (lane == 0) reinterpret_cast<volatile uint32_t*>(progress)[wave] = done;
  uint32_t mn = done;
#pragma unroll
  for (int w = 0; w < NW; w += 4) {
    const u32x4_t p = *reinterpret_cast<volatile u32x4_t*>(progress + w);
    mn = min(min(mn, min(p[0], p[1])), min(p[2], p[3]));
  }
  if (done > mn)
    __builtin_amdgcn_s_setprio(0);
  else
    __builtin_amdgcn_s_setprio(2);
}

}  // namespace
}  // namespace yrk
