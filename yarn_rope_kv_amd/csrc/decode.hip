// Split-K decode attention over a paged bf16, NVFP4 or INT8 group-64 KV cache
// (gfx950).
//
// One query per sequence, GQA: the G query heads of one KV head share every
// key and value they read ([P5] "Why NVFP4 KV changes the math": 4 KV heads x
// 256; 24 query heads).  Decode time is dominated by streaming the cache
// ([P1] "Two cards are faster than one, not just bigger": each card reading
// half the KV is what made TP2 faster), so the kernels are organised around
// HBM streaming:
//
//   split phase   grid (split, kv_head, seq), 4 waves per workgroup.  A
//                 split owns a contiguous range of pages; wave w of the
//                 workgroup takes pages w, w+4, ...  Both products run on
//                 the matrix cores with the G heads padded to a 16-column
//                 block, the loads of the wave's next pages in flight while
//                 one is computed.  Each wave keeps its own online softmax;
//                 the waves are combined at the end of the split and one
//                 partial (normalised output + log2-sum-exp) per query head
//                 goes to the workspace.
//   merge phase   grid (q_head, seq): log-sum-exp combination of the splits
//                 ([P3] "Limitations": the decode split policy).
//
// A bf16 cache is served by the multi-query kernels of the verify step run
// with one query (same partials, same merge).  This file holds the kernels of
// the quantised caches, NVFP4 pages ([P5] "Why NVFP4 KV changes the math":
// packed e2m1 codes, an e4m3 scale per 16 elements and a per-tensor fp32
// scale) and INT8 group-64 pages, whose codes are turned into fp16 in
// registers, exactly, with fp32 accumulation; the tensor scales are folded
// into the softmax scale and the output.
#include "attn_common.h"

namespace yrk {
namespace {

// ---- NVFP4 on the matrix cores ----------------------------------------------
//
// With 6 query heads per KV head, the scores of a page are a 16 x 16 product
// (16 tokens x 6 heads padded to 16) over the 256 head dims, and the output a
// 256 x 16 product over the page's tokens: the kernel runs both on
// v_mfma_f32_16x16x32_f16 and keeps only the dequantisation and the softmax
// on the vector ALUs.  A wave takes 32 tokens (two pages) per step.
//
//   dequant   the fp4 conversion with unit scale gives e2m1 in fp16 (the
//             scaled form multiplies by a power of two only: it takes the
//             exponent of its fp32 scale), and a packed fp16 multiply applies
//             the block scale q_s (e4m3, exact in fp16).  e2m1 x q_s has at
//             most 6 significant bits and lies in [2^-10, 2688]: exact.
//   S^T       = K Q^T.  Lane (t, kg) = (lane % 16, lane / 16) reads code bytes
//             [32kg, 32kg+32) of token row t (head dims [64kg, 64kg+64), scale
//             blocks 4kg..4kg+3: one scale dword) and supplies dims
//             64kg + 8j .. +7 at MFMA step j; the Q^T operand holds the same
//             dims of head t (zero for heads >= G), prescaled by a power of
//             two so that |q| < 2^15 fits fp16 (bf16 values are then exact).
//   softmax   lane (h, r) holds the scores of head h at tokens 4r..4r+3 of
//             both pages: the accumulator layout is the P^T operand of the
//             output product as it stands.  Online, log2 domain; the running
//             maximum m is raised (and O rescaled) only when a step exceeds
//             it by more than 1.  p = 2^(s - m + 14) <= 2^15 is rounded to
//             fp16 (nearest even); the row sums are a product of those same
//             values with ones.
//   O^T      += V^T P^T.  V is dequantised to fp16 into a per-wave LDS buffer
//             (token rows, 16-byte chunks swizzled); ds_read_b64_tr_b16 turns
//             4 rows x 4 dims per 16 lanes into the V^T operand: lane j of
//             lane group r gets dim 16i + j at tokens 4r..4r+3.
//   loads     the codes and scales of the wave's next 32 tokens are in flight
//             while the current ones are computed.

constexpr int kUnitPages = 2;                            // pages per wave step
// One NVFP4 workgroup per CU, 8 waves (2 per SIMD) whose issue priority
// favours the waves that are behind (balance_issue).  Two 4-wave workgroups
// on a CU ran at very different speeds: the first placed on each CU finished
// its equal share ~12% earlier, and the CU spent the rest of the split at
// half occupancy.  Measured per 1M-token layer: 230 us as two 4-wave
// workgroups per CU, 224 us as one 8-wave workgroup, 221 us with the
// priority balance (a counter handing steps to whichever wave asked first
// reached 218 us, but the sums then depend on the timing: no longer
// byte-reproducible).
constexpr int kWavesF4 = 8;
constexpr int kThreadsF4 = 64 * kWavesF4;
constexpr int kStageBytes = kWavesF4 * kUnitPages * kBlockSize * kRowBytesF16;   // 128 KiB
constexpr int kAheadF4 = 1;                              // wave steps in flight beyond the one computed
constexpr int kVtAhead = 4;                              // V^T operands in flight ahead of their products

// Block scales (e4m3 bytes 2 H and 2 H + 1 of w) as an fp16 pair, one packed
// conversion.  The hardware fp8 conversion decodes OCP E4M3FN exactly, and
// every e4m3 value (0 and 2^-9 .. 448) is an fp16 value.  (Two scales per
// instruction: one per block, converted to fp32 and repacked, took two
// instructions per block, 48 more per kernel and ~1 us more per 1M-token
// layer.)
template <bool H>
__device__ __forceinline__ uint32_t block_scale_pair(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, H));
}

// Eight e2m1 codes (one dword; element 2j in the low nibble of byte j) ->
// eight fp16 values code x q_s, exactly, q_s being half `which` of a scale
// pair (the packed multiply selects that half for both lanes of the pair):
// the unit-scale fp4 conversion gives the e2m1 value (the scaled form
// multiplies by a power of two only, so the block scale is applied
// separately), and e2m1 x q_s has at most 6 significant bits in
// [2^-10, 2688], which fp16 holds.
__device__ __forceinline__ uint4 fp4x8_to_f16(uint32_t w, uint32_t pair, int which) {
  const f16x2_t p2 = __builtin_bit_cast(f16x2_t, pair);
  const f16x2_t m = which ? __builtin_shufflevector(p2, p2, 1, 1) : __builtin_shufflevector(p2, p2, 0, 0);
  const f16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * m;
  const f16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * m;
  const f16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * m;
  const f16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * m;
  return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                    __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
}

// One lane's share of the two pages of a wave step.
struct F4Unit {
  u32x4_t kc[kUnitPages][2], vc[kUnitPages][2]; // code bytes [32kg, 32kg+32) of row t
  uint32_t ks[kUnitPages], vs[kUnitPages];      // scale bytes 4kg..4kg+3 of row t
  bool ok[kUnitPages];                          // page present and inside the split
};

// Q^T operand of the score product for lane (lo, hi): head lo of the group
// (zero for heads >= G), 8 dims per MFMA step (dims 64 hi .. 64 hi + 63, or
// the per-group order of the INT8 kernel), in fp16
// after a power-of-two prescale that puts the largest |q| of the group in
// [2^14, 2^15) (bf16 values are then exact in fp16).  Returns the factor that
// undoes the prescale.
template <int G>
__device__ __forceinline__ float load_q_f16(const DecodeArgs& a, int s, int g, int lo, int hi,
                                            uint4 (&qop)[8], bool grouped = false) {
  uint4 qraw[8];
  float qmax = 0.f;
  const uint16_t* qrow = a.q + ((int64_t)s * a.num_q_heads + (int64_t)g * G + lo) * kHeadDim;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    // step j: dims 64 hi + 8 j .. +7, or (grouped) 64 (j / 2) + 32 (j % 2) + 8 hi .. +7
    const int d0 = grouped ? 64 * (j >> 1) + 32 * (j & 1) + 8 * hi : 64 * hi + 8 * j;
    qraw[j] = lo < G ? *reinterpret_cast<const uint4*>(qrow + d0) : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {qraw[j].x, qraw[j].y, qraw[j].z, qraw[j].w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      qmax = fmaxf(qmax, fmaxf(fabsf(bf16_lo(w[e])), fabsf(bf16_hi(w[e]))));
  }
  qmax = max_over_row_groups(qmax);
#pragma unroll
  for (int sh = 1; sh < 16; sh <<= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, sh));
  // 2^(14 - e): the largest |q| lands in [2^14, 2^15)
  const int qe = (int)((__float_as_uint(qmax) >> 23) & 0xFF);
  const int pe = qmax > 0.f ? min(max(268 - qe, 1), 254) : 127;
  const float qpre = __uint_as_float((uint32_t)pe << 23);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t w[4] = {qraw[j].x, qraw[j].y, qraw[j].z, qraw[j].w};
    uint32_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = pk_f16(bf16_lo(w[e]) * qpre, bf16_hi(w[e]) * qpre);
    qop[j] = make_uint4(h[0], h[1], h[2], h[3]);
  }
  return __uint_as_float((uint32_t)(254 - pe) << 23);
}

// End of a split of the matrix-core kernels: combine the 4 waves through LDS
// (the staging buffer, once every wave is done with it) and write one
// normalised partial + log2-sum-exp per query head.  Lane (lo, hi) holds
// O^T rows 16 i + 4 hi .. +3 of head lo; l and O carry a factor
// 2^kPShiftF4; vS multiplies every value (1 for a cache without one).
template <int G, int NW = kWaves>
__device__ __forceinline__ void finish_split_mfma(const DecodeArgs& a, int s, int g, int split,
                                                  uint8_t* stage, const floatx4_t (&o)[16],
                                                  const floatx4_t& lsum, float m, float vS,
                                                  int wave, int lo, int hi) {
  __syncthreads();
  float* sm_o = reinterpret_cast<float*>(stage);   // [NW][G][256]
  float* sm_m = sm_o + NW * G * kHeadDim;          // [NW][G]
  float* sm_l = sm_m + NW * G;                     // [NW][G]
  if (lo < G) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      *reinterpret_cast<floatx4_t*>(sm_o + (wave * G + lo) * kHeadDim + 16 * i + 4 * hi) = o[i] * vS;
    if (hi == 0) {
      sm_m[wave * G + lo] = m - kPShiftF4;
      sm_l[wave * G + lo] = lsum[0];
    }
  }
  __syncthreads();
  const int nsp = a.plan.num_splits;
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += 64 * NW) {
    const int h = idx / kHeadDim;
    const int d = idx % kHeadDim;
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w * G + h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sc = fast_exp2(sm_m[w * G + h] - M);
      L += sm_l[w * G + h] * sc;
      O += sm_o[(w * G + h) * kHeadDim + d] * sc;
    }
    const int qh = g * G + h;
    const int64_t slot = ((int64_t)s * a.num_q_heads + qh) * nsp + split;
    a.ws_o[slot * kHeadDim + d] = L > 0.f ? O / L : 0.f;
    if (d == 0) a.ws_lse[slot] = L > 0.f ? M + __log2f(L) : -INFINITY;
  }
}

template <int G>
__global__ __launch_bounds__(kThreadsF4, 1) void decode_split_nvfp4(DecodeArgs a) {
  static_assert(G >= 1 && G <= 16, "heads of a group fill at most one MFMA column block");
  static_assert((kWavesF4 * G * kHeadDim + 2 * kWavesF4 * G) * 4 <= kStageBytes,
                "split combine reuses the staging buffer");
  __shared__ __attribute__((aligned(16))) uint8_t stage[kStageBytes];
  __shared__ __attribute__((aligned(16))) uint32_t progress[kWavesF4];   // steps done per wave
  const int split = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int lo = lane & 15, hi = lane >> 4;

  int64_t len = a.seq_lens[s];
  if (len > a.max_seq_len) {
    if (threadIdx.x == 0 && split == 0 && g == 0) err_flag(a.err, kErrPosition);
    len = a.max_seq_len;
  }
  if (len < 0) len = 0;
  const int64_t tok0 = (int64_t)split * a.plan.tokens_per_split;
  const int64_t tok1 = min(len, tok0 + a.plan.tokens_per_split);
  if (threadIdx.x < kWavesF4) progress[threadIdx.x] = 0;
  __syncthreads();

  floatx4_t o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  floatx4_t lsum = {0.f, 0.f, 0.f, 0.f};
  float m = kNegBig;
  float vS = 1.0f;

  if (tok1 > tok0) {
    const float kS = *a.k_tensor_scale;
    vS = *a.v_tensor_scale;
    uint4 qop[8];
    float c = 0.f;   // set once the first step's loads are in flight (below)

    const uint8_t* Kc = static_cast<const uint8_t*>(a.k);
    const uint8_t* Vc = static_cast<const uint8_t*>(a.v);
    const int64_t page0 = tok0 / kBlockSize;
    const int64_t npages = (tok1 - tok0 + kBlockSize - 1) / kBlockSize;
    const int64_t nunits = (npages + kUnitPages - 1) / kUnitPages;
    uint8_t* my_stage = stage + wave * (kUnitPages * kBlockSize * kRowBytesF16);

    auto load_unit = [&](int64_t u, F4Unit& U) {
#pragma unroll
      for (int p = 0; p < kUnitPages; ++p) {
        const int64_t pi = kUnitPages * u + p;
        int64_t base = 0, ts = 0;
        bool ok = false;
        if (pi < npages) {
          ok = page_base(a, s, g, page0 + pi, kHeadDim / 16, &base, &ts);
          if (!ok && lane == 0) err_flag(a.err, kErrBlockId);
        }
        U.ok[p] = ok;
        const u32x4_t z = {0u, 0u, 0u, 0u};
        u32x4_t k0 = z, k1 = z, v0 = z, v1 = z;
        uint32_t ksc = 0, vsc = 0;
        if (ok) {
          const int64_t rowblk = base + lo * ts;   // row t's first 16-element block
          const uint8_t* kp = Kc + rowblk * 8 + 32 * hi;
          const uint8_t* vp = Vc + rowblk * 8 + 32 * hi;
          k0 = *reinterpret_cast<const u32x4_t*>(kp);
          k1 = *reinterpret_cast<const u32x4_t*>(kp + 16);
          v0 = *reinterpret_cast<const u32x4_t*>(vp);
          v1 = *reinterpret_cast<const u32x4_t*>(vp + 16);
          ksc = *reinterpret_cast<const uint32_t*>(a.k_scale + rowblk + 4 * hi);
          vsc = *reinterpret_cast<const uint32_t*>(a.v_scale + rowblk + 4 * hi);
        }
        U.kc[p][0] = k0;
        U.kc[p][1] = k1;
        U.vc[p][0] = v0;
        U.vc[p][1] = v1;
        U.ks[p] = ksc;
        U.vs[p] = vsc;
      }
    };

    const uint4 ones = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
    auto compute_unit = [&](int64_t u, F4Unit& U) {
      const int64_t ut0 = (page0 + kUnitPages * u) * kBlockSize;   // first token of the step
      // the same for every lane: both pages present and inside the split
      bool full = ut0 + kUnitPages * kBlockSize <= tok1;
#pragma unroll
      for (int p = 0; p < kUnitPages; ++p) full = full && U.ok[p];
      // tokens of the step that are attended: [0, nvalid) per page, or none
      int nv[kUnitPages];
#pragma unroll
      for (int p = 0; p < kUnitPages; ++p)
        nv[p] = U.ok[p] ? (int)max((int64_t)0, min((int64_t)kBlockSize, tok1 - ut0 - p * kBlockSize)) : 0;
      if (!full) {
        // V rows outside the split or the sequence, or of a masked page, get
        // weight 0; stale bytes there may decode to NaN (0 * NaN is not 0),
        // so they are staged as zeros
#pragma unroll
        for (int p = 0; p < kUnitPages; ++p) {
          const bool keep = lo < nv[p];
          U.vc[p][0] = keep ? U.vc[p][0] : u32x4_t{0u, 0u, 0u, 0u};
          U.vc[p][1] = keep ? U.vc[p][1] : u32x4_t{0u, 0u, 0u, 0u};
          U.vs[p] = keep ? U.vs[p] : 0u;
        }
      }
      // stage V as fp16: row lo, logical chunks 8 hi .. 8 hi + 7
#pragma unroll
      for (int p = 0; p < kUnitPages; ++p) {
        const uint32_t bs[2] = {block_scale_pair<false>(U.vs[p]), block_scale_pair<true>(U.vs[p])};
        const uint32_t w[8] = {U.vc[p][0][0], U.vc[p][0][1], U.vc[p][0][2], U.vc[p][0][3],
                               U.vc[p][1][0], U.vc[p][1][1], U.vc[p][1][2], U.vc[p][1][3]};
        uint8_t* row = my_stage + (p * kBlockSize + lo) * kRowBytesF16;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<uint4*>(row + ((8 * hi + j) ^ vswz(lo)) * 16) =
              fp4x8_to_f16(w[j], bs[j >> 2], (j >> 1) & 1);
      }
      // S^T = K Q^T, one accumulator chain per page
      floatx4_t sacc[kUnitPages];
#pragma unroll
      for (int p = 0; p < kUnitPages; ++p) sacc[p] = floatx4_t{0.f, 0.f, 0.f, 0.f};
      uint32_t kb[kUnitPages][2];
#pragma unroll
      for (int p = 0; p < kUnitPages; ++p) {
        kb[p][0] = block_scale_pair<false>(U.ks[p]);
        kb[p][1] = block_scale_pair<true>(U.ks[p]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int p = 0; p < kUnitPages; ++p) {
          const uint32_t w = U.kc[p][j >> 2][j & 3];
          sacc[p] = mfma_f16(fp4x8_to_f16(w, kb[p][j >> 2], (j >> 1) & 1), qop[j], sacc[p]);
        }
      // online softmax over the unit's 32 tokens (lane: head lo, tokens 4hi..4hi+3 of each page)
      float x[kUnitPages][4];
      float mx = -INFINITY;
#pragma unroll
      for (int p = 0; p < kUnitPages; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = sacc[p][e] * c;
          x[p][e] = full || 4 * hi + e < nv[p] ? v : -INFINITY;
          mx = fmaxf(mx, x[p][e]);
        }
      mx = max_over_row_groups(mx);
      // the running maximum is raised (and O rescaled) only when a step
      // exceeds it by more than kRescaleF4
      const bool grow = mx > m + kRescaleF4;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float mn = grow ? mx : m;
        const float alpha = fast_exp2(m - mn);
        m = mn;
#pragma unroll
        for (int i = 0; i < 16; ++i) o[i] *= alpha;
        lsum *= alpha;
      }
      const float mp = m - kPShiftF4;
      uint4 pop;
      pop.x = pk_f16(fast_exp2(x[0][0] - mp), fast_exp2(x[0][1] - mp));
      pop.y = pk_f16(fast_exp2(x[0][2] - mp), fast_exp2(x[0][3] - mp));
      pop.z = pk_f16(fast_exp2(x[1][0] - mp), fast_exp2(x[1][1] - mp));
      pop.w = pk_f16(fast_exp2(x[1][2] - mp), fast_exp2(x[1][3] - mp));
      lsum = mfma_f16(ones, pop, lsum);
      // O^T += V^T P^T: k order = tokens 4hi..4hi+3 of page 0, then of page 1
      wave_lds_sync();
      auto read_vt = [&](int i) {
        const uint2 w0 = vt_operand(my_stage, i, lo, hi);
        const uint2 w1 = vt_operand(my_stage + kBlockSize * kRowBytesF16, i, lo, hi);
        return make_uint4(w0.x, w0.y, w1.x, w1.y);
      };
      // V^T operands read kVtAhead products ahead, so that LDS latency overlaps
      // the products (the compiler would otherwise read each just before use)
      uint4 vt[kVtAhead];
#pragma unroll
      for (int i = 0; i < kVtAhead; ++i) vt[i] = read_vt(i);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        o[i] = mfma_f16(vt[i % kVtAhead], pop, o[i]);
        if (i + kVtAhead < 16) vt[i % kVtAhead] = read_vt(i + kVtAhead);
        __builtin_amdgcn_sched_barrier(0);
      }
      wave_lds_sync();
    };

    // wave w takes steps w, w + kWavesF4, ...; the next one is loaded while
    // one is computed
    F4Unit R[kAheadF4 + 1];
    uint32_t done = 0;
#pragma unroll
    for (int k = 0; k < kAheadF4; ++k) load_unit(wave + k * kWavesF4, R[k]);
    // scores in log2 units: q.k * softmax scale * log2(e), with the K tensor
    // scale and the q prescale (a power of two) folded in; the query is read
    // while the first step's loads are in flight
    c = a.scale_log2 * kS * load_q_f16<G>(a, s, g, lo, hi, qop);
    for (int64_t u = wave; u < nunits; u += (kAheadF4 + 1) * kWavesF4) {
#pragma unroll
      for (int b = 0; b <= kAheadF4; ++b) {
        const int64_t uu = u + b * kWavesF4;
        load_unit(uu + kAheadF4 * kWavesF4, R[(b + kAheadF4) % (kAheadF4 + 1)]);
        if (uu < nunits) compute_unit(uu, R[b]);
        balance_issue<kWavesF4>(progress, ++done, wave, lane);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }

  finish_split_mfma<G, kWavesF4>(a, s, g, split, stage, o, lsum, m, vS, wave, lo, hi);
}

// ---- INT8 group-64 on the matrix cores ------------------------------------------
//
// The NVFP4 kernel's structure with 16-token steps (the codes take twice the
// registers per token) and v_mfma_f32_16x16x16_f16 for the output product.
// Everything stays exact up to the fp32 accumulation: the codes go to the
// matrix cores as fp16 integers, and the group scales are applied on the
// other side of each product.
//   codes     a byte c turns into fp16 1152 + c exactly (0x64 placed above
//             c ^ 0x80 by a byte permute) and one packed subtraction gives c.
//   S^T       = sum over the 4 scale groups g of s_tg * (K_g Q_g^T): each
//             MFMA step covers 32 dims of one group (lane group kg supplies
//             dims 64g + 32j + 8kg .. +7), so a group's two steps accumulate
//             T_g alone and the scales multiply T_g in fp32 (lane (h, r)
//             holds tokens 4r..4r+3, whose scale rows it reads).
//   O^T      += V^T (P o s_g)^T: V is staged as exact fp16 codes; 16 output
//             dims lie in one group, and the P^T operand of those products is
//             P times the token's group scale, rounded to fp16 like P.  A page
//             whose largest V scale is at least 1 counts as higher in the
//             running maximum by one more than that scale's binary exponent,
//             so every p * s stays below 2^15 (fp16 ends at 65504).  The row
//             sums use P itself.  K = 16 tokens: the S^T accumulator is the
//             P^T operand, one transposing LDS read per 16 dims is V^T.


// Two 4-wave workgroups per CU: one 8-wave workgroup with the priority
// balance of the NVFP4 kernel measured 1% slower here (405.7 against
// 401.8 us per 1M-token layer).
constexpr int kWavesI8 = 4;
constexpr int kThreadsI8 = 64 * kWavesI8;
constexpr int kStageBytesI8 = kWavesI8 * kBlockSize * kRowBytesF16;   // 32 KiB
// Steps in flight beyond the one computed.  The kernel waits on memory far
// more than it computes (a page is ~380 vector instructions and 25 MFMAs),
// so the registers go to a deeper ring: the Q^T operands live in LDS (read
// at every step) instead of 32 registers, and each lane loads only its own
// row's group scales and fetches the 4 rows it needs from their lanes
// (ds_bpermute) when it computes, 4 registers per step instead of 16.
// Measured per 1M-token layer: 0.443 ms with one step ahead, 0.407 ms with
// two (about 240 registers, no spills).
constexpr int kAheadI8 = 2;
constexpr int kQOpBytesI8 = 8 * 64 * 16;                            // Q^T operands in LDS

// One lane's share of one page.
struct I8Unit {
  u32x2_t kc[8];            // K: step j's 8 code bytes of row t (dims of group j / 2)
  u32x4_t vc[4];            // V: code bytes [64 kg, 64 kg + 64) of row t
  u32x2_t ks, vs;           // row t's four binary16 group scales
  bool ok;                  // page present and inside the split
};

template <int G>
__global__ __launch_bounds__(kThreadsI8, 2) void decode_split_int8(DecodeArgs a) {
  static_assert(G >= 1 && G <= 16, "heads of a group fill at most one MFMA column block");
  static_assert((kWavesI8 * G * kHeadDim + 2 * kWavesI8 * G) * 4 <= kStageBytesI8 + kQOpBytesI8,
                "split combine reuses the staging buffer");
  __shared__ __attribute__((aligned(16))) uint8_t stage[kStageBytesI8 + kQOpBytesI8];
  const int split = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int lo = lane & 15, hi = lane >> 4;

  int64_t len = a.seq_lens[s];
  if (len > a.max_seq_len) {
    if (threadIdx.x == 0 && split == 0 && g == 0) err_flag(a.err, kErrPosition);
    len = a.max_seq_len;
  }
  if (len < 0) len = 0;
  const int64_t tok0 = (int64_t)split * a.plan.tokens_per_split;
  const int64_t tok1 = min(len, tok0 + a.plan.tokens_per_split);

  floatx4_t o[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  floatx4_t lsum = {0.f, 0.f, 0.f, 0.f};
  float m = kNegBig;

  if (tok1 > tok0) {
    uint4 qop[8];   // step j = 2 g + j2: dims 64 g + 32 j2 + 8 hi .. +7 of head lo
    const float c = a.scale_log2 * load_q_f16<G>(a, s, g, lo, hi, qop, true);
    uint4* qlds = reinterpret_cast<uint4*>(stage + kStageBytesI8);   // [step][lane]
    if (wave == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) qlds[j * 64 + lane] = qop[j];
    }
    __syncthreads();   // tok1 > tok0 is the same for the whole workgroup

    const uint8_t* Kc = static_cast<const uint8_t*>(a.k);
    const uint8_t* Vc = static_cast<const uint8_t*>(a.v);
    const uint16_t* Ks = reinterpret_cast<const uint16_t*>(a.k_scale);
    const uint16_t* Vs = reinterpret_cast<const uint16_t*>(a.v_scale);
    const int64_t page0 = tok0 / kBlockSize;
    const int64_t npages = (tok1 - tok0 + kBlockSize - 1) / kBlockSize;
    uint8_t* my_stage = stage + wave * (kBlockSize * kRowBytesF16);

    auto load_unit = [&](int64_t pi, I8Unit& U) {
      int64_t base = 0, ts = 0;   // in rows
      bool ok = false;
      if (pi < npages) {
        ok = page_base(a, s, g, page0 + pi, 1, &base, &ts);
        if (!ok && lane == 0) err_flag(a.err, kErrBlockId);
      }
      U.ok = ok;
      const u32x2_t z2 = {0u, 0u};
      const u32x4_t z4 = {0u, 0u, 0u, 0u};
      u32x2_t kc[8], ks = z2, vs = z2;
      u32x4_t vc[4];
#pragma unroll
      for (int j = 0; j < 8; ++j) kc[j] = z2;
#pragma unroll
      for (int i = 0; i < 4; ++i) vc[i] = z4;
      if (ok) {
        const int64_t row = base + lo * ts;
        const uint8_t* kp = Kc + row * kHeadDim + 8 * hi;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          kc[j] = *reinterpret_cast<const u32x2_t*>(kp + 64 * (j >> 1) + 32 * (j & 1));
        const u32x4_t* vp = reinterpret_cast<const u32x4_t*>(Vc + row * kHeadDim + 64 * hi);
#pragma unroll
        for (int i = 0; i < 4; ++i) vc[i] = vp[i];
        ks = *reinterpret_cast<const u32x2_t*>(Ks + row * (kHeadDim / 64));
        vs = *reinterpret_cast<const u32x2_t*>(Vs + row * (kHeadDim / 64));
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) U.kc[j] = kc[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) U.vc[i] = vc[i];
      U.ks = ks;
      U.vs = vs;
    };

    const uint2 ones = make_uint2(0x3C003C00u, 0x3C003C00u);
    auto compute_unit = [&](int64_t pi, I8Unit& U) {
      const int64_t pt0 = (page0 + pi) * kBlockSize;   // first token of the page
      const bool full = U.ok && pt0 + kBlockSize <= tok1;   // the same for every lane
      const int nv = U.ok ? (int)max((int64_t)0, min((int64_t)kBlockSize, tok1 - pt0)) : 0;
      if (!full) {
        // rows outside the split or the sequence, or of a masked page, get
        // weight 0; their stale codes and scales become zeros (0 * NaN is not 0)
        const bool keep = lo < nv;
#pragma unroll
        for (int i = 0; i < 4; ++i) U.vc[i] = keep ? U.vc[i] : u32x4_t{0u, 0u, 0u, 0u};
        U.vs = keep ? U.vs : u32x2_t{0u, 0u};
        U.ks = keep ? U.ks : u32x2_t{0u, 0u};
      }
      // the group scales of rows 4 hi .. 4 hi + 3 (row r's are in lane r)
      u32x2_t ksr[4], vsr[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int src = 4 * (4 * hi + e);
        ksr[e] = u32x2_t{(uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)U.ks.x),
                         (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)U.ks.y)};
        vsr[e] = u32x2_t{(uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)U.vs.x),
                         (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)U.vs.y)};
      }
      // stage V codes as fp16 integers: row lo, logical chunks 8 hi .. 8 hi + 7
      {
        uint8_t* row = my_stage + lo * kRowBytesF16;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<uint4*>(row + ((8 * hi + j) ^ vswz(lo)) * 16) =
              i8x8_to_f16(U.vc[j >> 1][2 * (j & 1)], U.vc[j >> 1][2 * (j & 1) + 1]);
      }
      // T_g = K_g Q_g^T per scale group, then S^T = sum_g s_tg T_g in fp32
      floatx4_t tg[4];
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) tg[gg] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        tg[j >> 1] = mfma_f16(i8x8_to_f16(U.kc[j][0], U.kc[j][1]), qlds[j * 64 + lane],
                              tg[j >> 1]);
      float x[4];
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // copy the vector elements out first: a bit cast of a vector element
        // lvalue reads the vector's first element whatever the index
        const uint32_t w01 = ksr[e].x, w23 = ksr[e].y;
        const f16x2_t s01 = __builtin_bit_cast(f16x2_t, w01);
        const f16x2_t s23 = __builtin_bit_cast(f16x2_t, w23);
        float v = tg[0][e] * (float)s01[0];
        v = fmaf(tg[1][e], (float)s01[1], v);
        v = fmaf(tg[2][e], (float)s23[0], v);
        v = fmaf(tg[3][e], (float)s23[1], v);
        x[e] = full || 4 * hi + e < nv ? v * c : -INFINITY;
        mx = fmaxf(mx, x[e]);
      }
      mx = max_over_row_groups(mx);
      // p is multiplied by the token's V group scale in fp16 below: the page
      // counts as higher in the running maximum by 1 + the largest scale's
      // binary exponent (0 if it is below 1), so every p * s stays below
      // 2^15 (the softmax does not depend on the constant taken off a row)
      mx += vscale_shift(vsr);
      const bool grow = mx > m + kRescaleF4;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float mn = grow ? mx : m;
        const float alpha = fast_exp2(m - mn);
        m = mn;
#pragma unroll
        for (int i = 0; i < 16; ++i) o[i] *= alpha;
        lsum *= alpha;
      }
      const float mp = m - kPShiftF4;
      uint2 pop;
      pop.x = pk_f16(fast_exp2(x[0] - mp), fast_exp2(x[1] - mp));
      pop.y = pk_f16(fast_exp2(x[2] - mp), fast_exp2(x[3] - mp));
      lsum = mfma_f16_k16(ones, pop, lsum);
      // P^T operands with the V group scales of tokens 4hi .. 4hi+3 folded in
      uint2 pg[4];
      {
        const f16x2_t p01 = __builtin_bit_cast(f16x2_t, pop.x);
        const f16x2_t p23 = __builtin_bit_cast(f16x2_t, pop.y);
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int dw = gg >> 1;
          const uint32_t sel = (gg & 1) ? 0x07060302u : 0x05040100u;
          const f16x2_t s01 = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(vsr[1][dw], vsr[0][dw], sel));
          const f16x2_t s23 = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_perm(vsr[3][dw], vsr[2][dw], sel));
          pg[gg] = make_uint2(__builtin_bit_cast(uint32_t, p01 * s01),
                              __builtin_bit_cast(uint32_t, p23 * s23));
        }
      }
      // O^T += V^T (P o s_g)^T
      wave_lds_sync();
      auto read_vt = [&](int i) { return vt_operand(my_stage, i, lo, hi); };
      uint2 vt[kVtAhead];
#pragma unroll
      for (int i = 0; i < kVtAhead; ++i) vt[i] = read_vt(i);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        o[i] = mfma_f16_k16(vt[i % kVtAhead], pg[i >> 2], o[i]);
        if (i + kVtAhead < 16) vt[i % kVtAhead] = read_vt(i + kVtAhead);
        __builtin_amdgcn_sched_barrier(0);
      }
      wave_lds_sync();
    };

    // wave w takes pages w, w + kWavesI8, ...
    I8Unit R[kAheadI8 + 1];
#pragma unroll
    for (int k = 0; k < kAheadI8; ++k) load_unit(wave + k * kWavesI8, R[k]);
    for (int64_t u = wave; u < npages; u += (kAheadI8 + 1) * kWavesI8) {
#pragma unroll
      for (int b = 0; b <= kAheadI8; ++b) {
        const int64_t uu = u + b * kWavesI8;
        load_unit(uu + kAheadI8 * kWavesI8, R[(b + kAheadI8) % (kAheadI8 + 1)]);
        if (uu < npages) compute_unit(uu, R[b]);
      }
    }
  }
  finish_split_mfma<G, kWavesI8>(a, s, g, split, stage, o, lsum, m, 1.0f, wave, lo, hi);
}

// ---- merge ------------------------------------------------------------------

// Grid (4 x q_head, seq), 1024 threads: a workgroup owns 64 head dims of one
// (sequence, query head); its 16 waves each walk every 16th split (the walk
// is serial within a wave, so more waves shorten it: measured 2% on a
// whole decode call at 12 q / 2 KV heads, whose 256 splits made the merge
// 15 us long), and the 16 partial (max, sum, weighted output) triples are
// combined through LDS:
// out = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M), M = max_s lse_s.
// Splits that saw no token carry lse = -inf and weigh nothing.  With at most
// 4 splits per wave (64 in all, as in the 1M-token decode), a wave loads its
// maxima and outputs in one round instead of waiting for the maxima first
// (about 1 us of a 219 us NVFP4 decode call).
constexpr int kMergeGroups = 16;
constexpr int kMergeDims = kHeadDim / 4;

__global__ __launch_bounds__(64 * kMergeGroups) void decode_merge(DecodeArgs a) {
  __shared__ float sm_m[kMergeGroups], sm_l[kMergeGroups];
  __shared__ float sm_o[kMergeGroups][kMergeDims];
  const int qh = blockIdx.x >> 2, chunk = blockIdx.x & 3, s = blockIdx.y;
  const int grp = threadIdx.x >> 6, dl = threadIdx.x & 63;
  const int d = chunk * kMergeDims + dl;
  const int nsp = a.plan.num_splits;
  const int64_t slot0 = ((int64_t)s * a.num_q_heads + qh) * nsp;
  const float* lse = a.ws_lse + slot0;
  const float* o = a.ws_o + slot0 * kHeadDim + d;
  float M = -INFINITY;
  float L = 0.f, O = 0.f;
  if (nsp <= 4 * kMergeGroups) {
    // at most 4 splits per wave: their maxima and outputs are loaded in one
    // round (the sums below run in the same order as the general loop's,
    // with weight 0 for the slots past nsp, so the result is the same)
    float lv[4], ov[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sp = grp + u * kMergeGroups;
      lv[u] = sp < nsp ? lse[sp] : -INFINITY;
      ov[u] = sp < nsp ? o[(int64_t)sp * kHeadDim] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) M = fmaxf(M, lv[u]);
    if (M != -INFINITY) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = fast_exp2(lv[u] - M);
        L += w;
        O = fmaf(w, ov[u], O);
      }
    }
  } else {
  for (int sp = grp; sp < nsp; sp += kMergeGroups) M = fmaxf(M, lse[sp]);
  if (M != -INFINITY) {
    int sp = grp;
    for (; sp + 3 * kMergeGroups < nsp; sp += 4 * kMergeGroups) {
      float w[4], v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        w[u] = fast_exp2(lse[sp + u * kMergeGroups] - M);
        v[u] = o[(int64_t)(sp + u * kMergeGroups) * kHeadDim];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        L += w[u];
        O = fmaf(w[u], v[u], O);
      }
    }
    for (; sp < nsp; sp += kMergeGroups) {
      const float w = fast_exp2(lse[sp] - M);
      L += w;
      O = fmaf(w, o[(int64_t)sp * kHeadDim], O);
    }
  }
  }
  if (dl == 0) {
    sm_m[grp] = M;
    sm_l[grp] = L;
  }
  sm_o[grp][dl] = O;
  __syncthreads();
  if (grp == 0) {
    float Mt = -INFINITY;
#pragma unroll
    for (int g2 = 0; g2 < kMergeGroups; ++g2) Mt = fmaxf(Mt, sm_m[g2]);
    float res = 0.f;
    if (Mt != -INFINITY) {
      float Lt = 0.f, Ot = 0.f;
#pragma unroll
      for (int g2 = 0; g2 < kMergeGroups; ++g2) {
        const float sc = sm_m[g2] == -INFINITY ? 0.f : fast_exp2(sm_m[g2] - Mt);
        Lt += sm_l[g2] * sc;
        Ot += sm_o[g2][dl] * sc;
      }
      res = Ot / Lt;
    }
    const int64_t oi = ((int64_t)s * a.num_q_heads + qh) * kHeadDim + d;
    if (a.out_f32)
      static_cast<float*>(a.out)[oi] = res;
    else
      static_cast<uint16_t*>(a.out)[oi] = f32_to_bf16(res);
  }
}

template <int G>
hipError_t launch_split(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.plan.num_splits, a.geo.num_kv_heads, a.num_seqs);
  if (a.dtype == 2) return launch(decode_split_int8<G>, grid, dim3(kThreadsI8), 0, st, a);
  return launch(decode_split_nvfp4<G>, grid, dim3(kThreadsF4), 0, st, a);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  if (a.dtype == 0) {
    // bf16: the verify kernels with one query at position len - 1, which sees
    // every cached token; an empty sequence gives zeros and is no error
    VerifyArgs v;
    v.d = a;
    v.num_queries = 1;
    v.min_len = 0;
    return launch_verify(v, st);
  }
  hipError_t e;
  switch (a.group) {
    case 1: e = launch_split<1>(a, st); break;
    case 2: e = launch_split<2>(a, st); break;
    case 3: e = launch_split<3>(a, st); break;
    case 4: e = launch_split<4>(a, st); break;
    case 6: e = launch_split<6>(a, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return launch_decode_merge(a, st);
}

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t st) {
  return launch(decode_merge, dim3(4 * a.num_q_heads, a.num_seqs), dim3(64 * kMergeGroups), 0,
                st, a);
}

}  // namespace yrk
