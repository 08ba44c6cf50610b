// Multi-query split-K decode attention over a paged bf16 or INT8 group-64 KV
// cache (gfx950): the verify step of speculative decoding, where num_queries
// consecutive tokens of a sequence (the last accepted one and the drafted
// ones) attend to the cache at once ([P1] "Things that bit me" and [P3]
// "Limitations": a verify round evaluates K + 1 query columns; [P3] "Usage":
// 1 to 5 draft tokens, so 2 to 6 queries).  Their keys and values are in the
// cache already; query i of a sequence of len cached tokens sits at position
// len - num_queries + i and sees keys 0 .. len - num_queries + i.  With one
// query (at len - 1, seeing every cached token) the bf16 kernel is also the
// single-query decode kernel of a bf16 cache.
//
// With G query heads per KV head, one KV head serves R = num_queries x G
// query rows (row r = query r / G, head r % G of the group).  Every key is
// used by all R rows, so the rows share each load, and with R up to 48 the
// two products are dense enough for the matrix cores:
//
//   grid      (split, kv_head, seq), 4 waves; a split owns a contiguous token
//             range and wave w takes its pages w, w + 4, ... (16 tokens each);
//             where registers allow, the next page's loads are in flight while
//             one is computed.
//   S^T       = K Q^T on v_mfma_f32_16x16x32_bf16, one 16-row column block of
//             Q at a time (C = ceil(R / 16) blocks).  Lane (t, kg) loads 16
//             bytes of key row t per step (head dims 32 j + 8 kg .. +7; every
//             load instruction reads 64 contiguous bytes of 16 rows), which is
//             the A operand as loaded.  The Q^T operands of the workgroup's R
//             rows sit in LDS, read once per step and block.
//   softmax   per row, log2 domain, in the accumulator layout: lane (h, r)
//             holds tokens 4r .. 4r + 3 of row h.  The running maximum is
//             raised (and O rescaled) only when a page exceeds it by more
//             than 1, so p = 2^(s - m) <= 2.  Keys past a row's own position
//             and past the split get p = 0.
//   O^T      += V^T P^T on the same instruction with its 32-long inner
//             dimension holding each token twice: p is split into
//             p_hi = bf16(p) and p_lo = bf16(p - p_hi), and the operand pair
//             (V^T, V^T) x (P_hi^T ; P_lo^T) sums V (p_hi + p_lo), so the
//             weights keep 16 significant bits instead of bf16's 8 at no
//             extra instruction.  V is staged into per-wave LDS (swizzled
//             rows) and read back transposed with ds_read_b64_tr_b16.  The
//             row sums are the same product with a ones operand.
//   finish    the 4 waves' partials of a column block are combined through
//             LDS into one normalised partial and log2-sum-exp per (query,
//             head, split); the decode merge then combines the splits.
#include "attn_common.h"

#include <type_traits>

namespace yrk {
namespace {

constexpr int kColRows = kVerifyColRows;                            // rows per MFMA column block
constexpr int kQOpBytes = 8 * 64 * 16;                              // Q^T operands of a block: 8 KiB
constexpr float kRescaleV = 1.0f;

__device__ __forceinline__ floatx4_t mfma_bf16(const u32x4_t& a, const u32x4_t& b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Two floats -> packed bf16, rounded to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){lo, hi}, b2_t));
}

// The P^T operand of 4 weights: bf16 high parts, then the bf16 residuals.
__device__ __forceinline__ u32x4_t split_weights(const float (&p)[4]) {
  const uint32_t h01 = pk_bf16(p[0], p[1]), h23 = pk_bf16(p[2], p[3]);
  const uint32_t l01 = pk_bf16(p[0] - bf16_lo(h01), p[1] - bf16_hi(h01));
  const uint32_t l23 = pk_bf16(p[2] - bf16_lo(h23), p[3] - bf16_hi(h23));
  return u32x4_t{h01, h23, l01, l23};
}

// Per column-block count C: pages a wave keeps in flight beyond the one it
// computes, and waves of the (one per CU) workgroup.  Two waves per SIMD
// matter more than a deeper register ring (measured at 4 queries, 1M
// tokens: 0.755 ms with two waves per SIMD and no ring against 0.815 ms with
// one and one page ahead); three column blocks hold 192 accumulator
// registers and leave room for one wave per SIMD.  Two waves per SIMD come
// from one 8-wave workgroup with the priority balance (balance_issue), not
// two 4-wave workgroups, whose first-placed one ran far ahead of the other:
// per 1M-token layer at 1, 2 and 4 queries 725, 727 and 731 us against 732,
// 736 and 752 us.  Three column blocks leave one wave per SIMD, and there the
// page loop is pipelined (kPipelined): 6 queries 858 -> 737 us.  (The same
// pipelining of the INT8 kernel, whose pages carry far more vector work and
// which then keeps one page ahead instead of two, measured 857 against
// 828 us.)
template <int C> struct VerifyTune;
template <> struct VerifyTune<1> {
  static constexpr int kAhead = 1, kWaves = verify_waves(1, 0);
  static constexpr bool kPipelined = false;
};
template <> struct VerifyTune<2> {
  static constexpr int kAhead = 0, kWaves = verify_waves(2, 0);
  static constexpr bool kPipelined = false;
};
template <> struct VerifyTune<3> {
  static constexpr int kAhead = 1, kWaves = verify_waves(3, 0);
  static constexpr bool kPipelined = true;
};

// One lane's share of one page: 16-byte chunks 4 j + kg of key and value
// row t (head dims 32 j + 8 kg .. +7).
struct VUnit {
  u32x4_t k[8], v[8];
  bool ok;                  // page present and inside the split
};

template <int C>
__global__ __launch_bounds__(64 * VerifyTune<C>::kWaves, 1) void verify_split_bf16(
    VerifyArgs va) {
  constexpr int AHEAD = VerifyTune<C>::kAhead;
  constexpr int NW = VerifyTune<C>::kWaves;   // one workgroup per CU, NW / 4 waves per SIMD
  constexpr int NT = 64 * NW;
  static_assert(C >= 1 && C <= 3 && AHEAD >= 0 && AHEAD <= 2, "verify kernel shape");
  // one staged V page per wave; two where the page loop is pipelined
  constexpr bool PIPE = VerifyTune<C>::kPipelined;
  constexpr int kStagePages = PIPE ? 2 : 1;
  constexpr int kStageV = NW * kStagePages * kBlockSize * kRowBytesF16;
  constexpr int kFinish = (NW * kColRows * kHeadDim + 2 * NW * kColRows) * 4;
  constexpr int kLds = kStageV + C * kQOpBytes > kFinish ? kStageV + C * kQOpBytes : kFinish;
  const DecodeArgs& a = va.d;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
  __shared__ __attribute__((aligned(16))) uint32_t progress[NW];   // pages done per wave
  const int split = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int lo = lane & 15, hi = lane >> 4;
  const int G = a.group, nq = va.num_queries, R = nq * G;

  int64_t len = a.seq_lens[s];
  if (len > a.max_seq_len) {
    if (threadIdx.x == 0 && split == 0 && g == 0) err_flag(a.err, kErrPosition);
    len = a.max_seq_len;
  }
  if (len < va.min_len && threadIdx.x == 0 && split == 0 && g == 0) err_flag(a.err, kErrPosition);
  if (len < 0) len = 0;
  const int64_t qpos0 = len - nq;   // position of query 0 (negative only when flagged)
  const int64_t tok0 = (int64_t)split * a.plan.tokens_per_split;
  const int64_t tok1 = min(len, tok0 + a.plan.tokens_per_split);

  // Q^T operands: block c, step j, lane l at ((c * 8 + j) * 64 + l) * 16
  // bytes: row 16 c + l % 16, head dims 32 j + 8 (l / 16) .. +7 (zero rows
  // beyond R)
  u32x4_t* qop = reinterpret_cast<u32x4_t*>(lds + kStageV);
  if (threadIdx.x < NW) progress[threadIdx.x] = 0;
  for (int idx = threadIdx.x; idx < C * 8 * 64; idx += NT) {
    const int l = idx & 63, j = (idx >> 6) & 7, c = idx >> 9;
    const int r = kColRows * c + (l & 15);
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (r < R) {
      const int64_t h = (int64_t)g * G + r % G;
      const uint16_t* qrow = a.q + (((int64_t)s * nq + r / G) * a.num_q_heads + h) * kHeadDim;
      v = *reinterpret_cast<const u32x4_t*>(qrow + 32 * j + 8 * (l >> 4));
    }
    qop[idx] = v;
  }
  // the last key position lane lo's row of each block may see
  int64_t last[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int r = kColRows * c + lo;
    last[c] = qpos0 + (r < R ? r / G : nq - 1);
  }
  __syncthreads();

  floatx4_t o[C][16], lsum[C];
  float m[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
#pragma unroll
    for (int i = 0; i < 16; ++i) o[c][i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    lsum[c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    m[c] = kNegBig;
  }

  if (tok1 > tok0) {
    const uint16_t* K = static_cast<const uint16_t*>(a.k);
    const uint16_t* V = static_cast<const uint16_t*>(a.v);
    const int64_t page0 = tok0 / kBlockSize;
    const int64_t npages = (tok1 - tok0 + kBlockSize - 1) / kBlockSize;
    uint8_t* my_stage = lds + wave * (kStagePages * kBlockSize * kRowBytesF16);
    const float cl2 = a.scale_log2;
    const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};

    auto load_unit = [&](int64_t pi, VUnit& U) {
      int64_t base = 0, ts = 0;   // in elements
      bool ok = false;
      if (pi < npages) {
        ok = page_base(a, s, g, page0 + pi, kHeadDim, &base, &ts);
        if (!ok && lane == 0) err_flag(a.err, kErrBlockId);
      }
      U.ok = ok;
      const u32x4_t z = {0u, 0u, 0u, 0u};
      u32x4_t k[8], v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) k[j] = v[j] = z;
      if (ok) {
        const int64_t row = base + lo * ts;
        const u32x4_t* kp = reinterpret_cast<const u32x4_t*>(K + row) + hi;
        const u32x4_t* vp = reinterpret_cast<const u32x4_t*>(V + row) + hi;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          k[j] = kp[4 * j];
          v[j] = vp[4 * j];
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        U.k[j] = k[j];
        U.v[j] = v[j];
      }
    };

    // tokens of page pi that lie in the split (0 for a masked page), and
    // whether every row sees all of them
    auto page_extent = [&](int64_t pi, bool ok, int* nv, bool* full) {
      const int64_t pt0 = (page0 + pi) * kBlockSize;   // first token of the page
      *nv = ok ? (int)max((int64_t)0, min((int64_t)kBlockSize, tok1 - pt0)) : 0;
      *full = *nv == kBlockSize && pt0 + kBlockSize - 1 <= qpos0;
    };

    // stage V of the page into `stage`: row lo, logical chunks 4 j + hi
    auto stage_v = [&](int64_t pi, VUnit& U, uint8_t* stage) {
      int nv;
      bool full;
      page_extent(pi, U.ok, &nv, &full);
      if (nv < kBlockSize) {
        // rows outside the split or the sequence, or of a masked page, get
        // weight 0; their stale values become zeros (0 * NaN is not 0)
        const bool keep = lo < nv;
#pragma unroll
        for (int j = 0; j < 8; ++j) U.v[j] = keep ? U.v[j] : u32x4_t{0u, 0u, 0u, 0u};
      }
      uint8_t* row = stage + lo * kRowBytesF16;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<u32x4_t*>(row + ((4 * j + hi) ^ vswz(lo)) * 16) = U.v[j];
    };

    // S^T = K Q^T of the page, per column block
    auto scores = [&](const VUnit& U, floatx4_t (&sc)[C]) {
#pragma unroll
      for (int c = 0; c < C; ++c) sc[c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int c = 0; c < C; ++c) sc[c] = mfma_bf16(U.k[j], qop[(c * 8 + j) * 64 + lane], sc[c]);
      }
    };

    // masks, the lazy rescale of O and the row sums, and the P^T operands
    auto softmax = [&](int64_t pi, bool ok, const floatx4_t (&sc)[C], u32x4_t (&pop)[C]) {
      int nv;
      bool full;
      page_extent(pi, ok, &nv, &full);
      const int64_t pt0 = (page0 + pi) * kBlockSize;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        float x[4];
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool vis = full || (4 * hi + e < nv && pt0 + 4 * hi + e <= last[c]);
          x[e] = vis ? sc[c][e] * cl2 : -INFINITY;
          mx = fmaxf(mx, x[e]);
        }
        mx = max_over_row_groups(mx);
        const bool grow = mx > m[c] + kRescaleV;
        if (__builtin_amdgcn_ballot_w64(grow)) {
          const float mn = grow ? mx : m[c];
          const float alpha = fast_exp2(m[c] - mn);
          m[c] = mn;
#pragma unroll
          for (int i = 0; i < 16; ++i) o[c][i] *= alpha;
          lsum[c] *= alpha;
        }
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = fast_exp2(x[e] - m[c]);
        pop[c] = split_weights(p);
        lsum[c] = mfma_bf16(ones, pop[c], lsum[c]);
      }
    };

    // O^T += V^T (P_hi + P_lo)^T from the staged page
    auto pv = [&](const uint8_t* stage, const u32x4_t (&pop)[C]) {
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint2 vt = vt_operand(stage, i, lo, hi);
        const u32x4_t av = {vt.x, vt.y, vt.x, vt.y};
#pragma unroll
        for (int c = 0; c < C; ++c) o[c][i] = mfma_bf16(av, pop[c], o[c][i]);
      }
      wave_lds_sync();
    };

    auto compute_unit = [&](int64_t pi, VUnit& U) {
      stage_v(pi, U, my_stage);
      floatx4_t sc[C];
      scores(U, sc);
      u32x4_t pop[C];
      softmax(pi, U.ok, sc, pop);
      pv(my_stage, pop);
    };

    // wave w takes pages w, w + NW, ...
    if constexpr (PIPE) {
      // One wave per SIMD: nothing else fills the matrix core while a page's
      // chain (scores, then the softmax on the vector ALUs, then the value
      // products) runs.  So the scores of page n + 1 go to the matrix core
      // ahead of page n's value products, and its softmax follows them (the
      // rescale of O after page n's products, as in the plain order), with
      // page n + 1's V staged in the other half of the wave's staging.  The
      // operations on O, the row sums and the running maxima are those of
      // the plain loop, in the same order: the results are the same bits.
      // Page n + 2 loads while page n + 1 is scored.
      static_assert(AHEAD == 1, "the pipelined loop keeps one page ahead");
      VUnit U[2];
      u32x4_t pop[C];
      load_unit(wave, U[0]);
      load_unit(wave + NW, U[1]);
      {
        stage_v(wave, U[0], my_stage);
        floatx4_t sc[C];
        scores(U[0], sc);
        softmax(wave, U[0].ok, sc, pop);
      }
      // one step: page u's value products, page u + NW's scores and softmax;
      // Ucur held page u (scored and staged a step ago) and takes page u + 2 NW
      auto step = [&](int64_t u, VUnit& Ucur, VUnit& Unxt, uint8_t* st_cur, uint8_t* st_nxt) {
        const int64_t un = u + NW;
        floatx4_t sc[C];
        const bool has_next = un < npages;
        const bool next_ok = Unxt.ok;
        if (has_next) {
          stage_v(un, Unxt, st_nxt);
          scores(Unxt, sc);
        }
        load_unit(u + 2 * NW, Ucur);
        pv(st_cur, pop);
        if (has_next) softmax(un, next_ok, sc, pop);
      };
      uint8_t* st0 = my_stage;
      uint8_t* st1 = my_stage + kBlockSize * kRowBytesF16;
      // unrolled by two so that the ring's registers are named statically
      for (int64_t u = wave; u < npages; u += 2 * NW) {
        step(u, U[0], U[1], st0, st1);
        if (u + NW < npages) step(u + NW, U[1], U[0], st1, st0);
      }
    } else {
      VUnit U[AHEAD + 1];
      uint32_t done = 0;
#pragma unroll
      for (int k = 0; k < AHEAD; ++k) load_unit(wave + k * NW, U[k]);
      for (int64_t u = wave; u < npages; u += (AHEAD + 1) * NW) {
#pragma unroll
        for (int b = 0; b <= AHEAD; ++b) {
          const int64_t uu = u + b * NW;
          load_unit(uu + AHEAD * NW, U[(b + AHEAD) % (AHEAD + 1)]);
          if (uu < npages) compute_unit(uu, U[b]);
          if constexpr (NW == 8) balance_issue<NW>(progress, ++done, wave, lane);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // combine the NW waves, one column block at a time
  float* sm_o = reinterpret_cast<float*>(lds);     // [NW][16][256]
  float* sm_m = sm_o + NW * kColRows * kHeadDim;
  float* sm_l = sm_m + NW * kColRows;
  const int nsp = a.plan.num_splits;
  const int64_t rows_per_seq = (int64_t)nq * a.num_q_heads;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i)
      *reinterpret_cast<floatx4_t*>(sm_o + (wave * kColRows + lo) * kHeadDim + 16 * i + 4 * hi) =
          o[c][i];
    if (hi == 0) {
      sm_m[wave * kColRows + lo] = m[c];
      sm_l[wave * kColRows + lo] = lsum[c][0];
    }
    __syncthreads();
    // NT / 256 rows of the block per pass, thread % 256 = head dim
    for (int row = threadIdx.x / kHeadDim; row < kColRows; row += NT / kHeadDim) {
      const int r = kColRows * c + row;
      if (r >= R) break;
      const int d = threadIdx.x % kHeadDim;
      float M = kNegBig;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w * kColRows + row]);
      float L = 0.f, Ov = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float sc = fast_exp2(sm_m[w * kColRows + row] - M);
        L += sm_l[w * kColRows + row] * sc;
        Ov += sm_o[(w * kColRows + row) * kHeadDim + d] * sc;
      }
      const int64_t hh = (int64_t)(r / G) * a.num_q_heads + (int64_t)g * G + r % G;
      const int64_t slot = ((int64_t)s * rows_per_seq + hh) * nsp + split;
      a.ws_o[slot * kHeadDim + d] = L > 0.f ? Ov / L : 0.f;
      if (d == 0) a.ws_lse[slot] = L > 0.f ? M + __log2f(L) : -INFINITY;
    }
  }
}

// ---- INT8 group-64 cache -----------------------------------------------------
//
// The same rows, column blocks, masks and combine over an INT8 group-64
// cache, with the INT8 decode kernel's exact integer path: the codes enter
// the matrix cores as fp16 integers (v_mfma_f32_16x16x32_f16 for the scores
// and for the values of two pages), each key step covers 32 dims of one scale group
// so that a group's partial products T_g are scaled by the token's key group
// scale in fp32, and the value group scales ride on the fp16 weights
// (p = 2^(s - m + 14), the page counted higher in the running maximum by 1 +
// its largest V scale's exponent so that p * s stays below 2^15).  The Q^T
// operands are fp16 after one power-of-two prescale shared by the R rows,
// which puts the largest |q| in [2^14, 2^15) (bf16 values are exact there).

// Used for one column block (up to 2 queries at GQA 6; two and three go to
// the team kernel below).  Measured per 1M-token layer (2, 4, 6 queries at
// GQA 6), as two 4-wave workgroups per CU: C = 1 0.427 ms with one page ahead
// (0.443 with two); C = 2 0.464 ms without a ring; C = 3, one workgroup per
// CU, 0.941 / 0.897 / 0.819 ms with 0 / 1 / 2 pages ahead (one wave per SIMD
// leaves latency exposed).  One 8-wave workgroup with the priority balance:
// 1 and 2 queries 399 and 407 us against 409 and 413 us; 4 queries the same
// (476 / 474 us).  A wave step now covers two pages, with no step ahead:
// one softmax over their 32 tokens and the value products on the 32-long
// inner dimension, as in the team kernel (C = 1: 406 against 416 us with
// one page a step and one page ahead; at C = 2 the two-page step spilled 28
// registers, 995 us).
template <int C> struct VerifyTuneI8;
template <> struct VerifyTuneI8<1> { static constexpr int kAhead = 0, kWaves = verify_waves(1, 2); };

// One lane's share of one page.
struct I8VUnit {
  u32x2_t kc[8];   // K: step j's 8 code bytes of row t (dims 64 (j/2) + 32 (j%2) + 8 kg .. +7)
  u32x4_t vc[4];   // V: code bytes [64 kg, 64 kg + 64) of row t
  u32x2_t ks, vs;  // row t's four binary16 group scales
  bool ok;         // page present and inside the split
};

template <int C>
__global__ __launch_bounds__(64 * VerifyTuneI8<C>::kWaves, 1) void verify_split_int8(
    VerifyArgs va) {
  constexpr int AHEAD = VerifyTuneI8<C>::kAhead;
  constexpr int NW = VerifyTuneI8<C>::kWaves;   // one workgroup per CU, NW / 4 waves per SIMD
  constexpr int NT = 64 * NW;
  static_assert(C == 1 && AHEAD >= 0 && AHEAD <= 2, "verify kernel shape");
  constexpr int kStageV = NW * 2 * kBlockSize * kRowBytesF16; // two V pages per wave
  constexpr int kFinish = (NW * kColRows * kHeadDim + 2 * NW * kColRows) * 4;
  constexpr int kUse = kStageV + C * kQOpBytes + NW * 4;
  constexpr int kLds = kUse > kFinish ? kUse : kFinish;
  const DecodeArgs& a = va.d;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLds];
  __shared__ __attribute__((aligned(16))) uint32_t progress[NW];   // pages done per wave
  const int split = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int lo = lane & 15, hi = lane >> 4;
  const int G = a.group, nq = va.num_queries, R = nq * G;

  int64_t len = a.seq_lens[s];
  if (len > a.max_seq_len) {
    if (threadIdx.x == 0 && split == 0 && g == 0) err_flag(a.err, kErrPosition);
    len = a.max_seq_len;
  }
  if (len < va.min_len && threadIdx.x == 0 && split == 0 && g == 0) err_flag(a.err, kErrPosition);
  if (len < 0) len = 0;
  const int64_t qpos0 = len - nq;
  const int64_t tok0 = (int64_t)split * a.plan.tokens_per_split;
  const int64_t tok1 = min(len, tok0 + a.plan.tokens_per_split);

  // Q^T operands: block c, step j, lane l at ((c * 8 + j) * 64 + l) * 16
  // bytes: row 16 c + l % 16, head dims 64 (j / 2) + 32 (j % 2) + 8 (l / 16)
  // .. +7, as fp16 after the shared prescale (zero rows beyond R)
  auto q_chunk = [&](int idx) {
    const int l = idx & 63, j = (idx >> 6) & 7, c = idx >> 9;
    const int r = kColRows * c + (l & 15);
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (r < R) {
      const int64_t h = (int64_t)g * G + r % G;
      const uint16_t* qrow = a.q + (((int64_t)s * nq + r / G) * a.num_q_heads + h) * kHeadDim;
      v = *reinterpret_cast<const u32x4_t*>(qrow + 64 * (j >> 1) + 32 * (j & 1) + 8 * (l >> 4));
    }
    return v;
  };
  float* red = reinterpret_cast<float*>(lds + kStageV + C * kQOpBytes);   // [NW]
  if (threadIdx.x < NW) progress[threadIdx.x] = 0;
  float qmax = 0.f;
  for (int idx = threadIdx.x; idx < C * 8 * 64; idx += NT) {
    const u32x4_t v = q_chunk(idx);
#pragma unroll
    for (int w = 0; w < 4; ++w) qmax = fmaxf(qmax, fmaxf(fabsf(bf16_lo(v[w])), fabsf(bf16_hi(v[w]))));
  }
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, sh));
  if (lane == 0) red[wave] = qmax;
  __syncthreads();
  qmax = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) qmax = fmaxf(qmax, red[w]);
  // 2^(14 - e): the largest |q| lands in [2^14, 2^15)
  const int qe = (int)((__float_as_uint(qmax) >> 23) & 0xFF);
  const int pe = qmax > 0.f ? min(max(268 - qe, 1), 254) : 127;
  const float qpre = __uint_as_float((uint32_t)pe << 23);
  const float cl2 = a.scale_log2 * __uint_as_float((uint32_t)(254 - pe) << 23);
  uint4* qop = reinterpret_cast<uint4*>(lds + kStageV);
  for (int idx = threadIdx.x; idx < C * 8 * 64; idx += NT) {
    const u32x4_t v = q_chunk(idx);
    uint32_t h4[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) h4[w] = pk_f16(bf16_lo(v[w]) * qpre, bf16_hi(v[w]) * qpre);
    qop[idx] = make_uint4(h4[0], h4[1], h4[2], h4[3]);
  }
  int64_t last[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int r = kColRows * c + lo;
    last[c] = qpos0 + (r < R ? r / G : nq - 1);
  }
  __syncthreads();

  floatx4_t o[C][16], lsum[C];
  float m[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
#pragma unroll
    for (int i = 0; i < 16; ++i) o[c][i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    lsum[c] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    m[c] = kNegBig;
  }

  if (tok1 > tok0) {
    const uint8_t* Kc = static_cast<const uint8_t*>(a.k);
    const uint8_t* Vc = static_cast<const uint8_t*>(a.v);
    const uint16_t* Ks = reinterpret_cast<const uint16_t*>(a.k_scale);
    const uint16_t* Vs = reinterpret_cast<const uint16_t*>(a.v_scale);
    const int64_t page0 = tok0 / kBlockSize;
    const int64_t npages = (tok1 - tok0 + kBlockSize - 1) / kBlockSize;
    uint8_t* my_stage = lds + wave * (2 * kBlockSize * kRowBytesF16);
    const uint4 ones = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);

    auto load_unit = [&](int64_t pi, I8VUnit& U) {
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

    // one step: pages 2 uu and 2 uu + 1, one softmax over their 32 tokens,
    // the value products on the 32-long inner dimension (k order: tokens
    // 4 hi .. 4 hi + 3 of the first page, then of the second)
    auto compute_pair = [&](int64_t uu, I8VUnit (&U2)[2]) {
      float x[C][2][4];
      u32x2_t vsr[2][4];
      float vsh = 0.f;
      int nvp[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        I8VUnit& U = U2[p];
        const int64_t pt0 = (page0 + 2 * uu + p) * kBlockSize;
        nvp[p] = U.ok ? (int)max((int64_t)0, min((int64_t)kBlockSize, tok1 - pt0)) : 0;
        if (nvp[p] < kBlockSize) {
          // rows outside the split or the sequence, or of a masked page, get
          // weight 0; their stale codes and scales become zeros (0 * NaN is not 0)
          const bool keep = lo < nvp[p];
#pragma unroll
          for (int i = 0; i < 4; ++i) U.vc[i] = keep ? U.vc[i] : u32x4_t{0u, 0u, 0u, 0u};
          U.ks = keep ? U.ks : u32x2_t{0u, 0u};
          U.vs = keep ? U.vs : u32x2_t{0u, 0u};
        }
        // stage V codes as fp16 integers: row lo, logical chunks 8 hi .. 8 hi + 7
        uint8_t* row = my_stage + (p * kBlockSize + lo) * kRowBytesF16;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<uint4*>(row + ((8 * hi + j) ^ vswz(lo)) * 16) =
              i8x8_to_f16(U.vc[j >> 1][2 * (j & 1)], U.vc[j >> 1][2 * (j & 1) + 1]);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        I8VUnit& U = U2[p];
        const int64_t pi = 2 * uu + p;
        const int64_t pt0 = (page0 + pi) * kBlockSize;   // first token of the page
        const int nv = nvp[p];
        // every row sees every token of the page (the same for all lanes)
        const bool full = nv == kBlockSize && pt0 + kBlockSize - 1 <= qpos0;
        // the group scales of rows 4 hi .. 4 hi + 3 (row r's are in lane r)
        u32x2_t ksr[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int src = 4 * (4 * hi + e);
          ksr[e] = u32x2_t{(uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)U.ks.x),
                           (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)U.ks.y)};
          vsr[p][e] = u32x2_t{(uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)U.vs.x),
                              (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)U.vs.y)};
        }
        // T_g = K_g Q_g^T per scale group and column block (each key step's
        // codes are converted once for all blocks)
        floatx4_t tg[C][4];
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
          for (int gg = 0; gg < 4; ++gg) tg[c][gg] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint4 kf = i8x8_to_f16(U.kc[j][0], U.kc[j][1]);
#pragma unroll
          for (int c = 0; c < C; ++c)
            tg[c][j >> 1] = mfma_f16(kf, qop[(c * 8 + j) * 64 + lane], tg[c][j >> 1]);
        }
        vsh = fmaxf(vsh, vscale_shift(vsr[p]));
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w01 = ksr[e].x, w23 = ksr[e].y;   // copies: see the INT8 decode kernel
            const f16x2_t s01 = __builtin_bit_cast(f16x2_t, w01);
            const f16x2_t s23 = __builtin_bit_cast(f16x2_t, w23);
            float v = fmaf(tg[c][0][e], (float)s01[0], 0.f);
            v = fmaf(tg[c][1][e], (float)s01[1], v);
            v = fmaf(tg[c][2][e], (float)s23[0], v);
            v = fmaf(tg[c][3][e], (float)s23[1], v);
            v *= cl2;
            asm volatile("" : "+v"(v));
            const bool vis = full || (4 * hi + e < nv && pt0 + 4 * hi + e <= last[c]);
            x[c][p][e] = vis ? v : -INFINITY;
          }
      }
      uint4 pg[C][4];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        float mx = -INFINITY;
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int e = 0; e < 4; ++e) mx = fmaxf(mx, x[c][p][e]);
        mx = max_over_row_groups(mx) + vsh;
        const bool grow = mx > m[c] + kRescaleF4;
        if (__builtin_amdgcn_ballot_w64(grow)) {
          const float mn = grow ? mx : m[c];
          const float alpha = fast_exp2(m[c] - mn);
          m[c] = mn;
#pragma unroll
          for (int i = 0; i < 16; ++i) o[c][i] *= alpha;
          lsum[c] *= alpha;
        }
        const float mp = m[c] - kPShiftF4;
        uint2 pop[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          pop[p].x = pk_f16(fast_exp2(x[c][p][0] - mp), fast_exp2(x[c][p][1] - mp));
          pop[p].y = pk_f16(fast_exp2(x[c][p][2] - mp), fast_exp2(x[c][p][3] - mp));
        }
        lsum[c] = mfma_f16(ones, make_uint4(pop[0].x, pop[0].y, pop[1].x, pop[1].y), lsum[c]);
        // P^T operands with the V group scales of tokens 4 hi .. 4 hi + 3
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int dw = gg >> 1;
          const uint32_t sel = (gg & 1) ? 0x07060302u : 0x05040100u;
          uint32_t w[4];
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const f16x2_t p01 = __builtin_bit_cast(f16x2_t, pop[p].x);
            const f16x2_t p23 = __builtin_bit_cast(f16x2_t, pop[p].y);
            const f16x2_t s01 = __builtin_bit_cast(
                f16x2_t, __builtin_amdgcn_perm(vsr[p][1][dw], vsr[p][0][dw], sel));
            const f16x2_t s23 = __builtin_bit_cast(
                f16x2_t, __builtin_amdgcn_perm(vsr[p][3][dw], vsr[p][2][dw], sel));
            w[2 * p] = __builtin_bit_cast(uint32_t, p01 * s01);
            w[2 * p + 1] = __builtin_bit_cast(uint32_t, p23 * s23);
          }
          pg[c][gg] = make_uint4(w[0], w[1], w[2], w[3]);
        }
      }
      // O^T += V^T (P o s_g)^T; 16 output dims lie in one scale group
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint2 va = vt_operand(my_stage, i, lo, hi);
        const uint2 vb = vt_operand(my_stage + kBlockSize * kRowBytesF16, i, lo, hi);
        const uint4 vt = make_uint4(va.x, va.y, vb.x, vb.y);
#pragma unroll
        for (int c = 0; c < C; ++c) o[c][i] = mfma_f16(vt, pg[c][i >> 2], o[c][i]);
      }
      wave_lds_sync();
    };

    // wave w takes page pairs w, w + NW, ...
    const int64_t npairs = (npages + 1) / 2;
    I8VUnit U[AHEAD + 1][2];
    uint32_t done = 0;
#pragma unroll
    for (int k = 0; k < AHEAD; ++k) {
      load_unit(2 * (wave + k * NW), U[k][0]);
      load_unit(2 * (wave + k * NW) + 1, U[k][1]);
    }
    for (int64_t u = wave; u < npairs; u += (AHEAD + 1) * NW) {
#pragma unroll
      for (int b = 0; b <= AHEAD; ++b) {
        const int64_t uu = u + b * NW;
        load_unit(2 * (uu + AHEAD * NW), U[(b + AHEAD) % (AHEAD + 1)][0]);
        load_unit(2 * (uu + AHEAD * NW) + 1, U[(b + AHEAD) % (AHEAD + 1)][1]);
        if (uu < npairs) compute_pair(uu, U[b]);
        if constexpr (NW == 8) balance_issue<NW>(progress, ++done, wave, lane);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }

  // combine the 4 waves, one column block at a time (l and O carry 2^kPShiftF4)
  float* sm_o = reinterpret_cast<float*>(lds);     // [NW][16][256]
  float* sm_m = sm_o + NW * kColRows * kHeadDim;
  float* sm_l = sm_m + NW * kColRows;
  const int nsp = a.plan.num_splits;
  const int64_t rows_per_seq = (int64_t)nq * a.num_q_heads;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i)
      *reinterpret_cast<floatx4_t*>(sm_o + (wave * kColRows + lo) * kHeadDim + 16 * i + 4 * hi) =
          o[c][i];
    if (hi == 0) {
      sm_m[wave * kColRows + lo] = m[c] - kPShiftF4;
      sm_l[wave * kColRows + lo] = lsum[c][0];
    }
    __syncthreads();
    for (int row = threadIdx.x / kHeadDim; row < kColRows; row += NT / kHeadDim) {
      const int r = kColRows * c + row;
      if (r >= R) break;
      const int d = threadIdx.x % kHeadDim;
      float M = kNegBig;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w * kColRows + row]);
      float L = 0.f, Ov = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float sc = fast_exp2(sm_m[w * kColRows + row] - M);
        L += sm_l[w * kColRows + row] * sc;
        Ov += sm_o[(w * kColRows + row) * kHeadDim + d] * sc;
      }
      const int64_t hh = (int64_t)(r / G) * a.num_q_heads + (int64_t)g * G + r % G;
      const int64_t slot = ((int64_t)s * rows_per_seq + hh) * nsp + split;
      a.ws_o[slot * kHeadDim + d] = L > 0.f ? Ov / L : 0.f;
      if (d == 0) a.ws_lse[slot] = L > 0.f ? M + __log2f(L) : -INFINITY;
    }
  }
}

// ---- INT8 cache, 2 or 3 column blocks: a team of 4 waves per split --------
//
// Keeping two or three column blocks' accumulators in each wave, as the
// kernel above does for one (128 or 192 registers), leaves one wave to run a
// page's whole chain (conversion, score products, softmax on the vector ALUs,
// value products) with at most two waves per SIMD to cover its latencies.
// Here a
// workgroup of 4 waves walks the split's pages together, two pages a step:
//
//   compute   waves 0 .. C-1, one per column block (64 accumulator
//             registers): score products from the staged K, one softmax
//             over the step's 32 tokens, value products from the staged V
//             on the 32-long inner dimension, for its 16 rows;
//   loading   each page's 512 16-byte code chunks are 8 groups of 64 (4 of
//             K rows, 4 of V rows); every wave loads whole groups of the
//             pages kTeamAhead + 1 steps ahead and converts them to fp16
//             integers into the staged pages, the waves without column
//             block the most of them (C = 3: 5 groups on wave 3, one on each
//             compute wave; C = 2: 4 on each of waves 2 and 3, none on the
//             compute waves); the first wave without column block also
//             stages the group scales, the page's valid rows and its
//             largest V scale;
//   staging   two LDS buffers of two pages: in step p the compute waves read
//             the pages of step p while every wave writes its groups of step
//             p + 1 into the other buffer (last read in step p - 1); one
//             workgroup barrier ends each step.  K rows and V rows share one
//             swizzle (tswz).
//
// The arithmetic per row is the INT8 kernel's above (same prescale of Q,
// exact integer codes, K group scales on the per-group partial products, V
// group scales on the fp16 weights, the V-scale shift of the running
// maximum), with the running maximum and the rescale taken once per two
// pages; a wave's rows see the split's pages in order, so each compute wave
// writes its rows' normalised partials itself.
//
// Launched for two and three column blocks (3-8 queries at GQA 6), two teams
// per CU.
// 6 queries over a 1M-token layer: 826 us on the kernel above, 634 us here
// with one page a step, 550 us with two, 520 us with the V-scale maximum
// taken once per page by the loader and the scores masked by a select
// instead of a branch per element.  Two column blocks (3-4 queries) run here
// too, with the two waves without column block converting every group: 4
// queries 478 -> 450-459 us against the kernel above (with one group on each
// compute wave and 3 on each of the others, the same as the kernel above,
// 465-476 us).  Measured on the way: one wave per
// column block with no loader wave (each wave loading and converting its
// share, 3-wave teams) 679 us; a single loader wave converting every group,
// 594-614 us with one page a step and 563 us with two (the loader is then
// the slowest wave of each step); the loader filling an LDS ring with direct
// loads 742 us; the value products of page p issued among the scores of page
// p + 1, 694 us; loads two to four steps ahead instead of one, slower (more
// registers, longer unrolled code).

// Staged rows keep 16-byte chunk c of row t at position c ^ tswz(t).  tswz is
// a bijection of 0..15 (so the 16 rows of one score operand read, one chunk
// index, fall into 16 distinct bank groups) that gives rows 4r .. 4r + 3
// distinct bits 1-2 and rows 0..3 / 4..7 (8..11 / 12..15) distinct bit 3, so
// that each 32-lane half of a transposing V read (8 rows x 32 bytes) covers
// all 64 banks once.
__device__ __forceinline__ int tswz(int t) {
  return ((t & 3) << 1) | ((t >> 3) & 1) | (((t >> 2) & 1) << 3);
}

// A buffer resource over nbytes from p (raw addressing, no stride): loads
// at offsets past nbytes return zeros without touching memory.  The
// arguments are uniform; they are read from the first lane so that the
// descriptor is built in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_range(const void* p, uint32_t nbytes) {
  const uint64_t addr = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
  void* base = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0,
                                           (int)__builtin_amdgcn_readfirstlane(nbytes), 0x00020000);
}

constexpr int kTeamWaves = 4;
constexpr int kTeamAhead = 0;   // further steps a wave's loads run ahead of the step it stages

// Code-chunk groups (of 8 per page) that wave w loads and converts: groups
// team_group(C, w, 0 .. team_groups(C, w) - 1).
constexpr int team_groups(int C, int w) { return w < C ? (C == 3 ? 1 : 0) : (C == 3 ? 5 : 4); }
constexpr int team_group(int C, int w, int i) {
  return w < C ? 8 - C + w : (C == 3 ? i : 4 * (w - C) + i);
}

// One wave's share of one page: NG groups (16 codes per lane each) and, on
// the first wave without column block, lanes 0..15, row lane's K and V
// group scales.
template <int NG>
struct TeamShare {
  u32x4_t code[NG > 0 ? NG : 1];
  u32x2_t ks, vs;
  bool ok;   // page present and inside the split
};

template <int C>
__global__ __launch_bounds__(64 * kTeamWaves) __attribute__((amdgpu_waves_per_eu(2))) void verify_team_int8(
    VerifyArgs va) {
  constexpr int NW = kTeamWaves;
  constexpr int NU = kTeamAhead + 1;
  constexpr int kChunks = 2 * kBlockSize * kHeadDim / 16;   // 512: K rows' chunks, then V's
  constexpr int kStK = 0;
  constexpr int kStV = kBlockSize * kRowBytesF16;
  constexpr int kStS = 2 * kBlockSize * kRowBytesF16;       // K scale rows, then V's (8 B each)
  constexpr int kStN = kStS + 2 * kBlockSize * 8;           // valid rows, largest V scale bits (2 ints)
  constexpr int kStage = kStN + 16;                          // 16,656 B per staged page
  constexpr int kPP = 2;                                     // pages per step
  constexpr int kStep = kPP * kStage;                        // one staged step (kPP pages)
  constexpr int kDummy = 2 * kStep;                          // writes that are not kept
  static_assert(C >= 2 && C <= 3, "team kernel shape");
  static_assert(team_groups(C, 0) * C + team_groups(C, C) * (NW - C) == kChunks / 64,
                "every code group has one wave");
  const DecodeArgs& a = va.d;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kDummy + 64 * 16];
  __shared__ float red[NW];
  const int split = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lo = lane & 15, hi = lane >> 4;
  const int G = a.group, nq = va.num_queries, R = nq * G;

  int64_t len = a.seq_lens[s];
  if (len > a.max_seq_len) {
    if (threadIdx.x == 0 && split == 0 && g == 0) err_flag(a.err, kErrPosition);
    len = a.max_seq_len;
  }
  if (len < va.min_len && threadIdx.x == 0 && split == 0 && g == 0) err_flag(a.err, kErrPosition);
  if (len < 0) len = 0;
  const int64_t qpos0 = len - nq;
  const int64_t tok0 = (int64_t)split * a.plan.tokens_per_split;
  const int64_t tok1 = min(len, tok0 + a.plan.tokens_per_split);
  const int npages = tok1 > tok0 ? (int)((tok1 - tok0 + kBlockSize - 1) / kBlockSize) : 0;
  const int64_t page0 = tok0 / kBlockSize;
  const bool paged = a.geo.paged;
  const int64_t ts = paged ? 1 : a.geo.num_kv_heads;   // rows between a page's tokens
  const uint8_t* Kc = static_cast<const uint8_t*>(a.k);
  const uint8_t* Vc = static_cast<const uint8_t*>(a.v);
  const uint16_t* Ks = reinterpret_cast<const uint16_t*>(a.k_scale);
  const uint16_t* Vs = reinterpret_cast<const uint16_t*>(a.v_scale);
  typedef const __attribute__((address_space(4))) int32_t const_i32;
  const const_i32* trow =
      (const const_i32*)(const void*)(a.block_tables + (int64_t)s * a.block_table_stride);
  const bool has_scale = wave == C && lane < kBlockSize;
  const uint32_t sc_off = has_scale ? (uint32_t)(lane * ts * 8) : 0xFFFFFFF0u;

  auto team_barrier = []() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // The step loop shared by both roles; step u covers pages 2u and 2u + 1.
  // Step u stages this wave's groups of step u + 1 into buffer (u + 1) % 2,
  // issues the loads of its groups of step u + 1 + kTeamAhead into the units
  // step u + 1 came from (U[q % NU] holds step q), then runs body(u) and the
  // barrier.  The loop starts 2 NU steps early, with steps on pages before
  // the first (empty ranges, staged into a buffer that is not read), so that
  // every step is alike and the waits for a step's loads leave the later
  // steps' loads in flight; body does nothing for u < 0.  The table entries
  // of a block of 2 NU steps are scalar loads at the block's start (the
  // scalar counter, which each step's barrier drains).  The loop is unrolled
  // over a block so that units and buffers are named statically.
  auto run_steps = [&](auto tag, auto loader, auto&& body) {
    constexpr int NG = decltype(tag)::value;
    constexpr bool LOADER = decltype(loader)::value;   // the waves without column block
    constexpr int NA = NG > 0 ? NG : 1;   // (no zero-length arrays in device code)
    uint32_t code_off[NA], st_off[NA][2];
    const uint8_t* code_base[NA];
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int grp = team_group(C, wave < C ? 0 : C, i) + (wave < C ? wave : (C == 3 ? 0 : 4 * (wave - C)));
      const int ci = (64 * grp + lane) & 255;
      const int t = ci >> 4, c16 = ci & 15;
      code_off[i] = (uint32_t)(t * ts * kHeadDim + 16 * c16);
      code_base[i] = grp < 4 ? Kc : Vc;
      const uint32_t row = (grp < 4 ? kStK : kStV) + t * kRowBytesF16;
      st_off[i][0] = row + (((2 * c16) ^ tswz(t)) * 16);
      st_off[i][1] = row + (((2 * c16 + 1) ^ tswz(t)) * 16);
    }
    auto load_share = [&](int pi, int32_t entry, TeamShare<NG>& U) {
      const int nv = min(kBlockSize, (int)(tok1 - tok0) - kBlockSize * pi);
      const int32_t blk = __builtin_amdgcn_readfirstlane(entry);
      const bool in = pi >= 0 && pi < npages;
      const bool blk_ok = !paged || (blk >= 0 && blk < a.geo.num_blocks);
      if (in && !blk_ok && threadIdx.x == 0) err_flag(a.err, kErrBlockId);
      const bool ok = in && blk_ok;
      const int64_t base = paged ? ((int64_t)blk * a.geo.num_kv_heads + g) * kBlockSize
                                 : (page0 + pi) * kBlockSize * a.geo.num_kv_heads + g;
      U.ok = ok;
      // the ranges end after row nv - 1: rows past the split load as zeros
      const uint32_t rows = ok ? (uint32_t)((nv - 1) * ts + 1) : 0u;
#pragma unroll
      for (int i = 0; i < NG; ++i)
        U.code[i] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                         byte_range(code_base[i] + base * kHeadDim, rows * kHeadDim), code_off[i], 0, 0));
      if constexpr (LOADER) {
        // (on every loader wave, so that their loads count alike; only the
        // first one's lanes 0..15 have offsets inside the range)
        U.ks = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(
                                               byte_range(Ks + base * 4, rows * 8), sc_off, 0, 0));
        U.vs = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(
                                               byte_range(Vs + base * 4, rows * 8), sc_off, 0, 0));
      }
    };
    auto stage_share = [&](const TeamShare<NG>& U, int pi, uint8_t* st) {
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        *reinterpret_cast<uint4*>(st + st_off[i][0]) = i8x8_to_f16(U.code[i][0], U.code[i][1]);
        *reinterpret_cast<uint4*>(st + st_off[i][1]) = i8x8_to_f16(U.code[i][2], U.code[i][3]);
      }
      if constexpr (LOADER) {
        // scale rows and the page's valid rows (0 for a masked page) from the
        // first loader wave; the other lanes write to the dummy area
        *reinterpret_cast<u32x2_t*>(has_scale ? st + kStS + 8 * lane : lds + kDummy + 8 * lane) = U.ks;
        *reinterpret_cast<u32x2_t*>(has_scale ? st + kStS + 8 * (kBlockSize + lane)
                                              : lds + kDummy + 8 * lane) = U.vs;
        // the largest V group scale of the page's rows, as binary16 bits
        // (non-negative binary16 bits order like their values; rows past the
        // page's end and other lanes hold zeros)
        uint32_t vm = max(max(U.vs[0] & 0xffffu, U.vs[0] >> 16), max(U.vs[1] & 0xffffu, U.vs[1] >> 16));
        vm = max(vm, (uint32_t)__builtin_amdgcn_mov_dpp((int)vm, 0x128, 0xf, 0xf, false));
        vm = max(vm, (uint32_t)__builtin_amdgcn_mov_dpp((int)vm, 0x124, 0xf, 0xf, false));
        vm = max(vm, (uint32_t)__builtin_amdgcn_mov_dpp((int)vm, 0x4e, 0xf, 0xf, false));
        vm = max(vm, (uint32_t)__builtin_amdgcn_mov_dpp((int)vm, 0xb1, 0xf, 0xf, false));
        *reinterpret_cast<int2*>(wave == C && lane == 0 ? st + kStN : lds + kDummy + 8 * lane) =
            make_int2(U.ok ? min(kBlockSize, (int)(tok1 - tok0) - kBlockSize * pi) : 0, (int)vm);
      }
    };
    // (the units start as values the compiler cannot see through, so that it
    // does not fold the first steps into a prologue of their own)
    TeamShare<NG> U[NU][kPP];
#pragma unroll
    for (int k = 0; k < NU; ++k)
#pragma unroll
      for (int pp = 0; pp < kPP; ++pp) {
#pragma unroll
        for (int i = 0; i < NG; ++i) {
          u32x4_t z = {0u, 0u, 0u, 0u};
          asm volatile("" : "+v"(z));
          U[k][pp].code[i] = z;
        }
        u32x2_t z2 = {0u, 0u};
        asm volatile("" : "+v"(z2));
        U[k][pp].ks = U[k][pp].vs = z2;
        U[k][pp].ok = false;
      }
    const int nsteps = (npages + kPP - 1) / kPP;
    for (int p0 = -2 * NU;; p0 += 2 * NU) {
      int32_t ids[2 * NU][kPP];
#pragma unroll
      for (int b = 0; b < 2 * NU; ++b)
#pragma unroll
        for (int pp = 0; pp < kPP; ++pp) {
          const int q = min(max(kPP * (p0 + b + 1 + NU) + pp, 0), max(npages - 1, 0));
          ids[b][pp] = paged && npages > 0 ? trow[page0 + q] : 0;
        }
#pragma unroll
      for (int b = 0; b < 2 * NU; ++b) {
        const int ui = p0 + b;   // step: pages kPP ui .. kPP ui + kPP - 1
        if (ui >= nsteps) return;
#pragma unroll
        for (int pp = 0; pp < kPP; ++pp)
          stage_share(U[(b + 1) % NU][pp], kPP * (ui + 1) + pp,
                      lds + ((b + 1) & 1) * kStep + pp * kStage);
#pragma unroll
        for (int pp = 0; pp < kPP; ++pp)
          load_share(kPP * (ui + 1 + NU) + pp, ids[b][pp], U[(b + 1) % NU][pp]);
        body(ui, lds + (b & 1) * kStep);
        team_barrier();
      }
    }
  };

  if (wave >= C) {
    red[wave] = 0.f;
    __syncthreads();   // the Q maxima
    run_steps(std::integral_constant<int, team_groups(C, C)>{}, std::true_type{},
              [](int, const uint8_t*) {});
  } else {
    // Q^T operand of block `wave`, step j: row 16 wave + lo, head dims
    // 32 j + 8 hi .. +7 (zero beyond R); the prescale is shared by all R
    // rows, so every wave's maximum goes through LDS
    const int r = kColRows * wave + lo;
    u32x4_t qraw[8];
    float qmax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      qraw[j] = u32x4_t{0u, 0u, 0u, 0u};
      if (r < R) {
        const int64_t h = (int64_t)g * G + r % G;
        const uint16_t* qrow = a.q + (((int64_t)s * nq + r / G) * a.num_q_heads + h) * kHeadDim;
        qraw[j] = *reinterpret_cast<const u32x4_t*>(qrow + 32 * j + 8 * hi);
      }
#pragma unroll
      for (int w = 0; w < 4; ++w)
        qmax = fmaxf(qmax, fmaxf(fabsf(bf16_lo(qraw[j][w])), fabsf(bf16_hi(qraw[j][w]))));
    }
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) qmax = fmaxf(qmax, __shfl_xor(qmax, sh));
    if (lane == 0) red[wave] = qmax;
    __syncthreads();   // the Q maxima
    qmax = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) qmax = fmaxf(qmax, red[w]);
    const int qe = (int)((__float_as_uint(qmax) >> 23) & 0xFF);
    const int pe = qmax > 0.f ? min(max(268 - qe, 1), 254) : 127;
    const float qpre = __uint_as_float((uint32_t)pe << 23);
    const float cl2 = a.scale_log2 * __uint_as_float((uint32_t)(254 - pe) << 23);
    uint4 qf[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t h4[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) h4[w] = pk_f16(bf16_lo(qraw[j][w]) * qpre, bf16_hi(qraw[j][w]) * qpre);
      qf[j] = make_uint4(h4[0], h4[1], h4[2], h4[3]);
    }
    const int64_t last = qpos0 + (r < R ? r / G : nq - 1);
    // last key of this lane's row relative to the split's first token
    const int last_rel = (int)max((int64_t)-1, min(last - tok0, (int64_t)INT32_MAX));
    floatx4_t o[16], lsum = floatx4_t{0.f, 0.f, 0.f, 0.f};
    float m = kNegBig;
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    // the V^T operand for head dims 16 i .. 16 i + 15 (as vt_operand, rows in
    // the tswz layout): lane (lo, hi) gets dim 16 i + lo at tokens 4 hi .. +3
    const int vt_row = 4 * hi + (lo >> 2);
    const uint32_t vt_base = kStV + vt_row * kRowBytesF16 + 8 * (lo & 1);
    auto vt_read = [&](const uint8_t* st, int i) {
      const int chunk = 2 * i + ((lo & 3) >> 1);
      const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_short4_t*)(void*)(st + vt_base + ((chunk ^ tswz(vt_row)) * 16)));
      return __builtin_bit_cast(uint2, v);
    };

    // one step: pages A = kPP ui (staged at st) and B = A + 1 (at st + kStage),
    // one softmax over their 32 tokens, the value products on the 32-long
    // inner dimension (k order: tokens 4 hi .. 4 hi + 3 of A, then of B)
    auto compute_step = [&](int ui, const uint8_t* st) {
      if (ui < 0) return;
      float x[kPP][4];
      u32x2_t vsr[kPP][4];
      float mx = -INFINITY;
      uint32_t vsb = 0;   // largest V scale bits of the step's tokens (this lane's rows)
#pragma unroll
      for (int pp = 0; pp < kPP; ++pp) {
        const uint8_t* sp = st + pp * kStage;
        const int pi = kPP * ui + pp;
        // rows of the page inside the split, 0 for a masked page
        const int2 hdr = *reinterpret_cast<const int2*>(sp + kStN);
        const int nv = __builtin_amdgcn_readfirstlane(hdr.x);
        vsb = max(vsb, (uint32_t)__builtin_amdgcn_readfirstlane(hdr.y));
        // tokens 4 hi + e this lane's row sees: those below lim
        const int lim = min(nv, max(0, last_rel - kBlockSize * pi + 1));
        // group scales of tokens 4 hi .. 4 hi + 3 (K, then V)
        const u32x4_t* srow = reinterpret_cast<const u32x4_t*>(sp + kStS + 32 * hi);
        const u32x4_t k01 = srow[0], k23 = srow[1];
        const u32x4_t v01 = srow[8], v23 = srow[9];
        const u32x2_t ksr[4] = {{k01[0], k01[1]}, {k01[2], k01[3]}, {k23[0], k23[1]}, {k23[2], k23[3]}};
        vsr[pp][0] = u32x2_t{v01[0], v01[1]};
        vsr[pp][1] = u32x2_t{v01[2], v01[3]};
        vsr[pp][2] = u32x2_t{v23[0], v23[1]};
        vsr[pp][3] = u32x2_t{v23[2], v23[3]};
        // T_g = K_g Q_g^T per scale group
        floatx4_t tg[4];
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) tg[gg] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        const uint8_t* krow = sp + kStK + lo * kRowBytesF16;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint4 kf = *reinterpret_cast<const uint4*>(krow + (((4 * j + hi) ^ tswz(lo)) * 16));
          tg[j >> 1] = mfma_f16(kf, qf[j], tg[j >> 1]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // copy the vector elements out first: a bit cast of a vector element
          // lvalue reads the vector's first element whatever the index
          const uint32_t w01 = ksr[e].x, w23 = ksr[e].y;
          const f16x2_t s01 = __builtin_bit_cast(f16x2_t, w01);
          const f16x2_t s23 = __builtin_bit_cast(f16x2_t, w23);
          // (every term a mixed multiply-add; the score is computed on every
          // lane and the mask selects, with no branch per element)
          float v = fmaf(tg[0][e], (float)s01[0], 0.f);
          v = fmaf(tg[1][e], (float)s01[1], v);
          v = fmaf(tg[2][e], (float)s23[0], v);
          v = fmaf(tg[3][e], (float)s23[1], v);
          v *= cl2;
          asm volatile("" : "+v"(v));
          x[pp][e] = 4 * hi + e < lim ? v : -INFINITY;
          mx = fmaxf(mx, x[pp][e]);
        }
      }
      // the V-scale shift of the running maximum over the step's tokens (as
      // vscale_shift: non-negative binary16 bits order like their values)
      const float vsh = (float)max(0, (int)((vsb >> 10) & 31u) - 14);
      mx = max_over_row_groups(mx) + vsh;
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
      uint2 pop[kPP];
#pragma unroll
      for (int pp = 0; pp < kPP; ++pp) {
        pop[pp].x = pk_f16(fast_exp2(x[pp][0] - mp), fast_exp2(x[pp][1] - mp));
        pop[pp].y = pk_f16(fast_exp2(x[pp][2] - mp), fast_exp2(x[pp][3] - mp));
      }
      lsum = mfma_f16(make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u),
                      make_uint4(pop[0].x, pop[0].y, pop[1].x, pop[1].y), lsum);
      // P^T operands with the V group scales of tokens 4 hi .. 4 hi + 3
      uint4 pg[4];
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int dw = gg >> 1;
        const uint32_t sel = (gg & 1) ? 0x07060302u : 0x05040100u;
        uint32_t w[4];
#pragma unroll
        for (int pp = 0; pp < kPP; ++pp) {
          const f16x2_t p01 = __builtin_bit_cast(f16x2_t, pop[pp].x);
          const f16x2_t p23 = __builtin_bit_cast(f16x2_t, pop[pp].y);
          const f16x2_t s01 = __builtin_bit_cast(
              f16x2_t, __builtin_amdgcn_perm(vsr[pp][1][dw], vsr[pp][0][dw], sel));
          const f16x2_t s23 = __builtin_bit_cast(
              f16x2_t, __builtin_amdgcn_perm(vsr[pp][3][dw], vsr[pp][2][dw], sel));
          w[2 * pp] = __builtin_bit_cast(uint32_t, p01 * s01);
          w[2 * pp + 1] = __builtin_bit_cast(uint32_t, p23 * s23);
        }
        pg[gg] = make_uint4(w[0], w[1], w[2], w[3]);
      }
      // O^T += V^T (P o s_g)^T; 16 output dims lie in one scale group
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint2 va = vt_read(st, i), vb = vt_read(st + kStage, i);
        o[i] = mfma_f16(make_uint4(va.x, va.y, vb.x, vb.y), pg[i >> 2], o[i]);
      }
    };
    run_steps(std::integral_constant<int, team_groups(C, 0)>{}, std::false_type{}, compute_step);

    // this wave's rows: normalised partial and log2-sum-exp (l and O carry 2^kPShiftF4)
    if (r < R) {
      const int nsp = a.plan.num_splits;
      const int64_t rows_per_seq = (int64_t)nq * a.num_q_heads;
      const int64_t hh = (int64_t)(r / G) * a.num_q_heads + (int64_t)g * G + r % G;
      const int64_t slot = ((int64_t)s * rows_per_seq + hh) * nsp + split;
      const float L = lsum[0];
      float* dst = a.ws_o + slot * kHeadDim + 4 * hi;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        floatx4_t v = floatx4_t{0.f, 0.f, 0.f, 0.f};
        if (L > 0.f) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = o[i][e] / L;
        }
        *reinterpret_cast<floatx4_t*>(dst + 16 * i) = v;
      }
      if (hi == 0) a.ws_lse[slot] = L > 0.f ? (m - kPShiftF4) + __log2f(L) : -INFINITY;
    }
  }
}

int column_blocks(int rows) { return (rows + kColRows - 1) / kColRows; }

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, hipStream_t st) {
  const DecodeArgs& d = a.d;
  const int rows = a.num_queries * d.group;
  const dim3 grid(d.plan.num_splits, d.geo.num_kv_heads, d.num_seqs);
  hipError_t e;
  const bool i8 = d.dtype == 2;
  const dim3 block(64 * verify_waves(column_blocks(rows), d.dtype));
  switch (column_blocks(rows)) {
    case 1: e = i8 ? launch(verify_split_int8<1>, grid, block, 0, st, a)
                   : launch(verify_split_bf16<1>, grid, block, 0, st, a); break;
    case 2: e = i8 ? launch(verify_team_int8<2>, grid, block, 0, st, a)
                   : launch(verify_split_bf16<2>, grid, block, 0, st, a); break;
    case 3: e = i8 ? launch(verify_team_int8<3>, grid, block, 0, st, a)
                   : launch(verify_split_bf16<3>, grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  DecodeArgs m = d;
  m.num_q_heads = a.num_queries * d.num_q_heads;   // output rows [seq][query][head]
  return launch_decode_merge(m, st);
}

}  // namespace yrk
