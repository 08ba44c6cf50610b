// Split-K decode attention over a paged bf16 or NVFP4 KV cache (gfx950).
//
// One query per sequence, GQA: the G query heads of one KV head share every
// key and value they read ([P5] "Why NVFP4 KV changes the math": 4 KV heads x
// 256; 24 query heads).  Decode time is dominated by streaming the cache
// ([P1] "Two cards are faster than one, not just bigger": each card reading
// half the KV is what made TP2 faster), so the kernel is organised around
// HBM streaming:
//
//   split phase   grid (split, kv_head, seq), 4 waves per workgroup.  A
//                 split owns a contiguous range of pages; wave w of the
//                 workgroup takes pages w, w+4, ...  For each 16-token page
//                 the wave issues all of its K and V loads at once (16 KiB
//                 for bf16: 16 x 16-byte loads per lane) and then computes.
//                 Lane l = 16 r + c handles tokens 4j + r (j < 4) of the page
//                 and head dims [8c, 8c+8) and [128+8c, 128+8c+8): every load
//                 instruction reads 4 tokens x 256 contiguous bytes.
//                 Scores: v_dot2_f32_bf16 partial dots, summed over the 16
//                 lanes of a DPP row.  Each row keeps its own online softmax
//                 (max, sum, acc[G][16] in fp32 registers); rows, then waves,
//                 are merged at the end of the split and one partial
//                 (normalised output + log-sum-exp) per query head goes to
//                 the workspace.
//   merge phase   grid (q_head, seq): log-sum-exp combination of the splits
//                 ([P3] "Limitations": the decode split policy).
//
// NVFP4 pages ([P5] "Why NVFP4 KV changes the math") are read as packed
// e2m1 codes and e4m3 scales: lane (r, c) reads, per token, the 8 code bytes
// of head dims [16c, 16c+16) and that block's scale byte, and dequantises in
// registers (the hardware fp4 -> bf16 conversion, then a bf16 dot with q and
// one scale multiply per 16 elements; the tensor scales are folded into the
// softmax scale and the output).
#include "device_common.h"
#include "yrk_internal.h"

namespace yrk {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima

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
    const int64_t blk = a.block_tables[(int64_t)s * a.block_table_stride + page];
    if (blk < 0 || blk >= a.geo.num_blocks) return false;
    *base = ((blk * a.geo.num_kv_heads + g) * kBlockSize) * row_elems;
    *tstride = row_elems;
  } else {
    *base = (page * kBlockSize * a.geo.num_kv_heads + g) * row_elems;
    *tstride = (int64_t)a.geo.num_kv_heads * row_elems;
  }
  return true;
}

// Per-row online softmax update for one page: scores sc[j][h] already in the
// log2 domain (masked tokens at -inf).  Returns the probabilities in sc.
template <int G>
__device__ __forceinline__ void softmax_update(float (&sc)[4][G], float (&m)[G], float (&l)[G],
                                               float (&acc)[G][16]) {
  bool grow = false;
  float mnew[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = fmaxf(fmaxf(sc[0][h], sc[1][h]), fmaxf(sc[2][h], sc[3][h]));
    mnew[h] = fmaxf(m[h], mx);
    grow |= mnew[h] > m[h];
  }
  if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float alpha = fast_exp2(m[h] - mnew[h]);
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[h][e] *= alpha;
      m[h] = mnew[h];
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[j][h] = fast_exp2(sc[j][h] - m[h]);
      l[h] += sc[j][h];
    }
  }
}

// End of a split: merge the 4 rows of each wave, then the 4 waves through
// LDS, and write one normalised partial + log2-sum-exp per query head.
// dim_of(e) maps accumulator slot e of lane c to its head dimension.
template <int G, typename DimOf>
__device__ __forceinline__ void finish_split(const DecodeArgs& a, int s, int g, int split,
                                             float (&m)[G], float (&l)[G], float (&acc)[G][16],
                                             DimOf dim_of) {
  __shared__ float sm_acc[kWaves][G][kHeadDim];
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_l[kWaves][G];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = fmaxf(m[h], __shfl_xor(m[h], 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float alpha = fast_exp2(m[h] - M);
    float lh = l[h] * alpha;
    lh += __shfl_xor(lh, 16);
    lh += __shfl_xor(lh, 32);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float v = acc[h][e] * alpha;
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      acc[h][e] = v;
    }
    m[h] = M;
    l[h] = lh;
  }
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sm_acc[wave][h][dim_of(c, e)] = acc[h][e];
      if (c == 0) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();
  const int nsp = a.plan.num_splits;
  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += kThreads) {
    const int h = idx / kHeadDim;
    const int d = idx % kHeadDim;
    float M = kNegBig;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sc = fast_exp2(sm_m[w][h] - M);
      L += sm_l[w][h] * sc;
      O += sm_acc[w][h][d] * sc;
    }
    const int qh = g * G + h;
    const int64_t slot = ((int64_t)s * a.num_q_heads + qh) * nsp + split;
    a.ws_o[slot * kHeadDim + d] = L > 0.f ? O / L : 0.f;
    if (d == 0) a.ws_lse[slot] = L > 0.f ? M + __log2f(L) : -INFINITY;
  }
}

template <int G>
__global__ __launch_bounds__(kThreads, 2) void decode_split_bf16(DecodeArgs a) {
  const int split = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane >> 4, c = lane & 15;

  int64_t len = a.seq_lens[s];
  if (len > a.max_seq_len) {
    if (threadIdx.x == 0 && split == 0 && g == 0) err_flag(a.err, kErrPosition);
    len = a.max_seq_len;
  }
  if (len < 0) len = 0;
  const int64_t tok0 = (int64_t)split * a.plan.tokens_per_split;
  const int64_t tok1 = min(len, tok0 + a.plan.tokens_per_split);

  float m[G], l[G], acc[G][16];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[h][e] = 0.f;
  }

  if (tok1 > tok0) {
    // q slices of this lane: dims [8c, 8c+8) and [128+8c, 128+8c+8) of each head
    uint4 qa[G][2];
    const uint16_t* qbase = a.q + ((int64_t)s * a.num_q_heads + (int64_t)g * G) * kHeadDim;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      qa[h][0] = *reinterpret_cast<const uint4*>(qbase + h * kHeadDim + 8 * c);
      qa[h][1] = *reinterpret_cast<const uint4*>(qbase + h * kHeadDim + 128 + 8 * c);
    }
    const uint16_t* K = static_cast<const uint16_t*>(a.k);
    const uint16_t* V = static_cast<const uint16_t*>(a.v);
    const int64_t page0 = tok0 / kBlockSize;
    const int64_t npages = (tok1 - tok0 + kBlockSize - 1) / kBlockSize;
    for (int64_t pi = wave; pi < npages; pi += kWaves) {
      const int64_t page = page0 + pi;
      int64_t base = 0, ts = 0;
      const bool ok = page_base(a, s, g, page, kHeadDim, &base, &ts);
      if (!ok && lane == 0) err_flag(a.err, kErrBlockId);
      uint4 kr[4][2], vr[4][2];
      if (ok) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint16_t* kp = K + base + (4 * j + r) * ts + 8 * c;
          kr[j][0] = *reinterpret_cast<const uint4*>(kp);
          kr[j][1] = *reinterpret_cast<const uint4*>(kp + 128);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint16_t* vp = V + base + (4 * j + r) * ts + 8 * c;
          vr[j][0] = *reinterpret_cast<const uint4*>(vp);
          vr[j][1] = *reinterpret_cast<const uint4*>(vp + 128);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          kr[j][0] = kr[j][1] = vr[j][0] = vr[j][1] = make_uint4(0, 0, 0, 0);
      }
      float sc[4][G];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float d = 0.f;
          d = dot2_bf16(qa[h][0].x, kr[j][0].x, d);
          d = dot2_bf16(qa[h][0].y, kr[j][0].y, d);
          d = dot2_bf16(qa[h][0].z, kr[j][0].z, d);
          d = dot2_bf16(qa[h][0].w, kr[j][0].w, d);
          d = dot2_bf16(qa[h][1].x, kr[j][1].x, d);
          d = dot2_bf16(qa[h][1].y, kr[j][1].y, d);
          d = dot2_bf16(qa[h][1].z, kr[j][1].z, d);
          d = dot2_bf16(qa[h][1].w, kr[j][1].w, d);
          sc[j][h] = d;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t tok = page * kBlockSize + 4 * j + r;
        const bool valid = ok && tok < tok1;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float d = row16_sum(sc[j][h]);
          sc[j][h] = valid ? d * a.scale_log2 : -INFINITY;
        }
      }
      softmax_update<G>(sc, m, l, acc);
      // Rows past the end of the sequence (or of a masked page) hold whatever
      // the pool holds; their weight is 0, but 0 * NaN is not, so clear them.
      if (!ok || (page + 1) * kBlockSize > tok1) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (!(ok && page * kBlockSize + 4 * j + r < tok1))
            vr[j][0] = vr[j][1] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float vf[16];
        const uint32_t w[8] = {vr[j][0].x, vr[j][0].y, vr[j][0].z, vr[j][0].w,
                               vr[j][1].x, vr[j][1].y, vr[j][1].z, vr[j][1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          vf[2 * e] = bf16_lo(w[e]);
          vf[2 * e + 1] = bf16_hi(w[e]);
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float p = sc[j][h];
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
        }
      }
    }
  }
  finish_split<G>(a, s, g, split, m, l, acc,
                  [](int cc, int e) { return e < 8 ? 8 * cc + e : 128 + 8 * cc + (e - 8); });
}

// ---- NVFP4 ----------------------------------------------------------------

// Eight e2m1 codes (one 32-bit word, element 2j in the low nibble of byte j)
// -> eight bf16 values as four packed pairs, via the gfx950 fp4 -> bf16
// conversion with unit scale.
__device__ __forceinline__ void fp4x8_to_bf16(uint32_t w, uint32_t (&out)[4]) {
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0));
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1));
  out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2));
  out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3));
}

// OCP E4M3FN scale byte (sign clear, not NaN) -> fp32, exact: normal codes
// become (1 + m/8) 2^(e-7) by placing the fields, subnormals m 2^-9.
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  const uint32_t e = (byte >> 3) & 15u, m = byte & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
}

template <int G>
__global__ __launch_bounds__(kThreads, 2) void decode_split_nvfp4(DecodeArgs a) {
  const int split = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane >> 4, c = lane & 15;

  int64_t len = a.seq_lens[s];
  if (len > a.max_seq_len) {
    if (threadIdx.x == 0 && split == 0 && g == 0) err_flag(a.err, kErrPosition);
    len = a.max_seq_len;
  }
  if (len < 0) len = 0;
  const int64_t tok0 = (int64_t)split * a.plan.tokens_per_split;
  const int64_t tok1 = min(len, tok0 + a.plan.tokens_per_split);

  float m[G], l[G], acc[G][16];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegBig;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[h][e] = 0.f;
  }

  if (tok1 > tok0) {
    const float kS = *a.k_tensor_scale;
    const float vS = *a.v_tensor_scale;
    const float qk_scale = a.scale_log2 * kS;
    // q slice of this lane: dims [16c, 16c+16) of each head
    uint4 qa[G][2];
    const uint16_t* qbase = a.q + ((int64_t)s * a.num_q_heads + (int64_t)g * G) * kHeadDim;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      qa[h][0] = *reinterpret_cast<const uint4*>(qbase + h * kHeadDim + 16 * c);
      qa[h][1] = *reinterpret_cast<const uint4*>(qbase + h * kHeadDim + 16 * c + 8);
    }
    const uint8_t* Kc = static_cast<const uint8_t*>(a.k);
    const uint8_t* Vc = static_cast<const uint8_t*>(a.v);
    const int64_t page0 = tok0 / kBlockSize;
    const int64_t npages = (tok1 - tok0 + kBlockSize - 1) / kBlockSize;
    for (int64_t pi = wave; pi < npages; pi += kWaves) {
      const int64_t page = page0 + pi;
      // rows are counted in 16-element scale blocks: 8 code bytes, 1 scale byte each
      int64_t base = 0, ts = 0;
      const bool ok = page_base(a, s, g, page, kHeadDim / 16, &base, &ts);
      if (!ok && lane == 0) err_flag(a.err, kErrBlockId);
      uint2 kc[4], vc[4];
      uint32_t ksc[4], vsc[4];
      if (ok) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t blk = base + (4 * j + r) * ts + c;
          kc[j] = *reinterpret_cast<const uint2*>(Kc + blk * 8);
          vc[j] = *reinterpret_cast<const uint2*>(Vc + blk * 8);
          ksc[j] = a.k_scale[blk];
          vsc[j] = a.v_scale[blk];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kc[j] = vc[j] = make_uint2(0, 0);
          ksc[j] = vsc[j] = 0;
        }
      }
      float sc[4][G];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t kb[8];
        fp4x8_to_bf16(kc[j].x, *reinterpret_cast<uint32_t(*)[4]>(&kb[0]));
        fp4x8_to_bf16(kc[j].y, *reinterpret_cast<uint32_t(*)[4]>(&kb[4]));
        const float bs = e4m3_to_f32(ksc[j]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float d = 0.f;
          d = dot2_bf16(qa[h][0].x, kb[0], d);
          d = dot2_bf16(qa[h][0].y, kb[1], d);
          d = dot2_bf16(qa[h][0].z, kb[2], d);
          d = dot2_bf16(qa[h][0].w, kb[3], d);
          d = dot2_bf16(qa[h][1].x, kb[4], d);
          d = dot2_bf16(qa[h][1].y, kb[5], d);
          d = dot2_bf16(qa[h][1].z, kb[6], d);
          d = dot2_bf16(qa[h][1].w, kb[7], d);
          sc[j][h] = d * bs;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t tok = page * kBlockSize + 4 * j + r;
        const bool valid = ok && tok < tok1;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float d = row16_sum(sc[j][h]);
          sc[j][h] = valid ? d * qk_scale : -INFINITY;
        }
      }
      softmax_update<G>(sc, m, l, acc);
      // Stale codes and scales decode to finite values, so p = 0 already
      // cancels them; clearing keeps masked rows exactly out of the sum.
      if (!ok || (page + 1) * kBlockSize > tok1) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (!(ok && page * kBlockSize + 4 * j + r < tok1)) {
            vc[j] = make_uint2(0, 0);
            vsc[j] = 0;
          }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float vf[16];
        uint32_t vb[8];
        fp4x8_to_bf16(vc[j].x, *reinterpret_cast<uint32_t(*)[4]>(&vb[0]));
        fp4x8_to_bf16(vc[j].y, *reinterpret_cast<uint32_t(*)[4]>(&vb[4]));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          vf[2 * e] = bf16_lo(vb[e]);
          vf[2 * e + 1] = bf16_hi(vb[e]);
        }
        const float bs = e4m3_to_f32(vsc[j]);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float p = sc[j][h] * bs;
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
        }
      }
    }
    // the V tensor scale multiplies every value: apply it once
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[h][e] *= vS;
  }
  finish_split<G>(a, s, g, split, m, l, acc, [](int cc, int e) { return 16 * cc + e; });
}

// ---- merge ------------------------------------------------------------------

// Grid (4 x q_head, seq), 256 threads: a workgroup owns 64 head dims of one
// (sequence, query head); its 4 waves each walk every 4th split, and the 4
// partial (max, sum, weighted output) triples are combined through LDS:
// out = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M), M = max_s lse_s.
// Splits that saw no token carry lse = -inf and weigh nothing.
constexpr int kMergeGroups = 4;
constexpr int kMergeDims = kHeadDim / 4;

__global__ __launch_bounds__(256) void decode_merge(DecodeArgs a) {
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
  for (int sp = grp; sp < nsp; sp += kMergeGroups) M = fmaxf(M, lse[sp]);
  float L = 0.f, O = 0.f;
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
  if (a.dtype == 0) return launch(decode_split_bf16<G>, grid, dim3(kThreads), 0, st, a);
  return launch(decode_split_nvfp4<G>, grid, dim3(kThreads), 0, st, a);
}

}  // namespace

DecodePlan plan_decode(int32_t num_seqs, int32_t num_kv_heads, int64_t max_seq_len) {
  // Enough workgroups to cover the 256 compute units twice over (two
  // resident per CU), but never fewer than one page per wave per split.
  const int64_t target_wgs = 1024;
  const int64_t unit = (int64_t)kWaves * kBlockSize;           // 64 tokens
  const int64_t units = (int64_t)num_seqs * num_kv_heads;
  const int64_t chunks = (max_seq_len + unit - 1) / unit;      // 64-token chunks
  int64_t splits = (target_wgs + units - 1) / units;
  if (splits > chunks) splits = chunks;
  if (splits < 1) splits = 1;
  int64_t per = (chunks + splits - 1) / splits;                // chunks per split
  DecodePlan p;
  p.tokens_per_split = per * unit;
  p.num_splits = (int32_t)((chunks + per - 1) / per);
  if (p.num_splits < 1) p.num_splits = 1;
  return p;
}

size_t decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, const DecodePlan& p) {
  const size_t slots = (size_t)num_seqs * num_q_heads * p.num_splits;
  const size_t o = slots * kHeadDim * sizeof(float);
  const size_t lse = slots * sizeof(float);
  return ((o + 255) / 256) * 256 + ((lse + 255) / 256) * 256;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
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
  return launch(decode_merge, dim3(4 * a.num_q_heads, a.num_seqs), dim3(256), 0, st, a);
}

}  // namespace yrk
