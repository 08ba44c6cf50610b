// Chunked causal prefill attention on bf16 matrix cores (gfx950).
//
// [P1] "Against vLLM: prefill loses, decode wins": a long prompt is prefilled
// in chunks; each chunk's queries attend causally to everything already in
// the cache plus the chunk itself.  Query i of a chunk starting at position
// P0 sees keys 0 .. P0 + i.
//
// Work decomposition
//   rows       a (token, query head) pair is one row, R = 6 x token + head
//              within the GQA group of KV head g.  A workgroup owns 128
//              consecutive rows (about 21 tokens x the 6 heads that share g),
//              so every K/V tile staged in LDS serves the whole group.
//   workgroup  4 waves, one per SIMD, so a wave may hold 512 registers (Q and
//              O for 32 rows of head dim 256 take 192 of them).
//   wave       32 rows as 2 blocks of 16.  Per 32-key tile, with
//              v_mfma_f32_16x16x32_bf16:
//                S^T[32 keys x 32 rows]  = K . Q^T        32 MFMA
//                O^T[256 x 32 rows]     += V^T . P^T      32 MFMA
//              Each K or V operand read from LDS feeds both row blocks.  The
//              S^T accumulator gives lane l (row l%16 of a block, quad q =
//              l/16) keys 16kb + 4q + i (kb < 2, i < 4).  The P^T operand of
//              the 32-key PV step needs, in lane l, operand slots 8q .. 8q+7;
//              mapping slot 8q + m to key 16(m/4) + 4q + m%4 makes them
//              exactly the lane's own scores, so P goes from the softmax into
//              the PV MFMA without a shuffle.  V^T follows the same key
//              order: LDS holds V as [key/4][dim][4 keys], one 8-byte read
//              per operand half.
//   softmax    online, per row, log2 domain.  The running maximum is raised
//              (and O rescaled) only when a tile's maximum exceeds it by more
//              than 8, so p <= 2^8 and O is rarely touched.  P is rounded to
//              bf16 for the MFMA and the row sum adds the same rounded values.
//   masking    a row at position p sees keys <= p; only tiles that reach past
//              the smallest row position of the workgroup test it per key.
//   staging    every thread loads 4 V rows x 8 dims (transposed in registers
//              into the 4-key groups) and 4 K chunks; the next tile's global
//              loads are in flight while the current tile is computed.
//   order      workgroups are numbered so that each XCD (block id mod 8) runs
//              one KV head: the tiles of that head stream through one L2.
#include "device_common.h"
#include "yrk_internal.h"

namespace yrk {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kGroup = 6;                 // query heads per KV head
constexpr int kWavesP = 4;
constexpr int kPThreads = 64 * kWavesP;   // 256
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerWG = kRowsPerWave * kWavesP;   // 128 (token, head) rows
constexpr int kRB = kRowsPerWave / 16;    // 2 row blocks per wave
constexpr int kKStride = kHeadDim + 8;    // LDS row stride of K (elements), 16 B pad
constexpr float kRescale = 8.0f;          // lazy-rescale threshold (log2 units)
constexpr float kNegBig = -1.0e30f;       // finite start for the running maximum
#ifndef YRK_PREFILL_KEYS
#define YRK_PREFILL_KEYS 32
#endif
constexpr int kPrefillKeys = YRK_PREFILL_KEYS;   // keys per tile (32 or 64)

template <int NK>
struct Smem {
  uint16_t k[NK][kKStride];               // K tile, one row per key
  uint2 vt[NK / 4][kHeadDim];             // V tile as [key/4][dim][4 keys]
};

__device__ __forceinline__ floatx4_t mfma16(const uint4& a, const uint4& b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// The pages of one key tile, resolved once per workgroup (uniform values):
// element offset of each page's first row for KV head g, or -1 when the page
// holds no visible key (past kend) or is not a valid pool page.
template <int NK>
struct TilePages {
  int64_t base[NK / kBlockSize];
  bool bad;   // a page with visible keys is missing from the pool
};

template <int NK>
__device__ __forceinline__ TilePages<NK> tile_pages(const PrefillArgs& a, int g, int64_t k0,
                                                    int64_t kend) {
  TilePages<NK> tp;
  tp.bad = false;
#pragma unroll
  for (int j = 0; j < NK / kBlockSize; ++j) {
    const int64_t key = k0 + j * kBlockSize;
    int64_t base = -1;
    if (key < kend) {
      if (a.geo.paged) {
        const int64_t p = key / kBlockSize;
        const int64_t blk = p < a.block_table_len ? (int64_t)a.block_table[p] : -1;
        if (blk >= 0 && blk < a.geo.num_blocks)
          base = (blk * a.geo.num_kv_heads + g) * kBlockSize * kHeadDim;
      } else if (key < a.geo.num_blocks * kBlockSize) {
        base = (key * a.geo.num_kv_heads + g) * kHeadDim;
      }
      if (base < 0) tp.bad = true;
    }
    tp.base[j] = base;
  }
  return tp;
}

// Element offset of key k0 + kk (0 <= kk < NK), or -1 for a key not to load.
template <int NK>
__device__ __forceinline__ int64_t tile_row(const PrefillArgs& a, const TilePages<NK>& tp,
                                            int64_t k0, int kk, int64_t kend) {
  const int64_t base = tp.base[kk / kBlockSize];
  if (base < 0 || k0 + kk >= kend) return -1;
  const int slot = kk % kBlockSize;
  return base + (int64_t)slot * (a.geo.paged ? kHeadDim : (int64_t)a.geo.num_kv_heads * kHeadDim);
}

template <int NK>
struct Stage {
  uint4 v[NK / 8];   // (NK/32) groups of 4 keys x 8 dims
  uint4 k[NK / 8];   // K chunks t + 256 i
};

// Rows of keys that are never attended (at or past kend) load as zeros: a
// masked key has weight 0, but 0 * NaN from an unwritten row would not be 0.
template <int NK>
__device__ __forceinline__ void stage_load(const PrefillArgs& a, const TilePages<NK>& tp,
                                           int64_t k0, int64_t kend, Stage<NK>& st) {
  const int t = threadIdx.x;
  const int c = t & 31;
#pragma unroll
  for (int u = 0; u < NK / 32; ++u) {
    const int kg = (t >> 5) + 8 * u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t row = tile_row<NK>(a, tp, k0, 4 * kg + j, kend);
      st.v[4 * u + j] = row >= 0 ? *reinterpret_cast<const uint4*>(a.v + row + 8 * c)
                                 : make_uint4(0, 0, 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < NK / 8; ++i) {
    const int chunk = t + kPThreads * i;
    const int64_t row = tile_row<NK>(a, tp, k0, chunk >> 5, kend);
    st.k[i] = row >= 0 ? *reinterpret_cast<const uint4*>(a.k + row + 8 * (chunk & 31))
                       : make_uint4(0, 0, 0, 0);
  }
}

template <int NK>
__device__ __forceinline__ void stage_store(const Stage<NK>& st, Smem<NK>& sm) {
  const int t = threadIdx.x;
  const int c = t & 31;
#pragma unroll
  for (int u = 0; u < NK / 32; ++u) {
    const int kg = (t >> 5) + 8 * u;
    const uint4* r = &st.v[4 * u];
    const uint32_t w0[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
    const uint32_t w1[4] = {r[1].x, r[1].y, r[1].z, r[1].w};
    const uint32_t w2[4] = {r[2].x, r[2].y, r[2].z, r[2].w};
    const uint32_t w3[4] = {r[3].x, r[3].y, r[3].z, r[3].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // word i of a row holds dims 8c + 2i (low half) and 8c + 2i + 1 (high half)
      uint2 lo, hi;
      lo.x = (w0[i] & 0xffffu) | (w1[i] << 16);
      lo.y = (w2[i] & 0xffffu) | (w3[i] << 16);
      hi.x = (w0[i] >> 16) | (w1[i] & 0xffff0000u);
      hi.y = (w2[i] >> 16) | (w3[i] & 0xffff0000u);
      sm.vt[kg][8 * c + 2 * i] = lo;
      sm.vt[kg][8 * c + 2 * i + 1] = hi;
    }
  }
#pragma unroll
  for (int i = 0; i < NK / 8; ++i) {
    const int chunk = t + kPThreads * i;
    *reinterpret_cast<uint4*>(&sm.k[chunk >> 5][8 * (chunk & 31)]) = st.k[i];
  }
}

template <int NK>
__global__ __launch_bounds__(kPThreads, 1) void prefill_kernel(PrefillArgs a, int32_t tiles,
                                                               int32_t xcd_share) {
  constexpr int KB = NK / 16;             // 16-key blocks per tile
  __shared__ Smem<NK> sm;
  // block id -> (KV head, row tile): XCD x = b % 8 serves head x / xcd_share
  const int b = blockIdx.x;
  int g, tile;
  if (xcd_share > 0) {
    const int xcd = b & 7;
    g = xcd / xcd_share;
    tile = (b >> 3) * xcd_share + xcd % xcd_share;
  } else {
    g = b % a.geo.num_kv_heads;
    tile = b / a.geo.num_kv_heads;
  }
  if (g >= a.geo.num_kv_heads || tile >= tiles) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int64_t row0 = (int64_t)tile * kRowsPerWG;   // first (token, head) row

  // rows of this lane: row block rb -> R = row0 + 32 wave + 16 rb + r16 = 6 token + head
  int64_t tok[kRB], pos[kRB];
  int head[kRB];
  bool valid[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int64_t R = row0 + kRowsPerWave * wave + 16 * rb + r16;
    tok[rb] = R / kGroup;
    head[rb] = (int)(R % kGroup);
    valid[rb] = tok[rb] < a.num_q_tokens;
    pos[rb] = a.q_start + (valid[rb] ? tok[rb] : a.num_q_tokens - 1);
  }

  // Q^T operands: lane holds, per 32-dim step ks, dims 32ks + 8q4 .. +8 of its row
  uint4 qreg[kRB][8];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const uint16_t* qrow = a.q + (tok[rb] * a.num_q_heads + g * kGroup + head[rb]) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qreg[rb][ks] = valid[rb] ? *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * q4)
                               : make_uint4(0, 0, 0, 0);
  }

  floatx4_t o[16][kRB];
#pragma unroll
  for (int d = 0; d < 16; ++d)
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) o[d][rb] = floatx4_t{};
  float m_run[kRB], l_run[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    m_run[rb] = kNegBig;
    l_run[rb] = 0.f;
  }

  const int64_t first_tok = row0 / kGroup;
  const int64_t last_tok = min((row0 + kRowsPerWG - 1) / kGroup, a.num_q_tokens - 1);
  const int64_t kend = a.q_start + last_tok + 1;    // keys [0, kend) are ever visible
  const int64_t ntiles = (kend + NK - 1) / NK;
  const int64_t diag_from = a.q_start + first_tok;   // smallest row position here

  // pages are resolved two tiles ahead, the tile's rows one tile ahead
  TilePages<NK> tp_st = tile_pages<NK>(a, g, 0, kend);   // pages of the rows held in st
  Stage<NK> st;
  stage_load<NK>(a, tp_st, 0, kend, st);
  TilePages<NK> tp_next = tile_pages<NK>(a, g, NK, kend);
  for (int64_t it = 0; it < ntiles; ++it) {
    const int64_t k0 = it * NK;
    const TilePages<NK> tp = tp_st;   // pages of the tile computed in this iteration
    const bool bad = tp.bad;
    __syncthreads();                  // the previous tile is no longer read
    stage_store<NK>(st, sm);
    __syncthreads();
    if (it + 1 < ntiles) {
      stage_load<NK>(a, tp_next, k0 + NK, kend, st);
      tp_st = tp_next;
      tp_next = tile_pages<NK>(a, g, k0 + 2 * NK, kend);
    }
    if (bad && threadIdx.x == 0) set_error(a.err, kErrBlockId);

    // S^T = K Q^T
    floatx4_t sacc[KB][kRB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) sacc[kb][rb] = floatx4_t{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint4 kop = *reinterpret_cast<const uint4*>(&sm.k[16 * kb + r16][32 * ks + 8 * q4]);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) sacc[kb][rb] = mfma16(kop, qreg[rb][ks], sacc[kb][rb]);
      }
    }

    // A key is masked if it lies past the row's position, or (rare) in a page
    // that is missing from the pool.
    const bool need_mask = k0 + NK - 1 > diag_from || k0 + NK > kend || bad;
    uint4 pop[NK / 32][kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      float sv[4 * KB];
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = sacc[kb][rb][i] * a.scale_log2;
          if (need_mask) {
            const int kk = 16 * kb + 4 * q4 + i;
            if (k0 + kk > pos[rb] || (bad && tile_row<NK>(a, tp, k0, kk, kend) < 0)) v = -INFINITY;
          }
          sv[4 * kb + i] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool raise = mx > m_run[rb] + kRescale;
      if (__builtin_amdgcn_ballot_w64(raise)) {
        const float alpha = raise ? fast_exp2(m_run[rb] - mx) : 1.0f;
        if (raise) m_run[rb] = mx;
        l_run[rb] *= alpha;
#pragma unroll
        for (int d = 0; d < 16; ++d) o[d][rb] *= alpha;
      }
      float lsum = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < NK / 32; ++s2) {
        uint32_t pb[4];
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const int e = 8 * s2 + i;
          pb[i >> 1] = pack_bf16x2(fast_exp2(sv[e] - m_run[rb]), fast_exp2(sv[e + 1] - m_run[rb]));
          lsum += bf16_lo(pb[i >> 1]) + bf16_hi(pb[i >> 1]);
        }
        pop[s2][rb] = make_uint4(pb[0], pb[1], pb[2], pb[3]);
      }
      l_run[rb] += lsum;
    }

    // O^T += V^T P^T: per 32-key step s2, operand keys {32s2 + 4q4..+3} and
    // {32s2 + 16 + 4q4..+3}; 16 tiles of 16 dims
#pragma unroll
    for (int s2 = 0; s2 < NK / 32; ++s2) {
#pragma unroll
      for (int d = 0; d < 16; ++d) {
        const int dim = 16 * d + r16;
        const uint2 a0 = sm.vt[8 * s2 + q4][dim];
        const uint2 a1 = sm.vt[8 * s2 + 4 + q4][dim];
        const uint4 vop = make_uint4(a0.x, a0.y, a1.x, a1.y);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) o[d][rb] = mfma16(vop, pop[s2][rb], o[d][rb]);
      }
    }
  }

  // row sums over the 4 quads, normalise, store dims 16d + 4q4 .. +3
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    float lt = l_run[rb];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (valid[rb]) {
      const float inv = lt > 0.f ? 1.0f / lt : 0.f;
      uint16_t* orow = a.out + (tok[rb] * a.num_q_heads + g * kGroup + head[rb]) * kHeadDim;
#pragma unroll
      for (int d = 0; d < 16; ++d) {
        uint2 w;
        w.x = pack_bf16x2(o[d][rb][0] * inv, o[d][rb][1] * inv);
        w.y = pack_bf16x2(o[d][rb][2] * inv, o[d][rb][3] * inv);
        *reinterpret_cast<uint2*>(orow + 16 * d + 4 * q4) = w;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  if (a.group != kGroup) return hipErrorInvalidValue;
  const int64_t rows = a.num_q_tokens * kGroup;
  const int32_t tiles = (int32_t)((rows + kRowsPerWG - 1) / kRowsPerWG);
  const int H = a.geo.num_kv_heads;
  int32_t share = 0;
  int64_t blocks = (int64_t)tiles * H;
  if (H <= 8 && 8 % H == 0) {
    share = 8 / H;   // XCDs per KV head
    blocks = 8 * (((int64_t)tiles + share - 1) / share);
  }
  return launch(prefill_kernel<kPrefillKeys>, dim3((unsigned)blocks), dim3(kPThreads), 0, s, a,
                tiles, share);
}

}  // namespace yrk
