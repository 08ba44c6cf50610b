// Chunked causal prefill attention on bf16 matrix cores (gfx950).
//
// [P1] "Against vLLM: prefill loses, decode wins": a long prompt is prefilled
// in chunks; each chunk's queries attend causally to everything already in
// the cache plus the chunk itself.  Query i of a chunk starting at position
// P0 sees keys 0 .. P0 + i.
//
// Work decomposition
//   rows       a (token, query head) pair is one row, R = 6 x token + head
//              within the GQA group of KV head g.  A workgroup owns 192
//              consecutive rows (32 tokens x the 6 heads that share g), so
//              every K/V tile in LDS serves the whole group.
//   workgroup  4 waves, one per SIMD (a wave may hold 512 registers; Q and O
//              for 48 rows of head dim 256 take 288).
//   wave       48 rows as 3 blocks of 16.  Per 32 keys, with
//              v_mfma_f32_16x16x32_bf16:
//                S^T[32 keys x 48 rows]  = K . Q^T        48 MFMA
//                O^T[256 x 48 rows]     += V^T . P^T      48 MFMA
//                row sums                 = P . ones        3 MFMA
//              The S^T accumulator gives lane l (row l%16 of a block, quad q =
//              l/16) keys 16kb + 4q + i (i < 4).  The P^T operand of a 32-key
//              PV step needs, in lane l, operand slots 8q .. 8q+7; mapping
//              slot 8q + m to key 16(m/4) + 4q + m%4 makes them exactly the
//              lane's own scores, so P goes from the softmax into the PV MFMA
//              without a shuffle.
//   LDS ring   K and V tiles arrive by direct global-to-LDS loads (16 bytes
//              per lane, no registers), NST tiles deep, so NST-1 tiles are in
//              flight while one is computed.  Rows keep the cache's natural
//              [key][256] layout with 16-byte chunk c of row r stored at
//              position c ^ (r % 16); the loads fetch the chunks in that
//              permuted order, and both operand reads below touch 16
//              different chunk positions per 16 lanes.
//                K^T operand: one 16-byte read per lane.
//                V^T operand: two ds_read_b64_tr_b16 per lane.  In each
//              16-lane group that instruction hands lane j element j%4 of the
//              8 bytes lane 4r + j/4 addressed, as its slot r; pointing lane
//              L at key 4q + L/4, dims 16d + 4(L%4) .. +3 gives lane j the
//              values of dim 16d + j at keys 4q .. 4q+3 -- the V^T operand
//              in the key order of P^T.
//   softmax    log2 domain, with a fixed maximum per row: each row takes off
//              the maximum of its first key tile (keys 0..31, which every
//              causal row sees) and keeps it for every later tile, so the
//              tile loop carries no running maximum and never rescales O.
//              The first tile adds exactly 1 to the row sum l and every p is
//              at most l; a wave whose rows end with l > 2^64 or a
//              non-finite O sets its flag word in the workspace, and a
//              second launch on the same grid recomputes those workgroups
//              with a running maximum raised lazily (by more than 8, so
//              p <= 2^8) and O rescaled; its other workgroups return at once.
//              P is rounded to bf16 for the MFMA and the row sum adds the
//              same rounded values.
//   masking    a row at position p sees keys <= p; only tiles that reach past
//              the smallest row position of the workgroup test it per key.
//              Rows that are never attended (past the chunk, or in a page
//              missing from the pool) are loaded from the query buffer
//              instead, so the masked products are 0 x finite.
//   order      workgroups are numbered so that each XCD (block id mod 8) runs
//              one KV head: the tiles of that head stream through one L2.
#include <type_traits>

#include "device_common.h"
#include "yrk_internal.h"

namespace yrk {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

constexpr int kGroup = kPrefillGroup;     // query heads per KV head
constexpr int kWavesP = kPrefillWaves;
constexpr int kPThreads = 64 * kWavesP;   // 256
constexpr int kRowsPerWave = 48;
constexpr int kRowsPerWG = kRowsPerWave * kWavesP;   // 192 (token, head) rows = 32 tokens
static_assert(kRowsPerWG == kPrefillRowsPerWG, "the planner's workgroup rows");
constexpr int kRB = kRowsPerWave / 16;    // 3 row blocks per wave
constexpr int kChunks = kHeadDim * 2 / 16;   // 16-byte chunks per row
constexpr float kRescale = 8.0f;          // lazy-rescale threshold (log2 units)
constexpr float kMaxRowSum = 0x1p64f;     // main kernel: largest row sum it accepts
constexpr float kNegBig = -1.0e30f;       // finite start for the running maximum
constexpr int kNK = 32;                   // keys per tile
constexpr int kNST = 4;                   // tiles in the LDS ring
// 32-dim score steps (0..7) after which the two load groups of a full page
// go out.  A direct load holds the issuing wave for tens of cycles; issued
// among the score products, that time overlaps the products already in the
// matrix core.  Measured per 8,192-token chunk: 188 ms with groups after
// steps 0 and 3 (188-190 ms for other pairs), 200 ms with all 8 loads ahead
// of the products, 194-200 ms with four groups of two (one more M0 write
// each), 195-198 ms with one group among the PV products.
constexpr int kLoadStep0 = 0;
constexpr int kLoadStep1 = 3;
// Score step after which the next tile's load is planned (fast_plan): its
// scalar arithmetic issues while the matrix core works.  Planned at the loop
// head, between the barrier and the first product, the chunk took 188 ms;
// planned here, 183.5 ms.
constexpr int kPlanStep = 5;

template <int NK>
struct Tile {
  uint4 kv[2][NK][kChunks];               // [K or V][key][chunk position]
};

__device__ __forceinline__ floatx4_t mfma16(const uint4& a, const uint4& b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// LDS position of logical 16-byte chunk c of ring row r is c ^ swz(r).  swz
// permutes the bits of r % 16 so that (a) 8 rows starting at a multiple of 8
// get distinct values mod 8, and the K operand reads (8 lanes, one row each,
// 16 bytes) cover all 32 banks; (b) 4 rows starting at a multiple of 4 differ
// in bits 1-2, and the transposing V reads (4 rows x 32 bytes per 16 lanes)
// land in 4 distinct 8-bank groups.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8); }

// Two floats to packed bf16 with the hardware conversion (round to nearest
// even, as f32_to_bf16 above for finite values).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){lo, hi}, b2_t));
}

// Maximum over the four lanes l, l^16, l^32, l^48 (one row's 4 quads) with
// cross-row lane swaps: each swap leaves a lane holding its own value and
// its partner's, in one order or the other.
__device__ __forceinline__ float quad_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Compiler-level fence plus the hardware workgroup barrier, without the
// memory-counter drain a full __syncthreads() implies (loads of later tiles
// must stay in flight across it).
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16 bytes per lane from global memory straight into LDS: lane l reads
// base + voff_l and its bytes land at lds_base + 16 l.  Written as inline
// assembly so that the compiler does not treat the ring as one aliasing LDS
// store stream (it would drain every tile in flight before the first LDS
// read); the ring's own vmcnt waits and barriers order the accesses.  The
// asm sets M0 (the LDS base of the direct load) and lists it as clobbered;
// the compiler warns that it does not preserve M0 across the asm, which is
// harmless here: no compiler-generated instruction in these kernels reads
// or writes M0 (checked in the generated assembly).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_base) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t ub = ((uint64_t)hi << 32) | lo;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(ub)
               : "memory", "m0");
}

// Four 1 KiB direct loads behind one M0 write: load k (0..3) reads
// base + v_k + 1024 k and lands at lds_base + 1024 k + 16 lane (the
// instruction offset moves the global and the LDS address alike).  Each M0
// write ahead of a direct load costs the wave about as much as a fifth load.
__device__ __forceinline__ void dma16x4(const void* base, uint32_t v0, uint32_t v1, uint32_t v2,
                                        uint32_t v3, uint32_t lds_base) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t ub = ((uint64_t)hi << 32) | lo;
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "global_load_lds_dwordx4 %1, %5\n\t"
      "global_load_lds_dwordx4 %2, %5 offset:1024\n\t"
      "global_load_lds_dwordx4 %3, %5 offset:2048\n\t"
      "global_load_lds_dwordx4 %4, %5 offset:3072"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(ub)
      : "memory", "m0");
}
#pragma clang diagnostic pop

typedef __attribute__((address_space(4))) const int32_t const_i32_t;

// Block ids of the two 16-key pages of a 32-key tile, read ahead of use
// through the constant address space (the compiler loads them with scalar
// loads).  Page indices past the table are clamped into it; such pages hold
// no visible key (the host checks that the table covers the chunk), so
// their ids are never used.
struct PageIds {
  int32_t id[2];
};

template <bool PAGED>
__device__ __forceinline__ PageIds load_page_ids(const PrefillArgs& a, int32_t j) {
  PageIds r{{0, 0}};
  if constexpr (PAGED) {
    const_i32_t* bt = (const_i32_t*)a.block_table;
    const int32_t last = (int32_t)min(a.block_table_len, (int64_t)INT32_MAX) - 1;
    r.id[0] = bt[min(2 * j, last)];
    r.id[1] = bt[min(2 * j + 1, last)];
  }
  return r;
}

// One wave's share of a tile load: tensor w/2 (K, then V) of page w%2 of
// tile j (keys 32j ..), moved by 8 direct loads of 1 KiB (rows 2i and 2i+1,
// lane l taking the chunk that belongs at position l % 32 of row 2i + l/32;
// the per-lane byte offsets within a page are the same for every page).  In a page that is only partly visible, rows past kend are clamped
// to the last visible one; a page with no visible row (or missing from the
// pool) is replaced by query rows: every loaded value is finite and never
// attended.  Key and page indices fit in 32 bits (the host rejects chunks
// that end past 2^31-1), so the planning stays on the scalar unit.
struct PageLoad {
  const uint16_t* src;   // first row of the page (valid when present)
  uint32_t lds0;         // LDS byte address of the page's first row in the slot
  int32_t last;          // last visible row of the page
  bool present;          // in the pool and holding visible rows
  bool full;             // present with all 16 rows visible
};

// Plans the load of tile j; returns the tile's missing-page mask (bit p: page
// p holds visible keys but is not in the pool; the same in every wave).
template <bool PAGED>
__device__ __forceinline__ uint32_t plan_tile(const PrefillArgs& a, int g, int wave, int32_t j,
                                              int32_t kend, PageIds ids, Tile<32>& t,
                                              PageLoad& pl) {
  const int32_t nb = (int32_t)min(a.geo.num_blocks, (int64_t)INT32_MAX);
  const int64_t nkeys = a.geo.num_blocks * kBlockSize;
  uint32_t missing = 0;
  int64_t base[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int32_t key = 32 * j + kBlockSize * p;
    bool ok;
    if constexpr (PAGED) {
      ok = ids.id[p] >= 0 && ids.id[p] < nb;
      base[p] = ((int64_t)ids.id[p] * a.geo.num_kv_heads + g) * (kBlockSize * kHeadDim);
    } else {
      ok = key < nkeys;
      base[p] = ((int64_t)key * a.geo.num_kv_heads + g) * kHeadDim;
    }
    const bool visible = key < kend;
    if (visible && !ok) missing |= 1u << p;
    if (!visible || !ok) base[p] = -1;
  }
  const int tensor = wave >> 1;
  const int p = wave & 1;
  const int64_t b = p ? base[1] : base[0];
  const int32_t key0 = 32 * j + kBlockSize * p;
  pl.src = (tensor ? a.v : a.k) + (b >= 0 ? b : 0);
  pl.lds0 = (uint32_t)(uintptr_t)(lds_void_t*)(void*)(&t.kv[tensor][kBlockSize * p][0]);
  pl.last = kend - 1 - key0;
  pl.present = b >= 0;
  pl.full = b >= 0 && key0 + kBlockSize <= kend;
  return missing;
}

// The common case of plan_tile, cheap enough to run among the score products
// one tile ahead: a tile whose 32 keys are all visible and whose two pages
// are in the pool (bounds checked as in plan_tile) needs only the source
// address of this wave's page, `base` + index x `step` (the wave's tensor
// and KV head folded into `base`; the index is the page id, or the first
// key of the page in the contiguous layout).  Anything else takes plan_tile.
struct FastPlan {
  const uint16_t* src;
  bool fast;
};

template <bool PAGED>
__device__ __forceinline__ FastPlan fast_plan(const PrefillArgs& a, int wave, int32_t j,
                                              int32_t kend, PageIds ids, const uint16_t* base,
                                              int64_t step) {
  FastPlan f;
  const int p = wave & 1;
  if constexpr (PAGED) {
    const uint32_t nb = (uint32_t)min(a.geo.num_blocks, (int64_t)INT32_MAX);
    const bool ok = (uint32_t)ids.id[0] < nb && (uint32_t)ids.id[1] < nb;
    f.fast = ok && 32 * j + 32 <= kend;
    f.src = base + (int64_t)(p ? ids.id[1] : ids.id[0]) * step;
  } else {
    const int64_t nkeys = a.geo.num_blocks * kBlockSize;
    f.fast = 32 * j + 32 <= kend && (int64_t)(32 * j + 32) <= nkeys;
    f.src = base + (int64_t)(32 * j + kBlockSize * p) * step;
  }
  // The values are the same in every lane; saying so keeps them (and the
  // loop-head branch on `fast`) on the scalar unit.  Left to the compiler,
  // the plan carried across iterations was taken as per-lane and the kernel
  // spilled hundreds of registers.
  // (The builtin returns a signed int: each half goes through uint32_t before
  // it is widened, or a low half with bit 31 set would fill the high half.)
  f.fast = __builtin_amdgcn_readfirstlane((uint32_t)f.fast) != 0;
  const uint64_t u = (uint64_t)f.src;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)u);
  f.src = (const uint16_t*)(((uint64_t)hi << 32) | lo);
  return f;
}

// Direct load i (0..7) of a page that is only partly visible or not present.
__device__ __forceinline__ void load_rows(const PrefillArgs& a, const PageLoad& pl, int i,
                                          uint32_t stride_b) {
  const int lane = threadIdx.x & 63;
  int row = 2 * i + (lane >> 5);
  if (pl.present) {
    if (row > pl.last) row = pl.last;
    dma16(pl.src, (uint32_t)row * stride_b + 16u * (uint32_t)((lane & 31) ^ swz(row)),
          pl.lds0 + 1024u * i);
  } else {
    dma16(a.q, 16u * (uint32_t)(lane & 31), pl.lds0 + 1024u * i);
  }
}

// Half h (rows 0-7 or 8-15) of a page with all 16 rows visible: 4 direct
// loads behind one M0 write.  `voffq` holds the per-lane offsets of a full
// page less the instruction offset each load carries.
__device__ __forceinline__ void load_full_half(const PageLoad& pl, const uint32_t (&voffq)[8],
                                               int h) {
  if (h == 0) dma16x4(pl.src, voffq[0], voffq[1], voffq[2], voffq[3], pl.lds0);
  else dma16x4(pl.src, voffq[4], voffq[5], voffq[6], voffq[7], pl.lds0 + 4096u);
}

// The 8 direct loads of a planned page.
__device__ __forceinline__ void load_page(const PrefillArgs& a, const PageLoad& pl,
                                          const uint32_t (&voffq)[8], uint32_t stride_b) {
  if (pl.full) {
    load_full_half(pl, voffq, 0);
    load_full_half(pl, voffq, 1);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) load_rows(a, pl, i, stride_b);
  }
}

template <int NK, int NST>
__device__ __forceinline__ void wait_tile(int32_t tiles_after) {
  // my loads of the tile to compute are done once at most tiles_after later
  // tiles' loads (NK/4 instructions each) are still outstanding
  constexpr int P = NK / 4;
  if (tiles_after >= 3 && NST > 3) wait_vm<3 * P>();
  else if (tiles_after >= 2 && NST > 2) wait_vm<2 * P>();
  else if (tiles_after >= 1) wait_vm<P>();
  else wait_vm<0>();
}

// FALLBACK = false: the main kernel.  Each row's maximum is fixed at the
// maximum of its first key tile (the softmax is the same for any constant
// subtracted from a row's scores; only the range of exp2 limits the choice).
// The tile loop then needs neither a running maximum nor its cross-lane
// reduction, keeps O in AGPRs and spills nothing (a spill reloaded ahead of
// the loop makes the compiler leave counter waits inside it that stall on
// the tiles in flight).  After the loop each wave checks that its rows
// stayed in range and records a flag in the workspace (one word per wave)
// when they did not.
// FALLBACK = true: launched right after on the same grid; a workgroup with
// a flag set recomputes its rows with a running maximum that is raised (and
// O rescaled) whenever a tile exceeds it by more than kRescale, and every
// other workgroup returns at once.
template <int NK, int NST, bool PAGED, bool FALLBACK>
__global__ __launch_bounds__(kPThreads, 1) void prefill_kernel(PrefillArgs a, int32_t tiles,
                                                               int32_t xcd_share) {
  static_assert(NST == 4, "ring depth (slot arithmetic assumes a power of two)");
  static_assert(NK == 32, "tile keys");
  constexpr int KB = NK / 16;             // 16-key blocks per tile
  __shared__ Tile<NK> ring[NST];
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
  if (g >= a.geo.num_kv_heads || tile >= tiles) {
    // a workgroup of the rounded-up grid with no rows: its flags read clear
    if (!FALLBACK && (threadIdx.x & 63) == 0) a.flags[4 * (int64_t)b + (threadIdx.x >> 6)] = 0;
    return;
  }
  if constexpr (FALLBACK) {
    // the same decision in every wave of the workgroup
    const uint32_t* f = a.flags + 4 * (int64_t)b;
    if ((f[0] | f[1] | f[2] | f[3]) == 0) return;
  }

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q4 = lane >> 4;
  const int64_t row0 = (int64_t)tile * kRowsPerWG;   // first (token, head) row

  // rows of this lane: row block rb -> R = row0 + 48 wave + 16 rb + r16 = 6 token + head
  int64_t tok[kRB];
  int32_t pos[kRB];                                   // positions fit in 32 bits
  int head[kRB];
  bool valid[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int64_t R = row0 + kRowsPerWave * wave + 16 * rb + r16;
    tok[rb] = R / kGroup;
    head[rb] = (int)(R % kGroup);
    valid[rb] = tok[rb] < a.num_q_tokens;
    pos[rb] = (int32_t)(a.q_start + (valid[rb] ? tok[rb] : a.num_q_tokens - 1));
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

  // Q is in registers before the ring starts: a wait the compiler sees here
  // keeps it from waiting on Q (and so on every tile in flight) inside the loop.
  __builtin_amdgcn_s_waitcnt(0);

  floatx4_t o[16][kRB];
#pragma unroll
  for (int d = 0; d < 16; ++d)
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) o[d][rb] = floatx4_t{};
  // running maximum (log2 units) and row sums; lsum[rb] = ones . P^T, so
  // every element holds the lane's row sum of the rounded P values
  float m_run[kRB];
  floatx4_t lsum[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    m_run[rb] = kNegBig;
    lsum[rb] = floatx4_t{};
  }
  const uint4 ones = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
  const float c2 = a.scale_log2;

  const int64_t first_tok = row0 / kGroup;
  const int64_t last_tok = min((row0 + kRowsPerWG - 1) / kGroup, a.num_q_tokens - 1);
  const int32_t kend = (int32_t)(a.q_start + last_tok + 1);   // keys [0, kend) are ever visible
  const int32_t ntiles = (kend + NK - 1) / NK;
  const int32_t diag_from = (int32_t)(a.q_start + first_tok);  // smallest row position here

  // per-lane byte offsets of the direct loads within a page, less the
  // instruction offset of each (see load_page; never negative)
  const uint32_t stride_b =
      2u * (uint32_t)(a.geo.paged ? kHeadDim : a.geo.num_kv_heads * kHeadDim);
  uint32_t voff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 2 * i + (lane >> 5);
    voff[i] = (uint32_t)row * stride_b + 16u * (uint32_t)((lane & 31) ^ swz(row)) -
              1024u * (uint32_t)(i & 3);
  }

  // missing-page masks of the tiles in the ring, 2 bits per slot
  uint32_t missing = 0;
  uint32_t any_missing = 0;

  // prologue: tiles 0 .. NST-2 in flight, and the page ids of tile NST-1
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
    if (s < ntiles) {
      PageLoad pl;
      missing |= plan_tile<PAGED>(a, g, wave, s, kend, load_page_ids<PAGED>(a, s), ring[s], pl)
                 << (2 * s);
      load_page(a, pl, voff, stride_b);
    }
  PageIds ids_next = load_page_ids<PAGED>(a, NST - 1);

  // V^T operand d of a tile: keys 0 .. 31, dims 16d .. +15.  Lane (r16, q4)
  // points its two transposing reads at keys 4q4 + r16/4 (+16) and dims
  // 16d + 4(r16%4) .. +3.
  const int kq = 4 * q4 + (r16 >> 2);            // key within the 16-key half, 0..15
  const int coff = (r16 & 3) >> 1;               // chunk within the 32-byte dim span
  const int boff = (r16 & 1) * 8;                // byte within the chunk
  auto read_v = [&](const Tile<NK>& t, int d) {
    const int c = 2 * d + coff;
    const char* p0 = reinterpret_cast<const char*>(&t.kv[1][kq][c ^ swz(kq)]) + boff;
    const char* p1 = reinterpret_cast<const char*>(&t.kv[1][16 + kq][c ^ swz(kq)]) + boff;
    const short4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(void*)(p0));
    const short4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)(void*)(p1));
    const uint2 w0 = __builtin_bit_cast(uint2, v0);
    const uint2 w1 = __builtin_bit_cast(uint2, v1);
    return make_uint4(w0.x, w0.y, w1.x, w1.y);
  };
  constexpr int kVAhead = 6;                     // V^T operands read ahead of their MFMAs (even, <= 16)
  uint4 vpre[kVAhead];
  auto read_v_first = [&](const Tile<NK>& t) {
#pragma unroll
    for (int d = 0; d < kVAhead; ++d) vpre[d] = read_v(t, d);
  };

  // Scores of the tile in `t` (keys k0 ..): S^T = K Q^T, kept raw (the
  // scale, > 0, is applied inside the exponent) and masked.  K operands are
  // read four 32-dim steps ahead of their MFMAs, so that LDS latency overlaps
  // the products (the compiler would otherwise wait for each read just
  // before its use).
  float sv[kRB][4 * KB];
  float mxs[kRB];
  auto scores = [&]<bool VPRE, class Hook>(const Tile<NK>& t, int32_t k0, uint32_t miss,
                                           const Tile<NK>& tv, Hook&& hook) {
    constexpr int kKAhead = 3;
    uint4 kop[8][KB];
#pragma unroll
    for (int ks = 0; ks < kKAhead; ++ks)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) kop[ks][kb] = t.kv[0][16 * kb + r16][(4 * ks + q4) ^ swz(r16)];
    __builtin_amdgcn_sched_barrier(0);
    floatx4_t sacc[KB][kRB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) sacc[kb][rb] = floatx4_t{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks + kKAhead < 8) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          kop[ks + kKAhead][kb] = t.kv[0][16 * kb + r16][(4 * (ks + kKAhead) + q4) ^ swz(r16)];
      }
      if constexpr (VPRE) {
        // the first V operands of the tile whose products follow, two per
        // step over the last kVAhead / 2 steps
        if (ks >= 8 - kVAhead / 2) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int d = 2 * (ks - (8 - kVAhead / 2)) + j;
            vpre[d] = read_v(tv, d);
          }
        }
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          sacc[kb][rb] = mfma16(kop[ks][kb], qreg[rb][ks], sacc[kb][rb]);
      hook(ks);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[rb][4 * kb + i] = sacc[kb][rb][i];
    // Masking, only on tiles that reach past the smallest row position or
    // the visible range, or hold a missing page: key 16kb + 4q4 + i is kept
    // when it is at most the row's position and its page is present.
    if (k0 + NK - 1 > diag_from || k0 + NK > kend || miss != 0) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        const int lim = pos[rb] - k0 - 4 * q4;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int limk = ((miss >> kb) & 1u) ? -1 : lim - 16 * kb;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sv[rb][4 * kb + i] = i <= limk ? sv[rb][4 * kb + i] : -INFINITY;
        }
      }
    }
  };

  // Row maxima of sv (log2 units) and P = exp2(scale S - m) in bf16, for
  // the (re)start of the pipeline below.
  auto tile_max = [&]() {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      float mx = sv[rb][0];
#pragma unroll
      for (int e = 1; e < 4 * KB; ++e) mx = fmaxf(mx, sv[rb][e]);
      mxs[rb] = quad_max(mx) * c2;
    }
  };
  auto make_p = [&](uint4 (&p)[kRB]) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const float negm = -m_run[rb];
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        w[e >> 1] = cvt_pk_bf16(fast_exp2(fmaf(sv[rb][e], c2, negm)),
                                fast_exp2(fmaf(sv[rb][e + 1], c2, negm)));
      p[rb] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  };

  // O^T += V^T P^T and the row sums (ones . P^T) for the tile in `t`, whose
  // first V operands are in vpre.  With SM, the softmax of the next tile
  // (scores in sv) runs between the products: one exponential per MFMA pair,
  // filling the cycles the matrix core is busy; pn receives its P and mxs
  // its row maxima.
  auto pv = [&]<bool SM>(const Tile<NK>& t, const uint4(&pc)[kRB], uint4(&pn)[kRB]) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) lsum[rb] = mfma16(ones, pc[rb], lsum[rb]);
    uint4 vr[kVAhead];
#pragma unroll
    for (int d = 0; d < kVAhead; ++d) vr[d] = vpre[d];
    float negm[kRB], mx[kRB], xe = 0.f;
    uint32_t w[kRB][4];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) negm[rb] = -m_run[rb];
    __builtin_amdgcn_sched_barrier(0);
    // softmax item i = (row block i / 8, score i % 8) follows product 2i
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      const uint4 vop = vr[d % kVAhead];
      if (d + kVAhead < 16) vr[d % kVAhead] = read_v(t, d + kVAhead);
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        o[d][rb] = mfma16(vop, pc[rb], o[d][rb]);
        __builtin_amdgcn_sched_barrier(0);
        const int m = d * kRB + rb;
        if constexpr (SM) {
          if (m % 2 == 0 && m / 2 < 8 * kRB) {
            const int r = m / 16, e = (m / 2) % 8;
            float x = fast_exp2(fmaf(sv[r][e], c2, negm[r]));
            // instruction selection orders pure arithmetic freely; the
            // empty asm pins this exponential to its slot between products
            asm volatile("" : "+v"(x));
            if (e & 1) w[r][e >> 1] = cvt_pk_bf16(xe, x);
            else xe = x;
            mx[r] = e ? fmaxf(mx[r], sv[r][e]) : sv[r][e];
            if (e == 7) mxs[r] = quad_max(mx[r]) * c2;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (SM) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        pn[rb] = make_uint4(w[rb][0], w[rb][1], w[rb][2], w[rb][3]);
        // P is dead on the (rare) rescale path, so the compiler would sink
        // its exponentials below the branch, out of the gaps between the
        // products; this empty use keeps them here.
        asm volatile("" ::"v"(pn[rb].x), "v"(pn[rb].y), "v"(pn[rb].z), "v"(pn[rb].w));
      }
    }
  };

  // Software pipeline over key tiles, NST deep ring, one barrier per tile.
  // Iteration it: wait for this wave's loads of tile it+1, barrier (every
  // wave's loads of tile it+1 landed, and every wave is done with tile it-1,
  // whose slot the next load reuses), start tile it+NST-1, then S(it+1) on
  // the matrix cores, then PV(it) with the softmax of tile it+1 between its
  // products.  A tile whose maximum rises past a row's running maximum by
  // more than the threshold leaves the loop after PV(it): the maximum is
  // raised, O and the row sums are rescaled and its P is recomputed; this
  // happens on the first tile and rarely after it, so O is only ever touched
  // by the MFMAs inside the loop.
  __builtin_amdgcn_s_waitcnt(0xC07F);   // pending scalar loads only (see below)
  wait_tile<NK, NST>(min(NST - 2, ntiles - 1));
  wg_barrier();
  any_missing |= missing & 3u;
  scores.template operator()<false>(ring[0], 0, missing & 3u, ring[0], [](int) {});
  tile_max();
  uint4 pcur[kRB], pnext[kRB];
  int32_t it = 0;
  if constexpr (!FALLBACK) {
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) m_run[rb] = fmaxf(mxs[rb], kNegBig);
    make_p(pcur);
    // Tile t+NST-1 is loaded in iteration t, planned among the score products
    // of iteration t-1 (fast_plan) from page ids read at the end of iteration
    // t-2; only tiles that fast_plan declines are planned at the loop head.
    const int tensor = wave >> 1;
    const uint16_t* page_base =
        (tensor ? a.v : a.k) + (int64_t)g * (PAGED ? kBlockSize * kHeadDim : kHeadDim);
    const int64_t page_step = (int64_t)a.geo.num_kv_heads * (PAGED ? kBlockSize * kHeadDim : kHeadDim);
    const uint32_t lds_wave = (uint32_t)(uintptr_t)(lds_void_t*)(void*)(
        &ring[0].kv[tensor][kBlockSize * (wave & 1)][0]);
    PageIds ids_plan = ids_next;                              // tile NST-1
    FastPlan fp = fast_plan<PAGED>(a, wave, NST - 1, kend, ids_plan, page_base, page_step);
    ids_next = load_page_ids<PAGED>(a, NST);                  // tile NST
    __builtin_amdgcn_s_waitcnt(0xC07F);   // pending scalar loads only
    for (; it + 1 < ntiles; ++it) {
      const uint32_t cslot = (uint32_t)it & (NST - 1), nslot = (uint32_t)(it + 1) & (NST - 1),
                     islot = (uint32_t)(it + NST - 1) & (NST - 1);
      wait_tile<NK, NST>(min(NST - 3, ntiles - 2 - it));
      wg_barrier();
      // the page ids read at the end of the last iteration: waited for here,
      // where no LDS read is in flight
      __builtin_amdgcn_s_waitcnt(0xC07F);
      // load tile it+NST-1 into the slot tile it-1 used; a full page's 8
      // loads go out in two groups of four among the score products below
      const bool load = it + NST - 1 < ntiles;
      PageLoad pl;
      if (load) {
        uint32_t m = 0;
        if (fp.fast) {
          pl.src = fp.src;
          pl.lds0 = lds_wave + islot * (uint32_t)sizeof(Tile<NK>);
          pl.present = true;
          pl.full = true;
        } else {
          m = plan_tile<PAGED>(a, g, wave, it + NST - 1, kend, ids_plan, ring[islot], pl);
          if (!pl.full) load_page(a, pl, voff, stride_b);
        }
        missing = (missing & ~(3u << (2 * islot))) | (m << (2 * islot));
      }
      const uint32_t miss = (missing >> (2 * nslot)) & 3u;
      any_missing |= miss;
      const PageIds ids_new = ids_next;
      scores.template operator()<true>(ring[nslot], (it + 1) * NK, miss, ring[cslot], [&](int ks) {
        if (load && pl.full && (ks == kLoadStep0 || ks == kLoadStep1))
          load_full_half(pl, voff, ks == kLoadStep0 ? 0 : 1);
        if (ks == kPlanStep) {
          ids_plan = ids_new;
          fp = fast_plan<PAGED>(a, wave, it + NST, kend, ids_new, page_base, page_step);
        }
      });
      pv.template operator()<true>(ring[cslot], pcur, pnext);
      ids_next = load_page_ids<PAGED>(a, it + NST + 1);   // planned in the next iteration
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) pcur[rb] = pnext[rb];
    }
  } else {
  for (;;) {
    float alpha[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const bool raise = mxs[rb] > m_run[rb] + kRescale;
      alpha[rb] = raise ? fast_exp2(m_run[rb] - mxs[rb]) : 1.0f;
      if (raise) m_run[rb] = mxs[rb];
      lsum[rb] *= alpha[rb];
    }
    // one accumulator at a time, so that O never needs VGPR copies at once
#pragma unroll
    for (int d = 0; d < 16; ++d)
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        o[d][rb] *= alpha[rb];
        __builtin_amdgcn_sched_barrier(0);
      }
    make_p(pcur);
    // Pending scalar loads on entry would make every LDS wait in the loop a
    // full one: wait for them here (lgkmcnt only; tiles stay in flight).
    __builtin_amdgcn_s_waitcnt(0xC07F);
    bool raised = false;
    for (; it + 1 < ntiles; ++it) {
      const uint32_t cslot = (uint32_t)it & (NST - 1), nslot = (uint32_t)(it + 1) & (NST - 1),
                     islot = (uint32_t)(it + NST - 1) & (NST - 1);
      wait_tile<NK, NST>(min(NST - 3, ntiles - 2 - it));
      wg_barrier();
      // plan tile it+NST-1 into the slot tile it-1 used; a full page's 8
      // loads go out in two groups of four among the score products below
      const bool load = it + NST - 1 < ntiles;
      PageLoad pl;
      if (load) {
        const uint32_t m = plan_tile<PAGED>(a, g, wave, it + NST - 1, kend, ids_next,
                                            ring[islot], pl);
        missing = (missing & ~(3u << (2 * islot))) | (m << (2 * islot));
        if (!pl.full) load_page(a, pl, voff, stride_b);
      }
      const uint32_t miss = (missing >> (2 * nslot)) & 3u;
      any_missing |= miss;
      scores.template operator()<true>(ring[nslot], (it + 1) * NK, miss, ring[cslot], [&](int ks) {
        if (load && pl.full && (ks == kLoadStep0 || ks == kLoadStep1))
          load_full_half(pl, voff, ks == kLoadStep0 ? 0 : 1);
      });
      pv.template operator()<true>(ring[cslot], pcur, pnext);
      ids_next = load_page_ids<PAGED>(a, it + NST);   // for the next iteration's load
      bool r = false;
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) r |= mxs[rb] > m_run[rb] + kRescale;
      if (__builtin_amdgcn_ballot_w64(r)) {
        raised = true;
        ++it;
        break;
      }
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) pcur[rb] = pnext[rb];
    }
    if (!raised) break;
  }
  }
  read_v_first(ring[(uint32_t)it & (NST - 1)]);
  pv.template operator()<false>(ring[(uint32_t)it & (NST - 1)], pcur, pnext);

  if (any_missing && threadIdx.x == 0) set_error(a.err, kErrBlockId);

  if constexpr (!FALLBACK) {
    // With the maximum fixed, every p of a row is at most its row sum l (the
    // first tile's maximum contributes exactly 1 and no p is negative): if l
    // <= 2^64 and O is finite, no step overflowed and 1/l is a normal number,
    // so the result is as accurate as with a running maximum.  Otherwise
    // (scores far above the first tile's, or non-finite inputs) the wave is
    // flagged and the second launch recomputes its workgroup.
    bool bad = false;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      bool rbad = !(lsum[rb][0] <= kMaxRowSum);
#pragma unroll
      for (int d = 0; d < 16; ++d)
#pragma unroll
        for (int e = 0; e < 4; ++e) rbad |= !__builtin_isfinite(o[d][rb][e]);
      bad |= valid[rb] && rbad;
    }
    const bool flagged = __builtin_amdgcn_ballot_w64(bad) != 0;
    if (lane == 0) a.flags[4 * (int64_t)b + wave] = flagged ? 1u : 0u;
  }

  // normalise by the row sum and store dims 16d + 4q4 .. +3
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const float lt = lsum[rb][0];
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
  const PrefillGrid gr = prefill_grid(a.num_q_tokens, a.geo.num_kv_heads);
  auto main_kernel = a.geo.paged ? prefill_kernel<kNK, kNST, true, false>
                                 : prefill_kernel<kNK, kNST, false, false>;
  auto fallback = a.geo.paged ? prefill_kernel<kNK, kNST, true, true>
                              : prefill_kernel<kNK, kNST, false, true>;
  hipError_t e = launch(main_kernel, dim3((unsigned)gr.blocks), dim3(kPThreads), 0, s, a,
                        gr.tiles, gr.share);
  if (e != hipSuccess) return e;
  return launch(fallback, dim3((unsigned)gr.blocks), dim3(kPThreads), 0, s, a, gr.tiles,
                gr.share);
}

}  // namespace yrk
