// Internal launch interface between the C-ABI layer (capi.cpp, host
// validation) and the gfx950 kernels (*.hip).  Every launcher assumes its
// arguments were validated by the caller and only enqueues work.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace yrk {

constexpr int kHeadDim = 256;   // elements per head this build supports
constexpr int kBlockSize = 16;  // tokens per KV page
constexpr int kMaxRotaryHalf = 128;

// Launch shapes that the host planners (plan.cpp) and the kernels share.
constexpr int kAttnWaves = 4;          // waves per split-K attention workgroup
constexpr int kVerifyColRows = 16;     // query rows per MFMA column block of the verify kernels
// Waves per workgroup of the verify kernels by column blocks (1..3) and
// cache format: one workgroup per CU with two waves per SIMD where the
// registers allow; three column blocks hold 192 accumulator registers and
// leave room for one wave per SIMD (bf16), while over the INT8 cache two and
// three column blocks run as teams of 4 waves (one per column block, the
// rest loading), two per CU.
constexpr int verify_waves(int column_blocks, int32_t dtype) {
  return column_blocks <= 1 || (column_blocks == 2 && dtype != 2) ? 8 : 4;
}
constexpr int verify_wgs_per_cu(int column_blocks, int32_t dtype) {
  return column_blocks >= 2 && dtype == 2 ? 2 : 1;
}
constexpr int kPrefillGroup = 6;       // query heads per KV head of the prefill kernel
constexpr int kPrefillWaves = 4;
constexpr int kPrefillRowsPerWG = 192; // (token, head) rows per prefill workgroup: 32 tokens
constexpr uint32_t kErrBlockId = 1u;   // same bits as YRK_DEVERR_BLOCK_ID
constexpr uint32_t kErrPosition = 2u;  // same bits as YRK_DEVERR_POSITION

struct RopeArgs {
  uint16_t* x;
  int64_t num_tokens;
  int32_t num_heads;
  int32_t head_dim;
  int64_t token_stride;
  int32_t half;                    // rotary_dim / 2
  const int32_t* positions;
  uint32_t* err;                   // nullable; negative positions set kErrPosition
  double mscale;
  double inv_freq[kMaxRotaryHalf];
};
hipError_t launch_rope(const RopeArgs& a, hipStream_t s);

// Where one token row of one KV head lives.
struct KvGeometry {
  int32_t num_kv_heads;
  int32_t paged;
  int64_t num_blocks;
};

struct AppendArgs {
  KvGeometry geo;
  int32_t dtype;
  const uint16_t* k_src;
  const uint16_t* v_src;
  int64_t num_tokens;
  const int32_t* block_table;
  int64_t block_table_len;
  const int32_t* positions;
  uint32_t* err;
  void* k_dst;
  void* v_dst;
  uint8_t* k_scale_dst;
  uint8_t* v_scale_dst;
  const float* k_tensor_scale;
  const float* v_tensor_scale;
};
hipError_t launch_append(const AppendArgs& a, hipStream_t s);

// Rope and append in one pass: the new tokens' queries are roped in place
// and their keys roped on the way into the cache (rotary_dim 64 of 256).
constexpr int kFusedRopePairs = 32;
struct RopeAppendArgs {
  AppendArgs ap;             // ap.k_src holds the keys before rope
  uint16_t* q;               // nullable: [num_tokens] rows of num_q_heads heads, roped in place
  int32_t num_q_heads;
  int64_t q_token_stride;    // elements
  double mscale;
  double inv_freq[kFusedRopePairs];
  int32_t waves_per_token;   // set by launch_rope_append: 1, or 4 for a few tokens
};
hipError_t launch_rope_append(const RopeAppendArgs& a, hipStream_t s);

hipError_t launch_tensor_scale(const uint16_t* x, int64_t n, float* out, hipStream_t s);

struct DecodePlan {
  int32_t num_splits;
  int64_t tokens_per_split;  // multiple of 4 * kBlockSize
};
// Splits of units (sequence, KV head) x max_seq_len tokens into at most
// target_wgs workgroups when units allow (64-token granularity).
DecodePlan split_plan(int64_t units, int64_t max_seq_len, int64_t target_wgs);
DecodePlan plan_decode(int32_t num_seqs, int32_t num_kv_heads, int64_t max_seq_len,
                       int32_t dtype);
size_t decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, const DecodePlan& p);

struct DecodeArgs {
  KvGeometry geo;
  int32_t dtype;
  int32_t group;        // q heads per kv head
  int32_t num_q_heads;
  int32_t num_seqs;
  const uint16_t* q;
  const void* k;
  const void* v;
  const uint8_t* k_scale;
  const uint8_t* v_scale;
  const float* k_tensor_scale;
  const float* v_tensor_scale;
  const int32_t* block_tables;
  int64_t block_table_stride;
  const int32_t* seq_lens;
  int64_t max_seq_len;
  float scale_log2;     // softmax scale * log2(e)
  void* out;
  int32_t out_f32;
  float* ws_o;          // [S][Hq][splits][256]
  float* ws_lse;        // [S][Hq][splits]   (log2 domain)
  uint32_t* err;
  DecodePlan plan;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

// Device scratch of yrk_decode_attention_noalloc: a file-scope device array
// of kNoAllocScratchBytes per GPU (noalloc.hip).  device_scratch() returns
// its device address on the current device, looked up on the first call
// there and kept per device.
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
hipError_t device_scratch(void** ptr);
// The log-sum-exp merge of the split partials alone: one output row per
// (sequence, a.num_q_heads row) from a.ws_o / a.ws_lse.
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t s);

// Multi-query decode (speculative verify): num_queries consecutive queries
// per sequence, causal among themselves; the rows of one KV head's group are
// (query i, head j) = i * group + j, at most kVerifyMaxRows of them.
constexpr int kVerifyMaxRows = 48;
struct VerifyArgs {
  DecodeArgs d;           // d.num_q_heads: query heads per token
  int32_t num_queries;
  int32_t min_len;        // shorter sequences are flagged: num_queries for verify,
                          // 0 when single-query decode runs on these kernels
};
DecodePlan plan_verify(int32_t num_seqs, int32_t num_kv_heads, int32_t rows, int64_t max_seq_len,
                       int32_t dtype);
hipError_t launch_verify(const VerifyArgs& a, hipStream_t s);

struct PrefillArgs {
  KvGeometry geo;
  int32_t group;
  int32_t num_q_heads;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t num_q_tokens;
  int64_t q_start;
  const int32_t* block_table;
  int64_t block_table_len;
  float scale_log2;
  uint16_t* out;
  uint32_t* err;
  uint32_t* flags;           // one word per wave of the main kernel (workspace)
};
// Prefill launch grid: `tiles` workgroup row tiles of kPrefillRowsPerWG rows
// per KV head; with `share` > 0 the workgroups are numbered so that each XCD
// (block id mod 8) serves one KV head, `share` XCDs per head.
struct PrefillGrid {
  int32_t tiles, share;
  int64_t blocks;
};
PrefillGrid prefill_grid(int64_t num_q_tokens, int32_t num_kv_heads);
// Bytes of prefill workspace: one flag word per wave of the launch grid
// (0 when the shape is not supported; the call then fails on its own).
size_t prefill_workspace_bytes(int64_t num_q_tokens, int32_t num_q_heads);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);

}  // namespace yrk
