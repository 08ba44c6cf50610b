// Host-side launch planning of the attention kernels: the split-K partition
// of decode and verify, the workspace each needs, and the prefill grid.
// Plain host code (no kernel in this file), shared by the C-ABI layer and
// the launchers; the launch shapes it assumes are the constants in
// yrk_internal.h that the kernels are built with.
#include "yrk_internal.h"

namespace yrk {

// Workgroups a decode launch aims for: one round of them, two waves per
// SIMD.  The bf16 cache runs the one-query verify kernel (one 8-wave
// workgroup per CU), NVFP4 one 8-wave workgroup per CU, INT8 two 4-wave
// workgroups.  Measured: more rounds were slower (two rounds of 4-wave bf16
// workgroups 1.5% at 24 q / 4 KV heads and 10% at 12 q / 2 KV heads, where a
// split then holds only 2,048 tokens; NVFP4 8-wave workgroups: 512 and
// 1,024 of them 6% and 15% slower than 256).
constexpr int64_t kTargetWgsBf16 = 256;
constexpr int64_t kTargetWgsF4 = 256;
constexpr int64_t kTargetWgsI8 = 512;
constexpr int64_t kComputeUnits = 256;

DecodePlan split_plan(int64_t units, int64_t max_seq_len, int64_t target_wgs) {
  const int64_t unit = (int64_t)kAttnWaves * kBlockSize;        // 64 tokens
  // 64-token chunks; at least one, so that an empty range still gets a
  // split (its workgroups find no page and write empty partials)
  int64_t chunks = (max_seq_len + unit - 1) / unit;
  if (chunks < 1) chunks = 1;
  // as many splits as keep units x splits within the target: workgroups
  // beyond one round would run after it, few of them and alone (15
  // sequences x 4 KV heads: 8 splits, 480 workgroups, rather than 540)
  int64_t splits = target_wgs / units;
  if (splits > chunks) splits = chunks;
  if (splits < 1) splits = 1;
  const int64_t per = (chunks + splits - 1) / splits;           // chunks per split
  DecodePlan p;
  p.tokens_per_split = per * unit;
  p.num_splits = (int32_t)((chunks + per - 1) / per);
  if (p.num_splits < 1) p.num_splits = 1;
  return p;
}

DecodePlan plan_decode(int32_t num_seqs, int32_t num_kv_heads, int64_t max_seq_len,
                       int32_t dtype) {
  const int64_t target_wgs =
      dtype == 0 ? kTargetWgsBf16 : (dtype == 1 ? kTargetWgsF4 : kTargetWgsI8);
  return split_plan((int64_t)num_seqs * num_kv_heads, max_seq_len, target_wgs);
}

// One round of workgroups over the compute units.
DecodePlan plan_verify(int32_t num_seqs, int32_t num_kv_heads, int32_t rows, int64_t max_seq_len,
                       int32_t dtype) {
  const int column_blocks = (rows + kVerifyColRows - 1) / kVerifyColRows;
  return split_plan((int64_t)num_seqs * num_kv_heads, max_seq_len,
                    kComputeUnits * verify_wgs_per_cu(column_blocks, dtype));
}

size_t decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, const DecodePlan& p) {
  const size_t slots = (size_t)num_seqs * num_q_heads * p.num_splits;
  const size_t o = slots * kHeadDim * sizeof(float);
  const size_t lse = slots * sizeof(float);
  return ((o + 255) / 256) * 256 + ((lse + 255) / 256) * 256;
}

PrefillGrid prefill_grid(int64_t num_q_tokens, int32_t num_kv_heads) {
  PrefillGrid gr;
  gr.tiles = (int32_t)((num_q_tokens * kPrefillGroup + kPrefillRowsPerWG - 1) /
                       kPrefillRowsPerWG);
  gr.share = 0;
  gr.blocks = (int64_t)gr.tiles * num_kv_heads;
  if (num_kv_heads <= 8 && 8 % num_kv_heads == 0) {
    gr.share = 8 / num_kv_heads;   // XCDs per KV head
    gr.blocks = 8 * (((int64_t)gr.tiles + gr.share - 1) / gr.share);
  }
  return gr;
}

size_t prefill_workspace_bytes(int64_t num_q_tokens, int32_t num_q_heads) {
  if (num_q_tokens <= 0 || num_q_tokens > INT32_MAX || num_q_heads <= 0 ||
      num_q_heads % kPrefillGroup)
    return 0;
  return (size_t)prefill_grid(num_q_tokens, num_q_heads / kPrefillGroup).blocks * kPrefillWaves *
         sizeof(uint32_t);
}

}  // namespace yrk
