/*
 * yrk.h -- C ABI of libyrk: YaRN-roped, GQA, paged long-context attention
 * for AMD Instinct MI355X (gfx950).
 *
 * One data-parallel hot path: rotate queries and keys with a YaRN-stretched
 * rotary table, append keys and values to a paged bf16, NVFP4 or INT8 KV cache,
 * and run split-K decode attention and chunked causal prefill attention over
 * that cache.
 *
 * Pages the definitions come from (cited by title and section):
 *   [P1] "A 1,048,576-token context on two RTX 5090s: forking a C++ inference
 *        engine for tensor-parallel and YaRN" (portfolio-site-axx.pages.dev)
 *   [P3] "NInfer -- Windows 11 TP2 fork" README (git.onestrm.cn mirror)
 *   [P5] "262,144 Tokens on One RTX 5090: Qwen3.8-27B with an NVFP4 KV Cache
 *        That Actually Works" (stondo.github.io)
 *
 * Conventions for every entry point:
 *   - Pointers named *_dev are device pointers; everything else is host.
 *   - The caller owns every buffer.  The library allocates nothing and keeps
 *     no mutable global state; calls are thread-safe.
 *   - Work is enqueued on `stream` and is asynchronous; device faults surface
 *     at the caller's next synchronisation.
 *   - Return value: YRK_OK (0) or a negative status.  Every error that the
 *     host can detect is returned before anything is enqueued, so a failed
 *     call writes nothing.  Errors only the device can see (a block id
 *     outside the pool, a position beyond the block table) set bits in the
 *     optional device word *dev_error_word (bitwise OR of YRK_DEVERR_*); the
 *     offending write or read is skipped (a skipped key is masked out).
 *   - bf16 is the bit pattern of IEEE binary32's upper 16 bits.
 */
#ifndef YRK_H
#define YRK_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define YRK_OK 0
#define YRK_EINVAL (-1)  /* null pointer, bad shape, parameter outside its domain */
#define YRK_ERANGE (-2)  /* a length or position beyond what the buffers / table can hold */
#define YRK_ENOTSUP (-3) /* a shape or dtype this build has no kernel for */
#define YRK_ENOSPC (-4)  /* workspace smaller than the size query returned */
#define YRK_EDEVICE (-5) /* the HIP runtime refused a launch */

#define YRK_DEVERR_BLOCK_ID 1u  /* a block-table entry outside [0, num_blocks) */
#define YRK_DEVERR_POSITION 2u  /* a position < 0 or beyond the table / capacity */

#define YRK_KV_BF16 0
#define YRK_KV_NVFP4 1
#define YRK_KV_INT8 2

#define YRK_OUT_BF16 0
#define YRK_OUT_F32 1

/*
 * YaRN parameters ([P1] "YaRN, and matching what vLLM actually does";
 * [P3] "YaRN reference and drift guard" and "Usage").
 *   rope_theta               rotary base (1e7 for the workload)
 *   head_dim                 elements per head (256)
 *   rotary_dim               leading dimensions that rotate (64); even, <= head_dim
 *   factor                   YaRN scale s; finite, in [1, 64]; 1 = plain RoPE
 *   original_max_position    trained window (262,144)
 *   correction_max_position  length used for the correction range; 0 = the
 *                            original window (the paper's formula, range
 *                            (14, 22)); 4 x original reproduces the deployed
 *                            range (16, 24)
 *   beta_fast, beta_slow     turn counts bounding the correction range (32, 1)
 *   mscale                   attention temperature on cos/sin; <= 0 derives
 *                            0.1 ln s + 1 (1 when s == 1)
 * Positions beyond original x factor are allowed: the window limit is a
 * serving rule, not a limit of the arithmetic.
 */
typedef struct yrk_yarn_params {
  double rope_theta;
  int32_t head_dim;
  int32_t rotary_dim;
  double factor;
  int64_t original_max_position;
  int64_t correction_max_position;
  double beta_fast;
  double beta_slow;
  double mscale;
} yrk_yarn_params;

/*
 * One layer's KV cache, in caller-owned device memory.
 *
 * paged = 1 (the HND page layout of [P5] "Validation before vibes"; pages
 * of [P1] "Things that bit me"; one shared pool, [P3] "Current limits"):
 *   bf16:  k, v          [num_blocks][num_kv_heads][block_size][head_dim]       bf16
 *   NVFP4: k, v          [num_blocks][num_kv_heads][block_size][head_dim / 2]   packed e2m1
 *          k_scale, v_scale [num_blocks][num_kv_heads][block_size][head_dim / 16] e4m3
 *   INT8:  k, v          [num_blocks][num_kv_heads][block_size][head_dim]       int8
 *          k_scale, v_scale [num_blocks][num_kv_heads][block_size][head_dim / 64] binary16
 *   Logical token n of a sequence is block table[n / block_size], slot
 *   n % block_size.
 * paged = 0 (contiguous): the same rows as [capacity][num_kv_heads][row];
 *   capacity = num_blocks * block_size; token n is row n; no block table.
 *
 * NVFP4 element codes: sign bit | 3-bit e2m1 magnitude; element 2j in the
 * low nibble of byte j of a row.  One OCP E4M3FN scale per 16 consecutive
 * head-dim elements.  k_tensor_scale_dev / v_tensor_scale_dev point to the
 * fp32 tensor scale S of each tensor (device memory, one float).  The
 * dequantised value is e2m1(code) * e4m3(scale) * S.
 *
 * INT8 group-64 ([P3] memory table, [P1] "And the memory picture": the
 * deployed 1M-token format, 16.5 KiB per token per device with the scale
 * planes, which fixes 2-byte scales): one binary16 scale per 64 consecutive
 * head-dim elements of a row, s = RNE(max |x| / 127) saturating at 65504,
 * and two's-complement codes clamp(RNE(x / s), -127, 127) (0 when s is 0);
 * the dequantised value is code * s.  The rounding rules are this library's
 * reading.  The tensor-scale pointers are not used.
 *
 * This build supports head_dim 256 and block_size 16.  k, v and (NVFP4,
 * INT8) k_scale, v_scale must be 16-byte aligned, the tensor-scale pointers
 * 4-byte aligned (YRK_EINVAL otherwise, from every entry point).
 */
typedef struct yrk_kv_layer {
  int32_t dtype;          /* YRK_KV_BF16, YRK_KV_NVFP4 or YRK_KV_INT8 */
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int64_t num_blocks;
  int32_t paged;
  int32_t reserved;       /* must be 0 */
  void* k;
  void* v;
  void* k_scale;
  void* v_scale;
  const float* k_tensor_scale_dev;
  const float* v_tensor_scale_dev;
} yrk_kv_layer;

/*
 * yrk_yarn_table -- host only.  The rotary inverse-frequency table of [P1]
 * "YaRN, and matching what vLLM actually does": theta_i = rope_theta^(-2i/d)
 * blended by a linear ramp over the correction range [low, high] between
 * theta_i (below low) and theta_i / s (from high up), with
 * corr(r) = d ln(L / (2 pi r)) / (2 ln rope_theta), low = floor(corr(beta_fast)),
 * high = ceil(corr(beta_slow)), clamped to [0, d-1].
 *   inv_freq_out   rotary_dim / 2 doubles (nullable)
 *   mscale_out, corr_low_out, corr_high_out   (each nullable)
 * Errors: YRK_EINVAL for null params or a parameter outside its domain.
 */
int yrk_yarn_table(const yrk_yarn_params* params, double* inv_freq_out, double* mscale_out,
                   int32_t* corr_low_out, int32_t* corr_high_out);

/*
 * yrk_yarn_rope_apply -- rotate in place the first rotary_dim elements of
 * each head of x: pair (i, i + rotary_dim/2) turns by position * inv_freq_i,
 * cos and sin scaled by mscale ([P1] "YaRN, and matching what vLLM actually
 * does": mscale sits inside the rope on the rotary dimensions only; [P3]
 * "YaRN reference and drift guard": 64 of 256 dimensions).  The angle and
 * the rotation are computed in fp64 and rounded once to bf16 (RNE);
 * elements from rotary_dim on are not touched.
 *   x_dev          bf16, token t head h at x + t*token_stride + h*head_dim
 *   num_tokens     >= 0 (0 is a no-op)
 *   num_heads      > 0, num_heads*head_dim <= token_stride
 *   positions_dev  int32 [num_tokens], each >= 0; a token with a negative
 *                  position is left unchanged and sets YRK_DEVERR_POSITION
 *   dev_error_word nullable device uint32 (see the conventions above)
 * Errors: YRK_EINVAL (null, bad params/shape), YRK_ENOTSUP (rotary_dim > 256;
 * refused before the table is built, whatever head_dim allows).
 */
int yrk_yarn_rope_apply(const yrk_yarn_params* params, void* x_dev, int64_t num_tokens,
                        int32_t num_heads, int64_t token_stride, const int32_t* positions_dev,
                        uint32_t* dev_error_word, hipStream_t stream);

/*
 * yrk_nvfp4_tensor_scale -- S = fl32(amax / (6 * 448)) of n bf16 values,
 * amax = max |x|; amax == 0 gives S = 1.  Written to *scale_out_dev (one
 * float, device).  This is the per-tensor scale of the NVFP4 format ([P5]
 * "Why NVFP4 KV changes the math"; the tensor scale chosen as amax / (6*448)).
 * Errors: YRK_EINVAL (null, n < 0).
 */
int yrk_nvfp4_tensor_scale(const void* x_dev, int64_t n, float* scale_out_dev,
                           hipStream_t stream);

/*
 * yrk_kv_append_quantize -- write num_tokens new keys and values of one
 * sequence into the cache.  Token t (k/v rows [num_tokens][num_kv_heads]
 * [head_dim] bf16, contiguous) goes to logical position positions_dev[t].
 *   bf16 cache:  an exact copy.
 *   NVFP4 cache: per 16-element block, scale = RNE_e4m3(max|x| / (6 S)),
 *                saturating at 448; codes = sign | RNE_e2m1(|x| / (e4m3(scale) S)),
 *                ties to the even code, saturating at 6 ([P5] "Why NVFP4 KV
 *                changes the math").  The decisions are exact: they equal
 *                rounding the exact real quotients.
 *   INT8 cache:  per 64-element group, scale = RNE_binary16(max|x| / 127),
 *                saturating at 65504; codes = clamp(RNE(x / scale), -127,
 *                127), 0 for a zero scale (the reading stated at
 *                yrk_kv_layer).  Both quotients are fp64 divisions rounded
 *                once, which equals rounding the exact quotients.
 *   block_table_dev   int32 [block_table_len] (paged); NULL for contiguous
 *   dev_error_word    nullable device uint32; positions outside the table or
 *                     capacity, or table entries outside the pool, set a bit
 *                     and that token is skipped.
 * Errors: YRK_EINVAL, YRK_ENOTSUP (layout other than head_dim 256 / block 16).
 */
int yrk_kv_append_quantize(const yrk_kv_layer* layer, const void* k_dev, const void* v_dev,
                           int64_t num_tokens, const int32_t* block_table_dev,
                           int64_t block_table_len, const int32_t* positions_dev,
                           uint32_t* dev_error_word, hipStream_t stream);

/*
 * yrk_rope_append -- one pass for the new tokens of a step: their queries
 * are roped in place and their keys roped on the way into the cache (then
 * copied or quantised as yrk_kv_append_quantize does), values appended
 * unroped.  The results are bit-identical to yrk_yarn_rope_apply on q and
 * on k followed by yrk_kv_append_quantize; the pass saves writing and
 * re-reading the roped keys and one launch per tensor ([P1] "YaRN, and
 * matching what vLLM actually does": mscale on cos/sin inside the rope, on
 * the rotary dimensions only).  Token t's query and key share position
 * positions_dev[t] (a decode step's query and its own key; the queries of
 * a verify round and their keys).
 *   params           YaRN parameters; this pass needs head_dim 256 and
 *                    rotary_dim 64 (yrk_yarn_rope_apply takes others)
 *   q_dev            nullable: bf16 [num_tokens] rows of num_q_heads heads
 *                    of head_dim, q_token_stride elements apart (a multiple
 *                    of 4, at least num_q_heads * head_dim), 8-byte aligned;
 *                    roped in place whatever the table says, except for a
 *                    negative position (left unchanged, flagged)
 *   k_dev, v_dev     bf16 [num_tokens][num_kv_heads][head_dim], contiguous,
 *                    16-byte aligned, keys not yet roped; not modified
 *   block_table_dev  int32 [block_table_len] (paged); NULL for contiguous
 *   dev_error_word   nullable; positions outside the table or capacity, or
 *                    table entries outside the pool, set a bit and that
 *                    token's key and value are skipped
 * Errors: YRK_EINVAL (parameters as for yrk_yarn_rope_apply, nulls, shapes,
 * alignment), YRK_ENOTSUP (head_dim or rotary_dim other than 256 / 64, or
 * a layout other than head_dim 256 / block 16).
 */
int yrk_rope_append(const yrk_kv_layer* layer, const yrk_yarn_params* params, void* q_dev,
                    int32_t num_q_heads, int64_t q_token_stride, const void* k_dev,
                    const void* v_dev, int64_t num_tokens, const int32_t* block_table_dev,
                    int64_t block_table_len, const int32_t* positions_dev,
                    uint32_t* dev_error_word, hipStream_t stream);

/*
 * yrk_decode_workspace_size -- bytes of device workspace that
 * yrk_decode_attention needs for these sizes (the split partials: per
 * sequence, query head and split, head_dim fp32 plus one fp32 log-sum-exp).
 * Returns 0 for invalid sizes.
 */
size_t yrk_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int64_t max_seq_len);

/*
 * yrk_decode_attention -- one query per sequence attends to that sequence's
 * seq_lens[s] cached tokens (logical positions 0 .. seq_lens[s]-1; the
 * query's own key is not among them).  Query head h reads KV head
 * h / (num_q_heads / num_kv_heads).  Logits are softmax_scale * <q, k>
 * (0 selects 1/sqrt(head_dim); YaRN adds no attention-level factor, [P1]
 * "YaRN, and matching what vLLM actually does").  The cache is split into
 * token ranges processed in parallel across compute units and merged by
 * log-sum-exp ([P3] "Limitations": the decode split policy).
 * seq_lens[s] == 0 gives a zero output row (max_seq_len 0 is allowed).
 * Over a bf16 cache both products run on the matrix cores (the verify
 * kernels with one query, whose P keeps 16 significant bits).  Over an
 * NVFP4 cache the keys and values are dequantised to fp16 exactly for the
 * matrix cores.  Over an
 * INT8 cache the codes enter the matrix cores as exact fp16 integers: each
 * scale group's partial key products are scaled in fp32, and the value
 * scales multiply the (fp16) attention weights, so no dequantised value is
 * ever rounded.
 *   q_dev            bf16 [num_seqs][num_q_heads][head_dim] (already roped)
 *   block_tables_dev int32 [num_seqs][block_table_stride] (paged); NULL for
 *                    contiguous (num_seqs must then be 1)
 *   seq_lens_dev     int32 [num_seqs], each in [0, max_seq_len]; larger values
 *                    are clamped to max_seq_len and flagged
 *   out_dev          [num_seqs][num_q_heads][head_dim], bf16 or fp32 (out_dtype)
 *   workspace_dev    >= yrk_decode_workspace_size(...) bytes, 16-byte aligned
 *   dev_error_word   nullable; see the conventions above
 * Errors: YRK_EINVAL, YRK_ERANGE (max_seq_len beyond table or capacity),
 * YRK_ENOTSUP (head_dim != 256, group size not in {1,2,3,4,6}),
 * YRK_ENOSPC.
 */
int yrk_decode_attention(const yrk_kv_layer* layer, const void* q_dev, int32_t num_seqs,
                         int32_t num_q_heads, const int32_t* block_tables_dev,
                         int64_t block_table_stride, const int32_t* seq_lens_dev,
                         int64_t max_seq_len, float softmax_scale, void* out_dev,
                         int32_t out_dtype, void* workspace_dev, size_t workspace_bytes,
                         uint32_t* dev_error_word, hipStream_t stream);

/*
 * yrk_decode_attention_noalloc -- yrk_decode_attention without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * split partials go to a device array inside the library of
 * YRK_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the library runs on
 * holds until the process ends; the call allocates nothing.  The array's
 * address on a device is looked up on the first call made with that device
 * current, and every later call on that device uses it; the caller's stream
 * must belong to the current device.  Calls that overlap on one GPU (other
 * streams, other threads) share the array and race: serialise them.
 * Arguments, results and errors are those of yrk_decode_attention, plus
 * YRK_ENOSPC when the shapes need more than YRK_NOALLOC_SCRATCH_BYTES of
 * partials (yrk_decode_workspace_size() > the scratch size; 16 MiB covers,
 * e.g., one sequence of any length at 24 q / 4 KV heads, or 15 sequences),
 * and YRK_EDEVICE when the array's address cannot be looked up.
 */
#define YRK_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int yrk_decode_attention_noalloc(const yrk_kv_layer* layer, const void* q_dev, int32_t num_seqs,
                                 int32_t num_q_heads, const int32_t* block_tables_dev,
                                 int64_t block_table_stride, const int32_t* seq_lens_dev,
                                 int64_t max_seq_len, float softmax_scale, void* out_dev,
                                 int32_t out_dtype, uint32_t* dev_error_word,
                                 hipStream_t stream);

/*
 * yrk_verify_workspace_size -- bytes of device workspace that
 * yrk_verify_attention needs for these shapes (the split partials of every
 * (sequence, query, query head)); 0 for invalid sizes.
 */
size_t yrk_verify_workspace_size(int32_t num_seqs, int32_t num_queries, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int64_t max_seq_len);

/*
 * yrk_verify_attention -- multi-query decode for speculative verify: the
 * last num_queries cached tokens of each sequence (the last accepted token
 * and the drafted ones) attend to the cache at once, causally among
 * themselves ([P1] "Things that bit me", [P3] "Limitations": a verify round
 * evaluates K + 1 query columns; [P3] "Usage": 1 to 5 draft tokens).
 * seq_lens[s] counts the sequence's cached tokens including those
 * num_queries, whose keys and values must be appended before the call;
 * query i sits at position seq_lens[s] - num_queries + i and attends to keys
 * 0 .. seq_lens[s] - num_queries + i.  Query head h reads KV head
 * h / (num_q_heads / num_kv_heads); logits are softmax_scale * <q, k> (0
 * selects 1/sqrt(head_dim)).  The split-K plan and the log-sum-exp merge are
 * those of yrk_decode_attention.  Over a bf16 cache both products run on
 * bf16 matrix cores with fp32 accumulation, and the attention weights enter
 * the value product as two bf16 terms (16 significant bits).  Over an INT8
 * cache the codes enter fp16 matrix cores as exact integers and the group
 * scales are applied as in yrk_decode_attention.
 *   q_dev            bf16 [num_seqs][num_queries][num_q_heads][head_dim]
 *                    (already roped at the queries' positions), 16-byte aligned
 *   block_tables_dev int32 [num_seqs][block_table_stride] (paged); NULL for
 *                    contiguous (num_seqs must then be 1)
 *   seq_lens_dev     int32 [num_seqs], each in [num_queries, max_seq_len];
 *                    larger values are clamped to max_seq_len and smaller
 *                    ones leave the queries at negative positions with zero
 *                    rows, both flagged (YRK_DEVERR_POSITION)
 *   out_dev          [num_seqs][num_queries][num_q_heads][head_dim], bf16 or
 *                    fp32 (out_dtype)
 *   workspace_dev    >= yrk_verify_workspace_size(...) bytes, 16-byte aligned
 *   dev_error_word   nullable; see the conventions above
 * Errors: YRK_EINVAL, YRK_ERANGE (max_seq_len beyond table or capacity),
 * YRK_ENOTSUP (an NVFP4 cache, head_dim != 256, group size not in
 * {1,2,3,4,6}, or more than 48 query rows per KV head:
 * num_queries * num_q_heads / num_kv_heads > 48), YRK_ENOSPC.
 */
int yrk_verify_attention(const yrk_kv_layer* layer, const void* q_dev, int32_t num_seqs,
                         int32_t num_queries, int32_t num_q_heads,
                         const int32_t* block_tables_dev, int64_t block_table_stride,
                         const int32_t* seq_lens_dev, int64_t max_seq_len, float softmax_scale,
                         void* out_dev, int32_t out_dtype, void* workspace_dev,
                         size_t workspace_bytes, uint32_t* dev_error_word, hipStream_t stream);

/*
 * yrk_prefill_workspace_size -- bytes of device workspace that
 * yrk_prefill_attention needs for num_q_tokens queries of num_q_heads heads
 * (GQA group 6): one 32-bit word per wave of its launch grid, 16 bytes per
 * 192 (token, head) rows rounded up to the XCD grid.  0 for an empty chunk or
 * an unsupported head_dim.
 */
size_t yrk_prefill_workspace_size(int64_t num_q_tokens, int32_t num_q_heads, int32_t head_dim);

/*
 * yrk_prefill_attention -- causal attention of one chunk of num_q_tokens
 * queries of one sequence at positions q_start_position .. +num_q_tokens-1
 * over that sequence's cache, whose tokens 0 .. q_start_position +
 * num_q_tokens - 1 must already be appended (the chunk's own keys
 * included).  Query i attends to keys 0 .. q_start_position + i
 * ([P1] "Against vLLM: prefill loses, decode wins": prompts are prefilled in
 * chunks; the chunk attends causally).  QK^T and PV run on bf16 matrix cores
 * with fp32 accumulation.
 *   q_dev        bf16 [num_q_tokens][num_q_heads][head_dim] (already roped)
 *   block_table_dev  int32 [block_table_len]; NULL for contiguous
 *   out_dev      bf16 [num_q_tokens][num_q_heads][head_dim]
 *   workspace_dev  device memory of at least yrk_prefill_workspace_size()
 *                bytes, 4-byte aligned, owned by the caller; the call writes
 *                it (no initial contents needed) and reads it back within the
 *                same stream.  The first launch subtracts from each row the
 *                maximum of its first 32 keys throughout; a wave whose row
 *                sums end above 2^64, or whose accumulators are not finite,
 *                sets its word, and a second launch recomputes that wave's
 *                workgroup with a rescaling running maximum.  Calls that
 *                share a workspace must not overlap.
 * Errors: YRK_EINVAL (also a null or misaligned workspace), YRK_ERANGE
 * (positions beyond table or capacity, or a chunk ending past 2^31 - 65),
 * YRK_ENOTSUP (dtype other than bf16,
 * head_dim != 256, group size other than 6), YRK_ENOSPC (workspace smaller
 * than yrk_prefill_workspace_size()).
 */
int yrk_prefill_attention(const yrk_kv_layer* layer, const void* q_dev, int64_t num_q_tokens,
                          int32_t num_q_heads, int64_t q_start_position,
                          const int32_t* block_table_dev, int64_t block_table_len,
                          float softmax_scale, void* out_dev, void* workspace_dev,
                          size_t workspace_bytes, uint32_t* dev_error_word, hipStream_t stream);

/* Human-readable text for a status code (static storage). */
const char* yrk_status_string(int status);

/* ABI version of this header (bumped on any incompatible change). */
int yrk_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* YRK_H */
