// The C ABI of libyrk (include/yrk.h): host-side validation, the YaRN table
// and planning; kernels are enqueued only after every check has passed, so a
// failed call writes nothing.
#include "yrk.h"

#include <cmath>
#include <string.h>

#include "yrk_internal.h"

static_assert(YRK_NOALLOC_SCRATCH_BYTES == yrk::kNoAllocScratchBytes, "one scratch size");

namespace {

constexpr int kAbiVersion = 2;

bool is_finite(double x) { return __builtin_isfinite(x); }

// Host-only YaRN table ([P1] "YaRN, and matching what vLLM actually does";
// [P3] "YaRN reference and drift guard").  Pair i of the rotary dims has the
// trained frequency theta_i = base^(-2i/d).  The correction range [low,
// high] holds the pairs whose number of full turns over the correction
// length L lies between beta_slow and beta_fast; below it frequencies are
// kept, from `high` up they are divided by the factor, in between a linear
// ramp blends the two.  inv_freq holds `capacity` doubles: a table of more
// pairs is refused (YRK_ENOTSUP) before anything is written.
int yarn_table(const yrk_yarn_params* p, double* inv_freq, int capacity, double* mscale,
               int32_t* lo_out, int32_t* hi_out) {
  if (!p) return YRK_EINVAL;
  const double base = p->rope_theta, s = p->factor;
  const int d = p->rotary_dim;
  if (!is_finite(base) || base <= 1.0) return YRK_EINVAL;
  if (d <= 0 || (d & 1) || d > p->head_dim || p->head_dim <= 0) return YRK_EINVAL;
  if (!is_finite(s) || s < 1.0 || s > 64.0) return YRK_EINVAL;
  if (p->original_max_position <= 0 || p->correction_max_position < 0) return YRK_EINVAL;
  if (!is_finite(p->beta_fast) || !is_finite(p->beta_slow) || p->beta_fast <= 0.0 ||
      p->beta_slow <= 0.0 || p->beta_slow > p->beta_fast)
    return YRK_EINVAL;
  if (!is_finite(p->mscale)) return YRK_EINVAL;
  if (inv_freq && d / 2 > capacity) return YRK_ENOTSUP;

  const double L = (double)(p->correction_max_position > 0 ? p->correction_max_position
                                                           : p->original_max_position);
  const double ln_base = log(base);
  // pair index at which a pair makes exactly `turns` full rotations over L
  auto pair_at_turns = [&](double turns) {
    return (double)d * log(L / (turns * 2.0 * M_PI)) / (2.0 * ln_base);
  };
  // low is clamped below at 0 and high above at d - 1.  Their other ends are
  // limited too, low to d and high to -1, in double before the conversion to
  // int32 (undefined out of range, which a base just above 1 reaches); no
  // weight changes, since the ramp is already 1 (low > d) or 0 (high < -1)
  // for every pair there.
  const double lo_d = floor(pair_at_turns(p->beta_fast));
  const double hi_d = ceil(pair_at_turns(p->beta_slow));
  const int32_t lo = lo_d < 0.0 ? 0 : (lo_d > (double)d ? d : (int32_t)lo_d);
  const int32_t hi = hi_d > (double)(d - 1) ? d - 1 : (hi_d < -1.0 ? -1 : (int32_t)hi_d);
  const double span = hi == lo ? 0.001 : (double)(hi - lo);
  if (inv_freq) {
    for (int i = 0; i < d / 2; ++i) {
      const double theta = pow(base, -2.0 * (double)i / (double)d);
      double w = ((double)i - (double)lo) / span;   // weight of the interpolated frequency
      w = w < 0.0 ? 0.0 : (w > 1.0 ? 1.0 : w);
      inv_freq[i] = theta * (1.0 - w) + (theta / s) * w;
    }
  }
  if (mscale) *mscale = p->mscale > 0.0 ? p->mscale : (s > 1.0 ? 1.0 + 0.1 * log(s) : 1.0);
  if (lo_out) *lo_out = lo;
  if (hi_out) *hi_out = hi;
  return YRK_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_layer(const yrk_kv_layer* L) {
  if (!L) return YRK_EINVAL;
  if (L->dtype != YRK_KV_BF16 && L->dtype != YRK_KV_NVFP4 && L->dtype != YRK_KV_INT8)
    return YRK_EINVAL;
  if (L->num_kv_heads <= 0 || L->head_dim <= 0 || L->block_size <= 0 || L->num_blocks <= 0)
    return YRK_EINVAL;
  if (L->paged != 0 && L->paged != 1) return YRK_EINVAL;
  if (L->reserved != 0) return YRK_EINVAL;
  if (L->num_blocks > INT32_MAX) return YRK_ERANGE;   // block ids are int32
  if (!L->k || !L->v) return YRK_EINVAL;
  if (L->dtype == YRK_KV_NVFP4 &&
      (!L->k_scale || !L->v_scale || !L->k_tensor_scale_dev || !L->v_tensor_scale_dev))
    return YRK_EINVAL;
  if (L->dtype == YRK_KV_INT8 && (!L->k_scale || !L->v_scale)) return YRK_EINVAL;
  // the kernels read code and value rows with 16-byte loads and the scale
  // planes as whole rows (16 e4m3 bytes, or 4 binary16 words), the tensor
  // scales as single floats
  if (!aligned16(L->k) || !aligned16(L->v)) return YRK_EINVAL;
  if (L->dtype != YRK_KV_BF16 && (!aligned16(L->k_scale) || !aligned16(L->v_scale)))
    return YRK_EINVAL;
  if (L->dtype == YRK_KV_NVFP4 && ((((uintptr_t)L->k_tensor_scale_dev) & 3u) != 0 ||
                                   (((uintptr_t)L->v_tensor_scale_dev) & 3u) != 0))
    return YRK_EINVAL;
  if (L->head_dim != yrk::kHeadDim || L->block_size != yrk::kBlockSize) return YRK_ENOTSUP;
  return YRK_OK;
}

yrk::KvGeometry geometry(const yrk_kv_layer* L) {
  yrk::KvGeometry g;
  g.num_kv_heads = L->num_kv_heads;
  g.paged = L->paged;
  g.num_blocks = L->num_blocks;
  return g;
}

// Whether `pages` 16-token pages hold `tokens` tokens (0 <= tokens; no overflow).
bool pages_hold(int64_t pages, int64_t tokens) {
  return pages >= (tokens + yrk::kBlockSize - 1) / yrk::kBlockSize;
}

// Launch-grid limits of the split-K attention kernels: sequences and KV heads
// are grid dimensions (at most 65,535), query heads index the merge grid.
constexpr int32_t kMaxSeqs = 65535, kMaxKvHeads = 256, kMaxQHeads = 4096;
bool shape_fits_grid(int64_t num_seqs, int64_t num_kv_heads, int64_t num_q_heads) {
  return num_seqs <= kMaxSeqs && num_kv_heads <= kMaxKvHeads && num_q_heads <= kMaxQHeads;
}

int launch_status(hipError_t e) { return e == hipSuccess ? YRK_OK : YRK_EDEVICE; }

// Decode attention behind both entry points.  workspace_dev == nullptr
// selects the library's device scratch (yrk_decode_attention_noalloc), taken
// only after every host check has passed; workspace_bytes is then its size.
int decode_call(const yrk_kv_layer* layer, const void* q_dev, int32_t num_seqs,
                int32_t num_q_heads, const int32_t* block_tables_dev,
                int64_t block_table_stride, const int32_t* seq_lens_dev, int64_t max_seq_len,
                float softmax_scale, void* out_dev, int32_t out_dtype, void* workspace_dev,
                size_t workspace_bytes, uint32_t* dev_error_word, hipStream_t stream) {
  int rc = check_layer(layer);
  if (rc) return rc;
  if (num_seqs <= 0 || num_q_heads <= 0 || max_seq_len < 0) return YRK_EINVAL;
  if (num_q_heads % layer->num_kv_heads) return YRK_EINVAL;
  if (!shape_fits_grid(num_seqs, layer->num_kv_heads, num_q_heads)) return YRK_ENOTSUP;
  if (out_dtype != YRK_OUT_BF16 && out_dtype != YRK_OUT_F32) return YRK_EINVAL;
  if (!q_dev || !seq_lens_dev || !out_dev) return YRK_EINVAL;
  if (!is_finite(softmax_scale) || softmax_scale < 0.0f) return YRK_EINVAL;
  if (!aligned16(q_dev) || !aligned16(workspace_dev)) return YRK_EINVAL;   // null is aligned
  const int group = num_q_heads / layer->num_kv_heads;
  if (group != 1 && group != 2 && group != 3 && group != 4 && group != 6)
    return YRK_ENOTSUP;
  if (layer->paged) {
    if (!block_tables_dev || block_table_stride <= 0) return YRK_EINVAL;
  } else if (num_seqs != 1) {
    return YRK_EINVAL;
  }
  if (max_seq_len > INT32_MAX) return YRK_ERANGE;
  if (!pages_hold(layer->paged ? block_table_stride : layer->num_blocks, max_seq_len))
    return YRK_ERANGE;
  yrk::DecodeArgs a;
  a.plan = yrk::plan_decode(num_seqs, layer->num_kv_heads, max_seq_len, layer->dtype);
  const size_t need = yrk::decode_workspace_bytes(num_seqs, num_q_heads, a.plan);
  if (workspace_bytes < need) return YRK_ENOSPC;
  if (!workspace_dev) {
    const hipError_t e = yrk::device_scratch(&workspace_dev);
    if (e != hipSuccess) return YRK_EDEVICE;
  }
  if (softmax_scale == 0.0f) softmax_scale = 1.0f / sqrtf((float)layer->head_dim);
  a.geo = geometry(layer);
  a.dtype = layer->dtype;
  a.group = group;
  a.num_q_heads = num_q_heads;
  a.num_seqs = num_seqs;
  a.q = static_cast<const uint16_t*>(q_dev);
  a.k = layer->k;
  a.v = layer->v;
  a.k_scale = static_cast<const uint8_t*>(layer->k_scale);
  a.v_scale = static_cast<const uint8_t*>(layer->v_scale);
  a.k_tensor_scale = layer->k_tensor_scale_dev;
  a.v_tensor_scale = layer->v_tensor_scale_dev;
  a.block_tables = layer->paged ? block_tables_dev : nullptr;
  a.block_table_stride = layer->paged ? block_table_stride : 0;
  a.seq_lens = seq_lens_dev;
  a.max_seq_len = max_seq_len;
  a.scale_log2 = (float)((double)softmax_scale * M_LOG2E);
  a.out = out_dev;
  a.out_f32 = out_dtype == YRK_OUT_F32;
  const size_t slots = (size_t)num_seqs * num_q_heads * a.plan.num_splits;
  a.ws_o = static_cast<float*>(workspace_dev);
  a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace_dev) +
                                      ((slots * yrk::kHeadDim * sizeof(float) + 255) / 256) * 256);
  a.err = dev_error_word;
  return launch_status(yrk::launch_decode(a, stream));
}


}  // namespace

extern "C" {

int yrk_abi_version(void) { return kAbiVersion; }

const char* yrk_status_string(int status) {
  switch (status) {
    case YRK_OK: return "ok";
    case YRK_EINVAL: return "invalid argument";
    case YRK_ERANGE: return "length or position out of range";
    case YRK_ENOTSUP: return "shape or dtype not supported by this build";
    case YRK_ENOSPC: return "workspace too small";
    case YRK_EDEVICE: return "HIP launch failed";
    default: return "unknown status";
  }
}

int yrk_yarn_table(const yrk_yarn_params* params, double* inv_freq_out, double* mscale_out,
                   int32_t* corr_low_out, int32_t* corr_high_out) {
  // the caller provides rotary_dim / 2 doubles
  return yarn_table(params, inv_freq_out, INT32_MAX, mscale_out, corr_low_out, corr_high_out);
}

int yrk_yarn_rope_apply(const yrk_yarn_params* params, void* x_dev, int64_t num_tokens,
                        int32_t num_heads, int64_t token_stride, const int32_t* positions_dev,
                        uint32_t* dev_error_word, hipStream_t stream) {
  yrk::RopeArgs a;
  int rc = yarn_table(params, a.inv_freq, yrk::kMaxRotaryHalf, &a.mscale, nullptr, nullptr);
  if (rc) return rc;
  if (num_tokens < 0 || num_heads <= 0) return YRK_EINVAL;
  if (token_stride < (int64_t)num_heads * params->head_dim) return YRK_EINVAL;
  if (num_tokens == 0) return YRK_OK;
  if (!x_dev || !positions_dev) return YRK_EINVAL;
  a.x = static_cast<uint16_t*>(x_dev);
  a.num_tokens = num_tokens;
  a.num_heads = num_heads;
  a.head_dim = params->head_dim;
  a.token_stride = token_stride;
  a.half = params->rotary_dim / 2;
  a.positions = positions_dev;
  a.err = dev_error_word;
  return launch_status(yrk::launch_rope(a, stream));
}

int yrk_nvfp4_tensor_scale(const void* x_dev, int64_t n, float* scale_out_dev,
                           hipStream_t stream) {
  if (n < 0 || !scale_out_dev || (n > 0 && !x_dev)) return YRK_EINVAL;
  if (((uintptr_t)scale_out_dev & 3u) != 0) return YRK_EINVAL;
  return launch_status(
      yrk::launch_tensor_scale(static_cast<const uint16_t*>(x_dev), n, scale_out_dev, stream));
}

int yrk_kv_append_quantize(const yrk_kv_layer* layer, const void* k_dev, const void* v_dev,
                           int64_t num_tokens, const int32_t* block_table_dev,
                           int64_t block_table_len, const int32_t* positions_dev,
                           uint32_t* dev_error_word, hipStream_t stream) {
  int rc = check_layer(layer);
  if (rc) return rc;
  if (num_tokens < 0) return YRK_EINVAL;
  if (layer->paged && (!block_table_dev || block_table_len <= 0)) return YRK_EINVAL;
  if (num_tokens == 0) return YRK_OK;
  if (!k_dev || !v_dev || !positions_dev) return YRK_EINVAL;
  if (!aligned16(k_dev) || !aligned16(v_dev) || !aligned16(layer->k) || !aligned16(layer->v))
    return YRK_EINVAL;
  yrk::AppendArgs a;
  a.geo = geometry(layer);
  a.dtype = layer->dtype;
  a.k_src = static_cast<const uint16_t*>(k_dev);
  a.v_src = static_cast<const uint16_t*>(v_dev);
  a.num_tokens = num_tokens;
  a.block_table = layer->paged ? block_table_dev : nullptr;
  a.block_table_len = layer->paged ? block_table_len : 0;
  a.positions = positions_dev;
  a.err = dev_error_word;
  a.k_dst = layer->k;
  a.v_dst = layer->v;
  a.k_scale_dst = static_cast<uint8_t*>(layer->k_scale);
  a.v_scale_dst = static_cast<uint8_t*>(layer->v_scale);
  a.k_tensor_scale = layer->k_tensor_scale_dev;
  a.v_tensor_scale = layer->v_tensor_scale_dev;
  return launch_status(yrk::launch_append(a, stream));
}

int yrk_rope_append(const yrk_kv_layer* layer, const yrk_yarn_params* params, void* q_dev,
                    int32_t num_q_heads, int64_t q_token_stride, const void* k_dev,
                    const void* v_dev, int64_t num_tokens, const int32_t* block_table_dev,
                    int64_t block_table_len, const int32_t* positions_dev,
                    uint32_t* dev_error_word, hipStream_t stream) {
  int rc = check_layer(layer);
  if (rc) return rc;
  yrk::RopeAppendArgs ra;
  rc = yarn_table(params, ra.inv_freq, yrk::kFusedRopePairs, &ra.mscale, nullptr, nullptr);
  if (rc) return rc;
  if (params->head_dim != yrk::kHeadDim || params->rotary_dim != 2 * yrk::kFusedRopePairs)
    return YRK_ENOTSUP;
  if (num_tokens < 0) return YRK_EINVAL;
  if (layer->paged && (!block_table_dev || block_table_len <= 0)) return YRK_EINVAL;
  if (q_dev) {
    if (num_q_heads <= 0 || q_token_stride < (int64_t)num_q_heads * yrk::kHeadDim ||
        q_token_stride % 4 != 0 || ((uintptr_t)q_dev & 7u) != 0)
      return YRK_EINVAL;
  }
  if (num_tokens == 0) return YRK_OK;
  if (!k_dev || !v_dev || !positions_dev) return YRK_EINVAL;
  if (!aligned16(k_dev) || !aligned16(v_dev) || !aligned16(layer->k) || !aligned16(layer->v))
    return YRK_EINVAL;
  ra.q = static_cast<uint16_t*>(q_dev);
  ra.num_q_heads = q_dev ? num_q_heads : 0;
  ra.q_token_stride = q_dev ? q_token_stride : 0;
  yrk::AppendArgs& a = ra.ap;
  a.geo = geometry(layer);
  a.dtype = layer->dtype;
  a.k_src = static_cast<const uint16_t*>(k_dev);
  a.v_src = static_cast<const uint16_t*>(v_dev);
  a.num_tokens = num_tokens;
  a.block_table = layer->paged ? block_table_dev : nullptr;
  a.block_table_len = layer->paged ? block_table_len : 0;
  a.positions = positions_dev;
  a.err = dev_error_word;
  a.k_dst = layer->k;
  a.v_dst = layer->v;
  a.k_scale_dst = static_cast<uint8_t*>(layer->k_scale);
  a.v_scale_dst = static_cast<uint8_t*>(layer->v_scale);
  a.k_tensor_scale = layer->k_tensor_scale_dev;
  a.v_tensor_scale = layer->v_tensor_scale_dev;
  return launch_status(yrk::launch_rope_append(ra, stream));
}

size_t yrk_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int64_t max_seq_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim != yrk::kHeadDim ||
      max_seq_len < 0 || max_seq_len > INT32_MAX ||
      !shape_fits_grid(num_seqs, num_kv_heads, num_q_heads))
    return 0;
  // the cache format is not an argument here: enough for either plan
  const size_t b16 = yrk::decode_workspace_bytes(
      num_seqs, num_q_heads, yrk::plan_decode(num_seqs, num_kv_heads, max_seq_len, YRK_KV_BF16));
  const size_t f4 = yrk::decode_workspace_bytes(
      num_seqs, num_q_heads, yrk::plan_decode(num_seqs, num_kv_heads, max_seq_len, YRK_KV_NVFP4));
  const size_t i8 = yrk::decode_workspace_bytes(
      num_seqs, num_q_heads, yrk::plan_decode(num_seqs, num_kv_heads, max_seq_len, YRK_KV_INT8));
  const size_t m = b16 > f4 ? b16 : f4;
  return m > i8 ? m : i8;
}

int yrk_decode_attention(const yrk_kv_layer* layer, const void* q_dev, int32_t num_seqs,
                         int32_t num_q_heads, const int32_t* block_tables_dev,
                         int64_t block_table_stride, const int32_t* seq_lens_dev,
                         int64_t max_seq_len, float softmax_scale, void* out_dev,
                         int32_t out_dtype, void* workspace_dev, size_t workspace_bytes,
                         uint32_t* dev_error_word, hipStream_t stream) {
  if (!workspace_dev) return YRK_EINVAL;
  return decode_call(layer, q_dev, num_seqs, num_q_heads, block_tables_dev, block_table_stride,
                     seq_lens_dev, max_seq_len, softmax_scale, out_dev, out_dtype, workspace_dev,
                     workspace_bytes, dev_error_word, stream);
}

int yrk_decode_attention_noalloc(const yrk_kv_layer* layer, const void* q_dev, int32_t num_seqs,
                                 int32_t num_q_heads, const int32_t* block_tables_dev,
                                 int64_t block_table_stride, const int32_t* seq_lens_dev,
                                 int64_t max_seq_len, float softmax_scale, void* out_dev,
                                 int32_t out_dtype, uint32_t* dev_error_word,
                                 hipStream_t stream) {
  // nullptr workspace: decode_call validates everything, then takes the
  // device scratch of the current device (no allocation anywhere)
  return decode_call(layer, q_dev, num_seqs, num_q_heads, block_tables_dev, block_table_stride,
                     seq_lens_dev, max_seq_len, softmax_scale, out_dev, out_dtype, nullptr,
                     yrk::kNoAllocScratchBytes, dev_error_word, stream);
}

size_t yrk_verify_workspace_size(int32_t num_seqs, int32_t num_queries, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int64_t max_seq_len) {
  if (num_seqs <= 0 || num_queries <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim != yrk::kHeadDim || max_seq_len < 0 || max_seq_len > INT32_MAX ||
      num_q_heads % num_kv_heads ||
      !shape_fits_grid(num_seqs, num_kv_heads, num_q_heads) || num_queries > yrk::kVerifyMaxRows)
    return 0;
  const int64_t rows = (int64_t)num_queries * (num_q_heads / num_kv_heads);
  if (rows > yrk::kVerifyMaxRows) return 0;
  // the cache format is not an argument here: enough for either plan
  size_t need = 0;
  for (int32_t dtype : {YRK_KV_BF16, YRK_KV_INT8}) {
    const yrk::DecodePlan p =
        yrk::plan_verify(num_seqs, num_kv_heads, (int32_t)rows, max_seq_len, dtype);
    const size_t b = yrk::decode_workspace_bytes(num_seqs, num_queries * num_q_heads, p);
    need = b > need ? b : need;
  }
  return need;
}

int yrk_verify_attention(const yrk_kv_layer* layer, const void* q_dev, int32_t num_seqs,
                         int32_t num_queries, int32_t num_q_heads,
                         const int32_t* block_tables_dev, int64_t block_table_stride,
                         const int32_t* seq_lens_dev, int64_t max_seq_len, float softmax_scale,
                         void* out_dev, int32_t out_dtype, void* workspace_dev,
                         size_t workspace_bytes, uint32_t* dev_error_word, hipStream_t stream) {
  int rc = check_layer(layer);
  if (rc) return rc;
  if (num_seqs <= 0 || num_queries <= 0 || num_q_heads <= 0 || max_seq_len < 0)
    return YRK_EINVAL;
  if (num_q_heads % layer->num_kv_heads) return YRK_EINVAL;
  if (!shape_fits_grid(num_seqs, layer->num_kv_heads, num_q_heads) ||
      num_queries > yrk::kVerifyMaxRows)
    return YRK_ENOTSUP;
  if (out_dtype != YRK_OUT_BF16 && out_dtype != YRK_OUT_F32) return YRK_EINVAL;
  if (!q_dev || !seq_lens_dev || !out_dev || !workspace_dev) return YRK_EINVAL;
  if (!is_finite(softmax_scale) || softmax_scale < 0.0f) return YRK_EINVAL;
  if (!aligned16(q_dev) || !aligned16(workspace_dev) || !aligned16(layer->k) ||
      !aligned16(layer->v))
    return YRK_EINVAL;
  if (layer->dtype == YRK_KV_NVFP4) return YRK_ENOTSUP;
  const int group = num_q_heads / layer->num_kv_heads;
  if (group != 1 && group != 2 && group != 3 && group != 4 && group != 6)
    return YRK_ENOTSUP;
  if ((int64_t)num_queries * group > yrk::kVerifyMaxRows) return YRK_ENOTSUP;
  if (layer->paged) {
    if (!block_tables_dev || block_table_stride <= 0) return YRK_EINVAL;
  } else if (num_seqs != 1) {
    return YRK_EINVAL;
  }
  if (max_seq_len > INT32_MAX) return YRK_ERANGE;
  if (!pages_hold(layer->paged ? block_table_stride : layer->num_blocks, max_seq_len))
    return YRK_ERANGE;
  yrk::VerifyArgs va;
  yrk::DecodeArgs& a = va.d;
  va.num_queries = num_queries;
  va.min_len = num_queries;
  a.plan = yrk::plan_verify(num_seqs, layer->num_kv_heads, num_queries * group, max_seq_len,
                            layer->dtype);
  const int32_t rows_per_seq = num_queries * num_q_heads;
  const size_t need = yrk::decode_workspace_bytes(num_seqs, rows_per_seq, a.plan);
  if (workspace_bytes < need) return YRK_ENOSPC;
  if (softmax_scale == 0.0f) softmax_scale = 1.0f / sqrtf((float)layer->head_dim);
  a.geo = geometry(layer);
  a.dtype = layer->dtype;
  a.group = group;
  a.num_q_heads = num_q_heads;
  a.num_seqs = num_seqs;
  a.q = static_cast<const uint16_t*>(q_dev);
  a.k = layer->k;
  a.v = layer->v;
  a.k_scale = static_cast<const uint8_t*>(layer->k_scale);   // INT8 group scales, else unused
  a.v_scale = static_cast<const uint8_t*>(layer->v_scale);
  a.k_tensor_scale = nullptr;
  a.v_tensor_scale = nullptr;
  a.block_tables = layer->paged ? block_tables_dev : nullptr;
  a.block_table_stride = layer->paged ? block_table_stride : 0;
  a.seq_lens = seq_lens_dev;
  a.max_seq_len = max_seq_len;
  a.scale_log2 = (float)((double)softmax_scale * M_LOG2E);
  a.out = out_dev;
  a.out_f32 = out_dtype == YRK_OUT_F32;
  const size_t slots = (size_t)num_seqs * rows_per_seq * a.plan.num_splits;
  a.ws_o = static_cast<float*>(workspace_dev);
  a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace_dev) +
                                      ((slots * yrk::kHeadDim * sizeof(float) + 255) / 256) * 256);
  a.err = dev_error_word;
  return launch_status(yrk::launch_verify(va, stream));
}

size_t yrk_prefill_workspace_size(int64_t num_q_tokens, int32_t num_q_heads, int32_t head_dim) {
  if (num_q_tokens < 0 || num_q_heads <= 0 || head_dim != yrk::kHeadDim) return 0;
  return yrk::prefill_workspace_bytes(num_q_tokens, num_q_heads);
}

int yrk_prefill_attention(const yrk_kv_layer* layer, const void* q_dev, int64_t num_q_tokens,
                          int32_t num_q_heads, int64_t q_start_position,
                          const int32_t* block_table_dev, int64_t block_table_len,
                          float softmax_scale, void* out_dev, void* workspace_dev,
                          size_t workspace_bytes, uint32_t* dev_error_word, hipStream_t stream) {
  int rc = check_layer(layer);
  if (rc) return rc;
  if (num_q_tokens < 0 || num_q_heads <= 0 || q_start_position < 0) return YRK_EINVAL;
  if (num_q_heads % layer->num_kv_heads) return YRK_EINVAL;
  if (!is_finite(softmax_scale) || softmax_scale < 0.0f) return YRK_EINVAL;
  if (layer->paged && (!block_table_dev || block_table_len <= 0)) return YRK_EINVAL;
  // the kernel forms key bounds up to two 32-key tiles past the chunk's end in int32
  if (q_start_position > INT32_MAX || num_q_tokens > INT32_MAX) return YRK_ERANGE;
  const int64_t end = q_start_position + num_q_tokens;
  if (end > (int64_t)INT32_MAX - 64) return YRK_ERANGE;
  if (!pages_hold(layer->paged ? block_table_len : layer->num_blocks, end)) return YRK_ERANGE;
  if (num_q_tokens == 0) return YRK_OK;
  if (!q_dev || !out_dev) return YRK_EINVAL;
  if (!aligned16(q_dev) || !aligned16(out_dev)) return YRK_EINVAL;
  if (layer->dtype != YRK_KV_BF16) return YRK_ENOTSUP;
  const int group = num_q_heads / layer->num_kv_heads;
  if (group != 6) return YRK_ENOTSUP;
  if (!workspace_dev || ((uintptr_t)workspace_dev & 3u) != 0) return YRK_EINVAL;
  if (workspace_bytes < yrk::prefill_workspace_bytes(num_q_tokens, num_q_heads)) return YRK_ENOSPC;
  if (softmax_scale == 0.0f) softmax_scale = 1.0f / sqrtf((float)layer->head_dim);
  yrk::PrefillArgs a;
  a.geo = geometry(layer);
  a.group = group;
  a.num_q_heads = num_q_heads;
  a.q = static_cast<const uint16_t*>(q_dev);
  a.k = static_cast<const uint16_t*>(layer->k);
  a.v = static_cast<const uint16_t*>(layer->v);
  a.num_q_tokens = num_q_tokens;
  a.q_start = q_start_position;
  a.block_table = layer->paged ? block_table_dev : nullptr;
  a.block_table_len = layer->paged ? block_table_len : 0;
  a.scale_log2 = (float)((double)softmax_scale * M_LOG2E);
  a.out = static_cast<uint16_t*>(out_dev);
  a.err = dev_error_word;
  a.flags = static_cast<uint32_t*>(workspace_dev);
  return launch_status(yrk::launch_prefill(a, stream));
}

}  // extern "C"
