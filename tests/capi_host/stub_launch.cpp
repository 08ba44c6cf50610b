// Host-only stand-ins for the kernel launchers of libyrk, for the sanitized
// CPU build of the C-ABI layer (capi.cpp + plan.cpp).  Nothing here touches a
// GPU.  Each stand-in checks the arguments the real launcher relies on and
// touches the first and last byte of every workspace region the real kernels
// write, so that AddressSanitizer reports a workspace the size queries made
// too small.  Pointers a test passes in are either real host buffers (the
// workspaces) or never dereferenced.
#include <stdio.h>
#include <stdlib.h>

#include "yrk_internal.h"

namespace {

[[noreturn]] void fail(const char* what) {
  fprintf(stderr, "stub launcher: %s\n", what);
  abort();
}

void touch(void* base, size_t first, size_t last) {
  volatile unsigned char* p = static_cast<volatile unsigned char*>(base);
  p[first] = p[first];
  p[last] = p[last];
}

void touch_partials(const yrk::DecodeArgs& a, int32_t rows_per_seq) {
  if (a.plan.num_splits < 1 || a.plan.tokens_per_split <= 0) fail("empty split plan");
  if ((int64_t)a.plan.num_splits * a.plan.tokens_per_split < a.max_seq_len)
    fail("the splits do not cover max_seq_len");
  const size_t slots = (size_t)a.num_seqs * rows_per_seq * a.plan.num_splits;
  touch(a.ws_o, 0, slots * yrk::kHeadDim * sizeof(float) - 1);
  touch(a.ws_lse, 0, slots * sizeof(float) - 1);
}

}  // namespace

namespace yrk {

long g_launches = 0;

hipError_t launch_rope(const RopeArgs& a, hipStream_t) {
  if (a.half < 1 || a.half > kMaxRotaryHalf || 2 * a.half > a.head_dim) fail("rope shape");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_append(const AppendArgs& a, hipStream_t) {
  if (a.num_tokens <= 0 || a.geo.num_kv_heads <= 0) fail("append shape");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_rope_append(const RopeAppendArgs& a, hipStream_t) {
  if (a.ap.num_tokens <= 0 || (a.q && a.num_q_heads <= 0)) fail("rope_append shape");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_tensor_scale(const uint16_t*, int64_t n, float*, hipStream_t) {
  if (n < 0) fail("tensor scale size");
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t) {
  if (a.group != 1 && a.group != 2 && a.group != 3 && a.group != 4 && a.group != 6)
    fail("decode group");
  if (a.max_seq_len < 0 || a.max_seq_len > INT32_MAX) fail("decode length");
  touch_partials(a, a.num_q_heads);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t) {
  touch_partials(a, a.num_q_heads);
  ++g_launches;
  return hipSuccess;
}

hipError_t launch_verify(const VerifyArgs& a, hipStream_t) {
  const int rows = a.num_queries * a.d.group;
  if (rows < 1 || rows > kVerifyMaxRows) fail("verify rows");
  touch_partials(a.d, a.num_queries * a.d.num_q_heads);
  ++g_launches;
  return hipSuccess;
}

hipError_t device_scratch(void** ptr) {
  // a host stand-in of the library's device scratch, of the same size
  static unsigned char* buf = static_cast<unsigned char*>(malloc(kNoAllocScratchBytes));
  *ptr = buf;
  return hipSuccess;
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t) {
  if (a.group != kPrefillGroup || a.num_q_tokens <= 0) fail("prefill shape");
  if (a.q_start + a.num_q_tokens > (int64_t)INT32_MAX - 64) fail("prefill positions");
  const PrefillGrid g = prefill_grid(a.num_q_tokens, a.geo.num_kv_heads);
  touch(a.flags, 0, (size_t)g.blocks * kPrefillWaves * sizeof(uint32_t) - 1);
  ++g_launches;
  return hipSuccess;
}

}  // namespace yrk
