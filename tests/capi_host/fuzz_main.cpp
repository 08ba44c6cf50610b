// Seeded fuzz of the C ABI's host-side validation, for a build of capi.cpp
// and plan.cpp with AddressSanitizer and UndefinedBehaviorSanitizer and the
// host-only launcher stand-ins (stub_launch.cpp); no GPU is involved.
//
// Every call must come back with a status of the header's set; a call that
// fails must have launched nothing; a workspace of the size the matching
// size query returned must never be refused as too small.  Stack or heap
// overruns and signed overflow abort the program under the sanitizers.
// Usage: capi_fuzz [iterations] [seed]
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <limits>

#include "yrk.h"

namespace yrk { extern long g_launches; }

namespace {

uint64_t g_state;
uint64_t next_u64() {   // SplitMix64 (Steele, Lea, Flood, OOPSLA 2014)
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
int pick(int n) { return (int)(next_u64() % (uint64_t)n); }
bool chance(int percent) { return pick(100) < percent; }

int32_t any_i32(int32_t good) {
  static const int32_t pool[] = {0, 1, -1, 2, 3, 4, 6, 12, 16, 24, 32, 48, 64, 255, 256, 257,
                                 258, 512, 8192, 1 << 20, INT32_MAX, INT32_MIN, INT32_MAX - 1};
  if (chance(70)) return good;
  if (chance(20)) return (int32_t)next_u64();
  return pool[pick(sizeof(pool) / sizeof(pool[0]))];
}
int64_t any_i64(int64_t good) {
  static const int64_t pool[] = {0, 1, -1, 16, 17, 4096, 4097, 1 << 20, (int64_t)1 << 31,
                                 INT32_MAX, (int64_t)INT32_MAX + 1, INT32_MAX - 64,
                                 INT32_MAX - 65, INT64_MAX, INT64_MIN, INT64_MAX / 16};
  if (chance(70)) return good;
  if (chance(20)) return (int64_t)next_u64();
  return pool[pick(sizeof(pool) / sizeof(pool[0]))];
}
double any_f64(double good) {
  static const double pool[] = {0.0, -0.0, 1.0, -1.0, 0.5, 4.0, 64.0, 65.0, 1e7, 1.0000001,
                                1e308, 1e-308, 32.0, 1e300,
                                std::numeric_limits<double>::quiet_NaN(),
                                std::numeric_limits<double>::infinity(),
                                -std::numeric_limits<double>::infinity()};
  if (chance(75)) return good;
  return pool[pick(sizeof(pool) / sizeof(pool[0]))];
}
void* any_ptr(uintptr_t good) {
  static const uintptr_t pool[] = {0, 0x10001, 0x10002, 0x10004, 0x10008, 0x20000};
  if (chance(85)) return (void*)good;
  return (void*)pool[pick(sizeof(pool) / sizeof(pool[0]))];
}

yrk_yarn_params random_params() {
  yrk_yarn_params p;
  p.rope_theta = any_f64(1e7);
  p.head_dim = any_i32(256);
  p.rotary_dim = any_i32(64);
  p.factor = any_f64(4.0);
  p.original_max_position = any_i64(262144);
  p.correction_max_position = any_i64(0);
  p.beta_fast = any_f64(32.0);
  p.beta_slow = any_f64(1.0);
  p.mscale = any_f64(0.0);
  return p;
}

yrk_kv_layer random_layer() {
  yrk_kv_layer L;
  L.dtype = any_i32(pick(3));
  L.num_kv_heads = any_i32(chance(50) ? 4 : 2);
  L.head_dim = any_i32(256);
  L.block_size = any_i32(16);
  L.num_blocks = any_i64(65536);
  L.paged = any_i32(chance(80) ? 1 : 0);
  L.reserved = chance(95) ? 0 : 1;
  L.k = any_ptr(0x100000);
  L.v = any_ptr(0x200000);
  L.k_scale = any_ptr(0x300000);
  L.v_scale = any_ptr(0x400000);
  L.k_tensor_scale_dev = (const float*)any_ptr(0x500000);
  L.v_tensor_scale_dev = (const float*)any_ptr(0x600000);
  return L;
}

long g_failures = 0;
void check(bool ok, const char* what, long iter) {
  if (!ok) {
    fprintf(stderr, "iteration %ld: %s\n", iter, what);
    ++g_failures;
  }
}

bool known_status(int s) { return s <= 0 && s >= -5; }

// A status came back from the set, and a refused call launched nothing.
void after_call(int status, long before, const char* name, long iter) {
  char msg[160];
  snprintf(msg, sizeof msg, "%s returned %d", name, status);
  check(known_status(status), msg, iter);
  if (status != YRK_OK) {
    snprintf(msg, sizeof msg, "%s failed with %d after launching", name, status);
    check(yrk::g_launches == before, msg, iter);
  }
}

void* host_buffer(size_t bytes) { return malloc(bytes ? bytes : 1); }

// Workspace bytes to pass: the size query's answer most of the time, one
// byte short now and then; an answer beyond 256 MiB (the shape is refused
// or absurd) is replaced by a small buffer.
size_t workspace_bytes(size_t need) {
  if (need > ((size_t)256 << 20)) return 4096;
  return chance(80) ? need : (need ? need - 1 : 64);
}

void fixed_cases() {
  // head_dim = rotary_dim beyond the library's rotary table: refused before
  // anything is written (this once overran a 128-entry stack array)
  yrk_kv_layer L;
  memset(&L, 0, sizeof L);
  L.dtype = YRK_KV_BF16; L.num_kv_heads = 4; L.head_dim = 256; L.block_size = 16;
  L.num_blocks = 64; L.paged = 1; L.k = (void*)0x100000; L.v = (void*)0x200000;
  for (int32_t d : {258, 512, 8192}) {
    yrk_yarn_params p = {1e7, d, d, 4.0, 262144, 0, 32.0, 1.0, 0.0};
    int s = yrk_yarn_rope_apply(&p, (void*)0x1000, 1, 24, 24 * 8192, (const int32_t*)0x2000,
                                nullptr, nullptr);
    check(s == YRK_ENOTSUP, "rope_apply: rotary_dim beyond 256 not refused with ENOTSUP", -1);
    s = yrk_rope_append(&L, &p, (void*)0x8000, 24, 24 * 256, (void*)0x1000, (void*)0x3000, 4,
                        (const int32_t*)0x4000, 4, (const int32_t*)0x5000, nullptr, nullptr);
    check(s == YRK_ENOTSUP, "rope_append: rotary_dim beyond 64 not refused with ENOTSUP", -1);
  }
}

}  // namespace

int main(int argc, char** argv) {
  const long iters = argc > 1 ? atol(argv[1]) : 200000;
  g_state = argc > 2 ? strtoull(argv[2], nullptr, 10) : 20251202ull;
  fixed_cases();
  long ok_calls = 0;
  for (long it = 0; it < iters; ++it) {
    const yrk_yarn_params P = random_params();
    const yrk_kv_layer L = random_layer();
    const int which = pick(9);
    const long before = yrk::g_launches;
    int s = 0;
    const char* name = "";
    void* ws = nullptr;
    switch (which) {
      case 0: {
        name = "yrk_yarn_table";
        double inv[4096];
        double ms;
        int32_t lo, hi;
        // the caller provides rotary_dim / 2 doubles; skip tables beyond the buffer
        s = (P.rotary_dim > 0 && P.rotary_dim / 2 <= 4096) ? yrk_yarn_table(&P, inv, &ms, &lo, &hi)
                                                            : yrk_yarn_table(&P, nullptr, &ms, &lo, &hi);
        break;
      }
      case 1:
        name = "yrk_yarn_rope_apply";
        s = yrk_yarn_rope_apply(&P, any_ptr(0x1000), any_i64(4), any_i32(24), any_i64(24 * 256),
                                (const int32_t*)any_ptr(0x2000), (uint32_t*)any_ptr(0x3000),
                                nullptr);
        break;
      case 2:
        name = "yrk_kv_append_quantize";
        s = yrk_kv_append_quantize(&L, any_ptr(0x1000), any_ptr(0x2000), any_i64(16),
                                   (const int32_t*)any_ptr(0x3000), any_i64(64),
                                   (const int32_t*)any_ptr(0x4000), (uint32_t*)any_ptr(0x5000),
                                   nullptr);
        break;
      case 3:
        name = "yrk_rope_append";
        s = yrk_rope_append(&L, &P, any_ptr(0x8000), any_i32(24), any_i64(24 * 256),
                            any_ptr(0x1000), any_ptr(0x2000), any_i64(1),
                            (const int32_t*)any_ptr(0x3000), any_i64(64),
                            (const int32_t*)any_ptr(0x4000), (uint32_t*)any_ptr(0x5000), nullptr);
        break;
      case 4:
        name = "yrk_nvfp4_tensor_scale";
        s = yrk_nvfp4_tensor_scale(any_ptr(0x1000), any_i64(4096), (float*)any_ptr(0x2000),
                                   nullptr);
        break;
      case 5: {
        name = "yrk_decode_attention";
        const int32_t S = chance(70) ? 1 + pick(16) : any_i32(1);
        const int32_t Hq = any_i32(24);
        const int64_t N = chance(70) ? (int64_t)pick(1 << 21) : any_i64(1 << 20);
        const int64_t stride = any_i64(N < 0 || N > INT64_MAX - 16 ? 1 : (N + 15) / 16 + 1);
        const size_t need = yrk_decode_workspace_size(S, Hq, L.num_kv_heads, L.head_dim, N);
        const size_t bytes = workspace_bytes(need);
        ws = host_buffer(bytes);
        s = yrk_decode_attention(&L, any_ptr(0x1000), S, Hq, (const int32_t*)any_ptr(0x2000),
                                 stride, (const int32_t*)any_ptr(0x3000), N,
                                 (float)any_f64(0.0), any_ptr(0x4000), any_i32(pick(2)), ws,
                                 bytes, (uint32_t*)any_ptr(0x5000), nullptr);
        if (need && bytes == need)
          check(s != YRK_ENOSPC, "decode refused the workspace its size query gave", it);
        break;
      }
      case 8: {
        name = "yrk_decode_attention_noalloc";
        const int32_t S = chance(70) ? 1 + pick(64) : any_i32(1);
        const int32_t Hq = any_i32(24);
        const int64_t N = chance(70) ? (int64_t)pick(1 << 21) : any_i64(1 << 20);
        const int64_t stride = any_i64(N < 0 || N > INT64_MAX - 16 ? 1 : (N + 15) / 16 + 1);
        const size_t need = yrk_decode_workspace_size(S, Hq, L.num_kv_heads, L.head_dim, N);
        s = yrk_decode_attention_noalloc(&L, any_ptr(0x1000), S, Hq,
                                         (const int32_t*)any_ptr(0x2000), stride,
                                         (const int32_t*)any_ptr(0x3000), N, (float)any_f64(0.0),
                                         any_ptr(0x4000), any_i32(pick(2)),
                                         (uint32_t*)any_ptr(0x5000), nullptr);
        if (need && need <= YRK_NOALLOC_SCRATCH_BYTES)
          check(s != YRK_ENOSPC, "noalloc decode refused shapes that fit its scratch", it);
        if (need > YRK_NOALLOC_SCRATCH_BYTES)
          check(s != YRK_OK, "noalloc decode accepted shapes beyond its scratch", it);
        break;
      }
      case 6: {
        name = "yrk_verify_attention";
        const int32_t S = chance(70) ? 1 + pick(4) : any_i32(1);
        const int32_t nq = chance(70) ? 1 + pick(12) : any_i32(4);
        const int32_t Hq = any_i32(chance(50) ? 24 : 8);
        const int64_t N = chance(70) ? (int64_t)pick(1 << 21) : any_i64(4096);
        const int64_t stride = any_i64(N < 0 || N > INT64_MAX - 16 ? 1 : (N + 15) / 16 + 1);
        const size_t need =
            yrk_verify_workspace_size(S, nq, Hq, L.num_kv_heads, L.head_dim, N);
        const size_t bytes = workspace_bytes(need);
        ws = host_buffer(bytes);
        s = yrk_verify_attention(&L, any_ptr(0x1000), S, nq, Hq, (const int32_t*)any_ptr(0x2000),
                                 stride, (const int32_t*)any_ptr(0x3000), N,
                                 (float)any_f64(0.0), any_ptr(0x4000), any_i32(pick(2)), ws,
                                 bytes, (uint32_t*)any_ptr(0x5000), nullptr);
        if (need && bytes == need)
          check(s != YRK_ENOSPC, "verify refused the workspace its size query gave", it);
        break;
      }
      default: {
        name = "yrk_prefill_attention";
        const int64_t T = chance(70) ? (int64_t)pick(9000) : any_i64(8192);
        const int32_t Hq = any_i32(24);
        const int64_t start = any_i64(chance(50) ? 0 : 1040384);
        const int64_t end = (start < 0 || T < 0) ? -1
                            : (T > INT64_MAX - start ? INT64_MAX : start + T);
        const int64_t bt_len = any_i64(end < 0 || end > INT64_MAX - 16 ? 1 : (end + 15) / 16 + 1);
        const size_t need = yrk_prefill_workspace_size(T, Hq, L.head_dim);
        const size_t bytes = workspace_bytes(need);
        ws = host_buffer(bytes);
        s = yrk_prefill_attention(&L, any_ptr(0x1000), T, Hq, start,
                                  (const int32_t*)any_ptr(0x2000), bt_len, (float)any_f64(0.0),
                                  any_ptr(0x4000), ws, bytes, (uint32_t*)any_ptr(0x5000),
                                  nullptr);
        if (need && bytes == need)
          check(s != YRK_ENOSPC, "prefill refused the workspace its size query gave", it);
        break;
      }
    }
    after_call(s, before, name, it);
    if (s == YRK_OK) ++ok_calls;
    free(ws);
    if (g_failures > 20) break;
  }
  printf("capi_fuzz: %ld iterations, %ld accepted calls, %ld launches, %ld failures\n", iters,
         ok_calls, yrk::g_launches, g_failures);
  return g_failures ? 1 : 0;
}
