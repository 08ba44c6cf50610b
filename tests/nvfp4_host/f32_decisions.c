// Host check of the NVFP4 append kernels' fp32 element decisions: the binary
// search over the e2m1 decision points with fused multiply-adds (as in
// nvfp4_code_f32) against the fp64 decisions of the definition (nvfp4_code),
// for every e4m3 block scale, every positive finite bf16 magnitude (on 11
// tensor scales, a stride of 61 on 389 more) and the bf16 neighbours of every
// decision point, over tensor scales in [2^-109, 2^100].  Exit status 0 when
// every decision agrees.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
static float bf16f(uint16_t b) { uint32_t u = (uint32_t)b << 16; float f; memcpy(&f, &u, 4); return f; }
static double e4m3v(int c) {  // OCP E4M3FN
  int e = (c >> 3) & 15, m = c & 7;
  if (e == 0) return ldexp(m, -9);
  return ldexp(8 + m, e - 10);
}
static unsigned code64(double a, double e) {
  if (!(e > 0)) return 0;
  return (a > 0.25 * e) + (a >= 0.75 * e) + (a > 1.25 * e) + (a >= 1.75 * e) + (a > 2.5 * e) +
         (a >= 3.5 * e) + (a > 5.0 * e);
}
static unsigned code32(float a, float e4, float S, int qs) {
  int c1 = fmaf(-1.75f * e4, S, a) >= 0.0f;
  int c2 = fmaf(-(c1 ? 3.5f : 0.75f) * e4, S, a) >= 0.0f;
  float t3 = c1 ? (c2 ? 5.0f : 2.5f) : (c2 ? 1.25f : 0.25f);
  int c3 = fmaf(-t3 * e4, S, a) > 0.0f;
  return qs == 0 ? 0 : (unsigned)(c1 * 4 + c2 * 2 + c3);
}
int main(void) {
  uint64_t x = 88172645463325252ull, n = 0, bad = 0;
  float Ss[4096]; int ns = 0;
  float edge[] = {1.0f, 0x1p-109f, 0x1p-100f, 0x1p100f, 0x1.fffffep99f, 0x1.000002p-109f, 1.0f / 2688.0f,
                  3.0f, 0.1f, 7e-30f, 1e30f};
  for (unsigned i = 0; i < sizeof edge / sizeof *edge; ++i) Ss[ns++] = edge[i];
  while (ns < 400) {  // random fp32 S in [2^-109, 2^100]
    x ^= x << 13; x ^= x >> 7; x ^= x << 17;
    int ex = (int)(x % 210) - 109;
    float m = 1.0f + (float)((x >> 20) & 0x7fffff) / 8388608.0f;
    Ss[ns++] = ldexpf(m, ex);
  }
  for (int si = 0; si < ns; ++si) {
    float S = Ss[si];
    if (!(S >= 0x1p-109f && S <= 0x1p100f)) continue;
    for (int qs = 0; qs < 0x7F; ++qs) {
      double e4 = e4m3v(qs);
      double eff = e4 * (double)S;
      float e4f = (float)e4;
      // all positive finite bf16 magnitudes and those near the decision points
      for (uint32_t b = 0; b < 0x7F80; b += (si < 11 ? 1 : 61)) {
        float a = bf16f((uint16_t)b);
        unsigned r64 = code64((double)a, eff), r32 = code32(a, e4f, S, qs);
        ++n;
        if (r64 != r32) { if (bad < 10) printf("mismatch S=%a qs=%d a=%a: %u vs %u\n", S, qs, a, r64, r32); ++bad; }
      }
      // the bf16 neighbours of every decision point t*eff
      static const double T[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
      for (int k = 0; k < 7; ++k) {
        float p = (float)(T[k] * eff);
        uint32_t u; memcpy(&u, &p, 4);
        uint32_t hb = u >> 16;
        for (int d = -3; d <= 3; ++d) {
          uint32_t b = hb + d;
          if (b >= 0x7F80) continue;
          float a = bf16f((uint16_t)b);
          unsigned r64 = code64((double)a, eff), r32 = code32(a, e4f, S, qs);
          ++n;
          if (r64 != r32) { if (bad < 10) printf("mismatch S=%a qs=%d a=%a: %u vs %u\n", S, qs, a, r64, r32); ++bad; }
        }
      }
    }
  }
  printf("checked %llu (a, e4, S) triples, %llu mismatches\n", (unsigned long long)n, (unsigned long long)bad);
  return bad != 0;
}
