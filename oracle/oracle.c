/*
 * oracle.c -- plain fp64 CPU oracle for YaRN-roped, GQA, paged long-context
 * attention (decode and chunked prefill) over a bf16, NVFP4 or INT8 KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg load this library.  The product path (the HIP library)
 * never calls it, and it shares no code, header, table or constant generator
 * with that path.
 *
 * Every function states the definition it writes out and the passage of the
 * source pages it follows.  Pages cited:
 *   [P1] "A 1,048,576-token context on two RTX 5090s: forking a C++ inference
 *        engine for tensor-parallel and YaRN" (portfolio-site-axx.pages.dev)
 *   [P3] "NInfer -- Windows 11 TP2 fork" README (git.onestrm.cn mirror)
 *   [P5] "262,144 Tokens on One RTX 5090: Qwen3.8-27B with an NVFP4 KV Cache
 *        That Actually Works" (stondo.github.io)
 *   [YaRN] Peng et al., "YaRN: Efficient Context Window Extension of Large
 *        Language Models", 2023 (cited by P1's references).
 *
 * Where the pages leave a step open, the reading taken is marked READING.
 * Parity status of each function is stated in its comment; all are pinned
 * except where it says "parity unpinned".
 *
 * Precision: fp64 throughout, compiled without fast-math or FMA contraction.
 */
#include <limits.h>
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bf16 <-> fp64                                                            */
/* ------------------------------------------------------------------------ */

/* bf16 bit pattern -> exact fp64 value. */
double orc_bf16_to_f64(uint16_t h) {
    union { float f; uint32_t u; } v;
    v.u = ((uint32_t)h) << 16;
    return (double)v.f;
}

/*
 * fp64 -> bf16, a single rounding to nearest, ties to even (no detour through
 * fp32, which could round twice).  bf16 keeps 8 significant bits; normal
 * exponents -126..127, subnormal step 2^-133.  Overflow -> inf, NaN -> 0x7fc0.
 */
uint16_t orc_f64_to_bf16(double x) {
    if (isnan(x)) return 0x7fc0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (a == 0.0) return sign;
    int e;
    double m = frexp(a, &e); /* a = m * 2^e, 0.5 <= m < 1 */
    int exp_unb = e - 1;     /* a = (2m) * 2^(e-1), 1 <= 2m < 2 */
    if (exp_unb >= -126) {
        double sig = nearbyint(ldexp(m, 8)); /* 128..256, exact scaling then RNE */
        if (sig == 256.0) { sig = 128.0; exp_unb += 1; }
        if (exp_unb > 127) return sign | 0x7f80;
        return sign | (uint16_t)((exp_unb + 127) << 7) | (uint16_t)((int)sig - 128);
    }
    /* subnormal: units of 2^-133, 0..128 (128 is the smallest normal) */
    double q = nearbyint(ldexp(a, 133));
    return sign | (uint16_t)(int)q;
}

void orc_round_bf16(const double *x, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_bf16(x[i]);
}

void orc_bf16_array_to_f64(const uint16_t *x, int64_t n, double *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_to_f64(x[i]);
}

/* ------------------------------------------------------------------------ */
/* C1: the YaRN frequency table                                              */
/* ------------------------------------------------------------------------ */

/*
 * Follows [P1] "YaRN, and matching what vLLM actually does" and [P3] "YaRN
 * reference and drift guard": a correction range of frequency-pair indices
 * decides which pairs are interpolated by the factor s and which keep their
 * trained frequency; mscale = 0.1 ln s + 1 multiplies cos/sin on the rotary
 * dimensions only.  The definition is [YaRN]'s "NTK-by-parts":
 *
 *   theta_i  = base^(-2i/d),                 i = 0 .. d/2-1, d = rotary dim
 *   corr(r)  = d * ln(L / (2 pi r)) / (2 ln base)
 *              (the pair index whose wavelength fits r full turns into L)
 *   low      = max(floor(corr(beta_fast)), 0)
 *   high     = min(ceil(corr(beta_slow)), d-1)          (READING: the clamps)
 *   ramp_i   = clamp((i - low) / (high - low), 0, 1)    (high == low -> +0.001, READING)
 *   inv_freq = theta_i / s * ramp_i + theta_i * (1 - ramp_i)
 *   mscale   = mscale_in if > 0, else 0.1 ln s + 1 for s > 1, else 1
 *
 * L is corr_max_pos when > 0, else orig_max_pos.  With base 1e7, d 64,
 * beta 32/1, the pages' two printed ranges come out: L = 262,144 -> (14, 22)
 * ("the paper's formula"), L = 4 x 262,144 -> (16, 24) ("as deployed").
 *
 * Returns 0, or -1 when a parameter is outside the domain where the
 * definition is meaningful.
 */
int orc_yarn_table(double base, int rot_dim, double factor, int64_t orig_max_pos,
                   int64_t corr_max_pos, double beta_fast, double beta_slow, double mscale_in,
                   double *inv_freq, double *mscale_out, int *low_out, int *high_out) {
    if (!(base > 1.0) || rot_dim <= 0 || (rot_dim & 1) || !(factor >= 1.0) || orig_max_pos <= 0 ||
        !(beta_fast > 0.0) || !(beta_slow > 0.0))
        return -1;
    const int half = rot_dim / 2;
    const double d = (double)rot_dim;
    const double L = (double)(corr_max_pos > 0 ? corr_max_pos : orig_max_pos);
    const double two_pi = 2.0 * 3.14159265358979323846;

    double corr_fast = d * log(L / (two_pi * beta_fast)) / (2.0 * log(base));
    double corr_slow = d * log(L / (two_pi * beta_slow)) / (2.0 * log(base));
    /* the clamps in double, as written: the unclamped ends can lie far outside
       the int range (a base just above 1), where a conversion is undefined */
    double lo = floor(corr_fast), hi = ceil(corr_slow);
    if (lo < 0.0) lo = 0.0;
    if (hi > d - 1.0) hi = d - 1.0;
    const int low = lo > (double)INT_MAX ? INT_MAX : (int)lo;
    const int high = hi < (double)INT_MIN ? INT_MIN : (int)hi;
    if (hi == lo) hi += 0.001;

    for (int i = 0; i < half; ++i) {
        double theta = pow(base, -2.0 * (double)i / d);
        double ramp = ((double)i - lo) / (hi - lo);
        if (ramp < 0.0) ramp = 0.0;
        if (ramp > 1.0) ramp = 1.0;
        inv_freq[i] = theta / factor * ramp + theta * (1.0 - ramp);
    }
    double ms;
    if (mscale_in > 0.0) ms = mscale_in;
    else ms = factor > 1.0 ? 0.1 * log(factor) + 1.0 : 1.0;
    if (mscale_out) *mscale_out = ms;
    if (low_out) *low_out = low;
    if (high_out) *high_out = high;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* C2: the rotation                                                          */
/* ------------------------------------------------------------------------ */

/*
 * Rotary embedding with the YaRN table ([P1] "YaRN, and matching what vLLM
 * actually does": mscale is applied to cos/sin on the rotary dimensions, no
 * attention-level factor; [P3] "YaRN reference and drift guard": 64 rotary
 * dimensions of each 256-dimension head).
 *
 * For token t at position p = pos[t], head h, pair i < d/2 (d = rot_dim):
 *   a = p * inv_freq[i]                      (fp64)
 *   c = mscale * cos a,  s = mscale * sin a
 *   y[i]       = x[i] c - x[i + d/2] s
 *   y[i + d/2] = x[i + d/2] c + x[i] s
 * and y[j] = x[j] for d <= j < head_dim.
 * READING: the pairing is "rotate half" (i with i + d/2) over the first d
 * dimensions; text positions are one-dimensional.  Pairing parity unpinned
 * against the deployed tables (they are not on the pages).
 *
 * x: bf16 [ntok][nheads] rows of head_dim, token stride tok_stride elements.
 * y: fp64 dense [ntok][nheads][head_dim].
 */
void orc_rope(const uint16_t *x, int64_t ntok, int nheads, int head_dim, int64_t tok_stride,
              int rot_dim, const int64_t *pos, const double *inv_freq, double mscale, double *y) {
    const int half = rot_dim / 2;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < ntok; ++t) {
        for (int h = 0; h < nheads; ++h) {
            const uint16_t *xr = x + t * tok_stride + (int64_t)h * head_dim;
            double *yr = y + (t * nheads + h) * (int64_t)head_dim;
            for (int i = 0; i < half; ++i) {
                double a = (double)pos[t] * inv_freq[i];
                double c = mscale * cos(a);
                double s = mscale * sin(a);
                double x1 = orc_bf16_to_f64(xr[i]);
                double x2 = orc_bf16_to_f64(xr[i + half]);
                yr[i] = x1 * c - x2 * s;
                yr[i + half] = x2 * c + x1 * s;
            }
            for (int j = rot_dim; j < head_dim; ++j) yr[j] = orc_bf16_to_f64(xr[j]);
        }
    }
}

/* Rope followed by the single bf16 rounding the cache/query storage applies. */
void orc_rope_bf16(const uint16_t *x, int64_t ntok, int nheads, int head_dim, int64_t tok_stride,
                   int rot_dim, const int64_t *pos, const double *inv_freq, double mscale,
                   uint16_t *y) {
    const int half = rot_dim / 2;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < ntok; ++t) {
        double row[4096];
        for (int h = 0; h < nheads; ++h) {
            const uint16_t *xr = x + t * tok_stride + (int64_t)h * head_dim;
            uint16_t *yr = y + (t * nheads + h) * (int64_t)head_dim;
            for (int i = 0; i < half; ++i) {
                double a = (double)pos[t] * inv_freq[i];
                double c = mscale * cos(a);
                double s = mscale * sin(a);
                double x1 = orc_bf16_to_f64(xr[i]);
                double x2 = orc_bf16_to_f64(xr[i + half]);
                row[i] = x1 * c - x2 * s;
                row[i + half] = x2 * c + x1 * s;
            }
            for (int i = 0; i < rot_dim; ++i) yr[i] = orc_f64_to_bf16(row[i]);
            for (int j = rot_dim; j < head_dim; ++j) yr[j] = xr[j];
        }
    }
}

/* ------------------------------------------------------------------------ */
/* C3: paging                                                                */
/* ------------------------------------------------------------------------ */

/*
 * Paged KV pool ([P1] "Things that bit me": page IDs per sequence; [P3]
 * "Current limits": one shared pool fixed at startup; [P5] "Validation
 * before vibes": the reader needs the HND layout).  READING of HND: a page
 * holds, per KV head, block_size consecutive tokens, each a contiguous row:
 *     pool byte offset of (block b, head h, slot j) = ((b*H + h)*block_size + j) * row_bytes
 * Logical token n of a sequence lives in block table[n / block_size], slot
 * n % block_size.
 *
 * Gathers logical rows [ntok][H][row_bytes] out of a pool.  Returns -1 if a
 * table entry is outside [0, num_blocks).
 */
int orc_gather_paged(const uint8_t *pool, int64_t num_blocks, int nheads, int block_size,
                     int64_t row_bytes, const int32_t *table, int64_t ntok, uint8_t *out) {
    for (int64_t n = 0; n < ntok; ++n) {
        int64_t b = table[n / block_size];
        if (b < 0 || b >= num_blocks) return -1;
        int64_t j = n % block_size;
        for (int h = 0; h < nheads; ++h) {
            const uint8_t *src = pool + ((b * nheads + h) * block_size + j) * row_bytes;
            memcpy(out + (n * nheads + h) * row_bytes, src, (size_t)row_bytes);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* C4: NVFP4                                                                 */
/* ------------------------------------------------------------------------ */

/*
 * NVFP4 KV ([P5] "Why NVFP4 KV changes the math": the KV cache itself is
 * quantised to NVFP4).  Format, as the workload fixes it: e2m1 element codes,
 * one e4m3 scale per 16 contiguous head-dim elements, one fp32 tensor scale S.
 *
 * e2m1: sign, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes
 *       {0, 0.5, 1, 1.5, 2, 3, 4, 6}; no inf/NaN.
 * e4m3 (OCP E4M3FN): sign, 4 exponent bits (bias 7), 3 mantissa bits;
 *       subnormals m/8 * 2^-6; max 448; 0x7F/0xFF are NaN; no inf.
 */
double orc_e2m1_value(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

double orc_e4m3_value(int code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/*
 * Tensor scale S = fl32(amax / (6 * 448)), amax = max |x| over the tensor.
 * READING: amax is taken per (layer, K or V) tensor; amax == 0 gives S = 1.
 */
float orc_nvfp4_tensor_scale(const uint16_t *x, int64_t n) {
    double amax = 0.0;
#pragma omp parallel for reduction(max : amax) schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double a = fabs(orc_bf16_to_f64(x[i]));
        if (a > amax) amax = a;
    }
    if (amax == 0.0) return 1.0f;
    return (float)(amax / 2688.0);
}

/*
 * Round a non-negative fp64 value to the nearest e4m3 code, ties to even
 * mantissa, saturating at 448 (0x7E).  Only exact scalings by powers of two
 * happen before the single nearbyint(), so the result is the correct
 * rounding of q.
 */
static int e4m3_rne_sat(double q) {
    if (!(q < 448.0)) return 0x7E;
    if (q < ldexp(1.0, -6)) {
        /* subnormal range: step 2^-9; a result of 8 is the smallest normal 0x08 */
        return (int)nearbyint(ldexp(q, 9));
    }
    int e;
    double m = frexp(q, &e); /* q = (2m) * 2^(e-1) */
    int ex = e - 1;
    double mm = nearbyint((2.0 * m - 1.0) * 8.0); /* 0..8 */
    if (mm == 8.0) { mm = 0.0; ex += 1; }
    int code = ((ex + 7) << 3) | (int)mm;
    if (code > 0x7E) code = 0x7E;
    return code;
}

/*
 * Quantise one bf16 tensor [ntok][nheads][head_dim] (head_dim % 16 == 0):
 *   for each 16-element block of one (token, head):
 *     b     = max |x_i|
 *     q_s   = RNE_e4m3(b / (6 S)), saturating at 448
 *     eff   = e4m3(q_s) * S                              (exact in fp64)
 *     code_i = sign(x_i) | RNE_e2m1(|x_i| / eff)  (ties to the even code,
 *              saturating at 6; eff == 0 gives magnitude 0)
 * The e2m1 rounding is done by exact comparison of |x_i| with the midpoints
 * m * eff (m in {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5}; every product is exact
 * in fp64), so no quotient is rounded before the decision.  b / (6 S) is an
 * fp64 quotient: b has 8 significant bits and 6S at most 27, so it never
 * lands on an e4m3 rounding midpoint unless the exact quotient does.
 * READING: the sign bit of x is kept, so -0 and tiny negatives give 0x8.
 *
 * codes:  one code per byte, [ntok][nheads][head_dim]
 * scales: [ntok][nheads][head_dim/16]
 */
void orc_nvfp4_quantize(const uint16_t *x, int64_t ntok, int nheads, int head_dim, float S,
                        uint8_t *codes, uint8_t *scales) {
    static const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
    const int nblk = head_dim / 16;
    const double Sd = (double)S;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < ntok; ++t) {
        for (int h = 0; h < nheads; ++h) {
            const uint16_t *xr = x + (t * nheads + h) * (int64_t)head_dim;
            uint8_t *cr = codes + (t * nheads + h) * (int64_t)head_dim;
            uint8_t *sr = scales + (t * nheads + h) * (int64_t)nblk;
            for (int blk = 0; blk < nblk; ++blk) {
                double b = 0.0;
                for (int i = 0; i < 16; ++i) {
                    double a = fabs(orc_bf16_to_f64(xr[blk * 16 + i]));
                    if (a > b) b = a;
                }
                int qs = e4m3_rne_sat(b / (6.0 * Sd));
                sr[blk] = (uint8_t)qs;
                double eff = orc_e4m3_value(qs) * Sd;
                double thr[7]; /* the midpoints of this block, m * eff */
                for (int k = 0; k < 7; ++k) thr[k] = mid[k] * eff;
                for (int i = 0; i < 16; ++i) {
                    uint16_t bits = xr[blk * 16 + i];
                    double a = fabs(orc_bf16_to_f64(bits));
                    int mag = 0;
                    if (eff > 0.0) {
                        for (int k = 0; k < 7; ++k) {
                            /* between code k and k+1: above the midpoint, or on it when k+1 is even */
                            if (a > thr[k] || (a == thr[k] && ((k + 1) & 1) == 0)) mag = k + 1;
                        }
                    }
                    cr[blk * 16 + i] = (uint8_t)(((bits >> 15) << 3) | mag);
                }
            }
        }
    }
}

/*
 * Packing of codes into bytes.  READING: element 2j goes to the low nibble
 * and element 2j+1 to the high nibble of byte j of a row.
 */
void orc_nvfp4_pack(const uint8_t *codes, int64_t n_pairs, uint8_t *packed) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n_pairs; ++j)
        packed[j] = (uint8_t)((codes[2 * j] & 0xF) | ((codes[2 * j + 1] & 0xF) << 4));
}

/* Dequantised value x^ = e2m1(code) * e4m3(scale) * S, exact in fp64. */
void orc_nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, int64_t ntok, int nheads,
                          int head_dim, float S, double *out) {
    const int nblk = head_dim / 16;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < ntok; ++t)
        for (int h = 0; h < nheads; ++h)
            for (int d = 0; d < head_dim; ++d) {
                int64_t r = t * nheads + h;
                out[r * head_dim + d] = orc_e2m1_value(codes[r * head_dim + d]) *
                                        orc_e4m3_value(scales[r * nblk + d / 16]) * (double)S;
            }
}

/* ------------------------------------------------------------------------ */
/* INT8 group-64 KV cache                                                   */
/* ------------------------------------------------------------------------ */
/*
 * [P3] "NInfer -- Windows 11 TP2 fork" (memory table) and [P1] "And the
 * memory picture": the deployed 1M-token cache is INT8 with groups of 64 and
 * takes 16.5 KiB per token per device, quantisation-scale planes included.
 * With 16 full-attention layers x 2 KV heads per device x 256 dims x (K, V)
 * one byte per element is 16 KiB, which leaves 512 B for 16 x 2 x 2 x 4
 * group scales: 2 bytes each.  The pages fix nothing else, so:
 * READING (symmetric absmax groups, the plainest scheme with one scale per
 * group): a group is 64 consecutive head dims of one (token, KV head);
 *   s    = RNE_fp16(max |x_i| / 127), saturating at 65504 (fp16 scales:
 *          READING, bf16 would give the same size)
 *   code = clamp(RNE(x_i / s), -127, 127) as a two's-complement byte, and 0
 *          when s == 0
 *   x^   = code * s
 */

/* IEEE binary16 bit pattern -> exact fp64 value (finite patterns). */
double orc_f16_value(uint16_t h) {
    int e = (h >> 10) & 0x1F, m = h & 0x3FF;
    double v = e ? ldexp(1.0 + m / 1024.0, e - 15) : ldexp((double)m, -24);
    if (e == 31) v = m ? NAN : INFINITY;
    return (h & 0x8000) ? -v : v;
}

/*
 * Non-negative fp64 -> nearest binary16, ties to even, saturating at the
 * largest finite value 65504 (READING).  Every step before the single
 * nearbyint() is an exact scaling by a power of two, so the result is the
 * correct rounding of x.
 */
uint16_t orc_f64_to_f16_sat(double x) {
    if (!(x < 65504.0)) return 0x7BFF;
    if (x < ldexp(1.0, -14))                       /* subnormal: step 2^-24 */
        return (uint16_t)nearbyint(ldexp(x, 24)); /* 1024 is the smallest normal, 0x0400 */
    int e;
    double f = frexp(x, &e);                        /* x = 2f * 2^(e-1), 2f in [1, 2) */
    int ex = e - 1;
    double mant = nearbyint((2.0 * f - 1.0) * 1024.0); /* 0 .. 1024 */
    if (mant == 1024.0) { mant = 0.0; ex += 1; }
    if (ex > 15) return 0x7BFF;
    return (uint16_t)(((ex + 15) << 10) | (int)mant);
}

/*
 * Quantise one bf16 tensor [ntok][nheads][head_dim] (head_dim % 64 == 0)
 * into codes [ntok][nheads][head_dim] (int8) and scales
 * [ntok][nheads][head_dim/64] (binary16 bits), by the rule above.
 * amax / 127 is an fp64 quotient: amax has 8 significant bits, so the exact
 * quotient is either an fp16 rounding midpoint exactly (and then so is the
 * fp64 value) or at least ~2^-20 of itself away from every midpoint, far
 * beyond fp64's error.  Likewise x / s (8 by 11 significant bits) is either
 * exactly a half-integer or at least 2^-12 away from one, so nearbyint of the
 * fp64 quotient is the rounding of the exact one.
 */
void orc_int8_quantize(const uint16_t *x, int64_t ntok, int nheads, int head_dim, int8_t *codes,
                       uint16_t *scales) {
    const int ngrp = head_dim / 64;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < ntok; ++t) {
        for (int h = 0; h < nheads; ++h) {
            const uint16_t *xr = x + (t * nheads + h) * (int64_t)head_dim;
            int8_t *cr = codes + (t * nheads + h) * (int64_t)head_dim;
            uint16_t *sr = scales + (t * nheads + h) * (int64_t)ngrp;
            for (int grp = 0; grp < ngrp; ++grp) {
                double amax = 0.0;
                for (int i = 0; i < 64; ++i) {
                    double a = fabs(orc_bf16_to_f64(xr[grp * 64 + i]));
                    if (a > amax) amax = a;
                }
                uint16_t sb = orc_f64_to_f16_sat(amax / 127.0);
                sr[grp] = sb;
                double sv = orc_f16_value(sb);
                for (int i = 0; i < 64; ++i) {
                    int c = 0;
                    if (sv > 0.0) {
                        double q = nearbyint(orc_bf16_to_f64(xr[grp * 64 + i]) / sv);
                        if (q > 127.0) q = 127.0;
                        if (q < -127.0) q = -127.0;
                        c = (int)q;
                    }
                    cr[grp * 64 + i] = (int8_t)c;
                }
            }
        }
    }
}

/* Dequantised value x^ = code * s, exact in fp64. */
void orc_int8_dequantize(const int8_t *codes, const uint16_t *scales, int64_t ntok, int nheads,
                         int head_dim, double *out) {
    const int ngrp = head_dim / 64;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < ntok; ++t)
        for (int h = 0; h < nheads; ++h)
            for (int d = 0; d < head_dim; ++d) {
                int64_t r = t * nheads + h;
                out[r * head_dim + d] = (double)codes[r * head_dim + d] *
                                        orc_f16_value(scales[r * ngrp + d / 64]);
            }
}

/* ------------------------------------------------------------------------ */
/* C5 / C6: attention                                                        */
/* ------------------------------------------------------------------------ */

/*
 * One cached key or value row (logical token n, KV head g) as fp64: either
 * the stored bf16 value, or the NVFP4 dequantised value.
 */
typedef struct {
    int kind; /* 0 = bf16 [N][Hkv][D] bit patterns; 1 = NVFP4 codes [N][Hkv][D] + scales [N][Hkv][D/16];
                 2 = INT8 codes [N][Hkv][D] + binary16 scales [N][Hkv][D/64] */
    const uint16_t *bf16;
    const uint8_t *codes;
    const uint8_t *scales;
    double S;
    /* NVFP4: orc_e2m1_value and orc_e4m3_value of every code, filled once by
       calling them (the same doubles; the products below are unchanged) */
    double e2m1[16], e4m3[256];
} orc_kv_view;

static void kv_view_tables(orc_kv_view *kv) {
    for (int c = 0; c < 16; ++c) kv->e2m1[c] = orc_e2m1_value(c);
    for (int c = 0; c < 256; ++c) kv->e4m3[c] = orc_e4m3_value(c);
}

static void kv_row(const orc_kv_view *kv, int64_t n, int g, int Hkv, int D, double *row) {
    int64_t r = n * Hkv + g;
    if (kv->kind == 0) {
        const uint16_t *p = kv->bf16 + r * D;
        for (int d = 0; d < D; ++d) row[d] = orc_bf16_to_f64(p[d]);
    } else if (kv->kind == 1) {
        const uint8_t *c = kv->codes + r * D;
        const uint8_t *s = kv->scales + r * (D / 16);
        for (int d = 0; d < D; ++d)
            row[d] = kv->e2m1[c[d] & 0xF] * kv->e4m3[s[d / 16]] * kv->S;
    } else {
        const int8_t *c = (const int8_t *)kv->codes + r * D;
        const uint16_t *s = (const uint16_t *)kv->scales + r * (D / 64);
        for (int d = 0; d < D; ++d) row[d] = (double)c[d] * orc_f16_value(s[d / 64]);
    }
}

/*
 * Single-query attention of query head h over cached tokens 0..N-1 of KV
 * head g = h / (Hq / Hkv) (READING: consecutive grouping of the GQA heads;
 * [P5] "Why NVFP4 KV changes the math": 4 KV heads x 256):
 *   z_n = scale * <q_h, K_n>
 *   o_h = sum_n softmax(z)_n V_n,   computed as exp(z_n - max z) / sum.
 * scale is the plain softmax scale (READING: 1/sqrt(D); [P1] rules out an
 * extra attention-level YaRN factor).  N == 0 gives o = 0 and lse = -inf.
 * lse_h = max z + ln sum exp(z - max z), the natural-log normaliser.
 * The sums run in token order.
 */
static void attend_one_head(const double *qh, const orc_kv_view *kview, const orc_kv_view *vview,
                            int g, int Hkv, int D, int64_t N, double scale, double *oh,
                            double *lse_h) {
    for (int d = 0; d < D; ++d) oh[d] = 0.0;
    if (N <= 0) {
        if (lse_h) *lse_h = -INFINITY;
        return;
    }
    double *z = (double *)malloc((size_t)N * sizeof(double));
    double *row = (double *)malloc((size_t)D * sizeof(double));
    double zmax = -INFINITY;
    for (int64_t n = 0; n < N; ++n) {
        kv_row(kview, n, g, Hkv, D, row);
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += qh[d] * row[d];
        z[n] = scale * acc;
        if (z[n] > zmax) zmax = z[n];
    }
    double l = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        double w = exp(z[n] - zmax);
        l += w;
        kv_row(vview, n, g, Hkv, D, row);
        for (int d = 0; d < D; ++d) oh[d] += w * row[d];
    }
    for (int d = 0; d < D; ++d) oh[d] /= l;
    if (lse_h) *lse_h = zmax + log(l);
    free(z);
    free(row);
}

/*
 * Decode attention for one sequence: q [Hq][D] fp64 (the roped query as the
 * kernel sees it), cache of N tokens, out [Hq][D], lse [Hq] (nullable).
 * kv_kind 0: k/v are bf16 [N][Hkv][D].  kv_kind 1: k/v are NVFP4 codes (one
 * per byte) [N][Hkv][D] with scales [N][Hkv][D/16] and tensor scales kS/vS.
 * kv_kind 2: k/v are INT8 codes [N][Hkv][D] with binary16 scales
 * [N][Hkv][D/64] (passed as bytes; kS/vS unused).
 * Heads are independent and run in parallel.
 */
int orc_decode_attention(const double *q, int Hq, int Hkv, int D, int64_t N, int kv_kind,
                         const void *k, const void *v, const uint8_t *k_scales,
                         const uint8_t *v_scales, float kS, float vS, double scale, double *out,
                         double *lse) {
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || N < 0) return -1;
    if (kv_kind < 0 || kv_kind > 2) return -1;
    if (kv_kind == 1 && D % 16) return -1;
    if (kv_kind == 2 && D % 64) return -1;
    orc_kv_view kview = {kv_kind, (const uint16_t *)k, (const uint8_t *)k, k_scales, (double)kS};
    orc_kv_view vview = {kv_kind, (const uint16_t *)v, (const uint8_t *)v, v_scales, (double)vS};
    kv_view_tables(&kview);
    kv_view_tables(&vview);
    const int group = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int h = 0; h < Hq; ++h)
        attend_one_head(q + (int64_t)h * D, &kview, &vview, h / group, Hkv, D, N, scale,
                        out + (int64_t)h * D, lse ? lse + h : NULL);
    return 0;
}

/*
 * Causal chunked prefill ([P1] "Against vLLM: prefill loses, decode wins":
 * prompts are prefilled in chunks into the cache; READING: standard causal
 * attention including the token itself, with the chunk's own keys already
 * appended).  Row r (query q[r] at position pos[r]) attends to cached tokens
 * 0..pos[r], i.e. it is the decode definition with N = pos[r] + 1.
 * q: [R][Hq][D] fp64; out: [R][Hq][D].  The KV arrays must cover max pos + 1
 * tokens.  Every (row, head) pair is independent; they run in parallel.
 */
int orc_prefill_attention(const double *q, const int64_t *pos, int64_t R, int Hq, int Hkv, int D,
                          int kv_kind, const void *k, const void *v, const uint8_t *k_scales,
                          const uint8_t *v_scales, float kS, float vS, double scale, double *out) {
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || R < 0) return -1;
    if (kv_kind < 0 || kv_kind > 2) return -1;
    if (kv_kind == 1 && D % 16) return -1;
    if (kv_kind == 2 && D % 64) return -1;
    for (int64_t r = 0; r < R; ++r)
        if (pos[r] < 0) return -1;
    orc_kv_view kview = {kv_kind, (const uint16_t *)k, (const uint8_t *)k, k_scales, (double)kS};
    orc_kv_view vview = {kv_kind, (const uint16_t *)v, (const uint8_t *)v, v_scales, (double)vS};
    kv_view_tables(&kview);
    kv_view_tables(&vview);
    const int group = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t r = 0; r < R; ++r)
        for (int h = 0; h < Hq; ++h)
            attend_one_head(q + (r * Hq + h) * (int64_t)D, &kview, &vview, h / group, Hkv, D,
                            pos[r] + 1, scale, out + (r * Hq + h) * (int64_t)D, NULL);
    return 0;
}

/* Threads an OpenMP loop of this library runs on (reported next to timings;
 * no arithmetic depends on it). */
int orc_num_threads(void) { return omp_get_max_threads(); }
