/*
 * Seeded synthetic inputs, host side.
 *
 * This module is shared by the oracle and by the GPU path and holds none of
 * the attention / rope / quantisation arithmetic.  It only turns (seed,
 * stream, index) into bf16 bit patterns.
 *
 * Generator: the counter form of SplitMix64 (G. Steele, D. Lea, C. Flood,
 * "Fast Splittable Pseudorandom Number Generators", OOPSLA 2014).  The i-th
 * output of a stream with initial state k is mix(k + (i+1)*GAMMA), so any
 * element can be drawn independently of the others.  The stream key is itself
 * mix(seed*GAMMA ^ stream*ODD).  synth_dev.hip implements the same definition
 * for the device; tests compare the two on sampled slices.
 *
 * Normal values: the top 16 bits of a draw index a 65,536-entry bf16 table of
 * N(0,1) quantiles that the Python side builds once (scipy ndtri, fp64, then
 * round-to-nearest-even to bf16) and passes in.
 */
#include <stdint.h>
#include <stddef.h>

#define SM_GAMMA 0x9e3779b97f4a7c15ULL
#define SM_ODD 0xd1342543de82ef95ULL

static inline uint64_t sm_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

static inline uint64_t sm_key(uint64_t seed, uint64_t stream) {
    return sm_mix((seed * SM_GAMMA) ^ (stream * SM_ODD));
}

static inline uint64_t sm_draw(uint64_t key, uint64_t idx) {
    return sm_mix(key + (idx + 1) * SM_GAMMA);
}

/* fp32 -> bf16, round to nearest even (inputs here are finite). */
static inline uint16_t f32_to_bf16_rne(float f) {
    union { float f; uint32_t u; } v;
    v.f = f;
    uint32_t u = v.u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static inline float bf16_to_f32(uint16_t h) {
    union { float f; uint32_t u; } v;
    v.u = ((uint32_t)h) << 16;
    return v.f;
}

/* Raw 64-bit draws, for tests of the generator itself. */
void synth_draws(uint64_t seed, uint64_t stream, uint64_t start, int64_t count, uint64_t *out) {
    uint64_t key = sm_key(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) out[i] = sm_draw(key, start + (uint64_t)i);
}

/*
 * Fill out[t][h][d] (t < ntok, h < nheads, d < dim) for logical tokens
 * token0 .. token0+ntok-1 of one tensor:
 *   x = table[draw(seed, stream, (t_abs*nheads + h)*dim + d) >> 48]
 *   x *= chan_mul[h*dim + d]                 (if chan_mul != NULL; power-of-two multipliers keep it exact)
 *   if draw(seed, outlier_stream, same index) >> 40 < outlier_thresh:
 *       x = bf16_rne(fp32(x) * outlier_mul)  (element outliers)
 */
void synth_fill_bf16(uint64_t seed, uint64_t stream, int64_t token0, int64_t ntok, int32_t nheads,
                     int32_t dim, const uint16_t *table, const float *chan_mul,
                     uint64_t outlier_stream, uint32_t outlier_thresh, float outlier_mul,
                     uint16_t *out) {
    uint64_t key = sm_key(seed, stream);
    uint64_t okey = sm_key(seed, outlier_stream);
    int64_t row = (int64_t)nheads * dim;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < ntok; ++t) {
        uint64_t base = (uint64_t)(token0 + t) * (uint64_t)row;
        uint16_t *o = out + t * row;
        for (int64_t e = 0; e < row; ++e) {
            uint64_t idx = base + (uint64_t)e;
            uint16_t x = table[sm_draw(key, idx) >> 48];
            if (chan_mul) x = f32_to_bf16_rne(bf16_to_f32(x) * chan_mul[e]);
            if (outlier_thresh && (uint32_t)(sm_draw(okey, idx) >> 40) < outlier_thresh)
                x = f32_to_bf16_rne(bf16_to_f32(x) * outlier_mul);
            o[e] = x;
        }
    }
}
