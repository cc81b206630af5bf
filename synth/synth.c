/*
 * synth.c - seeded synthetic inputs for the MoE-layer workloads.
 *
 * This module performs no step of the MoE method (no routing, scoring,
 * permutation, FFN or combine).  It only draws random numbers and rounds the
 * drawn values into the storage formats the layer consumes.  Both the CPU
 * oracle and the GPU library receive the arrays it fills; neither links it.
 *
 * Random source: SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) with the "Mix13" finaliser
 * constants published by D. Stafford.  It is used counter-style: element i of
 * stream s under master seed S is a pure function of (S, s, i), so any slice of
 * a tensor (one expert, one token) can be regenerated on its own.
 *
 * Normal deviates: Irwin-Hall sum of twelve uniforms, centred (the classical
 * "sum of 12 uniforms minus 6" approximation of N(0,1); support +-6 sigma,
 * kurtosis 2.9).  Only integer operations and exact fp64 scalings are used,
 * so the result is identical on every IEEE machine.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (see build.py).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SM_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* Initial SplitMix64 state of stream `stream` under master seed `seed`. */
static inline uint64_t stream_state(uint64_t seed, uint64_t stream) {
    return sm_mix(sm_mix(seed + SM_GAMMA) ^ (stream * 0xD1B54A32D192ED03ULL + 1));
}

/* The i-th SplitMix64 output of a stream whose state is `st`. */
static inline uint64_t draw(uint64_t st, uint64_t i) { return sm_mix(st + (i + 1) * SM_GAMMA); }

/* Approximately N(0,1): twelve 16-bit uniforms from three draws, centred and
 * divided by 2^16 (each uniform has variance (2^32-1)/12, so the sum has
 * standard deviation sqrt(2^32-1), within 2^-33 of 2^16).  Exact in fp64. */
static inline double std_normal(uint64_t st, uint64_t i) {
    uint64_t s = 0;
    for (int d = 0; d < 3; ++d) {
        uint64_t r = draw(st, 3 * i + (uint64_t)d);
        s += (r & 0xFFFF) + ((r >> 16) & 0xFFFF) + ((r >> 32) & 0xFFFF) + (r >> 48);
    }
    return ((double)s - 393210.0) / 65536.0; /* 393210 = 12 * 32767.5 */
}

/* Uniform on [0,1) with 53 random bits. */
static inline double unit_uniform(uint64_t st, uint64_t i) {
    return (double)(draw(st, i) >> 11) * 0x1.0p-53;
}

static inline uint16_t f32_to_bf16_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u); /* quiet NaN */
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* IEEE binary16, round-to-nearest-even, directly from a double. */
static uint16_t f64_to_f16_bits(double d) {
    uint16_t sign = signbit(d) ? 0x8000u : 0;
    double a = fabs(d);
    if (isnan(d)) return 0x7E00u;
    if (a == 0.0) return sign;
    int e;
    double m = frexp(a, &e);         /* a = m * 2^e, m in [0.5, 1) */
    double r;
    if (e - 1 >= -14) {
        r = ldexp(rint(ldexp(m, 11)), e - 11); /* 11 significant bits */
    } else {
        r = ldexp(rint(ldexp(a, 24)), -24);    /* subnormal quantum 2^-24 */
    }
    if (r >= 65536.0) return (uint16_t)(sign | 0x7C00u); /* rounded past the largest finite */
    if (r == 0.0) return sign;
    m = frexp(r, &e);
    if (e - 1 >= -14) {
        uint32_t frac = (uint32_t)(ldexp(m, 11) - 1024.0); /* exact: 10 fraction bits */
        return (uint16_t)(sign | ((uint32_t)(e - 1 + 15) << 10) | frac);
    }
    return (uint16_t)(sign | (uint32_t)ldexp(r, 24));
}

static double f16_bits_to_f64(uint16_t h) {
    int ex = (h >> 10) & 0x1F, fr = h & 0x3FF;
    double v;
    if (ex == 0) v = ldexp((double)fr, -24);
    else if (ex == 31) v = fr ? NAN : INFINITY;
    else v = ldexp((double)(fr | 0x400), ex - 25);
    return (h & 0x8000u) ? -v : v;
}

/* Elements [start, start+n) of stream `stream`: mean + sigma * N(0,1), as fp32. */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n,
                      double mean, double sigma, float *out) {
    uint64_t st = stream_state(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        double v = mean + sigma * std_normal(st, start + (uint64_t)i);
        out[i] = (float)v;
    }
}

/* Same draws, stored as bf16 bits (fp32 first, then round-to-nearest-even). */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n,
                       double mean, double sigma, uint16_t *out) {
    uint64_t st = stream_state(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < (int64_t)n; ++i) {
        double v = mean + sigma * std_normal(st, start + (uint64_t)i);
        out[i] = f32_to_bf16_bits((float)v);
    }
}

/* Same draws quantised to int8 blocks of 32 along each row, one fp16 scale per
 * block: scale = fp16(amax/127), q = clamp(rint(w/scale), -127, 127); an
 * all-zero block gets scale 0 and q = 0.  Rows [row0, row0+n_rows) of a
 * row-major matrix with `cols` columns (cols % 32 == 0); element (r, c) is
 * draw index r*cols + c.  q: [n_rows, cols], scale: [n_rows, cols/32]. */
void synth_q8b32(uint64_t seed, uint64_t stream, uint64_t row0, uint64_t n_rows, uint64_t cols,
                 double sigma, int8_t *q, uint16_t *scale) {
    uint64_t st = stream_state(seed, stream);
    uint64_t nb = cols / 32;
#pragma omp parallel for schedule(static)
    for (int64_t rb = 0; rb < (int64_t)(n_rows * nb); ++rb) {
        uint64_t r = (uint64_t)rb / nb, b = (uint64_t)rb % nb;
        uint64_t base = (row0 + r) * cols + b * 32;
        double w[32], amax = 0.0;
        for (int j = 0; j < 32; ++j) {
            w[j] = sigma * std_normal(st, base + (uint64_t)j);
            if (fabs(w[j]) > amax) amax = fabs(w[j]);
        }
        uint16_t sb = f64_to_f16_bits(amax / 127.0);
        double sf = f16_bits_to_f64(sb);
        scale[r * nb + b] = sb;
        for (int j = 0; j < 32; ++j) {
            double v = sf > 0.0 ? rint(w[j] / sf) : 0.0;
            if (v > 127.0) v = 127.0;
            if (v < -127.0) v = -127.0;
            q[r * cols + b * 32 + (uint64_t)j] = (int8_t)v;
        }
    }
}

/* Elements [start, start+n) uniform on [lo, hi), as fp32. */
void synth_uniform_f32(uint64_t seed, uint64_t stream, uint64_t start, uint64_t n,
                       double lo, double hi, float *out) {
    uint64_t st = stream_state(seed, stream);
    for (uint64_t i = 0; i < n; ++i) out[i] = (float)(lo + (hi - lo) * unit_uniform(st, start + i));
}

/* A seeded popularity ranking of n experts (Fisher-Yates over draws of the
 * stream) and the skew bias b_e = -beta * ln(rank_e), rank 1 = hottest.
 * rank_out (optional) receives the 1-based ranks. */
void synth_zipf_bias(uint64_t seed, uint64_t stream, int32_t n, double beta,
                     float *bias_out, int32_t *rank_out) {
    uint64_t st = stream_state(seed, stream);
    int32_t perm[4096];
    if (n < 1 || n > 4096) return;
    for (int32_t i = 0; i < n; ++i) perm[i] = i;
    for (int32_t i = n - 1; i > 0; --i) {
        int32_t j = (int32_t)(draw(st, (uint64_t)(n - 1 - i)) % (uint64_t)(i + 1));
        int32_t t = perm[i];
        perm[i] = perm[j];
        perm[j] = t;
    }
    /* perm[p] = expert holding popularity position p (0 = hottest) */
    for (int32_t p = 0; p < n; ++p) {
        int32_t e = perm[p];
        if (rank_out) rank_out[e] = p + 1;
        bias_out[e] = (float)(-beta * log((double)(p + 1)));
    }
}
