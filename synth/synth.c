/*
 * Seeded synthetic inputs for the Q8_0 projection path.
 *
 * This module only draws random numbers. It holds none of the quantize,
 * normalisation or dot-product arithmetic: both the HIP path (through the
 * tests and the benchmark) and the CPU oracle receive the arrays it fills.
 *
 * Generator (counter based, so any element can be drawn on its own):
 *   fmix(z)            = SplitMix64 output finaliser
 *                        z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
 *                        z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31
 *   at(state, i)       = fmix(state + (i + 1) * 0x9E3779B97F4A7C15)
 *                        (the i-th output of SplitMix64 started at `state`)
 *   base(seed, stream) = at(seed, stream)
 *   bits(seed,stream,i)= at(base(seed, stream), i)
 *   u(i)               = (bits >> 11) * 2^-53                 in [0, 1)
 *   normal pair p      : u1 = u(2p), u2 = u(2p + 1)
 *                        r = sqrt(-2 ln(1 - u1)), t = 2 pi u2
 *                        z[2p] = r cos t, z[2p + 1] = r sin t  (Box-Muller)
 *   value              = (float)(mean + std * z)               (f64, then f32)
 *
 * Every element depends only on (seed, stream, index), never on the thread
 * count or on how a tensor is split into calls.
 */
#include <math.h>
#include <stdint.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t fmix(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ULL;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBULL;
    z ^= z >> 31;
    return z;
}

static inline uint64_t at(uint64_t state, uint64_t i) { return fmix(state + (i + 1) * GOLDEN); }

static inline double unit(uint64_t b) { return (double)(b >> 11) * (1.0 / 9007199254740992.0); }

uint64_t synth_splitmix_at(uint64_t state, uint64_t i) { return at(state, i); }

uint64_t synth_bits(uint64_t seed, uint64_t stream, uint64_t i) { return at(at(seed, stream), i); }

double synth_unit(uint64_t seed, uint64_t stream, uint64_t i) { return unit(synth_bits(seed, stream, i)); }

static inline double normal_at(uint64_t base, uint64_t i) {
    uint64_t p = i >> 1;
    double u1 = unit(at(base, 2 * p));
    double u2 = unit(at(base, 2 * p + 1));
    double r = sqrt(-2.0 * log(1.0 - u1));
    double t = 6.283185307179586 * u2;
    return (i & 1) ? r * sin(t) : r * cos(t);
}

/* out[j] = (float)(mean + std * z[offset + j]) for j < n */
void synth_normal_f32(uint64_t seed, uint64_t stream, int64_t offset, int64_t n, double mean,
                      double std, float* out) {
    uint64_t base = at(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) out[j] = (float)(mean + std * normal_at(base, (uint64_t)(offset + j)));
}

/* out[j] = (float)(lo + (hi - lo) * u[offset + j]) */
void synth_uniform_f32(uint64_t seed, uint64_t stream, int64_t offset, int64_t n, double lo, double hi,
                       float* out) {
    uint64_t base = at(seed, stream);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) out[j] = (float)(lo + (hi - lo) * unit(at(base, (uint64_t)(offset + j))));
}

/* out[j] = lo + floor(u[offset + j] * (hi - lo + 1)), an integer in [lo, hi] */
void synth_uniform_i8(uint64_t seed, uint64_t stream, int64_t offset, int64_t n, int lo, int hi, int8_t* out) {
    uint64_t base = at(seed, stream);
    double span = (double)(hi - lo + 1);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        int v = lo + (int)floor(unit(at(base, (uint64_t)(offset + j))) * span);
        if (v > hi) v = hi;
        out[j] = (int8_t)v;
    }
}

/* n pseudo-random bytes: byte i is the low byte of draw offset+i of the stream. */
void synth_bytes(uint64_t seed, uint64_t stream, int64_t offset, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)(synth_bits(seed, stream, (uint64_t)(offset + i)) & 0xFF);
}
