/*
 * CPU oracle for the Q8_0 quantized projection path -- TEST INFRASTRUCTURE.
 * See q8_oracle.h for who may use it and for the page titles cited below as
 * [P1], [P2], [P3].
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp (no -ffast-math). OpenMP only
 * splits independent rows or output pairs; the operation order inside each
 * result is fixed, so results do not depend on the thread count.
 */
#include "q8_oracle.h"

#include <math.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QK 32 /* elements per q8_0 block: [P1] s2.1, [P2] s2.1 */

int q8o_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the following oracle calls use (timing only; results do not depend on it). */
void q8o_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------
 * IEEE-754 binary16 conversion, written from the format definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; subnormals have
 * exponent field 0 and value frac * 2^-24. Rounding is to nearest, ties to
 * even; values at or above 65520 round to infinity.
 * ---------------------------------------------------------------------- */
uint16_t q8o_f32_to_f16(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t ef = (x >> 23) & 0xffu;
    uint32_t frac = x & 0x7fffffu;
    if (ef == 0xffu) { /* infinity or NaN (NaN stays quiet NaN) */
        return (uint16_t)(sign | 0x7c00u | (frac ? (0x200u | (frac >> 13)) : 0u));
    }
    if (ef == 0u) return (uint16_t)sign; /* f32 subnormal or zero: far below half the f16 subnormal step */
    int e = (int)ef - 127;               /* value = m * 2^(e-23), m = 2^23 + frac */
    uint32_t m = 0x800000u | frac;
    if (e > 15) return (uint16_t)(sign | 0x7c00u);
    if (e >= -14) {
        /* normal target: keep 11 significant bits, drop 13 */
        uint32_t q = m >> 13, rem = m & 0x1fffu;
        if (rem > 0x1000u || (rem == 0x1000u && (q & 1u))) q++;
        /* q in [1024, 2048]; a carry to 2048 moves into the next binade (and to inf past 65504) */
        uint32_t bits = ((uint32_t)(e + 15) << 10) + (q - 1024u);
        return (uint16_t)(sign | bits);
    }
    /* subnormal target: units of 2^-24, value in those units = m * 2^(e+1) */
    int shift = -(e + 1); /* >= 14 */
    if (shift > 24) return (uint16_t)sign; /* below half of the smallest step 2^-24 */
    uint32_t q = m >> shift;
    uint32_t rem = m & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q++;
    return (uint16_t)(sign | q); /* q == 1024 is the smallest normal, encoded the same way */
}

float q8o_f16_to_f32(uint16_t h) {
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t ef = (h >> 10) & 0x1fu;
    uint32_t frac = h & 0x3ffu;
    float v;
    if (ef == 0x1fu) {
        uint32_t bits = sign | 0x7f800000u | (frac << 13);
        memcpy(&v, &bits, 4);
        return v;
    }
    if (ef == 0u) {
        v = ldexpf((float)frac, -24); /* exact: frac < 2^10 */
    } else {
        v = ldexpf((float)(1024u + frac), (int)ef - 25);
    }
    return sign ? -v : v;
}

void q8o_f32_to_f16_array(const float* x, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = q8o_f32_to_f16(x[i]);
}

/* ------------------------------------------------------------------------
 * Activation quantize of one 32-element block.
 * [P2] s3.2 (phase-2 quantize body): amax = max |x_j|; d = amax / 127 in
 *   f32; q_j = rint of x_j scaled by 1/d, clamped; d stored as f16;
 *   ssum = sum of q_j (int16).
 * [P2] s2.1 gives the f16 d and int16 ssum packed into one 4-byte word.
 * Readings (pages silent or inconsistent):
 *   - x/d is an IEEE f32 division (not a multiply by a reciprocal);
 *   - rint rounds half to even;
 *   - a block with amax = 0 (so d = 0) stores d = 0, q = 0, ssum = 0;
 *   - the clamp is [-127, 127]; |x/d| <= 127 (+1 ulp) so -128 never occurs.
 * ---------------------------------------------------------------------- */
static void quantize_block(const float* x, uint16_t* d16, int8_t* q, int16_t* ssum) {
    float amax = 0.0f;
    for (int j = 0; j < QK; ++j) {
        float a = fabsf(x[j]);
        if (a > amax) amax = a;
    }
    float d = amax / 127.0f;
    *d16 = q8o_f32_to_f16(d);
    int s = 0;
    for (int j = 0; j < QK; ++j) {
        int v = 0;
        if (d != 0.0f) {
            v = (int)rintf(x[j] / d);
            if (v > 127) v = 127;
            if (v < -127) v = -127;
        }
        q[j] = (int8_t)v;
        s += v;
    }
    *ssum = (int16_t)s;
}

void q8o_quantize_rows(const float* x, int64_t rows, int64_t K, int8_t* qs, uint16_t* d16, int16_t* ssum) {
    int64_t nb = K / QK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            quantize_block(x + r * K + b * QK, d16 + r * nb + b, qs + r * K + b * QK, ssum + r * nb + b);
        }
    }
}

void q8o_pack_sd(const uint16_t* d16, const int16_t* ssum, int64_t n, uint32_t* sd) {
    for (int64_t i = 0; i < n; ++i) sd[i] = (uint32_t)d16[i] | ((uint32_t)(uint16_t)ssum[i] << 16);
}

/* ------------------------------------------------------------------------
 * PLANE64 layout: tokens grouped 64 at a time ([P2] s2.1: the token dimension
 * is grouped in 64s and padded), one 2048-byte qs tile and 64 scale words per
 * (group, 32-element chunk). The byte placement inside a tile is the one
 * the HIP library documents for its plane (the pages' XOR formula targets
 * another GPU's memory banks):
 *   token r = t mod 64 owns bytes [32r, 32r + 32) of the tile;
 *   its 16-byte half h (elements 16h..16h+15) sits at half position
 *   h ^ (((r >> 2) ^ (r >> 3)) & 1).
 * Tokens t >= T up to the 64-padded count are all zero ([P2] s3.1, tail fill).
 * ---------------------------------------------------------------------- */
int64_t q8o_plane_qs_offset(int64_t t, int64_t k, int64_t K) {
    int64_t nchunk = K / QK;
    int64_t g = t / 64, r = t % 64, c = k / QK, e = k % QK;
    int64_t h = (e / 16) ^ (((r >> 2) ^ (r >> 3)) & 1);
    return (g * nchunk + c) * 2048 + r * 32 + h * 16 + (e % 16);
}

int64_t q8o_plane_sd_index(int64_t t, int64_t c, int64_t K) {
    int64_t nchunk = K / QK;
    return (t / 64 * nchunk + c) * 64 + t % 64;
}

void q8o_encode_plane64(const int8_t* qs, const uint16_t* d16, const int16_t* ssum, int64_t T, int64_t K,
                        int8_t* pqs, uint32_t* psd) {
    int64_t nb = K / QK, tpad = (T + 63) / 64 * 64;
    for (int64_t t = 0; t < tpad; ++t) {
        for (int64_t k = 0; k < K; ++k) pqs[q8o_plane_qs_offset(t, k, K)] = (t < T) ? qs[t * K + k] : 0;
        for (int64_t c = 0; c < nb; ++c) {
            uint32_t w = 0;
            if (t < T) w = (uint32_t)d16[t * nb + c] | ((uint32_t)(uint16_t)ssum[t * nb + c] << 16);
            psd[q8o_plane_sd_index(t, c, K)] = w;
        }
    }
}

/* Inverse of the encode for rows t < T; returns the number of nonzero bytes
 * found in the padded tail (qs and scale words), which must be 0. */
int64_t q8o_decode_plane64(const int8_t* pqs, const uint32_t* psd, int64_t T, int64_t K, int8_t* qs,
                           uint16_t* d16, int16_t* ssum) {
    int64_t nb = K / QK, tpad = (T + 63) / 64 * 64, bad = 0;
    for (int64_t t = 0; t < tpad; ++t) {
        for (int64_t k = 0; k < K; ++k) {
            int8_t v = pqs[q8o_plane_qs_offset(t, k, K)];
            if (t < T) qs[t * K + k] = v;
            else bad += (v != 0);
        }
        for (int64_t c = 0; c < nb; ++c) {
            uint32_t w = psd[q8o_plane_sd_index(t, c, K)];
            if (t < T) {
                d16[t * nb + c] = (uint16_t)(w & 0xffffu);
                ssum[t * nb + c] = (int16_t)(uint16_t)(w >> 16);
            } else {
                bad += (w != 0);
            }
        }
    }
    return bad;
}

/* ------------------------------------------------------------------------
 * RMSNorm: [P2] s3.2 (rms_norm_f32 / phase 1 of the fused kernel):
 *   y_j = x_j * w_j / sqrt(mean_j(x_j^2) + eps), here in f64.
 * ---------------------------------------------------------------------- */
void q8o_rmsnorm_f64(const float* x, const float* w, int64_t rows, int64_t K, double eps, double* y) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float* xr = x + r * K;
        double ss = 0.0;
        for (int64_t j = 0; j < K; ++j) ss += (double)xr[j] * (double)xr[j];
        double inv = 1.0 / sqrt(ss / (double)K + eps);
        for (int64_t j = 0; j < K; ++j) y[r * K + j] = (double)xr[j] * inv * (double)w[j];
    }
}

/* SwiGLU: [P2] s3.2 (swiglu_f32 / phase 1): y = g / (1 + e^-g) * u, in f64. */
void q8o_swiglu_f64(const float* g, const float* u, int64_t n, double* y) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        double gv = (double)g[i];
        y[i] = gv / (1.0 + exp(-gv)) * (double)u[i];
    }
}

/* ------------------------------------------------------------------------
 * Weights. [P1] s2.1: a GGUF Q8_0 block is 34 bytes, alignment 2: f16 d at
 * +0, then int8 qs[32] at +2; block b of a row starts at byte 34*b. The f32
 * weights are quantized with the same per-block rule as activations.
 * ---------------------------------------------------------------------- */
void q8o_quantize_weights_gguf(const float* w, int64_t N, int64_t K, uint8_t* blocks) {
    int64_t nb = K / QK;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            uint16_t d16;
            int8_t q[QK];
            int16_t s;
            quantize_block(w + n * K + b * QK, &d16, q, &s);
            uint8_t* blk = blocks + (n * nb + b) * 34;
            blk[0] = (uint8_t)(d16 & 0xff); /* little-endian f16 */
            blk[1] = (uint8_t)(d16 >> 8);
            memcpy(blk + 2, q, QK);
        }
    }
}

void q8o_gguf_to_planar(const uint8_t* blocks, int64_t N, int64_t K, int8_t* qs, uint16_t* d) {
    int64_t nb = K / QK;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t* blk = blocks + (n * nb + b) * 34;
            d[n * nb + b] = (uint16_t)(blk[0] | (blk[1] << 8));
            memcpy(qs + n * K + b * QK, blk + 2, QK);
        }
    }
}

/* ------------------------------------------------------------------------
 * Block-scaled dot product of one weight row n with one activation row t
 * ([P1] s2.2: integer dot product per block, then the two block scales):
 *   isum_b = sum_{j<32} qw[n, 32b+j] * qa[t, 32b+j]            (exact int32)
 *   ref    = sum_b f16(dw[n,b]) * f16(da[t,b]) * isum_b        (f64)
 *   norm   = sum_b |f16(dw[n,b]) * f16(da[t,b]) * isum_b|
 * Each product dw*da*isum is exact in f64 (11+11+20 bits); only the sum over
 * b rounds.
 * ---------------------------------------------------------------------- */
static int32_t block_isum(const int8_t* a, const int8_t* b) {
    int32_t s = 0;
    for (int j = 0; j < QK; ++j) s += (int32_t)a[j] * (int32_t)b[j];
    return s;
}

static void dot_one(const int8_t* wq, const uint16_t* wd, int64_t K, const int8_t* aq, const uint16_t* ad,
                    double* ref, double* norm) {
    int64_t nb = K / QK;
    double s = 0.0, a = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
        int32_t is = block_isum(wq + b * QK, aq + b * QK);
        double term = (double)q8o_f16_to_f32(wd[b]) * (double)q8o_f16_to_f32(ad[b]) * (double)is;
        s += term;
        a += fabs(term);
    }
    *ref = s;
    *norm = a;
}

void q8o_dot_pairs(const int8_t* wq, const uint16_t* wd, int64_t N, int64_t K, const int8_t* aq,
                   const uint16_t* ad, int64_t T, const int64_t* pt, const int64_t* pn, int64_t npairs,
                   double* ref, double* norm) {
    (void)N;
    (void)T;
    int64_t nb = K / QK;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < npairs; ++i) {
        int64_t t = pt[i], n = pn[i];
        dot_one(wq + n * K, wd + n * nb, K, aq + t * K, ad + t * nb, ref + i, norm + i);
    }
}

void q8o_gemm_full(const int8_t* wq, const uint16_t* wd, int64_t N, int64_t K, const int8_t* aq,
                   const uint16_t* ad, int64_t T, double* ref, double* norm) {
    int64_t nb = K / QK;
#pragma omp parallel for schedule(static) collapse(2)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t n = 0; n < N; ++n) {
            dot_one(wq + n * K, wd + n * nb, K, aq + t * K, ad + t * nb, ref + t * N + n, norm + t * N + n);
        }
    }
}

void q8o_block_isums(const int8_t* wq, int64_t N, int64_t K, const int8_t* aq, int64_t T, int32_t* isum) {
    int64_t nb = K / QK;
#pragma omp parallel for schedule(static) collapse(2)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t b = 0; b < nb; ++b) {
                isum[(t * N + n) * nb + b] = block_isum(wq + n * K + b * QK, aq + t * K + b * QK);
            }
        }
    }
}

/* ------------------------------------------------------------------------
 * q4_K weights ([P3] s2, on dequantizing at matrix time, and spec point
 * 1): a super-block of 256 values in 144 bytes -- f16 d at +0, f16 dmin at +2,
 * 12 bytes of packed 6-bit sub-block scales and mins at +4, 128 bytes of
 * 4-bit values at +16. Sub-block s (values 32s..32s+31, s = 0..7) takes value
 * j from byte 16 + 32*(s/2) + j: its low nibble for even s, its high nibble
 * for odd s ([P3] s3.2, the unpack of the staging branch). The value is
 *   w = d * sc_s * nib - dmin * m_s          (nib unsigned, 0..15)
 * ([P3] s3.2: the scale times the unsigned nibble, minus dmin times the min).
 * The pages name the 6-bit decode (get_scale_min_k4) without giving its bit
 * layout; the GGUF q4_K layout is taken. Its pins (a worked example, and that
 * the 96 bits map one to one onto the sixteen 6-bit fields) fix it only up to
 * a permutation of bits: which bit goes where is that format's, unpinned by
 * the pages. With b the 12 bytes,
 *   s < 4 : sc = b[s] & 63,                     m = b[s+4] & 63
 *   s >= 4: sc = (b[s+4] & 15) | (b[s-4] >> 6) << 4,
 *           m  = (b[s+4] >> 4) | (b[s]   >> 6) << 4.
 * ---------------------------------------------------------------------- */
#define QK_K 256
#define Q4K_BYTES 144

void q4ko_scale_min(const uint8_t* b, int s, int* sc, int* m) {
    if (s < 4) {
        *sc = b[s] & 63;
        *m = b[s + 4] & 63;
    } else {
        *sc = (b[s + 4] & 15) | ((b[s - 4] >> 6) << 4);
        *m = (b[s + 4] >> 4) | ((b[s] >> 6) << 4);
    }
}

static int q4k_nibble(const uint8_t* blk, int s, int j) {
    uint8_t byte = blk[16 + 32 * (s / 2) + j];
    return (s % 2 == 0) ? (byte & 15) : (byte >> 4);
}

/* Decoded fields of [N][K/256] super-blocks: nib [N][K], d and dmin [N][K/256]
 * (f16 bits), sc and mn [N][K/32]. */
void q4ko_decode(const uint8_t* blocks, int64_t N, int64_t K, uint8_t* nib, uint16_t* d, uint16_t* dmin,
                 uint8_t* sc, uint8_t* mn) {
    int64_t nsb = K / QK_K;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t sb = 0; sb < nsb; ++sb) {
            const uint8_t* blk = blocks + (n * nsb + sb) * Q4K_BYTES;
            memcpy(&d[n * nsb + sb], blk, 2);
            memcpy(&dmin[n * nsb + sb], blk + 2, 2);
            for (int s = 0; s < 8; ++s) {
                int a, b;
                q4ko_scale_min(blk + 4, s, &a, &b);
                sc[n * (K / QK) + sb * 8 + s] = (uint8_t)a;
                mn[n * (K / QK) + sb * 8 + s] = (uint8_t)b;
                for (int j = 0; j < QK; ++j) nib[n * K + sb * QK_K + s * QK + j] = (uint8_t)q4k_nibble(blk, s, j);
            }
        }
    }
}

/* Element values w [N][K] in f64 (each exact: 11 + 6 + 4 bits, and 11 + 6 bits). */
void q4ko_dequant_f64(const uint8_t* blocks, int64_t N, int64_t K, double* w) {
    int64_t nsb = K / QK_K;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t sb = 0; sb < nsb; ++sb) {
            const uint8_t* blk = blocks + (n * nsb + sb) * Q4K_BYTES;
            uint16_t dh, mh;
            memcpy(&dh, blk, 2);
            memcpy(&mh, blk + 2, 2);
            double dd = q8o_f16_to_f32(dh), dm = q8o_f16_to_f32(mh);
            for (int s = 0; s < 8; ++s) {
                int a, b;
                q4ko_scale_min(blk + 4, s, &a, &b);
                for (int j = 0; j < QK; ++j)
                    w[n * K + sb * QK_K + s * QK + j] = dd * a * q4k_nibble(blk, s, j) - dm * b;
            }
        }
    }
}

/* One output cell against a q8_0 activation row (values aq, f16 scales ad,
 * block sums assum). Per 32-value sub-block b ([P2] s2.1: ssum is kept for the
 * min-term correction):
 *   isum_b = sum_j nib[32b+j] * qa[32b+j]                      (exact int32)
 *   term_b = f16(da_b) * (f16(d) * sc_b * isum_b - f16(dmin) * m_b * ssum_b)
 * which equals sum_j w_j * da_b * qa_j exactly. Each product is exact in f64;
 * only the sum over b rounds. norm sums the absolute values of both parts. */
static void q4k_dot_one(const uint8_t* row, int64_t K, const int8_t* aq, const uint16_t* ad, const int16_t* assum,
                        double* ref, double* norm) {
    int64_t nsb = K / QK_K;
    double s = 0.0, a = 0.0;
    for (int64_t sb = 0; sb < nsb; ++sb) {
        const uint8_t* blk = row + sb * Q4K_BYTES;
        uint16_t dh, mh;
        memcpy(&dh, blk, 2);
        memcpy(&mh, blk + 2, 2);
        double dd = q8o_f16_to_f32(dh), dm = q8o_f16_to_f32(mh);
        for (int sub = 0; sub < 8; ++sub) {
            int64_t b = sb * 8 + sub;
            int sc, m;
            q4ko_scale_min(blk + 4, sub, &sc, &m);
            int32_t is = 0;
            for (int j = 0; j < QK; ++j) is += (int32_t)q4k_nibble(blk, sub, j) * (int32_t)aq[b * QK + j];
            double da = q8o_f16_to_f32(ad[b]);
            double t1 = da * dd * sc * (double)is;
            double t2 = da * dm * m * (double)assum[b];
            s += t1 - t2;
            a += fabs(t1) + fabs(t2);
        }
    }
    *ref = s;
    *norm = a;
}

void q4ko_dot_pairs(const uint8_t* blocks, int64_t N, int64_t K, const int8_t* aq, const uint16_t* ad,
                    const int16_t* assum, int64_t T, const int64_t* pt, const int64_t* pn, int64_t npairs,
                    double* ref, double* norm) {
    (void)N;
    (void)T;
    int64_t nb = K / QK, rowbytes = (K / QK_K) * Q4K_BYTES;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < npairs; ++i) {
        int64_t t = pt[i], n = pn[i];
        q4k_dot_one(blocks + n * rowbytes, K, aq + t * K, ad + t * nb, assum + t * nb, ref + i, norm + i);
    }
}

void q4ko_gemm_full(const uint8_t* blocks, int64_t N, int64_t K, const int8_t* aq, const uint16_t* ad,
                    const int16_t* assum, int64_t T, double* ref, double* norm) {
    int64_t nb = K / QK, rowbytes = (K / QK_K) * Q4K_BYTES;
#pragma omp parallel for schedule(static) collapse(2)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t n = 0; n < N; ++n) {
            q4k_dot_one(blocks + n * rowbytes, K, aq + t * K, ad + t * nb, assum + t * nb, ref + t * N + n,
                        norm + t * N + n);
        }
    }
}
