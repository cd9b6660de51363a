/*
 * CPU oracle for the Q8_0 quantized projection path.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this code. The product path
 * (the HIP library and its Python binding) never does, and shares no code,
 * header, table or helper with it.
 *
 * Everything here is plain, slow and written to be read against the pages:
 *   [P1] "Part 4 - Lecture 05 - Fusion and the Activation-Quantization
 *        Discipline" (jared-hpc AI inference engineer roadmap)
 *   [P2] "54 - r51 - producer-fused A-quantize mode 1" (minfer CUDA
 *        optimization steps)
 *   [P3] "12 - r5-r6 re-ranking + structural rewrite spec" (minfer)
 * Floating-point references are computed in f64. The quantize itself is
 * defined in f32 (the pages fix d = amax/127 in f32 and rint of x/d), so it is
 * computed in f32 with IEEE basic operations only.
 */
#ifndef Q8_ORACLE_H
#define Q8_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* IEEE binary16 round-to-nearest-even conversion, including subnormals. */
uint16_t q8o_f32_to_f16(float f);
float q8o_f16_to_f32(uint16_t h);
void q8o_f32_to_f16_array(const float* x, int64_t n, uint16_t* out);

/* Activation quantize of [rows][K] f32 into q8_0 values. */
void q8o_quantize_rows(const float* x, int64_t rows, int64_t K, int8_t* qs, uint16_t* d16, int16_t* ssum);

/* ROW layout scale word: d16 | (uint16)ssum << 16. */
void q8o_pack_sd(const uint16_t* d16, const int16_t* ssum, int64_t n, uint32_t* sd);

/* PLANE64 layout (64-token groups, one 2048-byte tile per (group, chunk)). */
int64_t q8o_plane_qs_offset(int64_t t, int64_t k, int64_t K);
int64_t q8o_plane_sd_index(int64_t t, int64_t c, int64_t K);
void q8o_encode_plane64(const int8_t* qs, const uint16_t* d16, const int16_t* ssum, int64_t T, int64_t K,
                        int8_t* pqs, uint32_t* psd);
int64_t q8o_decode_plane64(const int8_t* pqs, const uint32_t* psd, int64_t T, int64_t K, int8_t* qs,
                           uint16_t* d16, int16_t* ssum);

/* Producers, f64 references. */
void q8o_rmsnorm_f64(const float* x, const float* w, int64_t rows, int64_t K, double eps, double* y);
void q8o_swiglu_f64(const float* g, const float* u, int64_t n, double* y);

/* Weights: quantize f32 [N][K] into GGUF Q8_0 blocks, and unpack blocks into planes. */
void q8o_quantize_weights_gguf(const float* w, int64_t N, int64_t K, uint8_t* blocks);
void q8o_gguf_to_planar(const uint8_t* blocks, int64_t N, int64_t K, int8_t* qs, uint16_t* d);

/* Block-scaled dot products. Activations are [T][K] values with d16 [T][K/32]. */
void q8o_dot_pairs(const int8_t* wq, const uint16_t* wd, int64_t N, int64_t K, const int8_t* aq,
                   const uint16_t* ad, int64_t T, const int64_t* pt, const int64_t* pn, int64_t npairs,
                   double* ref, double* norm);
void q8o_gemm_full(const int8_t* wq, const uint16_t* wd, int64_t N, int64_t K, const int8_t* aq,
                   const uint16_t* ad, int64_t T, double* ref, double* norm);
void q8o_block_isums(const int8_t* wq, int64_t N, int64_t K, const int8_t* aq, int64_t T, int32_t* isum);

/* q4_K weights (256-value super-blocks of 144 bytes) against q8_0 activations. */
void q4ko_scale_min(const uint8_t* b, int s, int* sc, int* m);
void q4ko_decode(const uint8_t* blocks, int64_t N, int64_t K, uint8_t* nib, uint16_t* d, uint16_t* dmin,
                 uint8_t* sc, uint8_t* mn);
void q4ko_dequant_f64(const uint8_t* blocks, int64_t N, int64_t K, double* w);
void q4ko_dot_pairs(const uint8_t* blocks, int64_t N, int64_t K, const int8_t* aq, const uint16_t* ad,
                    const int16_t* assum, int64_t T, const int64_t* pt, const int64_t* pn, int64_t npairs,
                    double* ref, double* norm);
void q4ko_gemm_full(const uint8_t* blocks, int64_t N, int64_t K, const int8_t* aq, const uint16_t* ad,
                    const int16_t* assum, int64_t T, double* ref, double* norm);

int q8o_num_threads(void);
void q8o_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
