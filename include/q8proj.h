/*
 * q8proj -- Q8_0 quantized projections for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libq8proj.so. Sources of the operations:
 *   [P1] "Part 4 - Lecture 05 - Fusion and the Activation-Quantization
 *        Discipline" (jared-hpc AI inference engineer roadmap)
 *   [P2] "54 - r51 - producer-fused A-quantize mode 1" (minfer)
 *   [P3] "12 - r5-r6 re-ranking + structural rewrite spec" (minfer)
 *
 * Conventions for every entry point below:
 *   - Pointers named in the argument lists are DEVICE pointers unless the
 *     comment says "host". The caller owns every buffer; the library never
 *     allocates, frees or caches device memory and keeps no state between
 *     calls ([P1] section 4: pass the buffer, do not cache it).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls enqueue their kernels on it and return without synchronising.
 *   - Arguments are validated on the host before anything is enqueued. On
 *     Q8_EINVAL, Q8_ESHAPE or Q8_EALIGN nothing was launched and no output byte
 *     was written. Q8_ELAUNCH means the HIP runtime refused a launch; the entry
 *     points that may make two launches back to back (q8_gemv_shared_multi_plus_f32
 *     and rmsnorm_quant_gemv_shared_multi_plus_f32 on shapes without their
 *     one-launch kernel) can have enqueued the first when the second is refused,
 *     and their outputs are then unspecified. Each launch's status is the one
 *     hipLaunchKernel returns for it: an error the caller's own earlier HIP work
 *     left pending (hipGetLastError) is never read, so it is not reported here.
 *   - Inputs are finite f32 values; the results for NaN or infinity inputs are
 *     unspecified (no fault). The producers' f32 outputs are within 1e-5
 *     relative of the exact value plus an absolute 2^-126 (rmsnorm_quant), or
 *     2^-126 * |up| + 2^-149 (swiglu_quant: silu(gate) is held to 2^-126 once it
 *     leaves f32's normal range, gate below about -87.3, and a product below
 *     that range rounds to f32's denormal step); the absolute parts matter only
 *     below f32's normal range. For rmsnorm_quant this holds for every finite
 *     x, including rows whose sum of squares overflows f32 (a rescaled second
 *     pass). Outputs must be representable (|y| below f32's maximum). A block
 *     whose d = amax/127 exceeds f16's maximum (amax above about 8.3e6) stores
 *     d = +infinity, the IEEE conversion's result.
 *   - Outputs must not alias inputs. Two consumers that must not overwrite
 *     each other's quantized activation use separate buffers ([P1] s4).
 *   - Calls with zero rows (rows == 0, T == 0, N == 0) are valid no-ops.
 *   - No C++ exception crosses this interface.
 *
 * Data formats
 *   q8_0 block: 32 elements, an f16 scale d and int8 values q, value = d*q
 *   ([P1] s2.1, [P2] s2.1).
 *
 *   Quantized activations (written by q8_quantize / rmsnorm_quant /
 *   swiglu_quant, read by q8_gemv and q8_gemm), for `rows` rows of width K:
 *     Q8_LAYOUT_ROW      qs [rows][K] int8, row-major;
 *                        sd [rows][K/32] uint32 = f16 bits of d | (uint16)ssum << 16,
 *                        where ssum is the int16 sum of the block's 32 q ([P2] s2.1).
 *     Q8_LAYOUT_PLANE64  tokens in groups of 64 ([P2] s2.1); with
 *                        ntb = ceil(rows/64), nchunk = K/32:
 *                        qs [ntb][nchunk][2048] int8: token r = t%64 of the group
 *                          owns bytes [32r, 32r+32) of the tile; its 16-byte half
 *                          h (elements 16h..16h+15 of the chunk) is stored at half
 *                          position h ^ (((r>>2) ^ (r>>3)) & 1);
 *                        sd [ntb][nchunk][64] uint32, same word as ROW, index r.
 *                        Tokens rows <= t < 64*ntb are written as zero bytes
 *                        ([P2] s3.1, the padded tail is part of the plane).
 *
 *   Weights (struct q8_weights, format Q8_WEIGHTS_Q8_0) are Q8_0 split into
 *     two planes: qs [N][K] int8 (row-major, 16-byte aligned) and d [N][K/32]
 *     f16 bits. q8_gemm also takes q4_K super-blocks (format Q8_WEIGHTS_Q4_K).
 *   q8_weights_repack converts GGUF Q8_0 blocks (34 bytes: f16 d at +0, int8
 *   qs[32] at +2, [P1] s2.1) into these planes once, at load time.
 */
#ifndef Q8PROJ_H
#define Q8PROJ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q8PROJ_ABI_VERSION 4

/* return codes */
#define Q8_OK 0
#define Q8_EINVAL (-1)  /* NULL required pointer, unknown layout, m out of range */
#define Q8_ESHAPE (-2)  /* negative size, K not a positive multiple of 32, K mismatch, ldc < N */
#define Q8_EALIGN (-3)  /* pointer not aligned as documented */
#define Q8_ELAUNCH (-4) /* the HIP runtime refused a launch (hipLaunchKernel's status for it) */
#define Q8_ENODEV (-5)  /* no usable gfx950 device for the calling thread */

/* activation layouts */
#define Q8_LAYOUT_ROW 0
#define Q8_LAYOUT_PLANE64 1

/* weight formats (q8_weights.format) */
#define Q8_WEIGHTS_Q8_0 0 /* Q8_0 split into the qs and d planes (every entry point) */
#define Q8_WEIGHTS_Q4_K 1 /* q4_K super-blocks (struct q4k_weights below) at qs, d unused: q8_gemm only */

typedef struct q8_weights {
    int64_t n;          /* output rows N */
    int64_t k;          /* reduction width K, a positive multiple of 32 (of 256 for Q8_WEIGHTS_Q4_K) */
    const int8_t* qs;   /* device, [N][K] int8, 16-byte aligned (Q4_K: the [N][K/256] x 144-byte blocks) */
    const uint16_t* d;  /* device, [N][K/32] f16 bits, 2-byte aligned (Q4_K: not read) */
    int64_t format;     /* Q8_WEIGHTS_Q8_0 (0, the value of a zero-initialised struct) or Q8_WEIGHTS_Q4_K;
                           entry points that do not take a format return Q8_EINVAL */
} q8_weights;

/* q4_K weights ([P3] s2-s3.2): row-major [N][K/256] super-blocks of 144 bytes
 * each -- f16 d at +0, f16 dmin at +2, 12 bytes of packed 6-bit sub-block
 * scales and mins at +4, 128 bytes of 4-bit values at +16. Value j of the
 * 32-value sub-block s is the low (s even) or high (s odd) nibble of byte
 * 16 + 32*(s/2) + j; w = d*sc_s*nib - dmin*m_s. The 6-bit fields: for s < 4,
 * sc = b[s] & 63 and m = b[s+4] & 63; for s >= 4, sc = (b[s+4] & 15) |
 * (b[s-4] >> 6) << 4 and m = (b[s+4] >> 4) | (b[s] >> 6) << 4, with b the
 * 12 scale bytes (the GGUF q4_K layout). */
typedef struct q4k_weights {
    int64_t n;              /* output rows N */
    int64_t k;              /* reduction width K, a positive multiple of 256 */
    const uint8_t* blocks;  /* device, [N][K/256] x 144 bytes, 16-byte aligned */
} q4k_weights;

/* ABI version (Q8PROJ_ABI_VERSION of the built library). */
int q8_abi_version(void);

/* Human-readable text of a return code (static storage). */
const char* q8_strerror(int code);

/*
 * Launch counters ([P1] s3: a tiny kernel's cost is set by how often it is
 * launched, not by its bytes; [P1] s5: count launches, and check the count
 * against the model's structure -- layers, consumers -- rather than trusting
 * a speedup). The library keeps one counter per entry point. Each counts the
 * kernel launches that entry point has enqueued since the library was loaded
 * or last reset: one per call that launched successfully. A call that returns
 * an error, or has nothing to do (zero rows), adds nothing. Launches recorded
 * into a HIP graph under stream capture count once, at capture; graph replays
 * do not pass through the library and are not counted. Counting is atomic,
 * process-wide and covers all devices.
 */
#define Q8_LAUNCH_QUANTIZE 0              /* q8_quantize */
#define Q8_LAUNCH_RMSNORM_QUANT 1         /* rmsnorm_quant */
#define Q8_LAUNCH_SWIGLU_QUANT 2          /* swiglu_quant */
#define Q8_LAUNCH_GEMV 3                  /* q8_gemv */
#define Q8_LAUNCH_GEMV_SHARED_MULTI 4     /* q8_gemv_shared_multi and q8_gemv_shared_multi_ex */
#define Q8_LAUNCH_GEMV_F32 5              /* q8_gemv_f32 */
#define Q8_LAUNCH_GEMM 6                  /* q8_gemm */
#define Q8_LAUNCH_GEMM_SHARED_MULTI 7     /* q8_gemm_shared_multi */
#define Q8_LAUNCH_Q4K_GEMM 8              /* q4k_gemm */
#define Q8_LAUNCH_WEIGHTS_REPACK 9        /* q8_weights_repack */
#define Q8_LAUNCH_GEMV_SHARED_MULTI_PLUS_F32 10  /* q8_gemv_shared_multi_plus_f32 (1 launch, or 2: see there) */
#define Q8_LAUNCH_RMSNORM_GEMV_STEP 11   /* rmsnorm_quant_gemv_shared_multi_plus_f32, one-launch form */
#define Q8_LAUNCH_COUNTERS 12

/* Copies the first min(n, Q8_LAUNCH_COUNTERS) counters, in the order of the
 * Q8_LAUNCH_* ids, into the host array counts. Returns Q8_LAUNCH_COUNTERS,
 * or Q8_EINVAL (nothing copied) when n < 0 or counts is NULL with n > 0. */
int q8_launch_counts(int64_t* counts, int n);

/* Sets every launch counter to zero. */
void q8_launch_counts_reset(void);

/* Name of the entry point counter `id` counts (static storage), or NULL when
 * id is not a Q8_LAUNCH_* id. */
const char* q8_launch_counter_name(int id);

/*
 * Bytes of the activation buffers for `rows` rows of width K in `layout`
 * (host only, no device call). Writes *qs_bytes and *sd_bytes.
 * Returns Q8_OK, Q8_EINVAL or Q8_ESHAPE.
 */
int q8_act_bytes(int64_t rows, int64_t k, int layout, size_t* qs_bytes, size_t* sd_bytes);

/*
 * Bytes of a PLANE64 activation of T tokens of width K ([P2] s2.1-s2.2: the
 * 64-token plane, ceil(T/64) groups of K/32 tiles of 2048 qs bytes and 64
 * scale words): q8_act_bytes(T, K, Q8_LAYOUT_PLANE64, ...). Host only.
 * Returns Q8_OK, Q8_EINVAL (NULL output) or Q8_ESHAPE.
 */
int q8_plane_bytes(int64_t t, int64_t k, size_t* qs_bytes, size_t* sd_bytes);

/*
 * Activation quantize ([P1] s3-s3.1: quantize once per activation and pass
 * the buffer to every consumer; [P2] s3.2 quantize body).
 * x: [rows][K] f32, 16-byte aligned. Per 32-element block:
 *   amax = max|x|, d = amax/127 (f32, IEEE divide), q = rint(x/d) (IEEE
 *   divide, ties to even) clamped to [-127, 127] (q = 0 when d == 0),
 *   stored d = f16(d) (round to nearest even), ssum = sum(q).
 * qs, sd: output buffers of q8_act_bytes(rows, K, layout); qs 16-byte and
 * sd 4-byte aligned.
 */
int q8_quantize(const float* x, int64_t rows, int64_t k, int layout, int8_t* qs, uint32_t* sd, void* stream);

/*
 * Fused RMSNorm + quantize ([P2] s2.3, s3.1, s3.2: the producer writes the
 * quantized activation in the same pass as its f32 output).
 * y[t][j] = x[t][j] * (1/sqrt(mean_j x[t][j]^2 + eps)) * w[j], f32.
 * The quantized output is q8_quantize applied to the y this call writes,
 * bit for bit. qs == NULL and sd == NULL: f32 output only (then `layout` is
 * ignored); either both or neither may be NULL. y == NULL (with qs and sd
 * given): the quantized output only, bit-identical to the one a call with y
 * writes, for consumers that read no f32 activation ([P2] s3.1, mode 2).
 * y and qs both NULL: Q8_EINVAL.
 * x, y: [rows][K] f32 (16-byte aligned), w: [K] f32 (16-byte aligned).
 */
int rmsnorm_quant(const float* x, const float* w, float eps, float* y, int64_t rows, int64_t k, int layout,
                  int8_t* qs, uint32_t* sd, void* stream);

/*
 * Fused SwiGLU + quantize ([P2] s3.2): y = gate / (1 + e^-gate) * up, f32,
 * and the quantized y as in rmsnorm_quant (NULL qs and sd: f32 only; NULL y:
 * the quantized output only, [P2] s3.1 mode 2).
 * gate, up, y: [rows][K] f32, 16-byte aligned.
 */
int swiglu_quant(const float* gate, const float* up, float* y, int64_t rows, int64_t k, int layout, int8_t* qs,
                 uint32_t* sd, void* stream);

/*
 * Batch-1 Q8_0 GEMV ([P1] s2.1-s2.4): y[n] = sum_b f16(dw[n,b]) * f16(da[b]) * isum[n,b],
 * isum[n,b] = sum_{j<32} qw[n,32b+j] * qa[32b+j] (exact int32).
 * W: host pointer to the weight descriptor. a_qs, a_sd: one ROW-layout
 * activation row of width W->k. y: [N] f32.
 * The number of lanes per row follows K/32. The rows per wave are 1 while the
 * activation fits a wave's registers (K <= 8192); for wider K they follow N
 * (a dispatch threshold: 2 from 2048 row slots, 4 from 16384). Every variant
 * gives bit-identical y.
 */
int q8_gemv(const q8_weights* W, const int8_t* a_qs, const uint32_t* a_sd, float* y, void* stream);

/*
 * Batch-1 Q8_0 GEMV on an f32 activation, quantized inside the same launch
 * ([P1] s3-s3.1: at decode a quantize launch costs far more than its bytes,
 * so launches should be removed; for an activation with a single consumer the
 * quantize moves into that consumer). x: [K] f32, 16-byte aligned, with
 * K = W->k <= 8192 (Q8_ESHAPE otherwise; wider activations are quantized once
 * with q8_quantize). Each workgroup quantizes x once into its shared memory
 * with the q8_quantize arithmetic, so y is bit-identical to q8_quantize(x)
 * followed by q8_gemv(W, ...). y: [N] f32.
 */
int q8_gemv_f32(const q8_weights* W, const float* x, float* y, void* stream);

/*
 * Several GEMVs that read the same activation, in one launch ([P1] s2.5,
 * s6: one activation feeding q/k/v/g, and the "more general grouped kernel"
 * for consumers of one activation at different N).
 * m: 1..8. W: host array of m host pointers, all with the same k. y: host
 * array of m device pointers, y[i] of length W[i]->n. Each y[i] is
 * bit-identical to q8_gemv(W[i], ...).
 */
int q8_gemv_shared_multi(int m, const q8_weights* const* W, const int8_t* a_qs, const uint32_t* a_sd,
                         float* const* y, void* stream);

/*
 * Same as q8_gemv_shared_multi with the rows-per-wave factor forced
 * (rows_per_wave in {0 = automatic, 1, 2, 4}); for tests and measurements.
 */
int q8_gemv_shared_multi_ex(int m, const q8_weights* const* W, const int8_t* a_qs, const uint32_t* a_sd,
                            float* const* y, int rows_per_wave, void* stream);

/*
 * q8_gemv_shared_multi(m, W, a_qs, a_sd, y) and q8_gemv_f32(Wx, x, yx) in one
 * launch ([P1] s6: the decode projections of a layer read a few activations at
 * different N; [P1] s3: at decode every launch costs microseconds while its
 * bytes cost less). The two GEMVs are independent: the grouped one reads the
 * ROW-layout q8_0 activation (a_qs, a_sd) and writes y[i]; the other reads the
 * f32 activation x of width Wx->k <= 8192, quantized inside the launch, and
 * writes yx. Arguments, layouts and errors are those of the two calls, and both
 * are validated before anything is launched. The outputs are bit-identical to
 * the two separate calls. One launch serves the grouped part at K in
 * (2048, 8192] together with the f32 part at Wx->k in (64, 512] (the rows per
 * wave that q8_gemv_plan picks for each part must be at most 2, and 1 for the
 * f32 part). Other shapes, or an empty part, make the two launches back to back.
 */
int q8_gemv_shared_multi_plus_f32(int m, const q8_weights* const* W, const int8_t* a_qs, const uint32_t* a_sd,
                                  float* const* y, const q8_weights* Wx, const float* x, float* yx, void* stream);

/*
 * The decode step of one layer's projections in one launch: rmsnorm_quant of
 * the single row x (width K = W[i]->k, ROW layout) and
 * q8_gemv_shared_multi_plus_f32 of its consumers ([P2] s2-s3: the producer
 * writes the q8_0 activation in the same pass as its f32 output, and the
 * consumers read it; [P1] s3: at decode a launch costs more than its bytes).
 * Inside the launch every workgroup of the grouped GEMV normalizes and
 * quantizes the row into its own LDS and reads its activation from there, so
 * no workgroup waits for another; x and w are read from HBM once per XCD.
 *   x, w: device f32, K values each, 16-byte aligned. eps: as rmsnorm_quant.
 *   y: device f32 [K] for the normalized row, or NULL for none. y may be x
 *     (in place); if y, a_qs or a_sd overlaps x or w, the call runs as the
 *     two calls below instead of one launch. The GEMV outputs must not
 *     overlap any input, as for the GEMV calls.
 *   a_qs, a_sd: device buffers (K bytes, K/32 words; 16- and 4-byte aligned)
 *     that receive the row's q8_0 activation, as rmsnorm_quant writes it.
 *   m, W, ys, Wx, x2, yx: as q8_gemv_shared_multi_plus_f32 (m, W, y, Wx, x, yx).
 *     Wx may be NULL: no f32-activation GEMV (x2 and yx are not read), as for
 *     an LM head after the output norm.
 * Every output is bit-identical to rmsnorm_quant followed by
 * q8_gemv_shared_multi_plus_f32 (q8_gemv_shared_multi when Wx is NULL). The
 * one launch serves the pair launch's shapes (see there; the grouped part at
 * K in (2048, 8192], one row per wave), with the f32 part empty or absent or
 * at K in (64, 512]; other shapes run those calls back to back (and count
 * under their names). Errors: those of the calls, all checked before anything
 * is launched; Q8_EINVAL for a NULL x or w.
 */
int rmsnorm_quant_gemv_shared_multi_plus_f32(const float* x, const float* w, float eps, float* y, int8_t* a_qs,
                                             uint32_t* a_sd, int m, const q8_weights* const* W, float* const* ys,
                                             const q8_weights* Wx, const float* x2, float* yx, void* stream);

/*
 * The GEMV launch plan for `total_rows` rows of width K (host only):
 * lanes per row, rows per wave and the grid size in workgroups.
 */
int q8_gemv_plan(int64_t total_rows, int64_t k, int rows_per_wave, int* lanes_per_row, int* rows_per_wave_out,
                 int64_t* workgroups);

/*
 * Prefill int8 GEMM ([P2] s2.1: the GEMM reads the pre-transposed quantized
 * plane in bulk; [P3] s2-s3): C[t][n] = sum_b f16(da[t,b]) * f16(dw[n,b]) * isum[t,n,b].
 * a_qs, a_sd: a PLANE64 activation of T tokens and width W->k.
 * C: [T][ldc] f32, row-major, ldc >= N; only columns n < N of rows t < T are
 * written. K <= 2^24 (Q8_ESHAPE otherwise).
 * W->format Q8_WEIGHTS_Q4_K takes the q4_K weights at W->qs (as q4k_gemm
 * below, the same bits); the launch counts under q8_gemm.
 */
int q8_gemm(const q8_weights* W, const int8_t* a_qs, const uint32_t* a_sd, int64_t t, float* c, int64_t ldc,
            void* stream);

/*
 * Several prefill GEMMs that read the same PLANE64 activation, in one launch:
 * the prefill counterpart of q8_gemv_shared_multi ([P1] s2.5, s6: consumers of
 * one activation in one grouped kernel; [P2] s1: q/k/v read one plane).
 * m: 1..8. W: host array of m host pointers, all with the same k. c: host
 * array of m device pointers; ldc: host array of m values; c[i] is
 * [T][ldc[i]] f32 with ldc[i] >= W[i]->n. Members with n == 0 are skipped.
 * Each c[i] is bit-identical to q8_gemm(W[i], a_qs, a_sd, t, c[i], ldc[i]).
 * Returns Q8_EINVAL (m out of range, NULL), Q8_ESHAPE (k differs, ldc < n,
 * K > 2^24, t < 0) or Q8_EALIGN before any launch.
 */
int q8_gemm_shared_multi(int m, const q8_weights* const* W, const int8_t* a_qs, const uint32_t* a_sd, int64_t t,
                         float* const* c, const int64_t* ldc, void* stream);

/*
 * Prefill GEMM with q4_K weights over a PLANE64 q8_0 activation ([P3] s2:
 * the weight side is staged as raw bytes and unpacked at matrix-op time):
 *   C[t][n] = sum over 32-value sub-blocks b of
 *             f16(da[t,b]) * (f16(d)*sc_b * isum[t,n,b] - f16(dmin)*m_b * ssum[t,b]),
 *   isum = sum_j nib[n, 32b+j] * qa[t, 32b+j], ssum = the activation block's
 *   stored sum of its q values ([P2] s2.1: kept for the min-term correction).
 * a_qs, a_sd: a PLANE64 activation of T tokens and width W->k. C: [T][ldc]
 * f32, ldc >= N; only columns n < N of rows t < T are written.
 * K a multiple of 256 and <= 2^24 (Q8_ESHAPE otherwise).
 */
int q4k_gemm(const q4k_weights* W, const int8_t* a_qs, const uint32_t* a_sd, int64_t t, float* c, int64_t ldc,
             void* stream);

/*
 * Load-time conversion of GGUF Q8_0 blocks (device, [N][K/32] x 34 bytes,
 * 2-byte aligned; [P1] s2.1) into the weight planes qs [N][K] and d [N][K/32]
 * (device). Pure byte movement.
 */
int q8_weights_repack(const void* gguf_blocks, int64_t n, int64_t k, int8_t* qs, uint16_t* d, void* stream);

/*
 * Measurement helper, not part of the projection path: the practical HBM read
 * rate of this GPU, the ceiling the path's bandwidth figures are read against
 * ([P1] s3: achieved bytes over time, against what the memory delivers). One
 * launch streams `bytes` (a multiple of 16) of the device buffer buf (16-byte
 * aligned) once, over `workgroups` workgroups of 256 lanes (1..65536), each
 * lane reading 16-byte words grid-stride with loads_per_lane (1, 2 or 4) loads
 * issued together; workgroup i writes an XOR of what it read to out[i]
 * (device, `workgroups` words). Not counted by the launch counters.
 */
int q8_hbm_read_probe(const void* buf, int64_t bytes, int workgroups, int loads_per_lane, uint32_t* out,
                      void* stream);

/*
 * Measurement helper, not part of the projection path: a plain stream of a
 * given read/write mix, the practical ceiling of a producer with that mix. One
 * launch reads `bytes` (a multiple of 16) from src0 and, when not NULL, from
 * src1, and writes `bytes` to dst when dst is not NULL (the XOR of the sources,
 * or a counter pattern with no source), over `workgroups` workgroups of 256
 * lanes (1..65536), 16-byte grid-stride words. With dst NULL, workgroup i
 * writes an XOR of what it read to out[i] (`workgroups` words; out is not used
 * otherwise). Device buffers, 16-byte aligned (out 4-byte). src1 without
 * src0, no source and no destination, or neither dst nor out: Q8_EINVAL; bytes
 * not a multiple of 16 or workgroups outside 1..65536: Q8_ESHAPE. Not counted
 * by the launch counters.
 */
int q8_hbm_stream_probe(const void* src0, const void* src1, void* dst, int64_t bytes, int workgroups, uint32_t* out,
                        void* stream);

#ifdef __cplusplus
}
#endif
#endif
