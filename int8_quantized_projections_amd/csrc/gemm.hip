// Prefill int8 GEMM on gfx950: q8_gemm.
//
// Sources: [P2] "r51 producer-fused A-quantize" s2.1 (the GEMM reads the
// pre-transposed, pre-swizzled activation plane by bulk copy, with no index
// arithmetic on the A side in the hot loop); [P3] "r5-r6 re-ranking +
// structural rewrite spec" s2-s3 (raw-byte staging, per-32-K rescale as the
// inner-loop cost).
//
// Design for gfx950:
//  - v_mfma_i32_32x32x32_i8: K = 32 is exactly one q8_0 block, so every MFMA
//    result is one block's exact int32 sum, ready for that block's two
//    scales. (The 16x16x64 form would add two blocks of different scales.)
//  - The MFMA accumulator input is a constant tile of 0x4B400000
//    (1.5 * 2^23 as f32), so the int32 result read as f32 is exactly
//    1.5 * 2^23 + isum (|isum| <= 32*127*127 < 2^22). Then
//      u   = fma(D, dw, -1.5*2^23*dw) = round(isum * dw)   (one rounding)
//      acc = fma(u, da, acc)
//    needs no int->float conversion.
//  - The per-row scale da of output register r lives in one VGPR per tile:
//    lane 16q+r holds da of the row that register r covers in row-group q,
//    and a DPP row_newbcast:r broadcast hands it to all 16 lanes.
//  - Workgroup tile: 64 tokens (one plane group) x 128 weight rows, 4 waves;
//    wave w owns weight rows 32w..32w+31 and both 32-token halves (two MFMA
//    tiles per K block). The A plane tile (8 chunks = 16 KB) is copied
//    verbatim into LDS; weight fragments are wave-private and are loaded
//    straight into VGPRs.
#include "q8_common.h"

#include <type_traits>

using namespace q8;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

namespace {

constexpr int kBN = 128;  // weight rows per workgroup
constexpr int kKT = 4;    // K blocks per LDS stage (double-buffered)
constexpr int kBias = 0x4B400000;
constexpr float kBiasF = 12582912.0f;  // 1.5 * 2^23

// acc[i] += u_i * (lane 16q + R_i's s), four at a time: v_fmac_f32_dpp with
// row_newbcast:R reads the scale from lane R of each 16-lane row, so the
// broadcast costs no extra instruction. The leading s_nop 1 covers the two
// wait states gfx9 requires between a VALU write of s and its DPP read.
#define Q8_FMAC_DPP4(a0, a1, a2, a3, sv, u0, u1, u2, u3, R0, R1, R2, R3)                  \
    asm("s_nop 1\n\t"                                                                     \
        "v_fmac_f32_dpp %0, %4, %5 row_newbcast:" #R0 " row_mask:0xf bank_mask:0xf\n\t"    \
        "v_fmac_f32_dpp %1, %4, %6 row_newbcast:" #R1 " row_mask:0xf bank_mask:0xf\n\t"    \
        "v_fmac_f32_dpp %2, %4, %7 row_newbcast:" #R2 " row_mask:0xf bank_mask:0xf\n\t"    \
        "v_fmac_f32_dpp %3, %4, %8 row_newbcast:" #R3 " row_mask:0xf bank_mask:0xf"         \
        : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3)                                            \
        : "v"(sv), "v"(u0), "v"(u1), "v"(u2), "v"(u3))

// One 32x32 tile's epilogue for one K block. d is the MFMA result reinterpreted
// as f32 as a whole vector (in this compiler, bit-casting a single
// ext_vector element yields element 0).
__device__ __forceinline__ void epilogue(float (&acc)[16], const v16f& d, float dw, float nbias, float s) {
    float u[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) u[r] = fmaf(d[r], dw, nbias);  // = round(isum * dw)
    Q8_FMAC_DPP4(acc[0], acc[1], acc[2], acc[3], s, u[0], u[1], u[2], u[3], 0, 1, 2, 3);
    Q8_FMAC_DPP4(acc[4], acc[5], acc[6], acc[7], s, u[4], u[5], u[6], u[7], 4, 5, 6, 7);
    Q8_FMAC_DPP4(acc[8], acc[9], acc[10], acc[11], s, u[8], u[9], u[10], u[11], 8, 9, 10, 11);
    Q8_FMAC_DPP4(acc[12], acc[13], acc[14], acc[15], s, u[12], u[13], u[14], u[15], 12, 13, 14, 15);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Global -> LDS direct copy of 16 (or 4) bytes per lane: lane i's bytes land at
// lds + 16*i (4*i). `lds` must be the same for the whole wave.
__device__ __forceinline__ void lds_copy16(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 16, 0, 0);
}
__device__ __forceinline__ void lds_copy4(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 4, 0, 0);
}

// Logical tile of physical workgroup p: workgroups are dealt to the 8 XCDs in
// turn, so give each XCD a contiguous range of logical tiles (neighbouring
// tiles share A or B strips in that XCD's L2).
__device__ __forceinline__ int64_t xcd_tile(int64_t p, int64_t tiles) {
    if (tiles % 8 != 0) return p;
    return (p % 8) * (tiles / 8) + p / 8;
}

__global__ __launch_bounds__(256) void k_gemm(const int8_t* __restrict__ aq, const uint32_t* __restrict__ asd,
                                              const int8_t* __restrict__ wq, const uint16_t* __restrict__ wd,
                                              float* __restrict__ C, int64_t T, int64_t N, int K, int nb, int64_t ldc,
                                              int n_tiles, int64_t tiles) {
    // Double-buffered stage of the A plane (kKT chunks of one 64-token group,
    // copied verbatim) and of its raw scale words.
    __shared__ __attribute__((aligned(16))) int8_t lds_a[2][kKT * kTileBytes];
    __shared__ __attribute__((aligned(16))) uint32_t lds_s[2][kKT * kGroup];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t tile = xcd_tile(blockIdx.x, tiles);
    const int nt = (int)(tile % n_tiles);
    const int64_t g = tile / n_tiles;
    const int64_t nrow = (int64_t)nt * kBN + wave * 32 + (lane & 31);
    const bool nvalid = nrow < N;
    const int khalf = lane >> 5;
    const int8_t* wrow = wq + (nvalid ? nrow : 0) * (int64_t)K + 16 * khalf;
    const uint16_t* drow = wd + (nvalid ? nrow : 0) * (int64_t)nb;

    // Output register r of lane l covers tile row 8(r/4) + 4(l/32) + r%4; the
    // lane that feeds register r's broadcast in row-group q is 16q + r.
    const int rr = lane & 15, qq = lane >> 4;
    const int srow = 8 * (rr >> 2) + 4 * (qq >> 1) + (rr & 3);
    // LDS byte offsets of this lane's A fragments (token 32h + lane%32, half khalf).
    int aoff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int i = 32 * h + (lane & 31);
        aoff[h] = i * 32 + (((khalf ^ (i >> 2) ^ (i >> 3)) & 1) * 16);
    }

    v16i bias;
#pragma unroll
    for (int i = 0; i < 16; ++i) bias[i] = kBias;
    float acc[2][16];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[h][i] = 0.0f;

    const int8_t* plane = aq + g * (int64_t)nb * kTileBytes;
    const uint32_t* splane = asd + g * (int64_t)nb * kGroup;
    const int nst = (nb + kKT - 1) / kKT;

    // Issue the copies of stage st into LDS buffer b. Each wave copies whole
    // 1 KB (A) or 256 B (scales) pieces, so the chunk a piece belongs to is
    // wave-uniform; chunks past K read a clamped (valid) address, never used.
    auto stage_a = [&](int st, int b) {
        const int c0 = st * kKT;
#pragma unroll
        for (int it = 0; it < kKT * kTileBytes / 16 / 256; ++it) {
            const int piece = it * 256 + wave * 64;  // first 16-byte piece of this wave
            const int c = min(c0 + piece / (kTileBytes / 16), nb - 1);
            const int8_t* src = plane + (int64_t)c * kTileBytes + (piece % (kTileBytes / 16)) * 16 + lane * 16;
            lds_copy16(src, &lds_a[b][piece * 16]);
        }
#pragma unroll
        for (int it = 0; it < kKT * kGroup / 256; ++it) {
            const int word = it * 256 + wave * 64;
            const int c = min(c0 + word / kGroup, nb - 1);
            lds_copy4(splane + (int64_t)c * kGroup + (word % kGroup) + lane, &lds_s[b][word]);
        }
    };
    auto stage_b = [&](int st, v4i (&bf)[kKT], uint32_t (&db)[kKT]) {
#pragma unroll
        for (int kb = 0; kb < kKT; ++kb) {
            const int c = min(st * kKT + kb, nb - 1);
            bf[kb] = *reinterpret_cast<const v4i*>(wrow + (int64_t)c * kQK);
            db[kb] = drow[c];
        }
    };

    // Compute stage st from LDS buffer `buf` and weight fragments bf/db.
    auto compute = [&](int st, int buf, const v4i (&bf)[kKT], const uint32_t (&db)[kKT]) {
        const int kc = min(kKT, nb - st * kKT);
        const int8_t* la = &lds_a[buf][0];
        const uint32_t* ls = &lds_s[buf][0];
        auto frags = [&](int kb, v4i (&af)[2], uint32_t (&sc)[2]) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                af[h] = *reinterpret_cast<const v4i*>(la + kb * kTileBytes + aoff[h]);
                sc[h] = ls[kb * kGroup + 32 * h + srow];
            }
        };
        // Pipeline over the 2*nk (block, half) tiles: the MFMA of the next tile is
        // issued before the epilogue of the current one, and the A fragments of
        // block kb+1 are read from LDS while block kb is being finished.
        auto run = [&](auto nk) {  // nk: std::integral_constant for full stages, int for the tail
            v4i af[2], an[2];
            uint32_t sc[2], sn[2];
            frags(0, af, sc);
            v16i d = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[0], bf[0], bias, 0, 0, 0);
#pragma unroll
            for (int kb = 0; kb < kKT; ++kb) {
                if (kb < nk) {
                    const float dw = nvalid ? f16_value(db[kb]) : 0.0f;
                    const float nbias = -kBiasF * dw;
                    if (kb + 1 < nk) frags(kb + 1, an, sn);
                    // tile (kb, 0) is in d; start (kb, 1)
                    const v16i d0 = d;
                    d = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[1], bf[kb], bias, 0, 0, 0);
                    epilogue(acc[0], __builtin_bit_cast(v16f, d0), dw, nbias, f16_value(sc[0]));
                    // tile (kb, 1) is in d; start (kb + 1, 0)
                    const v16i d1 = d;
                    if (kb + 1 < nk) d = __builtin_amdgcn_mfma_i32_32x32x32_i8(an[0], bf[kb + 1], bias, 0, 0, 0);
                    epilogue(acc[1], __builtin_bit_cast(v16f, d1), dw, nbias, f16_value(sc[1]));
                    af[0] = an[0];
                    af[1] = an[1];
                    sc[0] = sn[0];
                    sc[1] = sn[1];
                }
            }
        };
        if (kc == kKT)
            run(std::integral_constant<int, kKT>{});  // full stage: straight-line code, no joins
        else
            run(kc);
    };

    // Two register sets for the weight fragments, used alternately, so stage
    // st+1's fragments load while stage st computes without any copies.
    v4i b0[kKT], b1[kKT];
    uint32_t d0[kKT], d1[kKT];
    stage_a(0, 0);
    stage_b(0, b0, d0);
    __syncthreads();  // the compiler drains the copies (vmcnt) before the barrier
    for (int st = 0; st < nst; st += 2) {
        if (st + 1 < nst) {
            stage_a(st + 1, 1);
            stage_b(st + 1, b1, d1);
        }
        compute(st, 0, b0, d0);
        __syncthreads();
        if (st + 1 < nst) {
            if (st + 2 < nst) {
                stage_a(st + 2, 0);
                stage_b(st + 2, b0, d0);
            }
            compute(st + 1, 1, b1, d1);
            __syncthreads();
        }
    }

    if (nvalid) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t t = g * kGroup + 32 * h + 8 * (r >> 2) + 4 * khalf + (r & 3);
                if (t < T) C[t * ldc + nrow] = acc[h][r];
            }
        }
    }
}

}  // namespace

extern "C" int q8_gemm(const q8_weights* W, const int8_t* a_qs, const uint32_t* a_sd, int64_t t, float* c,
                       int64_t ldc, void* stream) {
    if (W == nullptr) return Q8_EINVAL;
    if (W->n < 0 || W->k <= 0 || (W->k % kQK) != 0 || W->k > ((int64_t)1 << 30) || t < 0) return Q8_ESHAPE;
    if (ldc < W->n) return Q8_ESHAPE;
    if (t == 0 || W->n == 0) return Q8_OK;
    if (W->qs == nullptr || W->d == nullptr || a_qs == nullptr || a_sd == nullptr || c == nullptr) return Q8_EINVAL;
    if (!q8h::aligned(W->qs, 16) || !q8h::aligned(W->d, 2) || !q8h::aligned(a_qs, 16) || !q8h::aligned(a_sd, 4) ||
        !q8h::aligned(c, 4))
        return Q8_EALIGN;
    const int nb = (int)(W->k / kQK);
    const int64_t ntb = q8h::ceil_div(t, kGroup);
    const int64_t n_tiles = q8h::ceil_div(W->n, kBN);
    const int64_t tiles = n_tiles * ntb;
    if (tiles > INT32_MAX) return Q8_ESHAPE;
    hipLaunchKernelGGL(k_gemm, dim3((unsigned)tiles), dim3(256), 0, (hipStream_t)stream, a_qs, a_sd, W->qs, W->d, c,
                       t, W->n, (int)W->k, nb, ldc, (int)n_tiles, tiles);
    return q8h::launch_status();
}
