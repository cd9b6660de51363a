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

using namespace q8;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

namespace {

constexpr int kBN = 128;  // weight rows per workgroup
constexpr int kKT = 8;    // K blocks per LDS stage
constexpr int kBias = 0x4B400000;
constexpr float kBiasF = 12582912.0f;  // 1.5 * 2^23

template <int R>
__device__ __forceinline__ float bcast_row(float s) {
    // row_newbcast always reads an existing lane of the same row, so the
    // bound_ctrl/old value never matters.
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x150 + R, 0xF, 0xF, true));
}

// d is the MFMA result reinterpreted as f32 as a whole vector: in this
// compiler, bit-casting a single ext_vector element yields element 0.
template <int R>
__device__ __forceinline__ void epilogue_r(float (&acc)[16], const v16f& d, float dw, float nbias, float s) {
    const float u = fmaf(d[R], dw, nbias);
    acc[R] = fmaf(u, bcast_row<R>(s), acc[R]);
}

__device__ __forceinline__ void epilogue(float (&acc)[16], const v16f& d, float dw, float nbias, float s) {
    epilogue_r<0>(acc, d, dw, nbias, s);
    epilogue_r<1>(acc, d, dw, nbias, s);
    epilogue_r<2>(acc, d, dw, nbias, s);
    epilogue_r<3>(acc, d, dw, nbias, s);
    epilogue_r<4>(acc, d, dw, nbias, s);
    epilogue_r<5>(acc, d, dw, nbias, s);
    epilogue_r<6>(acc, d, dw, nbias, s);
    epilogue_r<7>(acc, d, dw, nbias, s);
    epilogue_r<8>(acc, d, dw, nbias, s);
    epilogue_r<9>(acc, d, dw, nbias, s);
    epilogue_r<10>(acc, d, dw, nbias, s);
    epilogue_r<11>(acc, d, dw, nbias, s);
    epilogue_r<12>(acc, d, dw, nbias, s);
    epilogue_r<13>(acc, d, dw, nbias, s);
    epilogue_r<14>(acc, d, dw, nbias, s);
    epilogue_r<15>(acc, d, dw, nbias, s);
}

__global__ __launch_bounds__(256) void k_gemm(const int8_t* __restrict__ aq, const uint32_t* __restrict__ asd,
                                              const int8_t* __restrict__ wq, const uint16_t* __restrict__ wd,
                                              float* __restrict__ C, int64_t T, int64_t N, int K, int nb, int64_t ldc,
                                              int n_tiles) {
    __shared__ __attribute__((aligned(16))) int8_t lds_a[kKT * kTileBytes];
    __shared__ float lds_da[kKT * kGroup];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t tile = blockIdx.x;
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

    for (int c0 = 0; c0 < nb; c0 += kKT) {
        const int kc = min(kKT, nb - c0);
        __syncthreads();  // the previous stage's LDS reads are done
        // Stage the A tile (kc chunks of the plane, copied verbatim) and its scales. All
        // global loads are unconditional from clamped addresses so they issue together;
        // only the LDS stores are predicated.
        {
            const uint4* src = reinterpret_cast<const uint4*>(plane + (int64_t)c0 * kTileBytes);
            uint4* dst = reinterpret_cast<uint4*>(lds_a);
            const int na = kc * (kTileBytes / 16);
            uint4 av[kKT * kTileBytes / 16 / 256];
#pragma unroll
            for (int it = 0; it < kKT * kTileBytes / 16 / 256; ++it) {
                const int i = tid + 256 * it;
                av[it] = src[i < na ? i : na - 1];
            }
            const uint32_t* ssrc = splane + (int64_t)c0 * kGroup;
            const int ns = kc * kGroup;
            uint32_t sv[kKT * kGroup / 256];
#pragma unroll
            for (int it = 0; it < kKT * kGroup / 256; ++it) {
                const int i = tid + 256 * it;
                sv[it] = ssrc[i < ns ? i : ns - 1];
            }
#pragma unroll
            for (int it = 0; it < kKT * kTileBytes / 16 / 256; ++it) {
                const int i = tid + 256 * it;
                if (i < na) dst[i] = av[it];
            }
#pragma unroll
            for (int it = 0; it < kKT * kGroup / 256; ++it) {
                const int i = tid + 256 * it;
                if (i < ns) lds_da[i] = f16_value(sv[it]);
            }
        }
        v4i bf[kKT];
        float dwf[kKT];
#pragma unroll
        for (int kb = 0; kb < kKT; ++kb) {
            const int cb = c0 + kb < nb ? c0 + kb : nb - 1;
            bf[kb] = *reinterpret_cast<const v4i*>(wrow + (int64_t)cb * kQK);
            const uint16_t dbits = drow[cb];
            dwf[kb] = (kb < kc && nvalid) ? f16_value(dbits) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kb = 0; kb < kKT; ++kb) {
            if (kb < kc) {
                v4i af[2];
                float s[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int i = 32 * h + (lane & 31);
                    const int hh = (khalf ^ (i >> 2) ^ (i >> 3)) & 1;
                    af[h] = *reinterpret_cast<const v4i*>(lds_a + kb * kTileBytes + i * 32 + hh * 16);
                    s[h] = lds_da[kb * kGroup + 32 * h + srow];
                }
                const float nbias = -kBiasF * dwf[kb];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const v16i d = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[h], bf[kb], bias, 0, 0, 0);
                    epilogue(acc[h], __builtin_bit_cast(v16f, d), dwf[kb], nbias, s[h]);
                }
            }
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
                       t, W->n, (int)W->k, nb, ldc, (int)n_tiles);
    return q8h::launch_status();
}
