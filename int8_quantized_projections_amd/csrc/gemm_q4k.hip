// Prefill GEMM with q4_K weights on gfx950: q4k_gemm.
//
// Sources: [P3] "r5-r6 re-ranking + structural rewrite spec" s2 (the
// dequant-at-mma-time principle: the weight side sits in shared memory as raw
// q4_K bytes and is unpacked in registers inside the matrix loop) and s3.1-3.2
// (the 144-byte super-block: f16 d, f16 dmin, 12 bytes of 6-bit scales and
// mins, 128 bytes of 4-bit values; value = d*sc*nib - dmin*m); [P2] "r51
// producer-fused A-quantize" s2.1 (the activation plane, whose ssum carries
// the min term).
//
// Per 32-value sub-block b of weight row n and token t:
//   sum_j w_j * da*qa_j = da * (d*sc_b * isum_b - dmin*m_b * ssum_b),
//   isum_b = sum_j nib_j * qa_j  (exact: v_mfma_i32_32x32x32_i8 on the
//   unpacked nibbles 0..15, which are valid signed int8 values).
// The first term is the q8_gemm epilogue with dw replaced by d*sc_b. The min
// term, sum_b c[t][b] * e[n][b] with c = da*ssum and e = -dmin*m, is itself a
// small f32 matrix product (inner dimension K/32): per stage and 32x32 tile it
// is two v_mfma_f32_32x32x2_f32 accumulating into the same registers as the
// epilogue (all 32x32 MFMAs share one output layout), instead of one DPP FMA
// per element and block on the vector ALU, which bounds this kernel.
//
// Staging: a stage is half a super-block (4 sub-blocks = 128 K) and reuses the
// q8_gemm A side unchanged. The weight side copies, per row, the 16-byte
// header and the half's 64 value bytes: 80 bytes, a row stride that keeps the
// 16-lane fragment reads conflict-free. The header's scales are decoded once
// per stage; nibble pairs (sub-blocks 2i, 2i+1 share their bytes) are read
// once and unpacked with one AND (or shift and AND) per dword.
#include "gemm_common.h"

#include <type_traits>

using namespace q8;

namespace {

using namespace q8gemm;

constexpr int kQ4Block = 144;  // bytes per 256-value super-block
constexpr int kQ4Row = 80;     // LDS bytes per weight row per stage: header 16 + values 64
constexpr int kQ4Pieces = 5;   // 16-byte pieces per row per stage
static_assert(kKT == 4, "a stage is half a super-block");

// acc += A * B over one 32x32 tile: A[t][k] the token factors of two
// sub-blocks, B[k][n] the row factors (lane l holds A[l%32][l/32] and
// B[l/32][l%32]).
__device__ __forceinline__ void min_mfma(float (&acc)[16], float a, float b) {
    v16f x;
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = acc[i];
    x = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, x, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = x[i];
}

// 16 nibbles of a sub-block (low nibbles for even, high for odd sub-blocks) as
// 16 int8 values 0..15.
template <int ODD>
__device__ __forceinline__ v4i unpack(const v4i& raw) {
    v4i r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (ODD ? ((uint32_t)raw[i] >> 4) : (uint32_t)raw[i]) & 0x0F0F0F0Fu;
    return r;
}

// Scale and min of sub-block 4*HALF + kb from the 12 scale bytes held as three
// words y (bytes 0-3), z (4-7), w (8-11), in the 6-bit layout of the oracle.
template <int HALF>
__device__ __forceinline__ void scale_min(uint32_t y, uint32_t z, uint32_t w, int kb, uint32_t& sc, uint32_t& m) {
    const int sh = 8 * kb;
    if constexpr (HALF == 0) {
        sc = (y >> sh) & 63u;
        m = (z >> sh) & 63u;
    } else {
        sc = ((w >> sh) & 15u) | (((y >> (sh + 6)) & 3u) << 4);
        m = ((w >> (sh + 4)) & 15u) | (((z >> (sh + 6)) & 3u) << 4);
    }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_gemm_q4k(
    const int8_t* __restrict__ aq, const uint32_t* __restrict__ asd, const uint8_t* __restrict__ wblk,
    float* __restrict__ C, int64_t T, int64_t N, int K, int nb, int64_t ldc, int n_tiles, int64_t tiles) {
    // one variable per buffer, so that reading one buffer need not wait for the
    // copies into the other (see k_gemm)
    __shared__ __attribute__((aligned(16))) int8_t lds_a0[kKT * kTileBytes], lds_a1[kKT * kTileBytes];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b0[kBN * kQ4Row], lds_b1[kBN * kQ4Row];
    __shared__ __attribute__((aligned(16))) uint32_t lds_s0[kKT * kGroup], lds_s1[kKT * kGroup];
    auto lds_a = [&](int b) { return b ? lds_a1 : lds_a0; };
    auto lds_b = [&](int b) { return b ? lds_b1 : lds_b0; };
    auto lds_s = [&](int b) { return b ? lds_s1 : lds_s0; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int nt;
    int64_t g;
    tile_of(blockIdx.x, tiles, n_tiles, nt, g);
    const int64_t n0 = (int64_t)nt * kBN;
    const int64_t rowbytes = (int64_t)(K / 256) * kQ4Block;
    const int brow = wave * 32 + (lane & 31);  // this lane's weight row in the tile
    const int64_t nrow = n0 + brow;            // and its output column
    const bool nvalid = nrow < N;
    const int khalf = lane >> 5;

    const int rr = lane & 15, qq = lane >> 4;
    const int srow = 8 * (rr >> 2) + 4 * (qq >> 1) + (rr & 3);
    int aoff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int i = 32 * h + (lane & 31);
        aoff[h] = i * 32 + (((khalf ^ (i >> 2) ^ (i >> 3)) & 1) * 16);
    }
    const int bbase = brow * kQ4Row;  // this lane's row record in a stage

    v16i bias;
#pragma unroll
    for (int i = 0; i < 16; ++i) bias[i] = kBias;
    asm volatile("" : "+v"(bias));
    float acc[2][16];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[h][i] = 0.0f;

    const int8_t* plane = aq + g * (int64_t)nb * kTileBytes;
    const uint32_t* splane = asd + g * (int64_t)nb * kGroup;
    const int nst = nb / kKT;  // K is a multiple of 256: whole stages, an even count

    // Copies (all full stages): the A plane and its scale words as in q8_gemm;
    // the weight records as 640 16-byte slots (row = slot / 5, piece = slot % 5),
    // ten copy instructions, wave w taking instructions w, w+4, w+8. A slot's
    // source is the row's super-block plus a per-lane offset fixed for each half.
    const __amdgpu_buffer_rsrc_t r_a = make_rsrc(plane, (int64_t)nb * kTileBytes);
    const __amdgpu_buffer_rsrc_t r_s = make_rsrc(splane, (int64_t)nb * kGroup * 4);
    const __amdgpu_buffer_rsrc_t r_b = make_rsrc(wblk + n0 * rowbytes, (N - n0) * rowbytes);
    const uint32_t aoffs = (uint32_t)(wave * 1024 + lane * 16);
    const uint32_t soffs = (uint32_t)(wave * kGroup + lane) * 4;
    constexpr int kCopies = kBN * kQ4Pieces / 64;  // 10
    uint32_t boff[2][3];                           // [half][k]: instruction wave + 4k
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int slot = 64 * (wave + 4 * k) + lane;
        const int row = slot / kQ4Pieces, p = slot % kQ4Pieces;
        const uint32_t rowoff = (uint32_t)((min(n0 + row, N - 1) - n0) * rowbytes);
        boff[0][k] = rowoff + (p == 0 ? 0u : (uint32_t)(16 + 16 * (p - 1)));
        boff[1][k] = rowoff + (p == 0 ? 0u : (uint32_t)(16 + 64 + 16 * (p - 1)));
    }
    auto stage_copy = [&](int st, int b, auto half) {
        const int c0 = st * kKT;
#pragma unroll
        for (int it = 0; it < kKT * kTileBytes / 16 / 256; ++it)
            lds_copy16(r_a, aoffs, (uint32_t)(c0 * kTileBytes + it * 4096), &lds_a(b)[it * 4096 + wave * 1024]);
        lds_copy4(r_s, soffs, (uint32_t)(c0 * kGroup * 4), &lds_s(b)[wave * kGroup]);
        const uint32_t sb_off = (uint32_t)((st >> 1) * kQ4Block);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int i = wave + 4 * k;
            if (i < kCopies) lds_copy16(r_b, boff[decltype(half)::value][k], sb_off, &lds_b(b)[i * 1024]);
        }
    };

    // Compute one stage: `half` (a compile-time 0 or 1) selects the sub-blocks
    // 4*half .. 4*half+3 of the super-block.
    auto compute = [&](int buf, auto half) {
        constexpr int H = decltype(half)::value;
        const int8_t* la = &lds_a(buf)[0];
        const uint8_t* lb = &lds_b(buf)[bbase];
        const uint32_t* ls = &lds_s(buf)[0];
        // this row's header: f16 d, f16 dmin, 12 scale bytes
        const uint4 hdr = *reinterpret_cast<const uint4*>(lb);
        const float dd = f16_value(hdr.x), dm = f16_value(hdr.x >> 16);
        float dsc[kKT], em[kKT];
#pragma unroll
        for (int kb = 0; kb < kKT; ++kb) {
            uint32_t sc, m;
            scale_min<H>(hdr.y, hdr.z, hdr.w, kb, sc, m);
            dsc[kb] = dd * (float)sc;   // exact: 11 + 6 bits
            em[kb] = -(dm * (float)m);  // exact
        }
        // min-term operands: e of sub-blocks khalf and 2+khalf of this lane's
        // row; c of token 32h + lane%32 in the same sub-blocks
        float eb[2], ca[2][2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            eb[j] = khalf ? em[2 * j + 1] : em[2 * j];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t w = ls[(2 * j + khalf) * kGroup + 32 * h + (lane & 31)];
                ca[h][j] = f16_value(w) * (float)(int16_t)(w >> 16);  // exact: 11 + 12 bits
            }
        }
        v4i raw[2];  // value bytes of sub-block pairs (0,1) and (2,3), this lane's half
#pragma unroll
        for (int p = 0; p < 2; ++p) raw[p] = *reinterpret_cast<const v4i*>(lb + 16 + 32 * p + 16 * khalf);
        auto bfrag = [&](int kb) { return (kb & 1) ? unpack<1>(raw[kb >> 1]) : unpack<0>(raw[kb >> 1]); };
        auto afrags = [&](int kb, v4i (&af)[2], uint32_t (&sw)[2]) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                af[h] = *reinterpret_cast<const v4i*>(la + kb * kTileBytes + aoff[h]);
                sw[h] = ls[kb * kGroup + 32 * h + srow];
            }
        };
        v4i af[2], an[2], bf = bfrag(0), bn;
        uint32_t sw[2], sn[2];
        afrags(0, af, sw);
        v16i d = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[0], bf, bias, 0, 0, 0);
#pragma unroll
        for (int kb = 0; kb < kKT; ++kb) {
            float dw = dsc[kb];
            asm volatile("" : "+v"(dw));  // keep the FMAs below plain v_fma_f32
            const float nbias = -kBiasF * dw;
            if (kb + 1 < kKT) {
                afrags(kb + 1, an, sn);
                bn = bfrag(kb + 1);
            }
            const float s0 = f16_value(sw[0]), s1 = f16_value(sw[1]);
            const v16i d0 = d;
            d = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[1], bf, bias, 0, 0, 0);
            epilogue(acc[0], __builtin_bit_cast(v16f, d0), dw, nbias, s0);
            if (kb + 1 == kKT) {
                min_mfma(acc[0], ca[0][0], eb[0]);
                min_mfma(acc[0], ca[0][1], eb[1]);
            }
            const v16i d1 = d;
            if (kb + 1 < kKT) d = __builtin_amdgcn_mfma_i32_32x32x32_i8(an[0], bn, bias, 0, 0, 0);
            epilogue(acc[1], __builtin_bit_cast(v16f, d1), dw, nbias, s1);
            if (kb + 1 == kKT) {
                min_mfma(acc[1], ca[1][0], eb[0]);
                min_mfma(acc[1], ca[1][1], eb[1]);
            }
            af[0] = an[0];
            af[1] = an[1];
            bf = bn;
            sw[0] = sn[0];
            sw[1] = sn[1];
        }
    };

    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    stage_copy(0, 0, H0{});
    wait_copies();
    __syncthreads();
    for (int st = 0; st < nst; st += 2) {  // st even: half 0 in buffer 0; st+1: half 1 in buffer 1
        stage_copy(st + 1, 1, H1{});
        compute(0, H0{});
        wait_copies();
        __syncthreads();
        if (st + 2 < nst) stage_copy(st + 2, 0, H0{});
        compute(1, H1{});
        wait_copies();
        __syncthreads();
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

int launch_q4k_gemm(int counter, const q4k_weights* W, const int8_t* a_qs, const uint32_t* a_sd, int64_t t,
                    float* c, int64_t ldc, hipStream_t stream) {
    if (W == nullptr) return Q8_EINVAL;
    // K a multiple of 256 (whole super-blocks); K <= 2^24 keeps the in-tile offsets in 32 bits
    if (W->n < 0 || W->k <= 0 || (W->k % 256) != 0 || W->k > ((int64_t)1 << 24) || t < 0) return Q8_ESHAPE;
    if (ldc < W->n) return Q8_ESHAPE;
    if (W->n > 0 && (W->blocks == nullptr || c == nullptr)) return Q8_EINVAL;
    if (a_qs == nullptr || a_sd == nullptr) return Q8_EINVAL;
    if (!q8h::aligned(W->blocks, 16) || !q8h::aligned(a_qs, 16) || !q8h::aligned(a_sd, 4) || !q8h::aligned(c, 4))
        return Q8_EALIGN;
    if (t == 0 || W->n == 0) return Q8_OK;
    const int nb = (int)(W->k / kQK);
    const int64_t n_tiles = q8h::ceil_div(W->n, kBN);
    const int64_t tiles = n_tiles * q8h::ceil_div(t, kGroup);
    if (tiles > INT32_MAX) return Q8_ESHAPE;
    q8h::launch_kernel(k_gemm_q4k, dim3((unsigned)tiles), dim3(256), 0, stream, a_qs, a_sd, W->blocks, c, t, W->n,
                       (int)W->k, nb, ldc, (int)n_tiles, tiles);
    return q8h::launch_status(counter);
}

extern "C" int q4k_gemm(const q4k_weights* W, const int8_t* a_qs, const uint32_t* a_sd, int64_t t, float* c,
                        int64_t ldc, void* stream) {
    return launch_q4k_gemm(Q8_LAUNCH_Q4K_GEMM, W, a_qs, a_sd, t, c, ldc, (hipStream_t)stream);
}
