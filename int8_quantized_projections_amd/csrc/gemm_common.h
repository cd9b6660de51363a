// Shared pieces of the gfx950 int8 GEMM kernels (q8_gemm, q4k_gemm): the
// bias-reinterpret block-scale epilogue with DPP broadcast of the per-token
// scale, direct buffer -> LDS copies, and the XCD-aware tile order.
//
// Sources: [P2] "r51 producer-fused A-quantize" s2.1; [P3] "r5-r6 re-ranking +
// structural rewrite spec" s2-s3.
#pragma once

#include "q8_common.h"

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

namespace q8gemm {

using namespace q8;


constexpr int kBN = 128;  // weight rows per workgroup
constexpr int kKT = 4;    // K blocks per LDS stage (double-buffered)
constexpr int kBias = 0x4B400000;
constexpr float kBiasF = 12582912.0f;  // 1.5 * 2^23

// acc[i] += u_i * (lane 16q + R_i's s), four at a time: v_fmac_f32_dpp with
// row_newbcast:R reads the scale from lane R of each 16-lane row, so the
// broadcast costs no extra instruction. The leading s_nop 1 covers the two
// wait states gfx9 requires between a VALU write of s and its DPP read.
#define Q8_FMAC_DPP4(a0, a1, a2, a3, sv, u0, u1, u2, u3, R0, R1, R2, R3)                  \
    asm volatile("s_nop 1\n\t"                                                                     \
        "v_fmac_f32_dpp %0, %4, %5 row_newbcast:" #R0 " row_mask:0xf bank_mask:0xf\n\t"    \
        "v_fmac_f32_dpp %1, %4, %6 row_newbcast:" #R1 " row_mask:0xf bank_mask:0xf\n\t"    \
        "v_fmac_f32_dpp %2, %4, %7 row_newbcast:" #R2 " row_mask:0xf bank_mask:0xf\n\t"    \
        "v_fmac_f32_dpp %3, %4, %8 row_newbcast:" #R3 " row_mask:0xf bank_mask:0xf"         \
        : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3)                                            \
        : "v"(sv), "v"(u0), "v"(u1), "v"(u2), "v"(u3))

// The same without the leading s_nop, for the blocks after the first: s is
// not written between them. Both forms are volatile so that the compiler
// keeps their order: the block with the s_nop always runs first.
#define Q8_FMAC_DPP4_NONOP(a0, a1, a2, a3, sv, u0, u1, u2, u3, R0, R1, R2, R3)             \
    asm volatile("v_fmac_f32_dpp %0, %4, %5 row_newbcast:" #R0 " row_mask:0xf bank_mask:0xf\n\t"    \
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
    Q8_FMAC_DPP4_NONOP(acc[4], acc[5], acc[6], acc[7], s, u[4], u[5], u[6], u[7], 4, 5, 6, 7);
    Q8_FMAC_DPP4_NONOP(acc[8], acc[9], acc[10], acc[11], s, u[8], u[9], u[10], u[11], 8, 9, 10, 11);
    Q8_FMAC_DPP4_NONOP(acc[12], acc[13], acc[14], acc[15], s, u[12], u[13], u[14], u[15], 12, 13, 14, 15);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Buffer resource over `bytes` bytes from `base` (raw, stride 0; the third
// word's data format must be non-zero on gfx9). Reads past `bytes` return
// zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int nrec = (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, nrec, 0x00020000);
}

// Buffer -> LDS direct copy of 16 (or 4) bytes per lane from byte offset
// voff + soff of the resource: lane i's bytes land at lds + 16*i (4*i). `lds`
// and `soff` must be the same for the whole wave.
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void lds_copy4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 4, voff, soff, 0, 0);
}

// Wait until every global -> LDS copy this wave issued has landed
// (s_waitcnt vmcnt(0); the expcnt and lgkmcnt fields are left at their maxima).
__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Tile order: the n-tiles are cut into panels of kPanel; a panel's tiles are
// taken token group by token group. With each XCD given a contiguous range of
// this order, the ~96 tiles resident on one XCD span about 8 n-tiles x 12
// token groups, so the weight and activation strips they stream are shared in
// that XCD's L2 (in group-major order every XCD would stream the whole weight
// matrix, and a wide LM head would be read from HBM eight times).
constexpr int kPanel = 8;

__device__ __forceinline__ void tile_of(int64_t p, int64_t tiles, int n_tiles, int& nt, int64_t& g) {
    const int64_t L = xcd_contiguous(p, tiles);
    const int64_t ng = tiles / n_tiles;
    const int full = (n_tiles / kPanel) * kPanel;  // n-tiles in whole panels
    if (L < (int64_t)full * ng) {
        const int64_t r = L % ((int64_t)kPanel * ng);
        g = r / kPanel;
        nt = (int)(L / ((int64_t)kPanel * ng)) * kPanel + (int)(r % kPanel);
    } else {
        const int64_t r = L - (int64_t)full * ng;
        const int rem = n_tiles - full;
        g = r / rem;
        nt = full + (int)(r % rem);
    }
}

}  // namespace q8gemm
