// Shared device helpers of the gfx950 Q8_0 projection kernels.
//
// Wave64 throughout. A q8_0 block of 32 f32 values is held by 8 consecutive
// lanes, 4 values (one float4) per lane, so that every load and store of a
// row is a fully coalesced 16-byte-per-lane access and the per-block
// reductions (amax, ssum) are three DPP steps inside an 8-lane group.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <tuple>

#include "q8proj.h"

namespace q8 {

constexpr int kQK = 32;          // elements per q8_0 block
constexpr int kWave = 64;        // gfx950 wavefront size
constexpr int kGroup = 64;       // tokens per PLANE64 group
constexpr int kTileBytes = 2048; // qs bytes per (group, chunk) tile

// DPP controls (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm:[1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm:[2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i inside each 8 lanes
constexpr int kDppRowMirror = 0x140;     // lane i <- lane 15-i inside each 16 lanes

// Lane permutations inside rows of 16 lanes. Every lane of these patterns reads
// a lane of its own row, so no source is out of range; bound_ctrl then lets the
// compiler fold the move into the instruction that consumes it
// (v_add_f32_dpp, v_max_u32_dpp, ...), one instruction per step.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

// All-reduce over each aligned group of 8 lanes. After the two quad steps
// every lane holds its quad's result; the half-mirror step pairs lane i with
// lane 7-i, i.e. each quad with the other quad of its 8-lane group.
// umax8 takes the bit patterns of non-negative floats, whose unsigned order is
// their numeric order (the integer max needs no NaN canonicalization).
__device__ __forceinline__ uint32_t umax8(uint32_t a) {
    a = max(a, (uint32_t)dpp_i<kDppQuadXor1>((int)a));
    a = max(a, (uint32_t)dpp_i<kDppQuadXor2>((int)a));
    a = max(a, (uint32_t)dpp_i<kDppRowHalfMirror>((int)a));
    return a;
}

__device__ __forceinline__ int sum8(int s) {
    s += dpp_i<kDppQuadXor1>(s);
    s += dpp_i<kDppQuadXor2>(s);
    s += dpp_i<kDppRowHalfMirror>(s);
    return s;
}

__device__ __forceinline__ uint32_t fbits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __builtin_bit_cast(float, u); }

// amax / 127 correctly rounded (the IEEE quotient) in three instructions:
// q = amax * RN(1/127), then one fma correction of the remainder. Checked
// against the IEEE division for every non-negative f32, subnormals included
// (tests/test_quantize_arithmetic.py).
__device__ __forceinline__ float div127(float a) {
    constexpr float c = 1.0f / 127.0f;
    const float q = a * c;
    return fmaf(fmaf(-q, 127.0f, a), c, q);
}

// Half-integer margin of the reciprocal path: with |x/d| <= 128 and v_rcp_f32
// within one ulp, |x/d - x*r| <= 2^-16, so a residual |x*r - rint(x*r)| below
// 0.5 - 2^-14 puts x/d (and its f32 rounding) strictly inside the same integer's
// rounding interval.
constexpr float kHalfMargin = 0.5f - 0x1p-14f;

// True when d is a nonzero f32-subnormal: the reciprocal bound above needs a normal d.
__device__ __forceinline__ bool subnormal_nonzero(float d) { return fbits(d) - 1u < 0x007FFFFFu; }

// v plus the value of lane i ^ 16 (add_xor16) or i ^ 32 (add_xor32), with
// gfx950's v_permlane16_swap / v_permlane32_swap: the swap of 16-lane rows
// 0<->1 and 2<->3 (of the two 32-lane halves) in VALU registers, where a lane
// shuffle is an LDS round trip. The two operands come out as (lower row's,
// upper row's) in both rows, so the sum has the bits of v + shfl_xor(v, 16)
// (resp. 32) in every lane (f32 addition is commutative).
__device__ __forceinline__ float add_xor16(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ float add_xor32(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Sum over all 64 lanes with a fixed tree; every lane receives the same bits.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<kDppQuadXor1>(v);
    v += dpp_f<kDppQuadXor2>(v);
    v += dpp_f<kDppRowHalfMirror>(v);
    v += dpp_f<kDppRowMirror>(v);
    v = add_xor16(v);
    return add_xor32(v);
}

__device__ __forceinline__ uint32_t f16_bits(float d) {
    _Float16 h = (_Float16)d;  // v_cvt_f16_f32, round to nearest even, f16 denormals kept
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_value(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xFFFFu));
}

__device__ __forceinline__ int clamp127(float n) { return min(127, max(-127, (int)n)); }

struct Quant8 {
    uint32_t qs4;  // this lane's 4 int8 values, little-endian
    uint32_t sd;   // f16 bits of d | (uint16)ssum << 16, identical in all 8 lanes
};

__device__ __forceinline__ uint32_t pack4(int q0, int q1, int q2, int q3) {
    return (uint32_t)(q0 & 0xFF) | ((uint32_t)(q1 & 0xFF) << 8) | ((uint32_t)(q2 & 0xFF) << 16) |
           ((uint32_t)(q3 & 0xFF) << 24);
}

// The one quantize body of the library ([P2] section 3.2, phase 2): every
// producer (q8_quantize, rmsnorm_quant, swiglu_quant) calls it on the f32
// values it has just produced, so their quantized outputs are bit-identical
// by construction. The 8 lanes of an aligned group hold one 32-value block.
//
// q = rint(x / d) with x/d the correctly rounded f32 quotient, computed
// exactly but cheaply: n = rint(x * r) with r = rcp(d) is that integer unless
// the residual x*r - n comes within 2^-14 of a half (kHalfMargin); those
// lanes, and blocks with a subnormal d, redo their four values with the IEEE
// division. |x/d| <= 127 (+1 ulp) for a normal d, so the clamp only acts there.
__device__ __forceinline__ Quant8 quantize_block8(float4 v) {
    const uint32_t am = max(max(fbits(fabsf(v.x)), fbits(fabsf(v.y))), max(fbits(fabsf(v.z)), fbits(fabsf(v.w))));
    const float a = bitsf(umax8(am));  // exact in any order
    const float d = div127(a);
    const float r = d != 0.0f ? __builtin_amdgcn_rcpf(d) : 0.0f;  // d == 0: all q are 0
    float n0 = __builtin_rintf(v.x * r), n1 = __builtin_rintf(v.y * r), n2 = __builtin_rintf(v.z * r),
          n3 = __builtin_rintf(v.w * r);
    const float e = fmaxf(fmaxf(fabsf(fmaf(v.x, r, -n0)), fabsf(fmaf(v.y, r, -n1))),
                          fmaxf(fabsf(fmaf(v.z, r, -n2)), fabsf(fmaf(v.w, r, -n3))));
    if (e >= kHalfMargin || subnormal_nonzero(d)) {
        n0 = __builtin_rintf(v.x / d);
        n1 = __builtin_rintf(v.y / d);
        n2 = __builtin_rintf(v.z / d);
        n3 = __builtin_rintf(v.w / d);
    }
    const int q0 = clamp127(n0), q1 = clamp127(n1), q2 = clamp127(n2), q3 = clamp127(n3);
    const int s = sum8(q0 + q1 + q2 + q3);
    Quant8 res;
    res.qs4 = pack4(q0, q1, q2, q3);
    res.sd = f16_bits(d) | ((uint32_t)(uint16_t)(int16_t)s << 16);
    return res;
}

// quantize_block8's arithmetic for a whole 32-value block held by one lane
// (a consumer quantizing its own activation): the same bits. The IEEE division
// is redone for all 32 values when any of them is near a half-integer; for the
// others it gives the same integer as the reciprocal path. ssum is not formed.
__device__ __forceinline__ void quantize_lane32(const float4 (&v)[8], uint4& q0, uint4& q1, uint32_t& dbits) {
    uint32_t am = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        am = max(am, max(max(fbits(fabsf(v[i].x)), fbits(fabsf(v[i].y))),
                         max(fbits(fabsf(v[i].z)), fbits(fabsf(v[i].w)))));
    const float d = div127(bitsf(am));
    const float r = d != 0.0f ? __builtin_amdgcn_rcpf(d) : 0.0f;
    float n[32];
    float e = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float x4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            n[4 * i + c] = __builtin_rintf(x4[c] * r);
            e = fmaxf(e, fabsf(fmaf(x4[c], r, -n[4 * i + c])));
        }
    }
    if (e >= kHalfMargin || subnormal_nonzero(d)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            n[4 * i + 0] = __builtin_rintf(v[i].x / d);
            n[4 * i + 1] = __builtin_rintf(v[i].y / d);
            n[4 * i + 2] = __builtin_rintf(v[i].z / d);
            n[4 * i + 3] = __builtin_rintf(v[i].w / d);
        }
    }
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        w[i] = pack4(clamp127(n[4 * i]), clamp127(n[4 * i + 1]), clamp127(n[4 * i + 2]), clamp127(n[4 * i + 3]));
    q0 = make_uint4(w[0], w[1], w[2], w[3]);
    q1 = make_uint4(w[4], w[5], w[6], w[7]);
    dbits = f16_bits(d);
}

// Workgroup barrier for data exchanged through LDS by ordinary LDS stores:
// waits for this wave's LDS operations (lgkmcnt) but not for its global loads
// or its global -> LDS copies (vmcnt), which __syncthreads() would also wait
// for through its release fence. The memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Workgroups are dealt to the 8 XCDs in turn (workgroup p runs on XCD p % 8).
// Remap a linear workgroup index so that each XCD gets one contiguous range
// of logical indices (the first count % 8 XCDs one more than the others):
// neighbouring work items then share an XCD and its L2, e.g. the 64 rows of a
// plane tile, or the GEMM tiles that read the same operand strips.
__device__ __forceinline__ int64_t xcd_contiguous(int64_t p, int64_t count) {
    const int64_t x = p % 8, q = count / 8, r = count % 8;
    return x * q + (x < r ? x : r) + p / 8;
}

// PLANE64 addressing. Byte offset, inside the qs plane, of the 4-byte group
// holding elements e..e+3 (e % 4 == 0) of chunk c of token t.
__device__ __forceinline__ int64_t plane_qs_off(int64_t t, int c, int e, int nchunk) {
    const int64_t g = t >> 6;
    const int r = (int)(t & 63);
    const int h = ((e >> 4) ^ (r >> 2) ^ (r >> 3)) & 1;
    return (g * nchunk + c) * kTileBytes + r * 32 + h * 16 + (e & 15);
}

__device__ __forceinline__ int64_t plane_sd_idx(int64_t t, int c, int nchunk) {
    return ((t >> 6) * nchunk + c) * kGroup + (t & 63);
}

}  // namespace q8

// ---------------------------------------------------------------------------
// Host-side helpers shared by the entry points.
// ---------------------------------------------------------------------------
namespace q8h {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Launch counters of the entry points (Q8_LAUNCH_* ids), process-wide.
inline std::atomic<int64_t> launches[Q8_LAUNCH_COUNTERS];

// The first failure among the calling thread's launches since its last
// launch_status() (hipSuccess: none).
inline thread_local hipError_t launch_error = hipSuccess;

// Every kernel launch of the library: hipLaunchKernel returns the status of
// this launch alone, which is kept for launch_status(). The thread's pending
// HIP error (hipGetLastError) is never read, so an error left by the caller's
// own earlier work is not reported as the library's.
template <typename... P, typename... A>
inline void launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, size_t shmem, hipStream_t s, A... args) {
    static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
    std::tuple<P...> vals{static_cast<P>(args)...};
    void* ptrs[sizeof...(P) > 0 ? sizeof...(P) : 1];
    std::apply([&ptrs](auto&... v) {
        size_t i = 0;
        ((ptrs[i++] = static_cast<void*>(&v)), ...);
    }, vals);
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, shmem, s);
    if (e != hipSuccess && launch_error == hipSuccess) launch_error = e;
}

// Status of the launches the calling thread made since the last call; on
// success one launch is added to the entry point's counter.
inline int launch_status(int counter) {
    const hipError_t e = launch_error;
    launch_error = hipSuccess;
    if (e != hipSuccess) return Q8_ELAUNCH;
    launches[counter].fetch_add(1, std::memory_order_relaxed);
    return Q8_OK;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace q8h
