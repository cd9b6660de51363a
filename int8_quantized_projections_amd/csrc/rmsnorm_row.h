// RMSNorm + quantize device code shared by rmsnorm_quant (producers.hip) and
// the one-launch decode step (gemv.hip), so the two write the same bits.
//
// Sources: [P2] "r51 producer-fused A-quantize" s2-s3 (the fused producer, the
// 64-token plane and its zero tail), [P3] "r5-r6 rewrite spec" point 7
// (tree-reduced amax, packed stores).
#pragma once

#include "q8_common.h"

namespace q8 {
namespace {

// kDstStage: ROW addressing into a workgroup's LDS staging rows (row t of the
// workgroup's consecutive rows at t modulo its row count), written out as plane
// tiles by the caller.
enum Dst : int { kDstNone = 0, kDstRow = 1, kDstPlane = 2, kDstStage = 3 };

// Streaming accesses: the non-temporal bit, so the line does not displace
// others from L2 and the MALL. Measured per stream, not applied wholesale:
// - every f32 output y and the PLANE64 tile stores: 5.1 -> 5.4 TB/s on the
//   3325x18944 swiglu_quant with the plane, 3.2 -> 3.6 on the 3325x18944
//   rmsnorm_quant, and never slower;
// - the gate and up inputs of swiglu_quant (row layout 5.3 -> 6.1 TB/s);
// - not the single input of q8_quantize or rmsnorm_quant: there they measured
//   slower (rmsnorm_quant 3325x3584, 21 -> 25 us), as a row that the previous
//   kernel just wrote is often still in the MALL;
// - not the RMSNorm weight row, which every row reads.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream(const float* p) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(float* p, const float4& v) {
    const f32x4_t t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<f32x4_t*>(p));
}
__device__ __forceinline__ void store_stream(void* p, const uint4& v) {
    const u32x4_t t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4_t*>(p));
}

// Write this lane's 4 quantized values (and, from the group's first lane,
// the block's scale word) for element e..e+3 of chunk c of row t.
template <int D>
__device__ __forceinline__ void store_quant(const Quant8& r, int64_t t, int c, int e, int K, int nb, int8_t* qs,
                                            uint32_t* sd) {
    if constexpr (D == kDstRow || D == kDstStage) {
        *reinterpret_cast<uint32_t*>(qs + t * K + (int64_t)c * kQK + e) = r.qs4;
        if (e == 0) sd[t * nb + c] = r.sd;
    } else if constexpr (D == kDstPlane) {
        *reinterpret_cast<uint32_t*>(qs + plane_qs_off(t, c, e, nb)) = r.qs4;
        if (e == 0) sd[plane_sd_idx(t, c, nb)] = r.sd;
    }
}

// ---------------------------------------------------------------------------
// RMSNorm + quantize, the row arithmetic shared by every form of the producer
// ([P2] s3.2: scale = rsqrt(mean(x^2) + eps), y = x * scale * w, then the
// quantize of y). A row is spread over WPR waves of a workgroup of WAVES waves;
// lane i of the row (i = 64*(wave % WPR) + lane) holds float4 index
// i + 64*WPR*k, so 8 consecutive lanes hold one 32-value block. The sum of
// squares, and so every output bit, depends on K, WPR and NV only.
//
// A row whose f32 sum of squares overflows (|x| above about 1.8e19 / sqrt(K))
// takes a second pass over x * 2^-80, whose squares stay in range for any
// finite x and K <= 2^24: y = (x * 2^-80) * rsqrt(sum((x * 2^-80)^2) / K +
// eps * 2^-160) * w, the same value. Rows whose sum is finite keep the first
// pass's bits. Every wave of a workgroup takes the second reduction when any
// of its rows needs it, so the barrier inside is reached by all of them.
// ---------------------------------------------------------------------------
constexpr float kDown = 0x1p-80f;  // the second pass's prescale

// The row's total over its WPR waves, and (any_big) whether the total of any
// row of the workgroup is not finite -- the same answer in every wave of the
// workgroup. WPR > 1 combines the waves' partial sums in buf (WAVES floats of
// LDS) behind a barrier that every wave of the workgroup must reach.
template <int WPR, int WAVES>
__device__ __forceinline__ float rms_row_total(float ss, float* buf, bool& any_big) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    ss = wave_sum(ss);
    if constexpr (WPR > 1) {
        constexpr int kRowsPerWg = WAVES / WPR;
        if (lane == 0) buf[wave] = ss;
        lds_barrier();  // global loads and copies into LDS stay in flight
        float mine = 0.0f;
        bool any = false;
#pragma unroll
        for (int r = 0; r < kRowsPerWg; ++r) {
            float tot = buf[r * WPR];
#pragma unroll
            for (int i = 1; i < WPR; ++i) tot += buf[r * WPR + i];
            any |= !__builtin_isfinite(tot);
            if (r == wave / WPR) mine = tot;
        }
        any_big = any;
        return mine;
    } else {
        any_big = !__builtin_isfinite(ss);
        return ss;
    }
}

// The rest of the row once its share is in registers: v[k] holds x (float4
// index li + 64*WPR*k of row t, any value past K or for a padded row), wv[k]
// the same index of w. Writes y (unless NULL) and the quantized output of row
// t. part, part2: WAVES floats of LDS each (the two passes' partial sums).
// Every wave of the workgroup must call it.
// wv: the same indices of w, as a float4[NV] in registers or as WLds (read
// from LDS where used).
template <int D, int NV, int WPR, int WAVES, typename WV>
__device__ __forceinline__ void rms_finish(float4 (&v)[NV], const WV& wv, float eps,
                                           float* __restrict__ y, int64_t t, int64_t rows, int64_t tpad, int K,
                                           int nb, int8_t* __restrict__ qs, uint32_t* __restrict__ sd, float* part,
                                           float* part2) {
    constexpr int kStride = kWave * WPR;  // float4 stride between a lane's elements
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int li = (wave % WPR) * kWave + lane;  // lane index inside the row
    const bool live = t < rows;
    const bool inrow = t < tpad;  // uniform per wave
    const int n4 = K >> 2;
    // masks applied only after every load is in flight
#pragma unroll
    for (int k = 0; k < NV; ++k)
        if (!live || li + kStride * k >= n4) v[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        ss = fmaf(v[k].x, v[k].x, ss);
        ss = fmaf(v[k].y, v[k].y, ss);
        ss = fmaf(v[k].z, v[k].z, ss);
        ss = fmaf(v[k].w, v[k].w, ss);
    }
    bool any_big;
    ss = rms_row_total<WPR, WAVES>(ss, part, any_big);
    // [P2] s3.2: scale = rsqrt(ss/d + eps), y = x * scale * w.
    float scale = rsqrtf(ss / (float)K + eps), pre = 1.0f;
    if (any_big) {  // uniform over the workgroup
        float s2 = 0.0f;
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const float a = v[k].x * kDown, b = v[k].y * kDown, c = v[k].z * kDown, d = v[k].w * kDown;
            s2 = fmaf(a, a, s2);
            s2 = fmaf(b, b, s2);
            s2 = fmaf(c, c, s2);
            s2 = fmaf(d, d, s2);
        }
        bool unused;
        s2 = rms_row_total<WPR, WAVES>(s2, part2, unused);
        if (!__builtin_isfinite(ss)) {
            scale = rsqrtf(s2 / (float)K + eps * kDown * kDown);
            pre = kDown;
        }
    }
    if (!inrow) return;
    // y == NULL: the quantized output only, no f32 row is written
    float4* __restrict__ y4 = y != nullptr ? reinterpret_cast<float4*>(y + (live ? t : 0) * K) : nullptr;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int idx = li + kStride * k;
        float4 o;  // pre is 1 (exact) unless the row took the second pass
        o.x = v[k].x * pre * scale * wv[k].x;
        o.y = v[k].y * pre * scale * wv[k].y;
        o.z = v[k].z * pre * scale * wv[k].z;
        o.w = v[k].w * pre * scale * wv[k].w;
        if (y4 != nullptr && live && idx < n4) store_stream(reinterpret_cast<float*>(y4 + idx), o);
        v[k] = o;  // zero for padded rows and past K
    }
    if constexpr (D != kDstNone) {
        const int64_t tq = D == kDstStage ? t % (WAVES / WPR) : t;  // the staging row
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int c = (li + kStride * k) >> 3;
            if (c < nb) {
                const Quant8 r = quantize_block8(v[k]);
                store_quant<D>(r, tq, c, (lane & 7) * 4, K, nb, qs, sd);
            }
        }
    }
}

// w held in LDS (K float4-indexed values, zero past K): element k of a lane's
// share is read where it is used.
template <int WPR>
struct WLds {
    const float4* base;  // this lane's first element: w4 + li
    __device__ __forceinline__ float4 operator[](int k) const { return base[kWave * WPR * k]; }
};

// Loads of row t's share (see rms_finish): x from clamped, always-valid
// addresses (padded rows read row 0), w the same indices.
template <int NV, int WPR>
__device__ __forceinline__ void rms_load_x(float4 (&v)[NV], const float* __restrict__ x, int64_t t, int64_t rows,
                                           int K) {
    constexpr int kStride = kWave * WPR;
    const int li = ((threadIdx.x >> 6) % WPR) * kWave + (threadIdx.x & 63);
    const int n4 = K >> 2;
    const float4* __restrict__ x4 = reinterpret_cast<const float4*>(x + (t < rows ? t : 0) * K);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int idx = li + kStride * k;
        v[k] = x4[idx < n4 ? idx : n4 - 1];
    }
}

template <int NV, int WPR>
__device__ __forceinline__ void rms_load_w(float4 (&wv)[NV], const float* __restrict__ w, int K) {
    constexpr int kStride = kWave * WPR;
    const int li = ((threadIdx.x >> 6) % WPR) * kWave + (threadIdx.x & 63);
    const int n4 = K >> 2;
    const float4* __restrict__ w4 = reinterpret_cast<const float4*>(w);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int idx = li + kStride * k;
        wv[k] = w4[idx < n4 ? idx : n4 - 1];
    }
}

// RMSNorm + quantize of the rows of logical workgroup `wg` (WAVES / WPR rows).
// The row stays in registers (NV float4 per lane, K <= 256*WPR*NV) between the
// sum of squares and the output, so x is read once, and w is loaded in the
// same wave of loads. NV == 0: rows wider than the register budget; x is read
// twice (the second read hits L2), with the same per-lane order of the sum of
// squares. Every wave of the workgroup must call it. qs and sd may point to LDS.
template <int D, int NV, int WPR, int WAVES>
__device__ __forceinline__ void rmsnorm_rows(const float* __restrict__ x, const float* __restrict__ w, float eps,
                                             float* __restrict__ y, int64_t rows, int64_t tpad, int K, int nb,
                                             int8_t* __restrict__ qs, uint32_t* __restrict__ sd, int64_t wg) {
    static_assert(WAVES % WPR == 0, "whole rows per workgroup");
    constexpr int kRowsPerWg = WAVES / WPR;
    constexpr int kStride = kWave * WPR;  // float4 stride between a lane's elements
    __shared__ float part[WAVES];
    __shared__ float part2[WAVES];  // the rescaled second pass (a separate buffer: no wait for the first's readers)
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = wg * kRowsPerWg + wave / WPR;

    if constexpr (NV > 0) {
        float4 v[NV], wv[NV];
        rms_load_x<NV, WPR>(v, x, t, rows, K);
        rms_load_w<NV, WPR>(wv, w, K);
        __builtin_amdgcn_sched_barrier(0);  // keep every x and w load ahead of the math
        rms_finish<D, NV, WPR, WAVES>(v, wv, eps, y, t, rows, tpad, K, nb, qs, sd, part, part2);
    } else {
        const int li = (wave % WPR) * kWave + lane;  // lane index inside the row
        const bool live = t < rows;
        const bool inrow = t < tpad;  // uniform per wave
        const int n4 = K >> 2;
        const float4* __restrict__ x4 = reinterpret_cast<const float4*>(x + (live ? t : 0) * K);
        const float4* __restrict__ w4 = reinterpret_cast<const float4*>(w);
        float4* __restrict__ y4 = y != nullptr ? reinterpret_cast<float4*>(y + (live ? t : 0) * K) : nullptr;
        float ss = 0.0f;
        if (live) {
            for (int idx = li; idx < n4; idx += kStride) {
                const float4 a = x4[idx];
                ss = fmaf(a.x, a.x, ss);
                ss = fmaf(a.y, a.y, ss);
                ss = fmaf(a.z, a.z, ss);
                ss = fmaf(a.w, a.w, ss);
            }
        }
        bool any_big;
        ss = rms_row_total<WPR, WAVES>(ss, part, any_big);
        float scale = rsqrtf(ss / (float)K + eps), pre = 1.0f;
        if (any_big) {  // uniform over the workgroup
            float s2 = 0.0f;
            if (live) {
                for (int idx = li; idx < n4; idx += kStride) {
                    const float4 a = x4[idx];
                    const float p = a.x * kDown, q = a.y * kDown, r = a.z * kDown, u = a.w * kDown;
                    s2 = fmaf(p, p, s2);
                    s2 = fmaf(q, q, s2);
                    s2 = fmaf(r, r, s2);
                    s2 = fmaf(u, u, s2);
                }
            }
            bool unused;
            s2 = rms_row_total<WPR, WAVES>(s2, part2, unused);
            if (!__builtin_isfinite(ss)) {
                scale = rsqrtf(s2 / (float)K + eps * kDown * kDown);
                pre = kDown;
            }
        }
        if (!inrow) return;
        const int steps = (n4 + kStride - 1) / kStride;
        for (int k = 0; k < steps; ++k) {
            const int idx = li + kStride * k;
            const int ic = idx < n4 ? idx : n4 - 1;
            const float4 a = x4[ic];
            const float4 wq = w4[ic];
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
            if (live && idx < n4) {
                o.x = a.x * pre * scale * wq.x;
                o.y = a.y * pre * scale * wq.y;
                o.z = a.z * pre * scale * wq.z;
                o.w = a.w * pre * scale * wq.w;
                if (y4 != nullptr) store_stream(reinterpret_cast<float*>(y4 + idx), o);
            }
            if constexpr (D != kDstNone) {
                const int c = idx >> 3;
                if (c < nb) {
                    const Quant8 r = quantize_block8(o);
                    store_quant<D>(r, t, c, (lane & 7) * 4, K, nb, qs, sd);
                }
            }
        }
    }
}

}  // namespace
}  // namespace q8
