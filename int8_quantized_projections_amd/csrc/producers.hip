// Producers of quantized activations on gfx950: q8_quantize, rmsnorm_quant,
// swiglu_quant, and the load-time weight repack.
//
// Sources: [P1] "Fusion and the Activation-Quantization Discipline" s3-s4
// (quantize once, pass the buffer), [P2] "r51 producer-fused A-quantize"
// s2-s3 (fused producers, 64-token plane, zero tail), [P3] "r5-r6 rewrite
// spec" point 7 (tree-reduced amax, packed stores).
//
// Design (gfx950, not the pages' CUDA shapes): all three producers stream
// rows with 16-byte-per-lane coalesced loads and stores. Each 32-value block
// sits in 8 lanes, so the quantize runs from registers on the values the
// producer just computed -- no re-read of y, and the f32 store stays
// coalesced, which the pages had to trade against each other (their
// thread-per-chunk quantize body forced a re-read).
#include "q8_common.h"

using namespace q8;

namespace {

enum Dst : int { kDstNone = 0, kDstRow = 1, kDstPlane = 2 };

// Write this lane's 4 quantized values (and, from the group's first lane,
// the block's scale word) for element e..e+3 of chunk c of row t.
template <int D>
__device__ __forceinline__ void store_quant(const Quant8& r, int64_t t, int c, int e, int K, int nb, int8_t* qs,
                                            uint32_t* sd) {
    if constexpr (D == kDstRow) {
        *reinterpret_cast<uint32_t*>(qs + t * K + (int64_t)c * kQK + e) = r.qs4;
        if (e == 0) sd[t * nb + c] = r.sd;
    } else if constexpr (D == kDstPlane) {
        *reinterpret_cast<uint32_t*>(qs + plane_qs_off(t, c, e, nb)) = r.qs4;
        if (e == 0) sd[plane_sd_idx(t, c, nb)] = r.sd;
    }
}

// ---------------------------------------------------------------------------
// Element-wise producers (quantize of x, or swiglu then quantize).
// Grid: x = row (token, padded to 64 for PLANE64), y = chunk of units. A unit
// is 8 consecutive blocks = 256 floats = one float4 per lane. Each wave does
// UNR units, issuing all loads before any math.
// ---------------------------------------------------------------------------
constexpr int kUnr = 2;
constexpr int kWavesPerWg = 4;

template <int D, bool SWIGLU>
__global__ __launch_bounds__(256) void k_elementwise(const float* __restrict__ a, const float* __restrict__ b,
                                                     float* __restrict__ y, int64_t rows, int K, int nb,
                                                     int8_t* __restrict__ qs, uint32_t* __restrict__ sd) {
    const int64_t t = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int unit0 = (blockIdx.y * kWavesPerWg + wave) * kUnr;
    const bool live = t < rows;
    const int sub = lane & 7;
    float4 v[kUnr], w[kUnr];
    int blk[kUnr];
#pragma unroll
    for (int u = 0; u < kUnr; ++u) {
        blk[u] = (unit0 + u) * 8 + (lane >> 3);
        v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        w[u] = v[u];
        if (live && blk[u] < nb) {
            const int64_t off = t * K + (int64_t)blk[u] * kQK + sub * 4;
            v[u] = *reinterpret_cast<const float4*>(a + off);
            if constexpr (SWIGLU) w[u] = *reinterpret_cast<const float4*>(b + off);
        }
    }
#pragma unroll
    for (int u = 0; u < kUnr; ++u) {
        if (blk[u] >= nb) continue;  // whole 8-lane groups drop out together
        if constexpr (SWIGLU) {
            // [P2] s3.2: silu(g) * u with the plain expression.
            float4 o;
            o.x = v[u].x / (1.0f + expf(-v[u].x)) * w[u].x;
            o.y = v[u].y / (1.0f + expf(-v[u].y)) * w[u].y;
            o.z = v[u].z / (1.0f + expf(-v[u].z)) * w[u].z;
            o.w = v[u].w / (1.0f + expf(-v[u].w)) * w[u].w;
            if (!live) o = make_float4(0.f, 0.f, 0.f, 0.f);
            if (live) *reinterpret_cast<float4*>(y + t * K + (int64_t)blk[u] * kQK + sub * 4) = o;
            v[u] = o;
        }
        if constexpr (D != kDstNone) {
            const Quant8 r = quantize_block8(v[u]);  // padded rows hold zeros -> a zero block
            store_quant<D>(r, t, blk[u], sub * 4, K, nb, qs, sd);
        }
    }
}

// ---------------------------------------------------------------------------
// RMSNorm + quantize. One wave per row; the row stays in registers (NV
// float4 per lane, K <= 256*NV) between the sum of squares and the output,
// so x is read once. Lane l holds float4 index l + 64 i; the 8 lanes
// l = 8j..8j+7 of step i hold block 8i + j.
// NV == 0: rows wider than the register budget; x is read twice (the second
// read hits L2), with the same per-lane order of the sum of squares.
// ---------------------------------------------------------------------------
template <int D, int NV>
__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ x, const float* __restrict__ w, float eps,
                                                 float* __restrict__ y, int64_t rows, int64_t tpad, int K, int nb,
                                                 int8_t* __restrict__ qs, uint32_t* __restrict__ sd) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kWavesPerWg + wave;
    if (t >= tpad) return;  // uniform per wave
    const int n4 = K >> 2;
    const float4* __restrict__ x4 = reinterpret_cast<const float4*>(x + t * K);
    const float4* __restrict__ w4 = reinterpret_cast<const float4*>(w);
    float4* __restrict__ y4 = reinterpret_cast<float4*>(y + t * K);
    const bool live = t < rows;

    if constexpr (NV > 0) {
        float4 v[NV];
        float ss = 0.0f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int idx = lane + kWave * i;
            v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (live && idx < n4) v[i] = x4[idx];
        }
        if (live) {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                ss = fmaf(v[i].x, v[i].x, ss);
                ss = fmaf(v[i].y, v[i].y, ss);
                ss = fmaf(v[i].z, v[i].z, ss);
                ss = fmaf(v[i].w, v[i].w, ss);
            }
            ss = wave_sum(ss);
            // [P2] s3.2: scale = rsqrt(ss/d + eps), y = x * scale * w.
            const float scale = rsqrtf(ss / (float)K + eps);
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int idx = lane + kWave * i;
                if (idx < n4) {
                    const float4 wv = w4[idx];
                    float4 o;
                    o.x = v[i].x * scale * wv.x;
                    o.y = v[i].y * scale * wv.y;
                    o.z = v[i].z * scale * wv.z;
                    o.w = v[i].w * scale * wv.w;
                    y4[idx] = o;
                    v[i] = o;
                }
            }
        }
        if constexpr (D != kDstNone) {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int c = 8 * i + (lane >> 3);
                if (c < nb) {
                    const Quant8 r = quantize_block8(v[i]);
                    store_quant<D>(r, t, c, (lane & 7) * 4, K, nb, qs, sd);
                }
            }
        }
    } else {
        float scale = 0.0f;
        if (live) {
            float ss = 0.0f;
            for (int idx = lane; idx < n4; idx += kWave) {
                const float4 a = x4[idx];
                ss = fmaf(a.x, a.x, ss);
                ss = fmaf(a.y, a.y, ss);
                ss = fmaf(a.z, a.z, ss);
                ss = fmaf(a.w, a.w, ss);
            }
            ss = wave_sum(ss);
            scale = rsqrtf(ss / (float)K + eps);
        }
        const int steps = (n4 + kWave - 1) / kWave;
        for (int i = 0; i < steps; ++i) {
            const int idx = lane + kWave * i;
            const int c = 8 * i + (lane >> 3);
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
            if (live && idx < n4) {
                const float4 a = x4[idx];
                const float4 wv = w4[idx];
                o.x = a.x * scale * wv.x;
                o.y = a.y * scale * wv.y;
                o.z = a.z * scale * wv.z;
                o.w = a.w * scale * wv.w;
                y4[idx] = o;
            }
            if constexpr (D != kDstNone) {
                if (c < nb) {
                    const Quant8 r = quantize_block8(o);
                    store_quant<D>(r, t, c, (lane & 7) * 4, K, nb, qs, sd);
                }
            }
        }
    }
}

// GGUF Q8_0 blocks (34 bytes, 2-byte aligned: f16 d, int8 qs[32]) -> planes.
// Block b of the flat [N][K/32] block array maps to qs bytes [32b, 32b+32).
__global__ __launch_bounds__(256) void k_repack(const uint16_t* __restrict__ blocks, int64_t nblocks,
                                                int8_t* __restrict__ qs, uint16_t* __restrict__ d) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= nblocks) return;
    const uint16_t* src = blocks + b * 17;
    d[b] = src[0];
    uint32_t wv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) wv[j] = (uint32_t)src[1 + 2 * j] | ((uint32_t)src[2 + 2 * j] << 16);
    uint4* dst = reinterpret_cast<uint4*>(qs + b * kQK);
    dst[0] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    dst[1] = make_uint4(wv[4], wv[5], wv[6], wv[7]);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
int check_act_shape(int64_t rows, int64_t k) {
    if (rows < 0 || k <= 0 || (k % kQK) != 0) return Q8_ESHAPE;
    if (k > (int64_t)1 << 30 || rows > ((int64_t)1 << 31)) return Q8_ESHAPE;
    return Q8_OK;
}

int check_dst(int layout, const int8_t* qs, const uint32_t* sd, bool optional) {
    if (qs == nullptr && sd == nullptr) return optional ? Q8_OK : Q8_EINVAL;
    if (qs == nullptr || sd == nullptr) return Q8_EINVAL;
    if (layout != Q8_LAYOUT_ROW && layout != Q8_LAYOUT_PLANE64) return Q8_EINVAL;
    if (!q8h::aligned(qs, 16) || !q8h::aligned(sd, 4)) return Q8_EALIGN;
    return Q8_OK;
}

int64_t padded_rows(int64_t rows, int layout) {
    return layout == Q8_LAYOUT_PLANE64 ? q8h::ceil_div(rows, kGroup) * kGroup : rows;
}

template <bool SWIGLU>
int launch_elementwise(const float* a, const float* b, float* y, int64_t rows, int64_t k, int layout, int8_t* qs,
                       uint32_t* sd, hipStream_t s) {
    const int nb = (int)(k / kQK);
    const int64_t tpad = (qs == nullptr) ? rows : padded_rows(rows, layout);
    if (tpad == 0) return Q8_OK;
    const int units = (nb + 7) / 8;
    const dim3 grid((unsigned)tpad, (unsigned)q8h::ceil_div(units, kWavesPerWg * kUnr));
    if (qs == nullptr) {
        hipLaunchKernelGGL((k_elementwise<kDstNone, SWIGLU>), grid, dim3(256), 0, s, a, b, y, rows, (int)k, nb, qs, sd);
    } else if (layout == Q8_LAYOUT_ROW) {
        hipLaunchKernelGGL((k_elementwise<kDstRow, SWIGLU>), grid, dim3(256), 0, s, a, b, y, rows, (int)k, nb, qs, sd);
    } else {
        hipLaunchKernelGGL((k_elementwise<kDstPlane, SWIGLU>), grid, dim3(256), 0, s, a, b, y, rows, (int)k, nb, qs,
                           sd);
    }
    return q8h::launch_status();
}

template <int D>
void launch_rms(int nv, dim3 grid, hipStream_t s, const float* x, const float* w, float eps, float* y, int64_t rows,
                int64_t tpad, int k, int nb, int8_t* qs, uint32_t* sd) {
#define Q8_RMS_CASE(N)                                                                                         \
    case N:                                                                                                    \
        hipLaunchKernelGGL((k_rmsnorm<D, N>), grid, dim3(256), 0, s, x, w, eps, y, rows, tpad, k, nb, qs, sd); \
        break;
    switch (nv) {
        Q8_RMS_CASE(1)
        Q8_RMS_CASE(2)
        Q8_RMS_CASE(4)
        Q8_RMS_CASE(8)
        Q8_RMS_CASE(12)
        Q8_RMS_CASE(16)
        Q8_RMS_CASE(24)
        Q8_RMS_CASE(32)
        default:
            hipLaunchKernelGGL((k_rmsnorm<D, 0>), grid, dim3(256), 0, s, x, w, eps, y, rows, tpad, k, nb, qs, sd);
    }
#undef Q8_RMS_CASE
}

int rms_nv(int64_t k) {
    const int64_t need = q8h::ceil_div(k / 4, kWave);
    const int steps[] = {1, 2, 4, 8, 12, 16, 24, 32};
    for (int v : steps)
        if (need <= v) return v;
    return 0;
}

}  // namespace

extern "C" {

int q8_abi_version(void) { return Q8PROJ_ABI_VERSION; }

const char* q8_strerror(int code) {
    switch (code) {
        case Q8_OK: return "ok";
        case Q8_EINVAL: return "invalid argument (NULL pointer, unknown layout or count)";
        case Q8_ESHAPE: return "invalid shape (negative size, K not a positive multiple of 32, K mismatch, ldc < N)";
        case Q8_EALIGN: return "pointer not aligned as documented";
        case Q8_ELAUNCH: return "kernel launch failed";
        case Q8_ENODEV: return "no usable gfx950 device";
        default: return "unknown error";
    }
}

int q8_act_bytes(int64_t rows, int64_t k, int layout, size_t* qs_bytes, size_t* sd_bytes) {
    if (qs_bytes == nullptr || sd_bytes == nullptr) return Q8_EINVAL;
    if (layout != Q8_LAYOUT_ROW && layout != Q8_LAYOUT_PLANE64) return Q8_EINVAL;
    int rc = check_act_shape(rows, k);
    if (rc) return rc;
    const int64_t r = padded_rows(rows, layout);
    *qs_bytes = (size_t)(r * k);
    *sd_bytes = (size_t)(r * (k / kQK)) * sizeof(uint32_t);
    return Q8_OK;
}

int q8_quantize(const float* x, int64_t rows, int64_t k, int layout, int8_t* qs, uint32_t* sd, void* stream) {
    int rc = check_act_shape(rows, k);
    if (rc) return rc;
    if (x == nullptr) return Q8_EINVAL;
    if ((rc = check_dst(layout, qs, sd, false))) return rc;
    if (!q8h::aligned(x, 16)) return Q8_EALIGN;
    return launch_elementwise<false>(x, nullptr, nullptr, rows, k, layout, qs, sd, (hipStream_t)stream);
}

int swiglu_quant(const float* gate, const float* up, float* y, int64_t rows, int64_t k, int layout, int8_t* qs,
                 uint32_t* sd, void* stream) {
    int rc = check_act_shape(rows, k);
    if (rc) return rc;
    if (gate == nullptr || up == nullptr || y == nullptr) return Q8_EINVAL;
    if ((rc = check_dst(layout, qs, sd, true))) return rc;
    if (!q8h::aligned(gate, 16) || !q8h::aligned(up, 16) || !q8h::aligned(y, 16)) return Q8_EALIGN;
    return launch_elementwise<true>(gate, up, y, rows, k, layout, qs, sd, (hipStream_t)stream);
}

int rmsnorm_quant(const float* x, const float* w, float eps, float* y, int64_t rows, int64_t k, int layout,
                  int8_t* qs, uint32_t* sd, void* stream) {
    int rc = check_act_shape(rows, k);
    if (rc) return rc;
    if (x == nullptr || w == nullptr || y == nullptr) return Q8_EINVAL;
    if ((rc = check_dst(layout, qs, sd, true))) return rc;
    if (!q8h::aligned(x, 16) || !q8h::aligned(w, 16) || !q8h::aligned(y, 16)) return Q8_EALIGN;
    const int64_t tpad = (qs == nullptr) ? rows : padded_rows(rows, layout);
    if (tpad == 0) return Q8_OK;
    const dim3 grid((unsigned)q8h::ceil_div(tpad, kWavesPerWg));
    const int nv = rms_nv(k), nb = (int)(k / kQK);
    hipStream_t s = (hipStream_t)stream;
    if (qs == nullptr)
        launch_rms<kDstNone>(nv, grid, s, x, w, eps, y, rows, tpad, (int)k, nb, qs, sd);
    else if (layout == Q8_LAYOUT_ROW)
        launch_rms<kDstRow>(nv, grid, s, x, w, eps, y, rows, tpad, (int)k, nb, qs, sd);
    else
        launch_rms<kDstPlane>(nv, grid, s, x, w, eps, y, rows, tpad, (int)k, nb, qs, sd);
    return q8h::launch_status();
}

int q8_weights_repack(const void* gguf_blocks, int64_t n, int64_t k, int8_t* qs, uint16_t* d, void* stream) {
    int rc = check_act_shape(n, k);
    if (rc) return rc;
    if (gguf_blocks == nullptr || qs == nullptr || d == nullptr) return Q8_EINVAL;
    if (!q8h::aligned(gguf_blocks, 2) || !q8h::aligned(qs, 16) || !q8h::aligned(d, 2)) return Q8_EALIGN;
    const int64_t nblocks = n * (k / kQK);
    if (nblocks == 0) return Q8_OK;
    hipLaunchKernelGGL(k_repack, dim3((unsigned)q8h::ceil_div(nblocks, 256)), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const uint16_t*>(gguf_blocks), nblocks, qs, d);
    return q8h::launch_status();
}

}  // extern "C"
