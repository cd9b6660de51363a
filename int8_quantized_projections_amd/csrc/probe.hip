// HBM read probe: the practical read ceiling that the bandwidth figures of the
// projection path are read against ([P1] s3: a kernel's rate is its bytes over
// its time, judged against what the memory can deliver). A trivial kernel that
// streams a buffer once and does nothing else with it.
//
// Each lane reads 16-byte words, grid-stride, U loads per step (issued
// together, then consumed), XORs them, and every workgroup writes the XOR of
// its lanes, so no load is dead. Consecutive lanes read consecutive words: a
// wave's load instruction covers 1 KB of contiguous memory.
#include "q8_common.h"

namespace {

template <int U>
__global__ __launch_bounds__(256) void k_read_probe(const uint4* __restrict__ p, int64_t n16,
                                                    uint32_t* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = p[i + u * stride];
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {  // the last partial step
        const uint4 v = p[i];
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
    __shared__ uint32_t red[4];
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// Streams of equal length: NSRC sources read (0, 1 or 2) and, with W, one
// destination written, 16-byte grid-stride words, one load per source in flight
// per lane: a plain stream of the same read/write mix as a producer. Without a
// destination the XOR of what was read is written per workgroup to out.
template <int NSRC, bool W>
__global__ __launch_bounds__(256) void k_stream_probe(const uint4* __restrict__ s0, const uint4* __restrict__ s1,
                                                      uint4* __restrict__ dst, int64_t n16,
                                                      uint32_t* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    uint32_t acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
        uint4 v = make_uint4((uint32_t)i, 1u, 2u, 3u);
        if constexpr (NSRC >= 1) v = s0[i];
        if constexpr (NSRC >= 2) {
            const uint4 b = s1[i];
            v = make_uint4(v.x ^ b.x, v.y ^ b.y, v.z ^ b.z, v.w ^ b.w);
        }
        if constexpr (W)
            dst[i] = v;
        else
            acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if constexpr (!W) {
        for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
        __shared__ uint32_t red[4];
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
        __syncthreads();
        if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
    }
}

}  // namespace

extern "C" int q8_hbm_stream_probe(const void* src0, const void* src1, void* dst, int64_t bytes, int workgroups,
                                   uint32_t* out, void* stream) {
    const int nsrc = (src0 != nullptr) + (src1 != nullptr);
    if ((src1 != nullptr && src0 == nullptr) || (nsrc == 0 && dst == nullptr)) return Q8_EINVAL;
    if (dst == nullptr && out == nullptr) return Q8_EINVAL;
    if (bytes < 0 || bytes % 16 != 0 || workgroups < 1 || workgroups > 65536) return Q8_ESHAPE;
    if (!q8h::aligned(src0, 16) || !q8h::aligned(src1, 16) || !q8h::aligned(dst, 16) || !q8h::aligned(out, 4))
        return Q8_EALIGN;
    if (bytes == 0) return Q8_OK;
    const hipStream_t s = (hipStream_t)stream;
    const uint4* a = static_cast<const uint4*>(src0);
    const uint4* b = static_cast<const uint4*>(src1);
    uint4* d = static_cast<uint4*>(dst);
    const int64_t n16 = bytes / 16;
    const dim3 grid((unsigned)workgroups), block(256);
    if (dst == nullptr) {
        if (nsrc == 1)
            q8h::launch_kernel(k_stream_probe<1, false>, grid, block, 0, s, a, b, d, n16, out);
        else
            q8h::launch_kernel(k_stream_probe<2, false>, grid, block, 0, s, a, b, d, n16, out);
    } else if (nsrc == 0) {
        q8h::launch_kernel(k_stream_probe<0, true>, grid, block, 0, s, a, b, d, n16, out);
    } else if (nsrc == 1) {
        q8h::launch_kernel(k_stream_probe<1, true>, grid, block, 0, s, a, b, d, n16, out);
    } else {
        q8h::launch_kernel(k_stream_probe<2, true>, grid, block, 0, s, a, b, d, n16, out);
    }
    const hipError_t e = q8h::launch_error;
    q8h::launch_error = hipSuccess;
    return e == hipSuccess ? Q8_OK : Q8_ELAUNCH;
}

extern "C" int q8_hbm_read_probe(const void* buf, int64_t bytes, int workgroups, int loads_per_lane,
                                 uint32_t* out, void* stream) {
    if (buf == nullptr || out == nullptr) return Q8_EINVAL;
    if (bytes < 0 || bytes % 16 != 0 || workgroups < 1 || workgroups > 65536) return Q8_ESHAPE;
    if (loads_per_lane != 1 && loads_per_lane != 2 && loads_per_lane != 4) return Q8_EINVAL;
    if (!q8h::aligned(buf, 16) || !q8h::aligned(out, 4)) return Q8_EALIGN;
    if (bytes == 0) return Q8_OK;
    const hipStream_t s = (hipStream_t)stream;
    const uint4* p = static_cast<const uint4*>(buf);
    const int64_t n16 = bytes / 16;
    if (loads_per_lane == 1)
        q8h::launch_kernel(k_read_probe<1>, dim3((unsigned)workgroups), dim3(256), 0, s, p, n16, out);
    else if (loads_per_lane == 2)
        q8h::launch_kernel(k_read_probe<2>, dim3((unsigned)workgroups), dim3(256), 0, s, p, n16, out);
    else
        q8h::launch_kernel(k_read_probe<4>, dim3((unsigned)workgroups), dim3(256), 0, s, p, n16, out);
    const hipError_t e = q8h::launch_error;
    q8h::launch_error = hipSuccess;
    return e == hipSuccess ? Q8_OK : Q8_ELAUNCH;
}
