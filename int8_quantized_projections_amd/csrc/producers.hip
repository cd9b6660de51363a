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
#include "gemm_common.h"
#include "rmsnorm_row.h"

using namespace q8;

namespace {

// ---------------------------------------------------------------------------
// Element-wise producers (quantize of x, or swiglu then quantize). A unit is
// 8 consecutive blocks of one row = 256 floats = one float4 per lane. Each
// wave does kUnr units, one load step at a time; rows are padded to 64 for
// PLANE64.
// ---------------------------------------------------------------------------
constexpr int kUnr = 4;
constexpr int kSeq = 1;  // units per load step
constexpr int kWavesPerWg = 4;

// SwiGLU of one element ([P2] s3.2: silu(g) * u = g / (1 + e^-g) * u), written
// with e = e^-|g|, which lies in (0, 1] for every finite g, so nothing overflows:
// silu(g) = g / (1 + e) for g >= 0 and g * e / (1 + e) for g < 0. exp2f keeps
// results below 2^-126 as denormals (the compiler scales the hardware exp2
// there). silu(g) is then within about 6e-8 * |g| relative (the rounding of the
// exponent argument) plus a few ulp while it is an f32 normal, and within
// 2^-126 absolute below that (gate below about -87.3).
__device__ __forceinline__ float swiglu1(float g, float u) {
    const float e = exp2f(-fabsf(g) * 1.44269504088896341f);
    const float r = __builtin_amdgcn_rcpf(1.0f + e);
    return (g >= 0.0f ? g : g * e) * r * u;
}

__device__ __forceinline__ float4 swiglu4(const float4& g, const float4& u) {
    return make_float4(swiglu1(g.x, u.x), swiglu1(g.y, u.y), swiglu1(g.z, u.z), swiglu1(g.w, u.w));
}

template <int D, bool SWIGLU>
__global__ __launch_bounds__(256) void k_elementwise(const float* __restrict__ a, const float* __restrict__ b,
                                                     float* __restrict__ y, int64_t rows, int K, int nb, int upr,
                                                     int64_t units, int8_t* __restrict__ qs, uint32_t* __restrict__ sd) {
    // The work is a flat list of (row, unit) pairs, upr units per row (a unit
    // is 8 blocks = 256 values; the last unit of a row may be partial). ROW and
    // f32-only outputs take it row-major. PLANE64 takes it as (64-row group,
    // unit column, row in the group), so consecutive waves finish whole 2048-byte
    // tiles together. Wave w of logical workgroup L takes kUnr consecutive
    // pairs; logical workgroups are spread over the XCDs in contiguous ranges,
    // so each tile is assembled in one L2.
    const int64_t L = xcd_contiguous(blockIdx.x, gridDim.x);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane & 7;
    const int64_t first = (L * kWavesPerWg + wave) * kUnr;
    int blk[kUnr];
    int64_t trow[kUnr];
    bool live[kUnr];
#pragma unroll
    for (int u = 0; u < kUnr; ++u) {
        const int64_t un = first + u < units ? first + u : units - 1;  // wave-uniform
        int64_t col;
        if constexpr (D == kDstPlane) {
            const int64_t gj = un / kGroup;  // group * upr + unit column
            trow[u] = (gj / upr) * kGroup + un % kGroup;
            col = gj % upr;
        } else {
            trow[u] = un / upr;
            col = un % upr;
        }
        blk[u] = (int)col * 8 + (lane >> 3);
        if (first + u >= units) blk[u] = nb;  // past the end: no output
        live[u] = trow[u] < rows;
    }
    // PLANE64: this workgroup covers rows 16k..16k+15 of one 64-row group at one
    // 8-chunk column, i.e. a 512-byte slice of each of 8 tiles. The quantized
    // bytes are gathered in LDS and written as whole slices (16 bytes per lane).
    constexpr int kSlice = kWavesPerWg * kUnr;  // rows per workgroup (16)
    // the write-out below stores 16-row slices: 8 chunks x 512 bytes by 256 threads
    static_assert(kSlice * kQK == 512 && kWavesPerWg * 64 == 8 * 32, "16-row slices, 256 threads");
    constexpr int kCs = kSlice * 8 + 8;  // words per chunk slice, padded against bank conflicts
    __shared__ __attribute__((aligned(16))) uint32_t pq[D == kDstPlane ? 8 * kCs : 1];
    __shared__ uint32_t psd[D == kDstPlane ? 8 * kSlice : 1];
    // The units go in steps of kSeq: a step's loads are issued, then its math
    // and stores run. One unit per step measured as fast as issuing all kUnr
    // units' loads first (within 1-3%), with fewer registers live.
#pragma unroll
    for (int u0 = 0; u0 < kUnr; u0 += kSeq) {
        float4 v[kSeq], w[kSeq];
        // Unconditional loads from clamped, always-valid addresses (a load inside a
        // divergent branch serialises the stream); padded rows read row 0 and are
        // zeroed at use.
#pragma unroll
        for (int i = 0; i < kSeq; ++i) {
            const int u = u0 + i;
            const int bc = blk[u] < nb ? blk[u] : nb - 1;
            const int64_t off = (live[u] ? trow[u] : 0) * K + (int64_t)bc * kQK + sub * 4;
            if constexpr (SWIGLU) {  // two input streams: both read as streaming
                v[i] = load_stream(a + off);
                w[i] = load_stream(b + off);
            } else {  // one stream: ordinary loads measured faster
                v[i] = *reinterpret_cast<const float4*>(a + off);
            }
        }
#pragma unroll
        for (int i = 0; i < kSeq; ++i) {
            const int u = u0 + i;
            if (blk[u] >= nb) continue;  // whole 8-lane groups drop out together
            if constexpr (SWIGLU) {
                const float4 o = swiglu4(v[i], w[i]);
                if (y != nullptr && live[u])  // y == NULL: quantized output only
                    store_stream(y + trow[u] * K + (int64_t)blk[u] * kQK + sub * 4, o);
                v[i] = o;
            }
            if constexpr (D != kDstNone) {
                // padded rows (which loaded row 0) quantize a zero block: all bytes zero
                const Quant8 r = quantize_block8(live[u] ? v[i] : make_float4(0.f, 0.f, 0.f, 0.f));
                if constexpr (D == kDstPlane) {
                    const int rs = wave * kUnr + u;  // row in the slice
                    const int rt = (int)(trow[u] & 63);  // row in the tile (selects the half swizzle)
                    const int e = sub * 4;
                    const int h = ((e >> 4) ^ (rt >> 2) ^ (rt >> 3)) & 1;
                    const int cl = lane >> 3;  // chunk in the column
                    pq[cl * kCs + rs * 8 + h * 4 + ((e & 15) >> 2)] = r.qs4;
                    if (sub == 0) psd[cl * kSlice + rs] = r.sd;
                } else {
                    store_quant<D>(r, trow[u], blk[u], sub * 4, K, nb, qs, sd);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (D == kDstPlane) {
        __syncthreads();
        const int64_t g = trow[0] >> 6;  // same group and column for the whole workgroup
        const int r0 = (int)(trow[0] & 63) - wave * kUnr;  // first row of the slice
        // qs: 8 chunks x 512 bytes; thread i writes 16 bytes of chunk i / 32
        const int tid = threadIdx.x;
        const int cl = tid >> 5;
        const int64_t first_u = (L * kWavesPerWg) * kUnr;
        const int64_t col = (first_u / kGroup) % upr;
        const int c = (int)col * 8 + cl;
        if (c < nb) {
            const uint4 v4 = *reinterpret_cast<const uint4*>(&pq[cl * kCs + (tid & 31) * 4]);
            store_stream(qs + (g * nb + c) * kTileBytes + r0 * 32 + (tid & 31) * 16, v4);
        }
        if (tid < 8 * kSlice) {
            const int c2 = (int)col * 8 + tid / kSlice;
            if (c2 < nb) sd[(g * nb + c2) * kGroup + r0 + tid % kSlice] = psd[tid];
        }
    }
}

// ---------------------------------------------------------------------------
// q8_quantize (SWIGLU: swiglu_quant first) into PLANE64 for wide activations:
// each wave streams runs of RUN consecutive units (RUN KB of f32) of one row
// instead of 1 KB pieces of four rows.
// A workgroup covers 16 rows (one quarter of a 64-row group) by RUN units
// (8*RUN chunks): wave w takes rows 4w..4w+3 of the quarter, and for each row
// the RUN units in order. The quantized bytes are gathered in LDS and written as whole
// 512-byte tile slices, as in k_elementwise. Work items are ordered (group,
// 8*RUN-chunk column, quarter), so the four quarters of a tile run in consecutive
// workgroups of one XCD. The quantize arithmetic is the same function as
// every other producer's, so the plane has the same bits as k_elementwise's.
// Measured for q8_quantize (median us, k_elementwise -> 4 KB runs -> 2 KB
// runs): 3325x18944 62.2 -> 55.3 -> 51.6 (5.2 -> 6.25 TB/s), 2048x16384
// 35.5 -> 31.6 -> 30.7, 1024x18944 23.1 -> 22.2 -> 20.5, 3325x7168
// 26.8 -> 25.1 -> 23.5, 3325x3584 16.6 -> 18.7 (832 items) -> 15.0 (1456).
// With 4 KB runs 512x3584 took 11.0 us against 7.1: with fewer workgroups it
// loses once the grid no longer fills the chip, hence kRunMinWgs. For
// swiglu_quant it pays only without the f32 output and with 4 KB runs (plane
// only: 3325x18944 103.0 -> 101.4 us, 3325x7168 41.5 -> 38.3, 2048x16384
// 54.9 -> 53.6; 2 KB runs 102-103 us); with y it measured slower (152.3 ->
// 165.5 us with 4 KB runs, 156.5 with 2 KB), so that form keeps k_elementwise.
// SWIGLU computes silu(g) * u exactly as k_elementwise does (the same bits).
// ---------------------------------------------------------------------------
// Rows per workgroup (4 per wave). Whole 64-row groups per workgroup (16
// waves; each workgroup then writes whole tiles, a contiguous 16-32 KB run of
// the plane) measured slower: q8_quantize 3325x18944 51.0 -> 57.5 us,
// swiglu_quant with y 152.6 -> 171.5 us.
constexpr int kRunRows = 16;
constexpr int kRunMinWgs = 1024;  // fewer work items take k_elementwise
// units per row per wave (RUN x 1 KB of f32): 2 for q8_quantize, 4 for swiglu_quant
constexpr int run_units(bool swiglu) { return swiglu ? 4 : 2; }

template <bool SWIGLU, int RUN = run_units(SWIGLU), int QR = kRunRows>
__global__ __launch_bounds__(QR * 16) void k_quantize_plane_runs(const float* __restrict__ x,
                                                                 const float* __restrict__ xb, float* __restrict__ y,
                                                                 int64_t rows, int K, int nb, int ncol,
                                                                 int8_t* __restrict__ qs, uint32_t* __restrict__ sd) {
    constexpr int kChunks = RUN * 8;      // chunks per workgroup column
    constexpr int kParts = kGroup / QR;   // workgroups per 64-row group and column
    constexpr int kThreads = QR * 16;
    static_assert(kGroup % QR == 0 && kChunks * 2 * QR % kThreads == 0 && kChunks * QR % kThreads == 0,
                  "whole passes of the write-out");
    const int64_t L = xcd_contiguous(blockIdx.x, gridDim.x);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane & 7;
    const int64_t g = L / (kParts * (int64_t)ncol);  // 64-row group
    const int col = (int)((L / kParts) % ncol);      // 8*RUN-chunk column
    const int part = (int)(L % kParts);
    constexpr int kCs = QR * 8 + 8;  // words per chunk slice, padded against bank conflicts
    __shared__ __attribute__((aligned(16))) uint32_t pq[kChunks * kCs];
    __shared__ uint32_t psd[kChunks * QR];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rs = 4 * wave + i;        // row in the workgroup
        const int rt = QR * part + rs;      // row in the tile
        const int64_t t = g * kGroup + rt;
        const bool live = t < rows;
#pragma unroll
        for (int j = 0; j < RUN; ++j) {
            // one unit per step: its load, then its quantize (loads from clamped,
            // always-valid addresses; padded rows read row 0 and quantize zeros)
            const int cc = 8 * j + (lane >> 3);   // chunk in the column
            const int blk = kChunks * col + cc;
            const int bc = blk < nb ? blk : nb - 1;
            const int64_t off = (live ? t : 0) * K + (int64_t)bc * kQK + sub * 4;
            float4 v;
            float4 wv;
            if constexpr (SWIGLU) {
                v = load_stream(x + off);
                wv = load_stream(xb + off);
            } else {
                v = *reinterpret_cast<const float4*>(x + off);
            }
            if (blk < nb) {  // whole 8-lane groups drop out together
                if constexpr (SWIGLU) {
                    const float4 o = swiglu4(v, wv);
                    if (y != nullptr && live) store_stream(y + off, o);
                    v = o;
                }
                const Quant8 r = quantize_block8(live ? v : make_float4(0.f, 0.f, 0.f, 0.f));
                const int e = sub * 4;
                const int h = ((e >> 4) ^ (rt >> 2) ^ (rt >> 3)) & 1;
                pq[cc * kCs + rs * 8 + h * 4 + ((e & 15) >> 2)] = r.qs4;
                if (sub == 0) psd[cc * QR + rs] = r.sd;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __syncthreads();
    const int tid = threadIdx.x;
    // qs: 8*RUN chunks x (QR rows x 32 bytes), 16 bytes per thread and pass
#pragma unroll
    for (int it = 0; it < kChunks * 2 * QR / kThreads; ++it) {
        const int p = kThreads * it + tid;
        const int cc = p / (2 * QR), q = p % (2 * QR);
        const int c = kChunks * col + cc;
        if (c < nb) {
            const uint4 v4 = *reinterpret_cast<const uint4*>(&pq[cc * kCs + q * 4]);
            store_stream(qs + (g * nb + c) * kTileBytes + QR * part * kQK + q * 16, v4);
        }
    }
    // scale words: 8*RUN chunks x QR rows
#pragma unroll
    for (int it = 0; it < kChunks * QR / kThreads; ++it) {
        const int i = kThreads * it + tid;
        const int cc = i / QR, rs = i % QR;
        const int c = kChunks * col + cc;
        if (c < nb) sd[(g * nb + c) * kGroup + QR * part + rs] = psd[i];
    }
}

// RMSNorm + quantize kernel: WPR waves per row (see dispatch_rms); the row
// arithmetic is rmsnorm_rows in rmsnorm_row.h.
template <int D, int NV, int WPR, int WAVES = kWavesPerWg>
__global__ __launch_bounds__(WAVES * 64) void k_rmsnorm(const float* __restrict__ x, const float* __restrict__ w,
                                                        float eps, float* __restrict__ y, int64_t rows, int64_t tpad,
                                                        int K, int nb, int8_t* __restrict__ qs,
                                                        uint32_t* __restrict__ sd) {
    rmsnorm_rows<D, NV, WPR, WAVES>(x, w, eps, y, rows, tpad, K, nb, qs, sd, xcd_contiguous(blockIdx.x, gridDim.x));
}

// rmsnorm_quant into the PLANE64 layout for many rows: 16 waves, up to 8
// consecutive rows per workgroup, two waves per row with the row in registers
// (rms_finish: the same arithmetic and bits as the other two-wave forms). The
// rows' quantized blocks and scale words are staged in LDS and written as runs
// of the plane tiles (a 256-byte slice for 8 rows) and runs of scale words:
// written straight from each row, every block is one 32-byte piece and one
// 4-byte word, 2 KB and 256 bytes from the row's next block (measured: 27.4 us
// for 3325x3584, of which 6 us for the 13.4 MB of plane).
constexpr int kStageRows = 8;
constexpr int kStageMaxK = 4096;  // two waves x 64 lanes x 8 float4

// The balanced form, for up to 4096 padded rows (at most two of these
// workgroups per CU): a kernel that moves every byte once is held to a CU's
// share of the chip's bandwidth, so its time follows the most-loaded CU. With
// 8 rows per workgroup, 3328 rows are 416 workgroups: 160 CUs carry 16 rows and
// 96 carry 8 (measured: 2048 rows 14.2 us, 2560 rows 21.6 us, 3328 rows
// 24.8 us). Here the row pairs are dealt evenly to the CUs instead: CU c holds
// P or P + 1 pairs, up to 4 of them in workgroup c and the rest in workgroup
// c + kCUs (the first kCUs workgroups of a grid take one CU each before any CU
// takes a second), so no CU carries more than 2 * ceil(tpad / 512) rows, and a
// CU's first workgroup is full before its second takes rows (up to 2048 rows
// the second workgroups have none and exit). A workgroup's rows are
// contiguous, an even count of at most 8 starting at an even row, so the plane
// runs stay 64-byte aligned.
constexpr int kCUs = 256;                             // MI355X
constexpr int64_t kBalMaxRows = 2 * kCUs * kStageRows;  // 4096

// First row s and row count n of workgroup b of the balanced grid (2 * kCUs).
__device__ __forceinline__ void bal_rows(int b, int64_t tpad, int64_t& s, int& n) {
    const int u = (int)(tpad / 2);  // row pairs
    const int P = u / kCUs, r = u % kCUs;
    auto first = [](int p) { return 2 * min(p, kStageRows / 2); };       // rows of a CU's first workgroup, p pairs
    auto second = [](int p) { return 2 * max(p - kStageRows / 2, 0); };  // and of its second
    if (b < kCUs) {
        s = (int64_t)min(b, r) * first(P + 1) + (int64_t)max(0, b - r) * first(P);
        n = first(b < r ? P + 1 : P);
    } else {
        const int c = b - kCUs;
        s = (int64_t)r * first(P + 1) + (int64_t)(kCUs - r) * first(P) + (int64_t)min(c, r) * second(P + 1) +
            (int64_t)max(0, c - r) * second(P);
        n = second(c < r ? P + 1 : P);
    }
}

// BAL: the balanced rows above; else 8 consecutive rows per workgroup.
template <int NV, bool BAL>
__global__ __launch_bounds__(1024) void k_rmsnorm_plane8(const float* __restrict__ x, const float* __restrict__ w,
                                                         float eps, float* __restrict__ y, int64_t rows,
                                                         int64_t tpad, int K, int nb, int8_t* __restrict__ qs,
                                                         uint32_t* __restrict__ sd) {
    constexpr int kWaves = 2 * kStageRows;
    __shared__ __attribute__((aligned(16))) int8_t st_q[kStageRows * kStageMaxK];
    __shared__ uint32_t st_d[kStageRows * (kStageMaxK / kQK)];
    __shared__ __attribute__((aligned(16))) float4 st_w[kStageMaxK / 4];
    __shared__ float part[kWaves], part2[kWaves];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    int64_t s0;  // this workgroup's rows: s0 .. s0+n-1, staged in LDS at row % 8
    int n;
    if constexpr (BAL) {
        bal_rows(blockIdx.x, tpad, s0, n);
        if (n == 0) return;  // the whole workgroup: no barrier is left waiting
    } else {
        s0 = xcd_contiguous(blockIdx.x, gridDim.x) * kStageRows;
        n = kStageRows;
    }
    // a row slot past the workgroup's rows computes nothing it writes (t = tpad)
    const int64_t t = wave / 2 < n ? s0 + wave / 2 : tpad;
    // w once per workgroup, in LDS: one 1 KB copy per wave (bytes past K read as zeros),
    // so a lane holds only its x in registers (two workgroups fit a CU)
    q8gemm::lds_copy16(q8gemm::make_rsrc(w, (int64_t)K * 4), (uint32_t)(lane * 16), (uint32_t)(wave * 1024),
                       reinterpret_cast<int8_t*>(st_w) + wave * 1024);
    float4 v[NV];
    if (t < rows) {  // wave-uniform: padded and unused slots load nothing (their values are zeroed)
        rms_load_x<NV, 2>(v, x, t, rows, K);
    } else {
#pragma unroll
        for (int k = 0; k < NV; ++k) v[k] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    q8gemm::wait_copies();
    __syncthreads();
    const WLds<2> wl{st_w + (wave % 2) * kWave + lane};
    rms_finish<kDstStage, NV, 2, kWaves>(v, wl, eps, y, t, rows, tpad, K, nb, st_q, st_d, part, part2);
    __syncthreads();
    // chunk c of rows s0 .. s0+n-1 is a run of 32n contiguous bytes of a plane tile (of two
    // tiles when the rows cross a 64-token group); piece i = (c, row slot, half) in destination
    // order, each half taken from the source half it holds after the swizzle
    for (int i = (int)threadIdx.x; i < nb * kStageRows * 2; i += 1024) {
        const int c = i / (kStageRows * 2), j = (i >> 1) % kStageRows, hd = i & 1;
        if (j < n) {
            const int64_t tt = s0 + j, g = tt >> 6;
            const int row = (int)(tt & 63);
            const int hs = hd ^ (((row >> 2) ^ (row >> 3)) & 1);
            const uint4 q = *reinterpret_cast<const uint4*>(st_q + (int)(tt % kStageRows) * K + c * kQK + hs * 16);
            store_stream(qs + (g * nb + c) * kTileBytes + row * kQK + hd * 16, q);
        }
    }
    for (int i = (int)threadIdx.x; i < nb * kStageRows; i += 1024) {
        const int c = i / kStageRows, j = i % kStageRows;
        if (j < n) {
            const int64_t tt = s0 + j;
            sd[((tt >> 6) * nb + c) * kGroup + (tt & 63)] = st_d[(int)(tt % kStageRows) * nb + c];
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
    const int upr = (nb + 7) / 8;  // units per row
    const int64_t units = tpad * upr;
    const int64_t wgs = q8h::ceil_div(units, kWavesPerWg * kUnr);
    if (wgs > INT32_MAX) return Q8_ESHAPE;
    const dim3 grid((unsigned)wgs);
    // the 4 KB-run order: q8_quantize and the plane-only swiglu_quant (with an
    // f32 output as well, swiglu_quant measured faster in k_elementwise's order)
    if (!SWIGLU || y == nullptr) {
        if (qs != nullptr && layout == Q8_LAYOUT_PLANE64) {
            const int ncol = (int)q8h::ceil_div(nb, 8 * run_units(SWIGLU));
            const int64_t items = (tpad / kGroup) * ncol * (kGroup / kRunRows);
            if (items >= kRunMinWgs && items <= INT32_MAX) {
                q8h::launch_kernel(k_quantize_plane_runs<SWIGLU>, dim3((unsigned)items), dim3(kRunRows * 16), 0, s, a,
                                   b, y, rows, (int)k, nb, ncol, qs, sd);
                return q8h::launch_status(SWIGLU ? Q8_LAUNCH_SWIGLU_QUANT : Q8_LAUNCH_QUANTIZE);
            }
        }
    }
    if (qs == nullptr) {
        q8h::launch_kernel((k_elementwise<kDstNone, SWIGLU>), grid, dim3(256), 0, s, a, b, y, rows, (int)k, nb, upr,
                           units, qs, sd);
    } else if (layout == Q8_LAYOUT_ROW) {
        q8h::launch_kernel((k_elementwise<kDstRow, SWIGLU>), grid, dim3(256), 0, s, a, b, y, rows, (int)k, nb, upr,
                           units, qs, sd);
    } else {
        q8h::launch_kernel((k_elementwise<kDstPlane, SWIGLU>), grid, dim3(256), 0, s, a, b, y, rows, (int)k, nb, upr,
                           units, qs, sd);
    }
    return q8h::launch_status(SWIGLU ? Q8_LAUNCH_SWIGLU_QUANT : Q8_LAUNCH_QUANTIZE);
}

template <int D, int WPR, int WAVES = kWavesPerWg>
void launch_rms(int nv, dim3 grid, hipStream_t s, const float* x, const float* w, float eps, float* y, int64_t rows,
                int64_t tpad, int k, int nb, int8_t* qs, uint32_t* sd) {
    const dim3 block(WAVES * 64);
#define Q8_RMS_CASE(N)                                                                                           \
    case N:                                                                                                      \
        q8h::launch_kernel((k_rmsnorm<D, N, WPR, WAVES>), grid, block, 0, s, x, w, eps, y, rows, tpad, k, nb, qs, \
                           sd);                                                                                  \
        break;
    // at 1024 threads a lane has 128 VGPRs: more than 8 float4 per lane take the two-pass form
    if (WAVES > kWavesPerWg && nv > 8) nv = 0;
    switch (nv) {
        Q8_RMS_CASE(1)
        Q8_RMS_CASE(2)
        Q8_RMS_CASE(4)
        Q8_RMS_CASE(8)
        case 12:
        case 16:
        case 24:
        case 32:
            if constexpr (WAVES == kWavesPerWg) {
                switch (nv) {
                    Q8_RMS_CASE(12)
                    Q8_RMS_CASE(16)
                    Q8_RMS_CASE(24)
                    Q8_RMS_CASE(32)
                }
                break;
            }
            [[fallthrough]];
        default:
            q8h::launch_kernel((k_rmsnorm<D, 0, WPR, WAVES>), grid, block, 0, s, x, w, eps, y, rows, tpad, k, nb, qs,
                               sd);
    }
#undef Q8_RMS_CASE
}

// Float4 registers per lane for a row of width k spread over wpr waves
// (0 = too wide for registers: the two-pass form).
int rms_nv(int64_t k, int wpr) {
    const int64_t need = q8h::ceil_div(k / 4, (int64_t)kWave * wpr);
    const int steps[] = {1, 2, 4, 8, 12, 16, 24, 32};
    for (int v : steps)
        if (need <= v) return v;
    return 0;
}

// Waves per row: 16 (one 1024-thread workgroup per row) for a handful of rows,
// as at decode, where a row's latency is the cost: each lane then quantizes
// two blocks instead of eight; 4 up to 1024 rows; else 2 (half the row per wave
// keeps the kernel near 100 VGPRs, so enough waves are resident to stream).
int rms_wpr(int64_t rows) { return rows <= 16 ? 16 : rows < 1024 ? 4 : 2; }

template <int D>
void dispatch_rms(hipStream_t s, const float* x, const float* w, float eps, float* y, int64_t rows, int64_t tpad,
                  int k, int nb, int8_t* qs, uint32_t* sd) {
    const int wpr = rms_wpr(rows);
    const int nv = rms_nv(k, wpr);
    if (wpr == 16) {
        launch_rms<D, 16, 16>(nv, dim3((unsigned)tpad), s, x, w, eps, y, rows, tpad, k, nb, qs, sd);
        return;
    }
    if constexpr (D == kDstPlane) {
        // many rows held in registers: up to 8 rows per workgroup, the plane staged in LDS and
        // written in runs
        if (wpr == 2 && (nv == 4 || nv == 8) && k <= kStageMaxK) {
            const dim3 block(2 * kStageRows * 64);
            if (tpad <= kBalMaxRows) {  // rows dealt evenly to the CUs, two workgroups each
                const dim3 bgrid((unsigned)(2 * kCUs));
                if (nv == 4)
                    q8h::launch_kernel(k_rmsnorm_plane8<4, true>, bgrid, block, 0, s, x, w, eps, y, rows, tpad, k,
                                       nb, qs, sd);
                else
                    q8h::launch_kernel(k_rmsnorm_plane8<8, true>, bgrid, block, 0, s, x, w, eps, y, rows, tpad, k,
                                       nb, qs, sd);
                return;
            }
            const dim3 sgrid((unsigned)(tpad / kStageRows));
            if (nv == 4)
                q8h::launch_kernel(k_rmsnorm_plane8<4, false>, sgrid, block, 0, s, x, w, eps, y, rows, tpad, k, nb,
                                   qs, sd);
            else
                q8h::launch_kernel(k_rmsnorm_plane8<8, false>, sgrid, block, 0, s, x, w, eps, y, rows, tpad, k, nb,
                                   qs, sd);
            return;
        }
    }
    const dim3 grid((unsigned)q8h::ceil_div(tpad, kWavesPerWg / wpr));
    if (wpr == 4)
        launch_rms<D, 4>(nv, grid, s, x, w, eps, y, rows, tpad, k, nb, qs, sd);
    else
        launch_rms<D, 2>(nv, grid, s, x, w, eps, y, rows, tpad, k, nb, qs, sd);
}

}  // namespace

extern "C" {

int q8_abi_version(void) { return Q8PROJ_ABI_VERSION; }

int q8_launch_counts(int64_t* counts, int n) {
    if (n < 0 || (counts == nullptr && n > 0)) return Q8_EINVAL;
    for (int i = 0; i < n && i < Q8_LAUNCH_COUNTERS; ++i) counts[i] = q8h::launches[i].load(std::memory_order_relaxed);
    return Q8_LAUNCH_COUNTERS;
}

void q8_launch_counts_reset(void) {
    for (int i = 0; i < Q8_LAUNCH_COUNTERS; ++i) q8h::launches[i].store(0, std::memory_order_relaxed);
}

const char* q8_launch_counter_name(int id) {
    static const char* const names[Q8_LAUNCH_COUNTERS] = {
        "q8_quantize", "rmsnorm_quant", "swiglu_quant", "q8_gemv", "q8_gemv_shared_multi",
        "q8_gemv_f32", "q8_gemm", "q8_gemm_shared_multi", "q4k_gemm", "q8_weights_repack",
        "q8_gemv_shared_multi_plus_f32", "rmsnorm_quant_gemv_shared_multi_plus_f32"};
    return (id >= 0 && id < Q8_LAUNCH_COUNTERS) ? names[id] : nullptr;
}

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

int q8_plane_bytes(int64_t t, int64_t k, size_t* qs_bytes, size_t* sd_bytes) {
    return q8_act_bytes(t, k, Q8_LAYOUT_PLANE64, qs_bytes, sd_bytes);
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
    if (gate == nullptr || up == nullptr) return Q8_EINVAL;
    if ((rc = check_dst(layout, qs, sd, true))) return rc;
    if (y == nullptr && qs == nullptr) return Q8_EINVAL;  // nothing to produce
    if (!q8h::aligned(gate, 16) || !q8h::aligned(up, 16) || !q8h::aligned(y, 16)) return Q8_EALIGN;
    return launch_elementwise<true>(gate, up, y, rows, k, layout, qs, sd, (hipStream_t)stream);
}

int rmsnorm_quant(const float* x, const float* w, float eps, float* y, int64_t rows, int64_t k, int layout,
                  int8_t* qs, uint32_t* sd, void* stream) {
    int rc = check_act_shape(rows, k);
    if (rc) return rc;
    if (x == nullptr || w == nullptr) return Q8_EINVAL;
    if ((rc = check_dst(layout, qs, sd, true))) return rc;
    if (y == nullptr && qs == nullptr) return Q8_EINVAL;  // nothing to produce
    if (!q8h::aligned(x, 16) || !q8h::aligned(w, 16) || !q8h::aligned(y, 16)) return Q8_EALIGN;
    const int64_t tpad = (qs == nullptr) ? rows : padded_rows(rows, layout);
    if (tpad == 0) return Q8_OK;
    const int nb = (int)(k / kQK);
    hipStream_t s = (hipStream_t)stream;
    if (qs == nullptr)
        dispatch_rms<kDstNone>(s, x, w, eps, y, rows, tpad, (int)k, nb, qs, sd);
    else if (layout == Q8_LAYOUT_ROW)
        dispatch_rms<kDstRow>(s, x, w, eps, y, rows, tpad, (int)k, nb, qs, sd);
    else
        dispatch_rms<kDstPlane>(s, x, w, eps, y, rows, tpad, (int)k, nb, qs, sd);
    return q8h::launch_status(Q8_LAUNCH_RMSNORM_QUANT);
}

int q8_weights_repack(const void* gguf_blocks, int64_t n, int64_t k, int8_t* qs, uint16_t* d, void* stream) {
    int rc = check_act_shape(n, k);
    if (rc) return rc;
    if (gguf_blocks == nullptr || qs == nullptr || d == nullptr) return Q8_EINVAL;
    if (!q8h::aligned(gguf_blocks, 2) || !q8h::aligned(qs, 16) || !q8h::aligned(d, 2)) return Q8_EALIGN;
    const int64_t nblocks = n * (k / kQK);
    if (nblocks == 0) return Q8_OK;
    q8h::launch_kernel(k_repack, dim3((unsigned)q8h::ceil_div(nblocks, 256)), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const uint16_t*>(gguf_blocks), nblocks, qs, d);
    return q8h::launch_status(Q8_LAUNCH_WEIGHTS_REPACK);
}

}  // extern "C"
