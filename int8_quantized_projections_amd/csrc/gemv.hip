// Batch-1 Q8_0 GEMV on gfx950: q8_gemv and q8_gemv_shared_multi.
//
// Sources: [P1] "Fusion and the Activation-Quantization Discipline" s2.1
// (wide loads instead of per-byte loads of a 34-byte block), s2.2 (integer
// dot product instructions), s2.3 (several rows per unit of work reuse the
// activation, dispatched by an N threshold), s2.4 (width sized to K), s2.5
// and s6 (one activation feeding several projections in one launch), s8
// (bit identity across variants).
//
// Design for gfx950:
//  - Weights are split planes (qs [N][K] int8, d [N][K/32] f16), repacked
//    once at load, so every weight byte is streamed with 16-byte loads.
//  - W lanes work on one row (W = K/32 rounded up to a power of two, at most
//    64); lane u of a row handles blocks u, u+W, u+2W, ... in that order.
//    The quantized activation slice a lane needs stays in its VGPRs for the
//    whole kernel: waves are persistent and loop over row groups, so the
//    activation is read once per wave rather than once per row.
//  - Integer block sums use v_dot4_i32_i8 (8 per block); each block adds
//    (float)isum * (dw * da) into a per-lane f32 sum with one FMA.
//  - Per row: per-lane sums in block order, then a fixed butterfly over the
//    W lanes. The order depends on K only, so 1, 2 or 4 rows per wave and the
//    grouped launch give bit-identical outputs ([P1] s8 invariant).
#include "gemm_common.h"
#include "q8_common.h"
#include "rmsnorm_row.h"

#include <type_traits>

using namespace q8;

namespace {

constexpr int kMaxMats = 8;
constexpr int kWavesPerWg = 4;
constexpr int kMaxWaves = 256 * 16;  // persistent grid cap: 256 CUs x 16 resident waves
constexpr int64_t kMaxF32K = 8192;    // q8_gemv_f32: the activation fits one chunk (64 lanes x 4 blocks)

struct GemvArgs {
    const int8_t* wq[kMaxMats];
    const uint16_t* wd[kMaxMats];
    float* y[kMaxMats];
    int64_t off[kMaxMats];  // first global row of matrix i; INT64_MAX when unused
    int64_t total;          // total rows of all matrices
    const int8_t* safe_q;   // row 0 of a non-empty matrix: the address rows past `total` load from
    const uint16_t* safe_d;
};

// Row-wise all-reduce inside aligned groups of W lanes (W a power of two).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (W >= 2) v += dpp_f<kDppQuadXor1>(v);
    if constexpr (W >= 4) v += dpp_f<kDppQuadXor2>(v);
    if constexpr (W >= 8) v += dpp_f<kDppRowHalfMirror>(v);
    if constexpr (W >= 16) v += dpp_f<kDppRowMirror>(v);
    if constexpr (W >= 32) v = add_xor16(v);
    if constexpr (W >= 64) v = add_xor32(v);
    return v;
}

__device__ __forceinline__ int dot32(const uint4& w0, const uint4& w1, const uint4& a0, const uint4& a1) {
    int s = 0;
    s = __builtin_amdgcn_sdot4((int)w0.x, (int)a0.x, s, false);
    s = __builtin_amdgcn_sdot4((int)w0.y, (int)a0.y, s, false);
    s = __builtin_amdgcn_sdot4((int)w0.z, (int)a0.z, s, false);
    s = __builtin_amdgcn_sdot4((int)w0.w, (int)a0.w, s, false);
    s = __builtin_amdgcn_sdot4((int)w1.x, (int)a1.x, s, false);
    s = __builtin_amdgcn_sdot4((int)w1.y, (int)a1.y, s, false);
    s = __builtin_amdgcn_sdot4((int)w1.z, (int)a1.z, s, false);
    s = __builtin_amdgcn_sdot4((int)w1.w, (int)a1.w, s, false);
    return s;
}

// W: lanes per row. NBL: blocks per lane held in registers per K chunk
// (a chunk is W*NBL blocks; K wider than one chunk reloads the activation
// chunk per row group). R: rows per lane group per iteration. MULTI: rows
// are the concatenation of several matrices (the grouped launch); the
// per-row arithmetic is the same code either way. F32A: the activation is
// f32 (ax) and each lane quantizes the blocks it holds (one chunk only).
// The GEMV of one wave: wave `wave_id` of `nwaves` takes row groups wave_id,
// wave_id + nwaves, ...
// PREF: pre_q, pre_d (LDS) hold the wave's first row group, already copied
// there (one row, R == 1, W == 64, KSEQ == 1): for block column j, its two
// 16-byte halves at pre_q + 2048j (+1024) + 16*lane, and its f16 scales at
// pre_d, block b at byte 2b. The arithmetic is the same as from memory.
template <int W, int NBL, int R, bool MULTI, bool F32A, int KSEQ = 1, bool PREF = false>
__device__ __forceinline__ void gemv_run(const GemvArgs& args, const int8_t* __restrict__ aq,
                                         const uint32_t* __restrict__ asd, const float* __restrict__ ax, int K,
                                         int nb, int64_t groups, int64_t wave_id, int64_t nwaves,
                                         const int8_t* pre_q = nullptr, const uint16_t* pre_d = nullptr) {
    static_assert(!PREF || (R == 1 && W == kWave && KSEQ == 1 && !F32A), "first row from LDS: one row, 64 lanes");
    constexpr int G = kWave / W;  // row slots per wave
    constexpr int CH = W * NBL;   // blocks per chunk
    constexpr int kSeq = KSEQ < NBL ? KSEQ : NBL;  // block columns per load step
    const int lane = threadIdx.x & (kWave - 1);
    const int slot = lane / W, u = lane % W;
    const int nchunks = (nb + CH - 1) / CH;

    // Every load below is unconditional from a clamped, always-valid address and the
    // out-of-range contributions are zeroed afterwards: a load inside a divergent branch
    // makes the compiler wait for it before the join, which serialises the stream.
    uint4 a0[NBL], a1[NBL];
    float da[NBL];
    auto load_act = [&](int ch) {
#pragma unroll
        for (int j = 0; j < NBL; ++j) {
            const int b = ch * CH + u + j * W;
            const int bc = b < nb ? b : nb - 1;
            a0[j] = *reinterpret_cast<const uint4*>(aq + (int64_t)bc * kQK);
            a1[j] = *reinterpret_cast<const uint4*>(aq + (int64_t)bc * kQK + 16);
            da[j] = f16_value(asd[bc]);
        }
    };
    // F32A (one chunk, K <= 8192): the f32 blocks are loaded before the first row
    // group's weights and quantized after those weight loads are issued, so the
    // two cold accesses overlap.
    float4 xv[F32A ? NBL : 1][8];
    if constexpr (F32A) {
#pragma unroll
        for (int j = 0; j < NBL; ++j) {
            const int b = u + j * W;
            const int bc = b < nb ? b : nb - 1;
#pragma unroll
            for (int i = 0; i < 8; ++i) xv[j][i] = *reinterpret_cast<const float4*>(ax + (int64_t)bc * kQK + 4 * i);
        }
    } else if (nchunks == 1) {
        load_act(0);
    }

    // One row group; `first` (a compile-time flag) marks the wave's first group.
    auto body = [&](int64_t gi, auto first) {
        const int8_t* wrow[R];
        const uint16_t* drow[R];
        float* yout[R];
        bool valid[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = gi * (G * R) + r * G + slot;
            valid[r] = row < args.total;
            const int8_t* q = args.wq[0];
            const uint16_t* d = args.wd[0];
            float* yy = args.y[0];
            int64_t o = 0;
            if constexpr (MULTI) {  // the member matrix this row belongs to (rows are concatenated)
#pragma unroll
                for (int i = 1; i < kMaxMats; ++i) {
                    const bool in = row >= args.off[i];
                    q = in ? args.wq[i] : q;
                    d = in ? args.wd[i] : d;
                    yy = in ? args.y[i] : yy;
                    o = in ? args.off[i] : o;
                }
            }
            const int64_t local = valid[r] ? row - o : 0;
            wrow[r] = valid[r] ? q + local * K : args.safe_q;
            drow[r] = valid[r] ? d + local * nb : args.safe_d;
            yout[r] = yy + local;
        }
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.0f;

        const int nch = F32A ? 1 : nchunks;  // F32A: one chunk (a constant trip count keeps the order below)
        for (int ch = 0; ch < nch; ++ch) {
            if constexpr (!F32A)
                if (nchunks > 1) load_act(ch);
            bool inb[NBL];
#pragma unroll
            for (int j = 0; j < NBL; ++j) inb[j] = ch * CH + u + j * W < nb;
            // Block columns in steps of kSeq (one; two for short grids, see make_plan):
            // a step's loads are issued, then
            // consumed, before the next step's loads. Fewer bytes in flight per wave
            // measured faster: 4 -> 2 columns per step took the decode set from 5.24
            // to 5.5 TB/s, and 2 -> 1 the 152064x3584 GEMV from 100-100.5 to 97-98 us,
            // the decode pair from 33.1-33.5 to 31.6-31.8 us; the requests of all
            // waves then fall into fewer, denser address ranges. (A short grid, the
            // grouped x4 at 2.25 rows per wave, is the exception: 16.1 -> 17.6 us.)
            // The per-row order of the accumulation is unchanged (j ascending).
            // the first row group from the LDS copy made during the producer
            constexpr bool from_lds = PREF && decltype(first)::value;
            if constexpr (from_lds) q8gemm::wait_copies();  // this wave's own copies have landed
#pragma unroll
            for (int j0 = 0; j0 < NBL; j0 += kSeq) {
                uint4 w0[R][kSeq], w1[R][kSeq];
                uint16_t dw[R][kSeq];
#pragma unroll
                for (int r = 0; r < R; ++r) {
#pragma unroll
                    for (int jj = 0; jj < kSeq; ++jj) {
                        const int b = ch * CH + u + (j0 + jj) * W;
                        const int bc = b < nb ? b : nb - 1;
                        if constexpr (from_lds) {
                            w0[r][jj] = *reinterpret_cast<const uint4*>(pre_q + (j0 + jj) * 2048 + 16 * lane);
                            w1[r][jj] = *reinterpret_cast<const uint4*>(pre_q + (j0 + jj) * 2048 + 1024 + 16 * lane);
                            dw[r][jj] = pre_d[bc];
                        } else {
                            w0[r][jj] = *reinterpret_cast<const uint4*>(wrow[r] + (int64_t)bc * kQK);
                            w1[r][jj] = *reinterpret_cast<const uint4*>(wrow[r] + (int64_t)bc * kQK + 16);
                            dw[r][jj] = drow[r][bc];
                        }
                    }
                }
                if constexpr (F32A && decltype(first)::value) {
                    if (j0 == 0) {
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int j = 0; j < NBL; ++j) {
                            uint32_t dbits;
                            quantize_lane32(xv[j], a0[j], a1[j], dbits);
                            da[j] = f16_value(dbits);
                        }
                    }
                }
#pragma unroll
                for (int r = 0; r < R; ++r) {
#pragma unroll
                    for (int jj = 0; jj < kSeq; ++jj) {
                        const int j = j0 + jj;
                        const int isum = dot32(w0[r][jj], w1[r][jj], a0[j], a1[j]);
                        const float sc = inb[j] ? f16_value(dw[r][jj]) * da[j] : 0.0f;
                        acc[r] = fmaf((float)isum, sc, acc[r]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float v = group_sum<W>(acc[r]);
            if (u == 0 && valid[r]) *yout[r] = v;
        }
    };
    if (wave_id < groups) body(wave_id, std::true_type{});
    for (int64_t gi = wave_id + nwaves; gi < groups; gi += nwaves) body(gi, std::false_type{});
}

// F32A (q8_gemv_f32, K <= kMaxF32K): the workgroup first quantizes the f32
// activation into LDS, each 32-value block by 8 lanes with q8_quantize's
// arithmetic (quantize_block8: the same bits), then runs the GEMV from there.
// Every wave quantizing the whole activation itself, 32 values per lane with the
// one-lane form, cost 0.76 us of 4.2 us on 2048x2048.
template <int W, int NBL, int R, bool MULTI, bool F32A = false, int KSEQ = 1>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs args, const int8_t* __restrict__ aq,
                                              const uint32_t* __restrict__ asd, const float* __restrict__ ax, int K,
                                              int nb, int64_t groups) {
    const int64_t wave_id = (int64_t)blockIdx.x * kWavesPerWg + (threadIdx.x >> 6);
    const int64_t nwaves = (int64_t)gridDim.x * kWavesPerWg;
    if constexpr (F32A) {
        __shared__ __attribute__((aligned(16))) int8_t act_q[kMaxF32K];
        __shared__ uint32_t act_sd[kMaxF32K / kQK];
        // float4 i of x is element 4(i % 8) of block i / 8: the 8 lanes of a block are
        // consecutive lanes of one wave, all active or all not (nb * 8 is a multiple of 8)
        const float4* __restrict__ x4 = reinterpret_cast<const float4*>(ax);
        for (int i = (int)threadIdx.x; i < nb * 8; i += kWavesPerWg * kWave) {
            const Quant8 r = quantize_block8(x4[i]);
            *reinterpret_cast<uint32_t*>(act_q + 4 * i) = r.qs4;
            if ((i & 7) == 0) act_sd[i >> 3] = r.sd;
        }
        __syncthreads();
        gemv_run<W, NBL, R, MULTI, false, KSEQ>(args, act_q, act_sd, nullptr, K, nb, groups, wave_id, nwaves);
    } else {
        gemv_run<W, NBL, R, MULTI, false, KSEQ>(args, aq, asd, ax, K, nb, groups, wave_id, nwaves);
    }
}

// Two independent GEMVs in one launch: workgroups [0, wgs2) run the f32-activation
// GEMV (a2, its activation x2 quantized in the launch, W2 lanes per row), the rest
// the grouped GEMV over the q8_0 activation (a1). Each part runs exactly the
// code of its own kernel, so the outputs are those of the two launches.
template <int W, int NBL, int R, int W2>
__global__ __launch_bounds__(256) void k_gemv_pair(GemvArgs a1, const int8_t* __restrict__ aq,
                                                   const uint32_t* __restrict__ asd, int K1, int nb1,
                                                   int64_t groups1, GemvArgs a2, const float* __restrict__ x2,
                                                   int K2, int nb2, int64_t groups2, int wgs2) {
    const int w = threadIdx.x >> 6;
    if ((int)blockIdx.x < wgs2)
        gemv_run<W2, 1, 1, false, true>(a2, nullptr, nullptr, x2, K2, nb2, groups2,
                                        (int64_t)blockIdx.x * kWavesPerWg + w, (int64_t)wgs2 * kWavesPerWg);
    else
        gemv_run<W, NBL, R, true, false>(a1, aq, asd, nullptr, K1, nb1, groups1,
                                         (int64_t)(blockIdx.x - wgs2) * kWavesPerWg + w,
                                         (int64_t)(gridDim.x - wgs2) * kWavesPerWg);
}

// The one-launch decode step: rmsnorm_quant of one row and the paired GEMVs of
// its consumers ([P1] s3: at decode a launch costs more than its bytes; [P2]
// s2: the producer's q8_0 output is what the consumers read). Workgroups
// [0, wgs2) run the f32-activation GEMV; every other workgroup first runs the
// producer itself, the same code with the same 16-wave layout as the
// standalone rmsnorm_quant of one row (so the same bits), into its own LDS,
// then runs the grouped GEMV from that copy. The first grouped workgroup also
// writes y and the q8_0 activation to memory.
//
// Per workgroup that is 56 KB of L2 reads (x and w at K=7168; HBM serves them
// once per XCD) and a few hundred instructions, with no dependency between
// workgroups. Measured alternatives, per decode step (two launches: 33.9 us;
// this form, then with 240 grouped workgroups: 32.8 us):
//  - one producer workgroup that the others wait for (a flag in memory, an
//    agent-scope release and acquire, one poller per workgroup): 35.5 us, as
//    every load issued behind the first rows' weight loads, the producer's and
//    the polls alike, waits for that queue;
//  - this form with the first weight loads issued before the producer's
//    arithmetic: 32.9 us with the x and w loads after them, 35.7 us with the
//    x and w loads first (then the registers spill); with each wave's first
//    row copied into LDS by direct buffer -> LDS loads during the producer:
//    33.1 us;
//  - (with loads in steps of one block column; this form with 240 grouped
//    workgroups: 32.5 us) all 256 workgroups on the grouped GEMV, the f32
//    GEMV's groups taken by the waves with one row fewer: 34.2 us after their
//    rows, 33.1 us before. The grouped workgroup count is chosen in
//    launch_step3 (the step's time follows the rows per wave).
constexpr int kStepWaves = 16;    // waves per workgroup of the decode step
constexpr int kMaxStepK = 8192;   // the grouped part's K: one chunk of 64 lanes x 4 blocks

//
// PRE: every grouped wave copies its first row (weights and scales) into LDS
// with direct buffer -> LDS copies issued right after the producer's x and w
// loads, so the weight stream starts while the producer computes (a fixed
// number of copies per wave: the producer then waits for its own loads only).
// Needs K/32 even and 4-byte aligned scale rows (4-byte scale copies).
template <int NV, int NBL, int R, int W2, bool PRE>
__global__ __launch_bounds__(kStepWaves * 64) void k_decode_step(
    const float* __restrict__ xn, const float* __restrict__ wn, float eps, float* __restrict__ yn,
    int8_t* __restrict__ aq_out, uint32_t* __restrict__ asd_out, GemvArgs a1, int K1, int nb1, int64_t groups1,
    GemvArgs a2, const float* __restrict__ x2, int K2, int nb2, int64_t groups2, int wgs2) {
    __shared__ __attribute__((aligned(16))) int8_t act_q[kMaxStepK];
    __shared__ uint32_t act_sd[kMaxStepK / kQK];
    __shared__ __attribute__((aligned(16))) int8_t pre_q[PRE ? kStepWaves * NBL * 2048 : 16];
    __shared__ __attribute__((aligned(16))) uint32_t pre_d[PRE ? kStepWaves * 128 : 4];
    __shared__ float part[kStepWaves], part2[kStepWaves];
    const int w = threadIdx.x >> 6;
    const int b = (int)blockIdx.x;
    if (b < wgs2) {
        gemv_run<W2, 1, 1, false, true>(a2, nullptr, nullptr, x2, K2, nb2, groups2, (int64_t)b * kStepWaves + w,
                                        (int64_t)wgs2 * kStepWaves);
        return;
    }
    const bool writer = b == wgs2;
    // wave-uniform (scalar registers): the first row's member lookup below is scalar selects
    const int64_t wave_id = (int64_t)(b - wgs2) * kStepWaves + __builtin_amdgcn_readfirstlane(w);
    // the producer's loads first (they return in order), then the first-row copies
    float4 xv[NV], wv[NV];
    rms_load_x<NV, kStepWaves>(xv, xn, 0, 1, K1);
    rms_load_w<NV, kStepWaves>(wv, wn, K1);
    if constexpr (PRE) {
        const int lane = threadIdx.x & 63;
        // this wave's first row (row group wave_id, one row per group), as gemv_run finds it
        const int64_t row = wave_id;
        const bool valid = row < a1.total;
        const int8_t* q = a1.wq[0];
        const uint16_t* d = a1.wd[0];
        int64_t o = 0;
#pragma unroll
        for (int i = 1; i < kMaxMats; ++i) {
            const bool in = row >= a1.off[i];
            q = in ? a1.wq[i] : q;
            d = in ? a1.wd[i] : d;
            o = in ? a1.off[i] : o;
        }
        const int8_t* wrow = valid ? q + (row - o) * K1 : a1.safe_q;
        const uint16_t* drow = valid ? d + (row - o) * nb1 : a1.safe_d;
        const __amdgpu_buffer_rsrc_t rq = q8gemm::make_rsrc(wrow, K1);
        const __amdgpu_buffer_rsrc_t rd = q8gemm::make_rsrc(drow, (int64_t)nb1 * 2);
        int8_t* mq = pre_q + w * (NBL * 2048);
#pragma unroll
        for (int j = 0; j < NBL; ++j) {
            const int bl = lane + 64 * j;
            const uint32_t off = (uint32_t)((bl < nb1 ? bl : nb1 - 1) * kQK);
            q8gemm::lds_copy16(rq, off, 0u, mq + j * 2048);
            q8gemm::lds_copy16(rq, off + 16u, 0u, mq + j * 2048 + 1024);
        }
        q8gemm::lds_copy4(rd, (uint32_t)(4 * lane), 0u, &pre_d[w * 128]);
        q8gemm::lds_copy4(rd, (uint32_t)(4 * lane + 256), 0u, &pre_d[w * 128 + 64]);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load and copy issued ahead of the math
    rms_finish<kDstRow, NV, kStepWaves, kStepWaves>(xv, wv, eps, writer ? yn : nullptr, 0, 1, 1, K1, nb1, act_q,
                                                    act_sd, part, part2);
    lds_barrier();  // the activation in LDS is complete; the first-row copies stay in flight
    if (writer) {
        for (int i = (int)threadIdx.x; i < K1 / 16; i += kStepWaves * 64)
            reinterpret_cast<uint4*>(aq_out)[i] = reinterpret_cast<const uint4*>(act_q)[i];
        for (int i = (int)threadIdx.x; i < nb1; i += kStepWaves * 64) asd_out[i] = act_sd[i];
    }
    gemv_run<64, NBL, R, true, false, 1, PRE>(a1, act_q, act_sd, nullptr, K1, nb1, groups1, wave_id,
                                      (int64_t)((int)gridDim.x - wgs2) * kStepWaves,
                                      PRE ? pre_q + w * (NBL * 2048) : nullptr,
                                      PRE ? reinterpret_cast<const uint16_t*>(&pre_d[w * 128]) : nullptr);
}

struct Plan {
    int lanes;         // W
    int nbl;           // blocks per lane per chunk
    int rows;          // R
    int64_t groups;    // row groups
    int64_t workgroups;
    int kseq;          // block columns per load step
};

int lanes_for(int nb) {
    int w = 1;
    while (w < nb && w < kWave) w <<= 1;
    return w;
}

// Persistent grids: the number of slots (waves, or workgroups of the decode
// step) for `groups` units of work over at most `cap` slots. The fewest slots
// that keep the minimal number of rounds (units per slot), so every slot takes
// the same number or one fewer, when that removes at most 15% of the slots.
// Decode set, grouped x6 (21,600 rows): 3,600 waves instead of 4,096, 32.2-32.7
// -> 31.6-32.0 us; the one-launch step, 225 workgroups instead of 240,
// 32.5 -> 31.8 us. Grouped x4 (9,216 rows) would drop to 3,072 waves (3 rows
// each): the same time (17.6-17.7 us), and the limit keeps 4,096. The LM head
// goes from 4,096 to 4,002 waves, unchanged in time.
int64_t balanced_slots(int64_t groups, int64_t cap) {
    if (groups <= cap) return groups;
    const int64_t rounds = q8h::ceil_div(groups, cap);
    const int64_t even = q8h::ceil_div(groups, rounds);
    return even * 20 >= cap * 17 ? even : cap;
}

Plan make_plan(int64_t total, int nb, int force_rows) {
    Plan p;
    p.lanes = lanes_for(nb);
    const int64_t per_lane = (nb + p.lanes - 1) / p.lanes;
    p.nbl = per_lane <= 1 ? 1 : per_lane <= 2 ? 2 : 4;
    const int64_t slots = q8h::ceil_div(total, kWave / p.lanes);
    // [P1] s2.3: several rows per wave share one load of the activation but
    // divide the grid. Here the activation stays in a wave's registers for the
    // whole launch when K fits one chunk (64 lanes x 4 blocks, K <= 8192); then
    // extra rows only add loads in flight. One row per wave measured best, or
    // within 3% of the best, at every shape of 30 MB or more from N=1024 to
    // 152064 (decode set: 29.9 vs 32.5 us); launches under 10 us vary by up to
    // 20% either way without a trend. Wider K
    // reloads the activation chunks per row group, and there the rows per wave
    // follow N: 1 below 2048 row slots, 2 below 16384, 4 from there on
    // (K=18944, N=65536: 5.30 / 5.72 / 5.91 TB/s for 1 / 2 / 4).
    const int64_t nchunks = q8h::ceil_div(nb, (int64_t)p.lanes * p.nbl);
    if (force_rows > 0)
        p.rows = force_rows;
    else if (nchunks == 1)
        p.rows = 1;
    else
        p.rows = slots >= 16384 ? 4 : slots >= 2048 ? 2 : 1;
    p.groups = q8h::ceil_div(slots, p.rows);
    const int64_t waves = p.groups < kMaxWaves ? p.groups : balanced_slots(p.groups, kMaxWaves);
    p.workgroups = q8h::ceil_div(waves, kWavesPerWg);
    // Loads in steps of one block column measured faster on every long grid;
    // a short one (two or three rounds, the last at most half full) measured
    // faster with two: the grouped x4 (9,216 rows over 4,096 waves) 17.5-17.7
    // -> 16.1-16.2 us, while 12,288 rows (three full rounds) prefer one. The
    // accumulation order is the same either way.
    const int64_t rounds = q8h::ceil_div(p.groups, waves > 0 ? waves : 1);
    const int64_t last = p.groups - (rounds - 1) * waves;
    p.kseq = (nchunks == 1 && p.nbl >= 2 && rounds >= 2 && rounds <= 3 && 2 * last <= waves) ? 2 : 1;
    return p;
}

template <int W, int NBL, bool MULTI, bool F32A>
void launch_r(const Plan& p, dim3 grid, hipStream_t s, const GemvArgs& a, const int8_t* aq, const uint32_t* asd,
              const float* ax, int K, int nb) {
    if (p.rows == 4)
        q8h::launch_kernel((k_gemv<W, NBL, 4, MULTI, F32A>), grid, dim3(256), 0, s, a, aq, asd, ax, K, nb, p.groups);
    else if (p.rows == 2)
        q8h::launch_kernel((k_gemv<W, NBL, 2, MULTI, F32A>), grid, dim3(256), 0, s, a, aq, asd, ax, K, nb, p.groups);
    else if constexpr (W == kWave && NBL >= 2 && !F32A) {
        if (p.kseq == 2)
            q8h::launch_kernel((k_gemv<W, NBL, 1, MULTI, F32A, 2>), grid, dim3(256), 0, s, a, aq, asd, ax, K, nb,
                               p.groups);
        else
            q8h::launch_kernel((k_gemv<W, NBL, 1, MULTI, F32A>), grid, dim3(256), 0, s, a, aq, asd, ax, K, nb,
                               p.groups);
    } else
        q8h::launch_kernel((k_gemv<W, NBL, 1, MULTI, F32A>), grid, dim3(256), 0, s, a, aq, asd, ax, K, nb, p.groups);
}

template <bool MULTI, bool F32A>
void launch_m(const Plan& p, hipStream_t s, const GemvArgs& a, const int8_t* aq, const uint32_t* asd, const float* ax,
              int K, int nb) {
    const dim3 grid((unsigned)p.workgroups);
    switch (p.lanes) {
        case 1: launch_r<1, 1, MULTI, F32A>(p, grid, s, a, aq, asd, ax, K, nb); break;
        case 2: launch_r<2, 1, MULTI, F32A>(p, grid, s, a, aq, asd, ax, K, nb); break;
        case 4: launch_r<4, 1, MULTI, F32A>(p, grid, s, a, aq, asd, ax, K, nb); break;
        case 8: launch_r<8, 1, MULTI, F32A>(p, grid, s, a, aq, asd, ax, K, nb); break;
        case 16: launch_r<16, 1, MULTI, F32A>(p, grid, s, a, aq, asd, ax, K, nb); break;
        case 32: launch_r<32, 1, MULTI, F32A>(p, grid, s, a, aq, asd, ax, K, nb); break;
        default:
            if (p.nbl == 1)
                launch_r<64, 1, MULTI, F32A>(p, grid, s, a, aq, asd, ax, K, nb);
            else if (p.nbl == 2)
                launch_r<64, 2, MULTI, F32A>(p, grid, s, a, aq, asd, ax, K, nb);
            else
                launch_r<64, 4, MULTI, F32A>(p, grid, s, a, aq, asd, ax, K, nb);
    }
}

void launch(const Plan& p, bool multi, hipStream_t s, const GemvArgs& a, const int8_t* aq, const uint32_t* asd, int K,
            int nb) {
    if (multi)
        launch_m<true, false>(p, s, a, aq, asd, nullptr, K, nb);
    else
        launch_m<false, false>(p, s, a, aq, asd, nullptr, K, nb);
}

int check_weights(const q8_weights* w) {
    if (w == nullptr || w->format != Q8_WEIGHTS_Q8_0) return Q8_EINVAL;
    if (w->n < 0 || w->k <= 0 || (w->k % kQK) != 0 || w->k > ((int64_t)1 << 30)) return Q8_ESHAPE;
    if (w->n > 0 && (w->qs == nullptr || w->d == nullptr)) return Q8_EINVAL;
    if (!q8h::aligned(w->qs, 16) || !q8h::aligned(w->d, 2)) return Q8_EALIGN;
    return Q8_OK;
}

}  // namespace

namespace {

// A validated GEMV launch: its arguments and plan; `empty` when there is
// nothing to compute.
struct GemvJob {
    GemvArgs a{};
    Plan p{};
    int K = 0, nb = 0;
    bool multi = false, empty = true;
};

// Validation and launch arguments of the grouped GEMV (q8_gemv, q8_gemv_shared_multi).
int prepare_multi(int m, const q8_weights* const* W, const int8_t* a_qs, const uint32_t* a_sd,
                         float* const* y, int rows_per_wave, GemvJob& j) {
    if (m < 1 || m > kMaxMats || W == nullptr || y == nullptr) return Q8_EINVAL;
    if (rows_per_wave != 0 && rows_per_wave != 1 && rows_per_wave != 2 && rows_per_wave != 4) return Q8_EINVAL;
    GemvArgs& a = j.a;
    int64_t total = 0;
    const int64_t K = W[0] ? W[0]->k : 0;
    for (int i = 0; i < m; ++i) {
        int rc = check_weights(W[i]);
        if (rc) return rc;
        if (W[i]->k != K) return Q8_ESHAPE;
        if (y[i] == nullptr && W[i]->n > 0) return Q8_EINVAL;
        if (!q8h::aligned(y[i], 4)) return Q8_EALIGN;
        a.wq[i] = W[i]->qs;
        a.wd[i] = W[i]->d;
        a.y[i] = y[i];
        a.off[i] = total;
        total += W[i]->n;
    }
    for (int i = m; i < kMaxMats; ++i) {
        a.wq[i] = nullptr;
        a.wd[i] = nullptr;
        a.y[i] = nullptr;
        a.off[i] = INT64_MAX;
    }
    a.total = total;
    a.safe_q = nullptr;
    a.safe_d = nullptr;
    for (int i = m - 1; i >= 0; --i) {
        if (W[i]->n > 0) {
            a.safe_q = W[i]->qs;
            a.safe_d = W[i]->d;
        }
    }
    if (a_qs == nullptr || a_sd == nullptr) return Q8_EINVAL;
    if (!q8h::aligned(a_qs, 16) || !q8h::aligned(a_sd, 4)) return Q8_EALIGN;
    j.empty = total == 0;
    if (j.empty) return Q8_OK;
    j.K = (int)K;
    j.nb = (int)(K / kQK);
    j.p = make_plan(total, j.nb, rows_per_wave);
    // one non-empty member: the plain kernel, reading member 0's pointers
    int nonempty = 0, first = 0;
    for (int i = m - 1; i >= 0; --i)
        if (W[i]->n > 0) {
            ++nonempty;
            first = i;
        }
    j.multi = nonempty > 1;
    if (!j.multi) {
        a.wq[0] = a.wq[first];
        a.wd[0] = a.wd[first];
        a.y[0] = a.y[first];
    }
    return Q8_OK;
}

// Validation and launch arguments of the f32-activation GEMV (q8_gemv_f32).
int prepare_f32(const q8_weights* W, const float* x, float* y, GemvJob& j) {
    int rc = check_weights(W);
    if (rc) return rc;
    if (W->k > kMaxF32K) return Q8_ESHAPE;
    if (x == nullptr || (y == nullptr && W->n > 0)) return Q8_EINVAL;
    if (!q8h::aligned(x, 16) || !q8h::aligned(y, 4)) return Q8_EALIGN;
    j.empty = W->n == 0;
    if (j.empty) return Q8_OK;
    GemvArgs& a = j.a;
    for (int i = 0; i < kMaxMats; ++i) {
        a.wq[i] = W->qs;
        a.wd[i] = W->d;
        a.y[i] = y;
        a.off[i] = i == 0 ? 0 : INT64_MAX;
    }
    a.total = W->n;
    a.safe_q = W->qs;
    a.safe_d = W->d;
    j.K = (int)W->k;
    j.nb = (int)(W->k / kQK);
    j.p = make_plan(W->n, j.nb, 0);
    return Q8_OK;
}

void launch_multi(const GemvJob& j, hipStream_t s, const int8_t* a_qs, const uint32_t* a_sd) {
    launch(j.p, j.multi, s, j.a, a_qs, a_sd, j.K, j.nb);
}

void launch_f32(const GemvJob& j, hipStream_t s, const float* x) {
    launch_m<false, true>(j.p, s, j.a, nullptr, nullptr, x, j.K, j.nb);
}

// The pair kernel is instantiated for the grouped part with 64 lanes per row,
// 2 or 4 blocks per lane (K in (2048, 8192]) and 1 or 2 rows per wave, and the
// f32 part with 4, 8 or 16 lanes per row and one block per lane (K in (64, 512]).
bool pair_supported(const Plan& p1, const Plan& p2) {
    return p1.lanes == 64 && (p1.nbl == 2 || p1.nbl == 4) && (p1.rows == 1 || p1.rows == 2) && p2.nbl == 1 &&
           p2.rows == 1 && (p2.lanes == 4 || p2.lanes == 8 || p2.lanes == 16);
}

template <int NBL, int R, int W2>
void launch_pair3(const GemvJob& j1, const GemvJob& j2, hipStream_t s, const int8_t* a_qs,
                         const uint32_t* a_sd, const float* x) {
    // the grouped part is persistent: give it the resident slots the f32 part leaves,
    // so that no workgroup of it starts late (a tail with few waves in flight)
    const int wgs2 = (int)j2.p.workgroups;
    const int64_t cap = kMaxWaves / kWavesPerWg - wgs2;
    const int64_t wgs1 = j1.p.workgroups < cap ? j1.p.workgroups : (cap > 0 ? cap : 1);
    const dim3 grid((unsigned)(wgs1 + wgs2));
    q8h::launch_kernel((k_gemv_pair<64, NBL, R, W2>), grid, dim3(256), 0, s, j1.a, a_qs, a_sd, j1.K, j1.nb,
                       j1.p.groups, j2.a, x, j2.K, j2.nb, j2.p.groups, wgs2);
}

template <int NBL, int R>
void launch_pair2(const GemvJob& j1, const GemvJob& j2, hipStream_t s, const int8_t* a_qs,
                         const uint32_t* a_sd, const float* x) {
    if (j2.p.lanes == 4)
        launch_pair3<NBL, R, 4>(j1, j2, s, a_qs, a_sd, x);
    else if (j2.p.lanes == 8)
        launch_pair3<NBL, R, 8>(j1, j2, s, a_qs, a_sd, x);
    else
        launch_pair3<NBL, R, 16>(j1, j2, s, a_qs, a_sd, x);
}

void launch_pair(const GemvJob& j1, const GemvJob& j2, hipStream_t s, const int8_t* a_qs,
                        const uint32_t* a_sd, const float* x) {
    if (j1.p.nbl == 4) {
        if (j1.p.rows == 2)
            launch_pair2<4, 2>(j1, j2, s, a_qs, a_sd, x);
        else
            launch_pair2<4, 1>(j1, j2, s, a_qs, a_sd, x);
    } else {
        if (j1.p.rows == 2)
            launch_pair2<2, 2>(j1, j2, s, a_qs, a_sd, x);
        else
            launch_pair2<2, 1>(j1, j2, s, a_qs, a_sd, x);
    }
}

// The decode step's producer holds the row in NV float4 per lane over 16
// waves, as rmsnorm_quant does for one row: 1 for K <= 4096, 2 for K <= 8192.
int step_nv(int K) {
    const int need = (int)q8h::ceil_div(K / 4, (int64_t)kStepWaves * kWave);
    return need <= 1 ? 1 : need <= 2 ? 2 : 0;
}

// The one-launch step serves the pair kernel's shapes with one row per wave
// (the grouped part's plan at one K chunk, K <= 8192), with or without the
// f32 part.
bool step_supported(const GemvJob& j1, const GemvJob& j2) {
    const Plan& p1 = j1.p;
    const Plan& p2 = j2.p;
    const bool grouped_ok = !j1.empty && p1.lanes == 64 && (p1.nbl == 2 || p1.nbl == 4) && p1.rows == 1 &&
                            j1.K <= kMaxStepK && step_nv(j1.K) > 0 && (step_nv(j1.K) == 1) == (p1.nbl == 2);
    const bool f32_ok = j2.empty || (p2.nbl == 1 && p2.rows == 1 && (p2.lanes == 4 || p2.lanes == 8 || p2.lanes == 16));
    return grouped_ok && f32_ok;
}

template <int NV, int NBL, int W2>
void launch_step3(const GemvJob& j1, const GemvJob& j2, hipStream_t s, const float* x, const float* w, float eps,
                  float* y, int8_t* a_qs, uint32_t* a_sd, const float* x2) {
    // The f32 part needs one wave per row group; the grouped part takes the
    // resident 16-wave slots that leaves, balanced (balanced_slots: decode set,
    // 225 workgroups, 6 rows per wave: 31.8-31.9 us against 32.5 us with 240,
    // 5 or 6 rows per wave, and 34.3 with 224, 7 rows for 96 waves), and the
    // f32 part takes the slots this frees.
    const int64_t slots = kMaxWaves / kStepWaves;
    const int64_t waves2 = j2.empty ? 0 : j2.p.groups < kMaxWaves ? j2.p.groups : kMaxWaves;
    int64_t wgs2 = q8h::ceil_div(waves2, (int64_t)kStepWaves);
    const int64_t cap = slots - wgs2 > 0 ? slots - wgs2 : 1;
    const int64_t want = q8h::ceil_div(j1.p.groups, (int64_t)kStepWaves);
    int64_t wgs1 = want;
    if (want > cap) {
        // in workgroups: rows per workgroup round = kStepWaves
        wgs1 = q8h::ceil_div(balanced_slots(j1.p.groups, cap * kStepWaves), (int64_t)kStepWaves);
        if (wgs2 > 0) wgs2 = slots - wgs1;
    }
    const dim3 grid((unsigned)(wgs2 + wgs1));
    // the first-row copies need 4-byte scale copies: K/32 even and 4-byte aligned scale planes
    bool pre = j1.nb % 2 == 0;
    for (int i = 0; i < kMaxMats; ++i)
        if (j1.a.wd[i] != nullptr && !q8h::aligned(j1.a.wd[i], 4)) pre = false;
    if (pre)
        q8h::launch_kernel((k_decode_step<NV, NBL, 1, W2, true>), grid, dim3(kStepWaves * 64), 0, s, x, w, eps, y,
                           a_qs, a_sd, j1.a, j1.K, j1.nb, j1.p.groups, j2.a, x2, j2.K, j2.nb, j2.p.groups, (int)wgs2);
    else
        q8h::launch_kernel((k_decode_step<NV, NBL, 1, W2, false>), grid, dim3(kStepWaves * 64), 0, s, x, w, eps, y,
                           a_qs, a_sd, j1.a, j1.K, j1.nb, j1.p.groups, j2.a, x2, j2.K, j2.nb, j2.p.groups, (int)wgs2);
}

template <int NV, int NBL>
void launch_step2(const GemvJob& j1, const GemvJob& j2, hipStream_t s, const float* x, const float* w, float eps,
                  float* y, int8_t* a_qs, uint32_t* a_sd, const float* x2) {
    if (j2.empty || j2.p.lanes == 4)  // no f32 part: any instance, with no workgroup for it
        launch_step3<NV, NBL, 4>(j1, j2, s, x, w, eps, y, a_qs, a_sd, x2);
    else if (j2.p.lanes == 8)
        launch_step3<NV, NBL, 8>(j1, j2, s, x, w, eps, y, a_qs, a_sd, x2);
    else
        launch_step3<NV, NBL, 16>(j1, j2, s, x, w, eps, y, a_qs, a_sd, x2);
}

}  // namespace

extern "C" {

int q8_gemv_plan(int64_t total_rows, int64_t k, int rows_per_wave, int* lanes_per_row, int* rows_per_wave_out,
                 int64_t* workgroups) {
    if (total_rows < 0 || k <= 0 || (k % kQK) != 0) return Q8_ESHAPE;
    if (rows_per_wave != 0 && rows_per_wave != 1 && rows_per_wave != 2 && rows_per_wave != 4) return Q8_EINVAL;
    const Plan p = make_plan(total_rows, (int)(k / kQK), rows_per_wave);
    if (lanes_per_row) *lanes_per_row = p.lanes;
    if (rows_per_wave_out) *rows_per_wave_out = p.rows;
    if (workgroups) *workgroups = total_rows == 0 ? 0 : p.workgroups;
    return Q8_OK;
}

// The grouped GEMV behind q8_gemv, q8_gemv_shared_multi and _ex; `counter`
// names the entry point whose launch counter a launch adds to.
static int gemv_multi(int counter, int m, const q8_weights* const* W, const int8_t* a_qs, const uint32_t* a_sd,
                      float* const* y, int rows_per_wave, void* stream) {
    GemvJob j;
    int rc = prepare_multi(m, W, a_qs, a_sd, y, rows_per_wave, j);
    if (rc || j.empty) return rc;
    launch_multi(j, (hipStream_t)stream, a_qs, a_sd);
    return q8h::launch_status(counter);
}

int q8_gemv_shared_multi_ex(int m, const q8_weights* const* W, const int8_t* a_qs, const uint32_t* a_sd,
                            float* const* y, int rows_per_wave, void* stream) {
    return gemv_multi(Q8_LAUNCH_GEMV_SHARED_MULTI, m, W, a_qs, a_sd, y, rows_per_wave, stream);
}

int q8_gemv_shared_multi(int m, const q8_weights* const* W, const int8_t* a_qs, const uint32_t* a_sd,
                         float* const* y, void* stream) {
    return q8_gemv_shared_multi_ex(m, W, a_qs, a_sd, y, 0, stream);
}

int q8_gemv_f32(const q8_weights* W, const float* x, float* y, void* stream) {
    GemvJob j;
    int rc = prepare_f32(W, x, y, j);
    if (rc || j.empty) return rc;
    launch_f32(j, (hipStream_t)stream, x);
    return q8h::launch_status(Q8_LAUNCH_GEMV_F32);
}

int q8_gemv_shared_multi_plus_f32(int m, const q8_weights* const* W, const int8_t* a_qs, const uint32_t* a_sd,
                                  float* const* y, const q8_weights* Wx, const float* x, float* yx, void* stream) {
    GemvJob j1, j2;
    int rc = prepare_multi(m, W, a_qs, a_sd, y, 0, j1);
    if (rc) return rc;
    if ((rc = prepare_f32(Wx, x, yx, j2))) return rc;
    const hipStream_t s = (hipStream_t)stream;
    constexpr int ctr = Q8_LAUNCH_GEMV_SHARED_MULTI_PLUS_F32;
    if (!j1.empty && !j2.empty && pair_supported(j1.p, j2.p)) {
        launch_pair(j1, j2, s, a_qs, a_sd, x);
        return q8h::launch_status(ctr);
    }
    // one part empty, or shapes without a pair kernel: the two kernels back to back
    if (!j1.empty) {
        launch_multi(j1, s, a_qs, a_sd);
        if ((rc = q8h::launch_status(ctr))) return rc;
    }
    if (!j2.empty) {
        launch_f32(j2, s, x);
        if ((rc = q8h::launch_status(ctr))) return rc;
    }
    return Q8_OK;
}

int rmsnorm_quant_gemv_shared_multi_plus_f32(const float* x, const float* w, float eps, float* y, int8_t* a_qs,
                                             uint32_t* a_sd, int m, const q8_weights* const* W, float* const* ys,
                                             const q8_weights* Wx, const float* x2, float* yx, void* stream) {
    GemvJob j1, j2;
    int rc = prepare_multi(m, W, a_qs, a_sd, ys, 0, j1);
    if (rc) return rc;
    if (Wx != nullptr && (rc = prepare_f32(Wx, x2, yx, j2))) return rc;  // Wx == NULL: no f32 part
    if (x == nullptr || w == nullptr) return Q8_EINVAL;
    if (!q8h::aligned(x, 16) || !q8h::aligned(w, 16) || !q8h::aligned(y, 16)) return Q8_EALIGN;
    const int64_t K = W[0]->k;
    const hipStream_t s = (hipStream_t)stream;
    // One workgroup writes y and the activation while the others still read x
    // and w, so the one launch needs those outputs apart from x and w (an
    // in-place y = x runs as the two calls, which allow it).
    auto overlap = [](const void* a, int64_t na, const void* b, int64_t nb_) {
        const char* pa = static_cast<const char*>(a);
        const char* pb = static_cast<const char*>(b);
        return a != nullptr && b != nullptr && pa < pb + nb_ && pb < pa + na;
    };
    const bool apart = !overlap(y, 4 * K, x, 4 * K) && !overlap(y, 4 * K, w, 4 * K) &&
                       !overlap(a_qs, K, x, 4 * K) && !overlap(a_qs, K, w, 4 * K) &&
                       !overlap(a_sd, K / 8, x, 4 * K) && !overlap(a_sd, K / 8, w, 4 * K);
    if (apart && step_supported(j1, j2)) {
        if (j1.p.nbl == 2)
            launch_step2<1, 2>(j1, j2, s, x, w, eps, y, a_qs, a_sd, x2);
        else
            launch_step2<2, 4>(j1, j2, s, x, w, eps, y, a_qs, a_sd, x2);
        return q8h::launch_status(Q8_LAUNCH_RMSNORM_GEMV_STEP);
    }
    // other shapes: the producer, then the pair (or its two kernels)
    if ((rc = rmsnorm_quant(x, w, eps, y, 1, K, Q8_LAYOUT_ROW, a_qs, a_sd, stream))) return rc;
    if (Wx == nullptr) return q8_gemv_shared_multi(m, W, a_qs, a_sd, ys, stream);
    return q8_gemv_shared_multi_plus_f32(m, W, a_qs, a_sd, ys, Wx, x2, yx, stream);
}

int q8_gemv(const q8_weights* W, const int8_t* a_qs, const uint32_t* a_sd, float* y, void* stream) {
    if (W == nullptr) return Q8_EINVAL;
    const q8_weights* ws[1] = {W};
    float* ys[1] = {y};
    return gemv_multi(Q8_LAUNCH_GEMV, 1, ws, a_qs, a_sd, ys, 0, stream);
}

}  // extern "C"
