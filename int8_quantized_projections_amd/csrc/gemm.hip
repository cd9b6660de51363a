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
//    tiles per K block). Both operands and their scales go global -> LDS with
//    the direct copy, each copy instruction reading whole cache lines (8
//    lanes per 128-byte weight row): per-lane row-strided loads cost one L1
//    tag lookup per lane and made the vector-memory path the bottleneck.
#include "gemm_common.h"

using namespace q8;

namespace {

using namespace q8gemm;

constexpr int kPR = 2 * kKT;          // 16-byte pieces of a weight row per stage
constexpr int kRowB = kKT * 32;       // bytes of a weight row per stage
static_assert(kKT == 2 || kKT == 4, "stage of 2 or 4 blocks");

// The weight matrices of one launch: q8_gemm passes one, q8_gemm_shared_multi
// up to kMaxMembers that read the same activation plane. Their n-tiles are
// concatenated; member i owns tiles [tile0[i], tile0[i+1]).
constexpr int kMaxMembers = 8;
struct GemmMembers {
    const int8_t* wq[kMaxMembers];
    const uint16_t* wd[kMaxMembers];
    float* c[kMaxMembers];
    int64_t n[kMaxMembers];
    int64_t ldc[kMaxMembers];
    int tile0[kMaxMembers + 1];
    int m;
};

// a[i] for a wave-uniform i, as a chain of selects (a dynamic index into the
// by-value kernel argument would make the compiler copy it to scratch).
template <typename T>
__device__ __forceinline__ T pick(const T (&a)[kMaxMembers], int i) {
    T v = a[0];
#pragma unroll
    for (int j = 1; j < kMaxMembers; ++j) v = (i == j) ? a[j] : v;
    return v;
}

// Weight tile in LDS: 128 rows of kRowB bytes (kKT blocks); the 16-byte piece
// p (block p/2, half p%2) of tile row r sits at slot kPR*r + (p ^ wsw(r)). The
// copy reads each row's bytes with kPR consecutive lanes (whole cache-line
// runs), and the fragment read (32 consecutive rows, one piece) touches every
// bank group once per 8 or 16 lanes.
__device__ __forceinline__ int wsw(int r) {
    if constexpr (kPR == 8) return (r ^ (r >> 3)) & 7;
    return ((r >> 1) ^ (r >> 3)) & 3;
}

// DWL: the weight scales of a stage are copied into LDS with 4-byte copies of
// block pairs, which needs K/32 even (4-byte aligned pairs); otherwise every
// lane loads its own row's scales into registers one stage ahead.
// HV: 32-token halves of the plane group per workgroup. 2: the 64-token tile.
// 1: one half (two workgroups per 64-token tile), for grids with too few
// 64-token tiles to give every SIMD more than one wave; each output element is
// accumulated by the same instructions in the same order, so the bits are the
// same.
template <bool DWL, int HV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void k_gemm(
    const int8_t* __restrict__ aq, const uint32_t* __restrict__ asd, const GemmMembers M, int64_t T, int K, int nb,
    int n_tiles, int64_t tiles) {
    // Double-buffered stage: kKT chunks of one 64-token group of the A plane
    // (verbatim) with their scale words, and kKT blocks of the 128 weight rows
    // (swizzled as above) with their scales. Each buffer is a variable of its
    // own, so the compiler knows that the copies into one buffer and the reads
    // of the other do not alias. (With one array holding both buffers it made
    // the first read of every stage wait for all copies of the next stage, and
    // no copy overlapped the compute: 8% slower on 3325x3584x18944, 22% on
    // N=512.)
    static_assert(HV == 1 || HV == 2, "one or two 32-token halves");
    constexpr int kW = DWL ? kBN * kKT / 2 : 1;
    constexpr int kAB = HV * kTileBytes / 2;  // A bytes per block in LDS
    __shared__ __attribute__((aligned(16))) int8_t lds_a0[kKT * kAB], lds_a1[kKT * kAB];
    __shared__ __attribute__((aligned(16))) int8_t lds_b0[kBN * kKT * kQK], lds_b1[kBN * kKT * kQK];
    __shared__ __attribute__((aligned(16))) uint32_t lds_s0[kKT * kGroup], lds_s1[kKT * kGroup];
    __shared__ __attribute__((aligned(16))) uint32_t lds_w0[kW], lds_w1[kW];
    // buffer b of each (b is a compile-time constant at every use)
    auto lds_a = [&](int b) { return b ? lds_a1 : lds_a0; };
    auto lds_b = [&](int b) { return b ? lds_b1 : lds_b0; };
    auto lds_s = [&](int b) { return b ? lds_s1 : lds_s0; };
    auto lds_w = [&](int b) { return b ? lds_w1 : lds_w0; };
    static_assert(kKT * kGroup <= 256 && kBN * kKT / 2 <= 256, "one scale copy per wave at most");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int nt;
    int64_t g;
    tile_of(blockIdx.x, tiles, n_tiles, nt, g);
    int h0 = 0;  // HV == 1: the workgroup's half of plane group g
    if constexpr (HV == 1) {
        h0 = (int)(g & 1);
        g >>= 1;
    }
    // the member this tile belongs to (wave-uniform) and the tile inside it
    int mi = 0, tbase = 0;
#pragma unroll
    for (int i = 1; i < kMaxMembers; ++i) {
        if (i < M.m && nt >= M.tile0[i]) {
            mi = i;
            tbase = M.tile0[i];
        }
    }
    nt -= tbase;
    const int8_t* __restrict__ wq = pick(M.wq, mi);
    const uint16_t* __restrict__ wd = pick(M.wd, mi);
    float* __restrict__ C = pick(M.c, mi);
    const int64_t N = pick(M.n, mi);
    const int64_t ldc = pick(M.ldc, mi);
    const int64_t n0 = (int64_t)nt * kBN;
    const int brow = wave * 32 + (lane & 31);  // this lane's weight row in the tile
    const int64_t nrow = n0 + brow;            // and its output column
    const bool nvalid = nrow < N;
    const int khalf = lane >> 5;

    // Output register r of lane l covers tile row 8(r/4) + 4(l/32) + r%4; the
    // lane that feeds register r's broadcast in row-group q is 16q + r.
    const int rr = lane & 15, qq = lane >> 4;
    const int srow = 8 * (rr >> 2) + 4 * (qq >> 1) + (rr & 3);
    // LDS byte offsets of this lane's A fragments (token 32h + lane%32, half khalf)
    // and of its B fragment of block 0 (the XOR with wsw is linear in the block,
    // so block kb is at boff ^ (32 * kb)).
    int aoff[HV];
#pragma unroll
    for (int h = 0; h < HV; ++h) {
        const int i = 32 * h + (lane & 31);  // token in the LDS copy (HV == 1: in the half)
        aoff[h] = i * 32 + (((khalf ^ (i >> 2) ^ (i >> 3)) & 1) * 16);
    }
    const int boff = brow * kRowB + 16 * (khalf ^ wsw(brow));

    v16i bias;
#pragma unroll
    for (int i = 0; i < 16; ++i) bias[i] = kBias;
    // Opaque to the optimiser: held in 16 VGPRs for the whole kernel instead of
    // being re-created from scalar registers before the MFMAs of every stage.
    asm volatile("" : "+v"(bias));
    float acc[HV][16];
#pragma unroll
    for (int h = 0; h < HV; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[h][i] = 0.0f;

    const int8_t* plane = aq + g * (int64_t)nb * kTileBytes;
    const uint32_t* splane = asd + g * (int64_t)nb * kGroup;
    const int nst = (nb + kKT - 1) / kKT;

    // Issue the copies of stage st into LDS buffer b. Every copy instruction
    // fills one contiguous piece of LDS (1 KB, or 256 B). Each source is a
    // buffer resource over this workgroup's part of an operand; in a full stage
    // the byte offset is a per-lane offset fixed for the whole kernel plus a
    // wave-uniform stage offset, so the copies cost no vector ALU work. A tail
    // stage clamps every lane's block index to a valid block instead (those
    // blocks are never used).
    const __amdgpu_buffer_rsrc_t r_a = make_rsrc(plane, (int64_t)nb * kTileBytes);
    const __amdgpu_buffer_rsrc_t r_s = make_rsrc(splane, (int64_t)nb * kGroup * 4);
    const __amdgpu_buffer_rsrc_t r_b = make_rsrc(wq + n0 * (int64_t)K, (N - n0) * (int64_t)K);
    const __amdgpu_buffer_rsrc_t r_w = make_rsrc(wd + n0 * (int64_t)nb, (N - n0) * (int64_t)nb * 2);
    // HV == 2: copy `it` of wave w fills LDS bytes 4096 it + 1024 w .. of the stage (blocks 2it and
    // 2it + 1); HV == 1: wave w copies half h0 of block w
    const uint32_t aoffs = (uint32_t)(HV == 2 ? wave * 1024 + lane * 16 : wave * kTileBytes + h0 * 1024 + lane * 16);
    const uint32_t soffs = (uint32_t)(wave * kGroup + lane) * 4;
    // weights: wave w copies tile rows 32w .. 32w+31, 64/kPR rows per instruction
    auto brow_of = [&](int it) { return 32 * wave + (64 / kPR) * it + lane / kPR; };
    auto piece_of = [&](int it) { return (lane % kPR) ^ wsw(brow_of(it)); };  // block p/2, half p%2
    uint32_t boffs[kKT];  // this lane's copy `it`: byte offset from the tile's first row, block 0
#pragma unroll
    for (int it = 0; it < kKT; ++it)
        boffs[it] = (uint32_t)((min(n0 + brow_of(it), N - 1) - n0) * (int64_t)K) + (uint32_t)(piece_of(it) * 16);
    // weight scales: copy instruction w (w < kKT) takes rows (128/kKT)w .., kKT/2 block pairs per row
    constexpr int kPairs = kKT / 2;
    const int wpair = lane % kPairs;
    const uint32_t woffs =
        (uint32_t)((min(n0 + (128 / kKT) * wave + lane / kPairs, N - 1) - n0) * nb + 2 * wpair) * 2;
    auto stage_copy = [&](int st, int b) {
        const int c0 = st * kKT;
        if (c0 + kKT <= nb) {
#pragma unroll
            for (int it = 0; it < kKT * kAB / 16 / 256; ++it)
                lds_copy16(r_a, aoffs, (uint32_t)(c0 * kTileBytes + it * 4096), &lds_a(b)[it * 4096 + wave * 1024]);
            if (wave < kKT) lds_copy4(r_s, soffs, (uint32_t)(c0 * kGroup * 4), &lds_s(b)[wave * kGroup]);
#pragma unroll
            for (int it = 0; it < kKT; ++it)
                lds_copy16(r_b, boffs[it], (uint32_t)(c0 * kQK), &lds_b(b)[(wave * kKT + it) * 1024]);
            if constexpr (DWL)
                if (wave < kKT) lds_copy4(r_w, woffs, (uint32_t)(c0 * 2), &lds_w(b)[wave * 64]);
        } else {
#pragma unroll
            for (int it = 0; it < kKT * kAB / 16 / 256; ++it) {
                if constexpr (HV == 2) {
                    const int c = min(c0 + 2 * it + wave / 2, nb - 1);  // chunk of this wave's piece
                    lds_copy16(r_a, (uint32_t)(c * kTileBytes + (wave & 1) * 1024 + lane * 16), 0u,
                               &lds_a(b)[it * 4096 + wave * 1024]);
                } else {
                    const int c = min(c0 + wave, nb - 1);
                    lds_copy16(r_a, (uint32_t)(c * kTileBytes + h0 * 1024 + lane * 16), 0u, &lds_a(b)[wave * 1024]);
                }
            }
            if (wave < kKT)
                lds_copy4(r_s, (uint32_t)((min(c0 + wave, nb - 1) * kGroup + lane) * 4), 0u, &lds_s(b)[wave * kGroup]);
#pragma unroll
            for (int it = 0; it < kKT; ++it) {
                const int p = piece_of(it);
                const int c = min(c0 + (p >> 1), nb - 1);
                lds_copy16(r_b, boffs[it] + (uint32_t)((c - (p >> 1)) * kQK), 0u,
                           &lds_b(b)[(wave * kKT + it) * 1024]);
            }
            if constexpr (DWL) {
                if (wave < kKT) {
                    const int c = min(c0 + 2 * wpair, nb - 2);
                    lds_copy4(r_w, woffs + (uint32_t)((c - 2 * wpair) * 2), 0u, &lds_w(b)[wave * 64]);
                }
            }
        }
    };
    const _Float16* drow = reinterpret_cast<const _Float16*>(wd) + (nvalid ? nrow : 0) * (int64_t)nb;
    auto load_dw = [&](int st, h2 (&db)[kKT / 2]) {  // the register form (!DWL)
#pragma unroll
        for (int i = 0; i < kKT / 2; ++i) {
            h2 v;
            v.x = drow[min(st * kKT + 2 * i, nb - 1)];
            v.y = drow[min(st * kKT + 2 * i + 1, nb - 1)];
            db[i] = v;
        }
    };

    // Compute stage st from LDS buffer `buf` and weight scales db (two f16 per
    // register: block 2i in the low half, 2i+1 in the high half). A tail stage
    // runs the same straight-line code: its blocks past K hold copies of the
    // last block and get a weight scale of 0, which adds an exact zero.
    auto compute = [&](int st, int buf, h2 (&db)[kKT / 2]) {
        const int kc = nb - st * kKT;  // blocks of this stage inside K (>= 1)
        if (kc < kKT) {  // tail stage (wave-uniform): zero the scales of the blocks past K
#pragma unroll
            for (int kb = 1; kb < kKT; ++kb) {
                if (kb >= kc) {
                    if (kb & 1)
                        db[kb / 2].y = (_Float16)0.0f;
                    else
                        db[kb / 2].x = (_Float16)0.0f;
                }
            }
        }
        const int8_t* la = &lds_a(buf)[0];
        const int8_t* lb = &lds_b(buf)[0];
        const uint32_t* ls = &lds_s(buf)[0];
        auto frags = [&](int kb, v4i (&af)[HV], v4i& bf, uint32_t (&sc)[HV]) {
#pragma unroll
            for (int h = 0; h < HV; ++h) {
                af[h] = *reinterpret_cast<const v4i*>(la + kb * kAB + aoff[h]);
                sc[h] = ls[kb * kGroup + 32 * (HV == 2 ? h : h0) + srow];
            }
            bf = *reinterpret_cast<const v4i*>(lb + (boff ^ (32 * kb)));
        };
        // Pipeline over the HV*kKT (block, half) tiles: the MFMA of the next tile
        // is issued before the epilogue of the current one, and the fragments of
        // block kb+1 are read from LDS while block kb is being finished.
        v4i af[HV], an[HV], bf, bn;
        uint32_t sc[HV], sn[HV];
        frags(0, af, bf, sc);
        v16i d = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[0], bf, bias, 0, 0, 0);
#pragma unroll
        for (int kb = 0; kb < kKT; ++kb) {
            // (lanes of rows past N compute with row N-1's data and store nothing)
            float dw = (float)((kb & 1) ? db[kb / 2].y : db[kb / 2].x);
            // Opaque after the conversion, so the 32 FMAs below stay plain v_fma_f32:
            // folding the f16 operand into v_fma_mix_f32 makes each of them about
            // 1.5x as expensive on gfx950.
            asm volatile("" : "+v"(dw));
            const float nbias = -kBiasF * dw;
            if (kb + 1 < kKT) frags(kb + 1, an, bn, sn);
            if constexpr (HV == 2) {
                // tile (kb, 0) is in d; start (kb, 1)
                const v16i d0 = d;
                d = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[1], bf, bias, 0, 0, 0);
                epilogue(acc[0], __builtin_bit_cast(v16f, d0), dw, nbias, f16_value(sc[0]));
                // tile (kb, 1) is in d; start (kb + 1, 0)
                const v16i d1 = d;
                if (kb + 1 < kKT) d = __builtin_amdgcn_mfma_i32_32x32x32_i8(an[0], bn, bias, 0, 0, 0);
                epilogue(acc[1], __builtin_bit_cast(v16f, d1), dw, nbias, f16_value(sc[1]));
            } else {
                // block kb is in d; start kb + 1
                const v16i d0 = d;
                if (kb + 1 < kKT) d = __builtin_amdgcn_mfma_i32_32x32x32_i8(an[0], bn, bias, 0, 0, 0);
                epilogue(acc[0], __builtin_bit_cast(v16f, d0), dw, nbias, f16_value(sc[0]));
            }
#pragma unroll
            for (int h = 0; h < HV; ++h) {
                af[h] = an[h];
                sc[h] = sn[h];
            }
            bf = bn;
        }
    };
    auto lds_dw = [&](int buf, h2 (&db)[kKT / 2]) {
        if constexpr (kKT == 4) {
            const uint2 v = *reinterpret_cast<const uint2*>(&lds_w(buf)[brow * 2]);
            db[0] = __builtin_bit_cast(h2, v.x);
            db[1] = __builtin_bit_cast(h2, v.y);
        } else {
            db[0] = __builtin_bit_cast(h2, lds_w(buf)[brow]);
        }
    };

    // Each wave waits for its own copies (vmcnt) before the barrier that
    // publishes the stage to the other waves.
    h2 d0[kKT / 2], d1[kKT / 2];
    stage_copy(0, 0);
    if constexpr (!DWL) load_dw(0, d0);
    wait_copies();
    __syncthreads();
    for (int st = 0; st < nst; st += 2) {
        if (st + 1 < nst) {
            stage_copy(st + 1, 1);
            if constexpr (!DWL) load_dw(st + 1, d1);
        }
        if constexpr (DWL) lds_dw(0, d0);
        compute(st, 0, d0);
        wait_copies();
        __syncthreads();
        if (st + 1 < nst) {
            if (st + 2 < nst) {
                stage_copy(st + 2, 0);
                if constexpr (!DWL) load_dw(st + 2, d0);
            }
            if constexpr (DWL) lds_dw(1, d1);
            compute(st + 1, 1, d1);
            wait_copies();
            __syncthreads();
        }
    }

    if (nvalid) {
#pragma unroll
        for (int h = 0; h < HV; ++h) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t t = g * kGroup + 32 * (HV == 2 ? h : h0) + 8 * (r >> 2) + 4 * khalf + (r & 3);
                if (t < T) C[t * ldc + nrow] = acc[h][r];
            }
        }
    }
}

}  // namespace

namespace {

// A launch takes 32-token halves when every half-tile workgroup then has a CU
// of its own (2 x 64-token tiles <= the 256 CUs). Measured, bit-identical:
// 16 tiles (100x1024x4096) 32.1 -> 24.2 us, 32 tiles (512x512x3584) 28.9 ->
// 21.9 us; 208 tiles (3325x512x3584) 31.8 -> 30.9 us, 224 (512x3584x3584)
// 32.8 -> 33.0 us, and 448 or more tiles 10-17% slower, where the halves share
// CUs and each CU pulls more bytes per output.
constexpr int64_t kHalfTileMax = 128;

// Validation shared by q8_gemm and q8_gemm_shared_multi (the activation side is
// checked by the caller).
int check_member(const q8_weights* W, int64_t ldc, const float* c) {
    if (W == nullptr || W->format != Q8_WEIGHTS_Q8_0) return Q8_EINVAL;
    // K <= 2^24 keeps every in-tile byte offset of the weight copies in 32 bits.
    if (W->n < 0 || W->k <= 0 || (W->k % kQK) != 0 || W->k > ((int64_t)1 << 24)) return Q8_ESHAPE;
    if (ldc < W->n) return Q8_ESHAPE;
    if (W->n == 0) return Q8_OK;
    if (W->qs == nullptr || W->d == nullptr || c == nullptr) return Q8_EINVAL;
    if (!q8h::aligned(W->qs, 16) || !q8h::aligned(W->d, 2) || !q8h::aligned(c, 4)) return Q8_EALIGN;
    return Q8_OK;
}

int launch_gemm(int counter, int m, const q8_weights* const* W, const int8_t* a_qs, const uint32_t* a_sd, int64_t t,
                float* const* c, const int64_t* ldc, hipStream_t stream) {
    if (m < 1 || m > kMaxMembers || W == nullptr || c == nullptr || ldc == nullptr) return Q8_EINVAL;
    if (t < 0) return Q8_ESHAPE;
    int rc;
    for (int i = 0; i < m; ++i) {
        if ((rc = check_member(W[i], ldc[i], c[i]))) return rc;
        if (W[i]->k != W[0]->k) return Q8_ESHAPE;
    }
    if (a_qs == nullptr || a_sd == nullptr) return Q8_EINVAL;
    if (!q8h::aligned(a_qs, 16) || !q8h::aligned(a_sd, 4)) return Q8_EALIGN;
    if (t == 0) return Q8_OK;
    GemmMembers M = {};
    const int nb = (int)(W[0]->k / kQK);
    bool pairs = nb % 2 == 0;  // 4-byte scale pairs in LDS for every member, else the register form
    int64_t n_tiles = 0;
    M.m = 0;
    for (int i = 0; i < m; ++i) {
        if (W[i]->n == 0) continue;  // nothing to compute or write
        const int j = M.m++;
        M.wq[j] = W[i]->qs;
        M.wd[j] = W[i]->d;
        M.c[j] = c[i];
        M.n[j] = W[i]->n;
        M.ldc[j] = ldc[i];
        M.tile0[j] = (int)n_tiles;
        n_tiles += q8h::ceil_div(W[i]->n, kBN);
        pairs = pairs && q8h::aligned(W[i]->d, 4);
        if (n_tiles > INT32_MAX) return Q8_ESHAPE;
    }
    if (M.m == 0) return Q8_OK;
    M.tile0[M.m] = (int)n_tiles;
    for (int j = M.m; j < kMaxMembers; ++j) {  // unused slots repeat the last member (never selected)
        M.wq[j] = M.wq[M.m - 1];
        M.wd[j] = M.wd[M.m - 1];
        M.c[j] = M.c[M.m - 1];
        M.n[j] = M.n[M.m - 1];
        M.ldc[j] = M.ldc[M.m - 1];
        M.tile0[j + 1] = (int)n_tiles;
    }
    // A grid of few 64-token tiles leaves most CUs idle: then each workgroup
    // takes one 32-token half of a tile (the same per-element arithmetic and
    // bits, twice the workgroups).
    const bool half = n_tiles * q8h::ceil_div(t, kGroup) <= kHalfTileMax;
    const int64_t tiles = n_tiles * q8h::ceil_div(t, half ? kGroup / 2 : kGroup);
    if (tiles > INT32_MAX) return Q8_ESHAPE;
    auto go = [&](auto kernel) {
        q8h::launch_kernel(kernel, dim3((unsigned)tiles), dim3(256), 0, stream, a_qs, a_sd, M, t, (int)W[0]->k, nb,
                           (int)n_tiles, tiles);
    };
    if (pairs)
        half ? go(k_gemm<true, 1>) : go(k_gemm<true, 2>);
    else
        half ? go(k_gemm<false, 1>) : go(k_gemm<false, 2>);
    return q8h::launch_status(counter);
}

}  // namespace

// The q4_K GEMM (gemm_q4k.hip), counted under the given entry point.
int launch_q4k_gemm(int counter, const q4k_weights* W, const int8_t* a_qs, const uint32_t* a_sd, int64_t t,
                    float* c, int64_t ldc, hipStream_t stream);

extern "C" int q8_gemm(const q8_weights* W, const int8_t* a_qs, const uint32_t* a_sd, int64_t t, float* c,
                       int64_t ldc, void* stream) {
    if (W != nullptr && W->format == Q8_WEIGHTS_Q4_K) {
        const q4k_weights w4 = {W->n, W->k, reinterpret_cast<const uint8_t*>(W->qs)};
        return launch_q4k_gemm(Q8_LAUNCH_GEMM, &w4, a_qs, a_sd, t, c, ldc, (hipStream_t)stream);
    }
    return launch_gemm(Q8_LAUNCH_GEMM, 1, &W, a_qs, a_sd, t, &c, &ldc, (hipStream_t)stream);
}

extern "C" int q8_gemm_shared_multi(int m, const q8_weights* const* W, const int8_t* a_qs, const uint32_t* a_sd,
                                    int64_t t, float* const* c, const int64_t* ldc, void* stream) {
    return launch_gemm(Q8_LAUNCH_GEMM_SHARED_MULTI, m, W, a_qs, a_sd, t, c, ldc, (hipStream_t)stream);
}
