// a3+a4+a5 — weight-only linears (W8A16 = the pages' "q8", W4A16 = "q4") at
// small M (M <= 64 tokens), where the layer is bound by streaming the packed
// weights from HBM (aria project page, "Results": the 4-bit weights are what
// put the 1.2 B model on an 8 GB device).
//   W8A16: y = epilogue(s_w[n] * sum_k x[m][k] * q[n][k])
//   W4A16: y = epilogue(sum_k x[m][k] * fp16(q4[n][k] * s_g[n][k/32]))
//   W16A16 (the unquantized fp16 rung): y = epilogue(sum_k x[m][k] * wt[n][k])
// M > 64 runs the tiled kernel (gemm_tiled.hip).
//
// Design (gfx950): a workgroup of 4 waves owns 16*CG output channels; each
// wave streams one quarter of K for all of them.  A lane reads 16-byte runs of
// one channel's packed row (16 k at 8 bits, 32 k at 4 bits) and decodes them
// straight into v_mfma_f32_16x16x32_f16 B operands (no LDS for the weights:
// no other wave reuses them); the activations (tiny, L2-resident) are read
// as A operands with the same k permutation, once per column group set.
// Each wave issues all loads of a group of NS K-steps (bounds-checked buffer
// loads: past K or M they read zero, so there are no branches) before it
// decodes any of them; the four partial tiles are summed in LDS in a fixed
// order, so results are deterministic.

#include "common.h"
#include "decode.h"
#include "kernels.h"

namespace aria {

// s_waitcnt immediate (gfx9 encoding): at most `vm` vector memory operations
// and no LDS operations outstanding.
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4); }

constexpr int kNS4 = 3;   // 4-bit weights: NS = 3 steps of 128 k per wave and chunk

// K is cut into chunks of 4 * NS wave-steps (4 waves x NS steps x KPW k =
// 1536 k at either width); in chunk c, wave w takes steps (4c + w) NS ..
// (4c + w) NS + NS - 1.  Every kernel below uses this same split and the
// same order, so they produce bit-identical sums.
template <int BITS, int MT, int CG, int NS>
struct SkinnyRegs {
    static constexpr int KPL = BITS == 8 ? 16 : BITS == 4 ? 32 : 8;  // k per lane per 16-byte weight load
    static constexpr int NQ = KPL / 8;               // 16x16x32 MFMAs fed by one load
    static constexpr int KPW = 4 * KPL;              // k per wave step (4 lane groups)
    static constexpr int KCH = 4 * NS * KPW;         // k per chunk
    v4i w[NS][CG];
    v4i x[NS][NQ][MT];
    u32 sc[NS][CG];  // group scale bits (4-bit weights)
};

// Issue every load of one wave's share of chunk kc for output channels
// [n0, n0 + 16 CG).  Loads past K, N or M use an out-of-range offset: they read
// zero and move no data, so there are no branches.
template <int BITS, int MT, int CG, int NS, bool SCALES = true>
__device__ __forceinline__ void skinny_load(SkinnyRegs<BITS, MT, CG, NS>& R, rsrc_t rx, rsrc_t rw, rsrc_t rs,
                                            int M, int N, int K, int n0, int kc, int wave, int lane) {
    using RG = SkinnyRegs<BITS, MT, CG, NS>;
    const uint32_t rowbytes = BITS == 8 ? (uint32_t)K : BITS == 4 ? (uint32_t)K / 2 : (uint32_t)K * 2;
    const int G = K / 32;
    const int gsel = lane / 16;  // which k-run of a step this lane reads
#pragma unroll
    for (int j = 0; j < NS; j++) {
        const int st = (kc * 4 + wave) * NS + j;
        const int kb = st * RG::KPW + gsel * RG::KPL;  // first k of this lane's run
        const bool in = kb < K;
#pragma unroll
        for (int g = 0; g < CG; g++) {
            const int col = n0 + 16 * g + lane % 16;
            const bool ok = in && col < N;
            R.w[j][g] = buf_load16(rw, ok ? (uint32_t)col * rowbytes + (uint32_t)(BITS == 8 ? kb : BITS == 4 ? kb / 2 : 2 * kb) : OOB);
            if (BITS == 4 && SCALES)
                R.sc[j][g] = __builtin_amdgcn_raw_buffer_load_b16(rs, (int)(ok ? ((uint32_t)col * G + kb / 32) * 2 : OOB), 0, 0);
        }
#pragma unroll
        for (int q = 0; q < RG::NQ; q++)
#pragma unroll
            for (int t = 0; t < MT; t++) {
                const int m = t * 16 + lane % 16;
                R.x[j][q][t] = buf_load16(rx, in && m < M ? ((uint32_t)m * K + kb + 8 * q) * 2 : OOB);
            }
    }
}

// Decode the weights in registers straight into B operands and accumulate.
template <int BITS, int MT, int CG, int NS>
__device__ __forceinline__ void skinny_compute(const SkinnyRegs<BITS, MT, CG, NS>& R, v4f (&acc)[MT][CG]) {
    using RG = SkinnyRegs<BITS, MT, CG, NS>;
#pragma unroll
    for (int j = 0; j < NS; j++)
#pragma unroll
        for (int g = 0; g < CG; g++) {
            v4i d[RG::NQ];
            if constexpr (BITS == 8) {
                dec8(R.w[j][g], d[0], d[1]);
            } else if constexpr (BITS == 4) {
                dec4_bits(R.w[j][g], R.sc[j][g], d);
            } else {
                d[0] = R.w[j][g];   // fp16 weights: the load is the operand
            }
            // MFMA q of this run: the lane's 8 k are kb + 8q .. kb + 8q + 7 for its row and column
#pragma unroll
            for (int q = 0; q < RG::NQ; q++)
#pragma unroll
                for (int t = 0; t < MT; t++)
                    acc[t][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, R.x[j][q][t]),
                                                                       __builtin_bit_cast(v8h, d[q]), acc[t][g], 0, 0, 0);
        }
}

// Sum the four waves' partial tiles in a fixed order and apply the epilogue.
// `part` is reused, so callers that come back for another tile must pass a
// barrier first (done here at the end).
template <int BITS, int MT, int CG, class E>
__device__ __forceinline__ void skinny_finish(float (&part)[4][MT * 16][16 * CG + 1], v4f (&acc)[MT][CG],
                                              const half_t* S, half_t* Y, int M, int N, const E& epi, int n0,
                                              int wave, int lane) {
    constexpr int NC = 16 * CG;
    // 16x16 block layout: register r of lane l holds row 4*(l/16) + r, column l%16
#pragma unroll
    for (int t = 0; t < MT; t++)
#pragma unroll
        for (int g = 0; g < CG; g++)
#pragma unroll
            for (int r = 0; r < 4; r++) part[wave][t * 16 + 4 * (lane / 16) + r][16 * g + lane % 16] = acc[t][g][r];
    __syncthreads();
    const float alpha = load_alpha(epi);
    for (int o = threadIdx.x; o < MT * 16 * NC; o += 256) {
        const int row = o / NC, cc = o % NC, col = n0 + cc;
        if (row >= M || col >= N) continue;
        float v = ((part[0][row][cc] + part[1][row][cc]) + part[2][row][cc]) + part[3][row][cc];
        if (BITS == 8) v *= (float)S[col];
        const int64_t idx = (int64_t)row * N + col;
        Y[idx] = (half_t)epilogue_apply(v, idx, col, epi, alpha);
    }
    __syncthreads();
}

// The chunk loop with the group scales of each chunk (16 CG rows x KCH / 32
// groups, contiguous per row) fetched once per workgroup by LDS-DMA, 16 bytes
// per lane, instead of one 2-byte load per lane and weight load (4-bit
// weights, K % 256 == 0, so every 16-byte piece of scales lies inside one
// row).  The same values reach the same MFMAs as with direct loads.
template <int BITS, int MT, int CG, int NS>
__device__ __forceinline__ void skinny_chunks_lds_scales(rsrc_t rx, rsrc_t rw, rsrc_t rs, int M, int N, int K, int n0,
                                                         int wave, int lane, char* sct, v4f (&acc)[MT][CG]) {
    using RG = SkinnyRegs<BITS, MT, CG, NS>;
    constexpr int GCH = RG::KCH / 32;             // group scales per row and chunk
    constexpr int SROW = GCH * 2;                 // their bytes
    constexpr int SSLOTS = 16 * CG * SROW / 16;   // 16-byte pieces of the tile's scales
    static_assert(SROW % 16 == 0 && SSLOTS % WAVE == 0, "scale tile in whole waves of 16-byte pieces");
    const int G = K / 32;
    const int nkc = (K + RG::KCH - 1) / RG::KCH;
    for (int kc = 0; kc < nkc; kc++) {
#pragma unroll
        for (int r = 0; r < (SSLOTS + 255) / 256; r++) {
            const int first = r * 256 + wave * WAVE;   // this wave's first slot
            if (first < SSLOTS) {
                const int i = first + lane, row = i / (SROW / 16), piece = i % (SROW / 16);
                const int gi = kc * GCH + piece * 8;
                const bool ok = i < SSLOTS && n0 + row < N && gi < G;
                buf_load16_lds(rs, ok ? ((uint32_t)(n0 + row) * (uint32_t)G + (uint32_t)gi) * 2 : OOB, sct + first * 16);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        RG R;
        skinny_load<BITS, MT, CG, NS, false>(R, rx, rw, rs, M, N, K, n0, kc, wave, lane);
        __builtin_amdgcn_sched_barrier(0);
        // the scale pieces went out first: they are in LDS once no more than
        // this wave's weight and activation loads are outstanding
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(NS * CG + NS * RG::NQ * MT));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NS; j++)
#pragma unroll
            for (int c = 0; c < CG; c++) {
                const int row = 16 * c + lane % 16, gl = (wave * NS + j) * 4 + lane / 16;
                R.sc[j][c] = *reinterpret_cast<const uint16_t*>(sct + row * SROW + gl * 2);
            }
        skinny_compute(R, acc);
        if (kc + 1 < nkc) __syncthreads();   // before the next chunk's scales overwrite these
    }
}

// One linear: a workgroup of 4 waves per 16 CG output channels, one chunk of
// loads in flight at a time (every load of the chunk issued before any use).
template <int BITS, int MT, int CG, int NS>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(const half_t* __restrict__ X, const uint8_t* __restrict__ Bq,
                                                          const half_t* __restrict__ S, half_t* Y, int M, int N,
                                                          int K, Epi epi) {
    using RG = SkinnyRegs<BITS, MT, CG, NS>;
    __shared__ float part[4][MT * 16][16 * CG + 1];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), lane = threadIdx.x % WAVE;
    const int n0 = xcd_remap(blockIdx.x, gridDim.x) * 16 * CG;
    const rsrc_t rx = make_rsrc(X, (uint32_t)M * (uint32_t)K * 2);
    const rsrc_t rw = make_rsrc(Bq, (uint32_t)N * (BITS == 8 ? (uint32_t)K : BITS == 4 ? (uint32_t)K / 2 : (uint32_t)K * 2));
    const rsrc_t rs = make_rsrc(S, BITS == 4 ? (uint32_t)N * (uint32_t)(K / 32) * 2 : 0u);
    v4f acc[MT][CG];
#pragma unroll
    for (int t = 0; t < MT; t++)
#pragma unroll
        for (int g = 0; g < CG; g++) acc[t][g] = v4f{};
    constexpr bool LDS_SCALES = BITS == 4 && (16 * CG * (RG::KCH / 32) * 2 / 16) % WAVE == 0;
    __shared__ __attribute__((aligned(16))) char sct[LDS_SCALES ? 16 * CG * (RG::KCH / 32) * 2 : 16];
    bool done = false;
    if constexpr (LDS_SCALES) {
        if (K % 256 == 0) {
            skinny_chunks_lds_scales<BITS, MT, CG, NS>(rx, rw, rs, M, N, K, n0, wave, lane, sct, acc);
            done = true;
        }
    }
    if (!done) {
        const int nkc = (K + RG::KCH - 1) / RG::KCH;
        for (int kc = 0; kc < nkc; kc++) {
            RG R;
            skinny_load(R, rx, rw, rs, M, N, K, n0, kc, wave, lane);
            // keep the scheduler from sinking loads next to their uses, which
            // would serialise the chunk into several round trips to memory
            __builtin_amdgcn_sched_barrier(0);
            skinny_compute(R, acc);
        }
    }
    skinny_finish<BITS, MT, CG>(part, acc, S, Y, M, N, epi, n0, wave, lane);
}

// Several linears in one launch, one tile of 16 CG output channels per
// workgroup: the workgroups of problem p are [first_p, first_p + tiles_p) of
// one flat grid.  With 4-bit weights and K % 256 == 0 the group scales of the
// tile's chunk (16 CG rows x 48 groups, contiguous per row) are fetched once
// per workgroup by LDS-DMA, 16 bytes per lane, instead of one 2-byte load per
// lane and weight load: on this path it is the instruction count, not the
// bytes, that limits how fast the weights stream.
template <int BITS, int MT, int CG, int NS>
__global__ __launch_bounds__(256) void gemm_skinny_grouped_kernel(SkinnyGroup g) {
    using RG = SkinnyRegs<BITS, MT, CG, NS>;
    constexpr int GCH = RG::KCH / 32;             // group scales per row and chunk
    constexpr int SROW = GCH * 2;                 // their bytes
    constexpr int SSLOTS = 16 * CG * SROW / 16;   // 16-byte pieces of the tile's scales
    static_assert(SROW % 16 == 0 && SSLOTS % WAVE == 0, "scale tile in whole waves of 16-byte pieces");
    __shared__ float part[4][MT * 16][16 * CG + 1];
    __shared__ __attribute__((aligned(16))) char sct[BITS == 4 ? 16 * CG * SROW : 16];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), lane = threadIdx.x % WAVE;
    const int b = xcd_remap(blockIdx.x, gridDim.x);
    int pi = 0;
#pragma unroll
    for (int i = 1; i < kSkinnyGroupMax; i++)
        if (i < g.count && b >= g.p[i].first) pi = i;
    const SkinnyProblem& P = g.p[pi];
    const int n0 = (b - P.first) * 16 * CG;
    const int G = P.K / 32;
    const rsrc_t rx = make_rsrc(P.x, (uint32_t)P.M * (uint32_t)P.K * 2);
    const rsrc_t rw = make_rsrc(P.w, (uint32_t)P.N * (BITS == 8 ? (uint32_t)P.K : BITS == 4 ? (uint32_t)P.K / 2 : (uint32_t)P.K * 2));
    const rsrc_t rs = make_rsrc(P.s, BITS == 4 ? (uint32_t)P.N * (uint32_t)G * 2 : 0u);
    v4f acc[MT][CG];
#pragma unroll
    for (int t = 0; t < MT; t++)
#pragma unroll
        for (int c = 0; c < CG; c++) acc[t][c] = v4f{};
    const int nkc = (P.K + RG::KCH - 1) / RG::KCH;
    if (BITS == 4 && P.K % 256 == 0) {
        skinny_chunks_lds_scales<BITS, MT, CG, NS>(rx, rw, rs, P.M, P.N, P.K, n0, wave, lane, sct, acc);
    } else {
        for (int kc = 0; kc < nkc; kc++) {
            RG R;
            skinny_load(R, rx, rw, rs, P.M, P.N, P.K, n0, kc, wave, lane);
            __builtin_amdgcn_sched_barrier(0);
            skinny_compute(R, acc);
        }
    }
    skinny_finish<BITS, MT, CG>(part, acc, P.s, P.y, P.M, P.N, P.epi, n0, wave, lane);
}

// Streaming form of the grouped call for 4-bit weights at M <= 16 with K a
// multiple of 256 up to one chunk (1536) and N a multiple of 8: persistent
// workgroups, three per CU, each walk a contiguous run of units (32 output
// channels of one problem over all of K), loading the next unit while they
// decode one.
//  - A unit's weights (32 rows x up to 768 bytes) are loaded in whole lines:
//    each instruction moves 4 rows x 256 contiguous bytes (the register path
//    of the kernels above moves 16 rows x 64 bytes per instruction, which
//    streams ~25 % slower on MI355X).  The lanes then hold the wrong rows for
//    the MFMA layout, so the unit passes through LDS: stored with an XOR
//    swizzle, read back in the MFMA layout with 16 rows at one column landing
//    in 16 different bank groups.  The group scales (32 rows x K/32,
//    contiguous) travel the same way, and so do the epilogue operands.
//  - Each wave takes the same K-quarter, steps and MFMA order as in the
//    single-problem kernel and decodes the same bytes, and the four partial
//    tiles are summed in LDS in the same order, so the results are
//    bit-identical to one call per problem.
//  - Each wave keeps its quarter of the activations in registers for the
//    whole run (a workgroup's run never leaves its problem).
//  - One unit in flight per workgroup and three workgroups per CU measured
//    best: two units in flight per workgroup need two register sets, which
//    leaves room for only two workgroups per CU, and streamed slower.
constexpr int kStreamCh = 32;                 // output channels per unit
constexpr int kStreamWB = kStreamCh * 768;    // weight bytes of a unit's LDS stage (K <= 1536)
constexpr int kStreamSB = 4096;               // scale bytes of a stage (4 waves x 64 lanes x 16 bytes)
constexpr int kStreamPerCU = 3;               // workgroups per CU (LDS 40 KB, 164 VGPRs each)

__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// g.p[i].first is the first workgroup of problem i; each of its workgroups
// takes `units_per_wg` consecutive units of that problem (the last one fewer
// real units; the rest empty).  EPI: some problem of the group has a bias,
// residual or steering operand (without, a unit loads only weights and
// scales).
template <bool EPI>
__global__ __launch_bounds__(256, kStreamPerCU) void gemm_skinny_stream_kernel(SkinnyGroup g, int units_per_wg) {
    constexpr int BITS = 4, MT = 1, CG = kStreamCh / 16, NS = kNS4;
    using RG = SkinnyRegs<BITS, MT, CG, NS>;
    // One weight and scale stage: it is refilled at the start of the next
    // unit, after every wave has passed this unit's second barrier and so made
    // its last weight read.  The epilogue pieces are read after that barrier,
    // so they alternate between two small buffers.
    constexpr int EPB = 1280;   // residual 1024 B, bias 64 B, direction 128 B, pad
    __shared__ __attribute__((aligned(16))) char stage[kStreamWB + kStreamSB];
    __shared__ __attribute__((aligned(16))) char epi[2][EPB];
    __shared__ float part[4][MT * 16][16 * CG + 1];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), lane = threadIdx.x % WAVE;
    const int tid = (int)threadIdx.x;
    int pi = 0;
#pragma unroll
    for (int i = 1; i < kSkinnyGroupMax; i++)
        if (i < g.count && (int)blockIdx.x >= g.p[i].first) pi = i;
    const SkinnyProblem& P = g.p[pi];
    const int nunits = (P.N + kStreamCh - 1) / kStreamCh;
    // units [u0, uend) of problem pi; those past nunits are empty (their loads
    // read zeros, nothing is stored), so the loop below has no conditional
    // steps and the compiler's load counts stay exact
    const int u0 = ((int)blockIdx.x - P.first) * units_per_wg;
    const int uend = u0 + units_per_wg;
    const uint32_t rowb = (uint32_t)P.K / 2, G = (uint32_t)P.K / 32;
    const rsrc_t rw = make_rsrc(P.w, (uint32_t)P.N * rowb);
    const rsrc_t rs = make_rsrc(P.s, (uint32_t)P.N * G * 2);
    const rsrc_t ry = make_rsrc(P.y, (uint32_t)P.M * (uint32_t)P.N * 2);
    const EpiW& e = P.epi;
    const bool steer = e.steer_dir && e.steer_alpha;
    const rsrc_t rbias = make_rsrc(e.bias, e.bias ? (uint32_t)P.N * 2 : 0u);
    const rsrc_t rres = make_rsrc(e.residual, e.residual ? (uint32_t)P.M * (uint32_t)P.N * 2 : 0u);
    const rsrc_t rdir = make_rsrc(e.steer_dir, steer ? (uint32_t)P.N * 4 : 0u);
    const rsrc_t ralpha = make_rsrc(e.steer_alpha, steer ? 4u : 0u);

    // This lane's activations, loaded once: each wave reads only its quarter
    // of K, the same runs as in the single-problem kernel (row lane % 16,
    // k = kb + 8 q .. kb + 8 q + 7 for step j); zero past M and K.
    v4i xr[NS][RG::NQ];
    {
        const rsrc_t rx = make_rsrc(P.x, (uint32_t)P.M * (uint32_t)P.K * 2);
        const int m = lane % 16;
#pragma unroll
        for (int j = 0; j < NS; j++) {
            const int kb = (wave * NS + j) * RG::KPW + (lane / 16) * RG::KPL;
#pragma unroll
            for (int q = 0; q < RG::NQ; q++)
                xr[j][q] = buf_load16(rx, m < P.M && kb + 8 * q < P.K ? ((uint32_t)m * P.K + kb + 8 * q) * 2 : OOB);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // A unit's loads, 16-byte pieces per lane: six of weights and one of
    // scales, then (EPI) one each from the residual, the bias and the steering
    // direction (the unit's 16 x 32 residual block is 64 pieces, held by
    // threads 0..63; its 32 biases 4 pieces, threads 64..67; its 32 direction
    // entries 8 pieces, threads 68..75; every other lane reads out of range).
    // Every global read of a unit travels in this one stream of whole 16-byte
    // register tuples: the load counter is in order, so a read issued late
    // would wait for the unit in flight, and loop-carried values narrower than
    // a tuple get split and copied at the loop's back edge, where each copy
    // waits for its load.
    constexpr int NL = EPI ? 10 : 7;
    v4i RW[NL];
    // Per-lane parts of the offsets, fixed for the whole run.  A unit adds
    // only its first row; rows past N (the ragged last unit, the empty units)
    // lie past the end of the weight, scale, bias and direction buffers and
    // read zeros, and residual rows past M past the end of the residual, so
    // no load depends on the unit being real (a predicate there turns into
    // branches around the loads, and the compiler then waits for every load
    // in flight at the join).  With N a multiple of 8 no 16-byte piece
    // straddles column N; residual pieces of a ragged last unit's columns past
    // N land in the next row, and their outputs are not stored.
    uint32_t wofs[6];
#pragma unroll
    for (int i = 0; i < 6; i++) {
        const int b = 6 * wave + i, rg = b / 3, seg = b % 3;      // block b: rows 4 rg .. 4 rg + 3, bytes 256 seg ..
        const int r4 = lane / 16, c = (lane % 16) ^ (4 * (rg % 4) + r4);
        const uint32_t byte = 256u * seg + 16u * c;
        wofs[i] = byte < rowb ? (uint32_t)(4 * rg + r4) * rowb + byte : OOB;
    }
    const uint32_t sofs = (uint32_t)tid * 16;
    const uint32_t sofs_ok = sofs < (uint32_t)kStreamCh * G * 2 ? sofs : OOB;
    const uint32_t rofs = tid < 64 ? ((uint32_t)(tid / 4) * P.N + 8 * (tid % 4)) * 2 : OOB;
    const uint32_t bofs = tid >= 64 && tid < 68 ? (uint32_t)(tid - 64) * 16 : OOB;
    const uint32_t dofs = tid >= 68 && tid < 76 ? (uint32_t)(tid - 68) * 16 : OOB;
    const float alpha = steer ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ralpha, 0, 0, 0)) : 0.0f;
    // The prefetch past this workgroup's last unit (the loop's final pass) is
    // pushed 2^21 rows out, past every buffer, so it costs no traffic; done
    // with integer min / max, since a predicate here becomes a branch.
    auto issue = [&](int u) {
        const uint32_t n0 = (uint32_t)u * kStreamCh + (uint32_t)min(max(u - uend + 1, 0), 1) * (1u << 21);
#pragma unroll
        for (int i = 0; i < 6; i++) RW[i] = buf_load16(rw, wofs[i] + n0 * rowb);
        RW[6] = buf_load16(rs, sofs_ok + n0 * G * 2);
        if constexpr (EPI) {
            RW[7] = buf_load16(rres, rofs + n0 * 2);
            RW[8] = buf_load16(rbias, bofs + n0 * 2);
            RW[9] = buf_load16(rdir, dofs + n0 * 4);
        }
    };

    // Unit u's outputs from its four partial tiles (summed in the same order
    // as skinny_finish) and the epilogue of epilogue_apply on the operands
    // prefetched with the unit; thread o's outputs are rows o / 32 and
    // o / 32 + 8 of column o % 32.  The stores are range-checked buffer
    // stores, issued on every path (an out-of-range one is dropped).
    auto finish = [&](int u) {
        const bool real = u < nunits;
        const char* ep = epi[(u - u0) & 1];
        const int n0 = u * kStreamCh;
        constexpr int OUTS = MT * 16 * kStreamCh / 256;
#pragma unroll
        for (int k = 0; k < OUTS; k++) {
            const int o = tid + 256 * k;
            const int row = o / kStreamCh, cc = o % kStreamCh, col = n0 + cc;
            float v = ((part[0][row][cc] + part[1][row][cc]) + part[2][row][cc]) + part[3][row][cc];
            if (EPI && e.bias) v += (float)*reinterpret_cast<const half_t*>(ep + 1024 + cc * 2);
            if (e.gelu) v = gelu_tanh(v);
            if (EPI && e.residual) v += (float)*reinterpret_cast<const half_t*>(ep + row * 64 + cc * 2);
            if (EPI && alpha != 0.0f) v += alpha * *reinterpret_cast<const float*>(ep + 1088 + cc * 4);
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, (half_t)v), ry,
                                                  (int)(real && row < P.M && col < P.N ? ((uint32_t)row * P.N + col) * 2 : OOB), 0, 0);
        }
    };

    // Per unit: its loads into LDS, the next unit's loads issued, then the
    // previous unit's outputs stored.  A store pending at a wait for loads
    // makes the compiler wait for everything (loads and stores may complete
    // out of order), so the stores go out right after the next loads and have
    // a whole unit of decoding to complete in, instead of just before the
    // wait as at the end of their own unit.
    issue(u0);
    for (int u = u0; u < uend; u++) {
        // unit u into LDS: lane l of block b at slot l (the swizzle is in which
        // bytes the lane loaded)
#pragma unroll
        for (int i = 0; i < 6; i++) *reinterpret_cast<v4i*>(stage + (6 * wave + i) * 1024 + lane * 16) = RW[i];
        *reinterpret_cast<v4i*>(stage + kStreamWB + tid * 16) = RW[6];
        // the epilogue pieces (threads 0..75): residual rows at 64-byte pitch,
        // then bias, then direction
        if constexpr (EPI)
            if (tid < EPB / 16) *reinterpret_cast<v4i*>(epi[(u - u0) & 1] + tid * 16) = RW[7] | RW[8] | RW[9];
        issue(u + 1);
        if (u > u0) finish(u - 1);
        lds_barrier();   // unit u in LDS; every wave is done with unit u - 1's partial tiles

        v4f acc[CG];
#pragma unroll
        for (int c = 0; c < CG; c++) acc[c] = v4f{};
#pragma unroll
        for (int j = 0; j < NS; j++) {
#pragma unroll
            for (int c = 0; c < CG; c++) {
                // this lane's run: row R of the unit, bytes B .. B + 15 of the row
                const int R = 16 * c + lane % 16;
                const int B = 192 * wave + 64 * j + 16 * (lane / 16);
                const int rg = R / 4, r4 = R % 4, seg = B / 256, ch = (B % 256) / 16;
                const int slot = 16 * r4 + (ch ^ (4 * (rg % 4) + r4));
                const v4i w = *reinterpret_cast<const v4i*>(stage + (3 * rg + seg) * 1024 + slot * 16);
                const int gi = (wave * NS + j) * 4 + lane / 16;
                const u32 sb = *reinterpret_cast<const uint16_t*>(stage + kStreamWB + (R * (int)G + gi) * 2);
                v4i d[RG::NQ];
                dec4_bits(w, sb, d);
#pragma unroll
                for (int q = 0; q < RG::NQ; q++)
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, xr[j][q]),
                                                                    __builtin_bit_cast(v8h, d[q]), acc[c], 0, 0, 0);
            }
        }
#pragma unroll
        for (int c = 0; c < CG; c++)
#pragma unroll
            for (int r = 0; r < 4; r++) part[wave][4 * (lane / 16) + r][16 * c + lane % 16] = acc[c][r];
        // unit u's partial tiles complete; every wave is done reading the stage
        lds_barrier();
    }
    finish(uend - 1);
}

size_t wxa16_workspace_bytes(int, int64_t, int64_t, int64_t) { return 0; }

namespace {

// K-chunk of 1536 at every width: NS = 3 steps of 128 k (4-bit), 6 of 64 k
// (8-bit) or 12 of 32 k (fp16).
template <int BITS>
constexpr int kNS = BITS == 8 ? 6 : BITS == 4 ? 3 : 12;

// Compute units of the current device (queried once).
int skinny_cus() {
    static int cus = 0;
    if (!cus) {
        int dev = 0, n = 0;
        cus = hipGetDevice(&dev) == hipSuccess &&
                      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0
                  ? n
                  : 256;
    }
    return cus;
}

template <int BITS, int MT, int CG>
hipError_t launch_skinny_cg(const half_t* x, const uint8_t* wq, const half_t* s, half_t* y, int M, int N, int K,
                            const Epi& epi, hipStream_t st) {
    dim3 grid((N + 16 * CG - 1) / (16 * CG)), block(256);
    hipLaunchKernelGGL((gemm_skinny_kernel<BITS, MT, CG, kNS<BITS>>), grid, block, 0, st, x, wq, s, y, M, N, K, epi);
    return hipGetLastError();
}

// One workgroup per 16 output channels, or per 32 where that halves a grid of
// one to two workgroups per CU at M > 8: every workgroup reads all of X (for
// 16 rows four times the bytes of its 4-bit weights), so fewer workgroups
// read less of it.  Measured at K = 1536, one dependent launch per layer:
// M = 16, N = 4608 / 6144 / 8192: W4A16 6.5-6.6 -> 5.9-6.1 us, W8A16
// 6.7-7.0 -> 6.0-6.7 us; at M = 4 (X rows past M read nothing) it does not
// pay, nor beyond two workgroups per CU.  The sums are the same either way.
template <int BITS, int MT>
hipError_t launch_skinny_mt(const half_t* x, const uint8_t* wq, const half_t* s, half_t* y, int M, int N, int K,
                            const Epi& epi, hipStream_t st) {
    if constexpr (BITS != 16 && MT == 1) {
        const int cus = skinny_cus();
        if (M > 8 && N > 16 * cus && N <= 32 * cus) return launch_skinny_cg<BITS, MT, 2>(x, wq, s, y, M, N, K, epi, st);
    }
    return launch_skinny_cg<BITS, MT, 1>(x, wq, s, y, M, N, K, epi, st);
}

template <int BITS>
hipError_t launch_skinny(const half_t* x, const uint8_t* wq, const half_t* s, half_t* y, int M, int N, int K,
                         const Epi& epi, hipStream_t st) {
    if (M <= 16) return launch_skinny_mt<BITS, 1>(x, wq, s, y, M, N, K, epi, st);
    if (M <= 32) return launch_skinny_mt<BITS, 2>(x, wq, s, y, M, N, K, epi, st);
    return launch_skinny_mt<BITS, 4>(x, wq, s, y, M, N, K, epi, st);
}

// Grouped launches have tiles to spare, so each wave takes several column
// groups and reuses every activation fragment across them.
constexpr int kGroupedCG = 4;

template <int BITS, int MT>
hipError_t launch_grouped_tiles(const SkinnyGroup& g, int tiles, hipStream_t st) {
    hipLaunchKernelGGL((gemm_skinny_grouped_kernel<BITS, MT, kGroupedCG, kNS<BITS>>), dim3(tiles), dim3(256), 0, st, g);
    return hipGetLastError();
}

}  // namespace

// Every problem fits the streaming kernel: 4-bit, M <= 16, K % 256 == 0 and
// K <= 1536 (one chunk, so a unit is all of K).
bool stream_fits(int bits, const SkinnyGroup& g) {
    if (bits != 4) return false;
    for (int i = 0; i < g.count; i++)
        if (g.p[i].M > 16 || g.p[i].K % 256 != 0 || g.p[i].K > 1536 || g.p[i].N % 8 != 0 || g.p[i].N > (1 << 20))
            return false;
    return true;
}

hipError_t launch_skinny_grouped(int bits, SkinnyGroup& g, hipStream_t st) {
    if (g.count < 1 || g.count > kSkinnyGroupMax) return hipErrorInvalidValue;
    if (stream_fits(bits, g)) {
        // persistent workgroups, each a run of one problem's units: about
        // kStreamPerCU per CU in all
        int units = 0;
        bool epi = false;
        for (int i = 0; i < g.count; i++) {
            units += (g.p[i].N + kStreamCh - 1) / kStreamCh;
            epi = epi || g.p[i].epi.bias || g.p[i].epi.residual || (g.p[i].epi.steer_dir && g.p[i].epi.steer_alpha);
        }
        int cus = 0, dev = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        // the smallest run length whose workgroups (each problem's runs
        // rounded up on its own) all fit in one wave of resident workgroups
        const int slots = kStreamPerCU * cus;
        int per = (units + slots - 1) / slots;
        for (;; per++) {
            int need = 0;
            for (int i = 0; i < g.count; i++) need += ((g.p[i].N + kStreamCh - 1) / kStreamCh + per - 1) / per;
            if (need <= slots) break;
        }
        int wgs = 0;
        for (int i = 0; i < g.count; i++) {
            g.p[i].first = wgs;
            wgs += ((g.p[i].N + kStreamCh - 1) / kStreamCh + per - 1) / per;
        }
        if (epi) hipLaunchKernelGGL(gemm_skinny_stream_kernel<true>, dim3(wgs), dim3(256), 0, st, g, per);
        else hipLaunchKernelGGL(gemm_skinny_stream_kernel<false>, dim3(wgs), dim3(256), 0, st, g, per);
        return hipGetLastError();
    }
    int tiles = 0, maxm = 0;
    for (int i = 0; i < g.count; i++) {
        g.p[i].first = tiles;
        tiles += (g.p[i].N + 16 * kGroupedCG - 1) / (16 * kGroupedCG);
        maxm = g.p[i].M > maxm ? g.p[i].M : maxm;
    }
    if (maxm > 64) return hipErrorInvalidValue;
    if (bits == 8)
        return maxm <= 16 ? launch_grouped_tiles<8, 1>(g, tiles, st)
             : maxm <= 32 ? launch_grouped_tiles<8, 2>(g, tiles, st) : launch_grouped_tiles<8, 4>(g, tiles, st);
    return maxm <= 16 ? launch_grouped_tiles<4, 1>(g, tiles, st)
         : maxm <= 32 ? launch_grouped_tiles<4, 2>(g, tiles, st) : launch_grouped_tiles<4, 4>(g, tiles, st);
}

hipError_t launch_gemm_wxa16(int bits, const half_t* x, const void* wq, const half_t* s, half_t* y, int M,
                             int N, int K, const Epi& epi, void*, size_t, hipStream_t st) {
    const uint8_t* w = static_cast<const uint8_t*>(wq);
    if (M <= 64) {
        if (bits == 8) return launch_skinny<8>(x, w, s, y, M, N, K, epi, st);
        if (bits == 4) return launch_skinny<4>(x, w, s, y, M, N, K, epi, st);
        return launch_skinny<16>(x, w, s, y, M, N, K, epi, st);
    }
    return launch_gemm_tiled(bits == 8 ? 1 : bits == 4 ? 2 : 3, x, wq, s, nullptr, y, M, N, K, epi, st);
}

}  // namespace aria
