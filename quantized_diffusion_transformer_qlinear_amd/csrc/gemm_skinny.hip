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
template <int BITS, int MT, int CG>
__device__ __forceinline__ void skinny_finish(float (&part)[4][MT * 16][16 * CG + 1], v4f (&acc)[MT][CG],
                                              const half_t* S, half_t* Y, int M, int N, const Epi& epi, int n0,
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
    const int nkc = (K + RG::KCH - 1) / RG::KCH;
    for (int kc = 0; kc < nkc; kc++) {
        RG R;
        skinny_load(R, rx, rw, rs, M, N, K, n0, kc, wave, lane);
        // keep the scheduler from sinking loads next to their uses, which
        // would serialise the chunk into several round trips to memory
        __builtin_amdgcn_sched_barrier(0);
        skinny_compute(R, acc);
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
        // G % 8 == 0: every 16-byte piece of scales lies inside one row
        for (int kc = 0; kc < nkc; kc++) {
#pragma unroll
            for (int r = 0; r < (SSLOTS + 255) / 256; r++) {
                const int first = r * 256 + wave * WAVE;   // this wave's first slot
                if (first < SSLOTS) {
                    const int i = first + lane, row = i / (SROW / 16), piece = i % (SROW / 16);
                    const int gi = kc * GCH + piece * 8;
                    const bool ok = i < SSLOTS && n0 + row < P.N && gi < G;
                    buf_load16_lds(rs, ok ? ((uint32_t)(n0 + row) * (uint32_t)G + (uint32_t)gi) * 2 : OOB, sct + first * 16);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            RG R;
            skinny_load<BITS, MT, CG, NS, false>(R, rx, rw, rs, P.M, P.N, P.K, n0, kc, wave, lane);
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

size_t wxa16_workspace_bytes(int, int64_t, int64_t, int64_t) { return 0; }

namespace {

// K-chunk of 1536 at every width: NS = 3 steps of 128 k (4-bit), 6 of 64 k
// (8-bit) or 12 of 32 k (fp16).
template <int BITS>
constexpr int kNS = BITS == 8 ? 6 : BITS == 4 ? 3 : 12;

template <int BITS, int MT>
hipError_t launch_skinny_mt(const half_t* x, const uint8_t* wq, const half_t* s, half_t* y, int M, int N, int K,
                            const Epi& epi, hipStream_t st) {
    constexpr int CG = 1;
    dim3 grid((N + 16 * CG - 1) / (16 * CG)), block(256);
    hipLaunchKernelGGL((gemm_skinny_kernel<BITS, MT, CG, kNS<BITS>>), grid, block, 0, st, x, wq, s, y, M, N, K, epi);
    return hipGetLastError();
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

hipError_t launch_skinny_grouped(int bits, SkinnyGroup& g, hipStream_t st) {
    if (g.count < 1 || g.count > kSkinnyGroupMax) return hipErrorInvalidValue;
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
