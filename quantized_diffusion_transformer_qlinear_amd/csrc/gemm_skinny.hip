// a3+a4+a5 — weight-only linears (W8A16 = the pages' "q8", W4A16 = "q4") at
// small M (M <= 64 tokens), where the layer is bound by streaming the packed
// weights from HBM (aria project page, "Results": the 4-bit weights are what
// put the 1.2 B model on an 8 GB device).
//   W8A16: y = epilogue(s_w[n] * sum_k x[m][k] * q[n][k])
//   W4A16: y = epilogue(sum_k x[m][k] * fp16(q4[n][k] * s_g[n][k/32]))
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

template <int BITS, int MT, int CG, int NS>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(const half_t* __restrict__ X, const uint8_t* __restrict__ Bq,
                                                          const half_t* __restrict__ S, half_t* Y, int M, int N,
                                                          int K, Epi epi) {
    constexpr int KPL = BITS == 8 ? 16 : 32;  // k per lane per 16-byte weight load
    constexpr int NQ = KPL / 8;               // 16x16x32 MFMAs fed by one load
    constexpr int KPW = 4 * KPL;              // k per wave step (4 lane groups)
    constexpr int NC = 16 * CG;               // output channels per workgroup
    __shared__ float part[4][MT * 16][NC + 1];

    const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
    const int n0 = xcd_remap(blockIdx.x, gridDim.x) * NC;
    const int gsel = lane / 16;                // which k-run of a step this lane reads
    const uint32_t rowbytes = BITS == 8 ? (uint32_t)K : (uint32_t)K / 2;
    const int G = K / 32;
    const rsrc_t rx = make_rsrc(X, (uint32_t)M * (uint32_t)K * 2);
    const rsrc_t rw = make_rsrc(Bq, (uint32_t)N * rowbytes);
    const rsrc_t rs = make_rsrc(S, BITS == 4 ? (uint32_t)N * (uint32_t)G * 2 : 0u);

    // this wave's share of K, in whole steps
    const int steps = (K + KPW - 1) / KPW;
    const int s_beg = (steps * wave) / 4, s_end = (steps * (wave + 1)) / 4;

    v4f acc[MT][CG];
#pragma unroll
    for (int t = 0; t < MT; t++)
#pragma unroll
        for (int g = 0; g < CG; g++) acc[t][g] = v4f{};

    // Groups of NS steps: every load of a group is issued before any is used,
    // and no load is carried across iterations (so the waits stay exact).
    // Steps past this wave's share read as zero (out-of-range buffer offsets).
    for (int st0 = s_beg; st0 < s_end; st0 += NS) {
        v4i w[NS][CG], x[NS][NQ][MT];
        half_t sc[NS][CG];
#pragma unroll
        for (int j = 0; j < NS; j++) {
            const int st = st0 + j;
            const int kb = st * KPW + gsel * KPL;  // first k of this lane's run
            const bool in = st < s_end && kb < K;
#pragma unroll
            for (int g = 0; g < CG; g++) {
                const int col = n0 + 16 * g + lane % 16;
                const bool ok = in && col < N;
                w[j][g] = buf_load16(rw, ok ? (uint32_t)col * rowbytes + (uint32_t)(BITS == 8 ? kb : kb / 2) : OOB);
                if (BITS == 4) sc[j][g] = buf_load_h(rs, ok ? ((uint32_t)col * G + kb / 32) * 2 : OOB);
            }
#pragma unroll
            for (int q = 0; q < NQ; q++)
#pragma unroll
                for (int t = 0; t < MT; t++) {
                    const int m = t * 16 + lane % 16;
                    x[j][q][t] = buf_load16(rx, in && m < M ? ((uint32_t)m * K + kb + 8 * q) * 2 : OOB);
                }
        }
#pragma unroll
        for (int j = 0; j < NS; j++)
#pragma unroll
            for (int g = 0; g < CG; g++) {
                v4i d[NQ];
                if constexpr (BITS == 8) {
                    dec8(w[j][g], d[0], d[1]);
                } else {
                    dec4(w[j][g], sc[j][g], d);
                }
                // MFMA q of this run: the lane's 8 k are kb + 8q .. kb + 8q + 7 for its row and column
#pragma unroll
                for (int q = 0; q < NQ; q++)
#pragma unroll
                    for (int t = 0; t < MT; t++)
                        acc[t][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, x[j][q][t]),
                                                                           __builtin_bit_cast(v8h, d[q]), acc[t][g],
                                                                           0, 0, 0);
            }
    }

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
}

size_t wxa16_workspace_bytes(int, int64_t, int64_t, int64_t) { return 0; }

namespace {

template <int BITS, int MT>
hipError_t launch_skinny_mt(const half_t* x, const uint8_t* wq, const half_t* s, half_t* y, int M, int N, int K,
                            const Epi& epi, hipStream_t st) {
    constexpr int CG = 1, NS = BITS == 8 ? 8 : 4;
    dim3 grid((N + 16 * CG - 1) / (16 * CG)), block(256);
    hipLaunchKernelGGL((gemm_skinny_kernel<BITS, MT, CG, NS>), grid, block, 0, st, x, wq, s, y, M, N, K, epi);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_skinny(const half_t* x, const uint8_t* wq, const half_t* s, half_t* y, int M, int N, int K,
                         const Epi& epi, hipStream_t st) {
    if (M <= 16) return launch_skinny_mt<BITS, 1>(x, wq, s, y, M, N, K, epi, st);
    if (M <= 32) return launch_skinny_mt<BITS, 2>(x, wq, s, y, M, N, K, epi, st);
    return launch_skinny_mt<BITS, 4>(x, wq, s, y, M, N, K, epi, st);
}

}  // namespace

hipError_t launch_gemm_wxa16(int bits, const half_t* x, const void* wq, const half_t* s, half_t* y, int M,
                             int N, int K, const Epi& epi, void*, size_t, hipStream_t st) {
    const uint8_t* w = static_cast<const uint8_t*>(wq);
    if (M <= 64)
        return bits == 8 ? launch_skinny<8>(x, w, s, y, M, N, K, epi, st) : launch_skinny<4>(x, w, s, y, M, N, K, epi, st);
    return launch_gemm_tiled(bits == 8 ? 1 : 2, x, wq, s, nullptr, y, M, N, K, epi, st);
}

}  // namespace aria
