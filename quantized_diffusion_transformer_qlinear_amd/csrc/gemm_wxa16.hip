// a3+a4+a5 — weight-only linears (W8A16 = the pages' "q8", W4A16 = "q4"):
// packed weights are streamed from HBM, decoded to fp16 in registers, and
// contracted with fp16 activations on the fp16 matrix cores (fp32 accumulation).
//
// The aria project page ("What aria is", "Quantization that saves memory";
// "Results", the q8 / q4 columns) stores the transformer weights at 8 or 4 bits.
//   W8A16: y = epilogue(s_w[n] * sum_k x[m][k] * q[n][k])   (q -> fp16 is exact;
//          the per-channel scale is applied once, in the epilogue)
//   W4A16: y = epilogue(sum_k x[m][k] * fp16(q4[n][k] * s_g[n][k/32]))
//          (nibble -> signed int -> times its group scale, one fp16 rounding)
//
// M > 64 runs the tiled kernel (gemm_tiled.hip); this file holds the kernel
// for small M:
//  - skinny (M <= 64, bandwidth-bound): 4 waves per 16 output channels split K
//    four ways; each lane streams 16-byte runs of one channel's packed row and
//    decodes them straight into v_mfma_f32_16x16x32_f16 operands (no LDS for
//    the weights: no other wave reuses them); the four partial tiles are summed
//    in LDS in a fixed order, so results are deterministic.
#include "common.h"
#include "kernels.h"

namespace aria {

namespace {

// 16 int8 -> 16 fp16 (exact).
__device__ __forceinline__ void decode8(v4i w, v8h& lo, v8h& hi) {
#pragma unroll
    for (int d = 0; d < 4; d++) {
        const int word = w[d];
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const half_t h = (half_t)(float)((word << (24 - 8 * b)) >> 24);  // sign-extended byte
            if (d < 2) lo[d * 4 + b] = h; else hi[(d - 2) * 4 + b] = h;
        }
    }
}

// 32 nibbles (even k in the low nibble) -> 32 fp16 values q * s, one rounding each.
__device__ __forceinline__ void decode4(v4i w, float s, v8h out[4]) {
#pragma unroll
    for (int d = 0; d < 4; d++) {
        const int word = w[d];
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const int q = (word << (28 - 4 * e)) >> 28;  // sign-extended nibble e of the word
            out[d][e] = (half_t)((float)q * s);           // exact product in fp32, then RNE to fp16
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// skinny kernel: M <= 16 * MT, 4 waves x 16 output channels, K split over waves
// ---------------------------------------------------------------------------
template <int BITS, int MT>
__global__ __launch_bounds__(256) void gemm_wxa16_skinny_kernel(
    const half_t* __restrict__ X, const uint8_t* __restrict__ Bq, const half_t* __restrict__ S,
    half_t* Y, int M, int N, int K, Epi epi) {
    constexpr int KPL = BITS == 8 ? 16 : 32;  // k per lane per 16-byte load
    constexpr int KPW = KPL * 4;              // k per wave-wide load step (4 lane groups)
    __shared__ float part[4][MT][16][17];

    const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
    const int n0 = xcd_remap(blockIdx.x, gridDim.x) * 16;
    const int col = n0 + lane % 16;            // the channel this lane streams
    const int gsel = lane / 16;                // which k-run of the step
    const int gcol = min(col, N - 1);
    const int64_t rowbytes = BITS == 8 ? (int64_t)K : (int64_t)K / 2;
    const int G = K / 32;
    // this wave's share of K, in whole steps
    const int steps = (K + KPW - 1) / KPW;
    const int s_beg = (steps * wave) / 4, s_end = (steps * (wave + 1)) / 4;

    v4f acc[MT];
#pragma unroll
    for (int t = 0; t < MT; t++) acc[t] = v4f{};

    for (int st = s_beg; st < s_end; st++) {
        const int kb = st * KPW + gsel * KPL;   // first k of this lane's run
        const bool in = kb < K;
        const v4i w = in ? *reinterpret_cast<const v4i*>(Bq + gcol * rowbytes + (BITS == 8 ? kb : kb / 2)) : v4i{};
        v8h b[KPL / 8];
        if constexpr (BITS == 8) {
            decode8(w, b[0], b[1]);
        } else {
            const float s = in ? (float)S[(int64_t)gcol * G + kb / 32] : 0.0f;
            decode4(w, s, b);
        }
#pragma unroll
        for (int q = 0; q < KPL / 8; q++) {
            // MFMA q of this run: lane's 8 k are kb + 8q .. kb + 8q + 7 for its row/column
#pragma unroll
            for (int t = 0; t < MT; t++) {
                const int m = min(t * 16 + lane % 16, M - 1);
                const v8h a = in ? *reinterpret_cast<const v8h*>(X + (int64_t)m * K + kb + 8 * q) : v8h{};
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[q], acc[t], 0, 0, 0);
            }
        }
    }
    // 16x16 block layout: register r of lane l holds row 4*(l/16) + r, column l%16
#pragma unroll
    for (int t = 0; t < MT; t++)
#pragma unroll
        for (int r = 0; r < 4; r++) part[wave][t][4 * (lane / 16) + r][lane % 16] = acc[t][r];
    __syncthreads();

    const float alpha = load_alpha(epi);
    for (int o = threadIdx.x; o < MT * 256; o += 256) {
        const int t = o / 256, rr = (o % 256) / 16, cc = o % 16;
        const int row = t * 16 + rr, c = n0 + cc;
        if (row >= M || c >= N) continue;
        float v = ((part[0][t][rr][cc] + part[1][t][rr][cc]) + part[2][t][rr][cc]) + part[3][t][rr][cc];
        if (BITS == 8) v *= (float)S[c];
        const int64_t idx = (int64_t)row * N + c;
        Y[idx] = (half_t)epilogue_apply(v, idx, c, epi, alpha);
    }
}

size_t wxa16_workspace_bytes(int, int64_t, int64_t, int64_t) { return 0; }

template <int BITS>
static hipError_t launch_skinny(const half_t* x, const uint8_t* wq, const half_t* s, half_t* y, int M, int N, int K,
                                const Epi& epi, hipStream_t st) {
    dim3 grid((N + 15) / 16), block(256);
    if (M <= 16) hipLaunchKernelGGL((gemm_wxa16_skinny_kernel<BITS, 1>), grid, block, 0, st, x, wq, s, y, M, N, K, epi);
    else if (M <= 32) hipLaunchKernelGGL((gemm_wxa16_skinny_kernel<BITS, 2>), grid, block, 0, st, x, wq, s, y, M, N, K, epi);
    else hipLaunchKernelGGL((gemm_wxa16_skinny_kernel<BITS, 4>), grid, block, 0, st, x, wq, s, y, M, N, K, epi);
    return hipGetLastError();
}

hipError_t launch_gemm_wxa16(int bits, const half_t* x, const void* wq, const half_t* s, half_t* y, int M,
                             int N, int K, const Epi& epi, void*, size_t, hipStream_t st) {
    const uint8_t* w = static_cast<const uint8_t*>(wq);
    if (M <= 64)
        return bits == 8 ? launch_skinny<8>(x, w, s, y, M, N, K, epi, st) : launch_skinny<4>(x, w, s, y, M, N, K, epi, st);
    return launch_gemm_tiled(bits == 8 ? 1 : 2, x, wq, s, nullptr, y, M, N, K, epi, st);
}

}  // namespace aria
