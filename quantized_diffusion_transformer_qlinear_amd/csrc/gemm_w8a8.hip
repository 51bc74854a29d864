// a4+a5 — W8A8 contraction on the int8 matrix cores, with the fused epilogue.
//
// The aria project page ("Results", table "Quantization is close to free at
// 8-bit") runs W8A8 as 8-bit arithmetic on integer matrix units; it is the
// fastest GPU mode there.  Here:
//   acc[m][n] = sum_k Xq[m][k] * Wq[n][k]           (exact, int32)
//   y[m][n]   = epilogue(acc * s_a[m] * s_w[n])      (fp32, one fp16 rounding)
// Both operands are K-contiguous (Xq [M][K], Wq [N][K]), which is the layout an
// MFMA operand fragment wants: each lane holds 16 consecutive k of one row.
//
// Tiling (gfx950): a workgroup of WM x WN waves owns a BM x BN output tile and
// walks K in BK-byte steps through double-buffered LDS; each wave owns a
// (BM/WM) x (BN/WN) sub-tile of 32x32 blocks computed with
// v_mfma_i32_32x32x32_i8.  Global loads are 16 bytes per lane; the next K-step
// is fetched into registers while the current one is multiplied.
#include "common.h"
#include "kernels.h"

namespace aria {

namespace {

template <int BM, int BN, int BK, int WM, int WN>
struct W8A8Cfg {
    static constexpr int NT = WM * WN * WAVE;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    static constexpr int LDK = BK + 16;  // bytes per LDS row; the pad staggers rows over banks
    static constexpr int CPR = BK / 16;  // 16-byte chunks per row
    static constexpr int LA = BM * CPR / NT, LB = BN * CPR / NT;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be 32x32 blocks");
    static_assert((BM * CPR) % NT == 0 && (BN * CPR) % NT == 0, "tile loads must split evenly");
    static_assert(BK % 32 == 0, "BK must be a multiple of the MFMA K");
};

}  // namespace

template <int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__(WM * WN * WAVE) void gemm_w8a8_kernel(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, const half_t* __restrict__ sa,
    const half_t* __restrict__ sw, half_t* Y, int M, int N, int K, Epi epi) {
    using C = W8A8Cfg<BM, BN, BK, WM, WN>;
    __shared__ __attribute__((aligned(16))) int8_t As[2][BM * C::LDK];
    __shared__ __attribute__((aligned(16))) int8_t Bs[2][BN * C::LDK];

    const int ntm = (M + BM - 1) / BM;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int tm = bid % ntm, tn = bid / ntm;  // consecutive ids share a weight column block
    const int m0 = tm * BM, n0 = tn * BN;
    const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
    const int wm = wave / WN, wn = wave % WN;

    v16i acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; i++)
#pragma unroll
        for (int j = 0; j < C::FN; j++) acc[i][j] = v16i{};

    v4i ra[C::LA], rb[C::LB];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < C::LA; i++) {
            const int c = threadIdx.x + i * C::NT, row = c / C::CPR, k = k0 + (c % C::CPR) * 16;
            const int gm = min(m0 + row, M - 1);
            ra[i] = (k < K) ? *reinterpret_cast<const v4i*>(A + (int64_t)gm * K + k) : v4i{};
        }
#pragma unroll
        for (int i = 0; i < C::LB; i++) {
            const int c = threadIdx.x + i * C::NT, row = c / C::CPR, k = k0 + (c % C::CPR) * 16;
            const int gn = min(n0 + row, N - 1);
            rb[i] = (k < K) ? *reinterpret_cast<const v4i*>(B + (int64_t)gn * K + k) : v4i{};
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < C::LA; i++) {
            const int c = threadIdx.x + i * C::NT;
            *reinterpret_cast<v4i*>(&As[buf][(c / C::CPR) * C::LDK + (c % C::CPR) * 16]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < C::LB; i++) {
            const int c = threadIdx.x + i * C::NT;
            *reinterpret_cast<v4i*>(&Bs[buf][(c / C::CPR) * C::LDK + (c % C::CPR) * 16]) = rb[i];
        }
    };

    const int nk = (K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < BK / 32; kk++) {
            v4i a[C::FM], b[C::FN];
            const int koff = kk * 32 + (lane / 32) * 16;
#pragma unroll
            for (int i = 0; i < C::FM; i++)
                a[i] = *reinterpret_cast<const v4i*>(&As[buf][(wm * C::WTM + i * 32 + lane % 32) * C::LDK + koff]);
#pragma unroll
            for (int j = 0; j < C::FN; j++)
                b[j] = *reinterpret_cast<const v4i*>(&Bs[buf][(wn * C::WTN + j * 32 + lane % 32) * C::LDK + koff]);
#pragma unroll
            for (int i = 0; i < C::FM; i++)
#pragma unroll
                for (int j = 0; j < C::FN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

    // epilogue: 32x32 block layout — register r of lane l holds
    // row 8*(r/4) + 4*(l/32) + r%4, column l%32
    const float alpha = load_alpha(epi);
#pragma unroll
    for (int i = 0; i < C::FM; i++)
#pragma unroll
        for (int j = 0; j < C::FN; j++) {
            const int col = n0 + wn * C::WTN + j * 32 + lane % 32;
            if (col >= N) continue;
            const float swc = (float)sw[col];
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int row = m0 + wm * C::WTM + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
                if (row >= M) continue;
                const int64_t idx = (int64_t)row * N + col;
                const int32_t iv = acc[i][j][r];
                if (epi.acc_out) epi.acc_out[idx] = iv;
                float v = (float)iv * (float)sa[row] * swc;
                Y[idx] = (half_t)epilogue_apply(v, idx, col, epi, alpha);
            }
        }
}

hipError_t launch_gemm_w8a8(const int8_t* xq, const int8_t* wq, const half_t* sa, const half_t* sw,
                            half_t* y, int M, int N, int K, const Epi& epi, hipStream_t st) {
    constexpr int BM = 128, BN = 128, BK = 128, WM = 2, WN = 2;
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    hipLaunchKernelGGL((gemm_w8a8_kernel<BM, BN, BK, WM, WN>), dim3(tiles), dim3(WM * WN * WAVE), 0, st,
                       xq, wq, sa, sw, y, M, N, K, epi);
    return hipGetLastError();
}

}  // namespace aria
