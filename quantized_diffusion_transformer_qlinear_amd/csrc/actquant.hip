// a2 — per-token dynamic activation quantization for W8A8.
//
// The aria project page ("Results", table "Quantization is close to free at
// 8-bit") runs W8A8 as 8-bit arithmetic on integer matrix units, so the fp16
// activations are quantized per token (row) on the fly:
//   s_a[m] = fp16_RNE(max_k |x[m][k]| / 127),  xq[m][k] = clamp(RNE(x / s_a), -127, 127)
// bit-exact with the fp64 definition (the quotient is rounded through a
// per-row reciprocal with an exact tie test, which gives the same integers as
// an IEEE fp32 division; see below).  One wave per token row: every 16-byte load of
// the row is issued before any is used (bounds-checked buffer loads, so the
// K tail reads zeros without a branch), an in-register absmax, a cross-lane
// max, then 8-byte int8 stores with the non-temporal hint (out-of-range stores
// are dropped by the buffer range check; the hint measured +2 % on the W8A8
// 1.2B-scale step, although the next GEMM reads these bytes).
#include "common.h"
#include "kernels.h"

namespace aria {

namespace {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, WAVE));
    return v;
}

}  // namespace

template <int CH>  // CH 16-byte chunks per lane kept in registers (K <= CH * 512)
__global__ __launch_bounds__(256) void actquant_kernel(const half_t* __restrict__ x, int M, int K,
                                                       int8_t* __restrict__ xq, half_t* __restrict__ sa) {
    const int lane = threadIdx.x % WAVE;
    // the row is uniform over the wave; saying so keeps the buffer descriptors
    // in scalar registers (no per-lane waterfall around each load)
    const int m = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE);
    if (m >= M) return;
    const rsrc_t rx = make_rsrc(x + (int64_t)m * K, (uint32_t)K * 2);
    const rsrc_t rq = make_rsrc(xq + (int64_t)m * K, (uint32_t)K);
    v8h v[CH];
#pragma unroll
    for (int c = 0; c < CH; c++) v[c] = __builtin_bit_cast(v8h, buf_load16(rx, (uint32_t)(c * 512 + lane * 8) * 2));
    float a = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; c++)
#pragma unroll
        for (int e = 0; e < 8; e++) a = fmaxf(a, fabsf((float)v[c][e]));
    a = wave_max(a);
    const half_t sh = (half_t)(a / 127.0f);
    const float s = (float)sh;
    const float sdiv = s == 0.0f ? 1.0f : s;  // an all-zero row quantizes to zeros either way
    const float rcp = 1.0f / sdiv;            // correctly rounded, once per row
    if (lane == 0) sa[m] = sh;
#pragma unroll
    for (int c = 0; c < CH; c++) {
        u32 w[2];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            u32 packed = 0;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                // rint(x / s) without a division per element: x * RN(1/s)
                // is within 2^-23 relative of x / s, and for fp16 x and s a
                // quotient that is not exactly k + 1/2 lies at least ~3e-5
                // from one, so rint(x * RN(1/s)) agrees except at exact ties;
                // a tie x = (k + 1/2) s is detected exactly (the FMA residual
                // of the candidate k + 1/2 is exact and zero) and rounded from
                // the exact half-integer, which rint sends to the even side.
                // Checked on the host against rint(x / s) in fp32 for every
                // fp16 row maximum and every |x| <= it (1.0e9 pairs, 0 differ).
                const float xv = (float)v[c][4 * h + e];
                const float f = xv * rcp;
                const float qf = __builtin_floorf(f) + 0.5f;
                float r = __builtin_rintf(__builtin_fmaf(qf, sdiv, -xv) == 0.0f ? qf : f);
                r = fminf(fmaxf(r, -127.0f), 127.0f);
                packed |= ((u32)(int)r & 0xFFu) << (8 * e);
            }
            w[h] = packed;
        }
        buf_store8_nt(v2u{w[0], w[1]}, rq, (uint32_t)(c * 512 + lane * 8));
    }
}

hipError_t launch_actquant(const half_t* x, int64_t M, int64_t K, int8_t* xq, half_t* sa, hipStream_t st) {
    const int rows_per_block = 4;
    dim3 grid((unsigned)((M + rows_per_block - 1) / rows_per_block)), block(rows_per_block * WAVE);
    const int64_t ch = (K + 511) / 512;
    const int m = (int)M, k = (int)K;
    if (ch <= 1) hipLaunchKernelGGL(actquant_kernel<1>, grid, block, 0, st, x, m, k, xq, sa);
    else if (ch <= 2) hipLaunchKernelGGL(actquant_kernel<2>, grid, block, 0, st, x, m, k, xq, sa);
    else if (ch <= 3) hipLaunchKernelGGL(actquant_kernel<3>, grid, block, 0, st, x, m, k, xq, sa);
    else if (ch <= 4) hipLaunchKernelGGL(actquant_kernel<4>, grid, block, 0, st, x, m, k, xq, sa);
    else if (ch <= 6) hipLaunchKernelGGL(actquant_kernel<6>, grid, block, 0, st, x, m, k, xq, sa);
    else if (ch <= 8) hipLaunchKernelGGL(actquant_kernel<8>, grid, block, 0, st, x, m, k, xq, sa);
    else if (ch <= 12) hipLaunchKernelGGL(actquant_kernel<12>, grid, block, 0, st, x, m, k, xq, sa);
    else if (ch <= 16) hipLaunchKernelGGL(actquant_kernel<16>, grid, block, 0, st, x, m, k, xq, sa);
    else if (ch <= 32) hipLaunchKernelGGL(actquant_kernel<32>, grid, block, 0, st, x, m, k, xq, sa);
    else return hipErrorInvalidValue;  // K > 16384: rejected on the host before this point
    return hipGetLastError();
}

}  // namespace aria
