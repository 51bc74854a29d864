// a2 — per-token dynamic activation quantization for W8A8.
//
// The aria project page ("Results", table "Quantization is close to free at
// 8-bit") runs W8A8 as 8-bit arithmetic on integer matrix units, so the fp16
// activations are quantized per token (row) on the fly:
//   s_a[m] = fp16_RNE(max_k |x[m][k]| / 127),  xq[m][k] = clamp(RNE(x / s_a), -127, 127)
// bit-exact with the fp64 definition (the quotient is rounded through a
// per-row reciprocal with an exact tie test, which gives the same integers as
// an IEEE fp32 division; see quantize_row in rowops.h).  One wave per token row: every 16-byte load of
// the row is issued before any is used (bounds-checked buffer loads, so the
// K tail reads zeros without a branch), an in-register absmax, a cross-lane
// max, then 8-byte int8 stores with the non-temporal hint (out-of-range stores
// are dropped by the buffer range check; the hint measured +2 % on the W8A8
// 1.2B-scale step, although the next GEMM reads these bytes).
#include "common.h"
#include "kernels.h"
#include "rowops.h"

namespace aria {

template <int CH>  // CH 16-byte chunks per lane kept in registers (K <= CH * 512)
__global__ __launch_bounds__(256) void actquant_kernel(const half_t* __restrict__ x, int64_t ldx, int M, int K,
                                                       int8_t* __restrict__ xq, half_t* __restrict__ sa) {
    const int lane = threadIdx.x % WAVE;
    // the row is uniform over the wave; saying so keeps the buffer descriptors
    // in scalar registers (no per-lane waterfall around each load)
    const int m = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE);
    if (m >= M) return;
    const rsrc_t rx = make_rsrc(x + (int64_t)m * ldx, (uint32_t)K * 2);   // row m: K halves at stride ldx
    const rsrc_t rq = make_rsrc(xq + (int64_t)m * K, (uint32_t)K);
    v8h v[CH];
#pragma unroll
    for (int c = 0; c < CH; c++) v[c] = __builtin_bit_cast(v8h, buf_load16(rx, (uint32_t)(c * 512 + lane * 8) * 2));
    quantize_row<CH>(v, lane, m, rq, sa);
}

hipError_t launch_actquant(const half_t* x, int64_t M, int64_t K, int8_t* xq, half_t* sa, hipStream_t st,
                           int64_t ldx) {
    if (ldx == 0) ldx = K;
    const int rows_per_block = 4;
    dim3 grid((unsigned)((M + rows_per_block - 1) / rows_per_block)), block(rows_per_block * WAVE);
    const int64_t ch = (K + 511) / 512;
    const int m = (int)M, k = (int)K;
    if (ch <= 1) hipLaunchKernelGGL(actquant_kernel<1>, grid, block, 0, st, x, ldx, m, k, xq, sa);
    else if (ch <= 2) hipLaunchKernelGGL(actquant_kernel<2>, grid, block, 0, st, x, ldx, m, k, xq, sa);
    else if (ch <= 3) hipLaunchKernelGGL(actquant_kernel<3>, grid, block, 0, st, x, ldx, m, k, xq, sa);
    else if (ch <= 4) hipLaunchKernelGGL(actquant_kernel<4>, grid, block, 0, st, x, ldx, m, k, xq, sa);
    else if (ch <= 6) hipLaunchKernelGGL(actquant_kernel<6>, grid, block, 0, st, x, ldx, m, k, xq, sa);
    else if (ch <= 8) hipLaunchKernelGGL(actquant_kernel<8>, grid, block, 0, st, x, ldx, m, k, xq, sa);
    else if (ch <= 12) hipLaunchKernelGGL(actquant_kernel<12>, grid, block, 0, st, x, ldx, m, k, xq, sa);
    else if (ch <= 16) hipLaunchKernelGGL(actquant_kernel<16>, grid, block, 0, st, x, ldx, m, k, xq, sa);
    else if (ch <= 32) hipLaunchKernelGGL(actquant_kernel<32>, grid, block, 0, st, x, ldx, m, k, xq, sa);
    else return hipErrorInvalidValue;  // K > 16384: rejected on the host before this point
    return hipGetLastError();
}

}  // namespace aria
