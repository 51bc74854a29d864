// The DiT block's pre-norms (docshare paper page, Fig. 1 "DiT blocks"):
// LayerNorm over each token row of x fp16 [M][W] (Ba, Kiros, Hinton):
//   mu = mean x,  var = mean (x - mu)^2,  y = (x - mu) / sqrt(var + eps) * gamma + beta
// in fp32, rounded to fp16 once.  One wave per row, the row held in registers
// (W <= 16384): every 16-byte load of the row is issued before any use
// (bounds-checked buffer loads, so the tail reads zero without a branch);
// two passes over the registers (mean, then centred variance); wave-wide sums
// by lane shuffles; 16-byte stores.
#include "common.h"
#include "kernels.h"
#include "rowops.h"

namespace aria {

template <int CH>  // CH 16-byte chunks per lane (W <= CH * 512)
__global__ __launch_bounds__(256) void layernorm_kernel(const half_t* __restrict__ x, const half_t* __restrict__ gamma,
                                                        const half_t* __restrict__ beta, float eps, int M, int W,
                                                        half_t* __restrict__ y) {
    const int lane = threadIdx.x % WAVE;
    const int m = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE);
    if (m >= M) return;
    const rsrc_t rx = make_rsrc(x + (int64_t)m * W, (uint32_t)W * 2);
    v8h v[CH], o[CH];
#pragma unroll
    for (int c = 0; c < CH; c++) v[c] = __builtin_bit_cast(v8h, buf_load16(rx, (uint32_t)(c * 512 + lane * 8) * 2));
    layernorm_row<CH>(v, lane, W, eps, make_rsrc(gamma, (uint32_t)W * 2), make_rsrc(beta, (uint32_t)W * 2), o);
    const rsrc_t ry = make_rsrc(y + (int64_t)m * W, (uint32_t)W * 2);
#pragma unroll
    for (int c = 0; c < CH; c++)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, o[c]), ry, (int)(c * 512 + lane * 8) * 2, 0, 0);
}

// LayerNorm followed by the per-token quantization of its fp16 output, the
// row never leaving registers: the pre-norm of a W8A8 linear in one pass.
// The same row functions as the two separate kernels, so xq / s_a (and y,
// when asked for) are bit-identical to layernorm then actquant.
template <int CH>
__global__ __launch_bounds__(256) void layernorm_quant_kernel(const half_t* __restrict__ x,
                                                              const half_t* __restrict__ gamma,
                                                              const half_t* __restrict__ beta, float eps, int M, int W,
                                                              half_t* __restrict__ y, int8_t* __restrict__ xq,
                                                              half_t* __restrict__ sa) {
    const int lane = threadIdx.x % WAVE;
    const int m = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE);
    if (m >= M) return;
    const rsrc_t rx = make_rsrc(x + (int64_t)m * W, (uint32_t)W * 2);
    v8h v[CH], o[CH];
#pragma unroll
    for (int c = 0; c < CH; c++) v[c] = __builtin_bit_cast(v8h, buf_load16(rx, (uint32_t)(c * 512 + lane * 8) * 2));
    layernorm_row<CH>(v, lane, W, eps, make_rsrc(gamma, (uint32_t)W * 2), make_rsrc(beta, (uint32_t)W * 2), o);
    if (y) {
        const rsrc_t ry = make_rsrc(y + (int64_t)m * W, (uint32_t)W * 2);
#pragma unroll
        for (int c = 0; c < CH; c++)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, o[c]), ry, (int)(c * 512 + lane * 8) * 2, 0, 0);
    }
    quantize_row<CH>(o, lane, m, make_rsrc(xq + (int64_t)m * W, (uint32_t)W), sa);
}

hipError_t launch_layernorm(const half_t* x, const half_t* gamma, const half_t* beta, float eps, int64_t M, int64_t W,
                            half_t* y, hipStream_t st) {
    const int rows_per_block = 4;
    dim3 grid((unsigned)((M + rows_per_block - 1) / rows_per_block)), block(rows_per_block * WAVE);
    const int64_t ch = (W + 511) / 512;
    const int m = (int)M, w = (int)W;
#define ARIA_LN(C) hipLaunchKernelGGL(layernorm_kernel<C>, grid, block, 0, st, x, gamma, beta, eps, m, w, y)
    if (ch <= 1) ARIA_LN(1);
    else if (ch <= 2) ARIA_LN(2);
    else if (ch <= 3) ARIA_LN(3);
    else if (ch <= 4) ARIA_LN(4);
    else if (ch <= 6) ARIA_LN(6);
    else if (ch <= 8) ARIA_LN(8);
    else if (ch <= 12) ARIA_LN(12);
    else if (ch <= 16) ARIA_LN(16);
    else if (ch <= 32) ARIA_LN(32);
    else return hipErrorInvalidValue;  // W > 16384: rejected on the host before this point
#undef ARIA_LN
    return hipGetLastError();
}

hipError_t launch_layernorm_quant(const half_t* x, const half_t* gamma, const half_t* beta, float eps, int64_t M,
                                  int64_t W, half_t* y, int8_t* xq, half_t* sa, hipStream_t st) {
    const int rows_per_block = 4;
    dim3 grid((unsigned)((M + rows_per_block - 1) / rows_per_block)), block(rows_per_block * WAVE);
    const int64_t ch = (W + 511) / 512;
    const int m = (int)M, w = (int)W;
#define ARIA_LNQ(C) hipLaunchKernelGGL(layernorm_quant_kernel<C>, grid, block, 0, st, x, gamma, beta, eps, m, w, y, xq, sa)
    if (ch <= 1) ARIA_LNQ(1);
    else if (ch <= 2) ARIA_LNQ(2);
    else if (ch <= 3) ARIA_LNQ(3);
    else if (ch <= 4) ARIA_LNQ(4);
    else if (ch <= 6) ARIA_LNQ(6);
    else if (ch <= 8) ARIA_LNQ(8);
    else if (ch <= 12) ARIA_LNQ(12);
    else if (ch <= 16) ARIA_LNQ(16);
    else if (ch <= 32) ARIA_LNQ(32);
    else return hipErrorInvalidValue;  // W > 16384: rejected on the host before this point
#undef ARIA_LNQ
    return hipGetLastError();
}

}  // namespace aria
