// a2 — per-token dynamic activation quantization for W8A8.
//
// The aria project page ("Results", table "Quantization is close to free at
// 8-bit") runs W8A8 as 8-bit arithmetic on integer matrix units, so the fp16
// activations are quantized per token (row) on the fly:
//   s_a[m] = fp16_RNE(max_k |x[m][k]| / 127),  xq[m][k] = clamp(RNE(x / s_a), -127, 127)
// with the same fp32 route as the weight packer (bit-exact with the fp64
// definition; see qpack.hip).  One wave per token row: 16-byte loads along K,
// an in-register absmax, a cross-lane max, then 8-byte int8 stores.
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
__global__ __launch_bounds__(256) void actquant_kernel(const half_t* __restrict__ x, int64_t M, int64_t K,
                                                       int8_t* __restrict__ xq, half_t* __restrict__ sa) {
    const int lane = threadIdx.x % WAVE;
    const int64_t m = (int64_t)blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE;
    if (m >= M) return;
    const half_t* row = x + m * K;
    v8h v[CH];
    float a = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; c++) {
        const int64_t k = (int64_t)c * 512 + lane * 8;  // K % 32 == 0: a chunk is all in or all out
        if (k < K) {
            v[c] = *reinterpret_cast<const v8h*>(row + k);
#pragma unroll
            for (int e = 0; e < 8; e++) a = fmaxf(a, fabsf((float)v[c][e]));
        }
    }
    a = wave_max(a);
    const half_t sh = (half_t)(a / 127.0f);
    const float s = (float)sh;
    if (lane == 0) sa[m] = sh;
#pragma unroll
    for (int c = 0; c < CH; c++) {
        const int64_t k = (int64_t)c * 512 + lane * 8;
        if (k < K) {
            union { int8_t b[8]; uint2 u; } out;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                float r = (s == 0.0f) ? 0.0f : __builtin_rintf((float)v[c][e] / s);
                r = fminf(fmaxf(r, -127.0f), 127.0f);
                out.b[e] = (int8_t)(int)r;
            }
            *reinterpret_cast<uint2*>(xq + m * K + k) = out.u;
        }
    }
}

hipError_t launch_actquant(const half_t* x, int64_t M, int64_t K, int8_t* xq, half_t* sa, hipStream_t st) {
    const int rows_per_block = 4;
    dim3 grid((unsigned)((M + rows_per_block - 1) / rows_per_block)), block(rows_per_block * WAVE);
    const int64_t ch = (K + 511) / 512;
    if (ch <= 1) hipLaunchKernelGGL(actquant_kernel<1>, grid, block, 0, st, x, M, K, xq, sa);
    else if (ch <= 2) hipLaunchKernelGGL(actquant_kernel<2>, grid, block, 0, st, x, M, K, xq, sa);
    else if (ch <= 4) hipLaunchKernelGGL(actquant_kernel<4>, grid, block, 0, st, x, M, K, xq, sa);
    else if (ch <= 8) hipLaunchKernelGGL(actquant_kernel<8>, grid, block, 0, st, x, M, K, xq, sa);
    else if (ch <= 16) hipLaunchKernelGGL(actquant_kernel<16>, grid, block, 0, st, x, M, K, xq, sa);
    else if (ch <= 32) hipLaunchKernelGGL(actquant_kernel<32>, grid, block, 0, st, x, M, K, xq, sa);
    else return hipErrorInvalidValue;  // K > 16384: rejected on the host before this point
    return hipGetLastError();
}

}  // namespace aria
