// a1 — weight packing kernels (one-off, at load time).
//
// The aria project page ("What aria is", bullet "Quantization that saves
// memory") packs the transformer weights from fp16 down to 8 or 4 bits and
// releases the fp16 copy.  Symmetric absmax quantization with an fp16 scale:
//   s = fp16_RNE(max|v| / qmax),  q = clamp(RNE(v / s), -qmax, qmax),  s == 0 -> q = 0
// q8 : per output channel n over all K, qmax 127 -> Wq int8 [N][K], s [N]
// q4 : per (n, group of 32 k), qmax 7 -> two's-complement nibbles,
//      Wq4 uint8 [N][K/2], s [N][K/32]: each 32-bit word of a row holds eight
//      consecutive k, the even ones in the nibbles of its low half-word and
//      the odd ones in those of its high half-word (decode.h reads a (k, k+1)
//      pair out of the word with one mask)
//
// Bit-exactness with the fp64 definition: the scale is formed as an IEEE fp32
// quotient rounded to fp16 (equal to rounding the exact quotient, because fp32
// carries more than twice fp16's precision), and q uses an IEEE fp32 division
// followed by round-to-nearest-even (v_rndne_f32): the quotient of two fp16
// values is either exactly a half-integer or at least 2^-12 (relative) away
// from one, far beyond fp32's division error.  The library is therefore built
// without fast-math and with correctly rounded fp32 division.
#include "common.h"
#include "kernels.h"

namespace aria {

namespace {

constexpr int TILE_N = 64;  // output channels per workgroup
constexpr int TILE_K = 64;  // k rows per LDS tile
constexpr int LDS_STRIDE = TILE_N + 2;  // halfs; the +2 spreads column reads over banks

__device__ __forceinline__ int8_t quant_one(float v, float s, float qmax) {
    if (s == 0.0f) return 0;
    float r = __builtin_rintf(v / s);
    r = fminf(fmaxf(r, -qmax), qmax);
    return (int8_t)(int)r;
}

// Load a TILE_K x TILE_N tile of W (rows k0.., columns n0..) into LDS, zero outside.
__device__ __forceinline__ void load_tile(half_t (*tile)[LDS_STRIDE], const half_t* __restrict__ w,
                                          int64_t K, int64_t N, int64_t k0, int64_t n0) {
    for (int i = threadIdx.x; i < TILE_K * TILE_N; i += blockDim.x) {
        int r = i / TILE_N, c = i % TILE_N;
        int64_t k = k0 + r, n = n0 + c;
        tile[r][c] = (k < K && n < N) ? w[k * N + n] : (half_t)0.0f;
    }
}

}  // namespace

// q8: one workgroup per 64 output channels.  Pass 1 reduces max|w| per channel
// (coalesced along N), pass 2 quantizes 64x64 tiles through LDS and writes each
// channel's row of Wq contiguously along K (16 bytes per thread).
__global__ __launch_bounds__(256) void qpack8_kernel(const half_t* __restrict__ w, int64_t K, int64_t N,
                                                     int8_t* __restrict__ q, half_t* __restrict__ s) {
    __shared__ float red[4][TILE_N];
    __shared__ float scale[TILE_N];
    __shared__ half_t tile[TILE_K][LDS_STRIDE];
    const int64_t n0 = (int64_t)blockIdx.x * TILE_N;
    const int c = threadIdx.x % TILE_N, r = threadIdx.x / TILE_N;

    float a = 0.0f;
    if (n0 + c < N)
        for (int64_t k = r; k < K; k += 4) a = fmaxf(a, fabsf((float)w[k * N + n0 + c]));
    red[r][c] = a;
    __syncthreads();
    if (r == 0) {
        a = fmaxf(fmaxf(red[0][c], red[1][c]), fmaxf(red[2][c], red[3][c]));
        half_t sh = (half_t)(a / 127.0f);
        scale[c] = (float)sh;
        if (n0 + c < N) s[n0 + c] = sh;
    }
    __syncthreads();

    // thread -> (channel cn, 16-k segment seg) of the tile
    const int cn = threadIdx.x / 4, seg = threadIdx.x % 4;
    for (int64_t k0 = 0; k0 < K; k0 += TILE_K) {
        load_tile(tile, w, K, N, k0, n0);
        __syncthreads();
        const int64_t kb = k0 + seg * 16;
        if (n0 + cn < N && kb < K) {  // K % 32 == 0, so a 16-k segment is all in or all out
            const float sc = scale[cn];
            union { int8_t b[16]; v4i v; } out;
#pragma unroll
            for (int i = 0; i < 16; i++) out.b[i] = quant_one((float)tile[seg * 16 + i][cn], sc, 127.0f);
            *reinterpret_cast<v4i*>(q + (n0 + cn) * K + kb) = out.v;
        }
        __syncthreads();
    }
}

// q4: one workgroup per 64 output channels; each 64x64 tile holds two k-groups
// of 32; threads 0..127 own one (channel, group) each: absmax over 32 values,
// scale, quantize, and one 16-byte store of 32 nibbles.
__global__ __launch_bounds__(256) void qpack4_kernel(const half_t* __restrict__ w, int64_t K, int64_t N,
                                                     uint8_t* __restrict__ q4, half_t* __restrict__ s) {
    __shared__ half_t tile[TILE_K][LDS_STRIDE];
    const int64_t n0 = (int64_t)blockIdx.x * TILE_N;
    const int64_t G = K / 32;
    const int cn = threadIdx.x % TILE_N, g = threadIdx.x / TILE_N;  // g in 0..3, only 0..1 work
    for (int64_t k0 = 0; k0 < K; k0 += TILE_K) {
        load_tile(tile, w, K, N, k0, n0);
        __syncthreads();
        const int64_t kb = k0 + g * 32;
        if (g < 2 && n0 + cn < N && kb < K) {
            float a = 0.0f;
#pragma unroll
            for (int i = 0; i < 32; i++) a = fmaxf(a, fabsf((float)tile[g * 32 + i][cn]));
            half_t sh = (half_t)(a / 7.0f);
            const float sc = (float)sh;
            // word d of the group's 16 bytes holds k = 8d .. 8d + 7: the even
            // k in the nibbles of its low half-word, the odd k in its high one
            union { uint32_t w[4]; v4i v; } out;
#pragma unroll
            for (int d = 0; d < 4; d++) {
                uint32_t wd = 0;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int ev = quant_one((float)tile[g * 32 + 8 * d + 2 * i][cn], sc, 7.0f);
                    const int od = quant_one((float)tile[g * 32 + 8 * d + 2 * i + 1][cn], sc, 7.0f);
                    wd |= ((uint32_t)ev & 0xFu) << (4 * i);
                    wd |= ((uint32_t)od & 0xFu) << (16 + 4 * i);
                }
                out.w[d] = wd;
            }
            *reinterpret_cast<v4i*>(q4 + (n0 + cn) * (K / 2) + kb / 2) = out.v;
            s[(n0 + cn) * G + kb / 32] = sh;
        }
        __syncthreads();
    }
}

// The fp16 rung keeps fp16 weights in the same K-contiguous row layout as the
// packed ones: Wt[n][k] = W[k][n], a transpose through a 64x64 LDS tile
// (coalesced 128-byte rows on both sides).
__global__ __launch_bounds__(256) void pack16_kernel(const half_t* __restrict__ w, int K, int N, half_t* __restrict__ wt) {
    __shared__ half_t t[64][65];
    const int k0 = blockIdx.y * 64, n0 = blockIdx.x * 64, c = threadIdx.x % 64;
    for (int r = threadIdx.x / 64; r < 64; r += 4) {
        const int k = k0 + r, n = n0 + c;
        t[r][c] = (k < K && n < N) ? w[(int64_t)k * N + n] : (half_t)0.0f;
    }
    __syncthreads();
    for (int r = threadIdx.x / 64; r < 64; r += 4) {
        const int n = n0 + r, k = k0 + c;
        if (n < N && k < K) wt[(int64_t)n * K + k] = t[c][r];
    }
}

hipError_t launch_pack16(const half_t* w, int64_t K, int64_t N, half_t* wt, hipStream_t st) {
    dim3 grid((unsigned)((N + 63) / 64), (unsigned)((K + 63) / 64));
    hipLaunchKernelGGL(pack16_kernel, grid, dim3(256), 0, st, w, (int)K, (int)N, wt);
    return hipGetLastError();
}

hipError_t launch_qpack8(const half_t* w, int64_t K, int64_t N, int8_t* q, half_t* s, hipStream_t st) {
    dim3 grid((unsigned)((N + TILE_N - 1) / TILE_N));
    hipLaunchKernelGGL(qpack8_kernel, grid, dim3(256), 0, st, w, K, N, q, s);
    return hipGetLastError();
}

hipError_t launch_qpack4(const half_t* w, int64_t K, int64_t N, uint8_t* q4, half_t* s, hipStream_t st) {
    dim3 grid((unsigned)((N + TILE_N - 1) / TILE_N));
    hipLaunchKernelGGL(qpack4_kernel, grid, dim3(256), 0, st, w, K, N, q4, s);
    return hipGetLastError();
}

}  // namespace aria
