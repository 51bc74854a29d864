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

// ---------------------------------------------------------------------------
// N % 8 == 0 (every layer of the DiT and 1.2B-scale shapes): W is read in
// 16-byte chunks of 8 channels, and the work spreads over a 2-D grid of
// tiles instead of one workgroup per 64 channels walking all of K (which
// left most CUs idle and read W with 2-byte loads).  Same arithmetic per
// value as the kernels above, so the packed bytes are identical.

// q8 step 1: s[n] = fp16(max_k |W[k][n]| / 127) for 64 channels per
// workgroup; thread (r, cg) keeps the running maxima of channels
// n0 + 8 cg .. + 7 over rows k = r, r + 32, ...  The magnitudes are the
// fp16 values with the sign bit cleared, compared as halfs (a NaN is
// skipped, as fmaxf does).
__global__ __launch_bounds__(256) void qpack8_scale_kernel(const half_t* __restrict__ w, int64_t K, int64_t N,
                                                           half_t* __restrict__ s) {
    __shared__ v8h red[32][8];
    const int64_t n0 = (int64_t)blockIdx.x * TILE_N;
    const int cg = threadIdx.x % 8, r = threadIdx.x / 8;
    const bool in = n0 + 8 * cg < N;
    const rsrc_t rw = make_rsrc(w, (uint32_t)(K * N * 2));
    v2h mx[4] = {};
    const int64_t nk = (K - r + 31) / 32;   // rows r, r + 32, ... below K
    for (int64_t j = 0; j < nk; j += 4) {
        v4u v[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int64_t k = r + 32 * (j + u);
            v[u] = __builtin_bit_cast(v4u, buf_load16(rw, in && j + u < nk ? (uint32_t)((k * N + n0 + 8 * cg) * 2) : OOB));
        }
#pragma unroll
        for (int u = 0; u < 4; u++)
#pragma unroll
            for (int d = 0; d < 4; d++)
                mx[d] = __builtin_elementwise_max(mx[d], __builtin_bit_cast(v2h, v[u][d] & 0x7FFF7FFFu));
    }
    red[r][cg] = v8h{mx[0][0], mx[0][1], mx[1][0], mx[1][1], mx[2][0], mx[2][1], mx[3][0], mx[3][1]};
    __syncthreads();
    if (threadIdx.x < TILE_N) {
        const int c = threadIdx.x;
        float a = 0.0f;
        for (int i = 0; i < 32; i++) a = fmaxf(a, (float)red[i][c / 8][c % 8]);
        if (n0 + c < N) s[n0 + c] = (half_t)(a / 127.0f);
    }
}

// q8 step 2: a 128 k x 64 n tile per workgroup: each thread quantizes 8
// channels of one k from a 16-byte load, the codes go through LDS as
// [n][k] bytes, and each channel's 128 k leave as 16-byte stores.
constexpr int Q8_TK = 128;
__global__ __launch_bounds__(256) void qpack8_tile_kernel(const half_t* __restrict__ w, int64_t K, int64_t N,
                                                          const half_t* __restrict__ s, int8_t* __restrict__ q) {
    __shared__ __attribute__((aligned(16))) int8_t t[TILE_N][Q8_TK + 16];
    const int64_t n0 = (int64_t)blockIdx.x * TILE_N, k0 = (int64_t)blockIdx.y * Q8_TK;
    const int cg = threadIdx.x % 8;
    const bool in = n0 + 8 * cg < N;
    const rsrc_t rw = make_rsrc(w, (uint32_t)(K * N * 2));
    const v8h sc = in ? *reinterpret_cast<const v8h*>(s + n0 + 8 * cg) : v8h{};
    v4u v[Q8_TK * 8 / 256];
#pragma unroll
    for (int u = 0; u < Q8_TK * 8 / 256; u++) {
        const int64_t k = k0 + threadIdx.x / 8 + 32 * u;
        v[u] = __builtin_bit_cast(v4u, buf_load16(rw, in && k < K ? (uint32_t)((k * N + n0 + 8 * cg) * 2) : OOB));
    }
#pragma unroll
    for (int u = 0; u < Q8_TK * 8 / 256; u++) {
        const int kr = threadIdx.x / 8 + 32 * u;
        const v8h x = __builtin_bit_cast(v8h, v[u]);
#pragma unroll
        for (int e = 0; e < 8; e++) t[8 * cg + e][kr] = quant_one((float)x[e], (float)sc[e], 127.0f);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < TILE_N * Q8_TK / 16 / 256; u++) {
        const int i = threadIdx.x + 256 * u, n = i / (Q8_TK / 16), seg = i % (Q8_TK / 16);
        const int64_t k = k0 + 16 * seg;
        if (n0 + n < N && k < K)   // K % 32 == 0: a 16-k segment is all in or all out
            *reinterpret_cast<v4i*>(q + (n0 + n) * K + k) = *reinterpret_cast<const v4i*>(&t[n][16 * seg]);
    }
}

// q4: one 64 k x 64 n tile (two groups of 32 k) per workgroup, loaded in
// 16-byte chunks; then as qpack4_kernel: threads 0..127 own one (channel,
// group) each.
__global__ __launch_bounds__(256) void qpack4_tile_kernel(const half_t* __restrict__ w, int64_t K, int64_t N,
                                                          uint8_t* __restrict__ q4, half_t* __restrict__ s) {
    constexpr int TS = TILE_N + 8;   // halfs per LDS row: 16-byte aligned rows
    __shared__ __attribute__((aligned(16))) half_t tile[TILE_K][TS];
    const int64_t n0 = (int64_t)blockIdx.x * TILE_N, k0 = (int64_t)blockIdx.y * TILE_K;
    const int64_t G = K / 32;
    const rsrc_t rw = make_rsrc(w, (uint32_t)(K * N * 2));
#pragma unroll
    for (int u = 0; u < TILE_K * 8 / 256; u++) {
        const int i = threadIdx.x + 256 * u, r = i / 8, cg = i % 8;
        const int64_t k = k0 + r;
        const bool in = n0 + 8 * cg < N && k < K;
        *reinterpret_cast<v4i*>(&tile[r][8 * cg]) = buf_load16(rw, in ? (uint32_t)((k * N + n0 + 8 * cg) * 2) : OOB);
    }
    __syncthreads();
    const int cn = threadIdx.x % TILE_N, g = threadIdx.x / TILE_N;
    const int64_t kb = k0 + g * 32;
    if (g < 2 && n0 + cn < N && kb < K) {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; i++) a = fmaxf(a, fabsf((float)tile[g * 32 + i][cn]));
        const half_t sh = (half_t)(a / 7.0f);
        const float sc = (float)sh;
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
    if (N % 8 == 0) {
        const unsigned nb = (unsigned)((N + TILE_N - 1) / TILE_N);
        hipLaunchKernelGGL(qpack8_scale_kernel, dim3(nb), dim3(256), 0, st, w, K, N, s);
        hipLaunchKernelGGL(qpack8_tile_kernel, dim3(nb, (unsigned)((K + Q8_TK - 1) / Q8_TK)), dim3(256), 0, st, w, K, N,
                           (const half_t*)s, q);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((N + TILE_N - 1) / TILE_N));
    hipLaunchKernelGGL(qpack8_kernel, grid, dim3(256), 0, st, w, K, N, q, s);
    return hipGetLastError();
}

hipError_t launch_qpack4(const half_t* w, int64_t K, int64_t N, uint8_t* q4, half_t* s, hipStream_t st) {
    if (N % 8 == 0) {
        dim3 grid((unsigned)((N + TILE_N - 1) / TILE_N), (unsigned)((K + TILE_K - 1) / TILE_K));
        hipLaunchKernelGGL(qpack4_tile_kernel, grid, dim3(256), 0, st, w, K, N, q4, s);
        return hipGetLastError();
    }
    dim3 grid((unsigned)((N + TILE_N - 1) / TILE_N));
    hipLaunchKernelGGL(qpack4_kernel, grid, dim3(256), 0, st, w, K, N, q4, s);
    return hipGetLastError();
}

}  // namespace aria
