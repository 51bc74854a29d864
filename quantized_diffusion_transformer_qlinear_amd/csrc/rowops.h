// Per-row building blocks shared by the row kernels (activation quantizer,
// LayerNorm, and the two fused): one wave owns one row held in registers as
// CH 16-byte chunks per lane (element c * 512 + lane * 8 + e of the row in
// v[c][e]), so that the same arithmetic, in the same order, gives the same
// bits whichever kernel runs it.
#pragma once

#include "common.h"

namespace aria {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, WAVE));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, WAVE);
    return v;
}

// Per-token quantization of one row (a2; aria project page, "Results": W8A8
// runs 8-bit arithmetic on integer matrix units):
//   s_a = fp16_RNE(max |x| / 127),  xq = clamp(RNE(x / s_a), -127, 127),
// stored with the non-temporal hint (xq through `rq`, bounds-checked, so the
// zero tail past the row end is dropped; s_a by lane 0 at sa[m]).
template <int CH>
__device__ __forceinline__ void quantize_row(const v8h (&v)[CH], int lane, int m, rsrc_t rq, half_t* __restrict__ sa) {
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

// LayerNorm of one row of W elements (Ba, Kiros, Hinton; the DiT block's
// pre-norms): mu = mean x, var = mean (x - mu)^2 (two passes over the
// registers: no cancellation), o = fp16((x - mu) / sqrt(var + eps) * gamma + beta).
template <int CH>
__device__ __forceinline__ void layernorm_row(const v8h (&v)[CH], int lane, int W, float eps, rsrc_t rg, rsrc_t rb,
                                              v8h (&o)[CH]) {
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; c++)
#pragma unroll
        for (int e = 0; e < 8; e++) s += (float)v[c][e];
    const float mu = wave_sum(s) / (float)W;
    float q = 0.0f;
#pragma unroll
    for (int c = 0; c < CH; c++)
#pragma unroll
        for (int e = 0; e < 8; e++) {
            // the zero-filled tail past W must not count: its centred value is -mu
            const float d = (c * 512 + lane * 8 + e < W) ? (float)v[c][e] - mu : 0.0f;
            q += d * d;
        }
    const float inv = 1.0f / sqrtf(wave_sum(q) / (float)W + eps);
#pragma unroll
    for (int c = 0; c < CH; c++) {
        const uint32_t off = (uint32_t)(c * 512 + lane * 8) * 2;
        const v8h g = __builtin_bit_cast(v8h, buf_load16(rg, off));
        const v8h b = __builtin_bit_cast(v8h, buf_load16(rb, off));
#pragma unroll
        for (int e = 0; e < 8; e++) o[c][e] = (half_t)(((float)v[c][e] - mu) * inv * (float)g[e] + (float)b[e]);
    }
}

}  // namespace aria
