// Per-row building blocks shared by the row kernels (activation quantizer,
// LayerNorm, and the two fused): one wave owns one row held in registers as
// CH 16-byte chunks per lane (element c * 512 + lane * 8 + e of the row in
// v[c][e]), so that the same arithmetic, in the same order, gives the same
// bits whichever kernel runs it.
#pragma once

#include "common.h"

namespace aria {

// The largest of the wave's 64 values (non-negative integers, e.g. fp16
// magnitude bits), wave-uniform: DPP steps inside each row of 16 lanes (quad
// swaps, then the half-row and row mirrors), then the four row results
// through scalar registers.  Cheaper in latency than a chain of six lane
// shuffles through LDS.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));    // lanes xor 1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));    // lanes xor 2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));   // half-row mirror
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));   // row mirror
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// The sum of the wave's 64 values, wave-uniform: the same DPP steps inside
// each 16-lane row (a lane and its partner add the same two values, so every
// lane of a row ends with the same bits), then (r0 + r1) + (r2 + r3) of the
// four row sums read into scalar registers.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
    v = dpp_add<0xB1>(v);    // lanes xor 1
    v = dpp_add<0x4E>(v);    // lanes xor 2
    v = dpp_add<0x141>(v);   // half-row mirror
    v = dpp_add<0x140>(v);   // row mirror
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return (r0 + r1) + (r2 + r3);
}

// Per-token quantization of one row (a2; aria project page, "Results": W8A8
// runs 8-bit arithmetic on integer matrix units):
//   s_a = fp16_RNE(max |x| / 127),  xq = clamp(RNE(x / s_a), -127, 127),
// stored with the non-temporal hint (xq through `rq`, bounds-checked, so the
// zero tail past the row end is dropped; s_a by lane 0 at sa[m]).
template <int CH>
__device__ __forceinline__ void quantize_row(const v8h (&v)[CH], int lane, int m, rsrc_t rq, half_t* __restrict__ sa) {
    // max |x|: the fp16 magnitude bits order like the magnitudes, so an
    // integer max over (bits & 0x7FFF), two halves at a time, is exact
    typedef unsigned short v2us __attribute__((ext_vector_type(2)));
    v2us mx = {0, 0};
#pragma unroll
    for (int c = 0; c < CH; c++) {
        const v4u w = __builtin_bit_cast(v4u, v[c]);
#pragma unroll
        for (int d = 0; d < 4; d++) mx = __builtin_elementwise_max(mx, __builtin_bit_cast(v2us, w[d] & 0x7FFF7FFFu));
    }
    const uint32_t amax = wave_max_u32(mx[0] > mx[1] ? mx[0] : mx[1]);
    const float a = (float)__builtin_bit_cast(half_t, (uint16_t)amax);
    const half_t sh = (half_t)(a / 127.0f);
    const float s = (float)sh;
    const float sdiv = s == 0.0f ? 1.0f : s;  // an all-zero row quantizes to zeros either way
    const float rcp = 1.0f / sdiv;            // correctly rounded, once per row
    if (lane == 0) sa[m] = sh;
#pragma unroll
    for (int c = 0; c < CH; c++) {
        // rint(x / s) without a division per element: f = x * RN(1/s) is
        // within 127 * 2^-23 (~1.5e-5) of x / s, so rint(f) is rint(x / s)
        // unless f lies within 2^-15 of a half-integer; for fp16 x and s that
        // happens only at exact ties x = (k + 1/2) s, which are detected
        // exactly (the FMA residual of the candidate k + 1/2 is exact and
        // zero) and rounded from the exact half-integer, which rint sends to
        // the even side.  The tie test runs only for chunks where some lane
        // of the wave is near a half-integer.  Checked on the host against
        // rint(x / s) in fp32 for every fp16 row maximum and every |x| <= it
        // (1.0e9 pairs, 0 differ).  The near test takes the largest
        // |f - q| of the lane's 8 values (one max3 per two values instead of
        // a compare, a select and bit packing per value: the pass is bound
        // by its VALU work once the row is in registers).
        float f[8], q[8];
        float dmax = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            // x * RN(1/s) as an FMA with a +0 addend, so the fp16 -> fp32
            // conversion folds into it (v_fma_mix); it differs from the
            // product only by giving +0 for -0, which quantizes the same
            f[e] = __builtin_fmaf((float)v[c][e], rcp, 0.0f);
            q[e] = __builtin_rintf(f[e]);
            dmax = __builtin_fmaxf(dmax, __builtin_fabsf(f[e] - q[e]));
        }
        if (__builtin_amdgcn_ballot_w64(dmax >= 0.5f - 0x1p-15f) != 0) {
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const float xv = (float)v[c][e];
                const float qf = __builtin_floorf(f[e]) + 0.5f;
                q[e] = __builtin_rintf(__builtin_fmaf(qf, sdiv, -xv) == 0.0f ? qf : f[e]);
            }
        }
        u32 w[2];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            u32 b[4];
#pragma unroll
            // clamp to +-127 (med3: q is never a signalling NaN, so no
            // canonicalising max is needed), then the integer code
            for (int e = 0; e < 4; e++) b[e] = (u32)(int)__builtin_amdgcn_fmed3f(q[4 * h + e], -127.0f, 127.0f);
            // low bytes of the four codes, in order
            w[h] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[3], b[2], 0x0C0C0400u),
                                         __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u), 0x05040100u);
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
