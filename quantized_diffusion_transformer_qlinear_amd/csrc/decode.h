// Register decoders for packed weights (shared by the tiled and skinny GEMMs).
// Both build the fp16 bit pattern 0x6400 | u, whose value is 1024 + u for an
// integer u in [0, 1023], and subtract the bias with packed-half arithmetic:
// exact for the integer, then (4-bit) one multiply by the group scale, which
// rounds once to fp16.
#pragma once

#include "common.h"

namespace aria {

// 16 int8 (4 dwords) -> 16 fp16, exact: (b ^ 0x80) = q + 128 -> fp16(0x6400 | u) - 1152.
__device__ __forceinline__ void dec8(v4i w, v4i& lo, v4i& hi) {
    const v2h bias = {(half_t)1152.0f, (half_t)1152.0f};
    u32 o[8];
#pragma unroll
    for (int d = 0; d < 4; d++) {
        const u32 u = (u32)w[d] ^ 0x80808080u;
        const u32 p0 = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);  // bytes: u0, 64, u1, 64
        const u32 p1 = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);  // bytes: u2, 64, u3, 64
        v2h h0 = __builtin_bit_cast(v2h, p0) - bias;
        v2h h1 = __builtin_bit_cast(v2h, p1) - bias;
        o[2 * d] = __builtin_bit_cast(u32, h0);
        o[2 * d + 1] = __builtin_bit_cast(u32, h1);
    }
    lo = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
    hi = v4i{(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
}

// 8 ND nibbles (ND dwords; even k in the low nibble) -> 8 ND fp16 values
// fp16(q * s): (n ^ 8) = q + 8 -> fp16(0x6400 | u) - 1032 = q (exact) -> times s
// (one rounding).  `sc` holds the group scale in both halves.
template <int ND = 4>
__device__ __forceinline__ void dec4(v4i w, v2h sc, v4i out[ND]) {
    const v2h bias = {(half_t)1032.0f, (half_t)1032.0f};
#pragma unroll
    for (int d = 0; d < ND; d++) {
        const u32 u = (u32)w[d] ^ 0x88888888u;
        const u32 t0 = u & 0x0F0F0F0Fu;          // bytes: k0 k2 k4 k6
        const u32 t1 = (u >> 4) & 0x0F0F0F0Fu;   // bytes: k1 k3 k5 k7
        u32 o[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            // k = 2j (byte j of t0) in the low half, k = 2j+1 (byte j of t1) in the high half
            const u32 sel = 0x0C000C00u | (u32)j | ((u32)(4 + j) << 16);
            const u32 p = __builtin_amdgcn_perm(t1, t0, sel) | 0x64006400u;
            v2h h = (__builtin_bit_cast(v2h, p) - bias) * sc;
            o[j] = __builtin_bit_cast(u32, h);
        }
        out[d] = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
    }
}
template <int ND = 4>
__device__ __forceinline__ void dec4(v4i w, half_t s, v4i out[ND]) { dec4<ND>(w, v2h{s, s}, out); }
// ... with the scale given as its 16 bits in the low half of a dword (as a
// 16-bit buffer load returns it): kept in a dword, a scale array stays in
// registers.
__device__ __forceinline__ void dec4_bits(v4i w, u32 sbits, v4i out[4]) {
    dec4(w, __builtin_bit_cast(v2h, (sbits & 0xFFFFu) * 0x10001u), out);
}

}  // namespace aria
