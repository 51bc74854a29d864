// Register decoders for packed weights (shared by the tiled and skinny GEMMs).
// Both build fp16 bit patterns whose value is a fixed offset plus the unsigned
// code u (0x6400 | u = 1024 + u; for 4-bit codes also 0x5400 | u << 4 =
// 64 + u) and subtract the offset with packed-half arithmetic: exact for the
// integer, then (4-bit) one multiply by the group scale, which rounds once to
// fp16.
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
// fp16(q * s).  For the pair k = 2j, 2j+1 (byte j of a dword) a byte permute
// copies byte j into bytes 0 and 2; one three-input bit operation then keeps
// the low nibble in the low half and the high nibble at bits 4-7 of the high
// half, flips each nibble's top bit ((n ^ 8) = q + 8 = u) and sets the two
// exponents, so the low half reads 1024 + u (0x6400 | u: unit steps) and the
// high half 64 + u (0x5400 | u << 4: exponent 6, where mantissa bit 4 is
// worth 1).  One packed subtract of (1032, 72) leaves q exactly, one packed
// multiply by the group scale rounds once.  Four VALU ops per pair.
template <int ND = 4>
__device__ __forceinline__ void dec4(v4i w, v2h sc, v4i out[ND]) {
    const v2h bias = {(half_t)1032.0f, (half_t)72.0f};
#pragma unroll
    for (int d = 0; d < ND; d++) {
        const u32 u = (u32)w[d];
        u32 o[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            // selector bytes j, 0x0C (zero), j, 0x0C: the dword reads b_j, 0, b_j, 0
            const u32 b = __builtin_amdgcn_perm(0u, u, 0x0C000C00u | (u32)j | ((u32)j << 16));
            const u32 p = (b & 0x00F0000Fu) ^ 0x54806408u;
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
