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

// 8 ND nibbles (ND dwords) -> 8 ND fp16 values fp16(q * s).  Dword d holds
// k = 8d .. 8d + 7: the even k in the four nibbles of its low half-word, the
// odd k in those of its high half-word.  So one three-input bit operation on
// the dword keeps the pair (k, k + 1) of one nibble position from both halves,
// flips each nibble's top bit ((n ^ 8) = q + 8 = u) and sets the exponents:
// nibble 0 (bits 0-3 / 16-19) reads 1024 + u (0x6400 | u: unit steps), nibble
// 1 (bits 4-7 / 20-23) reads 64 + u (0x5400 | u << 4: exponent 6, where
// mantissa bit 4 is worth 1); nibbles 2 and 3 the same after an 8-bit shift.
// One packed subtract of the offset leaves q exactly, one packed multiply by
// the group scale rounds once.  13 VALU ops per 8 values.
template <int ND = 4>
__device__ __forceinline__ void dec4(v4i w, v2h sc, v4i out[ND]) {
    const v2h b0 = {(half_t)1032.0f, (half_t)1032.0f}, b1 = {(half_t)72.0f, (half_t)72.0f};
#pragma unroll
    for (int d = 0; d < ND; d++) {
        const u32 u = (u32)w[d], u8 = u >> 8;
        const u32 p0 = (u & 0x000F000Fu) ^ 0x64086408u;    // k 8d + 0, 1
        const u32 p1 = (u & 0x00F000F0u) ^ 0x54805480u;    // k 8d + 2, 3
        const u32 p2 = (u8 & 0x000F000Fu) ^ 0x64086408u;   // k 8d + 4, 5
        const u32 p3 = (u8 & 0x00F000F0u) ^ 0x54805480u;   // k 8d + 6, 7
        const v2h h0 = (__builtin_bit_cast(v2h, p0) - b0) * sc;
        const v2h h1 = (__builtin_bit_cast(v2h, p1) - b1) * sc;
        const v2h h2 = (__builtin_bit_cast(v2h, p2) - b0) * sc;
        const v2h h3 = (__builtin_bit_cast(v2h, p3) - b1) * sc;
        out[d] = v4i{(int)__builtin_bit_cast(u32, h0), (int)__builtin_bit_cast(u32, h1), (int)__builtin_bit_cast(u32, h2),
                     (int)__builtin_bit_cast(u32, h3)};
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
