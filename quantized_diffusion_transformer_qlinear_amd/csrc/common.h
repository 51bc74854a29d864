// Shared device helpers of the qlinear HIP library (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aria {

typedef _Float16 half_t;
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef uint32_t u32;
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// Epilogue operands as the kernels see them (already validated on the host).
struct Epi {
    const half_t* bias;      // [N] or null
    const half_t* residual;  // [M][N] or null (may alias y)
    const float* steer_dir;  // [N] or null
    const float* steer_alpha;  // device scalar or null
    int32_t* acc_out;        // W8A8 raw accumulators [M][N] or null
    int gelu;
    // optional: row maxima of the stored output for a later per-token
    // quantization of columns [rowmax_c0, rowmax_c1): rowmax[m * rowmax_ld + j]
    // = the largest fp16 magnitude bits over columns rowmax_c0 + 64 j .. + 63
    uint32_t* rowmax;
    int rowmax_ld, rowmax_c0, rowmax_c1;
};

// GELU, tanh form (Hendrycks & Gimpel): 0.5 y (1 + tanh(u)), u = sqrt(2/pi)(y + 0.044715 y^3).
// Uses 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)), with the hardware exp2 and reciprocal.
__device__ __forceinline__ float gelu_tanh(float y) {
    const float k2 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
    float u = y + 0.044715f * y * y * y;
    float e = __builtin_amdgcn_exp2f(k2 * u);
    return y * __builtin_amdgcn_rcpf(1.0f + e);
}

// Steering strength, read once per thread from device memory (0 if absent).
// The terms a weight-only linear of the grouped call takes (no raw
// accumulators, no row maxima): kept small because the grouped call's
// problem table travels as the kernel argument.
struct EpiW {
    const half_t* bias;
    const half_t* residual;
    const float* steer_dir;
    const float* steer_alpha;
    int gelu;
};

template <class E>
__device__ __forceinline__ float load_alpha(const E& e) {
    return (e.steer_dir && e.steer_alpha) ? __builtin_nontemporal_load(e.steer_alpha) : 0.0f;
}

// y (the dequantized accumulator) -> + bias -> GELU -> + residual -> + alpha d.
// `idx` is m * N + n.  E: Epi or EpiW.
template <class E>
__device__ __forceinline__ float epilogue_apply(float y, int64_t idx, int n, const E& e, float alpha) {
    if (e.bias) y += (float)e.bias[n];
    if (e.gelu) y = gelu_tanh(y);
    if (e.residual) y += (float)e.residual[idx];
    if (alpha != 0.0f) y += alpha * e.steer_dir[n];
    return y;
}

// Buffer resources: 32-bit offsets with hardware range checking; a load past
// num_records returns zero and a store past it is dropped, which keeps ragged
// edges branch-free.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t OOB = 0x80000000u;  // an offset past every buffer

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ v4i buf_load16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ v2u buf_load8(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ half_t buf_load_h(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(half_t, __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0));
}
// LDS-DMA: every lane's 16 bytes go straight from the buffer into LDS, lane l
// to lds_base + 16 l (`lds_base` is one address for the whole wave); an
// out-of-range lane writes zeros.  Counts as a vector memory load.
__device__ __forceinline__ void buf_load16_lds(rsrc_t r, uint32_t off, char* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, (int)off, 0, 0, 0);
}
// 8-byte store with the non-temporal cache policy (aux bit 1 = nt on gfx950):
// for outputs that the writing kernel never reads back.
__device__ __forceinline__ void buf_store8_nt(v2u v, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 2);
}

// XCD-aware remap of a linear workgroup id: the hardware deals workgroups
// round-robin over the 8 XCDs (id % 8); renumber so that consecutive logical
// ids land on the same XCD and therefore share its L2.
__device__ __forceinline__ int xcd_remap(int id, int total) {
    const int NX = 8;
    if (total % NX) return id;  // only exact multiples are remapped
    return (id % NX) * (total / NX) + id / NX;
}

}  // namespace aria
