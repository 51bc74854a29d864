// Internal launcher declarations (C++ linkage; the C-ABI lives in api.hip).
#pragma once

#include "common.h"

namespace aria {

hipError_t launch_qpack8(const half_t* w, int64_t K, int64_t N, int8_t* q, half_t* s, hipStream_t st);
hipError_t launch_qpack4(const half_t* w, int64_t K, int64_t N, uint8_t* q4, half_t* s, hipStream_t st);
// ldx: row stride of x in halves (0: K, rows contiguous)
hipError_t launch_actquant(const half_t* x, int64_t M, int64_t K, int8_t* xq, half_t* sa, hipStream_t st,
                           int64_t ldx = 0);
hipError_t launch_pack16(const half_t* w, int64_t K, int64_t N, half_t* wt, hipStream_t st);

// The DiT block's steps around the linears (layernorm.hip, attention.hip).
hipError_t launch_layernorm(const half_t* x, const half_t* gamma, const half_t* beta, float eps, int64_t M, int64_t W,
                            half_t* y, hipStream_t st);
// LayerNorm then per-token quantization of its fp16 output (y may be null).
hipError_t launch_layernorm_quant(const half_t* x, const half_t* gamma, const half_t* beta, float eps, int64_t M,
                                  int64_t W, half_t* y, int8_t* xq, half_t* sa, hipStream_t st);
hipError_t launch_attention(const half_t* qkv, int64_t M, int64_t W, int64_t H, int64_t S, half_t* out,
                            hipStream_t st);

// Per-token quantization inside the W8A8 contraction (mode 4): A is X fp16
// with row stride lda (halves); row m's scale comes from the row maxima a
// producing epilogue recorded (amax[m * amax_ld + j], j < K / 64, fp16
// magnitude bits); sa_out (or null) receives the scales.
struct AQuant {
    const uint32_t* amax;
    int amax_ld, lda;
    half_t* sa_out;
};

// Tiled contraction + epilogue for all modes (gemm_tiled.hip).  mode 0 = W8A8
// (a = Xq int8 [M][K], sa = per-token scales), 1 = W8A16, 2 = W4A16 (a = X fp16),
// 3 = W16A16, 4 = W8A8 quantizing a = X fp16 on the way in (aq required).
// With epi.rowmax set, only tiles whose waves are 64 columns wide are used.
hipError_t launch_gemm_tiled(int mode, const void* a, const void* bq, const half_t* s, const half_t* sa, half_t* y,
                             int M, int N, int K, const Epi& epi, hipStream_t st, const AQuant* aq = nullptr);

// Weight-only contraction + epilogue: A = X fp16 [M][K]; bits 8: B = Wq int8 [N][K] with
// per-channel scales s [N]; bits 4: B = Wq4 [N][K/2] with group scales s [N][K/32];
// bits 16: B = Wt fp16 [N][K], no scales.
// ws / ws_bytes: split-K partials for small M (may be null when not needed).
hipError_t launch_gemm_wxa16(int bits, const half_t* x, const void* wq, const half_t* s, half_t* y,
                             int M, int N, int K, const Epi& epi, void* ws, size_t ws_bytes,
                             hipStream_t st);
size_t wxa16_workspace_bytes(int bits, int64_t M, int64_t K, int64_t N);

// Grouped weight-only linears at small M (M <= 64): one launch for up to
// kSkinnyGroupMax problems, each problem's workgroups a slice of one grid.
// The problem table travels as the kernel argument (no device memory); the
// launcher fills in `first`.
constexpr int kSkinnyGroupMax = 32;
struct SkinnyProblem {
    const half_t* x;
    const uint8_t* w;
    const half_t* s;
    half_t* y;
    EpiW epi;
    int M, N, K;
    int first;  // first workgroup of this problem (set by the launcher)
};
struct SkinnyGroup {
    SkinnyProblem p[kSkinnyGroupMax];
    int count;
};
// the problem table is the kernel argument: keep it within 4 KB
static_assert(sizeof(SkinnyGroup) <= 4096, "grouped problem table exceeds 4 KB of kernel arguments");
hipError_t launch_skinny_grouped(int bits, SkinnyGroup& g, hipStream_t st);

}  // namespace aria
