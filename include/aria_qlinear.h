/*
 * aria_qlinear.h — C-ABI of the quantized linear layer ("qlinear") of a
 * diffusion-transformer denoising step, for AMD Instinct MI355X (gfx950).
 *
 * What it computes follows the aria pages ("A Quantized Native Runtime for
 * On-Device Semantic Audio Generation"):
 *   - project page, "What aria is", bullet "Quantization that saves memory":
 *     transformer weights are packed once from fp16 down to 8 or 4 bits and the
 *     fp16 copy is released, so the packed form replaces the footprint;
 *   - project page, "Results", table "Quantization is close to free at 8-bit":
 *     three precisions of the linear layers — q8 (8-bit weights, fp16
 *     activations; here W8A16), W8A8 (8-bit arithmetic on integer matrix
 *     units; here int8 x int8 -> int32) and q4 (4-bit weights; here W4A16).
 *     q8 and W8A8 have the same memory, so both read ONE stored int8 format;
 *   - project page, "Results", "Steering is real, inside a narrow window" and
 *     "Live steering while streaming": a direction d is added with strength
 *     alpha to one block's residual stream, alpha = 0 removes it with
 *     bit-identical output, and alpha lives inside a captured graph (so it is
 *     read from device memory here).
 * The pages do not give the formulas; the library uses these readings:
 *   scale s = fp16_RNE(max|v| / qmax), q = clamp(RNE(v / s), -qmax, qmax);
 *   qmax 127 for 8 bits, 7 for 4 bits; weights per output channel (8-bit) or
 *   per (output channel, group of 32 consecutive k) (4-bit); activations per
 *   token (row); s == 0 gives q == 0; every scale is stored as fp16;
 *   epilogue order: dequantize -> + bias -> GELU(tanh) -> + residual -> + alpha*d.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE memory owned by the caller unless stated otherwise.
 *     The library allocates nothing and keeps no state between calls, except
 *     the fixed device scratch of aria_qlinear_w8a8_noalloc.
 *   - Calls only enqueue work on `stream` (a hipStream_t; NULL = null stream);
 *     they never synchronise and never read device memory on the host, so they
 *     may be captured into a HIP graph.
 *   - All argument checks run on the host before anything is launched; on an
 *     error nothing is launched and a negative aria_status is returned.  A
 *     failed launch returns ARIA_E_HIP.  Errors inside a kernel surface at the
 *     caller's next synchronisation.  Inputs must be finite.
 *   - Shapes: M tokens, K inputs, N outputs; 1 <= M <= 2^30,
 *     1 <= N <= 2^30, 32 <= K <= 16384, K % 32 == 0 and N * K < 2^31 (the
 *     packed weights of one layer are addressed with 32-bit offsets).  Every
 *     pointer must be 16-byte aligned.
 *   - Layouts (row-major):
 *       X   fp16 [M][K]            activations
 *       W   fp16 [K][N]            unpacked weights (input of aria_qpack only)
 *       Wq  int8 [N][K]            8-bit weights, row n contiguous along K
 *       s_w fp16 [N]               8-bit weight scales
 *       Wq4 uint8 [N][K/2]         4-bit weights, two's complement nibbles:
 *                                  the little-endian 32-bit word d of row n
 *                                  (bytes 4d .. 4d+3) holds k = 8d .. 8d+7,
 *                                  k = 8d+2i in bits 4i .. 4i+3 and
 *                                  k = 8d+2i+1 in bits 16+4i .. 16+4i+3
 *       s_g fp16 [N][K/32]         4-bit group scales, group g = k in [32g, 32g+32)
 *       Wt  fp16 [N][K]            fp16 weights (the unquantized rung), row n = column n of W
 *       Y   fp16 [M][N]            output
 */
#ifndef ARIA_QLINEAR_H
#define ARIA_QLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* aria_stream_t; /* a hipStream_t */

enum aria_status {
    ARIA_OK = 0,
    ARIA_E_NULL = -1,        /* a required pointer is NULL                         */
    ARIA_E_SHAPE = -2,       /* M, K or N out of range, or K % 32 != 0             */
    ARIA_E_ALIGN = -3,       /* a pointer is not 16-byte aligned                   */
    ARIA_E_UNSUPPORTED = -4, /* bits not in {4, 8, 16}, group not 0 (8, 16) / 32 (4), or an option the call lacks */
    ARIA_E_WORKSPACE = -5,   /* workspace missing or smaller than required         */
    ARIA_E_HIP = -6,         /* the HIP runtime reported an error at launch        */
    ARIA_E_ALIAS = -7,       /* an output overlaps an input or another output      */
    ARIA_E_SCRATCH = -8      /* the shape needs more than the fixed scratch of the
                                allocation-free call (ARIA_NOALLOC_SCRATCH_BYTES)   */
};

enum aria_mode { ARIA_W8A8 = 0, ARIA_W8A16 = 1, ARIA_W4A16 = 2, ARIA_W16A16 = 3 };

/* Human-readable name of a status code (static storage, never NULL). */
const char* aria_status_string(int status);

/* Library ABI version (increments on incompatible change). */
int aria_abi_version(void);

/* Host-only: bytes of the packed weights and of their scales.
 *   bits 8, group 0 : q = K*N, s = 2*N
 *   bits 4, group 32: q = K*N/2, s = 2*N*(K/32)
 *   bits 16, group 0: q = 2*K*N, s = 0 (the fp16 rung; needs K*N < 2^30)
 * q_bytes / s_bytes are host pointers. */
int aria_qpack_bytes(int bits, int group, int64_t K, int64_t N, size_t* q_bytes, size_t* s_bytes);

/* a1 — pack fp16 weights W [K][N] (project page, "What aria is": weights from
 * fp16 down to 8 or 4 bits).  bits 8 / group 0 -> Wq int8 [N][K] + s_w fp16 [N];
 * bits 4 / group 32 -> Wq4 uint8 [N][K/2] + s_g fp16 [N][K/32]; bits 16 /
 * group 0 -> Wt fp16 [N][K], the unquantized weights in the same row layout
 * (s_out unused, may be NULL).  q_out and s_out must hold aria_qpack_bytes()
 * bytes.  Once the call has completed on the stream the caller may free W:
 * nothing later reads it. */
int aria_qpack(int bits, int group, const void* w_f16, int64_t K, int64_t N,
               void* q_out, void* s_out, aria_stream_t stream);

/* a2 — per-token dynamic activation quantization used by W8A8 (project page,
 * "Results": W8A8 runs 8-bit arithmetic, so activations become int8 too):
 * X fp16 [M][K] -> Xq int8 [M][K] + s_a fp16 [M].  Exposed for testing and for
 * callers that quantize once and reuse. */
int aria_quant_act(const void* x_f16, int64_t M, int64_t K, int8_t* xq, void* s_a_f16,
                   aria_stream_t stream);

/* a2 with a row stride: row m of X is the K halves at x + m * ldx (ldx >= K,
 * ldx % 8 == 0), e.g. a column block of a wider activation such as the V third
 * of a QKV output, quantized in place without a copy; Xq int8 [M][K] and
 * s_a fp16 [M] are contiguous and identical to aria_quant_act on the gathered
 * rows.  Feed them to aria_qlinear_w8a8_prequant. */
int aria_quant_act_strided(const void* x_f16, int64_t ldx, int64_t M, int64_t K, int8_t* xq,
                           void* s_a_f16, aria_stream_t stream);

/* a5 — epilogue applied to every output element y[m][n] (in fp32, then
 * rounded to fp16 once): dequantize, then each optional term in this order. */
typedef struct aria_epilogue {
    const void* bias;         /* fp16 [N] or NULL                                        */
    int32_t gelu;             /* 0 none, 1 GELU tanh form:
                                 0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3)))        */
    int32_t reserved;         /* must be 0                                               */
    const void* residual;     /* fp16 [M][N] or NULL; may be the same buffer as y        */
    const float* steer_dir;   /* fp32 [N] or NULL: steering direction d                  */
    const float* steer_alpha; /* DEVICE fp32 scalar alpha, or NULL; read by the kernel at
                                 run time (graph-updatable); alpha == 0 skips the term   */
    int32_t* acc_out;         /* W8A8 only, optional: the raw int32 accumulators [M][N]  */
} aria_epilogue;

/* Workspace (device bytes) the qlinear call needs for this shape; 0 = none.
 * W8A8 needs room for Xq int8 [M][K] and s_a fp16 [M] (256-byte aligned
 * parts); the weight-only modes currently need none, but callers should query
 * rather than assume.  A workspace may not overlap any other buffer of the
 * call (ARIA_E_ALIAS), and neither may the raw accumulators acc_out.
 *
 * Tile choice (M > 64) is automatic; the environment variable
 * ARIA_QLINEAR_TILE="BMxBNxWMxWN[xKS]" forces one of the library's tile
 * variants (a tuning and testing override; an unknown value is ignored). */
size_t aria_qlinear_workspace_bytes(int mode, int64_t M, int64_t K, int64_t N);

/* a2+a4+a5 — W8A8: Y = epilogue( (sum_k Xq[m][k] * Wq[n][k]) * s_a[m] * s_w[n] )
 * with Xq, s_a the per-token quantization of X (written to the workspace) and
 * an exact int32 accumulator.  epi may be NULL (plain output).  x must not
 * overlap y. */
int aria_qlinear_w8a8(const void* x_f16, int64_t M, int64_t K, int64_t N,
                      const int8_t* wq, const void* s_w_f16, const aria_epilogue* epi,
                      void* y_f16, void* ws, size_t ws_bytes, aria_stream_t stream);

/* Size of the library's fixed device scratch used by aria_qlinear_w8a8_noalloc
 * (one copy per GPU the library runs on, held until the process ends). */
#define ARIA_NOALLOC_SCRATCH_BYTES (24u << 20)

/* aria_qlinear_w8a8 for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, checks and results as aria_qlinear_w8a8 (bit-identical Y
 * and acc_out for the same inputs), but the quantized activations go to a
 * file-scope device array of ARIA_NOALLOC_SCRATCH_BYTES bytes owned by the
 * library instead of a caller workspace; the call allocates nothing (no
 * hipMalloc / hipFree, no allocating library routine).  Limit: the shape's
 * workspace, aria_qlinear_workspace_bytes(ARIA_W8A8, M, K, N) — Xq int8 [M][K]
 * plus s_a fp16 [M], each rounded up to 256 bytes — must fit in the scratch,
 * else ARIA_E_SCRATCH is returned and nothing is launched (M = 2048 allows
 * K up to 12288).  The first call on a GPU looks up the array's device address
 * there (ARIA_E_HIP if that fails).  Every call on one GPU uses the same array
 * and leaves its contents behind (each call overwrites what it reads before
 * reading it): calls that may overlap in time on one GPU — on different
 * streams, or from different threads — race and must be serialised by the
 * caller; aria_qlinear_w8a8 with a workspace per stream has no such limit. */
int aria_qlinear_w8a8_noalloc(const void* x_f16, int64_t M, int64_t K, int64_t N,
                              const int8_t* wq, const void* s_w_f16, const aria_epilogue* epi,
                              void* y_f16, aria_stream_t stream);

/* a3+a4+a5 — W8A16 (the pages' q8): Y = epilogue( s_w[n] * sum_k X[m][k] * Wq[n][k] )
 * with fp32 accumulation.  Reads the same Wq / s_w as W8A8. */
int aria_qlinear_w8a16(const void* x_f16, int64_t M, int64_t K, int64_t N,
                       const int8_t* wq, const void* s_w_f16, const aria_epilogue* epi,
                       void* y_f16, void* ws, size_t ws_bytes, aria_stream_t stream);

/* a3+a4+a5 — W4A16 (the pages' q4):
 * Y = epilogue( sum_k X[m][k] * fp16(q4[n][k] * s_g[n][k/32]) ) with fp32
 * accumulation; group must be 32. */
int aria_qlinear_w4a16(const void* x_f16, int64_t M, int64_t K, int64_t N,
                       const uint8_t* wq4, const void* s_g_f16, int group,
                       const aria_epilogue* epi, void* y_f16, void* ws, size_t ws_bytes,
                       aria_stream_t stream);

/* The fp16 rung (project page, "Results", table "Quantization is close to
 * free at 8-bit": fp16 is the row the quantized modes are timed against):
 * Y = epilogue( sum_k X[m][k] * Wt[n][k] ) with fp32 accumulation, Wt from
 * aria_qpack(16, 0, ...).  Same conventions and epilogue as the other modes;
 * K*N < 2^30. */
int aria_qlinear_w16a16(const void* x_f16, int64_t M, int64_t K, int64_t N, const void* wt_f16,
                        const aria_epilogue* epi, void* y_f16, void* ws, size_t ws_bytes,
                        aria_stream_t stream);

/* The DiT block's steps on either side of its linears (docshare paper page,
 * Fig. 1 "DiT blocks"; project page, "What aria is": the denoiser is a
 * transformer over latent tokens).  The pages name the block, not its
 * internals; these are the plain pre-norm transformer readings. */

/* LayerNorm of every row of X fp16 [M][W] (population variance, in fp32):
 * Y = (x - mean) / sqrt(var + eps) * gamma + beta, gamma / beta fp16 [W],
 * Y fp16 [M][W].  8 <= W <= 16384, W % 8 == 0, 0 <= eps <= 1.  y may be x
 * (in place) but must not partly overlap it. */
int aria_layernorm(const void* x_f16, int64_t M, int64_t W, const void* gamma_f16, const void* beta_f16,
                   float eps, void* y_f16, aria_stream_t stream);

/* LayerNorm as aria_layernorm, then the per-token quantization of its fp16
 * result as aria_quant_act, in one pass that keeps each row in registers: the
 * pre-norm in front of a W8A8 linear.  Xq int8 [M][W] and s_a fp16 [M] are
 * bit-identical to aria_layernorm followed by aria_quant_act on its output;
 * y (fp16 [M][W], the normalized rows) may be NULL when only the quantized
 * form is needed, or x (in place).  Shape rules are those of a W8A8 linear
 * with K = W (32 <= W <= 16384, W % 32 == 0); 0 <= eps <= 1.  xq and s_a must
 * not overlap x, y or each other. */
int aria_layernorm_quant(const void* x_f16, int64_t M, int64_t W, const void* gamma_f16, const void* beta_f16,
                         float eps, void* y_f16, int8_t* xq, void* s_a_f16, aria_stream_t stream);

/* a4+a5 — the W8A8 linear on activations quantized beforehand (by
 * aria_quant_act or aria_layernorm_quant): the GEMM and epilogue of
 * aria_qlinear_w8a8 without its quantization step, so the same Xq / s_a give
 * the same Y bit for bit.  Needs no workspace; xq and s_a must not overlap y. */
int aria_qlinear_w8a8_prequant(const int8_t* xq, const void* s_a_f16, int64_t M, int64_t K, int64_t N,
                               const int8_t* wq, const void* s_w_f16, const aria_epilogue* epi,
                               void* y_f16, aria_stream_t stream);

/* a2 fused into the chain (per-token quantization of one W8A8 linear's
 * input inside the linears around it; project page, "What aria is": the
 * denoising step replayed as one graph, and "Results", the W8A8 row of the
 * precision table).  The producer is aria_qlinear_w8a8
 * that also records, for a later W8A8 linear reading columns
 * [col0, col0 + ncols) of its output Y, the row maxima of those columns in
 * 64-column blocks:
 *   rowmax[m][j] = max over c in [col0 + 64 j, col0 + 64 j + 64) of
 *                  (bits of the stored fp16 y[m][c]) & 0x7FFF
 * (uint32 [M][ncols / 64]: the fp16 magnitude bits, which order like the
 * magnitudes).  col0 and ncols are multiples of 64, ncols >= 64,
 * col0 + ncols <= N, N % 8 == 0 (ARIA_E_SHAPE otherwise).  Y is bit-identical
 * to aria_qlinear_w8a8 on the same arguments.  rowmax must not overlap any
 * other argument (ARIA_E_ALIAS). */
int aria_qlinear_w8a8_rowmax(const void* x_f16, int64_t M, int64_t K, int64_t N, const int8_t* wq,
                             const void* s_w_f16, const aria_epilogue* epi, void* y_f16, void* ws,
                             size_t ws_bytes, uint32_t* rowmax, int64_t col0, int64_t ncols,
                             aria_stream_t stream);

/* The consumer: the W8A8 linear over X fp16 [M][K] stored at row stride ldx
 * halves (ldx >= K, ldx % 8 == 0; e.g. a column block of the producer's Y)
 * whose per-token scales come from the producer's row maxima (rowmax uint32
 * [M][K / 64], K % 64 == 0): s_a[m] = fp16(max_j rowmax[m][j] / 127), and X
 * is quantized with the arithmetic of aria_quant_act while the contraction
 * stages it, so no Xq is written.  Y, and s_a_out (fp16 [M], or NULL) when
 * given, are bit-identical to aria_quant_act_strided on the same X followed
 * by aria_qlinear_w8a8_prequant.  Needs no workspace; y must not overlap x or
 * rowmax, and s_a_out must not overlap any other argument (ARIA_E_ALIAS). */
int aria_qlinear_w8a8_fused(const void* x_f16, int64_t ldx, const uint32_t* rowmax, int64_t M, int64_t K,
                            int64_t N, const int8_t* wq, const void* s_w_f16, const aria_epilogue* epi,
                            void* y_f16, void* s_a_out_f16, aria_stream_t stream);

/* Multi-head softmax self-attention: qkv fp16 [M][3W] holds [Q | K | V]
 * column blocks (the QKV linear's output), head h of each at columns
 * h*64 .. h*64+63; the M rows are M / seq independent sequences of seq rows.
 *   out[i][h*64 + e] = sum_j softmax_j(q_i . k_j / 8) v_j[e]
 * with fp32 scores, softmax and accumulation, fp16 probabilities and output
 * out fp16 [M][W].  W must be heads * 64 (ARIA_E_UNSUPPORTED otherwise);
 * M % seq == 0; out must not overlap qkv. */
int aria_attention(const void* qkv_f16, int64_t M, int64_t W, int64_t heads, int64_t seq, void* out_f16,
                   aria_stream_t stream);

/* One weight-only linear of a grouped call: Y = epilogue(X * dequant(Wq)) as in
 * aria_qlinear_w8a16 / aria_qlinear_w4a16.  epi is a host pointer or NULL
 * (acc_out must be NULL). */
typedef struct aria_linear_problem {
    const void* x_f16;        /* X fp16 [M][K]                                             */
    int64_t M, K, N;
    const void* wq;           /* Wq int8 [N][K] (bits 8) or Wq4 uint8 [N][K/2] (bits 4)    */
    const void* s_f16;        /* s_w fp16 [N] (bits 8) or s_g fp16 [N][K/32] (bits 4)      */
    const aria_epilogue* epi; /* or NULL                                                   */
    void* y_f16;              /* Y fp16 [M][N]                                             */
} aria_linear_problem;

/* Several independent weight-only linears at small M in as few launches as
 * possible (one per 32 problems): the small-M regime of the 4-bit weights is
 * bound by streaming them from memory (project page, "Results": 4-bit weights
 * for small devices), and one launch per layer leaves it bound by launch cost
 * instead.  bits 8 / group 0 runs W8A16, bits 4 / group 32 runs W4A16.
 * Every problem is checked as the single call checks it, and in addition
 * 1 <= count <= 1024 (else ARIA_E_SHAPE) and M <= 64 (else ARIA_E_UNSUPPORTED).
 * The problems run concurrently, so no problem's y may overlap another
 * problem's x, weights, scales, bias, residual, d or y (ARIA_E_ALIAS).
 * `problems` is a host array, read only during the call.  Results are
 * bit-identical to one aria_qlinear_w8a16 / aria_qlinear_w4a16 call per problem. */
int aria_qlinear_grouped(int bits, int group, const aria_linear_problem* problems, int count,
                         aria_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* ARIA_QLINEAR_H */
