/*
 * aria qlinear ORACLE — test infrastructure only.
 *
 * A plain, slow, obviously correct CPU model of what the quantized linear layer
 * ("qlinear") of the aria runtime computes.  Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg may load it; the product path never does.
 * It shares no code, header, table or constant with the HIP library.
 *
 * Source pages (cited by title and section):
 *   [P4] "A Quantized Native Runtime for On-Device Semantic Audio Generation",
 *        project page (matteospanio.github.io/aria):
 *        - "What aria is", bullet "Quantization that saves memory": weights are
 *          packed from fp16 down to 8 or 4 bits and the fp16 copy is released.
 *        - "Results", table "Quantization is close to free at 8-bit": the modes
 *          q8 (8-bit weights, fp16 activations), W8A8 (8-bit operands
 *          multiplied on the integer matrix units) and q4 (4-bit weights).
 *        - "Results", "Steering is real, inside a narrow window" and "Sonic
 *          seasoning": a direction is added to one transformer block's residual
 *          stream; strength 0 removes it with bit-identical output.
 *   [P2] chatpaper abstract: the quantized copy replaces the fp16 footprint
 *        instead of adding to it.
 * The pages state the goal, not the formulas.  The formulas below are the plain
 * readings listed in the design notes (fp16 scales, absmax/qmax, round half to
 * even, qmax 127 / 7, group 32 along K, the 4-bit word layout below, epilogue order
 * scale -> bias -> GELU(tanh) -> residual -> alpha*d).
 *
 * Arithmetic: integers exactly in int64 (asserted to fit int32 where the GPU
 * keeps int32), reals in fp64.  Built with -ffp-contract=off, no fast-math.
 * Every function returns 0 on success and a negative number on a bad argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* C-1  IEEE 754 binary16 codec, written from the format's definition:        */
/*      1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent     */
/*      field 0 = zero/subnormal (value f * 2^-24), 31 = Inf/NaN.             */
/* ------------------------------------------------------------------------- */

double or_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* zero or subnormal */
    else if (e == 31)
        v = (f == 0) ? INFINITY : NAN;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Round half to even of a finite double, from the definition. */
double or_rne(double x)
{
    double fl = floor(x);
    double r = x - fl;                              /* exact for |x| < 2^52 */
    if (r > 0.5) return fl + 1.0;
    if (r < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;  /* tie: pick the even one */
}

/* fp64 -> binary16, round to nearest even, subnormals kept, overflow -> Inf. */
uint16_t or_f64_to_f16(double x)
{
    uint16_t sign = (signbit(x) ? 0x8000 : 0);
    double a = fabs(x);
    if (isnan(x)) return 0x7e00;
    if (a == 0.0) return sign;
    /* the grid spacing (quantum) of binary16 around a */
    int E;
    frexp(a, &E);                                   /* a = m * 2^E, m in [0.5, 1) */
    int e = E - 1;                                  /* a in [2^e, 2^(e+1)) */
    if (e < -14) e = -14;                           /* subnormal range: fixed quantum 2^-24 */
    double quantum = ldexp(1.0, e - 10);
    double n = or_rne(a / quantum);                 /* a/quantum is exact (power of two) */
    double v = n * quantum;                         /* the rounded magnitude, exact */
    if (v >= 65536.0) return sign | 0x7c00;         /* beyond max finite 65504 -> Inf */
    if (v < ldexp(1.0, -14))                        /* subnormal (or rounded to zero) */
        return sign | (uint16_t)(v / ldexp(1.0, -24));
    frexp(v, &E);
    e = E - 1;                                      /* v in [2^e, 2^(e+1)), e in [-14, 15] */
    uint16_t frac = (uint16_t)(v / ldexp(1.0, e - 10) - 1024.0);
    return sign | (uint16_t)((e + 15) << 10) | frac;
}

int or_f16_to_f64_array(const uint16_t* h, double* out, int64_t n)
{
    if (!h || !out || n < 0) return -1;
    for (int64_t i = 0; i < n; i++) out[i] = or_f16_to_f64(h[i]);
    return 0;
}

int or_f64_to_f16_array(const double* x, uint16_t* out, int64_t n)
{
    if (!x || !out || n < 0) return -1;
    for (int64_t i = 0; i < n; i++) out[i] = or_f64_to_f16(x[i]);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* C-2  Symmetric quantizer Q(v[0..L), qmax) -> (q[0..L), s)                  */
/*   a = max_i |v_i|;  s = fp16_RNE(a / qmax);                                */
/*   s == 0 -> all q = 0, else q_i = clamp(RNE(v_i / s), -qmax, qmax),        */
/*   dividing by the STORED fp16 scale.                                       */
/*   v is read with a stride (so a column of a row-major matrix can be fed);  */
/*   q is written contiguously.                                               */
/* ------------------------------------------------------------------------- */
int or_quant_sym(const uint16_t* v, int64_t L, int64_t stride, int qmax,
                 int8_t* q, uint16_t* s_out)
{
    if (!v || !q || !s_out || L <= 0 || stride <= 0 || qmax <= 0 || qmax > 127) return -1;
    double a = 0.0;
    for (int64_t i = 0; i < L; i++) {
        double t = fabs(or_f16_to_f64(v[i * stride]));
        if (!(t <= 65504.0)) return -2;             /* non-finite input */
        if (t > a) a = t;
    }
    uint16_t s = or_f64_to_f16(a / (double)qmax);
    double sd = or_f16_to_f64(s);
    *s_out = s;
    for (int64_t i = 0; i < L; i++) {
        if (sd == 0.0) { q[i] = 0; continue; }
        double r = or_rne(or_f16_to_f64(v[i * stride]) / sd);
        if (r > qmax) r = qmax;
        if (r < -qmax) r = -qmax;
        q[i] = (int8_t)r;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* a1  Weight packing.  W is fp16 [K][N] row-major (K inputs, N outputs).     */
/* q8: per output channel n, quantize the column W[:, n] with qmax 127;      */
/*     Wq int8 [N][K] (row n contiguous along K), s fp16 [N].                 */
/* q4: per (n, group g) quantize W[gG .. gG+G), n] with qmax 7; s fp16       */
/*     [N][K/G].  Row n of Wq4 is K/2 bytes: the codes of each run of eight   */
/*     consecutive k (k = 8d .. 8d+7) form its little-endian 32-bit word d    */
/*     (bytes 4d .. 4d+3), even k = 8d+2i in bits 4i .. 4i+3 and odd          */
/*     k = 8d+2i+1 in bits 16+4i .. 16+4i+3 (i = 0..3), as two's-complement   */
/*     nibbles.  (The byte layout is the library's own choice; with the even  */
/*     codes in one half-word and the odd ones in the other, one mask of a    */
/*     word yields the fp16 pair of two adjacent k.)                          */
/* ------------------------------------------------------------------------- */

/* Bit position of code k within its row's word k / 8 (layout above). */
static int or_q4_bit(int64_t k) { return (int)((k % 2) * 16 + ((k % 8) / 2) * 4); }

/* The nibble of code k in row q4r (K/2 bytes), two's complement -> int. */
static int or_q4_get(const uint8_t* q4r, int64_t k)
{
    const int bit = or_q4_bit(k);
    const int nib = (q4r[4 * (k / 8) + bit / 8] >> (bit % 8)) & 0xF;
    return nib >= 8 ? nib - 16 : nib;
}
int or_qpack8(const uint16_t* w, int64_t K, int64_t N, int8_t* q, uint16_t* s)
{
    if (!w || !q || !s || K <= 0 || N <= 0) return -1;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(|:bad)
    for (int64_t n = 0; n < N; n++)
        bad |= (or_quant_sym(w + n, K, N, 127, q + n * K, s + n) != 0);
    return bad ? -2 : 0;
}

int or_qpack4(const uint16_t* w, int64_t K, int64_t N, int64_t group, uint8_t* q4, uint16_t* s)
{
    if (!w || !q4 || !s || K <= 0 || N <= 0 || group <= 0 || (group % 2) || K % group || K % 8) return -1;
    int64_t G = K / group;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(|:bad)
    for (int64_t n = 0; n < N; n++) {
        int8_t* qcol = (int8_t*)malloc((size_t)K);
        if (!qcol) { bad = 1; continue; }
        for (int64_t g = 0; g < G; g++)
            bad |= (or_quant_sym(w + g * group * N + n, group, N, 7, qcol + g * group, s + n * G + g) != 0);
        uint8_t* row = q4 + n * (K / 2);
        memset(row, 0, (size_t)(K / 2));
        for (int64_t k = 0; k < K; k++) {
            const int bit = or_q4_bit(k);
            row[4 * (k / 8) + bit / 8] |= (uint8_t)((qcol[k] & 0xF) << (bit % 8));
        }
        free(qcol);
    }
    return bad ? -2 : 0;
}

/* Inverse of the nibble packing (two's complement 4-bit -> int8). */
int or_unpack4(const uint8_t* q4, int64_t K, int64_t N, int8_t* q)
{
    if (!q4 || !q || K <= 0 || N <= 0 || (K % 8)) return -1;
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) q[n * K + k] = (int8_t)or_q4_get(q4 + n * (K / 2), k);
    return 0;
}

/* a2  Per-token activation quantization: each row m of X fp16 [M][K]
 *     with qmax 127 -> Xq int8 [M][K], s_a fp16 [M]. */
int or_quant_act(const uint16_t* x, int64_t M, int64_t K, int8_t* xq, uint16_t* sa)
{
    if (!x || !xq || !sa || M <= 0 || K <= 0) return -1;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(|:bad)
    for (int64_t m = 0; m < M; m++)
        bad |= (or_quant_sym(x + m * K, K, 1, 127, xq + m * K, sa + m) != 0);
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------------------- */
/* C-4  Contractions.                                                         */
/* ------------------------------------------------------------------------- */

/* W8A8: acc[m][n] = sum_k xq[m][k] * wq[n][k], exact in int64; -3 if a sum
 * does not fit int32 (cannot happen for |q| <= 127 and K <= 133152). */
int or_gemm_i8(const int8_t* xq, const int8_t* wq, int64_t M, int64_t N, int64_t K, int32_t* acc)
{
    if (!xq || !wq || !acc || M <= 0 || N <= 0 || K <= 0) return -1;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(|:bad)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            int64_t t = 0;
            for (int64_t k = 0; k < K; k++) t += (int64_t)xq[m * K + k] * (int64_t)wq[n * K + k];
            if (t > INT32_MAX || t < INT32_MIN) bad = 1;
            acc[m * N + n] = (int32_t)t;
        }
    return bad ? -3 : 0;
}

/* W8A16: r[m][n] = s_w[n] * sum_k x[m][k] * wq[n][k]   (fp64). */
int or_ref_w8a16(const uint16_t* x, const int8_t* wq, const uint16_t* sw,
                 int64_t M, int64_t N, int64_t K, double* r)
{
    if (!x || !wq || !sw || !r || M <= 0 || N <= 0 || K <= 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        double* xr = (double*)malloc((size_t)K * sizeof(double));
        for (int64_t k = 0; k < K; k++) xr[k] = or_f16_to_f64(x[m * K + k]);
        for (int64_t n = 0; n < N; n++) {
            double t = 0.0;
            for (int64_t k = 0; k < K; k++) t += xr[k] * (double)wq[n * K + k];
            r[m * N + n] = or_f16_to_f64(sw[n]) * t;
        }
        free(xr);
    }
    return 0;
}

/* W4A16: r[m][n] = sum_k x[m][k] * (q4[n][k] * s4[n][k / group])   (fp64),
 * with q4 unpacked from the nibble layout above. */
int or_ref_w4a16(const uint16_t* x, const uint8_t* wq4, const uint16_t* sg, int64_t group,
                 int64_t M, int64_t N, int64_t K, double* r)
{
    if (!x || !wq4 || !sg || !r || M <= 0 || N <= 0 || K <= 0 || group <= 0 || K % group || (K % 8))
        return -1;
    int64_t G = K / group;
    /* dequantized weights, computed once: wd[n][k] = q * s (exact in fp64) */
    double* wd = (double*)malloc((size_t)(N * K) * sizeof(double));
    if (!wd) return -4;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            const int qv = or_q4_get(wq4 + n * (K / 2), k);
            wd[n * K + k] = (double)qv * or_f16_to_f64(sg[n * G + k / group]);
        }
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        double* xr = (double*)malloc((size_t)K * sizeof(double));
        for (int64_t k = 0; k < K; k++) xr[k] = or_f16_to_f64(x[m * K + k]);
        for (int64_t n = 0; n < N; n++) {
            double t = 0.0;
            for (int64_t k = 0; k < K; k++) t += xr[k] * wd[n * K + k];
            r[m * N + n] = t;
        }
        free(xr);
    }
    free(wd);
    return 0;
}

/* The fp16 rung of the precision ladder ([P4] "Results", table "Quantization
 * is close to free at 8-bit": fp16 is the row the quantized modes are timed
 * against).  Weights are kept as fp16, laid out like the packed ones: row n
 * holds column n of W, contiguous along K.  wt[n][k] = w[k][n] (a copy). */
int or_pack16(const uint16_t* w, int64_t K, int64_t N, uint16_t* wt)
{
    if (!w || !wt || K <= 0 || N <= 0) return -1;
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) wt[n * K + k] = w[k * N + n];
    return 0;
}

/* W16A16: r[m][n] = sum_k x[m][k] * wt[n][k]   (fp64). */
int or_ref_w16a16(const uint16_t* x, const uint16_t* wt, int64_t M, int64_t N, int64_t K, double* r)
{
    if (!x || !wt || !r || M <= 0 || N <= 0 || K <= 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        double* xr = (double*)malloc((size_t)K * sizeof(double));
        for (int64_t k = 0; k < K; k++) xr[k] = or_f16_to_f64(x[m * K + k]);
        for (int64_t n = 0; n < N; n++) {
            double t = 0.0;
            for (int64_t k = 0; k < K; k++) t += xr[k] * or_f16_to_f64(wt[n * K + k]);
            r[m * N + n] = t;
        }
        free(xr);
    }
    return 0;
}

/* W8A8 dequantization of the accumulator: y[m][n] = acc[m][n] * s_a[m] * s_w[n]. */
int or_scale_w8a8(const int32_t* acc, const uint16_t* sa, const uint16_t* sw,
                  int64_t M, int64_t N, double* y)
{
    if (!acc || !sa || !sw || !y || M <= 0 || N <= 0) return -1;
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            y[m * N + n] = (double)acc[m * N + n] * or_f16_to_f64(sa[m]) * or_f16_to_f64(sw[n]);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* C-5  Epilogue, in place on y fp64 [M][N]:                                  */
/*   y += bias[n];  y = gelu_tanh(y);  y += residual[m][n];  y += alpha*d[n]  */
/* each step only when its operand is given; the steering term is skipped    */
/* entirely when alpha == 0 or d is NULL ([P4] "Results": zero strength     */
/* leaves every output bit as without steering).                             */
/* GELU, tanh form (Hendrycks & Gimpel, "Gaussian Error Linear Units"):      */
/*   gelu(y) = 0.5 * y * (1 + tanh(sqrt(2/pi) * (y + 0.044715 * y^3)))       */
/* ------------------------------------------------------------------------- */
double or_gelu_tanh(double y)
{
    const double pi = 3.14159265358979323846;
    return 0.5 * y * (1.0 + tanh(sqrt(2.0 / pi) * (y + 0.044715 * y * y * y)));
}

int or_epilogue(double* y, int64_t M, int64_t N, const uint16_t* bias, int gelu,
                const uint16_t* residual, const float* d, float alpha)
{
    if (!y || M <= 0 || N <= 0) return -1;
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            double v = y[m * N + n];
            if (bias) v += or_f16_to_f64(bias[n]);
            if (gelu) v = or_gelu_tanh(v);
            if (residual) v += or_f16_to_f64(residual[m * N + n]);
            if (d && alpha != 0.0f) v += (double)alpha * (double)d[n];
            y[m * N + n] = v;
        }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* The steps on either side of the linears in a DiT block ([P5] Fig. 1 "DiT  */
/* blocks"; [P4] "What aria is": the denoiser is a transformer over latent   */
/* tokens).  The pages name the blocks but not their internals; the plain    */
/* readings (design notes R21-R23): a pre-norm LayerNorm per token over the  */
/* width, and multi-head softmax self-attention with 64-dimensional heads,   */
/* no mask and no position terms, within each sequence of S tokens.          */
/* ------------------------------------------------------------------------- */

/* LayerNorm over each row (Ba, Kiros, Hinton, "Layer Normalization"):
 *   mu = mean_k x[m][k];  var = mean_k (x[m][k] - mu)^2   (population)
 *   y[m][k] = (x[m][k] - mu) / sqrt(var + eps) * gamma[k] + beta[k]   (fp64). */
int or_layernorm(const uint16_t* x, const uint16_t* gamma, const uint16_t* beta, double eps,
                 int64_t M, int64_t W, double* y)
{
    if (!x || !gamma || !beta || !y || M <= 0 || W <= 0 || !(eps >= 0.0)) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        double mu = 0.0, var = 0.0;
        for (int64_t k = 0; k < W; k++) mu += or_f16_to_f64(x[m * W + k]);
        mu /= (double)W;
        for (int64_t k = 0; k < W; k++) {
            double c = or_f16_to_f64(x[m * W + k]) - mu;
            var += c * c;
        }
        var /= (double)W;
        double inv = 1.0 / sqrt(var + eps);
        for (int64_t k = 0; k < W; k++)
            y[m * W + k] = (or_f16_to_f64(x[m * W + k]) - mu) * inv * or_f16_to_f64(gamma[k]) +
                           or_f16_to_f64(beta[k]);
    }
    return 0;
}

/* Multi-head self-attention (Vaswani et al., "Attention Is All You Need"):
 * qkv fp16 [M][3W] holds [Q | K | V] column blocks, head h of each at columns
 * h*D .. h*D + D - 1 (D = W / H).  The M rows are M / S independent sequences
 * of S tokens.  For sequence b, head h, query i:
 *   s_j = (q_i . k_j) / sqrt(D),  p_j = exp(s_j - max s) / sum exp(...),
 *   out[i][h*D + e] = sum_j p_j v_j[e]                                  (fp64). */
int or_attention(const uint16_t* qkv, int64_t M, int64_t W, int64_t H, int64_t S, double* out)
{
    if (!qkv || !out || M <= 0 || W <= 0 || H <= 0 || S <= 0 || W % H || M % S) return -1;
    const int64_t D = W / H, ld = 3 * W;
    const double scale = 1.0 / sqrt((double)D);
#pragma omp parallel for schedule(static) collapse(2)
    for (int64_t b = 0; b < M / S; b++)
        for (int64_t h = 0; h < H; h++) {
            double* sc = (double*)malloc((size_t)S * sizeof(double));
            for (int64_t i = 0; i < S; i++) {
                const int64_t qi = (b * S + i) * ld + h * D;
                double mx = -INFINITY;
                for (int64_t j = 0; j < S; j++) {
                    const int64_t kj = (b * S + j) * ld + W + h * D;
                    double t = 0.0;
                    for (int64_t e = 0; e < D; e++) t += or_f16_to_f64(qkv[qi + e]) * or_f16_to_f64(qkv[kj + e]);
                    sc[j] = t * scale;
                    if (sc[j] > mx) mx = sc[j];
                }
                double sum = 0.0;
                for (int64_t j = 0; j < S; j++) {
                    sc[j] = exp(sc[j] - mx);
                    sum += sc[j];
                }
                for (int64_t e = 0; e < D; e++) {
                    double o = 0.0;
                    for (int64_t j = 0; j < S; j++) o += sc[j] * or_f16_to_f64(qkv[(b * S + j) * ld + 2 * W + h * D + e]);
                    out[(b * S + i) * W + h * D + e] = o / sum;
                }
            }
            free(sc);
        }
    return 0;
}
