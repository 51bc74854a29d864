// The C-ABI of the qlinear library (declared in include/aria_qlinear.h).
// Host-side only: validates every argument before anything is launched, lays
// out the caller's workspace, and enqueues the kernels on the caller's stream.
// No allocation, no synchronisation, no device reads on the host.
#include <atomic>
#include <mutex>

#include "../../include/aria_qlinear.h"
#include "common.h"
#include "kernels.h"

using namespace aria;

// The allocation-free W8A8 call keeps its quantized activations here: one copy
// of this array per GPU, created when the library's code is loaded on that GPU
// and held until the process ends.  In host code `scratch` names only a host
// stand-in; its device address on the current GPU comes from
// hipGetSymbolAddress (scratch_address below) and is the only form passed to
// kernels.
static __device__ __align__(256) unsigned char scratch[ARIA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 30;   // M and N limits (int indexing in kernels)
constexpr int64_t kMaxK = 16384;                 // activation-quant keeps a row in registers
constexpr size_t kAlign = 256;                    // workspace sub-buffer alignment
constexpr int kGroupedMax = 1024;                 // problems per grouped call
constexpr int64_t kGroupedMaxM = 64;              // the grouped path is the small-M kernel

inline bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int check_shape(int64_t M, int64_t K, int64_t N) {
    if (M < 1 || N < 1 || K < 32 || (K % 32) != 0) return ARIA_E_SHAPE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxK) return ARIA_E_SHAPE;
    // packed weights of one linear are addressed with 32-bit offsets
    if (M * N > ((int64_t)1 << 40) || M * K > ((int64_t)1 << 40) || N * K >= ((int64_t)1 << 31)) return ARIA_E_SHAPE;
    return ARIA_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Validate the epilogue and convert it to the kernels' form.
int make_epi(const aria_epilogue* e, int mode, int64_t M, int64_t N, const void* y, Epi* out) {
    *out = Epi{nullptr, nullptr, nullptr, nullptr, nullptr, 0};
    if (!e) return ARIA_OK;
    if (e->reserved != 0 || (e->gelu != 0 && e->gelu != 1)) return ARIA_E_UNSUPPORTED;
    if (e->acc_out && mode != ARIA_W8A8) return ARIA_E_UNSUPPORTED;
    if (e->steer_dir && !e->steer_alpha) return ARIA_E_NULL;
    if (!aligned16(e->bias) || !aligned16(e->residual) || !aligned16(e->steer_dir) ||
        !aligned16(e->steer_alpha) || !aligned16(e->acc_out))
        return ARIA_E_ALIGN;
    // the residual may be exactly y (in-place h += ...), but must not partly overlap it
    const size_t ybytes = (size_t)(M * N) * 2;
    if (e->residual && e->residual != y && overlap(e->residual, ybytes, y, ybytes)) return ARIA_E_ALIAS;
    // the raw accumulators are an output of their own
    const size_t abytes = (size_t)(M * N) * 4;
    if (e->acc_out && (overlap(e->acc_out, abytes, y, ybytes) || (e->residual && overlap(e->acc_out, abytes, e->residual, ybytes)) ||
                       (e->bias && overlap(e->acc_out, abytes, e->bias, (size_t)N * 2)) ||
                       (e->steer_dir && overlap(e->acc_out, abytes, e->steer_dir, (size_t)N * 4)) ||
                       (e->steer_alpha && overlap(e->acc_out, abytes, e->steer_alpha, 4))))
        return ARIA_E_ALIAS;
    out->bias = static_cast<const half_t*>(e->bias);
    out->residual = static_cast<const half_t*>(e->residual);
    out->steer_dir = e->steer_dir;
    out->steer_alpha = e->steer_dir ? e->steer_alpha : nullptr;
    out->acc_out = e->acc_out;
    out->gelu = e->gelu;
    return ARIA_OK;
}

size_t w8a8_ws(int64_t M, int64_t K) { return round_up((size_t)(M * K), kAlign) + round_up((size_t)M * 2, kAlign); }

// Does any buffer of the epilogue overlap [p, p + n)?  (The residual is
// checked against y by make_epi; here it is one more buffer.)
bool epi_overlaps(const aria_epilogue* e, int64_t M, int64_t N, const void* p, size_t n) {
    if (!e) return false;
    const size_t mn = (size_t)(M * N);
    return (e->bias && overlap(e->bias, (size_t)N * 2, p, n)) || (e->residual && overlap(e->residual, mn * 2, p, n)) ||
           (e->steer_dir && overlap(e->steer_dir, (size_t)N * 4, p, n)) ||
           (e->steer_alpha && overlap(e->steer_alpha, 4, p, n)) || (e->acc_out && overlap(e->acc_out, mn * 4, p, n));
}

// Device address of `scratch` on the current GPU, looked up once per device.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ARIA_E_HIP;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
                (void)hipGetLastError();
                return ARIA_E_HIP;
            }
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return ARIA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? ARIA_OK : ARIA_E_HIP; }

}  // namespace

extern "C" {

const char* aria_status_string(int s) {
    switch (s) {
        case ARIA_OK: return "ok";
        case ARIA_E_NULL: return "a required pointer is NULL";
        case ARIA_E_SHAPE: return "M, K or N out of range (1 <= M <= 2^30; 1 <= N <= 2^30; 32 <= K <= 16384; K % 32 == 0; N * K < 2^31)";
        case ARIA_E_ALIGN: return "a pointer is not 16-byte aligned";
        case ARIA_E_UNSUPPORTED: return "unsupported bits/group/epilogue option";
        case ARIA_E_WORKSPACE: return "workspace missing or too small";
        case ARIA_E_HIP: return "HIP runtime error at launch";
        case ARIA_E_ALIAS: return "output overlaps an input";
        case ARIA_E_SCRATCH: return "shape needs more than the library's fixed scratch (ARIA_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int aria_abi_version(void) { return 1; }

int aria_qpack_bytes(int bits, int group, int64_t K, int64_t N, size_t* q_bytes, size_t* s_bytes) {
    if (!q_bytes || !s_bytes) return ARIA_E_NULL;
    if (check_shape(1, K, N) != ARIA_OK) return ARIA_E_SHAPE;
    if (bits == 8 && group == 0) {
        *q_bytes = (size_t)(K * N);
        *s_bytes = (size_t)N * 2;
        return ARIA_OK;
    }
    if (bits == 4 && group == 32) {
        *q_bytes = (size_t)(K * N) / 2;
        *s_bytes = (size_t)N * (size_t)(K / 32) * 2;
        return ARIA_OK;
    }
    if (bits == 16 && group == 0) {
        if (K * N >= ((int64_t)1 << 30)) return ARIA_E_SHAPE;   // 2 K N bytes, 32-bit offsets
        *q_bytes = (size_t)(K * N) * 2;
        *s_bytes = 0;
        return ARIA_OK;
    }
    return ARIA_E_UNSUPPORTED;
}

int aria_qpack(int bits, int group, const void* w, int64_t K, int64_t N, void* q, void* s,
               aria_stream_t stream) {
    size_t qb, sb;
    const int rc = aria_qpack_bytes(bits, group, K, N, &qb, &sb);
    if (rc != ARIA_OK) return rc;
    if (!w || !q || (!s && bits != 16)) return ARIA_E_NULL;
    if (!aligned16(w) || !aligned16(q) || !aligned16(s)) return ARIA_E_ALIGN;
    if (overlap(w, (size_t)(K * N) * 2, q, qb) || (sb && overlap(w, (size_t)(K * N) * 2, s, sb))) return ARIA_E_ALIAS;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const half_t* wh = static_cast<const half_t*>(w);
    if (bits == 16) return hip_status(launch_pack16(wh, K, N, static_cast<half_t*>(q), st));
    if (bits == 8) return hip_status(launch_qpack8(wh, K, N, static_cast<int8_t*>(q), static_cast<half_t*>(s), st));
    return hip_status(launch_qpack4(wh, K, N, static_cast<uint8_t*>(q), static_cast<half_t*>(s), st));
}

int aria_quant_act(const void* x, int64_t M, int64_t K, int8_t* xq, void* sa, aria_stream_t stream) {
    if (check_shape(M, K, 1) != ARIA_OK) return ARIA_E_SHAPE;
    if (!x || !xq || !sa) return ARIA_E_NULL;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(sa)) return ARIA_E_ALIGN;
    if (overlap(x, (size_t)(M * K) * 2, xq, (size_t)(M * K))) return ARIA_E_ALIAS;
    (void)hipGetLastError();
    return hip_status(launch_actquant(static_cast<const half_t*>(x), M, K, xq, static_cast<half_t*>(sa),
                                      static_cast<hipStream_t>(stream)));
}

int aria_quant_act_strided(const void* x, int64_t ldx, int64_t M, int64_t K, int8_t* xq, void* sa,
                           aria_stream_t stream) {
    if (check_shape(M, K, 1) != ARIA_OK || ldx < K || ldx % 8 != 0 || ldx > ((int64_t)1 << 40) / M)
        return ARIA_E_SHAPE;
    if (!x || !xq || !sa) return ARIA_E_NULL;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(sa)) return ARIA_E_ALIGN;
    const size_t xb = (size_t)((M - 1) * ldx + K) * 2;   // first to last byte of the rows read
    if (overlap(x, xb, xq, (size_t)(M * K)) || overlap(x, xb, sa, (size_t)M * 2) ||
        overlap(xq, (size_t)(M * K), sa, (size_t)M * 2))
        return ARIA_E_ALIAS;
    (void)hipGetLastError();
    return hip_status(launch_actquant(static_cast<const half_t*>(x), M, K, xq, static_cast<half_t*>(sa),
                                      static_cast<hipStream_t>(stream), ldx));
}

size_t aria_qlinear_workspace_bytes(int mode, int64_t M, int64_t K, int64_t N) {
    if (check_shape(M, K, N) != ARIA_OK) return 0;
    switch (mode) {
        case ARIA_W8A8: return w8a8_ws(M, K);
        case ARIA_W8A16: return wxa16_workspace_bytes(8, M, K, N);
        case ARIA_W4A16: return wxa16_workspace_bytes(4, M, K, N);
        case ARIA_W16A16: return wxa16_workspace_bytes(16, M, K, N);
        default: return 0;
    }
}

}  // extern "C"

namespace {

// The W8A8 checks apart from those of the workspace.
int w8a8_check(const void* x, int64_t M, int64_t K, int64_t N, const int8_t* wq, const void* sw,
               const aria_epilogue* epi, void* y, Epi* e) {
    int rc = check_shape(M, K, N);
    if (rc != ARIA_OK) return rc;
    if (!x || !wq || !sw || !y) return ARIA_E_NULL;
    if (!aligned16(x) || !aligned16(wq) || !aligned16(sw) || !aligned16(y)) return ARIA_E_ALIGN;
    if (overlap(x, (size_t)(M * K) * 2, y, (size_t)(M * N) * 2)) return ARIA_E_ALIAS;
    return make_epi(epi, ARIA_W8A8, M, N, y, e);
}

// act-quant of X into the workspace (Xq int8 [M][K], then s_a fp16 [M] at the
// next 256-byte boundary), then the GEMM + epilogue reading it.
int w8a8_launch(const void* x, int64_t M, int64_t K, int64_t N, const int8_t* wq, const void* sw, const Epi& e,
                void* y, void* ws, hipStream_t st) {
    int8_t* xq = static_cast<int8_t*>(ws);
    half_t* sa = reinterpret_cast<half_t*>(static_cast<char*>(ws) + round_up((size_t)(M * K), kAlign));
    (void)hipGetLastError();
    int rc = hip_status(launch_actquant(static_cast<const half_t*>(x), M, K, xq, sa, st));
    if (rc != ARIA_OK) return rc;
    return hip_status(launch_gemm_tiled(0, xq, wq, static_cast<const half_t*>(sw), sa, static_cast<half_t*>(y),
                                        (int)M, (int)N, (int)K, e, st));
}

}  // namespace

extern "C" {

int aria_qlinear_w8a8(const void* x, int64_t M, int64_t K, int64_t N, const int8_t* wq, const void* sw,
                      const aria_epilogue* epi, void* y, void* ws, size_t ws_bytes, aria_stream_t stream) {
    Epi e;
    int rc = w8a8_check(x, M, K, N, wq, sw, epi, y, &e);
    if (rc != ARIA_OK) return rc;
    if (!aligned16(ws)) return ARIA_E_ALIGN;
    const size_t need = w8a8_ws(M, K);
    if (!ws || ws_bytes < need) return ARIA_E_WORKSPACE;
    // the workspace is written while x, the weights and the epilogue
    // operands are read, and y is written
    if (overlap(ws, need, x, (size_t)(M * K) * 2) || overlap(ws, need, y, (size_t)(M * N) * 2) ||
        overlap(ws, need, wq, (size_t)(N * K)) || overlap(ws, need, sw, (size_t)N * 2) ||
        epi_overlaps(epi, M, N, ws, need))
        return ARIA_E_ALIAS;
    return w8a8_launch(x, M, K, N, wq, sw, e, y, ws, static_cast<hipStream_t>(stream));
}

int aria_qlinear_w8a8_rowmax(const void* x, int64_t M, int64_t K, int64_t N, const int8_t* wq, const void* sw,
                             const aria_epilogue* epi, void* y, void* ws, size_t ws_bytes, uint32_t* rowmax,
                             int64_t col0, int64_t ncols, aria_stream_t stream) {
    Epi e;
    int rc = w8a8_check(x, M, K, N, wq, sw, epi, y, &e);
    if (rc != ARIA_OK) return rc;
    if (N % 8 != 0 || col0 < 0 || ncols < 64 || col0 % 64 != 0 || ncols % 64 != 0 || col0 + ncols > N)
        return ARIA_E_SHAPE;
    if (!rowmax) return ARIA_E_NULL;
    if (!aligned16(ws) || !aligned16(rowmax)) return ARIA_E_ALIGN;
    const size_t need = w8a8_ws(M, K);
    if (!ws || ws_bytes < need) return ARIA_E_WORKSPACE;
    const size_t rb = (size_t)M * (size_t)(ncols / 64) * 4;
    if (overlap(ws, need, x, (size_t)(M * K) * 2) || overlap(ws, need, y, (size_t)(M * N) * 2) ||
        overlap(ws, need, wq, (size_t)(N * K)) || overlap(ws, need, sw, (size_t)N * 2) ||
        epi_overlaps(epi, M, N, ws, need) || overlap(rowmax, rb, ws, need) || overlap(rowmax, rb, x, (size_t)(M * K) * 2) ||
        overlap(rowmax, rb, y, (size_t)(M * N) * 2) || overlap(rowmax, rb, wq, (size_t)(N * K)) ||
        overlap(rowmax, rb, sw, (size_t)N * 2) || epi_overlaps(epi, M, N, rowmax, rb))
        return ARIA_E_ALIAS;
    e.rowmax = rowmax;
    e.rowmax_ld = (int)(ncols / 64);
    e.rowmax_c0 = (int)col0;
    e.rowmax_c1 = (int)(col0 + ncols);
    return w8a8_launch(x, M, K, N, wq, sw, e, y, ws, static_cast<hipStream_t>(stream));
}

int aria_qlinear_w8a8_fused(const void* x, int64_t ldx, const uint32_t* rowmax, int64_t M, int64_t K, int64_t N,
                            const int8_t* wq, const void* sw, const aria_epilogue* epi, void* y, void* s_a_out,
                            aria_stream_t stream) {
    int rc = check_shape(M, K, N);
    if (rc != ARIA_OK) return rc;
    if (K % 64 != 0 || ldx < K || ldx % 8 != 0 || ldx > ((int64_t)1 << 40) / M || ldx >= ((int64_t)1 << 30))
        return ARIA_E_SHAPE;
    if (!x || !rowmax || !wq || !sw || !y) return ARIA_E_NULL;
    if (!aligned16(x) || !aligned16(rowmax) || !aligned16(wq) || !aligned16(sw) || !aligned16(y) ||
        !aligned16(s_a_out))
        return ARIA_E_ALIGN;
    const size_t xb = (size_t)((M - 1) * ldx + K) * 2, yb = (size_t)(M * N) * 2, rb = (size_t)(M * (K / 64)) * 4;
    if (overlap(x, xb, y, yb) || overlap(rowmax, rb, y, yb) ||
        (s_a_out && (overlap(s_a_out, (size_t)M * 2, y, yb) || overlap(s_a_out, (size_t)M * 2, x, xb) ||
                     overlap(s_a_out, (size_t)M * 2, rowmax, rb) || overlap(s_a_out, (size_t)M * 2, wq, (size_t)(N * K)) ||
                     overlap(s_a_out, (size_t)M * 2, sw, (size_t)N * 2) || epi_overlaps(epi, M, N, s_a_out, (size_t)M * 2))))
        return ARIA_E_ALIAS;
    Epi e;
    if ((rc = make_epi(epi, ARIA_W8A8, M, N, y, &e)) != ARIA_OK) return rc;
    const AQuant aq{rowmax, (int)(K / 64), (int)ldx, static_cast<half_t*>(s_a_out)};
    (void)hipGetLastError();
    return hip_status(launch_gemm_tiled(4, x, wq, static_cast<const half_t*>(sw), nullptr, static_cast<half_t*>(y),
                                        (int)M, (int)N, (int)K, e, static_cast<hipStream_t>(stream), &aq));
}

int aria_qlinear_w8a8_noalloc(const void* x, int64_t M, int64_t K, int64_t N, const int8_t* wq, const void* sw,
                              const aria_epilogue* epi, void* y, aria_stream_t stream) {
    Epi e;
    int rc = w8a8_check(x, M, K, N, wq, sw, epi, y, &e);
    if (rc != ARIA_OK) return rc;
    if (w8a8_ws(M, K) > (size_t)ARIA_NOALLOC_SCRATCH_BYTES) return ARIA_E_SCRATCH;
    void* ws = nullptr;
    if ((rc = scratch_address(&ws)) != ARIA_OK) return rc;
    return w8a8_launch(x, M, K, N, wq, sw, e, y, ws, static_cast<hipStream_t>(stream));
}

static int wxa16(int bits, const void* x, int64_t M, int64_t K, int64_t N, const void* wq, const void* s,
                 const aria_epilogue* epi, void* y, void* ws, size_t ws_bytes, aria_stream_t stream) {
    int rc = check_shape(M, K, N);
    if (rc != ARIA_OK) return rc;
    if (bits == 16 && K * N >= ((int64_t)1 << 30)) return ARIA_E_SHAPE;   // fp16 weights: 2 K N bytes
    if (!x || !wq || (!s && bits != 16) || !y) return ARIA_E_NULL;
    if (!aligned16(x) || !aligned16(wq) || !aligned16(s) || !aligned16(y) || !aligned16(ws)) return ARIA_E_ALIGN;
    if (overlap(x, (size_t)(M * K) * 2, y, (size_t)(M * N) * 2)) return ARIA_E_ALIAS;
    Epi e;
    const int mode = bits == 8 ? ARIA_W8A16 : bits == 4 ? ARIA_W4A16 : ARIA_W16A16;
    if ((rc = make_epi(epi, mode, M, N, y, &e)) != ARIA_OK) return rc;
    const size_t need = wxa16_workspace_bytes(bits, M, K, N);
    if (need && (!ws || ws_bytes < need)) return ARIA_E_WORKSPACE;
    if (need) {
        const size_t wb = bits == 8 ? (size_t)(N * K) : bits == 4 ? (size_t)(N * K) / 2 : (size_t)(N * K) * 2;
        const size_t sb = bits == 8 ? (size_t)N * 2 : bits == 4 ? (size_t)N * (size_t)(K / 32) * 2 : 0;
        if (overlap(ws, need, x, (size_t)(M * K) * 2) || overlap(ws, need, y, (size_t)(M * N) * 2) ||
            overlap(ws, need, wq, wb) || (sb && overlap(ws, need, s, sb)) || epi_overlaps(epi, M, N, ws, need))
            return ARIA_E_ALIAS;
    }
    (void)hipGetLastError();
    return hip_status(launch_gemm_wxa16(bits, static_cast<const half_t*>(x), wq, static_cast<const half_t*>(s),
                                        static_cast<half_t*>(y), (int)M, (int)N, (int)K, e, ws, ws_bytes,
                                        static_cast<hipStream_t>(stream)));
}

int aria_qlinear_w8a16(const void* x, int64_t M, int64_t K, int64_t N, const int8_t* wq, const void* sw,
                       const aria_epilogue* epi, void* y, void* ws, size_t ws_bytes, aria_stream_t stream) {
    return wxa16(8, x, M, K, N, wq, sw, epi, y, ws, ws_bytes, stream);
}

int aria_qlinear_w4a16(const void* x, int64_t M, int64_t K, int64_t N, const uint8_t* wq4, const void* sg,
                       int group, const aria_epilogue* epi, void* y, void* ws, size_t ws_bytes,
                       aria_stream_t stream) {
    if (group != 32) return ARIA_E_UNSUPPORTED;
    return wxa16(4, x, M, K, N, wq4, sg, epi, y, ws, ws_bytes, stream);
}

int aria_qlinear_grouped(int bits, int group, const aria_linear_problem* problems, int count,
                         aria_stream_t stream) {
    if (!((bits == 8 && group == 0) || (bits == 4 && group == 32))) return ARIA_E_UNSUPPORTED;
    if (!problems) return ARIA_E_NULL;
    if (count < 1 || count > kGroupedMax) return ARIA_E_SHAPE;
    const int mode = bits == 8 ? ARIA_W8A16 : ARIA_W4A16;
    // every problem on its own, as the single call checks it
    for (int i = 0; i < count; i++) {
        const aria_linear_problem& p = problems[i];
        int rc = check_shape(p.M, p.K, p.N);
        if (rc != ARIA_OK) return rc;
        if (p.M > kGroupedMaxM) return ARIA_E_UNSUPPORTED;
        if (!p.x_f16 || !p.wq || !p.s_f16 || !p.y_f16) return ARIA_E_NULL;
        if (!aligned16(p.x_f16) || !aligned16(p.wq) || !aligned16(p.s_f16) || !aligned16(p.y_f16)) return ARIA_E_ALIGN;
        if (overlap(p.x_f16, (size_t)(p.M * p.K) * 2, p.y_f16, (size_t)(p.M * p.N) * 2)) return ARIA_E_ALIAS;
        if (p.epi && p.epi->acc_out) return ARIA_E_UNSUPPORTED;
        Epi e;
        if ((rc = make_epi(p.epi, mode, p.M, p.N, p.y_f16, &e)) != ARIA_OK) return rc;
    }
    // the problems run concurrently: no output may touch another problem's buffers
    for (int i = 0; i < count; i++) {
        const aria_linear_problem& p = problems[i];
        const size_t yb = (size_t)(p.M * p.N) * 2;
        for (int j = 0; j < count; j++) {
            if (j == i) continue;
            const aria_linear_problem& q = problems[j];
            const size_t wb = bits == 8 ? (size_t)(q.N * q.K) : (size_t)(q.N * q.K) / 2;
            const size_t sb = bits == 8 ? (size_t)q.N * 2 : (size_t)q.N * (size_t)(q.K / 32) * 2;
            const size_t qy = (size_t)(q.M * q.N) * 2;
            if (overlap(p.y_f16, yb, q.x_f16, (size_t)(q.M * q.K) * 2) || overlap(p.y_f16, yb, q.wq, wb) ||
                overlap(p.y_f16, yb, q.s_f16, sb) || overlap(p.y_f16, yb, q.y_f16, qy))
                return ARIA_E_ALIAS;
            if (q.epi && ((q.epi->bias && overlap(p.y_f16, yb, q.epi->bias, (size_t)q.N * 2)) ||
                          (q.epi->residual && overlap(p.y_f16, yb, q.epi->residual, qy)) ||
                          (q.epi->steer_dir && overlap(p.y_f16, yb, q.epi->steer_dir, (size_t)q.N * 4))))
                return ARIA_E_ALIAS;
        }
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    for (int c0 = 0; c0 < count; c0 += kSkinnyGroupMax) {
        SkinnyGroup g{};
        g.count = count - c0 < kSkinnyGroupMax ? count - c0 : kSkinnyGroupMax;
        for (int i = 0; i < g.count; i++) {
            const aria_linear_problem& p = problems[c0 + i];
            SkinnyProblem& d = g.p[i];
            d.x = static_cast<const half_t*>(p.x_f16);
            d.w = static_cast<const uint8_t*>(p.wq);
            d.s = static_cast<const half_t*>(p.s_f16);
            d.y = static_cast<half_t*>(p.y_f16);
            Epi e;
            make_epi(p.epi, mode, p.M, p.N, p.y_f16, &e);   // validated above
            d.epi = EpiW{e.bias, e.residual, e.steer_dir, e.steer_alpha, e.gelu};
            d.M = (int)p.M, d.N = (int)p.N, d.K = (int)p.K;
        }
        const int rc = hip_status(launch_skinny_grouped(bits, g, st));
        if (rc != ARIA_OK) return rc;
    }
    return ARIA_OK;
}

int aria_layernorm(const void* x, int64_t M, int64_t W, const void* gamma, const void* beta, float eps, void* y,
                   aria_stream_t stream) {
    if (M < 1 || M > kMaxDim || W < 8 || W > kMaxK || W % 8 != 0) return ARIA_E_SHAPE;
    if (!(eps >= 0.0f) || eps > 1.0f) return ARIA_E_UNSUPPORTED;
    if (!x || !gamma || !beta || !y) return ARIA_E_NULL;
    if (!aligned16(x) || !aligned16(gamma) || !aligned16(beta) || !aligned16(y)) return ARIA_E_ALIGN;
    const size_t xb = (size_t)(M * W) * 2;
    if (y != x && overlap(x, xb, y, xb)) return ARIA_E_ALIAS;   // in place is fine: a row is read before written
    (void)hipGetLastError();
    return hip_status(launch_layernorm(static_cast<const half_t*>(x), static_cast<const half_t*>(gamma),
                                       static_cast<const half_t*>(beta), eps, M, W, static_cast<half_t*>(y),
                                       static_cast<hipStream_t>(stream)));
}

int aria_layernorm_quant(const void* x, int64_t M, int64_t W, const void* gamma, const void* beta, float eps,
                         void* y, int8_t* xq, void* sa, aria_stream_t stream) {
    // the quantized row feeds a W8A8 linear with K = W: its shape rules apply
    if (check_shape(M, W, 1) != ARIA_OK) return ARIA_E_SHAPE;
    if (!(eps >= 0.0f) || eps > 1.0f) return ARIA_E_UNSUPPORTED;
    if (!x || !gamma || !beta || !xq || !sa) return ARIA_E_NULL;
    if (!aligned16(x) || !aligned16(gamma) || !aligned16(beta) || !aligned16(y) || !aligned16(xq) || !aligned16(sa))
        return ARIA_E_ALIGN;
    const size_t xb = (size_t)(M * W) * 2;
    if (overlap(x, xb, xq, (size_t)(M * W)) || overlap(x, xb, sa, (size_t)M * 2) ||
        overlap(xq, (size_t)(M * W), sa, (size_t)M * 2) ||
        (y && y != x && overlap(x, xb, y, xb)) || (y && (overlap(y, xb, xq, (size_t)(M * W)) || overlap(y, xb, sa, (size_t)M * 2))))
        return ARIA_E_ALIAS;
    (void)hipGetLastError();
    return hip_status(launch_layernorm_quant(static_cast<const half_t*>(x), static_cast<const half_t*>(gamma),
                                             static_cast<const half_t*>(beta), eps, M, W, static_cast<half_t*>(y), xq,
                                             static_cast<half_t*>(sa), static_cast<hipStream_t>(stream)));
}

int aria_qlinear_w8a8_prequant(const int8_t* xq, const void* s_a, int64_t M, int64_t K, int64_t N, const int8_t* wq,
                               const void* sw, const aria_epilogue* epi, void* y, aria_stream_t stream) {
    int rc = check_shape(M, K, N);
    if (rc != ARIA_OK) return rc;
    if (!xq || !s_a || !wq || !sw || !y) return ARIA_E_NULL;
    if (!aligned16(xq) || !aligned16(s_a) || !aligned16(wq) || !aligned16(sw) || !aligned16(y)) return ARIA_E_ALIGN;
    const size_t yb = (size_t)(M * N) * 2;
    if (overlap(xq, (size_t)(M * K), y, yb) || overlap(s_a, (size_t)M * 2, y, yb)) return ARIA_E_ALIAS;
    Epi e;
    if ((rc = make_epi(epi, ARIA_W8A8, M, N, y, &e)) != ARIA_OK) return rc;
    (void)hipGetLastError();
    return hip_status(launch_gemm_tiled(0, xq, wq, static_cast<const half_t*>(sw), static_cast<const half_t*>(s_a),
                                        static_cast<half_t*>(y), (int)M, (int)N, (int)K, e,
                                        static_cast<hipStream_t>(stream)));
}

int aria_attention(const void* qkv, int64_t M, int64_t W, int64_t heads, int64_t seq, void* out, aria_stream_t stream) {
    if (M < 1 || M > kMaxDim || heads < 1 || seq < 1 || M % seq != 0) return ARIA_E_SHAPE;
    if (W != heads * 64) return ARIA_E_UNSUPPORTED;                      // 64-dimensional heads only
    if (seq * 3 * W * 2 >= ((int64_t)1 << 31) || heads > 65535 || M / seq > 65535) return ARIA_E_SHAPE;
    if (!qkv || !out) return ARIA_E_NULL;
    if (!aligned16(qkv) || !aligned16(out)) return ARIA_E_ALIGN;
    if (overlap(qkv, (size_t)(M * 3 * W) * 2, out, (size_t)(M * W) * 2)) return ARIA_E_ALIAS;
    (void)hipGetLastError();
    return hip_status(launch_attention(static_cast<const half_t*>(qkv), M, W, heads, seq, static_cast<half_t*>(out),
                                       static_cast<hipStream_t>(stream)));
}

int aria_qlinear_w16a16(const void* x, int64_t M, int64_t K, int64_t N, const void* wt, const aria_epilogue* epi,
                        void* y, void* ws, size_t ws_bytes, aria_stream_t stream) {
    return wxa16(16, x, M, K, N, wt, nullptr, epi, y, ws, ws_bytes, stream);
}

}  // extern "C"
