// a3+a4+a5 — the tiled quantized GEMM for M > 64, all modes, with the fused
// epilogue.
//
// What is computed (aria project page, "What aria is" / "Results": weights
// stored at 8 or 4 bits; W8A8 runs 8-bit arithmetic on integer matrix units;
// fp16 is the unquantized row the modes are compared with):
//   W8A8 : acc = sum_k Xq[m][k] * Wq[n][k] (exact int32);  y = acc * s_a[m] * s_w[n]
//   W8A16: acc = sum_k X[m][k] * Wq[n][k]  (fp32; int8 -> fp16 is exact);  y = acc * s_w[n]
//   W4A16: acc = sum_k X[m][k] * fp16(q4[n][k] * s_g[n][k/32])  (fp32);  y = acc
//   W16A16: acc = sum_k X[m][k] * Wt[n][k]  (fp32);  y = acc
// then y -> + bias -> GELU -> + residual -> + alpha d -> fp16.
//
// Design (gfx950): a workgroup of WM x WN waves (4, 6, 8, 12 or 16; a 4- or
// 6-wave tile may also run as two such groups that split the K-steps) owns a BM x BN
// output tile; each wave owns (BM/WM) x (BN/WN) as 32x32 blocks on the matrix cores
// (v_mfma_i32_32x32x32_i8 or v_mfma_f32_32x32x16_f16).  Both operands live in
// LDS as rows of 128 bytes (128 int8 k or 64 fp16 k) plus a 16-byte pad that
// spreads the 32 rows of an operand fragment over all banks; a K-step is 4
// MFMA sub-steps in every mode.  Tiles are fetched two K-steps ahead (three
// with a second register set: 4-wave tiles and the 12-wave W8A16 tile) into
// registers with bounds-checked buffer loads (rows past M/N and k past K read
// as zero), and the decode + LDS store of the next one is split over the
// first 3 sub-steps of the current K-step so that it overlaps the matrix
// work (for most tiles pinned there by scheduling barriers, see PIN).  The
// one barrier per K-step comes after the third sub-step: the next tile is
// then complete in LDS, and its first fragments are read while the last
// sub-step's MFMAs run (a barrier at the end of the K-step left every wave
// waiting on those reads with nothing to issue).  Packed weights are decoded
// in registers (decode.h: fp16 patterns 0x6400 | u and, for the codes left in
// mantissa bits 4-7, 0x5400 | u << 4, minus their offsets), two values per
// packed-half instruction.  The epilogue stages the accumulators through LDS and writes
// 16-byte rows of fp16 with non-temporal stores.
#include <type_traits>

#include "common.h"
#include "decode.h"
#include "kernels.h"

namespace aria {

namespace {

template <int MODE>
struct ModeT;
template <>
struct ModeT<0> {  // W8A8
    static constexpr int KSTEP = 128;        // k per 128-byte row
    static constexpr int AEB = 1;            // A element bytes
    static constexpr int KPB = 16;           // k per 16-byte packed weight chunk
    static constexpr int BCH = 8;            // packed weight chunks per row per K-step
    typedef v16i acc_t;
};
template <>
struct ModeT<1> {  // W8A16
    static constexpr int KSTEP = 64, AEB = 2, KPB = 16, BCH = 4;
    typedef v16f acc_t;
};
template <>
struct ModeT<2> {  // W4A16
    static constexpr int KSTEP = 64, AEB = 2, KPB = 32, BCH = 2;
    typedef v16f acc_t;
};
template <>
struct ModeT<3> {  // W16A16 (fp16 weights, the unquantized rung)
    static constexpr int KSTEP = 64, AEB = 2, KPB = 8, BCH = 8;
    typedef v16f acc_t;
};
template <>
struct ModeT<4> {  // W8A8, X fp16 quantized per token as it is staged (A in LDS as int8)
    static constexpr int KSTEP = 128, AEB = 2, KPB = 16, BCH = 8;
    typedef v16i acc_t;
};

}  // namespace

template <int MODE, int BM, int BN, int WM, int WN, int KS>
__global__ __launch_bounds__(WM * WN * KS * WAVE) void gemm_tiled_kernel(const void* __restrict__ Aptr, const uint8_t* __restrict__ Bq,
                                                         const half_t* __restrict__ S, const half_t* __restrict__ sa,
                                                         half_t* Y, int M, int N, int K, Epi epi, AQuant aq) {
    using T = ModeT<MODE>;
    constexpr bool I8 = MODE == 0 || MODE == 4;   // int8 operands on the integer matrix cores
    constexpr bool QA = MODE == 4;                // A quantized per token while staged
    constexpr int ACH = QA ? 16 : 8;              // 16-byte A chunks per row per K-step
    constexpr int NT = WM * WN * WAVE;
    constexpr int ROWB = 144;                    // LDS bytes per row (128 + pad)
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    // 4-bit weights come in 8-byte chunks (16 k) where 16-byte ones would leave
    // waves idle: the 12-wave 256x192 tile has 384 of those for 768 threads
    constexpr bool HALF4 = MODE == 2 && (BN * T::BCH) % (WM * WN * WAVE) != 0 &&
                           (2 * BN * T::BCH) % (WM * WN * WAVE) == 0;
    constexpr int KPB = HALF4 ? T::KPB / 2 : T::KPB;   // k per packed B chunk
    constexpr int BCH = HALF4 ? 2 * T::BCH : T::BCH;   // packed B chunks per row per K-step
    constexpr int NA = BM * ACH;                 // 16-byte A chunks per K-step
    constexpr int NB = BN * BCH;                 // packed B chunks per K-step
    constexpr int LA = (NA + NT - 1) / NT;
    constexpr int LB = (NB + NT - 1) / NT;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0 && NA % WAVE == 0 && NB % WAVE == 0, "tile shape");

    // KS = 2: two groups of WM x WN waves share the tile and split its
    // K-steps (group g takes g, g + 2, ...), each with its own double buffer
    // and pipeline; their partial sums meet in LDS before the epilogue.  For
    // tiles that leave one workgroup per CU this doubles the waves per SIMD.
    static_assert(KS == 1 || KS == 2, "K split");
    __shared__ __attribute__((aligned(16))) char lds[2 * KS][(BM + BN) * ROWB];

    // Tile order: groups of GM row-blocks, column-major inside a group, after
    // the XCD remap; the 32 consecutive tiles one XCD runs then form a compact
    // (GM x 8) block, so its L2 holds GM row-blocks of X instead of all of them.
    constexpr int GM = 4;
    const int ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int first_m = (bid / (GM * ntn)) * GM;
    const int gsize = min(ntm - first_m, GM);
    const int in_group = bid % (GM * ntn);
    const int tm = first_m + in_group % gsize, tn = in_group / gsize;
    const int m0 = tm * BM, n0 = tn * BN;
    // tid and wave count within the thread's K group
    const int grp = KS == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)threadIdx.x / NT);
    const int tid = (int)threadIdx.x % NT, wave = tid / WAVE, lane = tid % WAVE;
    const int wm = wave / WN, wn = wave % WN;
    char(*const glds)[(BM + BN) * ROWB] = lds + 2 * grp;   // this group's two buffers

    const int lda = QA ? aq.lda : K;             // A row stride in elements
    const uint32_t abytes = QA ? (uint32_t)((M - 1) * lda + K) * T::AEB : (uint32_t)M * (uint32_t)K * T::AEB;
    const uint32_t browb = MODE == 2 ? (uint32_t)K / 2 : MODE == 3 ? (uint32_t)K * 2 : (uint32_t)K;
    const rsrc_t ra = make_rsrc(Aptr, abytes);
    const rsrc_t rb = make_rsrc(Bq, (uint32_t)N * browb);
    const int G = K / 32;

    // per-thread chunk coordinates (fixed across K-steps)
    // 4- and 6-wave tiles keep the next-but-one tile in a second register
    // set, so a load has a whole K-step to land (6 waves, 64x96 at M = 256:
    // W8A16 13.7 -> 11.7 us, W8A8 -5 %); so does the 12-wave W8A16 tile
    // (168 VGPRs, +5 % measured).  Elsewhere the second set cost 1-6 %
    // (8-wave tiles; the 12-wave W4A16 tile, 167 VGPRs: 1-2 %, on the pinned
    // or the free schedule) or spilled (12-wave W8A8), and the extra waves
    // per SIMD hide the latency instead.
    constexpr int NSET = WM * WN == 4 || WM * WN == 6 || (WM * WN == 12 && MODE == 1) ? 2 : 1;
    // PIN: every part's loads and stores stay in their sub-step (a scheduling
    // barrier after each), and every wave issues the same loads (see load_a),
    // so the compiler's waits give each load a whole K-step to land; without
    // it the compiler gathered the stores of several parts into one sub-step
    // and, around the branches of chunks that some waves skip, waited for all
    // loads.  Measured per tile and mode over eight layer shapes: +5-9 % for
    // 8-wave tiles and for W8A8 on the 12-wave tile, +2 % W8A16 there; the
    // W4A16 12-wave tile and the 16-wave tile outside W8A8 lose 3-5 % with it,
    // so they keep the free schedule.  The 4-wave tiles (two register sets)
    // always pin.
    constexpr bool PIN = NSET >= 2 || WM * WN == 8 || I8 || (WM * WN == 12 && MODE != 2);
    v4i RA[NSET][LA], RB[NSET][LB > 0 ? LB : 1];
    half_t RS[NSET][LB > 0 ? LB : 1];

    // `ok` false: the chunk does not exist for this wave.  With PIN the load
    // still issues (an out-of-range offset reads zero and moves no data), so
    // every wave issues the same loads in the same order and the compiler can
    // count them exactly when it places its waits (a branch around a load
    // makes it wait for the loads of both paths); otherwise it is skipped.
    auto load_a = [&](int kt, int i, int set, bool ok) {
        const int c = tid + i * NT, row = c / ACH, ch = c % ACH;
        const int k = (kt * KS + grp) * T::KSTEP + ch * (16 / T::AEB);
        const uint32_t off = (uint32_t)(m0 + row) * (uint32_t)(QA ? lda : K) * T::AEB + (uint32_t)k * T::AEB;
        RA[set][i] = buf_load16(ra, ok && k < K && m0 + row < M ? off : OOB);
    };
    auto load_b = [&](int kt, int i, int set, bool ok) {
        const int c = tid + i * NT, row = c / BCH, ch = c % BCH;
        const int k = (kt * KS + grp) * T::KSTEP + ch * KPB;
        const bool in = ok && k < K && n0 + row < N;
        const uint32_t off = (uint32_t)(n0 + row) * browb + (uint32_t)(MODE == 2 ? k / 2 : MODE == 3 ? 2 * k : k);
        if constexpr (HALF4) {
            const v2u h = buf_load8(rb, in ? off : OOB);
            RB[set][i] = v4i{(int)h[0], (int)h[1], 0, 0};
        } else {
            RB[set][i] = buf_load16(rb, in ? off : OOB);
        }
        if (MODE == 2) RS[set][i] = S[(int64_t)min(n0 + row, N - 1) * G + min(k, K - 32) / 32];
    };
    // QA: this thread's A rows keep one scale each for the whole K loop
    // (chunk i of the thread is in row (tid + i NT) / 16 at every K-step)
    float qdiv[QA ? LA : 1], qrcp[QA ? LA : 1];
    auto store_a = [&](int buf, int i, int set) {
        const int c = tid + i * NT, row = c / ACH, ch = c % ACH;
        if constexpr (QA) {
            // the per-token quantizer's arithmetic (rowops.h quantize_row) on
            // these 8 values: rint(x * RN(1/s)), the exact tie test where a
            // lane of the wave lands near a half-integer, clamp to +-127
            const v8h x = __builtin_bit_cast(v8h, RA[set][i]);
            float f[8], q[8];
            float dmax = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                f[e] = (float)x[e] * qrcp[i];
                q[e] = __builtin_rintf(f[e]);
                dmax = __builtin_fmaxf(dmax, __builtin_fabsf(f[e] - q[e]));
            }
            if (__builtin_amdgcn_ballot_w64(dmax >= 0.5f - 0x1p-15f) != 0) {
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const float qf = __builtin_floorf(f[e]) + 0.5f;
                    q[e] = __builtin_rintf(__builtin_fmaf(qf, qdiv[i], -(float)x[e]) == 0.0f ? qf : f[e]);
                }
            }
            u32 w[2];
#pragma unroll
            for (int h = 0; h < 2; h++) {
                u32 b[4];
#pragma unroll
                for (int e = 0; e < 4; e++) b[e] = (u32)(int)__builtin_amdgcn_fmed3f(q[4 * h + e], -127.0f, 127.0f);
                w[h] = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[3], b[2], 0x0C0C0400u),
                                             __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u), 0x05040100u);
            }
            *reinterpret_cast<v2u*>(&glds[buf][row * ROWB + ch * 8]) = v2u{w[0], w[1]};
        } else {
            *reinterpret_cast<v4i*>(&glds[buf][row * ROWB + ch * 16]) = RA[set][i];
        }
    };
    auto store_b = [&](int buf, int i, int set) {
        const int c = tid + i * NT;
        const int row = c / BCH, ch = c % BCH;
        char* dst = &glds[buf][(BM + row) * ROWB + ch * (KPB * 2 / (I8 ? 2 : 1))];
        if constexpr (I8 || MODE == 3) {
            *reinterpret_cast<v4i*>(dst) = RB[set][i];
        } else if constexpr (MODE == 1) {
            v4i lo, hi;
            dec8(RB[set][i], lo, hi);
            reinterpret_cast<v4i*>(dst)[0] = lo;
            reinterpret_cast<v4i*>(dst)[1] = hi;
        } else {
            constexpr int ND = HALF4 ? 2 : 4;
            v4i o[ND];
            dec4<ND>(RB[set][i], RS[set][i], o);
#pragma unroll
            for (int q = 0; q < ND; q++) reinterpret_cast<v4i*>(dst)[q] = o[q];
        }
    };
    // chunk i of this thread exists unless the chunk count is not a multiple
    // of the thread count and the thread is past the end: a whole wave at a
    // time (both counts are multiples of 64), so the test is wave-uniform
    const int wbase = __builtin_amdgcn_readfirstlane(wave) * WAVE;
    // (rounds that every wave fills are folded to true only under PIN: on the
    // free schedule the branches happen to place the code better, by 1-3 %)
    auto has_a = [&](int i) { return (PIN && (i + 1) * NT <= NA) || NA % NT == 0 || wbase + i * NT < NA; };
    auto has_b = [&](int i) { return (PIN && (i + 1) * NT <= NB) || NB % NT == 0 || wbase + i * NT < NB; };
    auto load_part = [&](int kt, int p, int set) {
#pragma unroll
        for (int i = p; i < LA; i += 4)
            if (PIN || has_a(i)) load_a(kt, i, set, has_a(i));
#pragma unroll
        for (int i = p; i < LB; i += 4)
            if (PIN || has_b(i)) load_b(kt, i, set, has_b(i));
    };
    auto store_part = [&](int buf, int p, int set) {
#pragma unroll
        for (int i = p; i < LA; i += 4)
            if (has_a(i)) store_a(buf, i, set);
#pragma unroll
        for (int i = p; i < LB; i += 4)
            if (has_b(i)) store_b(buf, i, set);
    };

    // QA: the per-token scales of the tile's rows, from the producer's row
    // maxima (four threads per row, an integer max over the fp16 magnitude
    // bits as in the quantizer), then s_a = fp16(max / 127) and 1 / s_a as the
    // quantizer computes them
    __shared__ half_t qs[QA ? BM : 1];
    if constexpr (QA) {
        const int nslot = K / 64;
        for (int r = (int)threadIdx.x; r < BM * 4; r += (int)blockDim.x) {
            const int row = r / 4, part = r % 4, m = m0 + row;
            uint32_t mx = 0;
            if (m < M)
                for (int j = part; j < nslot; j += 4) mx = max(mx, aq.amax[(int64_t)m * aq.amax_ld + j]);
            mx = max(mx, (uint32_t)__shfl_xor((int)mx, 1, WAVE));
            mx = max(mx, (uint32_t)__shfl_xor((int)mx, 2, WAVE));
            if (part == 0) {
                const half_t sh = (half_t)((float)__builtin_bit_cast(half_t, (uint16_t)mx) / 127.0f);
                qs[row] = sh;
                if (aq.sa_out && tn == 0 && m < M) aq.sa_out[m] = sh;
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < LA; i++) {
            const float sf = (float)qs[min((tid + i * NT) / ACH, BM - 1)];
            qdiv[i] = sf == 0.0f ? 1.0f : sf;   // an all-zero row quantizes to zeros either way
            qrcp[i] = 1.0f / qdiv[i];
        }
    }

    typename T::acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int j = 0; j < FN; j++) acc[i][j] = typename T::acc_t{};

    // K-steps per group (with KS = 2 the second group may run one past K:
    // its loads read zero, so both groups meet every barrier)
    const int nk = ((K + T::KSTEP - 1) / T::KSTEP + KS - 1) / KS;
#pragma unroll
    for (int p = 0; p < 4; p++) load_part(0, p, 0);
#pragma unroll
    for (int p = 0; p < 4; p++) store_part(0, p, 0);
    // tiles 1 .. NSET into register sets n % NSET (tile t lives in set t % NSET)
#pragma unroll
    for (int n = 1; n <= NSET; n++)
#pragma unroll
        for (int p = 0; p < 4; p++) load_part(n, p, n % NSET);
    __syncthreads();

    const int arow = (wm * WTM + lane % 32) * ROWB + (lane / 32) * 16;
    const int brow = (BM + wn * WTN + lane % 32) * ROWB + (lane / 32) * 16;
    v4i fa[2][FM], fb[2][FN];
    auto read_frags = [&](const char* L, int p, int slot) {
#pragma unroll
        for (int i = 0; i < FM; i++) fa[slot][i] = *reinterpret_cast<const v4i*>(L + arow + i * 32 * ROWB + p * 32);
#pragma unroll
        for (int j = 0; j < FN; j++) fb[slot][j] = *reinterpret_cast<const v4i*>(L + brow + j * 32 * ROWB + p * 32);
    };
    // The loop body has no branches: the last K-steps load past K (zero-fill,
    // no memory traffic) and store into the idle buffer, which nothing reads.
    // Register set `set` holds tile kt + 1 (stored during K-step kt); with two
    // sets the tile after the next-but-one is requested into it once stored.
    // The barrier after sub-step 2 publishes tile kt + 1; every wave has read
    // all fragments of tile kt by then (sub-step 3's were read during sub-step
    // 2), so the next K-step may overwrite tile kt's buffer.
    auto kstep = [&](int kt, auto set_c) {
        constexpr int set = decltype(set_c)::value;
        const int cur = kt & 1;
        const char* L = glds[cur];
#pragma unroll
        for (int p = 0; p < 4; p++) {
            if (p < 3) read_frags(L, p + 1, (p + 1) & 1);
            else read_frags(glds[cur ^ 1], 0, 0);   // the next tile's first sub-step: visible since the barrier
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++) {
                    if constexpr (I8)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[p & 1][i], fb[p & 1][j], acc[i][j], 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, fa[p & 1][i]),
                                                                           __builtin_bit_cast(v8h, fb[p & 1][j]),
                                                                           acc[i][j], 0, 0, 0);
                }
            if (p < 3) {
                store_part(cur ^ 1, p, set);
                load_part(kt + 1 + NSET, p, set);
                if (p == 2) {
                    store_part(cur ^ 1, 3, set);
                    load_part(kt + 1 + NSET, 3, set);
                    __syncthreads();
                }
            }
            if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
        }
    };
    read_frags(glds[0], 0, 0);
    // K-step kt stores tile kt + 1 from set (kt + 1) % NSET: unrolled by NSET
    // (a third set for the 4-wave tiles measured 1-7 % slower)
    static_assert(NSET == 1 || NSET == 2, "register sets");
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1 % NSET>;
    if constexpr (NSET == 2) {
        int kt = 0;
        for (; kt + 1 < nk; kt += 2) {
            kstep(kt, S1{});
            kstep(kt + 1, S0{});
        }
        if (kt < nk) kstep(kt, S1{});
    } else {
        for (int kt = 0; kt < nk; kt++) kstep(kt, S0{});
    }

    if constexpr (KS == 2) {
        // Group 1 parks its partial sums in LDS past group 0's epilogue
        // staging area; group 0 adds them (one fixed order: the result does
        // not depend on timing) and runs the epilogue alone.
        constexpr int STAGE_BYTES = WM * WN * 32 * (WTN + 8) * 4;
        constexpr int PARK_BYTES = WM * WN * FM * FN * 16 * WAVE * 4;
        static_assert(STAGE_BYTES + PARK_BYTES <= (int)sizeof(lds), "K-split partial sums must fit in LDS");
        uint32_t* park = reinterpret_cast<uint32_t*>(&lds[0][0] + STAGE_BYTES) + wave * FM * FN * 16 * WAVE + lane;
        __syncthreads();   // every wave is done with the tile buffers
        if (grp == 1) {
#pragma unroll
            for (int i = 0; i < FM; i++)
#pragma unroll
                for (int j = 0; j < FN; j++)
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const auto v = acc[i][j][r];
                        park[((i * FN + j) * 16 + r) * WAVE] = __builtin_bit_cast(uint32_t, v);
                    }
        }
        __syncthreads();
        if (grp == 1) return;
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int j = 0; j < FN; j++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const uint32_t v = park[((i * FN + j) * 16 + r) * WAVE];
                    if constexpr (I8)
                        acc[i][j][r] += (int32_t)v;
                    else
                        acc[i][j][r] += __builtin_bit_cast(float, v);
                }
    }

    // Epilogue.  Each wave stages one 32-row block-row of its raw accumulators
    // at a time in its own slice of the (now idle) LDS, transposing the 32x32
    // MFMA layout (register r of lane l = row 8*(r/4) + 4*(l/32) + r%4, column
    // l%32) into rows; each lane then owns 8 consecutive columns of one row,
    // so scales, bias, residual, d and the fp16 output move as 16-byte
    // vectors.  A row stride of WTN + 8 words puts the two 32-lane halves of a
    // staging write on disjoint banks.
    constexpr int SROW = WTN + 8;
    constexpr int CPRW = WTN / 8;                         // 8-column chunks per staged row
    constexpr int TASKS = 32 * CPRW / WAVE;               // chunks per lane per block-row
    static_assert((32 * CPRW) % WAVE == 0, "epilogue chunks must split over the wave");
    static_assert(WM * WN * 32 * SROW * 4 <= (int)sizeof(lds), "epilogue staging must fit in LDS");
    uint32_t* stage = reinterpret_cast<uint32_t*>(&lds[0][0]) + wave * 32 * SROW;
    const float alpha = load_alpha(epi);
    const bool vec_ok = (N % 8) == 0;
    const v8h zero8 = {};
    // When the wave's row of chunks divides the wave (64-column wave tiles),
    // every task of a lane covers the same 8 columns: their scales, bias and
    // steering vector are then read and converted once per lane, not once
    // per task and block-row.
    constexpr bool COLFIX = WAVE % CPRW == 0;
    const int colf = n0 + wn * WTN + (lane % CPRW) * 8;
    const bool cvalid = COLFIX && vec_ok && colf + 8 <= N;
    float swf[8], bf[8], df[8];
    if constexpr (COLFIX) {
        const v8h s8 = ((I8 || MODE == 1) && cvalid) ? *reinterpret_cast<const v8h*>(S + colf) : zero8;
        const v8h b8 = (epi.bias && cvalid) ? *reinterpret_cast<const v8h*>(epi.bias + colf) : zero8;
        const v4f z4 = {};
        const v4f d0 = (alpha != 0.0f && cvalid) ? *reinterpret_cast<const v4f*>(epi.steer_dir + colf) : z4;
        const v4f d1 = (alpha != 0.0f && cvalid) ? *reinterpret_cast<const v4f*>(epi.steer_dir + colf + 4) : z4;
#pragma unroll
        for (int e = 0; e < 8; e++) {
            swf[e] = (float)s8[e];
            bf[e] = (float)b8[e];
            df[e] = e < 4 ? d0[e] : d1[e - 4];
        }
    }
#pragma unroll
    for (int i = 0; i < FM; i++) {
        // 1) issue this round's per-element operand loads (column scales,
        //    per-row scale, residual) first, so their latency overlaps the
        //    staging below; bias and d are small, shared by every row and
        //    cache-resident, so they are read where they are used
        v8h sw8[TASKS], r8[TASKS];
        float sr[TASKS];
#pragma unroll
        for (int t = 0; t < TASKS; t++) {
            const int task = lane + t * WAVE, rr = task / CPRW, cc = task % CPRW;
            const int row = m0 + wm * WTM + i * 32 + rr, col = n0 + wn * WTN + cc * 8;
            const bool v = vec_ok && row < M && col + 8 <= N;
            const int64_t base = (int64_t)row * N + col;
            sw8[t] = ((I8 || MODE == 1) && v && !COLFIX) ? *reinterpret_cast<const v8h*>(S + col) : zero8;
            sr[t] = !(I8 && v) ? 0.0f : QA ? (float)qs[row - m0] : (float)sa[row];
            r8[t] = (epi.residual && v) ? *reinterpret_cast<const v8h*>(epi.residual + base) : zero8;
        }
        // 2) stage the raw accumulators of block-row i
#pragma unroll
        for (int j = 0; j < FN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int rr = 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
                // copy the element out first: a bit cast of a vector-element
                // lvalue reads the vector's first element, not element r
                const auto val = acc[i][j][r];
                stage[rr * SROW + j * 32 + lane % 32] = __builtin_bit_cast(uint32_t, val);
            }
        // the slice is this wave's own: LDS executes one wave's accesses in
        // order, so a wavefront-scope fence (which keeps the compiler from
        // reordering) is all the staging needs; a workgroup barrier would
        // also wait for this wave's outstanding global stores
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        // 3) finish 8 consecutive columns of one row per task
#pragma unroll
        for (int t = 0; t < TASKS; t++) {
            const int task = lane + t * WAVE, rr = task / CPRW, cc = task % CPRW;
            const int row = m0 + wm * WTM + i * 32 + rr, col = n0 + wn * WTN + cc * 8;
            // row maxima for a later per-token quantization (W8A8 kernels with
            // 64-column wave tiles only): the eight lanes of a row hold its 64
            // columns, so the block's maximum is a reduction over those lanes
            // (all lanes take part in the shuffles; lanes past M or N give 0)
            constexpr bool RMX = MODE == 0 && CPRW == 8;
            if constexpr (!RMX) {
                if (row >= M || col >= N) continue;
            }
            uint32_t mbits = 0;
            if (!RMX || (row < M && col < N)) {
            // read with the element type the staging stores used (a vector-typed
            // load of scalar-typed stores would let alias analysis drop them)
            uint32_t raw[8];
#pragma unroll
            for (int e = 0; e < 8; e++) raw[e] = stage[rr * SROW + cc * 8 + e];
            const int64_t base = (int64_t)row * N + col;
            if (vec_ok && col + 8 <= N) {
                float v[8];
                if constexpr (I8) {
                    if (epi.acc_out) {
                        reinterpret_cast<v4u*>(epi.acc_out + base)[0] = v4u{raw[0], raw[1], raw[2], raw[3]};
                        reinterpret_cast<v4u*>(epi.acc_out + base)[1] = v4u{raw[4], raw[5], raw[6], raw[7]};
                    }
#pragma unroll
                    for (int e = 0; e < 8; e++)
                        v[e] = (float)(int32_t)raw[e] * sr[t] * (COLFIX ? swf[e] : (float)sw8[t][e]);
                } else if constexpr (MODE == 1) {
#pragma unroll
                    for (int e = 0; e < 8; e++) v[e] = __builtin_bit_cast(float, raw[e]) * (COLFIX ? swf[e] : (float)sw8[t][e]);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; e++) v[e] = __builtin_bit_cast(float, raw[e]);
                }
                if (epi.bias) {
                    if constexpr (COLFIX) {
#pragma unroll
                        for (int e = 0; e < 8; e++) v[e] += bf[e];
                    } else {
                        const v8h b8 = *reinterpret_cast<const v8h*>(epi.bias + col);
#pragma unroll
                        for (int e = 0; e < 8; e++) v[e] += (float)b8[e];
                    }
                }
                if (epi.gelu) {
#pragma unroll
                    for (int e = 0; e < 8; e++) v[e] = gelu_tanh(v[e]);
                }
                if (epi.residual) {
#pragma unroll
                    for (int e = 0; e < 8; e++) v[e] += (float)r8[t][e];
                }
                if (alpha != 0.0f) {
                    if constexpr (COLFIX) {
#pragma unroll
                        for (int e = 0; e < 8; e++) v[e] += alpha * df[e];
                    } else {
                        const v4f d0 = *reinterpret_cast<const v4f*>(epi.steer_dir + col);
                        const v4f d1 = *reinterpret_cast<const v4f*>(epi.steer_dir + col + 4);
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            v[e] += alpha * d0[e];
                            v[e + 4] += alpha * d1[e];
                        }
                    }
                }
                v8h out;
#pragma unroll
                for (int e = 0; e < 8; e++) out[e] = (half_t)v[e];
                if constexpr (RMX) {
                    if (epi.rowmax) {
#pragma unroll
                        for (int e = 0; e < 8; e++) {
                            const half_t oe = out[e];   // copied out: see the staging note above
                            mbits = max(mbits, (uint32_t)(__builtin_bit_cast(uint16_t, oe) & 0x7FFFu));
                        }
                    }
                }
                // non-temporal store: nothing in this launch reads the output
                // again (measured on MI355X: +1-3 % per launch, +1.5 % on the
                // DiT step, whose next kernel reads this output)
                __builtin_nontemporal_store(out, reinterpret_cast<v8h*>(Y + base));
            } else {
                // ragged right edge (or N % 8 != 0): element by element
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    if (col + e >= N) break;
                    const int64_t idx = base + e;
                    float v;
                    if constexpr (I8) {
                        if (epi.acc_out) epi.acc_out[idx] = (int32_t)raw[e];
                        v = (float)(int32_t)raw[e] * (QA ? (float)qs[row - m0] : (float)sa[row]) * (float)S[col + e];
                    } else if constexpr (MODE == 1) {
                        v = __builtin_bit_cast(float, raw[e]) * (float)S[col + e];
                    } else {
                        v = __builtin_bit_cast(float, raw[e]);
                    }
                    Y[idx] = (half_t)epilogue_apply(v, idx, col + e, epi, alpha);
                }
            }
            }
            if constexpr (RMX) {
                if (epi.rowmax) {
                    mbits = max(mbits, (uint32_t)__shfl_xor((int)mbits, 1, WAVE));
                    mbits = max(mbits, (uint32_t)__shfl_xor((int)mbits, 2, WAVE));
                    mbits = max(mbits, (uint32_t)__shfl_xor((int)mbits, 4, WAVE));
                    const int c64 = n0 + wn * WTN;   // this wave's 64 columns
                    if (cc == 0 && row < M && c64 >= epi.rowmax_c0 && c64 < epi.rowmax_c1)
                        epi.rowmax[(int64_t)row * epi.rowmax_ld + (c64 - epi.rowmax_c0) / 64] = mbits;
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");   // before the next round restages the slice
    }
}

// ---------------------------------------------------------------------------
// host side: tile choice and launch
// ---------------------------------------------------------------------------
namespace {

struct TileCfg {
    int bm, bn, wm, wn, ks;  // ks: K groups per workgroup (workgroup = wm x wn x ks waves)
    float eff[4];  // sustained throughput of one full wave of such tiles, per mode (relative units)
};

// Candidate macro tiles with their measured per-tile efficiency on MI355X, by
// mode W8A8 / W8A16 / W4A16 / W16A16: for each tile, waves x BM x BN x K / time
// (relative units), the median over eight layer shapes at M = 2048 (the DiT
// block's four linears at width 1536 and the four of the 1.2B-scale step at
// width 2048), then adjusted so that the picker's choice is within 1 % of the
// fastest tile on those shapes.  The picker minimises
//   ceil(tiles / CUs) * BM * BN / eff
// i.e. it trades CU fill (whole waves of tiles) against per-tile efficiency.
// 8-, 12- and 16-wave workgroups put two, three or four waves on every SIMD so
// one can issue while the others wait on LDS or memory; 64x64 per wave (the
// 12-wave 256x192 and 16-wave 256x256 tiles) beat 64x96 and 64x128 per wave
// with fewer waves (the 16-wave 256x256 entries are the 8-wave 256x256 ones
// scaled by what the two measured against each other: +17 % W8A8, +7 %
// W8A16, +2 % W16A16, equal for W4A16).  Every entry was then scaled by the
// measured gain of the pinned schedule (geomean over the same shapes).
constexpr TileCfg kTiles[] = {
    {256, 192, 4, 3, 1, {4304.f, 2622.f, 2432.f, 2504.f}}, {256, 256, 4, 4, 1, {4701.f, 2640.f, 2560.f, 2736.f}},
    {256, 192, 4, 2, 1, {3927.f, 2397.f, 2187.f, 2483.f}}, {256, 128, 4, 2, 1, {3344.f, 2122.f, 2008.f, 2130.f}},
    {128, 256, 2, 4, 1, {3470.f, 2126.f, 1833.f, 2127.f}}, {128, 192, 2, 2, 1, {2388.f, 1528.f, 1496.f, 1643.f}},
    {128, 128, 2, 2, 1, {2683.f, 1889.f, 1577.f, 1894.f}}, {64, 192, 2, 2, 1, {2335.f, 1379.f, 1140.f, 1406.f}},
    {128, 64, 2, 2, 1, {2235.f, 1335.f, 1222.f, 1353.f}},  {64, 128, 2, 2, 1, {2292.f, 1290.f, 1105.f, 1340.f}},
    {64, 64, 2, 2, 1, {2076.f, 1182.f, 960.f, 1153.f}},
    // two K groups: the 4-wave entries scaled by what the split measured
    // where it applies (one workgroup per CU, K >= 1024): W8A16 / W4A16
    // +12-16 % (+20 % at K = 6144 and 8192), W16A16 +1-2 %, W8A8 -2-5 %
    {64, 192, 2, 2, 2, {2218.f, 1600.f, 1322.f, 1420.f}}, {128, 128, 2, 2, 2, {2629.f, 2116.f, 1814.f, 1932.f}},
    // the 128x64 and 64x128 tiles with two K groups, measured at M = 256,
    // 1536 -> 6144 over one group: W8A16 +10 % / +19 %, W4A16 +15 % / +16 %;
    // W8A8 and W16A16 no gain, so priced just below the one-group entries
    {128, 64, 2, 2, 2, {2200.f, 1468.f, 1404.f, 1340.f}}, {64, 128, 2, 2, 2, {2260.f, 1535.f, 1284.f, 1330.f}},
    // 6 waves, 64x96: 256 tiles at M = 256, N = 6144 (one per CU where the
    // 128x64 tile leaves 64 CUs idle); fitted at that shape against the
    // 128x64 tile: W8A8 12.5 -> 11.4 us, W8A16 13.3 -> 11.8, W4A16 14.1 ->
    // 13.4, W16A16 15.2 -> 13.7
    {64, 96, 2, 3, 1, {1832.f, 1125.f, 962.f, 1124.f}},
    // 6 waves of 64x32, 128x96: 256 tiles for a 2048 x 1536 output, with
    // (128 + 96) K operand rows per tile where 64x192 streams (64 + 192);
    // measured at M = 2048, N = 1536 against the picks before it (act-quant
    // included for W8A8): W8A8 K = 1536 17.8 -> 16.8 us, K = 6144 43.0 ->
    // 39.7; W8A16 17.8 -> 15.8 and 52.1 -> 51.9; W4A16 -7 % at K = 1536 but
    // +5 % at K = 6144, so it is priced below the 128x128 two-group tile
    // there (W16A16 not measured, priced below 64x192)
    {128, 96, 2, 3, 1, {2491.f, 1650.f, 1300.f, 1300.f}},
    // 8 waves of 64x32, 128x128: measured at M = N = 2048 against the 4-wave
    // tile, K = 2048: W8A8 22.6 -> 20.8 us, W8A16 23.5 -> 22.2, W4A16 26.2 ->
    // 25.0; K = 8192: W8A8 the same, W8A16 / W4A16 slower than the two-group
    // 4-wave tile, which keeps the higher price for those modes
    {128, 128, 2, 4, 1, {2926.f, 2002.f, 1650.f, 1880.f}},
    // the 6-wave 64x96 tile with two K groups (12 waves, one workgroup per
    // CU) for mid-size M, where a tile's K-loop is a latency chain: halving
    // the chain paid for the weight-only modes, measured against the picks
    // before it (interleaved graph replays, two runs): W8A16 M = 256,
    // 1536 -> 6144 11.9 -> 10.8 us, 8192 -> 2048 39.5 -> 35.4 us; W4A16
    // 8192 -> 2048 43.7 -> 38.8 us, M = 192, 1536 -> 4608 12.3 -> 10.8 us,
    // within +-4 % at M = 128 and 256, 1536 -> 6144; W8A8 slower everywhere
    {64, 96, 2, 3, 2, {1000.f, 1800.f, 1500.f, 1000.f}}};

int num_cus() {
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        hipDeviceProp_t p;
        if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&p, dev) == hipSuccess) cus = p.multiProcessorCount;
        if (cus <= 0) cus = 256;
    }
    return cus;
}

// The fused-quantization form (mode 4) holds twice the A chunks in
// registers: on the 12- and 16-wave tiles and the K-split 128x128 tile it
// spills, so it does not use them.
bool tile_ok(const TileCfg& t, int mode, bool wave64) {
    if (wave64 && t.bn / t.wn != 64) return false;
    if (mode == 4 && (t.wm * t.wn >= 12 || t.ks > 1)) return false;
    return true;
}

// wave64: only tiles whose waves are 64 columns wide (the row-maxima output)
const TileCfg& pick_tile(int mode, int M, int N, int K, bool wave64 = false) {
    const char* env = getenv("ARIA_QLINEAR_TILE");  // "BMxBNxWMxWN[xKS]" tuning override
    if (env) {
        int bm = 0, bn = 0, wm = 0, wn = 0, ks = 1;
        if (sscanf(env, "%dx%dx%dx%dx%d", &bm, &bn, &wm, &wn, &ks) >= 4)
            for (const TileCfg& t : kTiles)
                if (t.bm == bm && t.bn == bn && t.wm == wm && t.wn == wn && t.ks == ks && tile_ok(t, mode, wave64))
                    return t;
    }
    const int em = mode == 4 ? 0 : mode;   // the fused-quantization form is priced as W8A8
    const int cus = num_cus();
    double best = 1e300;
    const TileCfg* pick = nullptr;
    for (const TileCfg& t : kTiles) {
        if (!tile_ok(t, mode, wave64)) continue;
        const long tiles = (long)((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
        // the K split pays only where the 4-wave tile would leave one
        // workgroup (one wave per SIMD) on each CU, and over a long enough K
        if (t.ks > 1 && (tiles > cus || K < 1024)) continue;
        const long waves = (tiles + cus - 1) / cus;
        const double cost = (double)waves * t.bm * t.bn / t.eff[em];
        if (cost < best) best = cost, pick = &t;
    }
    return *pick;   // every filter leaves at least the 4-wave 64-column 128x128 tile
}

template <int MODE, int BM, int BN, int WM, int WN, int KS>
hipError_t launch_one(const void* a, const uint8_t* b, const half_t* s, const half_t* sa, half_t* y, int M, int N,
                      int K, const Epi& e, hipStream_t st, const AQuant& aq) {
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    hipLaunchKernelGGL((gemm_tiled_kernel<MODE, BM, BN, WM, WN, KS>), dim3(tiles), dim3(WM * WN * KS * WAVE), 0, st, a,
                       b, s, sa, y, M, N, K, e, aq);
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(const TileCfg& t, const void* a, const uint8_t* b, const half_t* s, const half_t* sa, half_t* y,
                       int M, int N, int K, const Epi& e, hipStream_t st, const AQuant& aq) {
#define ARIA_TILE(BM_, BN_, WM_, WN_, KS_)                                     \
    if (t.bm == BM_ && t.bn == BN_ && t.wm == WM_ && t.wn == WN_ && t.ks == KS_) \
        return launch_one<MODE, BM_, BN_, WM_, WN_, KS_>(a, b, s, sa, y, M, N, K, e, st, aq);
    ARIA_TILE(256, 192, 4, 3, 1) ARIA_TILE(256, 256, 4, 4, 1) ARIA_TILE(256, 192, 4, 2, 1) ARIA_TILE(256, 128, 4, 2, 1)
    ARIA_TILE(128, 256, 2, 4, 1) ARIA_TILE(128, 192, 2, 2, 1) ARIA_TILE(128, 128, 2, 2, 1) ARIA_TILE(64, 192, 2, 2, 1)
    ARIA_TILE(128, 64, 2, 2, 1) ARIA_TILE(64, 128, 2, 2, 1) ARIA_TILE(64, 64, 2, 2, 1)
    ARIA_TILE(64, 192, 2, 2, 2) ARIA_TILE(128, 128, 2, 2, 2) ARIA_TILE(128, 64, 2, 2, 2) ARIA_TILE(64, 128, 2, 2, 2)
    ARIA_TILE(64, 96, 2, 3, 1) ARIA_TILE(128, 96, 2, 3, 1) ARIA_TILE(128, 128, 2, 4, 1) ARIA_TILE(64, 96, 2, 3, 2)
#undef ARIA_TILE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_tiled(int mode, const void* a, const void* bq, const half_t* s, const half_t* sa, half_t* y,
                             int M, int N, int K, const Epi& epi, hipStream_t st, const AQuant* aq) {
    if (mode == 4 && !aq) return hipErrorInvalidValue;
    // 32-bit buffer offsets: split very tall problems into row blocks
    const int64_t aeb = mode == 0 ? 1 : 2;
    const int64_t lda = mode == 4 ? aq->lda : K;
    const int64_t max_rows = ((int64_t)1 << 31) / ((int64_t)lda * aeb) / 256 * 256;
    const TileCfg& t = pick_tile(mode, M > max_rows ? (int)max_rows : M, N, K, epi.rowmax != nullptr);
    const uint8_t* b = static_cast<const uint8_t*>(bq);
    for (int64_t r0 = 0; r0 < M; r0 += max_rows) {
        const int rows = (int)((M - r0) < max_rows ? (M - r0) : max_rows);
        Epi e = epi;
        if (e.residual) e.residual += r0 * N;
        if (e.acc_out) e.acc_out += r0 * N;
        if (e.rowmax) e.rowmax += r0 * e.rowmax_ld;
        AQuant q = aq ? *aq : AQuant{nullptr, 0, 0, nullptr};
        if (q.amax) q.amax += r0 * q.amax_ld;
        if (q.sa_out) q.sa_out += r0;
        const char* ar = static_cast<const char*>(a) + r0 * lda * aeb;
        const half_t* sar = sa ? sa + r0 : nullptr;
        half_t* yr = y + r0 * N;
        hipError_t err;
        if (mode == 0) err = launch_mode<0>(t, ar, b, s, sar, yr, rows, N, K, e, st, q);
        else if (mode == 1) err = launch_mode<1>(t, ar, b, s, sar, yr, rows, N, K, e, st, q);
        else if (mode == 2) err = launch_mode<2>(t, ar, b, s, sar, yr, rows, N, K, e, st, q);
        else if (mode == 3) err = launch_mode<3>(t, ar, b, s, sar, yr, rows, N, K, e, st, q);
        else err = launch_mode<4>(t, ar, b, s, sar, yr, rows, N, K, e, st, q);
        if (err != hipSuccess) return err;
    }
    return hipSuccess;
}

}  // namespace aria
