// The DiT block's attention core between the QKV and out-projection linears
// (docshare paper page, Fig. 1 "DiT blocks"; project page, "What aria is": the
// denoiser is a transformer over latent tokens).  Multi-head softmax
// self-attention over [Q | K | V] = qkv fp16 [M][3W], head h of each block at
// columns h*64 .. h*64+63, within each sequence of S consecutive rows:
//   out[i][h*64 + e] = sum_j softmax_j(q_i . k_j / 8) v_j[e]     (64-dim heads)
//
// Design (gfx950, flash-attention style, one pass over the keys): a workgroup
// of 4 waves owns 128 queries of one (sequence, head); each wave keeps its 32
// queries' Q fragments in registers and computes S^T = K Q^T, so that a lane
// holds the scores of ONE query (column l % 32) for 32 keys: the running max
// needs one cross-lane exchange per key block instead of a reduction over 32
// lanes.  P^T (fp16) is fed straight from the score registers as the B
// operand of O^T += V^T P^T (the key order that the score layout implies is
// matched by how V^T is read from LDS), and of a ones-tile product that yields
// the softmax denominators on the matrix unit too.  Key blocks of 64 are
// double-buffered in LDS (K row-major with a 16-byte row pad, V transposed
// with 8-byte runs of four keys), the next block's loads are in flight during
// the current block's matrix work, one barrier per block.  Scores, the
// softmax statistics and the accumulators are fp32 (kept in VGPRs: the
// softmax touches them every block); P and the output are rounded to fp16.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace aria {

namespace {

constexpr int HD = 64;        // head dimension
constexpr int KB = 64;        // keys per block
constexpr int QW = 4;         // waves per workgroup (32 queries each)
constexpr int KROW = HD + 8;  // K rows in LDS, halves (16-byte pad)
constexpr int VROW = KB + 4;  // V^T rows in LDS, halves (136 bytes: the 8-byte runs of the
                              // V stores and of the fragment reads both spread over all banks)
// s_waitcnt immediate (gfx9 encoding) for vmcnt(0), expcnt and lgkmcnt(0)
constexpr int kWaitVm0 = 0x0070;

__device__ __forceinline__ float wave_xor32_max(float v) { return fmaxf(v, __shfl_xor(v, 32, WAVE)); }

}  // namespace

// PRE: read all of a block's K fragments before its score MFMAs, and its V^T
// fragments before the softmax so that their latency hides behind it (183
// VGPRs, two waves per SIMD, against 156 and three without).  Measured with 24
// heads of 1024 keys: -7 % at one sequence, -3 % to +2 % at two, but +5 % at
// four and eight, where the third wave per SIMD matters more; the launch picks
// it when the grid fits in two workgroups per CU.
template <bool PRE>
__global__ __launch_bounds__(QW * WAVE) void attention_kernel(const half_t* __restrict__ qkv, int M, int W, int S,
                                                              half_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) half_t Ks[2][KB][KROW];
    __shared__ __attribute__((aligned(16))) half_t Vt[2][HD][VROW];
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE, hl = lane / 32;
    const int h = blockIdx.y, seq = blockIdx.z;
    const int q0 = blockIdx.x * (QW * 32) + wave * 32;  // this wave's first query (within the sequence)
    const int ld = 3 * W;                               // qkv row stride, halves
    const int64_t row0 = (int64_t)seq * S;              // first row of the sequence
    const rsrc_t rq = make_rsrc(qkv + row0 * ld, (uint32_t)S * (uint32_t)ld * 2);

    // Cooperative K / V block loads, 16-byte chunks, four per thread; waves 0-1
    // fetch V, waves 2-3 fetch K (a wave-uniform split).  A V thread takes
    // four consecutive keys 4j .. 4j+3 of one 8-column piece p, so that it can
    // write V^T as 8-byte runs of four keys: Vt[8p + e][4j .. 4j+3].  A K thread
    // takes chunks c = t + 128 i (key c / 8, piece c % 8), stored row-major.
    const bool vthread = wave < 2;
    const int ct = vthread ? tid : tid - 2 * WAVE;   // 0 .. 127 within the role
    v4i rkv[4];
    auto load_kv = [&](int kb) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            int key, col;
            if (vthread) key = 4 * (ct / 8) + i, col = 2 * W + h * HD + (ct % 8) * 8;
            else key = (ct + 128 * i) / 8, col = W + h * HD + ((ct + 128 * i) % 8) * 8;
            const int j = kb + key;
            rkv[i] = buf_load16(rq, j < S ? ((uint32_t)j * ld + col) * 2 : OOB);
        }
    };
    auto store_kv = [&](int buf) {
        if (vthread) {
            const int j4 = 4 * (ct / 8), p8 = (ct % 8) * 8;
            v8h v[4];
#pragma unroll
            for (int i = 0; i < 4; i++) v[i] = __builtin_bit_cast(v8h, rkv[i]);
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const v2h lo = {v[0][e], v[1][e]}, hi = {v[2][e], v[3][e]};
                *reinterpret_cast<v2u*>(&Vt[buf][p8 + e][j4]) = v2u{__builtin_bit_cast(u32, lo), __builtin_bit_cast(u32, hi)};
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int c = ct + 128 * i;
                *reinterpret_cast<v4i*>(&Ks[buf][c / 8][(c % 8) * 8]) = rkv[i];
            }
        }
    };

    // Block 0's loads first, then Q^T fragments (B operand: lane = query
    // q0 + lane % 32, d = 16 t + 8 hl .. +7); every load before the loop has
    // landed before block 1 is requested, so no load is still pending at the
    // loop head (one that were would make each iteration wait for the
    // prefetched block as well).
    load_kv(0);
    v8h qf[4];
    {
        const int q = q0 + lane % 32;
#pragma unroll
        for (int t = 0; t < 4; t++)
            qf[t] = __builtin_bit_cast(v8h, buf_load16(rq, q < S ? ((uint32_t)q * ld + h * HD + 16 * t + 8 * hl) * 2 : OOB));
    }
    __builtin_amdgcn_sched_barrier(0);
    store_kv(0);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __builtin_amdgcn_sched_barrier(0);

    // Exponents in base 2: exp(s / sqrt(64)) = exp2(s * sl2).  m is the
    // reference the exponents are taken against (raw score units): it is
    // raised to the block maximum only when that exceeds it by more than
    // 2^kHeadroom in the exponentiated domain, so the rescaling of the sums and
    // accumulators is skipped for most blocks; P = exp2((s - m) sl2) stays
    // below 2^kHeadroom, well inside fp16.  The result does not depend on the
    // reference (it cancels in O / sum).
    constexpr float kHeadroom = 8.0f;
    const float sl2 = 0.125f * 1.4426950408889634f;
    float m = -INFINITY;
    v16f ot[2] = {v16f{}, v16f{}};
    // the softmax denominators come from the matrix unit as well: a 32-row
    // tile of ones times P^T gives every row the column sums of P^T, i.e.
    // each query's sum of the (fp16-rounded) weights that enter O
    v16f ls = {};
    v8h ones;
#pragma unroll
    for (int e = 0; e < 8; e++) ones[e] = (half_t)1.0f;
    const int nkb = (S + KB - 1) / KB, nfull = S / KB;
    if (nkb > 1) load_kv(KB);
    __syncthreads();
    auto block = [&](int b, auto masked_c) {
        constexpr bool masked = decltype(masked_c)::value;
        const int cur = b & 1, kb = b * KB;
        // S^T tiles: keys 32 jt + (row), queries (column = lane % 32)
        v16f st[2] = {v16f{}, v16f{}};
        auto vfrag = [&](int dt, int u) {
            const half_t* vr = &Vt[cur][32 * dt + lane % 32][16 * u + 4 * hl];
            const v2u lo = *reinterpret_cast<const v2u*>(vr);
            const v2u hi = *reinterpret_cast<const v2u*>(vr + 8);
            return __builtin_bit_cast(v8h, v4u{lo[0], lo[1], hi[0], hi[1]});
        };
        v8h vfr[2][4];
        if constexpr (PRE) {
            v8h kfr[2][4];
#pragma unroll
            for (int jt = 0; jt < 2; jt++)
#pragma unroll
                for (int t = 0; t < 4; t++) kfr[jt][t] = *reinterpret_cast<const v8h*>(&Ks[cur][32 * jt + lane % 32][16 * t + 8 * hl]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int jt = 0; jt < 2; jt++)
#pragma unroll
                for (int t = 0; t < 4; t++) st[jt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kfr[jt][t], qf[t], st[jt], 0, 0, 0);
#pragma unroll
            for (int dt = 0; dt < 2; dt++)
#pragma unroll
                for (int u = 0; u < 4; u++) vfr[dt][u] = vfrag(dt, u);
        } else {
#pragma unroll
            for (int jt = 0; jt < 2; jt++)
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    const v8h kf = *reinterpret_cast<const v8h*>(&Ks[cur][32 * jt + lane % 32][16 * t + 8 * hl]);
                    st[jt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[t], st[jt], 0, 0, 0);
                }
        }
        if constexpr (masked) {   // the partial last block: keys past S get no weight
#pragma unroll
            for (int jt = 0; jt < 2; jt++)
#pragma unroll
                for (int r = 0; r < 16; r++)
                    if (kb + 32 * jt + 8 * (r / 4) + 4 * hl + r % 4 >= S) st[jt][r] = -INFINITY;
        }
        // online softmax for this lane's query over the block's 64 keys
        float mb = -INFINITY;
#pragma unroll
        for (int jt = 0; jt < 2; jt++)
#pragma unroll
            for (int r = 0; r < 16; r++) mb = fmaxf(mb, st[jt][r]);
        mb = wave_xor32_max(mb);
        const bool raise = (mb - m) * sl2 > kHeadroom;   // always on the first block (m = -inf)
        if (__builtin_amdgcn_ballot_w64(raise)) {
            const float mn = raise ? mb : m;
            const float corr = __builtin_amdgcn_exp2f((m - mn) * sl2);   // 1 if not raised, 0 on the first block
            ls *= corr;
#pragma unroll
            for (int dt = 0; dt < 2; dt++) ot[dt] *= corr;
            m = mn;
        }
        const float off = -m * sl2;
        v8h pf[4];
#pragma unroll
        for (int u = 0; u < 4; u++)
#pragma unroll
            for (int e = 0; e < 8; e++)
                pf[u][e] = (half_t)__builtin_amdgcn_exp2f(__builtin_fmaf(st[u / 2][8 * (u % 2) + e], sl2, off));
        // O^T += V^T P^T over the block's 4 k-steps of 16 keys; register e of
        // P^T step u is key 16 u + 4 hl + 8 (e / 4) + e % 4
#pragma unroll
        for (int dt = 0; dt < 2; dt++)
#pragma unroll
            for (int u = 0; u < 4; u++)
                ot[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(PRE ? vfr[dt][u] : vfrag(dt, u), pf[u], ot[dt], 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 4; u++) ls = __builtin_amdgcn_mfma_f32_32x32x16_f16(ones, pf[u], ls, 0, 0, 0);
        // the next block: stored into the other buffer (free since the last
        // barrier), the one after it requested
        if (b + 1 < nkb) {
            store_kv(cur ^ 1);
            if (b + 2 < nkb) load_kv(kb + 2 * KB);
        }
        __syncthreads();
    };
    for (int b = 0; b < nfull; b++) block(b, std::false_type{});
    if (nfull < nkb) block(nfull, std::true_type{});

    // out[query][h*64 + d] = O^T[d][query] / sum; register r of tile dt is
    // d = 32 dt + 8 (r / 4) + 4 hl + r % 4: four consecutive d per 8-byte store
    const int q = q0 + lane % 32;
    if (q < S) {
        const float inv = 1.0f / ls[0];
        half_t* orow = out + (row0 + q) * W + h * HD;
#pragma unroll
        for (int dt = 0; dt < 2; dt++)
#pragma unroll
            for (int g = 0; g < 4; g++) {

                const float a0 = ot[dt][4 * g], a1 = ot[dt][4 * g + 1], a2 = ot[dt][4 * g + 2], a3 = ot[dt][4 * g + 3];
                const v2h p0 = {(half_t)(a0 * inv), (half_t)(a1 * inv)};
                const v2h p1 = {(half_t)(a2 * inv), (half_t)(a3 * inv)};
                *reinterpret_cast<v2u*>(orow + 32 * dt + 8 * g + 4 * hl) =
                    v2u{__builtin_bit_cast(u32, p0), __builtin_bit_cast(u32, p1)};
            }
    }
}

hipError_t launch_attention(const half_t* qkv, int64_t M, int64_t W, int64_t H, int64_t S, half_t* out,
                            hipStream_t st) {
    dim3 grid((unsigned)((S + QW * 32 - 1) / (QW * 32)), (unsigned)H, (unsigned)(M / S));
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        hipDeviceProp_t p;
        if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&p, dev) == hipSuccess) cus = p.multiProcessorCount;
        if (cus <= 0) cus = 256;
    }
    const int64_t wgs = (int64_t)grid.x * grid.y * grid.z;
    if (wgs <= 2 * (int64_t)cus)
        hipLaunchKernelGGL(attention_kernel<true>, grid, dim3(QW * WAVE), 0, st, qkv, (int)M, (int)W, (int)S, out);
    else
        hipLaunchKernelGGL(attention_kernel<false>, grid, dim3(QW * WAVE), 0, st, qkv, (int)M, (int)W, (int)S, out);
    return hipGetLastError();
}

}  // namespace aria
