// Decode-sized linear on gfx950: Y[M, N] = X[M, K] W[N, K]^T (+ bias) with
// M <= 64 tokens.
//
// At M <= 64 the arithmetic intensity is at most M flop per weight byte, far
// below the MI355X ridge (~315 flop/B): the kernel is bound by streaming W
// from HBM once. Design:
//   * Matrix cores still do the math (v_mfma_f32_16x16x32_bf16): the vector
//     ALU could not keep up with 16-64 flop per byte at 8 TB/s. W is the A
//     operand (16 weight rows per MFMA) and X^T the B operand (16 tokens), so
//     D[n][m] = Y[m][n] and each lane ends with 4 consecutive outputs of one
//     token row.
//   * W goes global -> VGPR directly, each lane fetching 16 contiguous bytes
//     of one row; all of a wave's k-steps are issued before the first MFMA so
//     that many loads are in flight per CU. Every load is unconditional
//     (out-of-range lanes read a clamped in-bounds address and are zeroed or
//     discarded at use) and LDS exchanges use LDS-only barriers, so each
//     s_waitcnt covers just the loads it needs (a load in a branch, or a full
//     __syncthreads(), would make it wait for all of them).
//   * X is staged once per workgroup in LDS (padded rows) and shared by the
//     waves that cover different weight rows, or, with one 16-row block per
//     workgroup, loaded per wave step by step together with the weights.
//   * K is split across the waves of a workgroup, summed through LDS in wave
//     order; each wave then finishes the token tiles it owns (mt = wk mod NWK).
//     If the weight has too few rows to fill 256 CUs, K is also split across
//     workgroups: each writes an fp32 partial tile to the workspace and the
//     last workgroup to arrive on a tile (one atomic counter per tile) sums
//     the partials in split order, so the result does not depend on arrival
//     order. Partials travel through relaxed device-scope atomic stores and
//     loads.
//   * Consecutive row tiles run on the same XCD (they share output lines),
//     and the kernel arguments the first loads need arrive in one batch.
//   * Fused epilogues. SwiGLU: each 16-row MFMA block holds 8 gate rows and
//     the same 8 up rows, so lanes 0-31 own gate outputs whose up partners
//     sit 32 lanes higher; one cross-lane swap pairs them and the block
//     writes 8 SwiGLU outputs per token. Reduce: the rank's rounded partial is
//     summed with the other ranks' partials in rank order and rounded once;
//     the owner waves load those partials right after the first weights.
//     Both give the same bits as the separate kernels.
#include <mutex>
#include <type_traits>

#include "common.h"
#include "kernels.h"

#ifndef TP_SKINNY_W_NT
#define TP_SKINNY_W_NT 0
#endif

namespace tpk {

namespace {

// XD = 0: X's K-chunk is staged once per workgroup in LDS (shared by the NWN
// waves that own different weight rows). XD = 1: every wave loads its own X
// fragments straight from global memory (L2-resident), which needs no LDS
// and no barrier before the MFMAs.
template <int MT, int KSTEPS, int NWN, int NWK, int XD>
struct SkinnyCfg {
    static constexpr int kThreads = 64 * NWN * NWK;
    static constexpr int kRows = 16 * NWN;             // weight rows per workgroup
    static constexpr int kWaveK = 32 * KSTEPS;         // K per wave
    static constexpr int kGroupK = kWaveK * NWK;       // K per workgroup
    static constexpr int kTokens = 16 * MT;
    static constexpr int kXStride = kGroupK + 8;       // LDS row stride (elements), 16 B pad
    static constexpr int kOwn = (MT + NWK - 1) / NWK;   // token tiles each wave finishes
    static constexpr int kRedBytes = NWK > 1 ? NWK * NWN * MT * 4 * 64 * 4 : 0;
    // LDS for xrows staged token rows plus the cross-wave reduction buffer
    static int lds_bytes(int xrows) { return (XD ? 0 : xrows * kXStride * 2) + kRedBytes; }
};

__device__ __forceinline__ void store_out4(const GemmArgs& a, int64_t m, int64_t n, const float* v) {
    // 4 consecutive outputs y[m, n..n+3] (+ bias), bf16 or fp32.
    float o[4] = {v[0], v[1], v[2], v[3]};
    if (a.bias != nullptr) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (n + i < a.N) o[i] += bf16_to_f32(reinterpret_cast<const uint16_t*>(a.bias)[n + i]);
    }
    const int64_t base = m * a.N + n;
    const bool full = (n + 3 < a.N) && (a.N % 4 == 0);
    if (a.out_dtype == TP_F32) {
        float* y = reinterpret_cast<float*>(a.y);
        if (full) {
            *reinterpret_cast<float4*>(y + base) = make_float4(o[0], o[1], o[2], o[3]);
        } else {
            for (int i = 0; i < 4; ++i) if (n + i < a.N) y[base + i] = o[i];
        }
    } else {
        uint16_t* y = reinterpret_cast<uint16_t*>(a.y);
        if (full) {
            *reinterpret_cast<uint2*>(y + base) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        } else {
            for (int i = 0; i < 4; ++i) if (n + i < a.N) y[base + i] = (uint16_t)f32_to_bf16(o[i]);
        }
    }
}

// Weight row of kernel row v, or -1 past the end. EPI_SWIGLU pairs gate and
// up rows in 16-row blocks: rows 8 b + r (r < 8) of gate and of up form block b.
template <int EPI>
__device__ __forceinline__ int64_t weight_row(const GemmArgs& a, int64_t v) {
    if constexpr (EPI != EPI_SWIGLU) return v < a.N ? v : -1;
    const int64_t j = (v >> 4) * 8 + (v & 7);
    if (j >= a.i_half) return -1;
    return (v & 8) ? a.i_half + j : j;
}

// Other ranks' values of one lane's 4 outputs, indexed by rank (the own slot
// unused): 4 bf16 (8 bytes) per rank, or 4 fp32 (16 bytes) for the _F32
// epilogues. When a wave finishes one token tile, the first tile's values are
// loaded right after its weights; otherwise (and for later tiles of a
// persistent loop, and in the last split) just before the sum. Reduce
// launches have N % 4 == 0, so a lane's 4 outputs are one aligned load per
// rank. The guards are uniform and one-sided (a branch that merged two values
// would make each load wait for the one before); lanes past the edge read the
// start of the peer's buffer instead and discard it. The _ADD epilogues also
// hold the lane's 4 residual values (read from y).
template <int EPI>
struct PeerVals {
    using V = typename std::conditional<epi_peers_f32(EPI), uint4, uint2>::type;
    V v[kMaxFusedPeers];
    uint2 res;
};

template <int EPI>
__device__ __forceinline__ void load_peers(const GemmArgs& a, int64_t m, int64_t n, PeerVals<EPI>& p) {
    using V = typename PeerVals<EPI>::V;
    constexpr int kElem = epi_peers_f32(EPI) ? 4 : 2;
    const bool ok = m < a.M && n < a.N;
    const int64_t base = ok ? m * a.N + n : 0;
#pragma unroll
    for (int r = 0; r < kMaxFusedPeers; ++r) {
        if (r < a.t && r != a.rank)
            p.v[r] = *reinterpret_cast<const V*>(reinterpret_cast<const unsigned char*>(a.peers[r]) + base * kElem);
    }
    if constexpr (epi_is_add(EPI))
        p.res = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.y) + base);
}

// Reduce epilogues: out[m, n..n+3] = bf16(sum over ranks in order from rank
// 0), the own partial as a partial buffer of the peers' dtype holds it
// (rounded to bf16, or the fp32 sum itself). _ADD: y[m, n..n+3] = bf16(y +
// that bf16 sum) (the residual stream).
template <int EPI>
__device__ __forceinline__ void reduce_out4(const GemmArgs& a, int64_t m, int64_t n, const float* v,
                                            const PeerVals<EPI>& p) {
    // Unrolled with constant indices (the values stay in registers); the
    // guards are uniform, so only the t ranks' iterations execute.
    float own[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) own[i] = epi_peers_f32(EPI) ? v[i] : round_bf16(v[i]);
    float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < kMaxFusedPeers; ++r) {
        if (r < a.t) {
            float q[4];
            if (r == a.rank) {
#pragma unroll
                for (int i = 0; i < 4; ++i) q[i] = own[i];
            } else if constexpr (epi_peers_f32(EPI)) {
                q[0] = __uint_as_float(p.v[r].x);
                q[1] = __uint_as_float(p.v[r].y);
                q[2] = __uint_as_float(p.v[r].z);
                q[3] = __uint_as_float(p.v[r].w);
            } else {
                q[0] = bf16_to_f32(p.v[r].x & 0xFFFFu);
                q[1] = bf16_to_f32(p.v[r].x >> 16);
                q[2] = bf16_to_f32(p.v[r].y & 0xFFFFu);
                q[3] = bf16_to_f32(p.v[r].y >> 16);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = r == 0 ? q[i] : o[i] + q[i];
        }
    }
    if constexpr (epi_is_add(EPI)) {
        const float res[4] = {bf16_to_f32(p.res.x & 0xFFFFu), bf16_to_f32(p.res.x >> 16),
                              bf16_to_f32(p.res.y & 0xFFFFu), bf16_to_f32(p.res.y >> 16)};
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = res[i] + round_bf16(o[i]);
    }
    uint16_t* y = reinterpret_cast<uint16_t*>(a.y) + m * a.N + n;
    *reinterpret_cast<uint2*>(y) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
}

// Final values of one lane: D rows n..n+3 (kernel row space) of token m.
// Every lane of the wave must call it (the SwiGLU pairing swaps lanes).
template <int EPI>
__device__ __forceinline__ void finish4(const GemmArgs& a, int64_t m, int64_t n, const float* v, int lane,
                                        const PeerVals<EPI>& peers) {
    if constexpr (EPI == EPI_SWIGLU) {
        float u[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = __shfl_xor(v[i], 32);
        const int64_t j = (n >> 4) * 8 + (n & 7);      // first of the 4 gate columns
        if (lane < 32 && m < a.M && j < a.i_half) {
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = silu_f32(round_bf16(v[i])) * round_bf16(u[i]);
            uint16_t* y = reinterpret_cast<uint16_t*>(a.y) + m * a.i_half + j;
            if (j + 3 < a.i_half && a.i_half % 4 == 0) {
                *reinterpret_cast<uint2*>(y) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
            } else {
                for (int i = 0; i < 4; ++i) if (j + i < a.i_half) y[i] = (uint16_t)f32_to_bf16(o[i]);
            }
        }
        return;
    }
    if (m >= a.M || n >= a.N) return;
    if constexpr (epi_is_reduce(EPI)) reduce_out4<EPI>(a, m, n, v, peers);
    else store_out4(a, m, n, v);
}

// NORM = 1 (X staged in LDS, one 16-row group): the RMSNorm of X's rows
// with gamma already folded into W (tp_fold_norm_weight): y = r_m (x_m .
// w'_n), r_m = 1 / sqrt(sum_k x_mk^2 / K + eps). sum_k x_mk^2 is the diagonal
// of X X^T, one more MFMA per k-step and token tile on the X fragments
// already in registers (the matrix cores idle otherwise), so the norm adds no
// per-element work. With K split across workgroups each publishes its share
// of the sums next to its partial tile and the last to arrive (one token
// tile), or the finish kernel of a two-launch split (up to 4 token tiles),
// adds them in split order.
template <int MT, int KSTEPS, int NWN, int NWK, int XD, int EPI, int NORM = 0>
__global__ void __launch_bounds__(64 * NWN * NWK)
skinny_kernel(GemmArgs a, int splits, int64_t ntiles, int xrows, float* __restrict__ ws,
              unsigned* __restrict__ counters) {
    using C = SkinnyCfg<MT, KSTEPS, NWN, NWK, XD>;
    static_assert(!NORM || (!XD && (MT == 1 || (MT == 4 && NWN <= 4)) && (MT == 4 || NWN == 1) && NWK > 1),
                  "the norm needs X staged in LDS (and one row group for one token tile)");
    __shared__ float s_gram[NORM ? NWK * MT * 4 * 64 : 1];    // NORM: each wave's X X^T fragments
    extern __shared__ __align__(16) unsigned char smem[];
    bf16_t* xs = reinterpret_cast<bf16_t*>(smem);                       // [xrows][kXStride]
    float* red = reinterpret_cast<float*>(smem + (XD ? 0 : (size_t)xrows * C::kXStride * 2));
    __shared__ unsigned s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave % NWN;
    const int wk = wave / NWN;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int split = blockIdx.y;
    const int64_t k_group = (int64_t)split * C::kGroupK;
    // Neighbouring row tiles share the 128-byte lines of the output (and of
    // the other ranks' partials). Workgroup b runs on XCD b mod 8, so an
    // unsplit grid hands each XCD a contiguous range of tiles (a permutation
    // of [0, grid) per round; later rounds add the grid size).
    // (Read without branching, so that every kernel argument the first loads
    // depend on arrives in one batch of scalar loads.)
    const unsigned gx = gridDim.x;
    // an empty asm that needs them: the compiler cannot defer these loads
    // past the first branch
    asm volatile("" ::"s"(splits), "s"(xrows), "s"(gx), "s"(a.t), "s"(a.rank));
    const bool remap = splits == 1 && gx % 8 == 0;
    int64_t tile = remap ? (int64_t)(blockIdx.x % 8) * (gx / 8) + blockIdx.x / 8 : (int64_t)blockIdx.x;

    const bf16_t* __restrict__ X = reinterpret_cast<const bf16_t*>(a.x);
    const bf16_t* __restrict__ W = reinterpret_cast<const bf16_t*>(a.w);

    // EPI_REDUCE with one token tile per wave: the owner waves load the other
    // ranks' values for the first tile right after its weights (step 2), so
    // they arrive while the weights stream; later tiles of a persistent loop
    // load theirs just before the sum.
    constexpr bool kReduce = epi_is_reduce(EPI);
    constexpr bool kPrefetchPeers = kReduce && C::kOwn == 1;
    PeerVals<EPI> peers;
    const int64_t m_own0 = 16 * wk + (lane & 15);          // token of the first owned tile
    bool first_tile = true;

    // 1. Stage X[0:xrows, k_group : k_group + kGroupK] into registers (issued
    //    first so that waiting for it does not wait for the weight stream).
    //    Only the xrows = min(M, 16 MT) real token rows are staged.
    constexpr int kXPerThread = XD ? 1 : (C::kTokens * (C::kGroupK / 8) + C::kThreads - 1) / C::kThreads;
    const int x_chunks = XD ? 0 : xrows * (C::kGroupK / 8);
    // Every load in this kernel is unconditional (out-of-range lanes read a
    // clamped in-bounds address and their values are replaced by zeros where
    // used), so the compiler can wait for exactly the loads it needs instead
    // of for all of them.
    uint4 xr[kXPerThread];
    if (!XD) {
#pragma unroll
        for (int j = 0; j < kXPerThread; ++j) {
            const int c = tid + j * C::kThreads;
            const int m = c / (C::kGroupK / 8);
            const int kc = c % (C::kGroupK / 8);
            const int64_t k = k_group + kc * 8;
            const bool ok = c < x_chunks && k < K;
            xr[j] = *reinterpret_cast<const uint4*>(X + (ok ? (int64_t)m * K + k : 0));
        }
    }

    // 2. Issue the first tile's weight loads (and, with XD, the wave's X
    //    fragments, which are the same for every tile).
    // Weight rows past the end read row 0 (their outputs are never stored);
    // k past K reads column 0 and is zeroed at the MFMA (k_ok).
    const int64_t k_wave = k_group + (int64_t)wk * C::kWaveK + 8 * (lane >> 4);
    uint4 wr[KSTEPS];
    auto load_w = [&](int64_t t, uint4* dst) {
        const int64_t row = weight_row<EPI>(a, t * C::kRows + wn * 16 + (lane & 15));
        const bf16_t* wrow = W + (row >= 0 ? row : 0) * K;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            const int64_t k = k_wave + 32 * s;
#if TP_SKINNY_W_NT
            dst[s] = ld_nt16(wrow + (k < K ? k : 0));
#else
            dst[s] = *reinterpret_cast<const uint4*>(wrow + (k < K ? k : 0));
#endif
        }
    };
    // XD: each step's weight and X fragments are issued together, so the
    //     MFMA of step s waits only for loads 0..s (the load counter is in
    //     order) and X never holds back the weight stream. They are read
    //     through buffer resources: one 32-bit offset per lane and row, the
    //     k-steps as immediate offsets, no clamping (a k past K reads the
    //     next row, or zeros past the extent, and meets a zeroed weight
    //     fragment at the MFMA; token rows past M read zeros and feed outputs
    //     that are never stored). Against 64-bit clamped addresses: Llama-8B
    //     t = 16 (64 tokens) o + sum 8.15 -> 8.0 us, down + sum 11.45 ->
    //     10.85; t = 8 o + sum 4.68 -> 4.58 (MI355X, timed alternately; the
    //     LDS-staged variants ran slower this way and keep plain loads).
    //     The host plans XD only for operands within kMaxBufferBytes.
    uint4 xd[XD ? KSTEPS : 1][XD ? MT : 1];
    if constexpr (XD) {
        const __amdgpu_buffer_rsrc_t rs_w = buffer_source(W, (EPI == EPI_SWIGLU ? 2 * a.i_half : N) * K * 2);
        const __amdgpu_buffer_rsrc_t rs_x = buffer_source(X, M * K * 2);
        const int64_t row = weight_row<EPI>(a, tile * C::kRows + wn * 16 + (lane & 15));
        const uint32_t w_off = (uint32_t)(((row >= 0 ? row : 0) * K + k_wave) * 2);
        const uint32_t x_off = (uint32_t)(((int64_t)(lane & 15) * K + k_wave) * 2);
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            wr[s] = buffer_ld16(rs_w, w_off + 64 * s);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) xd[s][mt] = buffer_ld16(rs_x, x_off + (uint32_t)(32 * mt * K) + 64 * s);
        }
    } else {
        load_w(tile, wr);
    }
    if constexpr (kPrefetchPeers) {
        if (splits == 1 && wk < MT) load_peers<EPI>(a, m_own0, tile * C::kRows + wn * 16 + 4 * (lane >> 4), peers);
    }

    // 3. X chunk -> LDS (zeros past K).
    if (!XD) {
#pragma unroll
        for (int j = 0; j < kXPerThread; ++j) {
            const int c = tid + j * C::kThreads;
            if (c < x_chunks) {
                const int m = c / (C::kGroupK / 8);
                const int kc = c % (C::kGroupK / 8);
                const bool ok = k_group + kc * 8 < K;
                *reinterpret_cast<uint4*>(xs + m * C::kXStride + kc * 8) = ok ? xr[j] : make_uint4(0u, 0u, 0u, 0u);
            }
        }
        lds_barrier();
    }


    const int xcol = wk * C::kWaveK + 8 * (lane >> 4);
    f32x4_t acc[MT];
    // Wave (wn, wk) finishes token tiles mt = wk + NWK o (o < kOwn): its own
    // accumulators when NWK == 1, else the in-order sum of the NWK waves'
    // accumulators read back from LDS.
    float fin[C::kOwn][4];
    // NORM: the row scale of each owned token tile's row lane % 16, from the
    // first tile (X is the same for all), and with K split this workgroup's
    // share of the row's sum of squares
    float rnorm[C::kOwn], ss_part[C::kOwn];
#pragma unroll
    for (int o = 0; o < C::kOwn; ++o) {
        rnorm[o] = 1.0f;
        ss_part[o] = 0.f;
    }
    for (;;) {
        const int64_t n_out = tile * C::kRows + wn * 16 + 4 * (lane >> 4);   // first of this lane's 4 rows

        // Prefetch the next tile's weights (unsplit grids with X staged in
        // LDS loop over tiles; XD grids have one workgroup per tile).
        const int64_t next = tile + gridDim.x;
        const bool has_next = !XD && splits == 1 && next < ntiles;
        uint4 wnext[XD ? 1 : KSTEPS];
        if constexpr (!XD) {
            if (has_next) load_w(next, wnext);
        }

        // 4. MFMAs: acc[mt] holds D[n = 4*(lane/16) + i][m = 16*mt + lane%16].
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        f32x4_t gram[NORM ? MT : 1];
#pragma unroll
        for (int mt = 0; mt < (NORM ? MT : 1); ++mt) gram[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            const bool k_ok = k_wave + 32 * s < K;
            const bf16x8_t av = __builtin_bit_cast(bf16x8_t, k_ok ? wr[s] : make_uint4(0u, 0u, 0u, 0u));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                uint4 xv;
                if (XD) {
                    xv = xd[XD ? s : 0][XD ? mt : 0];
                } else {
                    const int m = 16 * mt + (lane & 15);
                    xv = m < xrows ? *reinterpret_cast<const uint4*>(xs + m * C::kXStride + xcol + 32 * s)
                                   : make_uint4(0u, 0u, 0u, 0u);
                }
                acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, xv), acc[mt], 0, 0, 0);
                if (NORM && first_tile && wn == 0)       // one row group is enough
                    gram[NORM ? mt : 0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, xv), __builtin_bit_cast(bf16x8_t, xv), gram[NORM ? mt : 0], 0, 0, 0);
            }
        }

        // 5. Sum the NWK waves that share rows, in wave order, through LDS.
        if constexpr (NWK > 1) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    red[(((wk * NWN + wn) * MT + mt) * 4 + i) * 64 + lane] = acc[mt][i];
            // (the first row group computes X X^T and writes it)
            if (NORM && first_tile && wn == 0) {
#pragma unroll
                for (int mt = 0; mt < (NORM ? MT : 1); ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) s_gram[((wk * MT + mt) * 4 + i) * 64 + lane] = gram[mt][i];
            }
            lds_barrier();
#pragma unroll
            for (int o = 0; o < C::kOwn; ++o) {
                const int mt = wk + NWK * o;
                if (mt < MT) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float v = red[(((0 * NWN + wn) * MT + mt) * 4 + i) * 64 + lane];
#pragma unroll
                        for (int w = 1; w < NWK; ++w) v += red[(((w * NWN + wn) * MT + mt) * 4 + i) * 64 + lane];
                        fin[o][i] = v;
                    }
                }
            }
            if constexpr (NORM) {
                // X X^T[m][m] of token tile mt sits in lane m + 16 (m / 4),
                // element m % 4, of each wave's fragment for that tile;
                // summed over the waves in order.
                if (first_tile) {
                    const int m = lane & 15;
                    const int src = (m % 4) * 64 + m + 16 * (m / 4);
#pragma unroll
                    for (int o = 0; o < C::kOwn; ++o) {
                        const int mt = wk + NWK * o < MT ? wk + NWK * o : 0;   // unowned: any in-bounds tile
                        float ss = s_gram[mt * 4 * 64 + src];
#pragma unroll
                        for (int w = 1; w < NWK; ++w) ss += s_gram[(w * MT + mt) * 4 * 64 + src];
                        ss_part[o] = ss;
                        rnorm[o] = 1.0f / sqrtf(ss / (float)K + a.eps);
                    }
                }
                // with K split, the row's sum is complete only after the split
                if (splits == 1) {
#pragma unroll
                    for (int o = 0; o < C::kOwn; ++o)
#pragma unroll
                        for (int i = 0; i < 4; ++i) fin[o][i] *= rnorm[o];
                }
            }
            lds_barrier();     // the buffer is rewritten for the next tile
        } else {
#pragma unroll
            for (int o = 0; o < C::kOwn; ++o)
#pragma unroll
                for (int i = 0; i < 4; ++i) fin[o][i] = acc[o][i];
        }
        if (splits > 1) break;

#pragma unroll
        for (int o = 0; o < C::kOwn; ++o) {
            const int mt = wk + NWK * o;
            if (mt < MT) {                       // wave-uniform: every lane calls finish4
                const int64_t m = 16 * mt + (lane & 15);
                if constexpr (kReduce) {
                    if (!kPrefetchPeers || !first_tile) load_peers<EPI>(a, m, n_out, peers);
                }
                finish4<EPI>(a, m, n_out, fin[o], lane, peers);
            }
        }
        if (!has_next) return;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) wr[s] = wnext[XD ? 0 : s];
        tile = next;
        first_tile = false;
    }

    const int64_t n_out = tile * C::kRows + wn * 16 + 4 * (lane >> 4);   // first of this lane's 4 outputs

    // 6. K split across workgroups. The partial tile is published with
    //    relaxed device-scope atomic stores (global_store ... sc1: written
    //    through to the device-coherent level, no read-modify-write) and read
    //    back with relaxed device-scope atomic loads (sc1: never served from a
    //    stale line of another XCD's L2). Each thread waits until its stores
    //    are acknowledged before the barrier that precedes the arrival
    //    counter, so the last workgroup to arrive sees every partial. No
    //    agent-scope fence is used: on this GPU it writes back and
    //    invalidates the whole L2 of the XCD, once per workgroup.
    // 4 consecutive floats per lane: two 64-bit stores when 8-byte aligned.
    const bool pair = (N % 2 == 0) && (n_out + 3 < N);
    // counters == nullptr: the partial tiles are summed by skinny_split_finish
    // in a second launch (the kernel boundary publishes them): plain stores.
    if (counters == nullptr) {
        // NORM: this split's share of each row's sum of squares, [split][M]
        // after the partial tiles (every row tile computes the same; tile 0
        // publishes it)
        if (NORM && tile == 0 && wn == 0 && lane < 16) {
#pragma unroll
            for (int o = 0; o < C::kOwn; ++o) {
                const int mt = wk + NWK * o;
                const int64_t m = 16 * mt + lane;
                if (mt < MT && m < M) ws[(int64_t)splits * M * N + (int64_t)split * M + m] = ss_part[o];
            }
        }
#pragma unroll
        for (int o = 0; o < C::kOwn; ++o) {
            const int mt = wk + NWK * o;
            const int64_t m = 16 * mt + (lane & 15);
            if (mt < MT && m < M) {
                float* p = ws + ((int64_t)split * M + m) * N + n_out;
                if (pair) {
                    *reinterpret_cast<float2*>(p) = make_float2(fin[o][0], fin[o][1]);
                    *reinterpret_cast<float2*>(p + 2) = make_float2(fin[o][2], fin[o][3]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (n_out + i < N) p[i] = fin[o][i];
                }
            }
        }
        return;
    }
#pragma unroll
    for (int o = 0; o < C::kOwn; ++o) {
        const int mt = wk + NWK * o;
        const int64_t m = 16 * mt + (lane & 15);
        if (mt < MT && m < M) {
            float* p = ws + ((int64_t)split * M + m) * N + n_out;
            if (pair) {
                const uint64_t lo = (uint64_t)__float_as_uint(fin[o][0]) | ((uint64_t)__float_as_uint(fin[o][1]) << 32);
                const uint64_t hi = (uint64_t)__float_as_uint(fin[o][2]) | ((uint64_t)__float_as_uint(fin[o][3]) << 32);
                __hip_atomic_store(reinterpret_cast<uint64_t*>(p), lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(reinterpret_cast<uint64_t*>(p) + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (n_out + i < N)
                        __hip_atomic_store(p + i, fin[o][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    // NORM: this split's share of each row's sum of squares, after the
    // partial tiles ([split][tile][16] floats), published the same way
    float* const ws_ss = ws + (int64_t)splits * M * N;
    if (NORM && wk == 0 && lane < 16)
        __hip_atomic_store(ws_ss + ((int64_t)split * ntiles + tile) * 16 + lane, ss_part[0], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = atomicAdd(&counters[tile], 1u);
        s_last = (prev == (unsigned)(splits - 1)) ? 1u : 0u;
    }
    __syncthreads();
    if (s_last != 1u) return;

    // 7. Last workgroup on this tile: sum the partials in split order. The
    //    loads of up to 8 splits are issued back to back before any is used,
    //    so they cost one memory round trip, not one each.
    if constexpr (NORM) {
        // the row's sum of squares over the splits, in split order (one
        // token tile: the host finishes every split of 64 tokens in a second
        // launch, skinny_split_launches)
        float ss = 0.f;
        for (int sp0 = 0; sp0 < splits; sp0 += 8) {
            float t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int sp = sp0 + j < splits ? sp0 + j : splits - 1;
                t[j] = __hip_atomic_load(ws_ss + ((int64_t)sp * ntiles + tile) * 16 + (lane & 15), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (sp0 + j < splits) ss += t[j];
        }
        rnorm[0] = 1.0f / sqrtf(ss / (float)K + a.eps);
    }
#pragma unroll
    for (int o = 0; o < C::kOwn; ++o) {
        const int mt = wk + NWK * o;
        if (mt < MT) {                           // wave-uniform: every lane calls finish4
            const int64_t m = 16 * mt + (lane & 15);
            if constexpr (kReduce) load_peers<EPI>(a, m, n_out, peers);
            float v[4] = {0.f, 0.f, 0.f, 0.f};
            if (m < M && n_out < N) {
                for (int sp0 = 0; sp0 < splits; sp0 += 8) {
                    float t[8][4];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        t[j][0] = t[j][1] = t[j][2] = t[j][3] = 0.f;
                        if (sp0 + j < splits) {
                            float* p = ws + ((int64_t)(sp0 + j) * M + m) * N + n_out;
                            if (pair) {
                                const uint64_t lo = __hip_atomic_load(reinterpret_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                                const uint64_t hi = __hip_atomic_load(reinterpret_cast<uint64_t*>(p) + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                                t[j][0] = __uint_as_float((uint32_t)lo);
                                t[j][1] = __uint_as_float((uint32_t)(lo >> 32));
                                t[j][2] = __uint_as_float((uint32_t)hi);
                                t[j][3] = __uint_as_float((uint32_t)(hi >> 32));
                            } else {
#pragma unroll
                                for (int i = 0; i < 4; ++i)
                                    if (n_out + i < N)
                                        t[j][i] = __hip_atomic_load(p + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            }
                        }
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (sp0 + j < splits)
#pragma unroll
                            for (int i = 0; i < 4; ++i) v[i] += t[j][i];
                }
            }
            if constexpr (NORM) {
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] *= rnorm[0];
            }
            finish4<EPI>(a, m, n_out, v, lane, peers);
        }
    }
    if (tid == 0) atomicExch(&counters[tile], 0u);
}

// Second launch of a K split whose partial tiles were written without
// arrival counters: one thread per 4 consecutive outputs of the kernel's row
// space (EPI_SWIGLU: per 4 gate rows of a 16-row block, the up rows 8 higher),
// the splits summed in split order from 0.f, then the epilogue of the
// single-launch split: the same arithmetic, so the same bits.
template <int EPI>
__global__ void __launch_bounds__(256)
skinny_split_finish(GemmArgs a, int splits, const float* __restrict__ ws) {
    const int64_t M = a.M, N = a.N;
    const int64_t groups = EPI == EPI_SWIGLU ? N / 8 : (N + 3) / 4;   // per token row
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= M * groups) return;
    const int64_t m = g / groups;
    const int64_t q = g - m * groups;
    const int64_t n = EPI == EPI_SWIGLU ? 16 * (q >> 1) + 4 * (q & 1) : 4 * q;
    // The splits' values of 4 outputs at n0 (and, for SwiGLU, of the up
    // rows at n0 + 8), 8 splits per round: every load of a round is issued
    // before the first add, so a round costs one memory round trip; the adds
    // then run in split order from 0.f.
    constexpr int kRound = 8;
    constexpr int kCols = EPI == EPI_SWIGLU ? 2 : 1;
    const bool vec = n + 3 < N && N % 4 == 0;
    const bool norm = a.norm != 0;
    // with the norm, the splits' shares of the row's sum of squares ([split][M]
    // after the partial tiles) load in the same rounds
    const float* pss = ws + (int64_t)splits * M * N + m;
    float acc[kCols][4] = {};
    float ss = 0.f;
    for (int sp0 = 0; sp0 < splits; sp0 += kRound) {
        float4 t[kRound][kCols];
        float tss[kRound];
#pragma unroll
        for (int j = 0; j < kRound; ++j) {
            const int sp = sp0 + j < splits ? sp0 + j : splits - 1;   // clamped: in bounds, unused past splits
            tss[j] = norm ? pss[(int64_t)sp * M] : 0.f;
#pragma unroll
            for (int c = 0; c < kCols; ++c) {
                const int64_t n0 = n + 8 * c;
                const float* p = ws + ((int64_t)sp * M + m) * N + n0;
                if (vec) {
                    t[j][c] = *reinterpret_cast<const float4*>(p);
                } else {
                    t[j][c] = make_float4(n0 < N ? p[0] : 0.f, n0 + 1 < N ? p[1] : 0.f, n0 + 2 < N ? p[2] : 0.f,
                                          n0 + 3 < N ? p[3] : 0.f);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kRound; ++j) {
            if (sp0 + j < splits) {
#pragma unroll
                for (int c = 0; c < kCols; ++c) {
                    acc[c][0] += t[j][c].x;
                    acc[c][1] += t[j][c].y;
                    acc[c][2] += t[j][c].z;
                    acc[c][3] += t[j][c].w;
                }
                ss += tss[j];
            }
        }
    }
    if (norm) {
        // the row's sum of squares, summed in split order: the scale applies
        // before the epilogue
        const float r = 1.0f / sqrtf(ss / (float)a.K + a.eps);
#pragma unroll
        for (int c = 0; c < kCols; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[c][i] *= r;
    }
    float v[4] = {acc[0][0], acc[0][1], acc[0][2], acc[0][3]};
    if constexpr (EPI == EPI_SWIGLU) {
        const float u[4] = {acc[kCols - 1][0], acc[kCols - 1][1], acc[kCols - 1][2], acc[kCols - 1][3]};
        const int64_t j = (n >> 4) * 8 + (n & 7);      // first of the 4 gate columns
        if (j >= a.i_half) return;
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = silu_f32(round_bf16(v[i])) * round_bf16(u[i]);
        uint16_t* y = reinterpret_cast<uint16_t*>(a.y) + m * a.i_half + j;
        if (j + 3 < a.i_half && a.i_half % 4 == 0) {
            *reinterpret_cast<uint2*>(y) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        } else {
            for (int i = 0; i < 4; ++i) if (j + i < a.i_half) y[i] = (uint16_t)f32_to_bf16(o[i]);
        }
    } else if constexpr (epi_is_reduce(EPI)) {
        PeerVals<EPI> peers;
        load_peers<EPI>(a, m, n, peers);
        reduce_out4<EPI>(a, m, n, v, peers);
    } else {
        store_out4(a, m, n, v);
    }
}

typedef void (*SkinnyFn)(GemmArgs, int, int64_t, int, float*, unsigned*);
typedef int (*SkinnyLdsFn)(int);

// The norm-prologue kernel of a shape, for the column linears (EPI_STORE,
// EPI_SWIGLU), built for one 16-token tile with one row group, or four
// token tiles, X in LDS.
template <int MT, int KS, int NN, int NK, int XD, int EPI>
constexpr SkinnyFn skinny_norm_fn() {
    if constexpr (((MT == 1 && NN == 1) || MT == 4) && XD == 0 && NK > 1 && EPI <= EPI_SWIGLU)
        return skinny_kernel<MT, KS, NN, NK, XD, EPI, 1>;
    else
        return nullptr;
}

struct SkinnyEntry {
    int mt, ksteps, nwn, nwk, xd;
    SkinnyFn fn[kNumEpilogues];   // by epilogue (Epilogue's order)
    SkinnyFn fn_norm[2];   // with the norm prologue: EPI_STORE, EPI_SWIGLU (or nullptr)
    int threads;
    SkinnyLdsFn lds;
    int group_k;
};

#define TP_SK(MT, KS, NN, NK, XD)                                                                  \
    {MT, KS, NN, NK, XD,                                                                           \
     {skinny_kernel<MT, KS, NN, NK, XD, EPI_STORE>, skinny_kernel<MT, KS, NN, NK, XD, EPI_SWIGLU>,    \
      skinny_kernel<MT, KS, NN, NK, XD, EPI_REDUCE>, skinny_kernel<MT, KS, NN, NK, XD, EPI_REDUCE_ADD>, \
      skinny_kernel<MT, KS, NN, NK, XD, EPI_REDUCE_F32>,                                            \
      skinny_kernel<MT, KS, NN, NK, XD, EPI_REDUCE_ADD_F32>},                                       \
     {skinny_norm_fn<MT, KS, NN, NK, XD, EPI_STORE>(), skinny_norm_fn<MT, KS, NN, NK, XD, EPI_SWIGLU>()}, \
     SkinnyCfg<MT, KS, NN, NK, XD>::kThreads,                                                       \
     SkinnyCfg<MT, KS, NN, NK, XD>::lds_bytes, SkinnyCfg<MT, KS, NN, NK, XD>::kGroupK}
// M <= 16: every variant. M in (16, 64]: the ones that fit in registers.
#define TP_SK_MT1                                                                                    \
    TP_SK(1, 4, 4, 1, 0), TP_SK(1, 8, 4, 1, 0), TP_SK(1, 4, 2, 2, 0), TP_SK(1, 8, 2, 2, 0),             \
    TP_SK(1, 4, 1, 4, 0), TP_SK(1, 8, 1, 4, 0), TP_SK(1, 4, 4, 2, 0), TP_SK(1, 8, 4, 2, 0),             \
    TP_SK(1, 8, 4, 4, 0), TP_SK(1, 4, 4, 4, 0), TP_SK(1, 8, 1, 8, 0), TP_SK(1, 8, 2, 8, 0),             \
    TP_SK(1, 4, 2, 8, 0), TP_SK(1, 4, 1, 16, 0), TP_SK(1, 8, 1, 16, 0), TP_SK(1, 16, 1, 8, 0),          \
    TP_SK(1, 16, 2, 4, 0), TP_SK(1, 16, 4, 2, 0),                                                    \
    TP_SK(1, 4, 1, 4, 1), TP_SK(1, 8, 1, 4, 1), TP_SK(1, 8, 1, 8, 1), TP_SK(1, 4, 1, 16, 1),            \
    TP_SK(1, 8, 1, 16, 1), TP_SK(1, 16, 1, 8, 1), TP_SK(1, 4, 2, 8, 1), TP_SK(1, 20, 1, 8, 0)
#define TP_SK_MTN(MT)                                                                                \
    TP_SK(MT, 4, 4, 1, 0), TP_SK(MT, 8, 4, 1, 0), TP_SK(MT, 4, 2, 2, 0), TP_SK(MT, 8, 2, 2, 0),         \
    TP_SK(MT, 4, 1, 4, 0), TP_SK(MT, 8, 1, 4, 0), TP_SK(MT, 4, 4, 2, 0), TP_SK(MT, 8, 4, 2, 0),         \
    TP_SK(MT, 4, 4, 4, 0), TP_SK(MT, 4, 2, 8, 0), TP_SK(MT, 4, 1, 4, 1)

// (and variants whose k-steps cover the Llama-8B shards' K = 256, 896 and
// 1792 exactly, so that no wave loads X and W only to multiply zeros)
const SkinnyEntry kSkinnyTable[] = {TP_SK_MT1, TP_SK_MTN(2), TP_SK_MTN(4), TP_SK(4, 2, 1, 4, 1),
                                    TP_SK(1, 7, 1, 8, 0), TP_SK(1, 7, 1, 8, 1), TP_SK(4, 7, 1, 4, 0),
                                    TP_SK(4, 7, 1, 4, 1)};
#undef TP_SK_MT1
#undef TP_SK_MTN
#undef TP_SK

constexpr int kMaxLds = 160 * 1024 - 1024;   // dynamic LDS; the rest is the kernel's static LDS
constexpr int kNumSkinny = sizeof(kSkinnyTable) / sizeof(kSkinnyTable[0]);
constexpr int kSlots = kNumEpilogues + 2;     // kernels per entry: the epilogues, then the norm prologue's two
constexpr int kMaxDevices = 16;

// Per-device launch state, filled on first use: the dynamic-LDS limit set so
// far on each kernel, its occupancy at a given LDS size, the CU count. Read
// and written under one mutex, so concurrent host threads are safe.
struct DeviceLaunchState {
    int lds_attr[kNumSkinny][kSlots] = {};
    int occupancy[kNumSkinny][kSlots][2] = {};    // (lds bytes, workgroups per CU)
    int num_cus = 0;
};
std::mutex g_state_mu;
DeviceLaunchState g_state[kMaxDevices];

int find_skinny(const SkinnyPlan& p) {
    for (int i = 0; i < kNumSkinny; ++i) {
        const SkinnyEntry& e = kSkinnyTable[i];
        if (e.mt == p.mt && e.ksteps == p.ksteps && e.nwn == p.nwn && e.nwk == p.nwk && e.xd == p.xd) return i;
    }
    return -1;
}

int xrows_for(const SkinnyEntry& e, int64_t M) { return (int)(M < 16 * e.mt ? M : 16 * e.mt); }

SkinnyPlan make_plan(const SkinnyEntry& e, int64_t N, int64_t K) {
    SkinnyPlan p{e.mt, e.ksteps, e.nwn, e.nwk, e.xd, 1, 1};
    p.ntiles = (N + 16LL * e.nwn - 1) / (16LL * e.nwn);
    p.splits = (int)((K + e.group_k - 1) / e.group_k);
    return p;
}

}  // namespace

bool skinny_variant_exists(const SkinnyPlan& p) { return find_skinny(p) >= 0; }

bool skinny_plan_fits(const SkinnyPlan& p, int64_t M) {
    const int idx = find_skinny(p);
    if (idx < 0) return false;
    const SkinnyEntry& e = kSkinnyTable[idx];
    return e.lds(xrows_for(e, M)) <= kMaxLds;
}

// With the norm: one 16-token tile whose whole rows (K <= the variant's K
// coverage) sit in LDS.
bool skinny_norm_plan_fits(const SkinnyPlan& p, int64_t M, int64_t K) {
    (void)K;
    const int idx = find_skinny(p);
    if (idx < 0) return false;
    const SkinnyEntry& e = kSkinnyTable[idx];
    if (e.fn_norm[0] == nullptr || M > 16 * e.mt) return false;
    // dynamic LDS (staged rows, reduction buffer) + static (X X^T fragments, flags)
    return e.lds(xrows_for(e, M)) + e.nwk * e.mt * 4 * 64 * 4 + 512 <= 160 * 1024;
}

// Workspace floats a norm plan needs beyond the split partials: the splits'
// shares of the rows' sums of squares ([split][tile][16] for the single-
// launch exchange of one token tile, [split][M] beside the partials of a
// two-launch split).
int64_t skinny_norm_ss_floats(const SkinnyPlan& p, int64_t M) {
    if (p.splits <= 1) return 0;
    return p.mt == 4 ? (int64_t)p.splits * M : (int64_t)p.splits * p.ntiles * 16;
}

// Decode shape for a linear with the norm: as plan_skinny for M <= 16 (K
// split 4 ways over 1024-wide groups for weights with few 16-row tiles,
// otherwise the variant covering K in one workgroup with the least waste);
// for M in (16, 64] the plain linear's plan when it uses 64-token tiles and
// stages X in LDS (its K splits run in two launches); splits = 0 when none
// fits (the caller then normalises separately).
SkinnyPlan plan_skinny_norm(int64_t M, int64_t N, int64_t K, int64_t ws_floats, int64_t ws_counters) {
    struct Rule { int64_t kmax; int ks, nwn, nwk; };
    if (M > 16) {
        if (M <= 64) {
            const SkinnyPlan p = plan_skinny(M, N, K, ws_floats, ws_counters);
            const bool ws_ok =
                p.splits == 1 || skinny_workspace_floats(p, M, N) + skinny_norm_ss_floats(p, M) <= ws_floats;
            if (p.splits >= 1 && ws_ok && skinny_norm_plan_fits(p, M, K)) return p;
        }
        SkinnyPlan none{4, 0, 0, 0, 0, 0, 0};
        return none;
    }
    if ((N + 15) / 16 < 128 && K >= 2048) {
        SkinnyPlan p{1, 8, 1, 4, 0, 1, 1};
        const int idx = find_skinny(p);
        if (idx >= 0) {
            p = make_plan(kSkinnyTable[idx], N, K);
            // partial tiles, then each split's share of the rows' sums of squares
            const bool ws_ok = p.splits == 1 || (skinny_workspace_floats(p, M, N) + (int64_t)p.splits * p.ntiles * 16 <=
                                                     ws_floats &&
                                                 p.ntiles <= ws_counters);
            if (ws_ok && skinny_norm_plan_fits(p, M, K)) return p;
        }
    }
    static const Rule rules[] = {{512, 4, 1, 4}, {1024, 8, 1, 4}, {2048, 8, 1, 8}, {4096, 16, 1, 8}, {5120, 20, 1, 8}};
    for (const Rule& r : rules) {
        if (K > r.kmax) continue;
        SkinnyPlan p{1, r.ks, r.nwn, r.nwk, 0, 1, 1};
        const int idx = find_skinny(p);
        if (idx < 0) continue;
        p = make_plan(kSkinnyTable[idx], N, K);
        if (p.splits == 1 && skinny_norm_plan_fits(p, M, K)) return p;
    }
    SkinnyPlan none{1, 0, 0, 0, 0, 0, 0};
    return none;
}

// Pick the decode kernel shape for one linear, from MI355X sweeps of every
// variant at the Llama-8B decode shapes.
//
// M <= 16: one workgroup covers all of K for 16 weight rows (no exchange
// between workgroups) with the variant whose K coverage fits K with the least
// waste, except when the weight has too few 16-row tiles to fill the GPU,
// where K is split 4 ways (an exchange costs a few serialized memory round
// trips at the end of the kernel, worth it only then). M in (16, 64]: the
// measured winners per K and N for 64-token tiles (see below for the 32-token
// exception). Otherwise a cost model counts HBM bytes
// (the weight once, the fp32 partial round trip when K is split across
// workgroups, a quarter weight for X re-reads from L2) divided by how well the
// grid fills the 256 CUs.
SkinnyPlan plan_skinny(int64_t M, int64_t N, int64_t K, int64_t ws_floats, int64_t ws_counters) {
    // 17-32 tokens run the 64-token plans (rows past M masked), which beat
    // the 32-token tiles' cost-model choice (24 tokens, weights rotated past
    // the last-level cache: qkv 768 x 4096 10.7 -> 8.8 us, o 4096 x 512 with
    // the sum over 8 ranks 7.35 -> 5.23, gate_up 1792 x 4096 11.4 -> 10.7),
    // except on weights of more than 2048 rows with K in (1024, 2048]
    // (down 4096 x 1792 with the sum: 11.3 against 12.5 us).
    const bool tiles32 = M > 16 && M <= 32 && N > 2048 && K > 1024 && K <= 2048;
    const int mt = M <= 16 ? 1 : (tiles32 ? 2 : 4);
    struct Rule { int64_t kmax; int ks, nwn, nwk, xd; };
    auto first_fit = [&](const Rule* rules, int n, SkinnyPlan* out) {
        for (int i = 0; i < n; ++i) {
            const Rule& r = rules[i];
            if (K > r.kmax) continue;
            SkinnyPlan p{mt, r.ks, r.nwn, r.nwk, r.xd, 1, 1};
            const int idx = find_skinny(p);
            if (idx < 0 || !skinny_plan_fits(p, M)) continue;
            p = make_plan(kSkinnyTable[idx], N, K);
            if (p.splits > 1 && (p.splits * M * N > ws_floats || p.ntiles > ws_counters)) continue;
            *out = p;
            return true;
        }
        return false;
    };
    SkinnyPlan chosen;
    if (mt == 1) {
        // Few 16-row tiles (qkv-sized N): split K 4 ways over 1024-wide
        // groups; otherwise cover K in one workgroup.
        static const Rule few_tiles[] = {{1 << 30, 8, 1, 4, 0}};
        static const Rule rules[] = {
            {512, 4, 1, 4, 1}, {1024, 8, 1, 4, 1}, {1792, 7, 1, 8, 0}, {2048, 8, 1, 8, 0}, {4096, 16, 1, 8, 0},
            {5120, 20, 1, 8, 0},
        };
        if ((N + 15) / 16 < 128 && K >= 2048 && first_fit(few_tiles, 1, &chosen)) return chosen;
        if (first_fit(rules, 6, &chosen)) return chosen;
    } else if (mt == 4) {
        // M in (32, 64]: measured winners at the Llama-8B t=16 shard shapes
        // (weights rotated past the last-level cache, K splits in two
        // launches; gate_up 1792 x 4096: 64-row tiles split 8 ways, 14.2 us;
        // qkv 512 x 4096: 16-row tiles split 8 ways with X staged, 8.2 us;
        // o 4096 x 256 and down 4096 x 896 with the sum over 16 ranks: 4
        // waves whose k-steps cover K exactly, X loaded per wave, 6.4 and
        // 10.2 us against 7.6 and 11.1 for the next-larger coverage).
        static const Rule rules_small_n[] = {{256, 2, 1, 4, 1}, {512, 4, 1, 4, 1}, {896, 7, 1, 4, 1},
                                             {1024, 8, 1, 4, 0}, {1 << 30, 4, 1, 4, 0}};
        static const Rule rules_mid_n[] = {{256, 2, 1, 4, 1}, {512, 4, 1, 4, 1}, {896, 7, 1, 4, 1},
                                           {1024, 8, 1, 4, 0}, {1 << 30, 4, 4, 4, 0}};
        static const Rule rules[] = {{256, 2, 1, 4, 1}, {512, 4, 1, 4, 1}, {896, 7, 1, 4, 1},
                                     {1024, 8, 1, 4, 0}, {1 << 30, 8, 4, 2, 0}};
        if (first_fit(N <= 1024 ? rules_small_n : N <= 2048 ? rules_mid_n : rules, 5, &chosen)) return chosen;
    }
    SkinnyPlan best{mt, 8, 4, 2, 0, 0, 0};   // splits = 0: nothing fits (the caller reports it)
    double best_cost = -1.0;
    for (const SkinnyEntry& e : kSkinnyTable) {
        if (e.mt != mt || e.lds(xrows_for(e, M)) > kMaxLds) continue;
        const SkinnyPlan p = make_plan(e, N, K);
        if (p.splits > 1 && (p.splits * M * N > ws_floats || p.ntiles > ws_counters)) continue;
        if (p.splits > 65535) continue;
        const double wgs = (double)p.ntiles * (double)p.splits;
        double bytes = 2.0 * (double)N * (double)K;
        if (p.splits > 1) bytes += 8.0 * (double)p.splits * (double)M * (double)N;
        bytes += 0.25 * wgs * 16.0 * mt * (double)e.group_k * 2.0;
        double fill = wgs * e.threads / (256.0 * 512.0);
        if (fill > 1.0) fill = 1.0;
        const double cost = bytes / fill;
        if (best_cost < 0.0 || cost < best_cost) {
            best_cost = cost;
            best = p;
        }
    }
    return best;
}

int64_t skinny_workspace_floats(const SkinnyPlan& p, int64_t M, int64_t N) {
    return p.splits > 1 ? (int64_t)p.splits * M * N : 0;
}

hipError_t launch_skinny(const GemmArgs& a, const SkinnyPlan& p, const Workspace& ws, hipStream_t s) {
    const int idx = find_skinny(p);
    if (idx < 0) return hipErrorInvalidValue;
    const SkinnyEntry* e = &kSkinnyTable[idx];
    const int epi = a.epi;
    if (epi < 0 || epi >= kNumEpilogues) return hipErrorInvalidValue;
    const bool norm = a.norm != 0;
    if (norm && (epi > EPI_SWIGLU || !skinny_norm_plan_fits(p, a.M, a.K))) return hipErrorInvalidValue;
    const SkinnyFn fn = norm ? e->fn_norm[epi] : e->fn[epi];
    if (fn == nullptr) return hipErrorInvalidValue;
    const int slot = norm ? kNumEpilogues + epi : epi;      // launch state below is per function
    const int xrows = xrows_for(*e, a.M);
    const int lds = e->lds(xrows);
    if (lds > kMaxLds) return hipErrorInvalidValue;
    int dev = 0;
    hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) return he;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int64_t grid_x = p.ntiles;
    {
        std::lock_guard<std::mutex> lock(g_state_mu);
        DeviceLaunchState& st = g_state[dev];
        if (lds > 65536 && lds > st.lds_attr[idx][slot]) {
            he = hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
            if (he != hipSuccess) return he;
            st.lds_attr[idx][slot] = lds;
        }
        if (p.splits == 1 && !p.xd) {
            // Unsplit: as many workgroups as fit on the GPU at once, each
            // looping over row tiles (X is staged once per workgroup).
            if (st.num_cus == 0) {
                he = hipDeviceGetAttribute(&st.num_cus, hipDeviceAttributeMultiprocessorCount, dev);
                if (he != hipSuccess) return he;
            }
            int* occ = st.occupancy[idx][slot];
            if (occ[0] != lds || occ[1] == 0) {
                int per_cu = 0;
                he = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), e->threads,
                                                                  lds);
                if (he != hipSuccess) return he;
                occ[0] = lds;
                occ[1] = per_cu > 0 ? per_cu : 1;
            }
            const int64_t cap = (int64_t)occ[1] * st.num_cus;
            if (grid_x > cap) grid_x = cap;
        }
    }
    dim3 grid((unsigned)grid_x, (unsigned)p.splits);
    if (skinny_split_launches(p, a) == 2) {
        // The partial tiles in one launch, their sum and the epilogue in a
        // second: with 64 tokens a split tile holds up to 64 KB of partials
        // per split, which one last-arriving workgroup would read alone
        // (MI355X, Llama t = 16 gate_up: the 224 workgroups of 64-row
        // tiles finish their partials by ~10 us, the last arrivals then
        // take another 6-7 us).
        hipLaunchKernelGGL(fn, grid, dim3(e->threads), lds, s, a, p.splits, p.ntiles, xrows, ws.partials,
                           static_cast<unsigned*>(nullptr));
        he = hipGetLastError();
        if (he != hipSuccess) return he;
        const int64_t groups = epi == EPI_SWIGLU ? a.N / 8 : (a.N + 3) / 4;
        const int64_t threads = a.M * groups;
        const dim3 g2((unsigned)((threads + 255) / 256));
        switch (epi) {
        case EPI_STORE: hipLaunchKernelGGL(skinny_split_finish<EPI_STORE>, g2, dim3(256), 0, s, a, p.splits, ws.partials); break;
        case EPI_SWIGLU: hipLaunchKernelGGL(skinny_split_finish<EPI_SWIGLU>, g2, dim3(256), 0, s, a, p.splits, ws.partials); break;
        case EPI_REDUCE: hipLaunchKernelGGL(skinny_split_finish<EPI_REDUCE>, g2, dim3(256), 0, s, a, p.splits, ws.partials); break;
        case EPI_REDUCE_ADD: hipLaunchKernelGGL(skinny_split_finish<EPI_REDUCE_ADD>, g2, dim3(256), 0, s, a, p.splits, ws.partials); break;
        case EPI_REDUCE_F32: hipLaunchKernelGGL(skinny_split_finish<EPI_REDUCE_F32>, g2, dim3(256), 0, s, a, p.splits, ws.partials); break;
        case EPI_REDUCE_ADD_F32: hipLaunchKernelGGL(skinny_split_finish<EPI_REDUCE_ADD_F32>, g2, dim3(256), 0, s, a, p.splits, ws.partials); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    hipLaunchKernelGGL(fn, grid, dim3(e->threads), lds, s, a, p.splits, p.ntiles, xrows, ws.partials, ws.counters);
    return hipGetLastError();
}

// A K split at more than 32 tokens runs as two launches (with the norm, the
// splits' shares of the sums of squares go beside the partials and the
// second launch applies the scale): with 64 tokens a split tile holds 4-16 KB
// of partials per split per 16 rows, which the one last-arriving workgroup
// of the single-launch exchange would read alone after an arrival round trip
// (Llama t = 16 qkv, 16 rows x 8 splits: 10.0 us in one launch, 8.7 in two;
// gate_up, 64 rows x 8 splits: 16.8 in one, 14.4 in two).
int skinny_split_launches(const SkinnyPlan& p, const GemmArgs& a) {
    (void)a;
    return (p.splits > 1 && p.mt == 4) ? 2 : 1;
}

}  // namespace tpk
