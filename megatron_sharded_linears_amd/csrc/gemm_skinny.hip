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
//     that many loads are in flight per CU.
//   * X's K-chunk is loaded once per workgroup into LDS (padded rows) and
//     shared by the waves that cover different weight rows.
//   * K is split across the waves of a workgroup (summed through LDS) and, if
//     the weight has too few rows to fill 256 CUs, across workgroups: each
//     writes an fp32 partial tile to the workspace and the last workgroup to
//     arrive on a tile (one atomic counter per tile) sums the partials in
//     split order, so the result does not depend on arrival order.
#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

template <int MT, int KSTEPS, int NWN, int NWK>
struct SkinnyCfg {
    static constexpr int kThreads = 64 * NWN * NWK;
    static constexpr int kRows = 16 * NWN;             // weight rows per workgroup
    static constexpr int kWaveK = 32 * KSTEPS;         // K per wave
    static constexpr int kGroupK = kWaveK * NWK;       // K per workgroup
    static constexpr int kTokens = 16 * MT;
    static constexpr int kXStride = kGroupK + 8;       // LDS row stride (elements), 16 B pad
    static constexpr int kXBytes = kTokens * kXStride * 2;
    static constexpr int kRedBytes = NWK > 1 ? (NWK - 1) * NWN * MT * 4 * 64 * 4 : 0;
    static constexpr int kLdsBytes = kXBytes > kRedBytes ? kXBytes : kRedBytes;
};

__device__ __forceinline__ void store_out4(const GemmArgs& a, int64_t m, int64_t n, const float* v) {
    // 4 consecutive outputs y[m, n..n+3] (+ bias), bf16 or fp32.
    float o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float b = 0.f;
        if (a.bias != nullptr && n + i < a.N) b = bf16_to_f32(reinterpret_cast<const uint16_t*>(a.bias)[n + i]);
        o[i] = v[i] + b;
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

template <int MT, int KSTEPS, int NWN, int NWK>
__global__ void __launch_bounds__(64 * NWN * NWK)
skinny_kernel(GemmArgs a, int splits, float* __restrict__ ws, unsigned* __restrict__ counters) {
    using C = SkinnyCfg<MT, KSTEPS, NWN, NWK>;
    extern __shared__ __align__(16) unsigned char smem[];
    bf16_t* xs = reinterpret_cast<bf16_t*>(smem);
    __shared__ unsigned s_last;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave % NWN;
    const int wk = wave / NWN;
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t tile = blockIdx.x;
    const int split = blockIdx.y;
    const int64_t k_group = (int64_t)split * C::kGroupK;
    const int64_t n_wave = tile * C::kRows + wn * 16;

    const bf16_t* __restrict__ X = reinterpret_cast<const bf16_t*>(a.x);
    const bf16_t* __restrict__ W = reinterpret_cast<const bf16_t*>(a.w);

    // 1. Stage X[:, k_group : k_group + kGroupK] into registers (issued first so
    //    that waiting for it does not wait for the weight stream).
    constexpr int kXChunks = C::kTokens * (C::kGroupK / 8);
    constexpr int kXPerThread = (kXChunks + C::kThreads - 1) / C::kThreads;
    uint4 xr[kXPerThread];
#pragma unroll
    for (int j = 0; j < kXPerThread; ++j) {
        const int c = tid + j * C::kThreads;
        const int m = c / (C::kGroupK / 8);
        const int kc = c % (C::kGroupK / 8);
        const int64_t k = k_group + kc * 8;
        xr[j] = make_uint4(0u, 0u, 0u, 0u);
        if (c < kXChunks && m < M && k < K)
            xr[j] = *reinterpret_cast<const uint4*>(X + (int64_t)m * K + k);
    }

    // 2. Issue every weight load of this wave.
    const int64_t n_lane = n_wave + (lane & 15);
    const int64_t k_wave = k_group + (int64_t)wk * C::kWaveK + 8 * (lane >> 4);
    uint4 wr[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
        const int64_t k = k_wave + 32 * s;
        wr[s] = make_uint4(0u, 0u, 0u, 0u);
        if (n_lane < N && k < K)
            wr[s] = ld_nt16(W + n_lane * K + k);
    }

    // 3. X chunk -> LDS.
#pragma unroll
    for (int j = 0; j < kXPerThread; ++j) {
        const int c = tid + j * C::kThreads;
        if (c < kXChunks) {
            const int m = c / (C::kGroupK / 8);
            const int kc = c % (C::kGroupK / 8);
            *reinterpret_cast<uint4*>(xs + m * C::kXStride + kc * 8) = xr[j];
        }
    }
    __syncthreads();

    // 4. MFMAs: acc[mt] holds D[n = 4*(lane/16) + i][m = 16*mt + lane%16].
    f32x4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int xcol = wk * C::kWaveK + 8 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, wr[s]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const uint4 xv = *reinterpret_cast<const uint4*>(xs + (16 * mt + (lane & 15)) * C::kXStride + xcol + 32 * s);
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, xv), acc[mt], 0, 0, 0);
        }
    }

    // 5. Sum the NWK waves that share rows, in wave order, through LDS.
    if (NWK > 1) {
        __syncthreads();  // X chunk no longer needed: reuse its LDS
        float* red = reinterpret_cast<float*>(smem);
        if (wk > 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    red[((((wk - 1) * NWN + wn) * MT + mt) * 4 + i) * 64 + lane] = acc[mt][i];
        }
        __syncthreads();
        if (wk == 0) {
#pragma unroll
            for (int w = 1; w < NWK; ++w)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[mt][i] += red[((((w - 1) * NWN + wn) * MT + mt) * 4 + i) * 64 + lane];
        }
    }

    const int64_t n_out = n_wave + 4 * (lane >> 4);   // first of this lane's 4 outputs
    if (splits == 1) {
        if (wk == 0) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int64_t m = 16 * mt + (lane & 15);
                if (m < M && n_out < N) {
                    float v[4] = {acc[mt][0], acc[mt][1], acc[mt][2], acc[mt][3]};
                    store_out4(a, m, n_out, v);
                }
            }
        }
        return;
    }

    // 6. K split across workgroups: publish this split's partial tile.
    if (wk == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int64_t m = 16 * mt + (lane & 15);
            if (m < M) {
                float* p = ws + ((int64_t)split * M + m) * N;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (n_out + i < N) p[n_out + i] = acc[mt][i];
            }
        }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = atomicAdd(&counters[tile], 1u);
        s_last = (prev == (unsigned)(splits - 1)) ? 1u : 0u;
    }
    __syncthreads();
    if (s_last == 0u) return;
    __threadfence();

    // 7. Last workgroup on this tile: sum the partials in split order.
    if (wk == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int64_t m = 16 * mt + (lane & 15);
            if (m < M && n_out < N) {
                float v[4] = {0.f, 0.f, 0.f, 0.f};
                for (int sp = 0; sp < splits; ++sp) {
                    const float* p = ws + ((int64_t)sp * M + m) * N;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (n_out + i < N) v[i] += __builtin_nontemporal_load(p + n_out + i);
                }
                store_out4(a, m, n_out, v);
            }
        }
    }
    if (tid == 0) atomicExch(&counters[tile], 0u);
}

typedef void (*SkinnyFn)(GemmArgs, int, float*, unsigned*);

struct SkinnyEntry {
    int mt, ksteps, nwn, nwk;
    SkinnyFn fn;
    int threads;
    int lds;
};

#define TP_SK(MT, KS, NN, NK)                                                        \
    {MT, KS, NN, NK, skinny_kernel<MT, KS, NN, NK>, SkinnyCfg<MT, KS, NN, NK>::kThreads, \
     SkinnyCfg<MT, KS, NN, NK>::kLdsBytes}
#define TP_SK_MT(MT)                                                                  \
    TP_SK(MT, 4, 4, 1), TP_SK(MT, 8, 4, 1), TP_SK(MT, 4, 2, 2), TP_SK(MT, 8, 2, 2),     \
    TP_SK(MT, 4, 1, 4), TP_SK(MT, 8, 1, 4), TP_SK(MT, 4, 4, 2), TP_SK(MT, 8, 4, 2),     \
    TP_SK(MT, 8, 4, 4), TP_SK(MT, 4, 4, 4)

const SkinnyEntry kSkinnyTable[] = {TP_SK_MT(1), TP_SK_MT(2), TP_SK_MT(4)};
#undef TP_SK_MT
#undef TP_SK

const SkinnyEntry* find_skinny(const SkinnyPlan& p) {
    for (const SkinnyEntry& e : kSkinnyTable)
        if (e.mt == p.mt && e.ksteps == p.ksteps && e.nwn == p.nwn && e.nwk == p.nwk) return &e;
    return nullptr;
}

}  // namespace

bool skinny_variant_exists(const SkinnyPlan& p) { return find_skinny(p) != nullptr; }

// Pick the decode kernel shape for one linear. The cost model counts HBM
// bytes (the weight once, plus the fp32 partial round trip when K is split
// across workgroups, plus a quarter weight for X re-reads from L2) and
// divides by how well the grid fills the 256 CUs (at least 8 waves per CU).
SkinnyPlan plan_skinny(int64_t M, int64_t N, int64_t K) {
    const int mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    SkinnyPlan best{mt, 8, 4, 2, 1, 1};
    double best_cost = -1.0;
    for (const SkinnyEntry& e : kSkinnyTable) {
        if (e.mt != mt) continue;
        const int64_t rows = 16LL * e.nwn;
        const int64_t gk = 32LL * e.ksteps * e.nwk;
        const int64_t ntiles = (N + rows - 1) / rows;
        const int64_t splits = (K + gk - 1) / gk;
        if (splits > 1 && (splits * M * N > kSkinnyWsFloats || ntiles > kSkinnyWsCounters)) continue;
        if (splits > 65535) continue;
        const double wgs = (double)ntiles * (double)splits;
        double bytes = 2.0 * (double)N * (double)K;
        if (splits > 1) bytes += 8.0 * (double)splits * (double)M * (double)N;
        bytes += 0.25 * wgs * 16.0 * mt * (double)gk * 2.0;
        double fill = wgs * e.threads / (256.0 * 512.0);
        if (fill > 1.0) fill = 1.0;
        const double cost = bytes / fill;
        if (best_cost < 0.0 || cost < best_cost) {
            best_cost = cost;
            best = SkinnyPlan{mt, e.ksteps, e.nwn, e.nwk, (int)splits, ntiles};
        }
    }
    return best;
}

int64_t skinny_workspace_floats(const SkinnyPlan& p, int64_t M, int64_t N) {
    return p.splits > 1 ? (int64_t)p.splits * M * N : 0;
}

hipError_t launch_skinny(const GemmArgs& a, const SkinnyPlan& p, const Workspace& ws, hipStream_t s) {
    const SkinnyEntry* e = find_skinny(p);
    if (e == nullptr) return hipErrorInvalidValue;
    if (e->lds > 65536) {
        const hipError_t ae = hipFuncSetAttribute(reinterpret_cast<const void*>(e->fn),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, e->lds);
        if (ae != hipSuccess) return ae;
    }
    dim3 grid((unsigned)p.ntiles, (unsigned)p.splits);
    hipLaunchKernelGGL(e->fn, grid, dim3(e->threads), e->lds, s, a, p.splits, ws.partials, ws.counters);
    return hipGetLastError();
}

}  // namespace tpk
