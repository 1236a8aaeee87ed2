// Prefill-sized linear on gfx950: Y[M, N] = X[M, K] W[N, K]^T (+ bias) with
// M > 64 tokens. These shard GEMMs are dense contractions well above the
// MI355X ridge point, so they are bound by the bf16 matrix cores.
//
// Tiling: a 256-thread workgroup owns a 128 (tokens) x 128 (weight rows)
// output tile and walks K in steps of 64. Both operands are K-contiguous; each
// k-tile of X and W is copied global -> VGPR -> LDS (rows padded by 16 bytes
// so the 16 lanes of an MFMA operand read hit distinct banks), double
// buffered so the next tile's global loads are in flight while the current
// one feeds the MFMAs. Each wave computes a 64 x 64 block as 4 x 4
// v_mfma_f32_16x16x32_bf16 with W as the A operand, so each lane ends with 4
// consecutive outputs of one token row.
#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

constexpr int kBM = 128;   // tokens per tile
constexpr int kBN = 128;   // weight rows per tile
constexpr int kBK = 64;    // K per stage
constexpr int kStride = kBK + 8;               // LDS row stride in elements
constexpr int kThreads = 256;
constexpr int kChunksPerThread = kBM * (kBK / 8) / kThreads;   // 4 (same for W)
constexpr int kStageElems = (kBM + kBN) * kStride;

__device__ __forceinline__ void store_out4(const GemmArgs& a, int64_t m, int64_t n, const float* v) {
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
        if (full) *reinterpret_cast<float4*>(y + base) = make_float4(o[0], o[1], o[2], o[3]);
        else for (int i = 0; i < 4; ++i) if (n + i < a.N) y[base + i] = o[i];
    } else {
        uint16_t* y = reinterpret_cast<uint16_t*>(a.y);
        if (full) *reinterpret_cast<uint2*>(y + base) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        else for (int i = 0; i < 4; ++i) if (n + i < a.N) y[base + i] = (uint16_t)f32_to_bf16(o[i]);
    }
}

__global__ void __launch_bounds__(kThreads)
tiled_kernel(GemmArgs a) {
    __shared__ __align__(16) bf16_t lds[2 * kStageElems];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;      // token half
    const int wn = wave & 1;       // weight-row half
    const int64_t M = a.M, N = a.N, K = a.K;
    const int64_t n0 = (int64_t)blockIdx.x * kBN;
    const int64_t m0 = (int64_t)blockIdx.y * kBM;
    const bf16_t* __restrict__ X = reinterpret_cast<const bf16_t*>(a.x);
    const bf16_t* __restrict__ W = reinterpret_cast<const bf16_t*>(a.w);

    uint4 xr[kChunksPerThread], wr[kChunksPerThread];

    auto load_tile = [&](int64_t k0) {
#pragma unroll
        for (int j = 0; j < kChunksPerThread; ++j) {
            const int c = tid + j * kThreads;
            const int r = c >> 3;
            const int64_t k = k0 + (c & 7) * 8;
            xr[j] = make_uint4(0u, 0u, 0u, 0u);
            wr[j] = make_uint4(0u, 0u, 0u, 0u);
            if (k < K) {
                if (m0 + r < M) xr[j] = *reinterpret_cast<const uint4*>(X + (m0 + r) * K + k);
                if (n0 + r < N) wr[j] = *reinterpret_cast<const uint4*>(W + (n0 + r) * K + k);
            }
        }
    };
    auto store_tile = [&](int stage) {
        bf16_t* xs = lds + stage * kStageElems;
        bf16_t* wsm = xs + kBM * kStride;
#pragma unroll
        for (int j = 0; j < kChunksPerThread; ++j) {
            const int c = tid + j * kThreads;
            const int r = c >> 3;
            const int kc = (c & 7) * 8;
            *reinterpret_cast<uint4*>(xs + r * kStride + kc) = xr[j];
            *reinterpret_cast<uint4*>(wsm + r * kStride + kc) = wr[j];
        }
    };

    f32x4_t acc[4][4];   // [weight block nb][token block mb]
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int64_t ktiles = (K + kBK - 1) / kBK;
    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int64_t kt = 0; kt < ktiles; ++kt) {
        const int stage = (int)(kt & 1);
        if (kt + 1 < ktiles) load_tile((kt + 1) * kBK);
        const bf16_t* xs = lds + stage * kStageElems;
        const bf16_t* wsm = xs + kBM * kStride;
#pragma unroll
        for (int s = 0; s < kBK / 32; ++s) {
            const int col = s * 32 + 8 * (lane >> 4);
            bf16x8_t av[4], bv[4];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
                av[nb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                    wsm + (wn * 64 + nb * 16 + (lane & 15)) * kStride + col));
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
                bv[mb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                    xs + (wm * 64 + mb * 16 + (lane & 15)) * kStride + col));
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
                    acc[nb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[nb], bv[mb], acc[nb][mb], 0, 0, 0);
        }
        if (kt + 1 < ktiles) store_tile(stage ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
        const int64_t n = n0 + wn * 64 + nb * 16 + 4 * (lane >> 4);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int64_t m = m0 + wm * 64 + mb * 16 + (lane & 15);
            if (m < M && n < N) {
                float v[4] = {acc[nb][mb][0], acc[nb][mb][1], acc[nb][mb][2], acc[nb][mb][3]};
                store_out4(a, m, n, v);
            }
        }
    }
}

}  // namespace

hipError_t launch_tiled(const GemmArgs& a, hipStream_t s) {
    dim3 grid((unsigned)((a.N + kBN - 1) / kBN), (unsigned)((a.M + kBM - 1) / kBM));
    hipLaunchKernelGGL(tiled_kernel, grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace tpk
