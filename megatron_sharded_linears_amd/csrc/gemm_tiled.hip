// Prefill-sized linear on gfx950: Y[M, N] = X[M, K] W[N, K]^T (+ bias) with
// M > 64 tokens. These shard GEMMs are dense contractions far above the
// MI355X ridge point (~315 flop/B), so they are bound by the bf16 matrix
// cores (2.5 PFLOP/s dense).
//
// Common to both kernels:
//   * v_mfma_f32_32x32x16_bf16 with W as the A operand (32 weight rows) and
//     X as the B operand (32 tokens): D[n][m] = Y[m][n].
//   * A workgroup owns a BN (weight rows) x BM (tokens) tile, split over
//     2 x WGM waves; each wave owns (BN/2) x (BM/WGM) as a grid of 32 x 32
//     MFMA blocks whose accumulators stay in registers (every access to them
//     uses compile-time indices).
//   * Tiles are numbered so that each of the 8 XCDs (workgroup id mod 8)
//     gets a contiguous range, walked in groups of 8 weight-row tiles with
//     the token tile fastest inside a group: the 32 tiles an XCD runs at
//     once share 8 W panels and 4 X panels, whose k-slices its L2 serves to
//     all of them (MI355X, against token-fastest order over whole columns:
//     Qwen-32B t = 8 o_proj 76.6 -> 66.2 us, gate_up 290 -> 283 us).
//   * Epilogue: accumulators go through LDS one block row at a time, then all
//     threads write rows of Y in runs of 4 outputs (bias added there; interior
//     tiles' bf16 outputs with the non-temporal hint).
//   * SwiGLU epilogue: a tile's first BN/2 rows are gate rows and its last
//     BN/2 the same up rows, i.e. the two wave rows' halves of the LDS slab,
//     so a thread reads a gate run and its up run and writes 4 outputs.
//
// tiled_dma_kernel (K % 32 == 0) and tiled_dma64_kernel (K % 64 == 0):
// k-tiles land in LDS by direct global -> LDS loads (buffer_load ... lds
// through buffer resources) in rings of 2-4 stages (details below).
// tiled_reg_kernel (any K % 8 == 0, and operands of 4 GiB or more): k-tiles
// of 64 go global -> VGPR -> LDS, double buffered, 128-byte rows
// XOR-swizzled by (row / 2) mod 8.
#include <atomic>

#include "common.h"
#include "kernels.h"

namespace tpk {

namespace {

constexpr int kBK = 64;         // K per stage
#ifndef TP_TILE_GROUP_N
#define TP_TILE_GROUP_N 8
#endif
constexpr int kThreads = 256;   // 4 waves, 2 x 2
constexpr int kXcds = 8;
constexpr int kCus = 256;       // MI355X compute units

// Tile t of an XCD-contiguous range -> (weight-row tile, token tile): groups
// of TP_TILE_GROUP_N weight-row tiles, token tiles walked within a group, so
// the tiles an XCD runs at once share TP_TILE_GROUP_N W panels and
// 32 / TP_TILE_GROUP_N X panels.
__device__ __forceinline__ void group_tile(int t, int tiles_n, int tiles_m, int& tn, int& tm) {
    constexpr int GN = TP_TILE_GROUP_N;
    const int per_group = GN * tiles_m;
    const int g = t / per_group;
    const int w = t - g * per_group;
    const int left = tiles_n - g * GN;
    const int gn = left < GN ? left : GN;
    tm = w / gn;
    tn = g * GN + (w - tm * gn);
}

template <int BN, int BM>
struct TileCfg {
    static constexpr int kWN = BN / 2;           // weight rows per wave
    static constexpr int kWM = BM / 2;           // tokens per wave
    static constexpr int kBlkN = kWN / 32;       // 32x32 blocks per wave along N
    static constexpr int kBlkM = kWM / 32;
    static constexpr int kWChunks = BN * (kBK / 8) / kThreads;   // 16-B loads per thread per k-tile
    static constexpr int kXChunks = BM * (kBK / 8) / kThreads;
    static constexpr int kStageElems = (BN + BM) * kBK;
    static constexpr int kLdsBytes = 2 * kStageElems * 2;
};

// Output row stride (elements) and SwiGLU up-row offset of a launch.
__device__ __forceinline__ int64_t out_ld(const GemmArgs& a) {
    return a.ldy != 0 ? a.ldy : (a.epi == EPI_SWIGLU ? a.i_half : a.N);
}
__device__ __forceinline__ int64_t up_rows(const GemmArgs& a) { return a.up_off != 0 ? a.up_off : a.i_half; }

// Weight row of kernel row v for tiles of BN rows, or -1 past the end.
// EPI_SWIGLU: tile b holds gate rows [b BN/2, (b+1) BN/2), then the same up rows.
template <int BN>
__device__ __forceinline__ int64_t tile_w_row(const GemmArgs& a, int64_t v) {
    if (a.epi != EPI_SWIGLU) return v < a.N ? v : -1;
    const int64_t j = (v / BN) * (BN / 2) + (v % (BN / 2));
    if (j >= a.i_half) return -1;
    return (v % BN) >= BN / 2 ? up_rows(a) + j : j;
}

// The DMA kernels read their sources through buffer resources (common.h):
// 32-bit lane offsets, and the k-tile's byte offset in the scalar offset
// operand. Against global_load_lds with 64-bit lane addresses this staged the
// same bytes 3-8% faster per prefill linear (MI355X, the Llama-8B t = 2 and
// Qwen-32B t = 8 shard shapes, timed alternately). The launcher keeps both
// extents within kMaxBufferBytes.

// Weight rows a launch reads: every row for a plain linear; gate rows
// [0, i_half) and up rows [up_rows, up_rows + i_half) with SwiGLU.
__host__ __device__ __forceinline__ int64_t w_rows_read(const GemmArgs& a) {
    return a.epi == EPI_SWIGLU ? (a.up_off != 0 ? a.up_off : a.i_half) + a.i_half : a.N;
}

// SwiGLU of 4 gate values and their up values: y[m, j..j+3], bf16, with the
// gate_up outputs rounded to bf16 first as the unfused path stores them.
__device__ __forceinline__ void swiglu4(float4 g, float4 u, float* o) {
    const float gv[4] = {g.x, g.y, g.z, g.w}, uv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = silu_f32(round_bf16(gv[i])) * round_bf16(uv[i]);
}

__device__ __forceinline__ void swiglu_out4(const GemmArgs& a, int64_t m, int64_t j, float4 g, float4 u) {
    float o[4];
    swiglu4(g, u, o);
    const int64_t ld = out_ld(a);
    uint16_t* y = reinterpret_cast<uint16_t*>(a.y) + m * ld + j;
    if (j + 3 < a.i_half && ld % 4 == 0) {
        *reinterpret_cast<uint2*>(y) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    } else {
        for (int i = 0; i < 4; ++i) if (j + i < a.i_half) y[i] = (uint16_t)f32_to_bf16(o[i]);
    }
}

// Element offset of (row, 16-byte chunk c) in a [rows][64] bf16 LDS tile.
__device__ __forceinline__ int swz(int row, int c) {
    return row * kBK + ((c ^ ((row >> 1) & 7)) << 3);
}

__device__ __forceinline__ void store_out4(const GemmArgs& a, int64_t m, int64_t n, const float* v) {
    float o[4] = {v[0], v[1], v[2], v[3]};
    if (a.bias != nullptr) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (n + i < a.N) o[i] += bf16_to_f32(reinterpret_cast<const uint16_t*>(a.bias)[n + i]);
    }
    const int64_t ld = out_ld(a);
    const int64_t base = m * ld + n;
    const bool full = (n + 3 < a.N) && (ld % 4 == 0);
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

// Tile epilogue, shared by the tiled kernels. The accumulators leave in
// block rows i (32 weight rows of each of the two wave halves): acc[i][j][e]
// holds D row 8 (e / 4) + 4 (lane / 32) + e % 4 and token lane % 32 of block
// (i, j). A block row goes to LDS with constant register indices, as
// slab[half][token][32 rows + pad], then every thread writes runs of 4 rows
// of Y. The loop over block rows is not unrolled and the generic store path
// (bias, ragged edges, fp32 or bf16) is a plain loop, so the epilogue's code
// stays small (fully unrolled, the kernel ran to ~18,000 instructions and
// its epilogue took 13 us per 256 x 256 tile; this form takes 8, about what
// a whole chip of tiles writing 128 KB each at once needs). Interior tiles
// without bias take a fast path that issues every slab read before the
// stores.
constexpr int kSlabStride = 36;                     // floats per token row (32 + pad)

template <int BN, int BM>
__device__ __forceinline__ bool tile_interior(const GemmArgs& a, int64_t m0, int64_t n0, int tile_n) {
    if (m0 + BM > a.M) return false;
    if (a.epi == EPI_SWIGLU) return (int64_t)(tile_n + 1) * (BN / 2) <= a.i_half && out_ld(a) % 4 == 0;
    return n0 + BN <= a.N && out_ld(a) % 4 == 0 && a.bias == nullptr;
}

// 4 bf16 outputs with the non-temporal hint: a wave of tiles writes its whole
// output in one burst at the end, which nothing in the launch reads back
// (Llama-8B t = 2: o 38.9 -> 37.4 us, gate_up + SwiGLU 214.6 -> 211.5, qkv and
// down ~1% faster; Qwen-32B t = 8 unchanged; timed alternately).
__device__ __forceinline__ void store_bf16x4_nt(uint16_t* p, float a0, float a1, float a2, float a3) {
    __builtin_nontemporal_store(u32x2_t{pack_bf16x2(a0, a1), pack_bf16x2(a2, a3)}, reinterpret_cast<u32x2_t*>(p));
}

template <int BN, int BM, int THREADS, int RED = 0>
__device__ __forceinline__ void store_block_row(const GemmArgs& a, const float* slab, int i, int tid, int64_t m0,
                                                int64_t n0, int tile_n, bool interior) {
    constexpr int kWN = BN / 2;
    constexpr int kRuns = 2 * BM * 8;               // (half, token, run of 4 rows)
    static_assert(kRuns % THREADS == 0, "store loop must divide evenly");
    static_assert((kRuns / 2) % THREADS == 0, "SwiGLU store loop must divide evenly");
    constexpr int kIt = kRuns / THREADS;
    constexpr int kItS = kRuns / 2 / THREADS;       // SwiGLU: gate half paired with up half
    const int64_t M = a.M, N = a.N, ld = out_ld(a);
    if (a.epi == EPI_SWIGLU) {
        if (interior) {
            float4 g[kItS], u[kItS];
#pragma unroll
            for (int it = 0; it < kItS; ++it) {
                const int q = tid + it * THREADS;
                g[it] = *reinterpret_cast<const float4*>(slab + (q >> 3) * kSlabStride + 4 * (q & 7));
                u[it] = *reinterpret_cast<const float4*>(slab + (BM + (q >> 3)) * kSlabStride + 4 * (q & 7));
            }
#pragma unroll
            for (int it = 0; it < kItS; ++it) {
                const int q = tid + it * THREADS;
                const int64_t j = (int64_t)tile_n * kWN + i * 32 + 4 * (q & 7);
                float o[4];
                swiglu4(g[it], u[it], o);
                store_bf16x4_nt(reinterpret_cast<uint16_t*>(a.y) + (m0 + (q >> 3)) * ld + j, o[0], o[1], o[2], o[3]);
            }
        } else {
#pragma unroll 1
            for (int it = 0; it < kItS; ++it) {
                const int q = tid + it * THREADS;
                const int mt = q >> 3;
                const int run = q & 7;
                const int64_t m = m0 + mt;
                const int64_t j = (int64_t)tile_n * kWN + i * 32 + 4 * run;
                if (m < M && j < a.i_half)
                    swiglu_out4(a, m, j, *reinterpret_cast<const float4*>(slab + mt * kSlabStride + 4 * run),
                                *reinterpret_cast<const float4*>(slab + (BM + mt) * kSlabStride + 4 * run));
            }
        }
        return;
    }
    // run q: half q / (8 BM), token (q mod 8 BM) / 8, rows 4 (q mod 8) of the block row
    auto token = [&](int q) { return (q % (BM * 8)) >> 3; };
    auto slab_at = [&](int q) { return slab + ((q / (BM * 8)) * BM + token(q)) * kSlabStride + 4 * (q & 7); };
    auto col = [&](int q) { return n0 + (q / (BM * 8)) * kWN + i * 32 + 4 * (q & 7); };
    if constexpr (RED) {
        // The sum over the ranks (t <= kTiledReduceRanks, bf16 partials
        // [M, N], N % 4 == 0): the rank's partial rounded to bf16 as a partial
        // buffer holds it, the t ranks added in rank order in fp32, one
        // rounding; the same bits as the GEMM into a buffer followed by the
        // reducer. The other ranks' 4 values of every run of this block row
        // are loaded before any is used (runs past the edge read the buffers'
        // start and store nothing).
        uint2 pv[kIt][kTiledReduceRanks];
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int q = tid + it * THREADS;
            const int64_t m = m0 + token(q), n = col(q);
            const int64_t off = (m < M && n < N) ? m * N + n : 0;
#pragma unroll
            for (int r = 0; r < kTiledReduceRanks; ++r)
                if (r < a.t && r != a.rank)
                    pv[it][r] = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.peers[r]) + off);
        }
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int q = tid + it * THREADS;
            const int64_t m = m0 + token(q), n = col(q);
            const float4 v = *reinterpret_cast<const float4*>(slab_at(q));
            const float own[4] = {round_bf16(v.x), round_bf16(v.y), round_bf16(v.z), round_bf16(v.w)};
            float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < kTiledReduceRanks; ++r) {
                if (r < a.t) {
                    float qv[4];
                    if (r == a.rank) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) qv[e] = own[e];
                    } else {
                        qv[0] = bf16_to_f32(pv[it][r].x & 0xFFFFu);
                        qv[1] = bf16_to_f32(pv[it][r].x >> 16);
                        qv[2] = bf16_to_f32(pv[it][r].y & 0xFFFFu);
                        qv[3] = bf16_to_f32(pv[it][r].y >> 16);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = r == 0 ? qv[e] : o[e] + qv[e];
                }
            }
            if (m < M && n < N)
                store_bf16x4_nt(reinterpret_cast<uint16_t*>(a.y) + m * N + n, o[0], o[1], o[2], o[3]);
        }
        return;
    }
    if (interior) {
        float4 v[kIt];
#pragma unroll
        for (int it = 0; it < kIt; ++it) v[it] = *reinterpret_cast<const float4*>(slab_at(tid + it * THREADS));
        if (a.out_dtype == TP_F32) {
#pragma unroll
            for (int it = 0; it < kIt; ++it) {
                const int q = tid + it * THREADS;
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.y) + (m0 + token(q)) * ld + col(q)) = v[it];
            }
        } else {
#pragma unroll
            for (int it = 0; it < kIt; ++it) {
                const int q = tid + it * THREADS;
                store_bf16x4_nt(reinterpret_cast<uint16_t*>(a.y) + (m0 + token(q)) * ld + col(q), v[it].x, v[it].y,
                                v[it].z, v[it].w);
            }
        }
        return;
    }
#pragma unroll 1
    for (int it = 0; it < kIt; ++it) {
        const int q = tid + it * THREADS;
        const int64_t m = m0 + token(q);
        const int64_t n = col(q);
        if (m < M && n < N) {
            const float4 v = *reinterpret_cast<const float4*>(slab_at(q));
            float o[4] = {v.x, v.y, v.z, v.w};
            store_out4(a, m, n, o);
        }
    }
}

// The whole epilogue: block rows one at a time through the slab at `lds`
// (the stage ring is free by then).
template <int BN, int BM, int THREADS, int BLKN, int BLKM, int WM_ROWS, int RED = 0, typename Acc>
__device__ __forceinline__ void tile_epilogue(const GemmArgs& a, unsigned char* lds, Acc& acc, int tid, int wn,
                                              int wm, int64_t m0, int64_t n0, int tile_n) {
    float* slab = reinterpret_cast<float*>(lds);
    const int lane = tid & 63;
    const bool interior = tile_interior<BN, BM>(a, m0, n0, tile_n);
#pragma unroll 1
    for (int i = 0; i < BLKN; ++i) {
        static_for<BLKN>([&](auto I) {
            if (i == decltype(I)::value) {
                static_for<BLKM>([&](auto j) {
                    const int mt = wm * WM_ROWS + j * 32 + (lane & 31);
                    static_for<4>([&](auto g) {
                        const f32x4_t v = {acc[I][j][4 * g], acc[I][j][4 * g + 1], acc[I][j][4 * g + 2],
                                           acc[I][j][4 * g + 3]};
                        *reinterpret_cast<f32x4_t*>(slab + (wn * BM + mt) * kSlabStride + 8 * g + 4 * (lane >> 5)) = v;
                    });
                });
            }
        });
        lds_barrier();
        store_block_row<BN, BM, THREADS, RED>(a, slab, i, tid, m0, n0, tile_n, interior);
        lds_barrier();
    }
}

template <int BN, int BM>
__global__ void __launch_bounds__(kThreads, 1)
tiled_reg_kernel(GemmArgs a, int tiles_n, int tiles_m) {
    using C = TileCfg<BN, BM>;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    bf16_t* lds = reinterpret_cast<bf16_t*>(lds_raw);

    // XCD-aware tile order: workgroups id, id + 8, id + 16, ... run on one XCD;
    // give each XCD a contiguous range of tiles, token tile fastest.
    const int ntiles = tiles_n * tiles_m;
    const int per_xcd = (ntiles + kXcds - 1) / kXcds;
    const int t = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
    if (t >= ntiles) return;
    int tile_n, tile_m;
    group_tile(t, tiles_n, tiles_m, tile_n, tile_m);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave >> 1;
    const int wm = wave & 1;
    const int64_t M = a.M, K = a.K;
    const int64_t n0 = (int64_t)tile_n * BN;
    const int64_t m0 = (int64_t)tile_m * BM;
    const bf16_t* __restrict__ X = reinterpret_cast<const bf16_t*>(a.x);
    const bf16_t* __restrict__ W = reinterpret_cast<const bf16_t*>(a.w);

    // Global -> VGPR staging of one k-tile. Thread tid loads chunk tid % 8 of
    // rows tid / 8 + 32 j: 8 consecutive lanes cover one 128-byte row segment.
    const int crow = tid >> 3;
    const int cchunk = tid & 7;
    u32x4_t wr[C::kWChunks], xr[C::kXChunks];     // native vectors: kept in VGPRs
#define TP_TILED_LOAD(K0)                                                                   \
    do {                                                                                    \
        const int64_t k_ = (K0) + cchunk * 8;                                               \
        const bool kin_ = k_ < K;                                                           \
        _Pragma("unroll") for (int j = 0; j < C::kWChunks; ++j) {                           \
            const int64_t r_ = tile_w_row<BN>(a, n0 + crow + 32 * j);                        \
            wr[j] = u32x4_t{0u, 0u, 0u, 0u};                                                \
            if (kin_ && r_ >= 0) wr[j] = *reinterpret_cast<const u32x4_t*>(W + r_ * K + k_); \
        }                                                                                   \
        _Pragma("unroll") for (int j = 0; j < C::kXChunks; ++j) {                           \
            const int64_t r_ = m0 + crow + 32 * j;                                          \
            xr[j] = u32x4_t{0u, 0u, 0u, 0u};                                                \
            if (kin_ && r_ < M) xr[j] = *reinterpret_cast<const u32x4_t*>(X + r_ * K + k_); \
        }                                                                                   \
    } while (0)
#define TP_TILED_STORE(STAGE)                                                               \
    do {                                                                                    \
        bf16_t* ws_ = lds + (STAGE) * C::kStageElems;                                       \
        bf16_t* xs_ = ws_ + BN * kBK;                                                       \
        _Pragma("unroll") for (int j = 0; j < C::kWChunks; ++j)                             \
            *reinterpret_cast<u32x4_t*>(ws_ + swz(crow + 32 * j, cchunk)) = wr[j];          \
        _Pragma("unroll") for (int j = 0; j < C::kXChunks; ++j)                             \
            *reinterpret_cast<u32x4_t*>(xs_ + swz(crow + 32 * j, cchunk)) = xr[j];          \
    } while (0)

    f32x16_t acc[C::kBlkN][C::kBlkM];
    static_for<C::kBlkN>([&](auto i) {
        static_for<C::kBlkM>([&](auto j) { acc[i][j] = f32x16_t{}; });
    });

    const int ktiles = (int)((K + kBK - 1) / kBK);
    TP_TILED_LOAD(0);
    TP_TILED_STORE(0);
    __syncthreads();
    if (ktiles > 1) TP_TILED_LOAD(kBK);

    // Operand reads: lane reads row (lane % 32) of a 32-row block, logical
    // chunk 2 s + lane / 32 for k16 step s. Fragments are double buffered:
    // the reads of step s + 1 are issued before the MFMAs of step s, so LDS
    // latency hides under 16 (at 256 x 256) back-to-back MFMAs.
    const int orow = lane & 31;
    const int ohalf = lane >> 5;
    bf16x8_t fa[2][C::kBlkN], fb[2][C::kBlkM];
    auto read_frags = [&](auto buf, const bf16_t* ws, const bf16_t* xs, int s) {
        const int c = 2 * s + ohalf;
        static_for<C::kBlkN>([&](auto i) {
            fa[buf][i] = __builtin_bit_cast(bf16x8_t,
                *reinterpret_cast<const u32x4_t*>(ws + swz(wn * C::kWN + i * 32 + orow, c)));
        });
        static_for<C::kBlkM>([&](auto j) {
            fb[buf][j] = __builtin_bit_cast(bf16x8_t,
                *reinterpret_cast<const u32x4_t*>(xs + swz(wm * C::kWM + j * 32 + orow, c)));
        });
    };
    read_frags(std::integral_constant<int, 0>{}, lds, lds + BN * kBK, 0);
    for (int kt = 0; kt < ktiles; ++kt) {
        const bf16_t* ws = lds + (kt & 1) * C::kStageElems;
        const bf16_t* xs = ws + BN * kBK;
        static_for<kBK / 16>([&](auto s) {
            constexpr int cur = s & 1;
            if constexpr (s + 1 < kBK / 16) read_frags(std::integral_constant<int, cur ^ 1>{}, ws, xs, s + 1);
            __builtin_amdgcn_sched_barrier(0);
            static_for<C::kBlkN>([&](auto i) {
                static_for<C::kBlkM>([&](auto j) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
                });
            });
            __builtin_amdgcn_sched_barrier(0);
        });
        if (kt + 1 < ktiles) TP_TILED_STORE((kt + 1) & 1);
        __syncthreads();
        if (kt + 2 < ktiles) TP_TILED_LOAD((int64_t)(kt + 2) * kBK);
        if (kt + 1 < ktiles) {
            const bf16_t* wn_ = lds + ((kt + 1) & 1) * C::kStageElems;
            read_frags(std::integral_constant<int, 0>{}, wn_, wn_ + BN * kBK, 0);
        }
    }

    tile_epilogue<BN, BM, kThreads, C::kBlkN, C::kBlkM, C::kWM>(a, lds_raw, acc, tid, wn, wm, m0, n0, tile_n);
}

#undef TP_TILED_LOAD
#undef TP_TILED_STORE

// ---------------------------------------------------------------------------
// Direct-to-LDS variant (K % 32 == 0): k-tiles of 32 land in LDS through
// global_load_lds_dwordx4 (no VGPR staging) in a ring of NS stages issued
// NS - 1 k-tiles ahead, so global latency hides behind several k-tiles of
// MFMAs. Waits are explicit: s_waitcnt vmcnt(n) for this wave's own DMA, then
// a barrier fenced for LDS only (not __syncthreads, whose release of all
// memory would wait for every outstanding DMA). Each iteration reads the step-1 fragments, runs the
// step-0 MFMAs, crosses the barrier for the next stage, issues the DMA three
// stages ahead into the slot freed by the previous iteration, reads the next
// stage's step-0 fragments and runs the step-1 MFMAs; the last k-tile runs
// after the loop (K >= 32: the launcher only sees validated shapes).
// LDS stage: W tile [BN][32] then X tile [BM][32], 64-byte rows, 16-byte
// chunks XOR-swizzled by (row / 4) mod 4; a lane's DMA destination is fixed
// (wave base + 16 * lane), so the swizzle is realized by choosing which
// global chunk each lane loads.

template <int BN, int BM, int NS, int WGM>
struct DmaCfg {
    static constexpr int kBK = 32;
    static constexpr int kWaves = 2 * WGM;                // 2 along weight rows x WGM along tokens
    static constexpr int kThreadsWG = 64 * kWaves;
    static constexpr int kWN = BN / 2, kWM = BM / WGM;
    static constexpr int kBlkN = kWN / 32, kBlkM = kWM / 32;
    static constexpr int kStageBytes = (BN + BM) * 64;
    static constexpr int kInstrW = BN / 16, kInstrX = BM / 16;
    static constexpr int kInstrPerWave = (kInstrW + kInstrX) / kWaves;
    static constexpr int kSlabBytes = 2 * BM * 36 * 4;
    static constexpr int kLdsBytes = NS * kStageBytes > kSlabBytes ? NS * kStageBytes : kSlabBytes;
    static_assert((kInstrW + kInstrX) % kWaves == 0, "DMA instructions must split evenly over the waves");
    static_assert(kBlkM >= 1, "at least one 32-token block per wave");
};

__device__ __forceinline__ int swz64(int row, int c) { return row * 64 + ((c ^ ((row >> 2) & 3)) << 4); }

// Barrier for the kernels that stream k-tiles into LDS with
// global_load_lds: this wave's LDS reads are complete (lgkmcnt 0) and every
// wave has arrived; which stages have landed is the caller's explicit
// vmcnt wait. lds_barrier's release fence covers LDS writes, and LDS DMA
// counts on vmcnt, so the compiler puts a vmcnt(0) in front of it: a ring
// of three or more stages would then keep no stage beyond the next one in
// flight across a barrier. The memory clobber keeps the compiler from
// moving LDS accesses across the barrier.
__device__ __forceinline__ void dma_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int BN, int BM, int NS, int WGM>
__global__ void __launch_bounds__(128 * WGM, 1)
tiled_dma_kernel(GemmArgs a, int tiles_n, int tiles_m) {
    using C = DmaCfg<BN, BM, NS, WGM>;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    unsigned char* lds8 = lds_raw;

    const int ntiles = tiles_n * tiles_m;
    const int per_xcd = (ntiles + kXcds - 1) / kXcds;
    const int t = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
    if (t >= ntiles) return;
    int tile_n, tile_m;
    group_tile(t, tiles_n, tiles_m, tile_n, tile_m);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave / WGM;
    const int wm = wave % WGM;
    const int64_t M = a.M, K = a.K;
    const int64_t n0 = (int64_t)tile_n * BN;
    const int64_t m0 = (int64_t)tile_m * BM;
    const bf16_t* __restrict__ X = reinterpret_cast<const bf16_t*>(a.x);
    const bf16_t* __restrict__ W = reinterpret_cast<const bf16_t*>(a.w);
    const int ktiles = (int)(K / C::kBK);

    // Per-lane DMA source rows (clamped into the matrix: rows past the end
    // only feed outputs that are never stored) and swizzled chunks, as byte
    // offsets into the weight's or X's buffer resource.
    const __amdgpu_buffer_rsrc_t rs_w = buffer_source(W, w_rows_read(a) * K * 2);
    const __amdgpu_buffer_rsrc_t rs_x = buffer_source(X, M * K * 2);
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // uniform: picks a resource
    uint32_t voff[C::kInstrPerWave];
    bool from_w[C::kInstrPerWave];
    int dst_off[C::kInstrPerWave];
    static_for<C::kInstrPerWave>([&](auto q) {
        const int instr = wave_s + C::kWaves * q;
        const bool is_w = instr < C::kInstrW;
        const int rbase = (is_w ? instr : instr - C::kInstrW) * 16;
        const int r = rbase + (lane >> 2);
        const int c = (lane & 3) ^ ((r >> 2) & 3);
        int64_t g;
        if (is_w) {
            g = tile_w_row<BN>(a, n0 + r);
            if (g < 0) g = 0;
        } else {
            g = m0 + r;
            if (g > M - 1) g = M - 1;
        }
        voff[q] = (uint32_t)((g * K + 8 * c) * 2);
        from_w[q] = is_w;
        dst_off[q] = (is_w ? 0 : BN * 64) + rbase * 64;
    });
    auto issue = [&](int kt) {
        unsigned char* base = lds8 + (kt % NS) * C::kStageBytes;
        const uint32_t k_bytes = (uint32_t)kt * (C::kBK * 2);
        static_for<C::kInstrPerWave>([&](auto q) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(from_w[q] ? rs_w : rs_x,
                                                     (__attribute__((address_space(3))) void*)(base + dst_off[q]), 16,
                                                     voff[q], k_bytes, 0, 0);
        });
    };

    f32x16_t acc[C::kBlkN][C::kBlkM];
    static_for<C::kBlkN>([&](auto i) {
        static_for<C::kBlkM>([&](auto j) { acc[i][j] = f32x16_t{}; });
    });

    const int orow = lane & 31;
    const int ohalf = lane >> 5;
    bf16x8_t fa[2][C::kBlkN], fb[2][C::kBlkM];
    auto read_frags = [&](auto buf, int kt, int s) {
        const unsigned char* ws = lds8 + (kt % NS) * C::kStageBytes;
        const unsigned char* xs = ws + BN * 64;
        const int c = 2 * s + ohalf;
        static_for<C::kBlkN>([&](auto i) {
            fa[buf][i] = __builtin_bit_cast(bf16x8_t,
                *reinterpret_cast<const u32x4_t*>(ws + swz64(wn * C::kWN + i * 32 + orow, c)));
        });
        static_for<C::kBlkM>([&](auto j) {
            fb[buf][j] = __builtin_bit_cast(bf16x8_t,
                *reinterpret_cast<const u32x4_t*>(xs + swz64(wm * C::kWM + j * 32 + orow, c)));
        });
    };
    auto mfmas = [&](auto buf) {
        static_for<C::kBlkN>([&](auto i) {
            static_for<C::kBlkM>([&](auto j) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
            });
        });
    };
    // wait until this wave's DMA of the stage `ahead` stages before the most
    // recently issued one has landed: `pending` stages may stay in flight
    auto wait_stage = [&](int pending) {
        if (pending <= 0) wait_vmcnt<0>();
        else if (pending == 1) wait_vmcnt<C::kInstrPerWave>();
        else wait_vmcnt<2 * C::kInstrPerWave>();
    };
    constexpr int kF0 = 0, kF1 = 1;

    // prologue: stages 0 .. NS-2 in flight, wait for stage 0
    const int pro = ktiles < NS - 1 ? ktiles : NS - 1;
    for (int kt = 0; kt < pro; ++kt) issue(kt);
    wait_stage(pro - 1);
    dma_barrier();
    read_frags(std::integral_constant<int, kF0>{}, 0, 0);

    // The last k-tile is peeled off so that the loop body has no branch
    // around the next stage's fragment reads: at such a join the compiler
    // waits for every LDS read in flight, so the step-1 MFMAs would wait for
    // the next stage's reads as well (3-5 % slower). (No scheduling barriers:
    // the compiler's interleaving of reads and MFMAs measured as fast as a
    // pinned one.)
    for (int kt = 0; kt + 1 < ktiles; ++kt) {
        read_frags(std::integral_constant<int, kF1>{}, kt, 1);
        mfmas(std::integral_constant<int, kF0>{});
        // stages issued after kt + 1: up to kt + NS - 2
        const int last = kt + NS - 2 < ktiles - 1 ? kt + NS - 2 : ktiles - 1;
        wait_stage(last - (kt + 1));
        dma_barrier();   // every wave's part of stage kt + 1 has landed; stage kt - 1 is free
        if (kt + NS - 1 < ktiles) issue(kt + NS - 1);
        read_frags(std::integral_constant<int, kF0>{}, kt + 1, 0);
        mfmas(std::integral_constant<int, kF1>{});
    }
    read_frags(std::integral_constant<int, kF1>{}, ktiles - 1, 1);
    mfmas(std::integral_constant<int, kF0>{});
    mfmas(std::integral_constant<int, kF1>{});
    wait_vmcnt<0>();
    __syncthreads();

    tile_epilogue<BN, BM, C::kThreadsWG, C::kBlkN, C::kBlkM, C::kWM>(a, lds8, acc, tid, wn, wm, m0, n0, tile_n);
}

// ---------------------------------------------------------------------------
// 64-wide k-tiles (K % 64 == 0): every DMA row segment is a whole 128-byte
// line (8 lanes x 16 B), where 32-wide k-tiles fetch each line in two halves
// a k-tile apart; and there is one barrier per 64 of K. On the prefill shard
// shapes it runs 3-10 % faster than the 32-wide kernel with the same tile. LDS stage: W tile [BN][64] then X tile [BM][64], 128-byte rows,
// 16-byte chunks XOR-swizzled by (row / 2) mod 8. A 16-byte LDS read is
// served 16 lanes at a time across 64 four-byte banks (256 bytes): the 16
// consecutive rows that 16 lanes read are 8 pairs of rows 128 bytes apart,
// and the swizzle gives the 8 rows of each parity 8 different 16-byte bank
// groups, so the 16 reads take all 64 banks once. (A swizzle by row mod 8
// sends rows r and r + 8 to the same banks: measured 0.96 bank-conflict
// cycles per LDS access on the 256 x 256 tile.) After the barrier of k-tile kt every
// wave has finished reading stage kt, so the DMA of k-tile kt + NS goes into
// its slot: NS stages are in flight from the prologue on.
template <int BN, int BM, int NS, int WGM>
struct Dma64Cfg {
    static constexpr int kBK = 64;
    static constexpr int kWaves = 2 * WGM;
    static constexpr int kThreadsWG = 64 * kWaves;
    static constexpr int kWN = BN / 2, kWM = BM / WGM;
    static constexpr int kBlkN = kWN / 32, kBlkM = kWM / 32;
    static constexpr int kStageBytes = (BN + BM) * 128;
    static constexpr int kInstrW = BN / 8, kInstrX = BM / 8;
    static constexpr int kInstrPerWave = (kInstrW + kInstrX) / kWaves;
    static constexpr int kSlabBytes = 2 * BM * 36 * 4;
    static constexpr int kLdsBytes = NS * kStageBytes > kSlabBytes ? NS * kStageBytes : kSlabBytes;
    static_assert((kInstrW + kInstrX) % kWaves == 0, "DMA instructions must split evenly over the waves");
    static_assert(kBlkM >= 1, "at least one 32-token block per wave");
    static_assert(NS >= 2 && NS * kInstrPerWave <= 63, "stages in flight must fit the load counter");
};

__device__ __forceinline__ int swz128(int row, int c) { return row * 128 + ((c ^ ((row >> 1) & 7)) << 4); }

template <int BN, int BM, int NS, int WGM, int RED = 0>
__global__ void __launch_bounds__(128 * WGM, (Dma64Cfg<BN, BM, NS, WGM>::kLdsBytes <= 80 * 1024 ? 2 : 1))
tiled_dma64_kernel(GemmArgs a, int tiles_n, int tiles_m) {
    using C = Dma64Cfg<BN, BM, NS, WGM>;
    extern __shared__ __align__(16) unsigned char lds_raw[];
    unsigned char* lds8 = lds_raw;

    const int ntiles = tiles_n * tiles_m;
    const int per_xcd = (ntiles + kXcds - 1) / kXcds;
    const int t = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
    if (t >= ntiles) return;
    int tile_n, tile_m;
    group_tile(t, tiles_n, tiles_m, tile_n, tile_m);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave / WGM;
    const int wm = wave % WGM;
    const int64_t M = a.M, K = a.K;
    const int64_t n0 = (int64_t)tile_n * BN;
    const int64_t m0 = (int64_t)tile_m * BM;
    const bf16_t* __restrict__ X = reinterpret_cast<const bf16_t*>(a.x);
    const bf16_t* __restrict__ W = reinterpret_cast<const bf16_t*>(a.w);
    const int ktiles = (int)(K / C::kBK);

    // Per-lane DMA source rows (clamped: rows past the end only feed outputs
    // that are never stored); lane l of an instruction fills LDS chunk l % 8
    // of row l / 8 with the global chunk that the swizzle puts there, read
    // at a byte offset into the weight's or X's buffer resource.
    const __amdgpu_buffer_rsrc_t rs_w = buffer_source(W, w_rows_read(a) * K * 2);
    const __amdgpu_buffer_rsrc_t rs_x = buffer_source(X, M * K * 2);
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // uniform: picks a resource
    uint32_t voff[C::kInstrPerWave];
    bool from_w[C::kInstrPerWave];
    int dst_off[C::kInstrPerWave];
    static_for<C::kInstrPerWave>([&](auto q) {
        const int instr = wave_s + C::kWaves * q;
        const bool is_w = instr < C::kInstrW;
        const int rbase = (is_w ? instr : instr - C::kInstrW) * 8;
        const int r = rbase + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        int64_t g;
        if (is_w) {
            g = tile_w_row<BN>(a, n0 + r);
            if (g < 0) g = 0;
        } else {
            g = m0 + r;
            if (g > M - 1) g = M - 1;
        }
        voff[q] = (uint32_t)((g * K + 8 * c) * 2);
        from_w[q] = is_w;
        dst_off[q] = (is_w ? 0 : BN * 128) + rbase * 128;
    });
    auto issue = [&](int kt) {
        unsigned char* base = lds8 + (kt % NS) * C::kStageBytes;
        const uint32_t k_bytes = (uint32_t)kt * (C::kBK * 2);
        static_for<C::kInstrPerWave>([&](auto q) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(from_w[q] ? rs_w : rs_x,
                                                     (__attribute__((address_space(3))) void*)(base + dst_off[q]), 16,
                                                     voff[q], k_bytes, 0, 0);
        });
    };

    f32x16_t acc[C::kBlkN][C::kBlkM];
    static_for<C::kBlkN>([&](auto i) {
        static_for<C::kBlkM>([&](auto j) { acc[i][j] = f32x16_t{}; });
    });

    const int orow = lane & 31;
    const int ohalf = lane >> 5;
    bf16x8_t fa[2][C::kBlkN], fb[2][C::kBlkM];
    // Fragments are read in the order the MFMAs below consume them (A0, every
    // B, then A1, A2, ...): LDS reads return in order, so the first MFMAs of
    // a step wait only for the first reads of the previous step.
    auto read_frags = [&](auto buf, int kt, int s) {
        const unsigned char* ws = lds8 + (kt % NS) * C::kStageBytes;
        const unsigned char* xs = ws + BN * 128;
        const int c = 2 * s + ohalf;
        auto read_a = [&](auto i) {
            fa[buf][i] = __builtin_bit_cast(bf16x8_t,
                *reinterpret_cast<const u32x4_t*>(ws + swz128(wn * C::kWN + i * 32 + orow, c)));
        };
        read_a(std::integral_constant<int, 0>{});
        static_for<C::kBlkM>([&](auto j) {
            fb[buf][j] = __builtin_bit_cast(bf16x8_t,
                *reinterpret_cast<const u32x4_t*>(xs + swz128(wm * C::kWM + j * 32 + orow, c)));
        });
        static_for<C::kBlkN - 1>([&](auto i) { read_a(std::integral_constant<int, decltype(i)::value + 1>{}); });
    };
    auto mfmas = [&](auto buf) {
        static_for<C::kBlkN>([&](auto i) {
            static_for<C::kBlkM>([&](auto j) {
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
            });
        });
    };
    // wait until at most `pending` of this wave's most recent stages are in flight
    auto wait_stage = [&](int pending) {
        if (pending <= 0) wait_vmcnt<0>();
        static_for<NS - 1>([&](auto p) {
            if (pending == decltype(p)::value + 1) wait_vmcnt<(decltype(p)::value + 1) * C::kInstrPerWave>();
        });
    };
    // Order of the reads and MFMAs that follow one another in the loop:
    // MFMA, read, MFMA, read, ..., then the rest. An MFMA goes first, so the
    // group's first MFMA waits only for the previous group's reads; left to
    // itself the compiler clusters reads behind waits here (9 % slower).
    auto pin_group = [&]() {
        constexpr int R = C::kBlkN + C::kBlkM, F = C::kBlkN * C::kBlkM;
        constexpr int P = R < F ? R : F;
        static_for<P>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
        });
        if constexpr (R > P) __builtin_amdgcn_sched_group_barrier(0x100, R - P, 0);
        if constexpr (F > P) __builtin_amdgcn_sched_group_barrier(0x008, F - P, 0);
    };
    constexpr int kF0 = 0, kF1 = 1;
    using F0 = std::integral_constant<int, kF0>;
    using F1 = std::integral_constant<int, kF1>;

    const int pro = ktiles < NS ? ktiles : NS;
    for (int kt = 0; kt < pro; ++kt) issue(kt);
    wait_stage(pro - 1);
    dma_barrier();
    read_frags(F0{}, 0, 0);

    // The last k-tile runs after the loop, so the loop body has no branch
    // around fragment reads (see the 32-wide kernel).
    for (int kt = 0; kt + 1 < ktiles; ++kt) {
        read_frags(F1{}, kt, 1);
        mfmas(F0{});
        pin_group();
        read_frags(F0{}, kt, 2);
        mfmas(F1{});
        pin_group();
        read_frags(F1{}, kt, 3);
        mfmas(F0{});
        pin_group();
        // stages issued after kt + 1: up to kt + NS - 1
        const int last = kt + NS - 1 < ktiles - 1 ? kt + NS - 1 : ktiles - 1;
        wait_stage(last - (kt + 1));
        dma_barrier();   // stage kt + 1 has landed; every wave is done with stage kt
        if (kt + NS < ktiles) issue(kt + NS);
        read_frags(F0{}, kt + 1, 0);
        mfmas(F1{});
        pin_group();
    }
    read_frags(F1{}, ktiles - 1, 1);
    mfmas(F0{});
    read_frags(F0{}, ktiles - 1, 2);
    mfmas(F1{});
    read_frags(F1{}, ktiles - 1, 3);
    mfmas(F0{});
    mfmas(F1{});
    wait_vmcnt<0>();
    __syncthreads();

    tile_epilogue<BN, BM, C::kThreadsWG, C::kBlkN, C::kBlkM, C::kWM, RED>(a, lds8, acc, tid, wn, wm, m0, n0, tile_n);
}

typedef void (*TiledFn)(GemmArgs, int, int);
struct TiledEntry {
    int bn, bm;
    int kmul;          // K must be a multiple of this
    TiledFn fn;
    int lds;
    int threads;
    bool buffer;       // sources read through buffer resources (extents < 4 GiB)
    TiledFn fn_red;    // the same tile with the sum over ranks as its epilogue, or null
};

#define TP_DMA(BN, BM, NS, WGM) \
    {BN, BM, 32, tiled_dma_kernel<BN, BM, NS, WGM>, DmaCfg<BN, BM, NS, WGM>::kLdsBytes, DmaCfg<BN, BM, NS, WGM>::kThreadsWG, \
     true, nullptr}
#define TP_DMA64(BN, BM, NS, WGM) \
    {BN, BM, 64, tiled_dma64_kernel<BN, BM, NS, WGM>, Dma64Cfg<BN, BM, NS, WGM>::kLdsBytes, \
     Dma64Cfg<BN, BM, NS, WGM>::kThreadsWG, true, tiled_dma64_kernel<BN, BM, NS, WGM, 1>}
const TiledEntry kTiled[] = {
    TP_DMA(256, 256, 4, 2),
    TP_DMA(256, 128, 4, 2),
    TP_DMA(128, 128, 4, 2),
    {128, 128, 8, tiled_reg_kernel<128, 128>, TileCfg<128, 128>::kLdsBytes, kThreads, false, nullptr},
    TP_DMA(256, 256, 4, 4),
    TP_DMA(256, 128, 4, 4),
    TP_DMA(128, 128, 4, 4),
    TP_DMA(192, 128, 4, 2),
    TP_DMA64(256, 256, 2, 4),
    TP_DMA64(256, 128, 3, 4),
    TP_DMA64(128, 128, 3, 4),
    TP_DMA64(192, 128, 3, 4),
    TP_DMA64(64, 64, 4, 2),
    TP_DMA64(128, 64, 4, 2),
    TP_DMA64(64, 64, 6, 1),
    TP_DMA64(128, 128, 2, 2),
    TP_DMA64(192, 256, 2, 4),
    TP_DMA64(128, 256, 3, 4),
};
#undef TP_DMA
#undef TP_DMA64
constexpr int kNumTiled = sizeof(kTiled) / sizeof(kTiled[0]);
constexpr int kRegVariant = 3;   // register-staged: plain global loads, any K % 8
constexpr int kMaxDevices = 16;
// Whether each kernel's dynamic-LDS limit is set, per device; setting it is
// idempotent, so a race between host threads only repeats the call.
std::atomic<bool> g_tiled_attr[kMaxDevices][2][kNumTiled] = {};   // [device][reduce epilogue][variant]

}  // namespace

int tiled_variant_count() { return kNumTiled; }

// Measured on MI355X at 64 tokens (weights rotated past the last-level
// cache): with K >= 2048 and at least 48 tiles of 64 weight rows, 64 x 64
// tiles streaming K through a 4-stage ring beat the decode kernel, whose
// K split then re-stages all 64 tokens' activations per 16 weight rows and
// sums fp32 partials across workgroups (LM head 8016 x 4096: 27.1 against
// 40.2 us; 3584 x 4096: 24.8 against 27.0 us). With fewer rows or shorter K
// the decode kernel wins (1792 x 4096: 17.3 against 24.5 us; 4096 x 896:
// 7.2 against 9.5 us). At 17-32 tokens only weights of LM-head size do
// (16032 x 4096 at 24 and 32 tokens: 30.7 and 30.9 against 49.5 and 54.6 us;
// 3584 x 4096: 20.8 and 21.0 against 16.7 and 17.8), and at 16 tokens none
// (16032 x 4096: 30.6 against 27.6 us).
bool tiled_wins_at_decode(const GemmArgs& a) {
    if (a.M <= 16 || a.K < 2048 || a.K % 64 != 0 || a.norm != 0) return false;
    if (a.epi != EPI_STORE && a.epi != EPI_SWIGLU) return false;
    const int64_t rows = a.epi == EPI_SWIGLU ? 2 * a.i_half : a.N;
    return (rows + 63) / 64 >= (a.M <= 32 ? 128 : 48);
}

namespace {

// Launch tiled kernel v over tokens [m0, M) of `a` (a contiguous block of
// X's and Y's rows).
hipError_t launch_variant(const GemmArgs& a, int v, int64_t m0, hipStream_t s) {
    const TiledEntry& e = kTiled[v];
    const int red = epi_is_reduce(a.epi) ? 1 : 0;
    const TiledFn fn = red ? e.fn_red : e.fn;
    if (fn == nullptr) return hipErrorInvalidValue;     // no reduce epilogue on this shape (the host avoids it)
    int dev = 0;
    hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) return he;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (!g_tiled_attr[dev][red][v].load(std::memory_order_acquire)) {
        he = hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, e.lds);
        if (he != hipSuccess) return he;
        g_tiled_attr[dev][red][v].store(true, std::memory_order_release);
    }
    GemmArgs b = a;
    const bool swiglu = a.epi == EPI_SWIGLU;
    if (swiglu) b.N = (int64_t)e.bn * ((a.i_half + e.bn / 2 - 1) / (e.bn / 2));
    if (m0 > 0) {
        const int64_t y_cols = a.ldy != 0 ? a.ldy : (swiglu ? a.i_half : a.N);
        const int64_t y_elem = a.out_dtype == TP_F32 ? 4 : 2;
        b.x = static_cast<const unsigned char*>(a.x) + m0 * a.K * 2;
        b.y = static_cast<unsigned char*>(a.y) + m0 * y_cols * y_elem;
        b.M = a.M - m0;
    }
    // Kernels that read through buffer resources address 32-bit byte
    // offsets: a weight or X of 4 GiB or more takes the register-staged
    // kernel (same MFMA, same K order, so the same bits).
    if (e.buffer && (w_rows_read(b) * b.K * 2 > kMaxBufferBytes || b.M * b.K * 2 > kMaxBufferBytes))
        return red ? hipErrorInvalidValue : launch_variant(a, kRegVariant, m0, s);
    const int tn = (int)((b.N + e.bn - 1) / e.bn);
    const int tm = (int)((b.M + e.bm - 1) / e.bm);
    const int ntiles = tn * tm;
    const int grid = ((ntiles + kXcds - 1) / kXcds) * kXcds;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(e.threads), e.lds, s, b, tn, tm);
    return hipGetLastError();
}

// Sustained bf16 rate of a whole chip's worth of each 64-wide-k-tile shape
// (TFLOP/s, MI355X counters at the prefill shard shapes: 2 x 256 x 256 and
// 256 x 128 on 8 waves, 192 x 128, 128 x 128), for the split below.
double tile_rate(int v) {
    switch (v) {
    case 8: return 990.0;
    case 9: return 830.0;
    case 11: return 745.0;
    case 10: return 600.0;
    default: return 0.0;
    }
}

// Estimated microseconds of variant v over tokens [m0, M): whole waves of
// tiles over the 256 CUs (a partly filled wave costs a full one).
double region_us(const GemmArgs& a, int v, int64_t m0) {
    const TiledEntry& e = kTiled[v];
    const int64_t rows = a.epi == EPI_SWIGLU ? (int64_t)e.bn * ((a.i_half + e.bn / 2 - 1) / (e.bn / 2)) : a.N;
    const int64_t tiles = ((rows + e.bn - 1) / e.bn) * ((a.M - m0 + e.bm - 1) / e.bm);
    const int64_t waves = (tiles + kCus - 1) / kCus;
    const double tile_flop = 2.0 * e.bn * e.bm * (double)a.K;
    return (double)waves * tile_flop / (tile_rate(v) * 1e12 / kCus) * 1e6;
}

}  // namespace

// EPI_SWIGLU: a.N is 2 * i_half on entry (used to pick the tile shape); the
// kernel's row space is then whole tiles of paired gate and up rows.
hipError_t launch_tiled(const GemmArgs& a, hipStream_t s, int variant) {
    // Kernel choice, from MI355X measurements at the Llama-8B and Qwen-32B
    // prefill shard shapes, all on 8 waves: 256 x 256 tiles when they give at
    // least 192 tiles; else 256 x 128 tiles when those do; else 128 x 128
    // tiles. K <= 1024 (where a tile's fixed prologue and epilogue weigh
    // most) takes 128 x 128 tiles: two 4-wave workgroups per CU with 64-wide
    // k-tiles when K % 64 == 0 (Qwen-32B t = 8 o_proj, K = 640: 42.3 -> 39.7
    // and 44.3 -> 43.3 us in two sweeps), else 32-wide k-tiles; otherwise 64-wide
    // k-tiles when K % 64 == 0, 32-wide ones when K % 32 == 0, and the
    // register-staged kernel for any other K. With 64-wide k-tiles, 256 x 128
    // tiles that leave CUs idle give way to 192 x 128 tiles when those fill
    // at most one pass of the chip (Llama-8B t = 2 qkv: 192 tiles of
    // 256 x 128 take 70 us, 256 of 192 x 128 take 62 us); to 128 x 256 tiles
    // (weight rows x tokens, three stages) when those fill 90-100% of one
    // pass (Llama-8B t = 2 down 118.5 -> 109.4 us, o 39.5 -> 37.6, against
    // the 128 x 128 tiles below; worse wherever they leave a pass part-full);
    // and otherwise to 128 x 128 tiles on 4 waves with two 64-wide stages,
    // small enough (64 KB of LDS, 134 VGPRs) for two workgroups per CU, whose
    // barriers and loads then interleave (Llama-8B t = 2 down 132.8 -> 124.3
    // us, o 44.6 -> 42.7, timed alternately with the 8-wave 256 x 128 tiles).
    auto tiles = [&](int bn, int bm) { return ((a.N + bn - 1) / bn) * ((a.M + bm - 1) / bm); };
    const int shape = tiles(256, 256) >= 192 ? 0 : tiles(256, 128) >= 192 ? 1 : 2;
    int best;
    if (a.M <= 64 && a.K % 64 == 0) best = 12;       // 64 x 64 tiles for decode sizes
    else if (a.K % 32 != 0) best = 3;
    else if (a.K <= 1024) best = a.K % 64 == 0 ? 15 : 6;
    else if (a.K % 64 != 0) best = 4 + shape;
    else if (shape == 1 && tiles(256, 128) < kCus && tiles(192, 128) <= kCus) best = 11;
    else if (shape == 1 && tiles(128, 256) <= kCus && tiles(128, 256) * 10 >= kCus * 9) best = 17;
    else if (shape == 1) best = 15;
    else best = 8 + shape;
    if (variant >= 0 && variant < kNumTiled && a.K % kTiled[variant].kmul == 0) return launch_variant(a, variant, 0, s);
    // the sum over ranks indexes the other ranks' [M, N] buffers with the
    // launch's own M and N: one launch over the whole product
    if (epi_is_reduce(a.epi)) return launch_variant(a, best, 0, s);
    // Weight-row split: when 256 x 256 tiles make between one and two waves,
    // one whole wave of them takes the first weight rows and a second launch
    // of 192 x 256 tiles (0.75 of the work per tile, one exact wave where the
    // shapes allow) takes the rest, instead of a second wave of 256 x 256
    // tiles that leaves CUs idle (Llama-8B t = 2 gate_up, 2048 x 14336 x
    // 4096: 256 + 256 tiles, 215 against 224 us, timed alternately; Qwen-32B
    // t = 8 gate_up, 256 + 240 tiles: no change). Each output keeps its
    // tile's K order, so the split changes no bit.
    if (best == 8) {
        const int64_t t8 = tiles(256, 256);
        const int64_t tm = (a.M + 255) / 256;
        const int64_t head_n = kCus / tm;
        const int64_t head_rows = head_n * 256;
        const int64_t tail_rows = a.N - head_rows;
        const int64_t tail_tiles = tail_rows > 0 ? ((tail_rows + 191) / 192) * tm : 0;
        if (t8 > kCus && t8 < 2 * kCus && head_n >= 1 && head_n * tm * 10 >= kCus * 9 && tail_rows > 0 &&
            tail_tiles <= kCus && tail_tiles * 10 >= kCus * 6) {
            const bool sw = a.epi == EPI_SWIGLU;
            const int64_t y_elem = a.out_dtype == TP_F32 ? 4 : 2;
            GemmArgs h = a, t = a;
            if (sw) {
                const int64_t g0 = head_rows / 2;      // gate rows in the head
                h.i_half = g0;
                h.N = 2 * g0;
                t.i_half = a.i_half - g0;
                t.N = 2 * t.i_half;
                t.w = static_cast<const unsigned char*>(a.w) + g0 * a.K * 2;
                t.y = static_cast<unsigned char*>(a.y) + g0 * 2;
                h.up_off = t.up_off = a.i_half;
                h.ldy = t.ldy = a.i_half;
            } else {
                h.N = head_rows;
                t.N = a.N - head_rows;
                t.w = static_cast<const unsigned char*>(a.w) + head_rows * a.K * 2;
                t.y = static_cast<unsigned char*>(a.y) + head_rows * y_elem;
                if (a.bias != nullptr) t.bias = static_cast<const unsigned char*>(a.bias) + head_rows * 2;
                h.ldy = t.ldy = a.N;
            }
            const hipError_t he = launch_variant(h, 8, 0, s);
            if (he != hipSuccess) return he;
            return launch_variant(t, 16, 0, s);
        }
    }
    // Wave quantisation: when the last wave of 256 x 256 tiles would leave
    // most CUs idle (Qwen-32B t = 8 down: 320 tiles, 1.25 waves), the
    // first token rows keep those tiles and the rest run as a second launch
    // of smaller tiles, if the estimate (whole waves at each shape's measured
    // rate, plus one launch) says so. Every tile shape sums K in the same
    // order with the same MFMA, so the split changes no bit of the result.
    if (best == 8) {
        const TiledEntry& big = kTiled[8];
        const double alone = region_us(a, 8, 0);
        double best_us = alone;
        int64_t best_m0 = 0;
        int best_tail = -1;
        for (int64_t m0 = big.bm; m0 < a.M; m0 += big.bm) {
            GemmArgs h = a;
            h.M = m0;                                   // the head: tokens [0, m0)
            const double head_us = region_us(h, 8, 0);
            for (int v : {9, 11, 10}) {
                const double us = head_us + region_us(a, v, m0) + 3.0;
                if (us < best_us) {
                    best_us = us;
                    best_m0 = m0;
                    best_tail = v;
                }
            }
        }
        if (best_tail >= 0 && best_us < 0.97 * alone) {
            GemmArgs h = a;
            h.M = best_m0;
            const hipError_t he = launch_variant(h, 8, 0, s);
            if (he != hipSuccess) return he;
            return launch_variant(a, best_tail, best_m0, s);
        }
    }
    return launch_variant(a, best, 0, s);
}

}  // namespace tpk
