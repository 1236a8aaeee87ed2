// HBM-bound kernels of the tensor-parallel linear path on gfx950:
// weight shard copy, SwiGLU, the partial-sum reducer, the masked vocab gather
// and the logits concatenation. All move 16-byte vectors per lane so that a
// wavefront touches 1 KiB of contiguous memory per access; none of them is a
// contraction, so none of them uses the matrix cores.
#include "common.h"
#include "kernels.h"
#include "layer_ops.h"

namespace tpk {

namespace {

constexpr int kThreads = 256;

// Enough workgroups to fill 256 CUs several times over, then grid-stride.
inline unsigned grid_for(int64_t work_items, int per_thread = 1) {
    int64_t blocks = (work_items + (int64_t)kThreads * per_thread - 1) / ((int64_t)kThreads * per_thread);
    if (blocks < 1) blocks = 1;
    if (blocks > 8192) blocks = 8192;
    return (unsigned)blocks;
}

// ----------------------------------------------------------------- shard copy

__device__ __forceinline__ int64_t shard_src_row(const ShardMap& m, int64_t i) {
    switch (m.kind) {
    case TP_W_QKV: {
        const int64_t d = m.head_dim;
        const int64_t q_rows = (int64_t)m.q_count * d;
        const int64_t kv_rows = (int64_t)m.kv_count * d;
        if (i < q_rows) return (int64_t)m.q_first * d + i;
        i -= q_rows;
        if (i < kv_rows) return ((int64_t)m.num_q_heads + m.kv_first) * d + i;
        i -= kv_rows;
        return ((int64_t)m.num_q_heads + m.num_kv_heads + m.kv_first) * d + i;
    }
    case TP_W_GATE_UP:
        if (i < m.inter_shard) return m.inter_first + i;
        return m.inter + m.inter_first + (i - m.inter_shard);
    case TP_W_EMBED:
    case TP_W_LM_HEAD: {
        const int64_t r = m.vocab_first + i;
        return r < m.vocab ? r : -1;
    }
    default:  // TP_W_O, TP_W_DOWN: same row, column window
        return i;
    }
}

__global__ void __launch_bounds__(kThreads)
shard_copy_kernel(ShardMap m, const uint4* __restrict__ src, uint4* __restrict__ dst) {
    const int64_t vec_per_row = m.dst_cols / 8;
    const int64_t total = m.dst_rows * vec_per_row;
    const int64_t src_vec_per_row = m.src_cols / 8;
    const int64_t col0 = m.src_col0 / 8;
    for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < total;
         v += (int64_t)gridDim.x * kThreads) {
        const int64_t i = v / vec_per_row;
        const int64_t c = v - i * vec_per_row;
        const int64_t r = shard_src_row(m, i);
        uint4 val = make_uint4(0u, 0u, 0u, 0u);
        if (r >= 0) val = src[r * src_vec_per_row + col0 + c];
        dst[v] = val;
    }
}

// --------------------------------------------------------------------- swiglu

__global__ void __launch_bounds__(kThreads)
swiglu_kernel(const uint4* __restrict__ gu, int64_t M, int64_t i_vec, uint4* __restrict__ out) {
    const int64_t total = M * i_vec;
    for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < total;
         v += (int64_t)gridDim.x * kThreads) {
        const int64_t m = v / i_vec;
        const int64_t j = v - m * i_vec;
        const uint4 gv = gu[m * 2 * i_vec + j];
        const uint4 uv = gu[m * 2 * i_vec + i_vec + j];
        float g[8], u[8], o[8];
        unpack_bf16x8(gv, g);
        unpack_bf16x8(uv, u);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = silu_f32(g[e]) * u[e];
        out[v] = pack_bf16x8(o);
    }
}

// --------------------------------------------------------------------- reduce

// Load 8 consecutive elements of a partial as fp32.
template <int IN_F32>
__device__ __forceinline__ void load8(const void* p, int64_t vec, float* f) {
    if (IN_F32) {
        const float4* q = reinterpret_cast<const float4*>(p) + 2 * vec;
        const float4 a = ld_nt16f(q);
        const float4 b = ld_nt16f(q + 1);
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    } else {
        const uint4 v = ld_nt16(reinterpret_cast<const uint4*>(p) + vec);
        unpack_bf16x8(v, f);
    }
}

template <int OUT_F32>
__device__ __forceinline__ void store8(void* p, int64_t vec, const float* f) {
    if (OUT_F32) {
        float4* q = reinterpret_cast<float4*>(p) + 2 * vec;
        q[0] = make_float4(f[0], f[1], f[2], f[3]);
        q[1] = make_float4(f[4], f[5], f[6], f[7]);
    } else {
        reinterpret_cast<uint4*>(p)[vec] = pack_bf16x8(f);
    }
}

template <int IN_F32>
__device__ __forceinline__ float load1(const void* p, int64_t i) {
    if (IN_F32) return reinterpret_cast<const float*>(p)[i];
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}

template <int OUT_F32>
__device__ __forceinline__ void store1(void* p, int64_t i, float f) {
    if (OUT_F32) reinterpret_cast<float*>(p)[i] = f;
    else reinterpret_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_bf16(f);
}

// Fixed summation order i = 0..t-1, accumulator initialised from partial 0:
// the result is bit-identical run to run, and -0.0 contributions leave every
// value (including a -0.0 or subnormal) unchanged. Each thread sums VPT
// vectors of 8 elements (v, v + TH, ...) per pass, issuing every load of the
// pass before the first add.
template <int IN_F32, int OUT_F32, int T, int VPT, int TH>
__global__ void __launch_bounds__(TH)
reduce_kernel(PartialPtrs ptrs, int t_rt, int64_t numel, void* out) {
    const int t = T > 0 ? T : t_rt;
    const int64_t nvec = numel / 8;
    for (int64_t base = (int64_t)blockIdx.x * TH * VPT + threadIdx.x; base < nvec;
         base += (int64_t)gridDim.x * TH * VPT) {
        if (T > 0) {
            float buf[VPT][T][8];
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                const int64_t v = base + (int64_t)j * TH;
                const int64_t vv = v < nvec ? v : base;   // clamped: loads stay unconditional and in bounds
#pragma unroll
                for (int i = 0; i < T; ++i) load8<IN_F32>(ptrs.p[i], vv, buf[j][i]);
            }
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                const int64_t v = base + (int64_t)j * TH;
#pragma unroll
                for (int i = 1; i < T; ++i)
#pragma unroll
                    for (int e = 0; e < 8; ++e) buf[j][0][e] += buf[j][i][e];
                if (v < nvec) store8<OUT_F32>(out, v, buf[j][0]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < VPT; ++j) {
                const int64_t v = base + (int64_t)j * TH;
                if (v >= nvec) break;
                float acc[8];
                load8<IN_F32>(ptrs.p[0], v, acc);
                for (int i = 1; i < t; ++i) {
                    float f[8];
                    load8<IN_F32>(ptrs.p[i], v, f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] += f[e];
                }
                store8<OUT_F32>(out, v, acc);
            }
        }
    }
    // tail (numel % 8 elements), one thread each
    const int64_t tail0 = nvec * 8;
    const int64_t g = (int64_t)blockIdx.x * TH + threadIdx.x;
    if (g < numel - tail0) {
        const int64_t i0 = tail0 + g;
        float acc = load1<IN_F32>(ptrs.p[0], i0);
        for (int i = 1; i < t; ++i) acc += load1<IN_F32>(ptrs.p[i], i0);
        store1<OUT_F32>(out, i0, acc);
    }
}

// Small sums (decode: a few rows) spread one vector per thread over as many
// workgroups as there are vectors / 256; large ones (prefill) run 512-thread
// workgroups with two vectors per thread in flight (measured on MI355X at
// 2048 x 4096, t = 2: 5.1 TB/s against 4.8 for the small-sum shape), for up
// to 8 bf16 partials (more would not fit in registers).
template <int IN_F32, int OUT_F32>
hipError_t reduce_dispatch(const PartialPtrs& ptrs, int t, int64_t numel, void* out, hipStream_t s) {
    const int64_t nvec = numel / 8;
    const bool wide = nvec >= 65536 && !IN_F32 && t <= 8;
    if (wide) {
        int64_t blocks = (nvec + 1023) / 1024;
        if (blocks > 8192) blocks = 8192;
        const dim3 grid((unsigned)blocks);
        switch (t) {
#define TP_REDUCE_WIDE(TT) \
        case TT: hipLaunchKernelGGL((reduce_kernel<IN_F32, OUT_F32, TT, 2, 512>), grid, dim3(512), 0, s, ptrs, t, numel, out); \
            return hipGetLastError();
        TP_REDUCE_WIDE(1) TP_REDUCE_WIDE(2) TP_REDUCE_WIDE(4) TP_REDUCE_WIDE(8)
#undef TP_REDUCE_WIDE
        default:
            hipLaunchKernelGGL((reduce_kernel<IN_F32, OUT_F32, 0, 2, 512>), grid, dim3(512), 0, s, ptrs, t, numel, out);
            return hipGetLastError();
        }
    }
    const unsigned grid = grid_for(nvec > 0 ? nvec : 1);
    switch (t) {
#define TP_REDUCE_CASE(TT) \
    case TT: hipLaunchKernelGGL((reduce_kernel<IN_F32, OUT_F32, TT, 1, kThreads>), dim3(grid), dim3(kThreads), 0, s, ptrs, t, numel, out); break;
    TP_REDUCE_CASE(1) TP_REDUCE_CASE(2) TP_REDUCE_CASE(4) TP_REDUCE_CASE(8) TP_REDUCE_CASE(16)
#undef TP_REDUCE_CASE
    default:
        hipLaunchKernelGGL((reduce_kernel<IN_F32, OUT_F32, 0, 1, kThreads>), dim3(grid), dim3(kThreads), 0, s, ptrs, t, numel, out);
    }
    return hipGetLastError();
}

// ------------------------------------------------ residual add + RMSNorm

// One workgroup per token row (the norm needs the whole row), 512 threads,
// each owning VPT vectors of 8 values, v = thread + 512 j. Every load of the
// row (the residual, gamma and, with T >= 0, all T partials) is issued before
// any is used, so a row costs one memory round trip, then one LDS reduction:
// at decode sizes (16 rows) the latency is the cost. The partials are summed
// in rank order from partial 0 and rounded to bf16 as the reducer stores them
// (T = 0: no add), added to the residual and rounded again; the new residual
// is written back. The squares are summed in a fixed tree (per thread in
// vector order, lane butterflies, then the waves in order), so results are
// the same run to run. out = bf16(h * r * gamma), r = 1 / sqrt(sum / H + eps).
// T = -1: runtime t, partials read in a loop (t not in 0, 1, 2, 4, 8, 16).
constexpr int kNormThreads = 512;

template <int IN_F32, int T, int VPT>
__global__ void __launch_bounds__(kNormThreads)
add_rmsnorm_kernel(PartialPtrs ptrs, int t_rt, uint16_t* __restrict__ residual, const uint16_t* __restrict__ gamma,
                   float eps, int64_t H, uint16_t* __restrict__ out) {
    constexpr int kInVec = IN_F32 ? 2 : 1;        // 16-byte loads per 8 values of a partial
    const int64_t m = blockIdx.x;
    const int64_t nvec = H / 8;
    uint4* res = reinterpret_cast<uint4*>(residual + m * H);
    // gamma == nullptr: unit weights (the loads then read the residual row
    // instead and their values are not used)
    const bool unit = gamma == nullptr;
    const uint4* g4 = reinterpret_cast<const uint4*>(unit ? residual + m * H : gamma);
    const int64_t row_vec = m * nvec * kInVec;     // first 16-byte vector of row m in a partial
    const int t = T >= 0 ? T : t_rt;

    int64_t vv[VPT];
    bool ok[VPT];
    uint4 rraw[VPT], graw[VPT];
    uint4 praw[VPT][(T > 0 ? T : 1) * kInVec];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        const int64_t v = threadIdx.x + (int64_t)kNormThreads * j;
        ok[j] = v < nvec;
        vv[j] = ok[j] ? v : 0;                     // clamped: loads stay in bounds and unconditional
        rraw[j] = res[vv[j]];
        graw[j] = g4[vv[j]];
        if constexpr (T > 0) {
#pragma unroll
            for (int i = 0; i < T; ++i)
#pragma unroll
                for (int q = 0; q < kInVec; ++q)
                    praw[j][i * kInVec + q] = reinterpret_cast<const uint4*>(ptrs.p[i])[row_vec + vv[j] * kInVec + q];
        }
    }

    float h[VPT][8];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        unpack_bf16x8(rraw[j], h[j]);
        if (t > 0) {
            float acc[8];
            auto part = [&](int i, float* f) {
                if constexpr (T > 0) {
                    if (IN_F32) {
                        const uint4 a = praw[j][i * kInVec], b = praw[j][i * kInVec + kInVec - 1];
                        f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y);
                        f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
                        f[4] = __uint_as_float(b.x); f[5] = __uint_as_float(b.y);
                        f[6] = __uint_as_float(b.z); f[7] = __uint_as_float(b.w);
                    } else {
                        unpack_bf16x8(praw[j][i], f);
                    }
                } else {
                    load8<IN_F32>(reinterpret_cast<const char*>(ptrs.p[i]) + row_vec * 16, vv[j], f);
                }
            };
            part(0, acc);
#pragma unroll
            for (int i = 1; i < t; ++i) {
                float f[8];
                part(i, f);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += f[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) h[j][e] = round_bf16(h[j][e] + round_bf16(acc[e]));
            if (ok[j]) res[vv[j]] = pack_bf16x8(h[j]);
        }
        if (ok[j]) {
#pragma unroll
            for (int e = 0; e < 8; ++e) ss += h[j][e] * h[j][e];
        }
    }
    if (out == nullptr) return;      // the sum and the residual add only (uniform)
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    __shared__ float wave_ss[kNormThreads / 64];
    if ((threadIdx.x & 63) == 0) wave_ss[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = wave_ss[0];
#pragma unroll
    for (int w = 1; w < kNormThreads / 64; ++w) tot += wave_ss[w];
    const float r = 1.0f / sqrtf(tot / (float)H + eps);
    uint4* o4 = reinterpret_cast<uint4*>(out + m * H);
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
        float g[8], y[8];
        unpack_bf16x8(graw[j], g);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = unit ? h[j][e] * r : h[j][e] * r * g[e];
        if (ok[j]) o4[vv[j]] = pack_bf16x8(y);
    }
}

template <int IN_F32, int T>
hipError_t add_rmsnorm_vpt(const PartialPtrs& ptrs, int t, int64_t M, int64_t H, uint16_t* res,
                           const uint16_t* g, float eps, uint16_t* o, hipStream_t s) {
    const int64_t nvec = H / 8;
    const dim3 grid((unsigned)M), block(kNormThreads);
    if (nvec <= kNormThreads)
        hipLaunchKernelGGL((add_rmsnorm_kernel<IN_F32, T, 1>), grid, block, 0, s, ptrs, t, res, g, eps, H, o);
    else if (nvec <= 2 * kNormThreads)   // 16 fp32 partials of 2 vectors would spill: loop instead
        hipLaunchKernelGGL((add_rmsnorm_kernel<IN_F32, (IN_F32 && T > 8 ? -1 : T), 2>), grid, block, 0, s, ptrs, t,
                           res, g, eps, H, o);
    // wider rows: partials read in a loop (all T partials of 4 or 8 vectors
    // per thread would not fit in registers)
    else if (nvec <= 4 * kNormThreads)
        hipLaunchKernelGGL((add_rmsnorm_kernel<IN_F32, -1, 4>), grid, block, 0, s, ptrs, t, res, g, eps, H, o);
    else
        hipLaunchKernelGGL((add_rmsnorm_kernel<IN_F32, -1, 8>), grid, block, 0, s, ptrs, t, res, g, eps, H, o);
    return hipGetLastError();
}

template <int IN_F32>
hipError_t add_rmsnorm_t(const PartialPtrs& ptrs, int t, int64_t M, int64_t H, uint16_t* res,
                         const uint16_t* g, float eps, uint16_t* o, hipStream_t s) {
    switch (t) {
    case 0: return add_rmsnorm_vpt<IN_F32, 0>(ptrs, t, M, H, res, g, eps, o, s);
    case 1: return add_rmsnorm_vpt<IN_F32, 1>(ptrs, t, M, H, res, g, eps, o, s);
    case 2: return add_rmsnorm_vpt<IN_F32, 2>(ptrs, t, M, H, res, g, eps, o, s);
    case 4: return add_rmsnorm_vpt<IN_F32, 4>(ptrs, t, M, H, res, g, eps, o, s);
    case 8: return add_rmsnorm_vpt<IN_F32, 8>(ptrs, t, M, H, res, g, eps, o, s);
    case 16: return add_rmsnorm_vpt<IN_F32, 16>(ptrs, t, M, H, res, g, eps, o, s);
    default: return add_rmsnorm_vpt<IN_F32, -1>(ptrs, t, M, H, res, g, eps, o, s);
    }
}

// --------------------------------------------------------- norm weight folding

// w_out[n, k] = bf16(w[n, k] * gamma[k]), 8 elements per thread (K % 8 == 0).
__global__ void __launch_bounds__(kThreads)
fold_norm_weight_kernel(const uint4* __restrict__ w, const uint4* __restrict__ gamma, int64_t k_vec, int64_t total,
                        uint4* __restrict__ out) {
    for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < total; v += (int64_t)gridDim.x * kThreads) {
        float x[8], g[8];
        unpack_bf16x8(w[v], x);
        unpack_bf16x8(gamma[v % k_vec], g);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= g[e];
        out[v] = pack_bf16x8(x);
    }
}


// ---------------------------------------------------------------- vocab embed

// One contribution of a vocab-parallel embedding: row ids[m] - lo of this
// shard's table when lo <= ids[m] < hi, else -0.0 in every element.
__global__ void __launch_bounds__(kThreads)
vocab_embed_kernel(const int32_t* __restrict__ ids, int64_t M, const uint4* __restrict__ table,
                   int64_t lo, int64_t hi, int64_t h_vec, uint4* __restrict__ out) {
    const uint4 neg_zero = make_uint4(0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u);
    const int64_t total = M * h_vec;
    for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < total;
         v += (int64_t)gridDim.x * kThreads) {
        const int64_t m = v / h_vec;
        const int64_t c = v - m * h_vec;
        const int64_t id = ids[m];
        uint4 val = neg_zero;
        if (id >= lo && id < hi) val = table[(id - lo) * h_vec + c];
        out[v] = val;
    }
}

// --------------------------------------------------------------- concat logits

// Vector path: v_shard % 8 == 0 and vocab % 8 == 0, so each 8-element output
// chunk comes from one shard and both sides are 16-byte aligned.
template <int F32>
__global__ void __launch_bounds__(kThreads)
concat_vec_kernel(PartialPtrs ptrs, int64_t M, int64_t v_shard, int64_t vocab, void* out) {
    const int64_t out_vec = vocab / 8;
    const int64_t total = M * out_vec;
    const int64_t sh_vec = v_shard / 8;
    for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < total;
         v += (int64_t)gridDim.x * kThreads) {
        const int64_t m = v / out_vec;
        const int64_t c = v - m * out_vec;   // output chunk in this row
        const int64_t r = c / sh_vec;
        const int64_t j = c - r * sh_vec;
        if (F32) {
            const float4* src = reinterpret_cast<const float4*>(ptrs.p[r]) + 2 * (m * sh_vec + j);
            float4* dst = reinterpret_cast<float4*>(out) + 2 * v;
            dst[0] = src[0];
            dst[1] = src[1];
        } else {
            reinterpret_cast<uint4*>(out)[v] = reinterpret_cast<const uint4*>(ptrs.p[r])[m * sh_vec + j];
        }
    }
}

// Element path for any v_shard / vocab.
template <int F32>
__global__ void __launch_bounds__(kThreads)
concat_elem_kernel(PartialPtrs ptrs, int64_t M, int64_t v_shard, int64_t vocab, void* out) {
    const int64_t total = M * vocab;
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * kThreads) {
        const int64_t m = e / vocab;
        const int64_t col = e - m * vocab;
        const int64_t r = col / v_shard;
        const int64_t j = col - r * v_shard;
        if (F32) reinterpret_cast<float*>(out)[e] = reinterpret_cast<const float*>(ptrs.p[r])[m * v_shard + j];
        else reinterpret_cast<uint16_t*>(out)[e] = reinterpret_cast<const uint16_t*>(ptrs.p[r])[m * v_shard + j];
    }
}

}  // namespace

hipError_t launch_shard_copy(const ShardMap& map, const void* full, void* shard, hipStream_t s) {
    const int64_t total = map.dst_rows * (map.dst_cols / 8);
    hipLaunchKernelGGL(shard_copy_kernel, dim3(grid_for(total)), dim3(kThreads), 0, s, map,
                       reinterpret_cast<const uint4*>(full), reinterpret_cast<uint4*>(shard));
    return hipGetLastError();
}

hipError_t launch_swiglu(const void* gu, int64_t M, int64_t i_shard, void* out, hipStream_t s) {
    const int64_t i_vec = i_shard / 8;
    hipLaunchKernelGGL(swiglu_kernel, dim3(grid_for(M * i_vec)), dim3(kThreads), 0, s,
                       reinterpret_cast<const uint4*>(gu), M, i_vec, reinterpret_cast<uint4*>(out));
    return hipGetLastError();
}

hipError_t launch_reduce(const PartialPtrs& ptrs, int t, int64_t numel, int in_dtype,
                         void* out, int out_dtype, hipStream_t s) {
    if (in_dtype == TP_F32)
        return out_dtype == TP_F32 ? reduce_dispatch<1, 1>(ptrs, t, numel, out, s)
                                   : reduce_dispatch<1, 0>(ptrs, t, numel, out, s);
    return out_dtype == TP_F32 ? reduce_dispatch<0, 1>(ptrs, t, numel, out, s)
                               : reduce_dispatch<0, 0>(ptrs, t, numel, out, s);
}

hipError_t launch_vocab_embed(const int32_t* ids, int64_t M, const void* table, int64_t lo,
                              int64_t hi, int64_t H, void* out, hipStream_t s) {
    const int64_t h_vec = H / 8;
    hipLaunchKernelGGL(vocab_embed_kernel, dim3(grid_for(M * h_vec)), dim3(kThreads), 0, s, ids, M,
                       reinterpret_cast<const uint4*>(table), lo, hi, h_vec, reinterpret_cast<uint4*>(out));
    return hipGetLastError();
}

hipError_t launch_concat(const PartialPtrs& ptrs, int t, int64_t M, int64_t v_shard,
                         int64_t vocab, int dtype, void* out, hipStream_t s) {
    (void)t;
    const bool vec = (v_shard % 8 == 0) && (vocab % 8 == 0);
    if (vec) {
        const unsigned g = grid_for(M * (vocab / 8));
        if (dtype == TP_F32) hipLaunchKernelGGL(concat_vec_kernel<1>, dim3(g), dim3(kThreads), 0, s, ptrs, M, v_shard, vocab, out);
        else hipLaunchKernelGGL(concat_vec_kernel<0>, dim3(g), dim3(kThreads), 0, s, ptrs, M, v_shard, vocab, out);
    } else {
        const unsigned g = grid_for(M * vocab);
        if (dtype == TP_F32) hipLaunchKernelGGL(concat_elem_kernel<1>, dim3(g), dim3(kThreads), 0, s, ptrs, M, v_shard, vocab, out);
        else hipLaunchKernelGGL(concat_elem_kernel<0>, dim3(g), dim3(kThreads), 0, s, ptrs, M, v_shard, vocab, out);
    }
    return hipGetLastError();
}

hipError_t launch_add_rmsnorm(const PartialPtrs& ptrs, int t, int in_dtype, int64_t M, int64_t H,
                              void* residual, const void* gamma, float eps, void* out, hipStream_t s) {
    if (H / 8 > 8 * kNormThreads) return hipErrorInvalidValue;   // H > 32768: rejected by the ABI
    uint16_t* res = reinterpret_cast<uint16_t*>(residual);
    const uint16_t* g = reinterpret_cast<const uint16_t*>(gamma);
    uint16_t* o = reinterpret_cast<uint16_t*>(out);
    return in_dtype == TP_F32 ? add_rmsnorm_t<1>(ptrs, t, M, H, res, g, eps, o, s)
                              : add_rmsnorm_t<0>(ptrs, t, M, H, res, g, eps, o, s);
}

hipError_t launch_fold_norm_weight(const void* w, int64_t N, int64_t K, const void* gamma, void* out, hipStream_t s) {
    const int64_t total = N * (K / 8);
    int64_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fold_norm_weight_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       static_cast<const uint4*>(w), static_cast<const uint4*>(gamma), K / 8, total,
                       static_cast<uint4*>(out));
    return hipGetLastError();
}

}  // namespace tpk
