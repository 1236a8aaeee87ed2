// One decode step of a rank's grouped-query attention on gfx950, with the
// KV-cache append folded in.
//
// A rank holds nq query heads and nkv KV heads (its share, KV heads possibly
// replicated); the G = nq / nkv query heads of a group read the same K and V.
// Decode attention is bound by reading the cache once: per (sequence, KV head)
// 2 (n) D bytes of bf16 K and V against 4 G (n) D flops, far below what the
// vector ALU sustains, so there are no MFMAs here. Design:
//   * Workgroups split the sequence: one per (chunk of 128 positions, KV
//     head, sequence). Each reads its K and V rows once for all G heads of the
//     group. D / 8 lanes hold one position (16 bytes each), so a wave covers
//     64 / (D / 8) positions per step; every K and V load of the chunk is
//     issued before the first is used (clamped addresses, masked results).
//   * The new token's K and V are read from the qkv output (its position is
//     lens[b]); the workgroup whose chunk holds that position also writes
//     them into the cache. No other workgroup of the launch reads that cache
//     row, so the append needs no ordering.
//   * Per chunk: scores in LDS, each wave takes whole heads for the max, the
//     exponentials and their sum; the weighted V rows are summed across the
//     position slots of a wave by lane swaps, then across the waves in order.
//   * Chunks are merged by the last workgroup to arrive on (sequence, KV
//     head) (one counter each, reset by that workgroup): partial results
//     travel through relaxed device-scope stores and loads and are combined
//     in chunk order with the usual max-rescaling, so the result does not
//     depend on arrival order.
#include "common.h"
#include "layer_ops.h"

namespace tpk {

namespace {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / 64;

template <int D, int G>
__global__ void __launch_bounds__(kAttnThreads)
decode_attention_kernel(AttnArgs a, float* __restrict__ ws, unsigned* __restrict__ counters) {
    constexpr int LP = D / 8;                        // lanes per position
    constexpr int PW = 64 / LP;                      // positions per wave step
    constexpr int STEPS = kAttnChunk / (kAttnWaves * PW);
    constexpr int REC = G * (D + 2);                 // floats of one chunk's partial: G x (o[D], m, l)
    static_assert(kAttnChunk % (kAttnWaves * PW) == 0, "chunk must split evenly over the waves");

    __shared__ float s_score[G][kAttnChunk];
    __shared__ float s_ml[G][2];
    __shared__ float s_acc[kAttnWaves][G][D];
    __shared__ unsigned s_last;

    const int ci = blockIdx.x, kvh = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = lane / LP, piece = lane % LP;
    const int nchunks = gridDim.x;
    const int32_t len = a.lens[b];
    const bool valid_seq = len >= 0 && len < a.L;
    const int n = valid_seq ? len + 1 : 0;           // keys: the cached ones and the new one
    const int p0 = ci * kAttnChunk;
    const int cnt = n - p0 < kAttnChunk ? n - p0 : kAttnChunk;   // positions of this chunk (<= 0: none)

    const uint16_t* qrow = a.qkv + b * a.qkv_stride;
    const uint16_t* k_new = qrow + (int64_t)(a.nq + kvh) * D + piece * 8;
    const uint16_t* v_new = qrow + (int64_t)(a.nq + a.nkv + kvh) * D + piece * 8;
    const int64_t cache_base = ((b * a.nkv + kvh) * a.L) * D + piece * 8;
    float* rec = ws + ((b * a.nkv + kvh) * nchunks + ci) * (int64_t)REC;

    if (cnt > 0) {
        // every K and V piece of the chunk, then the queries (pre-scaled)
        uint4 kr[STEPS], vr[STEPS];
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const int idx = (st * kAttnWaves + wave) * PW + sub;
            const int pos = p0 + (idx < cnt ? idx : cnt - 1);
            const bool is_new = pos == n - 1;
            const uint16_t* kp = is_new ? k_new : a.k_cache + cache_base + (int64_t)pos * D;
            const uint16_t* vp = is_new ? v_new : a.v_cache + cache_base + (int64_t)pos * D;
            kr[st] = *reinterpret_cast<const uint4*>(kp);
            vr[st] = *reinterpret_cast<const uint4*>(vp);
        }
        float qf[G][8];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            unpack_bf16x8(*reinterpret_cast<const uint4*>(qrow + (int64_t)(kvh * G + g) * D + piece * 8), qf[g]);
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[g][e] *= a.scale;
        }
        // the append: the lanes that hold the new row write it to the cache
        if (n - 1 >= p0 && n - 1 < p0 + kAttnChunk) {
#pragma unroll
            for (int st = 0; st < STEPS; ++st) {
                const int idx = (st * kAttnWaves + wave) * PW + sub;
                if (p0 + idx == n - 1) {
                    *reinterpret_cast<uint4*>(a.k_cache + cache_base + (int64_t)(n - 1) * D) = kr[st];
                    *reinterpret_cast<uint4*>(a.v_cache + cache_base + (int64_t)(n - 1) * D) = vr[st];
                }
            }
        }
        // scores
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const int idx = (st * kAttnWaves + wave) * PW + sub;
            float kf[8];
            unpack_bf16x8(kr[st], kf);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) d += qf[g][e] * kf[e];
#pragma unroll
                for (int o = 1; o < LP; o <<= 1) d += __shfl_xor(d, o);
                if (piece == 0 && idx < cnt) s_score[g][idx] = d;
            }
        }
        __syncthreads();
        // softmax statistics: wave w takes heads w, w + 4, ...
        for (int g = wave; g < G; g += kAttnWaves) {
            float m = -INFINITY;
            for (int i = lane; i < cnt; i += 64) m = fmaxf(m, s_score[g][i]);
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
            float l = 0.f;
            for (int i = lane; i < cnt; i += 64) {
                const float p = __expf(s_score[g][i] - m);
                s_score[g][i] = p;
                l += p;
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
            if (lane == 0) {
                s_ml[g][0] = m;
                s_ml[g][1] = l;
            }
        }
        __syncthreads();
        // weighted V rows: per lane over its positions, then over the
        // position slots of the wave, then over the waves
        float acc[G][8];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const int idx = (st * kAttnWaves + wave) * PW + sub;
            float vf[8];
            unpack_bf16x8(vr[st], vf);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float p = idx < cnt ? s_score[g][idx] : 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[g][e] += p * vf[e];
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float v = acc[g][e];
#pragma unroll
                for (int o = LP; o < 64; o <<= 1) v += __shfl_xor(v, o);
                acc[g][e] = v;
            }
        if (sub == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int e = 0; e < 8; ++e) s_acc[wave][g][piece * 8 + e] = acc[g][e];
        }
        __syncthreads();
        // publish this chunk's partial: o[G][D], then m and l per head
        for (int i = tid; i < G * D; i += kAttnThreads) {
            const int g = i / D, j = i % D;
            float v = s_acc[0][g][j];
#pragma unroll
            for (int w = 1; w < kAttnWaves; ++w) v += s_acc[w][g][j];
            __hip_atomic_store(rec + g * (D + 2) + j, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (tid < G) {
            __hip_atomic_store(rec + tid * (D + 2) + D, s_ml[tid][0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(rec + tid * (D + 2) + D + 1, s_ml[tid][1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    unsigned* ctr = counters + b * a.nkv + kvh;
    if (tid == 0) {
        const unsigned prev = atomicAdd(ctr, 1u);
        s_last = prev == (unsigned)(nchunks - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (s_last != 1u) return;

    // Last workgroup on (b, kvh): merge the chunks that hold positions, in
    // chunk order. A sequence with lens[b] outside [0, L) gets a zero row.
    // One memory round: each thread issues the loads of its outputs' partial
    // values for up to BATCH chunks and of the chunks' max and sum before any
    // is used; the weights w_c = e^(m_c - M) / sum_c' l_c' e^(m_c' - M) are
    // formed in LDS; each output sums w_c o_c in chunk order.
    constexpr int OPT = (G * D + kAttnThreads - 1) / kAttnThreads;   // outputs per thread
    constexpr int BATCH = OPT >= 8 ? 8 : 64 / OPT;                   // chunks per round of loads
    __shared__ float s_w[G][kAttnMaxChunks];
    __shared__ float s_m[G][kAttnMaxChunks];
    const int nvalid = (n + kAttnChunk - 1) / kAttnChunk;
    const float* base = ws + ((b * a.nkv + kvh) * nchunks) * (int64_t)REC;
    const int last_c = nvalid > 0 ? nvalid - 1 : 0;
    float part[OPT][BATCH];
#pragma unroll
    for (int q = 0; q < OPT; ++q) {
        const int i = tid + q * kAttnThreads < G * D ? tid + q * kAttnThreads : 0;
        const int g = i / D, j = i % D;
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
            const int c = k < last_c ? k : last_c;
            part[q][k] = __hip_atomic_load(base + c * REC + g * (D + 2) + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    for (int i = tid; i < G * nvalid; i += kAttnThreads) {
        const int g = i / nvalid, c = i % nvalid;
        const float* r = base + c * REC + g * (D + 2) + D;
        s_m[g][c] = __hip_atomic_load(r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_w[g][c] = __hip_atomic_load(r + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (tid < G) {
        float mx = -INFINITY;
        for (int c = 0; c < nvalid; ++c) mx = fmaxf(mx, s_m[tid][c]);
        float l = 0.f;
        for (int c = 0; c < nvalid; ++c) l += s_w[tid][c] * __expf(s_m[tid][c] - mx);
        for (int c = 0; c < nvalid; ++c) s_w[tid][c] = __expf(s_m[tid][c] - mx) / l;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < OPT; ++q) {
        const int i = tid + q * kAttnThreads;
        if (i < G * D) {
            const int g = i / D, j = i % D;
            float o = 0.f;
#pragma unroll
            for (int k = 0; k < BATCH; ++k)
                if (k < nvalid) o += s_w[g][k] * part[q][k];
            for (int c = BATCH; c < nvalid; ++c)   // more than BATCH chunks: one load each
                o += s_w[g][c] * __hip_atomic_load(base + c * REC + g * (D + 2) + j, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
            a.ctx[b * (int64_t)a.nq * D + (int64_t)(kvh * G + g) * D + j] = (uint16_t)f32_to_bf16(o);
        }
    }
    if (tid == 0) atomicExch(ctr, 0u);
}

typedef void (*AttnFn)(AttnArgs, float*, unsigned*);

template <int D>
AttnFn attn_for_group(int g) {
    switch (g) {
    case 1: return decode_attention_kernel<D, 1>;
    case 2: return decode_attention_kernel<D, 2>;
    case 3: return decode_attention_kernel<D, 3>;
    case 4: return decode_attention_kernel<D, 4>;
    case 5: return decode_attention_kernel<D, 5>;
    case 6: return decode_attention_kernel<D, 6>;
    case 7: return decode_attention_kernel<D, 7>;
    case 8: return decode_attention_kernel<D, 8>;
    default: return nullptr;
    }
}

}  // namespace

int64_t attention_workspace_floats(const AttnArgs& a) {
    const int64_t nchunks = (a.L + kAttnChunk - 1) / kAttnChunk;
    const int64_t g = a.nq / a.nkv;
    return a.B * a.nkv * nchunks * g * (a.head_dim + 2);
}

hipError_t launch_decode_attention(const AttnArgs& a, const Workspace& ws, hipStream_t s) {
    const int g = a.nq / a.nkv;
    AttnFn fn = nullptr;
    switch (a.head_dim) {
    case 32: fn = attn_for_group<32>(g); break;
    case 64: fn = attn_for_group<64>(g); break;
    case 128: fn = attn_for_group<128>(g); break;
    case 256: fn = attn_for_group<256>(g); break;
    default: break;
    }
    if (fn == nullptr) return hipErrorInvalidValue;
    const unsigned nchunks = (unsigned)((a.L + kAttnChunk - 1) / kAttnChunk);
    hipLaunchKernelGGL(fn, dim3(nchunks, (unsigned)a.nkv, (unsigned)a.B), dim3(kAttnThreads), 0, s, a,
                       ws.partials, ws.counters);
    return hipGetLastError();
}

}  // namespace tpk
