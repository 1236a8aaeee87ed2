// One decode step of a rank's grouped-query attention on gfx950, with the
// KV-cache append folded in.
//
// A rank holds nq query heads and nkv KV heads (its share, KV heads possibly
// replicated); the G = nq / nkv query heads of a group read the same K and V.
// Decode attention is bound by reading the cache once: per (sequence, KV
// head) 2 (n) D bytes of bf16 K and V. Two launches:
//
//   1. attn_chunk_kernel, one workgroup of 4 waves per (chunk of positions,
//      KV head, sequence). A chunk is 192 positions (64 at d = 256, where a
//      second 16-row block per wave would not fit in registers): at the
//      decode workloads' shapes it leaves the busiest CU the fewest cache
//      rows to stream (128 and 256 were slower), and being fixed, a
//      sequence's result does not depend on the batch around it. Every cache load of the chunk, the queries and the
//      new token's K and V are issued at the start, before the sequence length
//      arrives (the cache rows through a buffer resource over the (sequence,
//      KV head)'s L rows, so positions past L read zeros; rows past the
//      length are masked once it is known), so the loads cost one memory
//      round trip. Against clamped 64-bit addresses the buffer resource took
//      the 64-token workload's call (Llama-8B t = 16) from 21.2 to 19.8 us
//      and left the 16-token one at 12.1-12.2 us.
//        * Scores on the matrix cores: v_mfma_f32_16x16x32_bf16 with 16 cache
//          rows as the A operand and the group's query heads (padded to 16)
//          as the B operand, so every lane ends with 4 whole dot products and
//          no cross-lane reduction is needed.
//        * Softmax statistics per wave (max and sum of its positions, per
//          head); the probabilities go through a wave-private LDS slab to the
//          layout of the V loads, where each lane owns 8 consecutive columns
//          of V and sums p * v over its positions.
//        * The waves' sums are rescaled to the chunk's max and written, with
//          that max and the chunk's sum of exponentials, as one record per
//          (chunk, head) to the workspace (plain stores: the kernel boundary
//          makes them visible to the merge).
//      The workgroup whose chunk holds the new token's position replaces the
//      stale cache row in registers and writes the new K and V into the caches
//      (the append); no other workgroup reads that row.
//   2. attn_merge_kernel, one thread per output column: the records of the
//      chunks in use are combined in chunk order with the usual max
//      rescaling, so the result does not depend on scheduling.
#include "common.h"
#include "layer_ops.h"

namespace tpk {

namespace {

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = kAttnThreads / 64;

template <int D, int G, int NB>
__global__ void __launch_bounds__(kAttnThreads)
attn_chunk_kernel(AttnArgs a, float* __restrict__ ws) {
    constexpr int WP = 16 * NB;                      // positions per wave (NB MFMA blocks of 16)
    constexpr int CH = WP * kAttnWaves;              // positions per workgroup
    constexpr int KS = D / 32;                       // MFMA k-steps per block
    constexpr int LPR = D / 8;                       // lanes per V row (16 bytes each)
    constexpr int RPI = 64 / LPR;                    // V rows per wave load
    constexpr int VSTEPS = WP / RPI;                 // V loads per lane
    constexpr int GP = G <= 4 ? 4 : 8;               // heads, padded, per LDS probability row
    constexpr int RED = G > 4 ? 2 : 1;               // row groups folded by a lane swap first
    constexpr int RG = RPI / RED;                    // row groups per wave kept in LDS
    constexpr int REC = G * (D + 2);                 // floats of one chunk's record
    static_assert(WP % 16 == 0 && WP % RPI == 0, "wave positions must split into blocks and V steps");

    __shared__ __align__(16) float s_p[kAttnWaves][WP][GP];         // probabilities (wave-private)
    __shared__ float s_ml[kAttnWaves][2][GP];                      // per wave and head: max, sum
    __shared__ __align__(16) float s_o[kAttnWaves * RG][G][D];     // per row group: sum of p v

    const int ci = blockIdx.x, kvh = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p0 = ci * CH;
    const int pw = p0 + wave * WP;                   // first position of this wave

    const uint16_t* qrow = a.qkv + b * a.qkv_stride;
    const uint16_t* k_new = qrow + (int64_t)(a.nq + kvh) * D;
    const uint16_t* v_new = qrow + (int64_t)(a.nq + a.nkv + kvh) * D;
    const int64_t cache0 = (b * a.nkv + kvh) * a.L * D;

    // 1. Loads. MFMA operand lanes: row (cache position or head) lane & 15,
    //    8-element group lane >> 4 of each 32-wide k-step. V lanes: row
    //    lane / LPR of each step, columns vd .. vd + 7.
    const int32_t len = a.lens[b];
    const int kr = lane & 15, kq = lane >> 4;
    const int vr = lane / LPR, vd = 8 * (lane % LPR);
    const __amdgpu_buffer_rsrc_t rs_k = buffer_source(a.k_cache + cache0, a.L * D * 2);
    const __amdgpu_buffer_rsrc_t rs_v = buffer_source(a.v_cache + cache0, a.L * D * 2);
    uint4 kf[NB][KS];
#pragma unroll
    for (int bl = 0; bl < NB; ++bl) {
        const int pos = pw + 16 * bl + kr;
        const uint32_t off = (uint32_t)(((int64_t)pos * D + 8 * kq) * 2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[bl][ks] = buffer_ld16(rs_k, off + 64 * ks);
    }
    uint4 vf[VSTEPS];
#pragma unroll
    for (int st = 0; st < VSTEPS; ++st) {
        const int pos = pw + st * RPI + vr;
        vf[st] = buffer_ld16(rs_v, (uint32_t)(((int64_t)pos * D + vd) * 2));
    }
    // query head kr of the group (lanes past G read head 0; their columns of
    // the scores are never used) and the new token's K in the same layout
    const int qh = kr < G ? kr : 0;
    uint4 qf[KS], knf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        qf[ks] = *reinterpret_cast<const uint4*>(qrow + (int64_t)(kvh * G + qh) * D + 32 * ks + 8 * kq);
        knf[ks] = *reinterpret_cast<const uint4*>(k_new + 32 * ks + 8 * kq);
    }
    const uint4 vn = *reinterpret_cast<const uint4*>(v_new + vd);

    // 2. Positions 0 .. n-1 are in use: the cached ones and the new token at
    //    n - 1 = lens[b] (none when lens[b] is outside [0, L)). The new row
    //    replaces the stale cache row and is appended by the lanes holding it.
    const bool valid = len >= 0 && (int64_t)len < a.L;
    const int n = valid ? len + 1 : 0;
#pragma unroll
    for (int bl = 0; bl < NB; ++bl) {
        const int pos = pw + 16 * bl + kr;
        if (pos == n - 1) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                kf[bl][ks] = knf[ks];
                *reinterpret_cast<uint4*>(a.k_cache + cache0 + (int64_t)pos * D + 32 * ks + 8 * kq) = knf[ks];
            }
        }
    }
#pragma unroll
    for (int st = 0; st < VSTEPS; ++st) {
        const int pos = pw + st * RPI + vr;
        if (pos == n - 1) {
            vf[st] = vn;
            *reinterpret_cast<uint4*>(a.v_cache + cache0 + (int64_t)pos * D + vd) = vn;
        }
        // rows past the end may hold anything (NaN included): their weight is 0
        if (pos >= n) vf[st] = make_uint4(0u, 0u, 0u, 0u);
    }

    // 3. Scores: sc[bl][r] = K[pw + 16 bl + 4 kq + r] . Q[head kr].
    f32x4_t sc[NB];
#pragma unroll
    for (int bl = 0; bl < NB; ++bl) {
        sc[bl] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            sc[bl] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[bl][ks]),
                                                             __builtin_bit_cast(bf16x8_t, qf[ks]), sc[bl], 0, 0, 0);
    }

    // 4. Per-wave softmax statistics of each head: the 4 lanes of a head
    //    (kq = 0..3) hold its WP scores. A wave with no position in use keeps
    //    max -inf and sum 0 and contributes nothing.
    float s[NB][4];
    float mx = -INFINITY;
#pragma unroll
    for (int bl = 0; bl < NB; ++bl)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int pos = pw + 16 * bl + 4 * kq + r;
            s[bl][r] = pos < n ? sc[bl][r] * a.scale : -INFINITY;
            mx = fmaxf(mx, s[bl][r]);
        }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mref = mx == -INFINITY ? 0.f : mx;
    float l = 0.f;
#pragma unroll
    for (int bl = 0; bl < NB; ++bl)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            s[bl][r] = __expf(s[bl][r] - mref);
            l += s[bl][r];
        }
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (kr < G) {
#pragma unroll
        for (int bl = 0; bl < NB; ++bl)
#pragma unroll
            for (int r = 0; r < 4; ++r) s_p[wave][16 * bl + 4 * kq + r][kr] = s[bl][r];
        if (kq == 0) {
            s_ml[wave][0][kr] = mx;
            s_ml[wave][1][kr] = l;
        }
    }
    lds_barrier();

    // 5. Weighted V rows: each lane over its VSTEPS positions, for every head.
    float acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
#pragma unroll
    for (int st = 0; st < VSTEPS; ++st) {
        float p[GP];
#pragma unroll
        for (int q = 0; q < GP / 4; ++q) {
            const float4 p4 = *reinterpret_cast<const float4*>(&s_p[wave][st * RPI + vr][4 * q]);
            p[4 * q] = p4.x;
            p[4 * q + 1] = p4.y;
            p[4 * q + 2] = p4.z;
            p[4 * q + 3] = p4.w;
        }
        float v[8];
        unpack_bf16x8(vf[st], v);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] += p[g] * v[e];
    }
    if constexpr (RED == 2) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] += __shfl_xor(acc[g][e], 32);
    }
    if (RED == 1 || lane < 32) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float* dst = &s_o[wave * RG + vr][g][vd];
            *reinterpret_cast<float4*>(dst) = make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
        }
    }
    lds_barrier();

    // 6. The chunk's record per head: sum over waves of e^(m_w - m) o_w (row
    //    groups and waves in order), then m = max_w m_w and sum_w e^(m_w - m) l_w.
    if (n <= p0) return;                              // no position of this chunk in use
    float* rec = ws + ((b * a.nkv + kvh) * gridDim.x + ci) * (int64_t)REC;
    for (int i = tid; i < G * D; i += kAttnThreads) {
        const int g = i / D, j = i - g * D;
        float m = -INFINITY;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) m = fmaxf(m, s_ml[w][0][g]);
        float o = 0.f, lc = 0.f;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) {
            const float f = __expf(s_ml[w][0][g] - m);
            float ow = 0.f;
#pragma unroll
            for (int r = 0; r < RG; ++r) ow += s_o[w * RG + r][g][j];
            o += f * ow;
            lc += f * s_ml[w][1][g];
        }
        rec[g * (D + 2) + j] = o;
        if (j == 0) {
            rec[g * (D + 2) + D] = m;
            rec[g * (D + 2) + D + 1] = lc;
        }
    }
}

// Records of the chunks 0 .. ceil(n / chunk) - 1 of (sequence, KV head),
// combined in chunk order, MB chunks per round of loads:
// ctx = sum_c e^(m_c - M) o_c / sum_c e^(m_c - M) l_c with M the running max.
// The first round's loads do not wait for the sequence length (they cover
// the first MB chunks of the cache; records past the ones in use are left
// over from other calls and are never used).
template <int D, int G>
__global__ void __launch_bounds__(D)
attn_merge_kernel(AttnArgs a, const float* __restrict__ ws, int nchunks, int chunk) {
    constexpr int REC = G * (D + 2);
    constexpr int MB = 32;
    const int g = blockIdx.x, kvh = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int j = threadIdx.x;
    const float* base = ws + (b * a.nkv + kvh) * (int64_t)nchunks * REC + g * (D + 2);
    const int32_t len = a.lens[b];
    float mc[MB], lc[MB], oc[MB];
    auto load = [&](int c0, int cmax) {
#pragma unroll
        for (int k = 0; k < MB; ++k) {
            const int c = c0 + k < cmax ? c0 + k : cmax - 1;
            mc[k] = base[(int64_t)c * REC + D];
            lc[k] = base[(int64_t)c * REC + D + 1];
            oc[k] = base[(int64_t)c * REC + j];
        }
    };
    load(0, nchunks);
    const bool valid = len >= 0 && (int64_t)len < a.L;
    const int n = valid ? len + 1 : 0;
    const int nvalid = (n + chunk - 1) / chunk;
    float M = -INFINITY, lsum = 0.f, o = 0.f;
    for (int c0 = 0; c0 < nvalid; c0 += MB) {
        if (c0 > 0) load(c0, nvalid);
        float Mn = M;
#pragma unroll
        for (int k = 0; k < MB; ++k)
            if (c0 + k < nvalid) Mn = fmaxf(Mn, mc[k]);
        const float f = __expf(M - Mn);               // 0 on the first round (M = -inf)
        lsum *= f;
        o *= f;
#pragma unroll
        for (int k = 0; k < MB; ++k)
            if (c0 + k < nvalid) {
                const float e = __expf(mc[k] - Mn);
                lsum += e * lc[k];
                o += e * oc[k];
            }
        M = Mn;
    }
    // a sequence with no position in use gets a zero row
    a.ctx[b * (int64_t)a.nq * D + (int64_t)(kvh * G + g) * D + j] =
        (uint16_t)f32_to_bf16(nvalid > 0 ? o / lsum : 0.f);
}

// MFMA blocks of 16 positions per wave (a chunk is 64 NB positions)
template <int D>
constexpr int attn_nb() { return D > 128 ? 1 : 3; }

struct AttnFns {
    void (*chunk)(AttnArgs, float*);
    void (*merge)(AttnArgs, const float*, int, int);
};

template <int D, int G>
AttnFns attn_fns() {
    return AttnFns{attn_chunk_kernel<D, G, attn_nb<D>()>, attn_merge_kernel<D, G>};
}

template <int D>
AttnFns attn_for_group(int g) {
    switch (g) {
    case 1: return attn_fns<D, 1>();
    case 2: return attn_fns<D, 2>();
    case 3: return attn_fns<D, 3>();
    case 4: return attn_fns<D, 4>();
    case 5: return attn_fns<D, 5>();
    case 6: return attn_fns<D, 6>();
    case 7: return attn_fns<D, 7>();
    case 8: return attn_fns<D, 8>();
    default: return AttnFns{nullptr, nullptr};
    }
}

int attn_chunk(int head_dim) { return head_dim > 128 ? 64 * attn_nb<256>() : 64 * attn_nb<128>(); }

}  // namespace

int64_t attention_workspace_floats(const AttnArgs& a) {
    const int64_t ch = attn_chunk(a.head_dim);
    const int64_t nchunks = (a.L + ch - 1) / ch;
    const int64_t g = a.nq / a.nkv;
    return a.B * a.nkv * nchunks * g * (a.head_dim + 2);
}

hipError_t launch_decode_attention(const AttnArgs& a, const Workspace& ws, hipStream_t s) {
    const int g = a.nq / a.nkv;
    AttnFns fn{nullptr, nullptr};
    switch (a.head_dim) {
    case 32: fn = attn_for_group<32>(g); break;
    case 64: fn = attn_for_group<64>(g); break;
    case 128: fn = attn_for_group<128>(g); break;
    case 256: fn = attn_for_group<256>(g); break;
    default: break;
    }
    if (fn.chunk == nullptr) return hipErrorInvalidValue;
    const int chunk = attn_chunk(a.head_dim);
    const int nchunks = (int)((a.L + chunk - 1) / chunk);
    hipLaunchKernelGGL(fn.chunk, dim3((unsigned)nchunks, (unsigned)a.nkv, (unsigned)a.B), dim3(kAttnThreads), 0, s,
                       a, ws.partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn.merge, dim3((unsigned)g, (unsigned)a.nkv, (unsigned)a.B), dim3((unsigned)a.head_dim), 0, s,
                       a, static_cast<const float*>(ws.partials), nchunks, chunk);
    return hipGetLastError();
}

}  // namespace tpk
