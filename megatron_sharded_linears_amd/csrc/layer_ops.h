// Internal launch interface of the layer operations around the linears: the
// residual add + RMSNorm (memops.hip) and the decode attention
// (attention.hip). As in kernels.h, arguments are validated by the ABI layer
// and each launcher returns the hipError_t of its launch.
#pragma once

#include "kernels.h"

namespace tpk {

// residual[m] = bf16(residual[m] + bf16(sum of the t partials' row m)) (t = 0:
// unchanged), out[m] = bf16(residual[m] * rsqrt-scale * gamma); one workgroup
// per row, M <= 2^31 - 1, H % 8 == 0, H <= 32768. out == nullptr: the
// residual update only; gamma == nullptr: unit weights.
// w_out[n, k] = bf16(w[n, k] * gamma[k]) for [N, K] bf16 (K % 8 == 0; may be in place).
hipError_t launch_fold_norm_weight(const void* w, int64_t N, int64_t K, const void* gamma, void* out, hipStream_t s);

hipError_t launch_add_rmsnorm(const PartialPtrs& ptrs, int t, int in_dtype, int64_t M, int64_t H,
                              void* residual, const void* gamma, float eps, void* out, hipStream_t s);

// One decode step of a rank's GQA attention. qkv: [B, (nq + 2 nkv) head_dim]
// bf16 rows [Q heads | K heads | V heads]; caches [B, nkv, L, head_dim] bf16;
// lens: [B] int32 on the device; ctx: [B, nq head_dim] bf16.
struct AttnArgs {
    const uint16_t* qkv;
    uint16_t* k_cache;
    uint16_t* v_cache;
    const int32_t* lens;
    uint16_t* ctx;
    int64_t B, L;
    int nq, nkv, head_dim;
    int64_t qkv_stride;   // elements per qkv row
    float scale;          // 1 / sqrt(head_dim)
};
constexpr int64_t kAttnMaxLen = 32768;   // cache positions per sequence
// floats of the per-chunk records (the chunk kernel writes, the merge reads)
int64_t attention_workspace_floats(const AttnArgs& a);
hipError_t launch_decode_attention(const AttnArgs& a, const Workspace& ws, hipStream_t s);

}  // namespace tpk
