// Internal launch interface between the C ABI (abi.cpp) and the kernels.
// Every launcher assumes its arguments were validated by the ABI layer and
// returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tp_shard.h"

namespace tpk {

// Row map of a weight shard copy (tp_shard_weights): destination row i of the
// shard reads source row src_row(i) starting at column src_col0, or is zero.
struct ShardMap {
    int kind;
    int64_t dst_rows, dst_cols;    // shard shape
    int64_t src_rows, src_cols;    // full shape
    int64_t src_col0;              // first source column (row-split kinds)
    // QKV
    int32_t head_dim, q_first, q_count, kv_first, kv_count, num_q_heads, num_kv_heads;
    // GATE_UP
    int64_t inter, inter_shard, inter_first;
    // EMBED / LM_HEAD
    int64_t vocab_first, vocab;
};

hipError_t launch_shard_copy(const ShardMap& map, const void* full, void* shard, hipStream_t s);

hipError_t launch_swiglu(const void* gu, int64_t M, int64_t i_shard, void* out, hipStream_t s);

struct PartialPtrs { const void* p[TP_MAX_SHARDS]; };
hipError_t launch_reduce(const PartialPtrs& ptrs, int t, int64_t numel, int in_dtype,
                         void* out, int out_dtype, hipStream_t s);

hipError_t launch_vocab_embed(const int32_t* ids, int64_t M, const void* table, int64_t lo,
                              int64_t hi, int64_t H, void* out, hipStream_t s);

hipError_t launch_concat(const PartialPtrs& ptrs, int t, int64_t M, int64_t v_shard,
                         int64_t vocab, int dtype, void* out, hipStream_t s);

// Epilogue of a linear.
enum Epilogue : int {
    EPI_STORE = 0,    // y = acc (+ bias), out_dtype
    EPI_SWIGLU = 1,   // weight rows [gate (i_half); up (i_half)]; y[m, j] = silu(bf16(g)) * bf16(u), bf16
    EPI_REDUCE = 2,   // y = bf16(sum over t partials in order), own = bf16(acc) at position `rank`
    EPI_REDUCE_ADD = 3,   // as EPI_REDUCE, then y = bf16(y + that sum): y is the residual, in place
    // The same two with fp32 peers: the own partial enters the sum unrounded.
    EPI_REDUCE_F32 = 4,
    EPI_REDUCE_ADD_F32 = 5,
};
constexpr int kNumEpilogues = 6;
constexpr bool epi_is_reduce(int e) { return e >= EPI_REDUCE && e != EPI_SWIGLU; }
constexpr bool epi_is_add(int e) { return e == EPI_REDUCE_ADD || e == EPI_REDUCE_ADD_F32; }
constexpr bool epi_peers_f32(int e) { return e == EPI_REDUCE_F32 || e == EPI_REDUCE_ADD_F32; }

constexpr int kMaxFusedPeers = 16;   // t limit of the fused reduce epilogue
constexpr int kTiledReduceRanks = 2;  // t limit of the sum over ranks in the prefill kernel's epilogue

// Linear Y[M, N] = X[M, K] W[N, K]^T (+ bias[N]); out_dtype TP_BF16 / TP_F32.
// With EPI_SWIGLU, N is the kernel's row space (groups of gate rows paired
// with the same up rows, see the kernels), the weight holds 2 * i_half rows
// and y is [M, i_half]. With the reduce epilogues (decode kernel only,
// N % 4 == 0), y is [M, N] bf16 and peers[i] ([M, N] bf16, or fp32 for the
// _F32 epilogues; i != rank) are the other ranks' partials.
struct GemmArgs {
    const void* x;
    const void* w;
    const void* bias;   // bf16 [N] or nullptr
    void* y;
    int64_t M, N, K;
    int out_dtype;
    int epi;
    int64_t i_half;     // EPI_SWIGLU
    int t, rank;        // EPI_REDUCE, EPI_REDUCE_ADD
    // norm != 0: the RMSNorm of X's rows with gamma folded into W (decode
    // kernel, one tile of X in LDS): y = acc / sqrt(mean_k x^2 + eps).
    int norm;
    float eps;
    const void* peers[kMaxFusedPeers];
    // Prefill kernels only (0: the defaults). ldy: elements between output
    // rows (N, or i_half with SwiGLU); up_off: weight rows from a gate row to
    // its up row (i_half). Set when a launch covers a block of the weight
    // rows of a larger product.
    int64_t ldy = 0;
    int64_t up_off = 0;
};

// Caller-owned scratch (the C ABI's workspace argument): fp32 partial tiles
// and one arrival counter per output tile for K split across workgroups, the
// attention's chunk records. Counters must be zero before a launch; every
// kernel that uses them leaves them zero again.
struct Workspace {
    float* partials;
    int64_t partial_floats;
    unsigned* counters;
    int64_t num_counters;
};

// Plan of a decode-sized (M <= 64) linear; describes how K is split.
// Largest extent in bytes that a buffer resource addresses with 32-bit
// offsets: the prefill DMA kernels and the decode kernel's per-wave loads
// read through buffer resources, so their operands stay at or below it (the
// launchers pick other kernels beyond).
constexpr int64_t kMaxBufferBytes = 0xFFFFFFFFLL;

struct SkinnyPlan {
    int mt;          // token tiles of 16
    int ksteps;      // 32-wide k steps per wave
    int nwn;         // waves along N per workgroup (16 rows each)
    int nwk;         // waves along K per workgroup
    int xd;          // 1: X fragments loaded per wave from global; 0: X staged in LDS
    int splits;      // workgroups along K
    int64_t ntiles;  // workgroups along N
};

// The workspace size the planner's choices were measured with.
constexpr int64_t kSkinnyWsFloats = (int64_t)4 << 20;   // 16 MiB
constexpr int64_t kSkinnyWsCounters = 65536;

// ws_floats / ws_counters: the scratch floats and counters a K split may use
// (zero: keep K in one workgroup).
SkinnyPlan plan_skinny(int64_t M, int64_t N, int64_t K, int64_t ws_floats, int64_t ws_counters);
bool skinny_variant_exists(const SkinnyPlan& p);
bool skinny_plan_fits(const SkinnyPlan& p, int64_t M);   // LDS need for M tokens within limits
// The norm prologue's plan (splits == 0: no variant stages whole rows of K
// for M tokens; normalise separately) and its fit test.
SkinnyPlan plan_skinny_norm(int64_t M, int64_t N, int64_t K, int64_t ws_floats, int64_t ws_counters);
bool skinny_norm_plan_fits(const SkinnyPlan& p, int64_t M, int64_t K);
int64_t skinny_norm_ss_floats(const SkinnyPlan& p, int64_t M);
int64_t skinny_workspace_floats(const SkinnyPlan& p, int64_t M, int64_t N);
// Launches a decode-sized linear takes under plan p (2: the split partial
// tiles, then their sum and the epilogue).
int skinny_split_launches(const SkinnyPlan& p, const GemmArgs& a);
hipError_t launch_skinny(const GemmArgs& a, const SkinnyPlan& p, const Workspace& ws, hipStream_t s);

// EPI_STORE or EPI_SWIGLU (a.N = 2 i_half). variant: a kernel index in
// [0, tiled_variant_count()), or -1 for the automatic choice; one whose K
// multiple the call does not meet is replaced by the automatic choice.
// Whether a decode-sized linear (M <= 64) runs faster on the tiled kernel's
// 64 x 64 tiles than on the decode kernel (store or SwiGLU epilogue only).
bool tiled_wins_at_decode(const GemmArgs& a);
hipError_t launch_tiled(const GemmArgs& a, hipStream_t s, int variant = -1);
int tiled_variant_count();

}  // namespace tpk
