// C ABI of libtpshard: host-side validation, shape queries, workspace
// management and dispatch to the gfx950 kernels. Every entry point checks its
// arguments before making any HIP call, so argument errors are reported (and
// testable) without a GPU. No C++ exception escapes: each entry point catches
// everything and maps it to a tp_status.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "kernels.h"
#include "layer_ops.h"
#include "tp_shard.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;   // sizes must fit the kernels' int ranges
constexpr int64_t kSkinnyMaxM = 64;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(int d) { return d == TP_BF16 || d == TP_F32; }

int check_cfg(const tp_model_cfg* c, int t) {
    if (c == nullptr) return TP_ERR_NULL;
    if (t < 1 || t > TP_MAX_SHARDS) return TP_ERR_RANGE;
    if (c->hidden <= 0 || c->num_q_heads <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0 ||
        c->intermediate <= 0 || c->vocab <= 0)
        return TP_ERR_SHAPE;
    if (c->num_kv_heads > c->num_q_heads || c->num_q_heads % c->num_kv_heads != 0) return TP_ERR_SHAPE;
    if (c->num_q_heads % t != 0) return TP_ERR_DIVISIBILITY;
    if (c->num_kv_heads >= t) {
        if (c->num_kv_heads % t != 0) return TP_ERR_DIVISIBILITY;
    } else if (t % c->num_kv_heads != 0) {
        return TP_ERR_DIVISIBILITY;
    }
    if (c->intermediate % t != 0) return TP_ERR_DIVISIBILITY;
    return TP_OK;
}

void kv_of_rank(const tp_model_cfg* c, int t, int rank, int* first, int* count) {
    if (c->num_kv_heads >= t) {
        *count = c->num_kv_heads / t;
        *first = rank * *count;
    } else {
        *count = 1;
        *first = rank / (t / c->num_kv_heads);
    }
}

// --------------------------------------------------------------- workspace

constexpr int64_t kWsFloats = tpk::kSkinnyWsFloats;
constexpr int64_t kWsCounters = tpk::kSkinnyWsCounters;

struct StreamWs {
    float* partials = nullptr;
    unsigned* counters = nullptr;
};

std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, StreamWs> g_ws;

int get_workspace(hipStream_t s, tpk::Workspace* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TP_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_ws_mu);
    StreamWs& w = g_ws[std::make_pair(dev, s)];
    if (w.partials == nullptr) {
        void* p = nullptr;
        void* c = nullptr;
        if (hipMalloc(&p, kWsFloats * sizeof(float)) != hipSuccess) return TP_ERR_ALLOC;
        if (hipMalloc(&c, kWsCounters * sizeof(unsigned)) != hipSuccess) {
            (void)hipFree(p);
            return TP_ERR_ALLOC;
        }
        if (hipMemset(c, 0, kWsCounters * sizeof(unsigned)) != hipSuccess) {
            (void)hipFree(p);
            (void)hipFree(c);
            return TP_ERR_HIP;
        }
        w.partials = static_cast<float*>(p);
        w.counters = static_cast<unsigned*>(c);
    }
    out->partials = w.partials;
    out->partial_floats = kWsFloats;
    out->counters = w.counters;
    out->num_counters = kWsCounters;
    return TP_OK;
}

// A process-wide override of the decode kernel's shape, for tuning and for
// tests that exercise every variant. Zero means automatic.
int g_force_ksteps = 0, g_force_nwn = 0, g_force_nwk = 0, g_force_xd = 0;

// Launch one validated linear. a.N is the kernel's row space (for EPI_SWIGLU
// on the decode kernel: 16-row blocks of 8 gate and 8 up rows).
// ws_limit: floats of the stream workspace's front a split-K plan may use
// (the rest may hold an operand the caller staged at the back).
int launch_linear(const tpk::GemmArgs& a, hipStream_t s, int64_t ws_limit = kWsFloats) {
    const int64_t M = a.M, N = a.N, K = a.K;
    hipError_t e;
    if (M <= kSkinnyMaxM) {
        tpk::SkinnyPlan p = tpk::plan_skinny(M, N, K, ws_limit);
        if (p.splits < 1) return TP_ERR_SHAPE;        // no variant's partials fit the workspace
        if (g_force_ksteps > 0) {
            tpk::SkinnyPlan f = p;
            f.ksteps = g_force_ksteps;
            f.nwn = g_force_nwn;
            f.nwk = g_force_nwk;
            f.xd = g_force_xd;
            f.ntiles = (N + 16LL * f.nwn - 1) / (16LL * f.nwn);
            const int64_t gk = 32LL * f.ksteps * f.nwk;
            f.splits = (int)((K + gk - 1) / gk);
            // a forced shape that does not fit this M (LDS) or the workspace
            // keeps the automatic plan
            const bool fits = f.splits == 1 || (tpk::skinny_workspace_floats(f, M, N) <= ws_limit &&
                                                f.ntiles <= kWsCounters && f.splits <= 65535);
            if (tpk::skinny_variant_exists(f) && tpk::skinny_plan_fits(f, M) && fits) p = f;
        }
        tpk::Workspace ws{nullptr, 0, nullptr, 0};
        if (p.splits > 1) {
            const int st = get_workspace(s, &ws);
            if (st != TP_OK) return st;
            if (tpk::skinny_workspace_floats(p, M, N) > std::min(ws.partial_floats, ws_limit) ||
                p.ntiles > ws.num_counters)
                return TP_ERR_SHAPE;
        }
        e = tpk::launch_skinny(a, p, ws, s);
    } else {
        e = tpk::launch_tiled(a, s);
    }
    return e == hipSuccess ? TP_OK : TP_ERR_HIP;
}

int check_linear(const void* x, int64_t M, int64_t K, const void* w, int64_t N, const void* y) {
    if (x == nullptr || w == nullptr || y == nullptr) return TP_ERR_NULL;
    if (M < 0 || N <= 0 || K <= 0 || M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return TP_ERR_SHAPE;
    if (K % 8 != 0) return TP_ERR_ALIGNMENT;
    if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return TP_ERR_ALIGNMENT;
    return TP_OK;
}

int run_linear(const void* x, int64_t M, int64_t K, const void* w, int64_t N, const void* bias,
               void* y, int out_dtype, void* stream) {
    const int st = check_linear(x, M, K, w, N, y);
    if (st != TP_OK) return st;
    if (!dtype_ok(out_dtype)) return TP_ERR_DTYPE;
    if (bias != nullptr && (reinterpret_cast<uintptr_t>(bias) & 1u)) return TP_ERR_ALIGNMENT;
    if (M == 0) return TP_OK;
    tpk::GemmArgs a{};
    a.x = x; a.w = w; a.bias = bias; a.y = y;
    a.M = M; a.N = N; a.K = K;
    a.out_dtype = out_dtype;
    a.epi = tpk::EPI_STORE;
    return launch_linear(a, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

const char* tp_status_string(int status) {
    switch (status) {
    case TP_OK: return "ok";
    case TP_ERR_NULL: return "a required pointer is NULL";
    case TP_ERR_SHAPE: return "negative, inconsistent or too large sizes";
    case TP_ERR_DIVISIBILITY: return "a tensor-parallel split rule does not hold (n_h % t, n_kv vs t, I % t)";
    case TP_ERR_ALIGNMENT: return "pointer not 16-byte aligned or a size not a multiple of 8";
    case TP_ERR_DTYPE: return "unknown dtype or weight kind";
    case TP_ERR_RANGE: return "t outside [1, 64] or rank outside [0, t)";
    case TP_ERR_HIP: return "the HIP runtime reported an error";
    case TP_ERR_ALLOC: return "workspace allocation failed";
    default: return "unknown status";
    }
}

int tp_full_shape(const tp_model_cfg* cfg, int kind, int64_t* rows, int64_t* cols) {
    if (cfg == nullptr || rows == nullptr || cols == nullptr) return TP_ERR_NULL;
    const int st = check_cfg(cfg, 1);
    if (st != TP_OK) return st;
    const int64_t H = cfg->hidden, d = cfg->head_dim;
    switch (kind) {
    case TP_W_QKV: *rows = ((int64_t)cfg->num_q_heads + 2LL * cfg->num_kv_heads) * d; *cols = H; break;
    case TP_W_O: *rows = H; *cols = (int64_t)cfg->num_q_heads * d; break;
    case TP_W_GATE_UP: *rows = 2LL * cfg->intermediate; *cols = H; break;
    case TP_W_DOWN: *rows = H; *cols = cfg->intermediate; break;
    case TP_W_EMBED:
    case TP_W_LM_HEAD: *rows = cfg->vocab; *cols = H; break;
    default: return TP_ERR_DTYPE;
    }
    return TP_OK;
}

int64_t tp_vocab_shard_rows(int64_t vocab, int t) {
    if (t < 1 || t > TP_MAX_SHARDS) return TP_ERR_RANGE;
    if (vocab <= 0) return TP_ERR_SHAPE;
    return (vocab + t - 1) / t;
}

int tp_shard_shape(const tp_model_cfg* cfg, int t, int kind, int64_t* rows, int64_t* cols) {
    if (cfg == nullptr || rows == nullptr || cols == nullptr) return TP_ERR_NULL;
    const int st = check_cfg(cfg, t);
    if (st != TP_OK) return st;
    const int64_t H = cfg->hidden, d = cfg->head_dim;
    int kv_first = 0, kv_count = 0;
    kv_of_rank(cfg, t, 0, &kv_first, &kv_count);
    switch (kind) {
    case TP_W_QKV: *rows = ((int64_t)cfg->num_q_heads / t + 2LL * kv_count) * d; *cols = H; break;
    case TP_W_O: *rows = H; *cols = (int64_t)cfg->num_q_heads / t * d; break;
    case TP_W_GATE_UP: *rows = 2LL * cfg->intermediate / t; *cols = H; break;
    case TP_W_DOWN: *rows = H; *cols = cfg->intermediate / t; break;
    case TP_W_EMBED:
    case TP_W_LM_HEAD: *rows = tp_vocab_shard_rows(cfg->vocab, t); *cols = H; break;
    default: return TP_ERR_DTYPE;
    }
    return TP_OK;
}

int tp_kv_heads_of_rank(const tp_model_cfg* cfg, int t, int rank, int* first, int* count) {
    if (cfg == nullptr || first == nullptr || count == nullptr) return TP_ERR_NULL;
    const int st = check_cfg(cfg, t);
    if (st != TP_OK) return st;
    if (rank < 0 || rank >= t) return TP_ERR_RANGE;
    kv_of_rank(cfg, t, rank, first, count);
    return TP_OK;
}

int tp_shard_weights(const tp_model_cfg* cfg, int t, int rank, int kind, const void* full_w,
                     void* shard_w, void* stream) {
    try {
        if (cfg == nullptr || full_w == nullptr || shard_w == nullptr) return TP_ERR_NULL;
        int st = check_cfg(cfg, t);
        if (st != TP_OK) return st;
        if (rank < 0 || rank >= t) return TP_ERR_RANGE;
        tpk::ShardMap m;
        std::memset(&m, 0, sizeof(m));
        m.kind = kind;
        st = tp_full_shape(cfg, kind, &m.src_rows, &m.src_cols);
        if (st != TP_OK) return st;
        st = tp_shard_shape(cfg, t, kind, &m.dst_rows, &m.dst_cols);
        if (st != TP_OK) return st;
        if (m.src_cols % 8 != 0 || m.dst_cols % 8 != 0) return TP_ERR_ALIGNMENT;
        if (!aligned16(full_w) || !aligned16(shard_w)) return TP_ERR_ALIGNMENT;
        if (m.src_rows * m.src_cols >= ((int64_t)1 << 40)) return TP_ERR_SHAPE;
        switch (kind) {
        case TP_W_QKV: {
            m.head_dim = cfg->head_dim;
            m.num_q_heads = cfg->num_q_heads;
            m.num_kv_heads = cfg->num_kv_heads;
            m.q_count = cfg->num_q_heads / t;
            m.q_first = rank * m.q_count;
            int f = 0, c = 0;
            kv_of_rank(cfg, t, rank, &f, &c);
            m.kv_first = f;
            m.kv_count = c;
            break;
        }
        case TP_W_GATE_UP:
            m.inter = cfg->intermediate;
            m.inter_shard = cfg->intermediate / t;
            m.inter_first = (int64_t)rank * m.inter_shard;
            break;
        case TP_W_O:
        case TP_W_DOWN:
            m.src_col0 = (int64_t)rank * m.dst_cols;
            break;
        case TP_W_EMBED:
        case TP_W_LM_HEAD:
            m.vocab = cfg->vocab;
            m.vocab_first = (int64_t)rank * m.dst_rows;
            break;
        default:
            return TP_ERR_DTYPE;
        }
        const hipError_t e = tpk::launch_shard_copy(m, full_w, shard_w, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? TP_OK : TP_ERR_HIP;
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_column_linear(const void* x, int64_t M, int64_t K, const void* w_shard, int64_t N,
                     const void* bias_or_null, void* y, void* stream) {
    try {
        return run_linear(x, M, K, w_shard, N, bias_or_null, y, TP_BF16, stream);
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_row_linear_partial(const void* x_shard, int64_t M, int64_t K_shard, const void* w_shard,
                          int64_t N, void* partial, int partial_dtype, void* stream) {
    try {
        return run_linear(x_shard, M, K_shard, w_shard, N, nullptr, partial, partial_dtype, stream);
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_lm_head_shard(const void* h, int64_t M, int64_t K, const void* w_lm_shard, int64_t v_shard,
                     void* logits_shard, int out_dtype, void* stream) {
    try {
        return run_linear(h, M, K, w_lm_shard, v_shard, nullptr, logits_shard, out_dtype, stream);
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_column_linear_swiglu(const void* x, int64_t M, int64_t K, const void* w_gate_up, int64_t i_shard,
                            void* act, void* stream) {
    try {
        if (i_shard <= 0 || i_shard >= kMaxDim / 2) return TP_ERR_SHAPE;
        const int st = check_linear(x, M, K, w_gate_up, 2 * i_shard, act);
        if (st != TP_OK) return st;
        if (M == 0) return TP_OK;
        tpk::GemmArgs a{};
        a.x = x; a.w = w_gate_up; a.y = act;
        a.M = M; a.K = K;
        a.out_dtype = TP_BF16;
        a.epi = tpk::EPI_SWIGLU;
        a.i_half = i_shard;
        // decode kernel: 16-row blocks of 8 gate + 8 up rows; tiled kernel:
        // 2 i_shard here, whole tiles of paired rows inside the launcher
        a.N = M <= kSkinnyMaxM ? 16 * ((i_shard + 7) / 8) : 2 * i_shard;
        return launch_linear(a, static_cast<hipStream_t>(stream));
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_row_linear_reduce(const void* x_shard, int64_t M, int64_t K_shard, const void* w_shard, int64_t N,
                         const void* const* partials, int t, int rank, void* out, void* stream) {
    try {
        const int st = check_linear(x_shard, M, K_shard, w_shard, N, out);
        if (st != TP_OK) return st;
        if (partials == nullptr) return TP_ERR_NULL;
        if (t < 1 || t > TP_MAX_SHARDS || rank < 0 || rank >= t) return TP_ERR_RANGE;
        for (int i = 0; i < t; ++i) {
            if (i == rank) continue;
            if (partials[i] == nullptr) return TP_ERR_NULL;
            if (!aligned16(partials[i])) return TP_ERR_ALIGNMENT;
            if (partials[i] == out) return TP_ERR_SHAPE;
        }
        if (M == 0) return TP_OK;
        hipStream_t s = static_cast<hipStream_t>(stream);
        tpk::GemmArgs a{};
        a.x = x_shard; a.w = w_shard; a.y = out;
        a.M = M; a.N = N; a.K = K_shard;
        a.out_dtype = TP_BF16;
        if (M <= kSkinnyMaxM && t <= tpk::kMaxFusedPeers && N % 4 == 0) {
            a.epi = tpk::EPI_REDUCE;
            a.t = t;
            a.rank = rank;
            for (int i = 0; i < t; ++i) a.peers[i] = i == rank ? nullptr : partials[i];
            return launch_linear(a, s);
        }
        // Two launches with the same arithmetic: the rank's bf16 partial is
        // written to `out`, then summed in place with the others in rank order.
        a.epi = tpk::EPI_STORE;
        const int st2 = launch_linear(a, s);
        if (st2 != TP_OK) return st2;
        tpk::PartialPtrs ptrs;
        std::memset(&ptrs, 0, sizeof(ptrs));
        for (int i = 0; i < t; ++i) ptrs.p[i] = i == rank ? out : partials[i];
        const hipError_t e = tpk::launch_reduce(ptrs, t, M * N, TP_BF16, out, TP_BF16, s);
        return e == hipSuccess ? TP_OK : TP_ERR_HIP;
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_swiglu(const void* gu, int64_t M, int64_t i_shard, void* out, void* stream) {
    try {
        if (gu == nullptr || out == nullptr) return TP_ERR_NULL;
        if (M < 0 || i_shard <= 0 || M >= kMaxDim || i_shard >= kMaxDim) return TP_ERR_SHAPE;
        if (i_shard % 8 != 0 || !aligned16(gu) || !aligned16(out)) return TP_ERR_ALIGNMENT;
        if (M == 0) return TP_OK;
        const hipError_t e = tpk::launch_swiglu(gu, M, i_shard, out, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? TP_OK : TP_ERR_HIP;
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_reduce_partials(const void* const* partials, int t, int64_t numel, int in_dtype, void* out,
                       int out_dtype, void* stream) {
    try {
        if (partials == nullptr || out == nullptr) return TP_ERR_NULL;
        if (t < 1 || t > TP_MAX_SHARDS) return TP_ERR_RANGE;
        if (numel < 0) return TP_ERR_SHAPE;
        if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return TP_ERR_DTYPE;
        tpk::PartialPtrs ptrs;
        std::memset(&ptrs, 0, sizeof(ptrs));
        for (int i = 0; i < t; ++i) {
            if (partials[i] == nullptr) return TP_ERR_NULL;
            if (!aligned16(partials[i])) return TP_ERR_ALIGNMENT;
            ptrs.p[i] = partials[i];
        }
        if (!aligned16(out)) return TP_ERR_ALIGNMENT;
        if (numel == 0) return TP_OK;
        const hipError_t e = tpk::launch_reduce(ptrs, t, numel, in_dtype, out, out_dtype,
                                                static_cast<hipStream_t>(stream));
        return e == hipSuccess ? TP_OK : TP_ERR_HIP;
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_vocab_embed(const int32_t* ids, int64_t M, const void* e_shard, int64_t vocab, int t, int rank,
                   int64_t H, void* out_partial, void* stream) {
    try {
        if (ids == nullptr || e_shard == nullptr || out_partial == nullptr) return TP_ERR_NULL;
        if (t < 1 || t > TP_MAX_SHARDS || rank < 0 || rank >= t) return TP_ERR_RANGE;
        if (M < 0 || vocab <= 0 || H <= 0 || M >= kMaxDim || vocab >= kMaxDim || H >= kMaxDim) return TP_ERR_SHAPE;
        if (H % 8 != 0 || !aligned16(e_shard) || !aligned16(out_partial) ||
            (reinterpret_cast<uintptr_t>(ids) & 3u))
            return TP_ERR_ALIGNMENT;
        if (M == 0) return TP_OK;
        const int64_t vs = (vocab + t - 1) / t;
        const int64_t lo = (int64_t)rank * vs;
        const int64_t hi = lo + vs < vocab ? lo + vs : vocab;
        const hipError_t e = tpk::launch_vocab_embed(ids, M, e_shard, lo, hi, H, out_partial,
                                                     static_cast<hipStream_t>(stream));
        return e == hipSuccess ? TP_OK : TP_ERR_HIP;
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_concat_logits(const void* const* shard_logits, int t, int64_t M, int64_t v_shard, int64_t vocab,
                     int dtype, void* out, void* stream) {
    try {
        if (shard_logits == nullptr || out == nullptr) return TP_ERR_NULL;
        if (t < 1 || t > TP_MAX_SHARDS) return TP_ERR_RANGE;
        if (!dtype_ok(dtype)) return TP_ERR_DTYPE;
        if (M < 0 || vocab <= 0 || M >= kMaxDim || vocab >= kMaxDim) return TP_ERR_SHAPE;
        if (v_shard != (vocab + t - 1) / t) return TP_ERR_SHAPE;
        tpk::PartialPtrs ptrs;
        std::memset(&ptrs, 0, sizeof(ptrs));
        for (int i = 0; i < t; ++i) {
            if (shard_logits[i] == nullptr) return TP_ERR_NULL;
            if (!aligned16(shard_logits[i])) return TP_ERR_ALIGNMENT;
            ptrs.p[i] = shard_logits[i];
        }
        if (!aligned16(out)) return TP_ERR_ALIGNMENT;
        if (M == 0) return TP_OK;
        const hipError_t e = tpk::launch_concat(ptrs, t, M, v_shard, vocab, dtype, out,
                                                static_cast<hipStream_t>(stream));
        return e == hipSuccess ? TP_OK : TP_ERR_HIP;
    } catch (...) {
        return TP_ERR_HIP;
    }
}

namespace {

constexpr int64_t kMaxNormWidth = 32768;   // one workgroup holds a whole row in registers

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

// Shared validation of the two add + RMSNorm calls; `inputs` are t buffers
// of M x H elements of in_dtype (t may be 0).
int add_rmsnorm_call(const void* const* inputs, int t, int in_dtype, int64_t M, int64_t H, void* residual,
                     const void* gamma, float eps, void* out, void* stream) {
    if (residual == nullptr || gamma == nullptr || out == nullptr) return TP_ERR_NULL;
    if (t < 0 || t > TP_MAX_SHARDS) return TP_ERR_RANGE;
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return TP_ERR_RANGE;
    if (!dtype_ok(in_dtype)) return TP_ERR_DTYPE;
    if (M < 0 || H <= 0 || M >= kMaxDim || H > kMaxNormWidth) return TP_ERR_SHAPE;
    if (H % 8 != 0 || !aligned16(residual) || !aligned16(gamma) || !aligned16(out)) return TP_ERR_ALIGNMENT;
    const int64_t act_bytes = M * H * 2, in_bytes = M * H * (in_dtype == TP_F32 ? 4 : 2);
    if (overlap(out, act_bytes, residual, act_bytes) || overlap(out, act_bytes, gamma, H * 2) ||
        overlap(residual, act_bytes, gamma, H * 2))
        return TP_ERR_SHAPE;
    tpk::PartialPtrs ptrs;
    std::memset(&ptrs, 0, sizeof(ptrs));
    for (int i = 0; i < t; ++i) {
        if (inputs[i] == nullptr) return TP_ERR_NULL;
        if (!aligned16(inputs[i])) return TP_ERR_ALIGNMENT;
        if (overlap(inputs[i], in_bytes, out, act_bytes) || overlap(inputs[i], in_bytes, residual, act_bytes))
            return TP_ERR_SHAPE;
        ptrs.p[i] = inputs[i];
    }
    if (M == 0) return TP_OK;
    const hipError_t e = tpk::launch_add_rmsnorm(ptrs, t, in_dtype, M, H, residual, gamma, eps, out,
                                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TP_OK : TP_ERR_HIP;
}

}  // namespace

int tp_add_rmsnorm(const void* x_or_null, int64_t M, int64_t H, void* residual, const void* gamma, float eps,
                   void* out, void* stream) {
    try {
        const void* in[1] = {x_or_null};
        return add_rmsnorm_call(in, x_or_null != nullptr ? 1 : 0, TP_BF16, M, H, residual, gamma, eps, out, stream);
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_reduce_add_rmsnorm(const void* const* partials, int t, int partial_dtype, int64_t M, int64_t H,
                          void* residual, const void* gamma, float eps, void* out, void* stream) {
    try {
        if (partials == nullptr) return TP_ERR_NULL;
        if (t < 1) return TP_ERR_RANGE;
        return add_rmsnorm_call(partials, t, partial_dtype, M, H, residual, gamma, eps, out, stream);
    } catch (...) {
        return TP_ERR_HIP;
    }
}

namespace {

// The back `bytes` of the stream workspace (whole 256-byte units) for an
// operand a fused call's two-launch path stages; *front is what stays free
// for the linear's own split-K partials.
int workspace_back(hipStream_t s, int64_t bytes, void** out, int64_t* front) {
    tpk::Workspace ws{nullptr, 0, nullptr, 0};
    const int st = get_workspace(s, &ws);
    if (st != TP_OK) return st;
    const int64_t need = (bytes + 255) / 256 * 256;
    if (need > ws.partial_floats * 4) return TP_ERR_SHAPE;
    *out = reinterpret_cast<char*>(ws.partials) + (ws.partial_floats * 4 - need);
    *front = ws.partial_floats - need / 4;
    return TP_OK;
}

// The linear a describes on RMS-normalised rows of a.x (unit weights: the
// norm's gamma is folded into a.w). One launch when the decode kernel can
// stage whole rows; otherwise the norm writes the normalised rows to the
// workspace and the plain linear reads them.
int run_norm_linear(tpk::GemmArgs a, hipStream_t s) {
    if (a.M <= kSkinnyMaxM) {
        const tpk::SkinnyPlan p = tpk::plan_skinny_norm(a.M, a.N, a.K);
        if (p.splits >= 1) {
            tpk::Workspace ws{nullptr, 0, nullptr, 0};
            if (p.splits > 1) {
                // partial tiles, then each split's share of the rows' sums of squares
                const int st = get_workspace(s, &ws);
                if (st != TP_OK) return st;
                if (tpk::skinny_workspace_floats(p, a.M, a.N) + (int64_t)p.splits * p.ntiles * 16 > ws.partial_floats ||
                    p.ntiles > ws.num_counters)
                    return TP_ERR_SHAPE;
            }
            const hipError_t e = tpk::launch_skinny(a, p, ws, s);
            return e == hipSuccess ? TP_OK : TP_ERR_HIP;
        }
    }
    void* xn = nullptr;
    int64_t front = 0;
    const int st = workspace_back(s, a.M * a.K * 2, &xn, &front);
    if (st != TP_OK) return st;
    tpk::PartialPtrs none;
    std::memset(&none, 0, sizeof(none));
    const hipError_t e = tpk::launch_add_rmsnorm(none, 0, TP_BF16, a.M, a.K, const_cast<void*>(a.x), nullptr, a.eps,
                                                 xn, s);
    if (e != hipSuccess) return TP_ERR_HIP;
    a.x = xn;
    a.norm = 0;
    return launch_linear(a, s, front);
}

int check_norm_input(const void* h, int64_t K, float eps, const void* y, int64_t M, int64_t n_bytes) {
    if (!(eps >= 0.0f) || !std::isfinite(eps)) return TP_ERR_RANGE;
    if (K > kMaxNormWidth) return TP_ERR_SHAPE;
    if (overlap(y, n_bytes, h, M * K * 2)) return TP_ERR_SHAPE;
    return TP_OK;
}

}  // namespace

int tp_fold_norm_weight(const void* w, int64_t N, int64_t K, const void* gamma, void* w_folded, void* stream) {
    try {
        if (w == nullptr || gamma == nullptr || w_folded == nullptr) return TP_ERR_NULL;
        if (N <= 0 || K <= 0 || N >= kMaxDim || K >= kMaxDim) return TP_ERR_SHAPE;
        if (K % 8 != 0 || !aligned16(w) || !aligned16(gamma) || !aligned16(w_folded)) return TP_ERR_ALIGNMENT;
        const int64_t bytes = N * K * 2;
        if ((w_folded != w && overlap(w_folded, bytes, w, bytes)) || overlap(w_folded, bytes, gamma, K * 2))
            return TP_ERR_SHAPE;
        const hipError_t e = tpk::launch_fold_norm_weight(w, N, K, gamma, w_folded, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? TP_OK : TP_ERR_HIP;
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_rmsnorm_column_linear(const void* h, float eps, int64_t M, int64_t K, const void* w_folded, int64_t N,
                             const void* bias_or_null, void* y, void* stream) {
    try {
        const void* w_shard = w_folded;
        int st = check_linear(h, M, K, w_shard, N, y);
        if (st != TP_OK) return st;
        st = check_norm_input(h, K, eps, y, M, M * N * 2);
        if (st != TP_OK) return st;
        if (bias_or_null != nullptr && (reinterpret_cast<uintptr_t>(bias_or_null) & 1u)) return TP_ERR_ALIGNMENT;
        if (M == 0) return TP_OK;
        tpk::GemmArgs a{};
        a.x = h; a.w = w_shard; a.bias = bias_or_null; a.y = y;
        a.M = M; a.N = N; a.K = K;
        a.out_dtype = TP_BF16;
        a.epi = tpk::EPI_STORE;
        a.norm = 1;
        a.eps = eps;
        return run_norm_linear(a, static_cast<hipStream_t>(stream));
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_rmsnorm_column_linear_swiglu(const void* h, float eps, int64_t M, int64_t K, const void* w_gate_up_folded,
                                    int64_t i_shard, void* act, void* stream) {
    try {
        const void* w_gate_up = w_gate_up_folded;
        if (i_shard <= 0 || i_shard >= kMaxDim / 2) return TP_ERR_SHAPE;
        int st = check_linear(h, M, K, w_gate_up, 2 * i_shard, act);
        if (st != TP_OK) return st;
        st = check_norm_input(h, K, eps, act, M, M * i_shard * 2);
        if (st != TP_OK) return st;
        if (M == 0) return TP_OK;
        tpk::GemmArgs a{};
        a.x = h; a.w = w_gate_up; a.y = act;
        a.M = M; a.K = K;
        a.out_dtype = TP_BF16;
        a.epi = tpk::EPI_SWIGLU;
        a.i_half = i_shard;
        a.N = M <= kSkinnyMaxM ? 16 * ((i_shard + 7) / 8) : 2 * i_shard;
        a.norm = 1;
        a.eps = eps;
        return run_norm_linear(a, static_cast<hipStream_t>(stream));
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_row_linear_reduce_add(const void* x_shard, int64_t M, int64_t K_shard, const void* w_shard, int64_t N,
                             const void* const* partials, int t, int rank, void* residual, void* stream) {
    try {
        const int st = check_linear(x_shard, M, K_shard, w_shard, N, residual);
        if (st != TP_OK) return st;
        if (partials == nullptr) return TP_ERR_NULL;
        if (t < 1 || t > TP_MAX_SHARDS || rank < 0 || rank >= t) return TP_ERR_RANGE;
        const int64_t bytes = M * N * 2;
        for (int i = 0; i < t; ++i) {
            if (i == rank) continue;
            if (partials[i] == nullptr) return TP_ERR_NULL;
            if (!aligned16(partials[i])) return TP_ERR_ALIGNMENT;
            if (overlap(partials[i], bytes, residual, bytes)) return TP_ERR_SHAPE;
        }
        if (overlap(x_shard, M * K_shard * 2, residual, bytes)) return TP_ERR_SHAPE;
        if (M == 0) return TP_OK;
        hipStream_t s = static_cast<hipStream_t>(stream);
        tpk::GemmArgs a{};
        a.x = x_shard; a.w = w_shard; a.y = residual;
        a.M = M; a.N = N; a.K = K_shard;
        a.out_dtype = TP_BF16;
        if (M <= kSkinnyMaxM && t <= tpk::kMaxFusedPeers && N % 4 == 0) {
            a.epi = tpk::EPI_REDUCE_ADD;
            a.t = t;
            a.rank = rank;
            for (int i = 0; i < t; ++i) a.peers[i] = i == rank ? nullptr : partials[i];
            return launch_linear(a, s);
        }
        // Two launches with the same arithmetic: the rank's bf16 partial goes
        // to the back of the workspace, then the sum over ranks in order is
        // added to the residual (the add + norm kernel without its norm).
        if (N % 8 != 0 || N > kMaxNormWidth) return TP_ERR_SHAPE;
        void* own = nullptr;
        int64_t front = 0;
        const int st2 = workspace_back(s, bytes, &own, &front);
        if (st2 != TP_OK) return st2;
        a.y = own;
        a.epi = tpk::EPI_STORE;
        const int st3 = launch_linear(a, s, front);
        if (st3 != TP_OK) return st3;
        tpk::PartialPtrs ptrs;
        std::memset(&ptrs, 0, sizeof(ptrs));
        for (int i = 0; i < t; ++i) ptrs.p[i] = i == rank ? own : partials[i];
        const hipError_t e = tpk::launch_add_rmsnorm(ptrs, t, TP_BF16, M, N, residual, nullptr, 0.0f, nullptr, s);
        return e == hipSuccess ? TP_OK : TP_ERR_HIP;
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_decode_attention(const void* qkv, int64_t B, int nq, int nkv, int head_dim, void* k_cache, void* v_cache,
                        int64_t L, const int32_t* lens, void* ctx, void* stream) {
    try {
        if (qkv == nullptr || k_cache == nullptr || v_cache == nullptr || lens == nullptr || ctx == nullptr)
            return TP_ERR_NULL;
        if (B < 0 || B > 65535 || L < 1 || L > tpk::kAttnMaxLen) return TP_ERR_SHAPE;
        if (nq < 1 || nkv < 1 || nkv > 65535 || nq % nkv != 0 || nq / nkv > 8) return TP_ERR_SHAPE;
        if (head_dim != 32 && head_dim != 64 && head_dim != 128 && head_dim != 256) return TP_ERR_SHAPE;
        if (!aligned16(qkv) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(ctx) ||
            (reinterpret_cast<uintptr_t>(lens) & 3u))
            return TP_ERR_ALIGNMENT;
        const int64_t qkv_row = (int64_t)(nq + 2 * nkv) * head_dim;
        const int64_t qkv_bytes = B * qkv_row * 2, cache_bytes = B * nkv * L * head_dim * 2,
                      ctx_bytes = B * nq * head_dim * 2;
        if (overlap(ctx, ctx_bytes, qkv, qkv_bytes) || overlap(ctx, ctx_bytes, k_cache, cache_bytes) ||
            overlap(ctx, ctx_bytes, v_cache, cache_bytes) || overlap(k_cache, cache_bytes, v_cache, cache_bytes) ||
            overlap(qkv, qkv_bytes, k_cache, cache_bytes) || overlap(qkv, qkv_bytes, v_cache, cache_bytes) ||
            overlap(lens, B * 4, ctx, ctx_bytes) || overlap(lens, B * 4, k_cache, cache_bytes) ||
            overlap(lens, B * 4, v_cache, cache_bytes))
            return TP_ERR_SHAPE;
        if (B == 0) return TP_OK;
        tpk::AttnArgs a;
        a.qkv = static_cast<const uint16_t*>(qkv);
        a.k_cache = static_cast<uint16_t*>(k_cache);
        a.v_cache = static_cast<uint16_t*>(v_cache);
        a.lens = lens;
        a.ctx = static_cast<uint16_t*>(ctx);
        a.B = B;
        a.L = L;
        a.nq = nq;
        a.nkv = nkv;
        a.head_dim = head_dim;
        a.qkv_stride = qkv_row;
        a.scale = 1.0f / std::sqrt((float)head_dim);
        hipStream_t s = static_cast<hipStream_t>(stream);
        tpk::Workspace ws{nullptr, 0, nullptr, 0};
        const int st = get_workspace(s, &ws);
        if (st != TP_OK) return st;
        if (tpk::attention_workspace_floats(a) > ws.partial_floats) return TP_ERR_SHAPE;
        const hipError_t e = tpk::launch_decode_attention(a, ws, s);
        return e == hipSuccess ? TP_OK : TP_ERR_HIP;
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_tune_skinny(int ksteps, int nwn, int nwk, int x_direct) {
    if (ksteps == 0 && nwn == 0 && nwk == 0) {
        g_force_ksteps = g_force_nwn = g_force_nwk = g_force_xd = 0;
        return TP_OK;
    }
    tpk::SkinnyPlan p{1, ksteps, nwn, nwk, x_direct ? 1 : 0, 1, 1};
    if (!tpk::skinny_variant_exists(p)) return TP_ERR_SHAPE;
    g_force_ksteps = ksteps;
    g_force_nwn = nwn;
    g_force_nwk = nwk;
    g_force_xd = x_direct ? 1 : 0;
    return TP_OK;
}

int tp_tune_tiled(int variant) {
    if (variant < -1 || variant >= tpk::tiled_variant_count()) return TP_ERR_RANGE;
    tpk::tiled_force_variant(variant);
    return TP_OK;
}

}  // extern "C"
