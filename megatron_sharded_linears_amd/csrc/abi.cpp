// C ABI of libtpshard: host-side validation, shape queries, kernel choice and
// dispatch to the gfx950 kernels. Every entry point checks its arguments
// before making any HIP call, so argument errors are reported (and testable)
// without a GPU. The library allocates no memory and keeps no state between
// calls beyond caches of kernel attributes: scratch is the caller's workspace
// argument. No C++ exception escapes: each entry point catches everything and
// maps it to a tp_status.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "abi_internal.h"
#include "kernels.h"
#include "layer_ops.h"
#include "tp_shard.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;   // sizes must fit the kernels' int ranges
constexpr int64_t kSkinnyMaxM = 64;
constexpr int64_t kMaxNormWidth = 32768;        // one workgroup holds a whole row in registers
constexpr int64_t kWsCounters = TP_WS_COUNTER_BYTES / 4;
static_assert(kWsCounters == tpk::kSkinnyWsCounters, "workspace counters");

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(int d) { return d == TP_BF16 || d == TP_F32; }
int64_t dtype_bytes(int d) { return d == TP_F32 ? 4 : 2; }

// Byte ranges [a, a + na) and [b, b + nb) intersect (empty ranges never do).
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    if (a == nullptr || b == nullptr || na <= 0 || nb <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

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

// The caller's workspace: counters at the front, fp32 scratch after them.
// A buffer shorter than the counters offers nothing.
int view_workspace(void* ws, int64_t bytes, tpk::Workspace* out) {
    *out = tpk::Workspace{nullptr, 0, nullptr, 0};
    if (bytes < 0) return TP_ERR_SHAPE;
    if (bytes == 0) return TP_OK;
    if (ws == nullptr) return TP_ERR_NULL;
    if (!aligned16(ws)) return TP_ERR_ALIGNMENT;
    if (bytes < TP_WS_COUNTER_BYTES) return TP_OK;
    out->counters = static_cast<unsigned*>(ws);
    out->num_counters = kWsCounters;
    out->partials = reinterpret_cast<float*>(static_cast<char*>(ws) + TP_WS_COUNTER_BYTES);
    out->partial_floats = (bytes - TP_WS_COUNTER_BYTES) / 4;
    return TP_OK;
}

// Whole 256-byte units at the back of the workspace's scratch for an operand
// a two-launch path stages; `front` keeps the rest for the linear's own
// split-K partials.
int workspace_back(const tpk::Workspace& ws, int64_t bytes, void** out, tpk::Workspace* front) {
    const int64_t floats = (bytes + 255) / 256 * 64;
    if (floats > ws.partial_floats) return TP_ERR_SHAPE;
    *out = ws.partials + (ws.partial_floats - floats);
    *front = ws;
    front->partial_floats = ws.partial_floats - floats;
    return TP_OK;
}

// ------------------------------------------------------------- kernel choice

bool plan_is_auto_decode(const tp_linear_plan& p) {
    return p.decode_ksteps == 0 && p.decode_nwn == 0 && p.decode_nwk == 0;
}

// The plan's decode shape exists for some token count, and prefill_tile is
// in range; otherwise TP_ERR_RANGE.
int check_plan(const tp_linear_plan& p) {
    if (p.prefill_tile < 0 || p.prefill_tile > tpk::tiled_variant_count()) return TP_ERR_RANGE;
    if (plan_is_auto_decode(p)) return TP_OK;
    for (int mt : {1, 2, 4}) {
        const tpk::SkinnyPlan sp{mt, p.decode_ksteps, p.decode_nwn, p.decode_nwk, p.decode_x_direct ? 1 : 0, 1, 1};
        if (tpk::skinny_variant_exists(sp)) return TP_OK;
    }
    return TP_ERR_RANGE;
}

bool split_fits(const tpk::SkinnyPlan& p, int64_t M, int64_t N, const tpk::Workspace& ws, int64_t extra_floats) {
    if (p.splits <= 1) return true;
    return p.splits <= 65535 && tpk::skinny_workspace_floats(p, M, N) + extra_floats <= ws.partial_floats &&
           p.ntiles <= ws.num_counters;
}

// Decode-kernel plan for a linear of M <= 64 tokens given the workspace;
// false when no decode variant fits (then the prefill kernel, which needs no
// scratch, or a two-launch path runs instead).
bool decode_plan(int64_t M, int64_t N, int64_t K, const tpk::Workspace& ws, const tp_linear_plan& over,
                 tpk::SkinnyPlan* out) {
    tpk::SkinnyPlan p = tpk::plan_skinny(M, N, K, ws.partial_floats, ws.num_counters);
    if (p.splits < 1) return false;
    if (!plan_is_auto_decode(over)) {
        tpk::SkinnyPlan f = p;
        f.ksteps = over.decode_ksteps;
        f.nwn = over.decode_nwn;
        f.nwk = over.decode_nwk;
        f.xd = over.decode_x_direct ? 1 : 0;
        f.ntiles = (N + 16LL * f.nwn - 1) / (16LL * f.nwn);
        const int64_t gk = 32LL * f.ksteps * f.nwk;
        f.splits = (int)((K + gk - 1) / gk);
        if (tpk::skinny_variant_exists(f) && tpk::skinny_plan_fits(f, M) && split_fits(f, M, N, ws, 0)) p = f;
    }
    // per-wave X loads read W and X through buffer resources (32-bit offsets)
    if (p.xd && (N * K * 2 > tpk::kMaxBufferBytes || M * K * 2 > tpk::kMaxBufferBytes)) return false;
    *out = p;
    return true;
}

// With the norm folded into the decode kernel (M <= 64 tokens on 16- or
// 64-token tiles, X staged in LDS by 16-row tile groups): the plan or false.
bool decode_norm_plan(int64_t M, int64_t N, int64_t K, const tpk::Workspace& ws, const tp_linear_plan& over,
                      tpk::SkinnyPlan* out) {
    if (M > 64) return false;
    tpk::SkinnyPlan p = tpk::plan_skinny_norm(M, N, K, ws.partial_floats, ws.num_counters);
    if (!plan_is_auto_decode(over)) {
        tpk::SkinnyPlan f{M <= 16 ? 1 : 4, over.decode_ksteps, over.decode_nwn, over.decode_nwk,
                          over.decode_x_direct ? 1 : 0, 1, 1};
        f.ntiles = (N + 16LL * f.nwn - 1) / (16LL * f.nwn);
        const int64_t gk = 32LL * f.ksteps * f.nwk;
        f.splits = (int)((K + gk - 1) / gk);
        if (tpk::skinny_norm_plan_fits(f, M, K) && split_fits(f, M, N, ws, tpk::skinny_norm_ss_floats(f, M)))
            p = f;
    }
    if (p.splits < 1) return false;
    *out = p;
    return true;
}

int hip_status(hipError_t e) { return e == hipSuccess ? TP_OK : TP_ERR_HIP; }

// One validated linear without the norm (EPI_STORE or EPI_SWIGLU, or a reduce
// epilogue whose decode plan the caller has checked). a.N is the kernel's row
// space for EPI_SWIGLU on the decode kernel (16-row blocks of 8 gate and 8
// up rows) and 2 i_half on the prefill kernel; this sets it.
int launch_linear(tpk::GemmArgs a, const tpk::Workspace& ws, const tp_linear_plan& over, hipStream_t s) {
    const bool swiglu = a.epi == tpk::EPI_SWIGLU;
    // an explicit prefill tile runs the tiled kernel at any token count
    const bool tiled_asked = over.prefill_tile > 0 && !tpk::epi_is_reduce(a.epi);
    const bool decode_asked = !plan_is_auto_decode(over);
    if (a.M <= kSkinnyMaxM && !tiled_asked && (decode_asked || !tpk::tiled_wins_at_decode(a))) {
        const int64_t n_rows = swiglu ? 16 * ((a.i_half + 7) / 8) : a.N;
        tpk::SkinnyPlan p;
        if (decode_plan(a.M, n_rows, a.K, ws, over, &p)) {
            a.N = n_rows;
            return hip_status(tpk::launch_skinny(a, p, ws, s));
        }
        if (tpk::epi_is_reduce(a.epi)) return TP_ERR_SHAPE;
    }
    if (swiglu) a.N = 2 * a.i_half;
    return hip_status(tpk::launch_tiled(a, s, over.prefill_tile - 1));
}

// The linear on RMS-normalised rows of a.x (unit weights: gamma is folded
// into a.w). One launch when the decode kernel can stage whole rows;
// otherwise the norm writes the normalised rows to the workspace and the
// plain linear reads them.
int launch_norm_linear(tpk::GemmArgs a, const tpk::Workspace& ws, const tp_linear_plan& over, hipStream_t s) {
    const int64_t n_rows = a.epi == tpk::EPI_SWIGLU ? 16 * ((a.i_half + 7) / 8) : a.N;
    tpk::SkinnyPlan p;
    if (a.M <= kSkinnyMaxM && decode_norm_plan(a.M, n_rows, a.K, ws, over, &p)) {
        a.N = n_rows;
        return hip_status(tpk::launch_skinny(a, p, ws, s));
    }
    void* xn = nullptr;
    tpk::Workspace front;
    const int st = workspace_back(ws, a.M * a.K * 2, &xn, &front);
    if (st != TP_OK) return st;
    tpk::PartialPtrs none;
    std::memset(&none, 0, sizeof(none));
    const hipError_t e =
        tpk::launch_add_rmsnorm(none, 0, TP_BF16, a.M, a.K, const_cast<void*>(a.x), nullptr, a.eps, xn, s);
    if (e != hipSuccess) return TP_ERR_HIP;
    a.x = xn;
    a.norm = 0;
    return launch_linear(a, front, over, s);
}

// The reduce epilogues: one launch when the decode kernel can sum the peers
// in its epilogue, otherwise the rank's partial is staged and summed by the
// reducer (EPI_REDUCE) or the add kernel (EPI_REDUCE_ADD), with the same
// arithmetic.
int launch_reduce_linear(tpk::GemmArgs a, const void* const* partials, int partial_dtype, const tpk::Workspace& ws,
                         const tp_linear_plan& over, hipStream_t s) {
    const bool add = a.epi == tpk::EPI_REDUCE_ADD;
    const bool f32 = partial_dtype == TP_F32;
    tpk::SkinnyPlan p;
    if (a.M <= kSkinnyMaxM && a.t <= tpk::kMaxFusedPeers && a.N % 4 == 0 &&
        decode_plan(a.M, a.N, a.K, ws, over, &p)) {
        a.epi = add ? (f32 ? tpk::EPI_REDUCE_ADD_F32 : tpk::EPI_REDUCE_ADD) : (f32 ? tpk::EPI_REDUCE_F32 : tpk::EPI_REDUCE);
        return hip_status(tpk::launch_skinny(a, p, ws, s));
    }
    // prefill sizes, two ranks, bf16 partials, automatic plan: the sum over
    // ranks in the 64-wide-k-tile kernel's epilogue (no staged partial, no
    // second launch; the same bits)
    if (a.M > kSkinnyMaxM && !add && !f32 && a.t <= tpk::kTiledReduceRanks && a.N % 4 == 0 && a.K % 64 == 0 &&
        over.prefill_tile == 0 && plan_is_auto_decode(over) && a.N * a.K * 2 <= tpk::kMaxBufferBytes &&
        a.M * a.K * 2 <= tpk::kMaxBufferBytes) {
        a.epi = tpk::EPI_REDUCE;
        return hip_status(tpk::launch_tiled(a, s, -1));
    }
    const int64_t own_bytes = a.M * a.N * dtype_bytes(partial_dtype);
    if (add && (a.N % 8 != 0 || a.N > kMaxNormWidth)) return TP_ERR_SHAPE;
    void* own = a.y;                  // EPI_REDUCE with bf16 partials: staged in `out`, summed in place
    tpk::Workspace front = ws;
    if (add || f32) {
        const int st = workspace_back(ws, own_bytes, &own, &front);
        if (st != TP_OK) return st;
    }
    void* const out = a.y;
    tpk::GemmArgs b = a;
    b.y = own;
    b.epi = tpk::EPI_STORE;
    b.out_dtype = partial_dtype;
    b.bias = nullptr;
    const int st = launch_linear(b, front, over, s);
    if (st != TP_OK) return st;
    tpk::PartialPtrs ptrs;
    std::memset(&ptrs, 0, sizeof(ptrs));
    for (int i = 0; i < a.t; ++i) ptrs.p[i] = i == a.rank ? own : partials[i];
    if (add)
        return hip_status(
            tpk::launch_add_rmsnorm(ptrs, a.t, partial_dtype, a.M, a.N, out, nullptr, 0.0f, nullptr, s));
    return hip_status(tpk::launch_reduce(ptrs, a.t, a.M * a.N, partial_dtype, out, TP_BF16, s));
}

// Validate one linear (every named linear call and tp_linear_ex) and fill
// the kernel arguments and the workspace view; host only.
int validate_linear(const tp_linear_call& c, tpk::GemmArgs* out, tpk::Workspace* ws_out) {
    if (c.x == nullptr || c.w == nullptr || c.y == nullptr) return TP_ERR_NULL;
    if (c.M < 0 || c.N <= 0 || c.K <= 0 || c.M >= kMaxDim || c.N >= kMaxDim / 2 || c.K >= kMaxDim) return TP_ERR_SHAPE;
    if (c.epilogue < TP_EPI_STORE || c.epilogue > TP_EPI_REDUCE_ADD) return TP_ERR_DTYPE;
    if (c.K % 8 != 0) return TP_ERR_ALIGNMENT;
    if (!aligned16(c.x) || !aligned16(c.w) || !aligned16(c.y)) return TP_ERR_ALIGNMENT;
    if (!dtype_ok(c.out_dtype)) return TP_ERR_DTYPE;
    int st = check_plan(c.plan);
    if (st != TP_OK) return st;
    const bool store = c.epilogue == TP_EPI_STORE, swiglu = c.epilogue == TP_EPI_SWIGLU;
    const bool reduce = c.epilogue == TP_EPI_REDUCE || c.epilogue == TP_EPI_REDUCE_ADD;
    if (!store && c.out_dtype != TP_BF16) return TP_ERR_DTYPE;
    if (c.bias != nullptr) {
        if (!store) return TP_ERR_SHAPE;
        if (reinterpret_cast<uintptr_t>(c.bias) & 1u) return TP_ERR_ALIGNMENT;
    }
    // byte extents: w holds 2 N rows [gate | up] for SwiGLU, y is [M, N]
    const int64_t x_bytes = c.M * c.K * 2, w_bytes = (swiglu ? 2 : 1) * c.N * c.K * 2;
    const int64_t y_bytes = c.M * c.N * dtype_bytes(c.out_dtype), b_bytes = c.N * 2;
    if (overlap(c.y, y_bytes, c.x, x_bytes) || overlap(c.y, y_bytes, c.w, w_bytes) ||
        overlap(c.y, y_bytes, c.bias, b_bytes))
        return TP_ERR_SHAPE;
    if (c.norm != 0) {
        if (reduce) return TP_ERR_SHAPE;
        if (!(c.eps >= 0.0f) || !std::isfinite(c.eps)) return TP_ERR_RANGE;
        if (c.K > kMaxNormWidth) return TP_ERR_SHAPE;
    }
    tpk::GemmArgs a{};
    if (reduce) {
        if (c.partials == nullptr) return TP_ERR_NULL;
        if (c.t < 1 || c.t > TP_MAX_SHARDS || c.rank < 0 || c.rank >= c.t) return TP_ERR_RANGE;
        if (!dtype_ok(c.partial_dtype)) return TP_ERR_DTYPE;
        const int64_t p_bytes = c.M * c.N * dtype_bytes(c.partial_dtype);
        for (int i = 0; i < c.t; ++i) {
            if (i == c.rank) continue;
            if (c.partials[i] == nullptr) return TP_ERR_NULL;
            if (!aligned16(c.partials[i])) return TP_ERR_ALIGNMENT;
            if (overlap(c.partials[i], p_bytes, c.y, y_bytes)) return TP_ERR_SHAPE;
            if (i < tpk::kMaxFusedPeers) a.peers[i] = c.partials[i];
        }
    }
    st = view_workspace(c.workspace, c.workspace_bytes, ws_out);
    if (st != TP_OK) return st;
    if (c.workspace != nullptr &&
        (overlap(c.workspace, c.workspace_bytes, c.x, x_bytes) || overlap(c.workspace, c.workspace_bytes, c.w, w_bytes) ||
         overlap(c.workspace, c.workspace_bytes, c.y, y_bytes)))
        return TP_ERR_SHAPE;
    a.x = c.x; a.w = c.w; a.bias = c.bias; a.y = c.y;
    a.M = c.M; a.N = c.N; a.K = c.K;
    a.out_dtype = c.out_dtype;
    a.epi = c.epilogue;
    a.i_half = swiglu ? c.N : 0;
    a.t = reduce ? c.t : 0;
    a.rank = reduce ? c.rank : 0;
    a.norm = c.norm != 0 ? 1 : 0;
    a.eps = c.eps;
    *out = a;
    return TP_OK;
}

int linear_call_impl(const tp_linear_call& c, hipStream_t s) {
    tpk::GemmArgs a;
    tpk::Workspace ws;
    const int st = validate_linear(c, &a, &ws);
    if (st != TP_OK) return st;
    if (c.M == 0) return TP_OK;
    if (c.epilogue == TP_EPI_REDUCE || c.epilogue == TP_EPI_REDUCE_ADD)
        return launch_reduce_linear(a, c.partials, c.partial_dtype, ws, c.plan, s);
    if (a.norm) return launch_norm_linear(a, ws, c.plan, s);
    return launch_linear(a, ws, c.plan, s);
}

// Alias so the named calls below read as before.
int linear_call(const tp_linear_call& c, hipStream_t s) { return linear_call_impl(c, s); }

tp_linear_call make_call(const void* x, int64_t M, int64_t K, const void* w, int64_t N, void* y, int out_dtype,
                         int epilogue, void* workspace, int64_t workspace_bytes) {
    tp_linear_call c;
    std::memset(&c, 0, sizeof(c));
    c.x = x; c.M = M; c.K = K; c.w = w; c.N = N; c.y = y;
    c.out_dtype = out_dtype;
    c.epilogue = epilogue;
    c.workspace = workspace;
    c.workspace_bytes = workspace_bytes;
    return c;
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
    const int64_t act_bytes = M * H * 2, in_bytes = M * H * dtype_bytes(in_dtype);
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
    return hip_status(tpk::launch_add_rmsnorm(ptrs, t, in_dtype, M, H, residual, gamma, eps, out,
                                              static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char* tp_status_string(int status) {
    switch (status) {
    case TP_OK: return "ok";
    case TP_ERR_NULL: return "a required pointer is NULL";
    case TP_ERR_SHAPE: return "negative, inconsistent or too large sizes, overlapping buffers, or too little workspace";
    case TP_ERR_DIVISIBILITY: return "a tensor-parallel split rule does not hold (n_h % t, n_kv vs t, I % t)";
    case TP_ERR_ALIGNMENT: return "pointer not 16-byte aligned or a size not a multiple of 8";
    case TP_ERR_DTYPE: return "unknown dtype, weight kind or epilogue";
    case TP_ERR_RANGE: return "t outside [1, 64], rank outside [0, t), eps not finite and >= 0, or an unknown kernel plan";
    case TP_ERR_HIP: return "the HIP runtime reported an error";
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

int64_t tp_workspace_bytes(void) { return TP_WS_COUNTER_BYTES + tpk::kSkinnyWsFloats * 4; }

int tp_prefill_tile_count(void) { return tpk::tiled_variant_count(); }

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
        if (overlap(shard_w, m.dst_rows * m.dst_cols * 2, full_w, m.src_rows * m.src_cols * 2)) return TP_ERR_SHAPE;
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
        return hip_status(tpk::launch_shard_copy(m, full_w, shard_w, static_cast<hipStream_t>(stream)));
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_linear_ex(const tp_linear_call* call, void* stream) {
    try {
        if (call == nullptr) return TP_ERR_NULL;
        return linear_call(*call, static_cast<hipStream_t>(stream));
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_column_linear(const void* x, int64_t M, int64_t K, const void* w_shard, int64_t N,
                     const void* bias_or_null, void* y, void* workspace, int64_t workspace_bytes, void* stream) {
    try {
        tp_linear_call c = make_call(x, M, K, w_shard, N, y, TP_BF16, TP_EPI_STORE, workspace, workspace_bytes);
        c.bias = bias_or_null;
        return linear_call(c, static_cast<hipStream_t>(stream));
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_row_linear_partial(const void* x_shard, int64_t M, int64_t K_shard, const void* w_shard,
                          int64_t N, void* partial, int partial_dtype, void* workspace, int64_t workspace_bytes,
                          void* stream) {
    try {
        const tp_linear_call c =
            make_call(x_shard, M, K_shard, w_shard, N, partial, partial_dtype, TP_EPI_STORE, workspace, workspace_bytes);
        return linear_call(c, static_cast<hipStream_t>(stream));
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_lm_head_shard(const void* h, int64_t M, int64_t K, const void* w_lm_shard, int64_t v_shard,
                     void* logits_shard, int out_dtype, void* workspace, int64_t workspace_bytes, void* stream) {
    try {
        const tp_linear_call c =
            make_call(h, M, K, w_lm_shard, v_shard, logits_shard, out_dtype, TP_EPI_STORE, workspace, workspace_bytes);
        return linear_call(c, static_cast<hipStream_t>(stream));
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_column_linear_swiglu(const void* x, int64_t M, int64_t K, const void* w_gate_up, int64_t i_shard,
                            void* act, void* workspace, int64_t workspace_bytes, void* stream) {
    try {
        const tp_linear_call c =
            make_call(x, M, K, w_gate_up, i_shard, act, TP_BF16, TP_EPI_SWIGLU, workspace, workspace_bytes);
        return linear_call(c, static_cast<hipStream_t>(stream));
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_row_linear_reduce(const void* x_shard, int64_t M, int64_t K_shard, const void* w_shard, int64_t N,
                         const void* const* partials, int partial_dtype, int t, int rank, void* out,
                         void* workspace, int64_t workspace_bytes, void* stream) {
    try {
        tp_linear_call c = make_call(x_shard, M, K_shard, w_shard, N, out, TP_BF16, TP_EPI_REDUCE, workspace,
                                     workspace_bytes);
        c.partials = partials;
        c.partial_dtype = partial_dtype;
        c.t = t;
        c.rank = rank;
        return linear_call(c, static_cast<hipStream_t>(stream));
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_row_linear_reduce_add(const void* x_shard, int64_t M, int64_t K_shard, const void* w_shard, int64_t N,
                             const void* const* partials, int partial_dtype, int t, int rank, void* residual,
                             void* workspace, int64_t workspace_bytes, void* stream) {
    try {
        tp_linear_call c = make_call(x_shard, M, K_shard, w_shard, N, residual, TP_BF16, TP_EPI_REDUCE_ADD, workspace,
                                     workspace_bytes);
        c.partials = partials;
        c.partial_dtype = partial_dtype;
        c.t = t;
        c.rank = rank;
        return linear_call(c, static_cast<hipStream_t>(stream));
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_rmsnorm_column_linear(const void* h, float eps, int64_t M, int64_t K, const void* w_folded, int64_t N,
                             const void* bias_or_null, void* y, void* workspace, int64_t workspace_bytes,
                             void* stream) {
    try {
        tp_linear_call c = make_call(h, M, K, w_folded, N, y, TP_BF16, TP_EPI_STORE, workspace, workspace_bytes);
        c.bias = bias_or_null;
        c.norm = 1;
        c.eps = eps;
        return linear_call(c, static_cast<hipStream_t>(stream));
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_rmsnorm_column_linear_swiglu(const void* h, float eps, int64_t M, int64_t K, const void* w_gate_up_folded,
                                    int64_t i_shard, void* act, void* workspace, int64_t workspace_bytes,
                                    void* stream) {
    try {
        tp_linear_call c =
            make_call(h, M, K, w_gate_up_folded, i_shard, act, TP_BF16, TP_EPI_SWIGLU, workspace, workspace_bytes);
        c.norm = 1;
        c.eps = eps;
        return linear_call(c, static_cast<hipStream_t>(stream));
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_swiglu(const void* gu, int64_t M, int64_t i_shard, void* out, void* stream) {
    try {
        if (gu == nullptr || out == nullptr) return TP_ERR_NULL;
        if (M < 0 || i_shard <= 0 || M >= kMaxDim || i_shard >= kMaxDim) return TP_ERR_SHAPE;
        if (i_shard % 8 != 0 || !aligned16(gu) || !aligned16(out)) return TP_ERR_ALIGNMENT;
        if (overlap(out, M * i_shard * 2, gu, M * i_shard * 4)) return TP_ERR_SHAPE;
        if (M == 0) return TP_OK;
        return hip_status(tpk::launch_swiglu(gu, M, i_shard, out, static_cast<hipStream_t>(stream)));
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
        const int64_t in_bytes = numel * dtype_bytes(in_dtype), out_bytes = numel * dtype_bytes(out_dtype);
        tpk::PartialPtrs ptrs;
        std::memset(&ptrs, 0, sizeof(ptrs));
        for (int i = 0; i < t; ++i) {
            if (partials[i] == nullptr) return TP_ERR_NULL;
            if (!aligned16(partials[i])) return TP_ERR_ALIGNMENT;
            // in place only as out == partials[0] with the same element size
            const bool in_place = i == 0 && partials[0] == out && in_dtype == out_dtype;
            if (!in_place && overlap(partials[i], in_bytes, out, out_bytes)) return TP_ERR_SHAPE;
            ptrs.p[i] = partials[i];
        }
        if (!aligned16(out)) return TP_ERR_ALIGNMENT;
        if (numel == 0) return TP_OK;
        return hip_status(tpk::launch_reduce(ptrs, t, numel, in_dtype, out, out_dtype, static_cast<hipStream_t>(stream)));
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
        const int64_t vs = (vocab + t - 1) / t;
        const int64_t out_bytes = M * H * 2;
        if (overlap(out_partial, out_bytes, ids, M * 4) || overlap(out_partial, out_bytes, e_shard, vs * H * 2))
            return TP_ERR_SHAPE;
        if (M == 0) return TP_OK;
        const int64_t lo = (int64_t)rank * vs;
        const int64_t hi = lo + vs < vocab ? lo + vs : vocab;
        return hip_status(
            tpk::launch_vocab_embed(ids, M, e_shard, lo, hi, H, out_partial, static_cast<hipStream_t>(stream)));
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
        const int64_t es = dtype_bytes(dtype);
        tpk::PartialPtrs ptrs;
        std::memset(&ptrs, 0, sizeof(ptrs));
        for (int i = 0; i < t; ++i) {
            if (shard_logits[i] == nullptr) return TP_ERR_NULL;
            if (!aligned16(shard_logits[i])) return TP_ERR_ALIGNMENT;
            if (overlap(shard_logits[i], M * v_shard * es, out, M * vocab * es)) return TP_ERR_SHAPE;
            ptrs.p[i] = shard_logits[i];
        }
        if (!aligned16(out)) return TP_ERR_ALIGNMENT;
        if (M == 0) return TP_OK;
        return hip_status(
            tpk::launch_concat(ptrs, t, M, v_shard, vocab, dtype, out, static_cast<hipStream_t>(stream)));
    } catch (...) {
        return TP_ERR_HIP;
    }
}

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

int tp_fold_norm_weight(const void* w, int64_t N, int64_t K, const void* gamma, void* w_folded, void* stream) {
    try {
        if (w == nullptr || gamma == nullptr || w_folded == nullptr) return TP_ERR_NULL;
        if (N <= 0 || K <= 0 || N >= kMaxDim || K >= kMaxDim) return TP_ERR_SHAPE;
        if (K % 8 != 0 || !aligned16(w) || !aligned16(gamma) || !aligned16(w_folded)) return TP_ERR_ALIGNMENT;
        const int64_t bytes = N * K * 2;
        if ((w_folded != w && overlap(w_folded, bytes, w, bytes)) || overlap(w_folded, bytes, gamma, K * 2))
            return TP_ERR_SHAPE;
        return hip_status(tpk::launch_fold_norm_weight(w, N, K, gamma, w_folded, static_cast<hipStream_t>(stream)));
    } catch (...) {
        return TP_ERR_HIP;
    }
}

int tp_decode_attention(const void* qkv, int64_t B, int nq, int nkv, int head_dim, void* k_cache, void* v_cache,
                        int64_t L, const int32_t* lens, void* ctx, void* workspace, int64_t workspace_bytes,
                        void* stream) {
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
        tpk::Workspace ws;
        const int st = view_workspace(workspace, workspace_bytes, &ws);
        if (st != TP_OK) return st;
        if (overlap(workspace, workspace_bytes, ctx, ctx_bytes) || overlap(workspace, workspace_bytes, qkv, qkv_bytes) ||
            overlap(workspace, workspace_bytes, k_cache, cache_bytes) ||
            overlap(workspace, workspace_bytes, v_cache, cache_bytes))
            return TP_ERR_SHAPE;
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
        if (tpk::attention_workspace_floats(a) > ws.partial_floats) return TP_ERR_SHAPE;
        if (B == 0) return TP_OK;
        return hip_status(tpk::launch_decode_attention(a, ws, static_cast<hipStream_t>(stream)));
    } catch (...) {
        return TP_ERR_HIP;
    }
}

}  // extern "C"

namespace tpabi {

int linear_call(const tp_linear_call& c, hipStream_t s) { return linear_call_impl(c, s); }

int linear_scratch_need(const tp_linear_call& c, int64_t* floats, int64_t* counters) {
    *floats = 0;
    *counters = 0;
    tp_linear_call v = c;
    v.workspace = nullptr;
    v.workspace_bytes = 0;
    tpk::GemmArgs a;
    tpk::Workspace none;
    const int st = validate_linear(v, &a, &none);
    if (st != TP_OK) return st;
    if (c.M == 0 || c.M > kSkinnyMaxM) return TP_OK;      // the prefill kernel needs no scratch
    // Only the plain and SwiGLU linears without the norm are asked about:
    // the plan launch_linear would take with the tuned workspace size.
    if (c.epilogue != TP_EPI_STORE && c.epilogue != TP_EPI_SWIGLU) return TP_ERR_SHAPE;
    if (c.norm != 0) return TP_ERR_SHAPE;
    const tpk::Workspace tuned{reinterpret_cast<float*>(16), tpk::kSkinnyWsFloats, reinterpret_cast<unsigned*>(16),
                               tpk::kSkinnyWsCounters};
    // as launch_linear: an explicit tile, or the tiled kernel's win at this
    // shape, runs the prefill kernel, which needs no scratch
    if (c.plan.prefill_tile > 0 || (plan_is_auto_decode(c.plan) && tpk::tiled_wins_at_decode(a))) return TP_OK;
    const int64_t n_rows = c.epilogue == TP_EPI_SWIGLU ? 16 * ((c.N + 7) / 8) : c.N;
    tpk::SkinnyPlan p;
    if (!decode_plan(c.M, n_rows, c.K, tuned, c.plan, &p)) return TP_OK;
    if (p.splits > 1) {
        *floats = tpk::skinny_workspace_floats(p, c.M, n_rows);
        *counters = p.ntiles;
    }
    return TP_OK;
}

}  // namespace tpabi
