// tp_column_linear_noalloc: tp_column_linear for callers that cannot
// allocate or pass device memory of their own (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation). The split-K scratch
// lives in a file-scope device array of fixed size instead of a workspace
// argument; each GPU the library runs on holds its copy until the process
// ends. Every call on one GPU shares that GPU's array, so calls that overlap
// on one GPU (two streams, or two host threads) race; calls ordered on one
// stream do not. The array keeps the last call's contents: its arrival
// counters must be zero before a call, and every call leaves them zero, so
// they are cleared once, by a fill kernel on the first call's stream on each
// device.
#include <cstring>
#include <mutex>

#include "abi_internal.h"
#include "kernels.h"

namespace {

// Layout of a workspace (tp_shard.h): TP_WS_COUNTER_BYTES of counters, then
// fp32 scratch; here 4 MiB of it.
constexpr int64_t kScratchFloats = (int64_t)1 << 20;
constexpr int64_t kScratchBytes = TP_WS_COUNTER_BYTES + kScratchFloats * 4;
constexpr int kMaxDevices = 16;

// In host code `scratch` is a stand-in, not a device address: only the
// pointer hipGetSymbolAddress returns (kept per device below) is passed on.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void zero_words(unsigned* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's copy of the array; on the first call on a device its
// counters are cleared on `s` (a fill kernel, so a capture records a node
// that replays harmlessly instead of a memset).
int device_scratch(hipStream_t s, void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return TP_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return TP_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return TP_ERR_HIP;
        const int64_t words = TP_WS_COUNTER_BYTES / 4;
        hipLaunchKernelGGL(zero_words, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s,
                           static_cast<unsigned*>(p), words);
        if (hipGetLastError() != hipSuccess) return TP_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return TP_OK;
}

}  // namespace

extern "C" int tp_column_linear_noalloc(const void* x, int64_t M, int64_t K, const void* w_shard, int64_t N,
                                        const void* bias_or_null, void* y, void* stream) {
    try {
        tp_linear_call c;
        std::memset(&c, 0, sizeof(c));
        c.x = x; c.M = M; c.K = K; c.w = w_shard; c.N = N; c.bias = bias_or_null; c.y = y;
        c.out_dtype = TP_BF16;
        c.epilogue = TP_EPI_STORE;
        // Host only: the arguments, and the scratch the plan tp_column_linear
        // takes with a workspace of tp_workspace_bytes() needs.
        int64_t floats = 0, counters = 0;
        int st = tpabi::linear_scratch_need(c, &floats, &counters);
        if (st != TP_OK) return st;
        if (floats > kScratchFloats || counters > TP_WS_COUNTER_BYTES / 4) return TP_ERR_SHAPE;
        if (M == 0) return TP_OK;
        hipStream_t s = static_cast<hipStream_t>(stream);
        void* ws = nullptr;
        st = device_scratch(s, &ws);
        if (st != TP_OK) return st;
        c.workspace = ws;
        c.workspace_bytes = kScratchBytes;
        return tpabi::linear_call(c, s);
    } catch (...) {
        return TP_ERR_HIP;
    }
}
