"""Benchmark of one tensor-parallel rank's share of the linear path on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--eager]
    python bench.py --summarize-trace PATH/TO/kernel_trace.csv

A step is one pass of the whole path over one batch of synthetic tokens, for
one rank r = 0 of a t-way split, with every input already resident in HBM:

    embedding   tp_vocab_embed (rank r) + tp_reduce_partials over t shards
    per layer   tp_column_linear (qkv) ;
                tp_row_linear_reduce (o, then the sum over ranks) ;
                tp_column_linear_swiglu (gate_up, then SwiGLU) ;
                tp_row_linear_reduce (down, then the sum over ranks)
    LM head     tp_lm_head_shard (rank r) + tp_concat_logits over t shards

At prefill sizes (more than 64 tokens) the row-parallel linears and the sums
are separate calls (tp_row_linear_partial + tp_reduce_partials). With
--separate every step is separate calls: gate_up, SwiGLU, o, reduce, down,
reduce; the other variant's step time is always reported as `alt_path`.

The other t-1 ranks' partial sums and logits (which would arrive over the
interconnect) are seeded synthetic buffers resident in HBM. Attention is not
on this path: o_proj reads a seeded synthetic context. gate_up reads the value
after all-reduce 1 and the next layer reads the value after all-reduce 2
(norms and residuals are not on this path). Weight shards are drawn on the
device from seeded generators; distinct per layer, so they stream from HBM.

The step's launches are captured once into a HIP graph; the timed region is K
replays of it (decode is launch-bound: ~200 small kernels per step). The same
calls issued eagerly from Python are timed too (`eager_ms_per_step`).

Prints ONE JSON line (the driver's contract). `value` is the shard-GEMM
TFLOP/s of the whole step: the flops of every shard GEMM in the step divided
by the time of the step. `roofline` is that of the decode-linear kernel (the
dominant one): each op's launches of one step (repeated to at least 32
launches) are captured into a graph of their own and replayed K times between
HIP events on the replaying stream, giving the average duration per launch. `cpu_baseline` is the float64 CPU
oracle on a bounded sample of the same per-rank work.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
METRIC = "shard-GEMM TFLOP/s + reduce GB/s (% roofline), Llama-8B t=8 decode B=16"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # defaults: 1000 timed steps (50 warm-up) at decode sizes, 50 (5) at
    # prefill sizes, so that every workload's run takes minutes
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default="llama8b_t8_decode_m16")
    p.add_argument("--eager", action="store_true", help="time eager launches instead of the captured step")
    p.add_argument("--separate", action="store_true",
                   help="time the step through the separate calls (no fused SwiGLU / reduce epilogues)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--step-only", action="store_true",
                   help="time the captured step only and print its figures (for a kernel trace of the step)")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--counters", action="store_true",
                   help="run under rocprofv3 --pmc: a plain copy of known size, then W+K eager steps; "
                        "prints what --summarize-counters needs and times nothing")
    return p.parse_args()


# ---------------------------------------------------------------- work model

def gemm_bytes(M, N, K, out_bytes=2):
    return 2 * N * K + 2 * M * K + out_bytes * M * N


def gemm_flops(M, N, K):
    return 2 * M * N * K


class Rank:
    """Every buffer of rank 0's share, resident on the device."""

    def __init__(self, w, lib, I, torch):
        self.w = w
        dev = "cuda"
        t, M, H, L = w.t, w.tokens, w.hidden, w.layers
        cfg = w.cfg()
        seed = 1000 * (w.index + 1)
        bf = torch.bfloat16

        def dn(shape, std, s):
            return I.device_normal_bf16(shape, std, seed + s, dev)

        self.shapes = {k: lib.tp_shard_shape(cfg, t, k) for k in lib.KIND}
        self.layers = []
        # Peers' partial sums for the two all-reduce sites: distinct per layer
        # while small (so no cache holds them across layers); shared by all
        # layers when a buffer is larger than 8 MiB (no cache can hold those).
        shared_peers = M * H * 2 > (8 << 20)
        if shared_peers:
            peers_o = [dn((M, H), 0.5, 10 + j) for j in range(t - 1)]
            peers_d = [dn((M, H), 0.5, 40 + j) for j in range(t - 1)]
        for l in range(L):
            s = 100 * (l + 1)
            self.layers.append({
                "qkv": dn(self.shapes["qkv"], 0.02, s + 1),
                "o": dn(self.shapes["o"], 0.02, s + 2),
                "gate_up": dn(self.shapes["gate_up"], 0.02, s + 3),
                "down": dn(self.shapes["down"], 0.02, s + 4),
                "ctx": dn((M, self.shapes["o"][1]), 1.0, s + 5),
                "peers_o": peers_o if shared_peers else [dn((M, H), 0.5, s + 10 + j) for j in range(t - 1)],
                "peers_d": peers_d if shared_peers else [dn((M, H), 0.5, s + 40 + j) for j in range(t - 1)],
                # RMSNorm weights (around 1) before attention and before the MLP
                "g_in": (1.0 + dn((H,), 0.1, s + 6).float()).to(bf),
                "g_post": (1.0 + dn((H,), 0.1, s + 7).float()).to(bf),
            })
        self.g_final = (1.0 + dn((H,), 0.1, 8).float()).to(bf)
        # Decode: the rank's KV caches (its query heads' KV heads, replicated
        # when there are fewer KV heads than ranks), KV_LEN tokens cached per
        # sequence, room for KV_CAP; the step appends one token at KV_LEN.
        d = w.head_dim
        self.nq_r = self.shapes["o"][1] // d
        self.nkv_r = (self.shapes["qkv"][0] // d - self.nq_r) // 2
        self.attn = M <= 64
        if self.attn:
            for l, Ld in enumerate(self.layers):
                s = 100 * (l + 1)
                Ld["k_cache"] = dn((M, self.nkv_r, KV_CAP, d), 1.0, s + 8)
                Ld["v_cache"] = dn((M, self.nkv_r, KV_CAP, d), 1.0, s + 9)
            self.kv_lens = torch.full((M,), KV_LEN, dtype=torch.int32, device=dev)
            self.ctx_attn = torch.empty((M, self.nq_r * d), dtype=bf, device=dev)
        self.x = dn((M, H), 1.0, 7)
        self.qkv = torch.empty((M, self.shapes["qkv"][0]), dtype=bf, device=dev)
        self.po = torch.empty((M, H), dtype=bf, device=dev)
        self.y1 = torch.empty((M, H), dtype=bf, device=dev)
        self.gu = torch.empty((M, self.shapes["gate_up"][0]), dtype=bf, device=dev)
        self.act = torch.empty((M, self.shapes["gate_up"][0] // 2), dtype=bf, device=dev)
        self.pd = torch.empty((M, H), dtype=bf, device=dev)
        self.h = torch.empty((M, H), dtype=bf, device=dev)
        self.xn = torch.empty((M, H), dtype=bf, device=dev)     # normalised activations
        self.vocab = w.has_vocab
        if self.vocab:
            vs = self.shapes["embed"][0]
            self.vs = vs
            self.ids = torch.randint(0, w.vocab, (M,), generator=torch.Generator().manual_seed(seed + 3),
                                     dtype=torch.int32).to(dev)
            self.embed = dn((vs, H), 0.02, 21)
            self.lm = dn((vs, H), 0.02, 22)
            self.peers_e = [dn((M, H), 0.02, 60 + j) for j in range(t - 1)]
            self.ze = torch.empty((M, H), dtype=bf, device=dev)
            Ms = w.lm_positions
            self.hs_rows = Ms
            self.logits = torch.empty((Ms, vs), dtype=bf, device=dev)
            self.peer_logits = [dn((Ms, vs), 1.0, 80 + j) for j in range(t - 1)]
            self.full_logits = torch.empty((Ms, w.vocab), dtype=bf, device=dev)

    def make_fp32_partials(self):
        """fp32 copies of the other ranks' partial sums and fp32 buffers for
        the rank's own (the variant that stores partials in fp32)."""
        import torch
        if hasattr(self, "po32"):
            return
        M, H = self.w.tokens, self.w.hidden
        self.po32 = torch.empty((M, H), dtype=torch.float32, device="cuda")
        self.pd32 = torch.empty((M, H), dtype=torch.float32, device="cuda")
        cache = {}
        for L in self.layers:
            for k in ("peers_o", "peers_d"):
                L[k + "32"] = [cache.setdefault(id(p), p.float()) for p in L[k]]

    def work(self):
        """Algorithmic flops and bytes per step, by op."""
        w = self.w
        M, H, t = w.tokens, w.hidden, w.t
        q, o, g, d = self.shapes["qkv"], self.shapes["o"], self.shapes["gate_up"], self.shapes["down"]
        ops = {
            "qkv": (w.layers, gemm_flops(M, q[0], q[1]), gemm_bytes(M, q[0], q[1])),
            "o": (w.layers, gemm_flops(M, o[0], o[1]), gemm_bytes(M, o[0], o[1])),
            "gate_up": (w.layers, gemm_flops(M, g[0], g[1]), gemm_bytes(M, g[0], g[1])),
            "down": (w.layers, gemm_flops(M, d[0], d[1]), gemm_bytes(M, d[0], d[1])),
            "swiglu": (w.layers, 0, 6 * M * (g[0] // 2)),
            "reduce": (2 * w.layers, 0, (2 * t + 2) * M * H),
            # fused calls: the linear reads the other ranks' partials / writes SwiGLU's output
            "o_reduce": (w.layers, gemm_flops(M, o[0], o[1]), gemm_bytes(M, o[0], o[1]) + 2 * (t - 1) * M * H),
            "gate_up_swiglu": (w.layers, gemm_flops(M, g[0], g[1]), 2 * g[0] * g[1] + 2 * M * g[1] + M * g[0]),
            "down_reduce": (w.layers, gemm_flops(M, d[0], d[1]), gemm_bytes(M, d[0], d[1]) + 2 * (t - 1) * M * H),
            # sum over ranks + residual add + RMSNorm: t partials and the residual
            # read, the residual and the normalised row written, gamma read
            "reduce_norm": (2 * w.layers, 0, (2 * t + 6) * M * H + 2 * H),
            "input_norm": (1, 0, 4 * M * H + 2 * H),
            # K and V of KV_LEN + 1 positions per (sequence, KV head), the qkv
            # rows read, the context written, the new K and V written
            "attention": (w.layers, 4 * M * self.nq_r * w.head_dim * (KV_LEN + 1),
                          2 * 2 * M * self.nkv_r * (KV_LEN + 1) * w.head_dim + 2 * M * q[0]
                          + 2 * M * self.nq_r * w.head_dim + 2 * 2 * M * self.nkv_r * w.head_dim),
        }
        if self.vocab:
            Ms, vs = self.hs_rows, self.vs
            ops["lm_head"] = (1, gemm_flops(Ms, vs, H), gemm_bytes(Ms, vs, H))
            lo, hi = 0, min(self.vs, w.vocab)                        # rank 0's vocab range
            owned = int(((self.ids >= lo) & (self.ids < hi)).sum().item())
            ops["embed"] = (1, 0, 4 * M + 2 * H * owned + 2 * M * H)
            ops["embed_reduce"] = (1, 0, (2 * t + 2) * M * H)
            ops["concat"] = (1, 0, 4 * Ms * w.vocab)
        return ops


def build_ops(R, lib, fused_swiglu=True, fused_reduce=True, fp32_partials=False):
    """The step as a list of (name, fn, args): every call of one pass. Fused
    calls replace gate_up + SwiGLU and a row-parallel linear + its reduce.
    fp32_partials: the row-parallel linears' partial sums (the rank's own and
    the other ranks') are stored in fp32 instead of bf16."""
    w = R.w
    t = w.t
    ops = []
    h = R.x
    if fp32_partials:
        R.make_fp32_partials()
    po, pd = (R.po32, R.pd32) if fp32_partials else (R.po, R.pd)
    pk_o, pk_d = ("peers_o32", "peers_d32") if fp32_partials else ("peers_o", "peers_d")
    if R.vocab:
        ops.append(("embed", lib.tp_vocab_embed, (R.ids, R.embed, w.vocab, t, 0, R.ze)))
        ops.append(("embed_reduce", lib.tp_reduce_partials, ([R.ze] + R.peers_e, R.h)))
        h = R.h
    for L in R.layers:
        ops.append(("qkv", lib.tp_column_linear, (h, L["qkv"], R.qkv)))
        if fused_reduce:
            ops.append(("o_reduce", lib.tp_row_linear_reduce, (L["ctx"], L["o"], [None] + L[pk_o], 0, R.y1)))
        else:
            ops.append(("o", lib.tp_row_linear_partial, (L["ctx"], L["o"], po)))
            ops.append(("reduce", lib.tp_reduce_partials, ([po] + L[pk_o], R.y1)))
        if fused_swiglu:
            ops.append(("gate_up_swiglu", lib.tp_column_linear_swiglu, (R.y1, L["gate_up"], R.act)))
        else:
            ops.append(("gate_up", lib.tp_column_linear, (R.y1, L["gate_up"], R.gu)))
            ops.append(("swiglu", lib.tp_swiglu, (R.gu, R.act)))
        if fused_reduce:
            ops.append(("down_reduce", lib.tp_row_linear_reduce, (R.act, L["down"], [None] + L[pk_d], 0, R.h)))
        else:
            ops.append(("down", lib.tp_row_linear_partial, (R.act, L["down"], pd)))
            ops.append(("reduce", lib.tp_reduce_partials, ([pd] + L[pk_d], R.h)))
        h = R.h
    if R.vocab:
        hs = h[h.shape[0] - R.hs_rows:]
        ops.append(("lm_head", lib.tp_lm_head_shard, (hs, R.lm, R.logits)))
        ops.append(("concat", lib.tp_concat_logits, ([R.logits] + R.peer_logits, w.vocab, R.full_logits)))
    return ops


def build_norm_ops(R, lib, eps=1e-5):
    """The step with the residual stream and the replicated RMSNorms of a
    Llama layer: input norm; qkv; o partial, then the sum over ranks fused with
    the residual add and the post-attention norm; gate_up + SwiGLU; down
    partial, then the sum, the add and the next norm (the next layer's input
    norm, or the final norm before the LM head)."""
    w = R.w
    ops = []
    res = R.x
    if R.vocab:
        ops.append(("embed", lib.tp_vocab_embed, (R.ids, R.embed, w.vocab, w.t, 0, R.ze)))
        ops.append(("embed_reduce", lib.tp_reduce_partials, ([R.ze] + R.peers_e, R.h)))
        res = R.h
    ops.append(("input_norm", lib.tp_add_rmsnorm, (None, res, R.layers[0]["g_in"], eps, R.xn)))
    for i, L in enumerate(R.layers):
        g_next = R.layers[i + 1]["g_in"] if i + 1 < len(R.layers) else R.g_final
        ops.append(("qkv", lib.tp_column_linear, (R.xn, L["qkv"], R.qkv)))
        ops.append(("o", lib.tp_row_linear_partial, (L["ctx"], L["o"], R.po)))
        ops.append(("reduce_norm", lib.tp_reduce_add_rmsnorm, ([R.po] + L["peers_o"], res, L["g_post"], eps, R.xn)))
        ops.append(("gate_up_swiglu", lib.tp_column_linear_swiglu, (R.xn, L["gate_up"], R.act)))
        ops.append(("down", lib.tp_row_linear_partial, (R.act, L["down"], R.pd)))
        ops.append(("reduce_norm", lib.tp_reduce_add_rmsnorm, ([R.pd] + L["peers_d"], res, g_next, eps, R.xn)))
    if R.vocab:
        hs = R.xn[R.xn.shape[0] - R.hs_rows:]
        ops.append(("lm_head", lib.tp_lm_head_shard, (hs, R.lm, R.logits)))
        ops.append(("concat", lib.tp_concat_logits, ([R.logits] + R.peer_logits, w.vocab, R.full_logits)))
    return ops


def fold_norm_weights(R, lib):
    """Load-time copies of the weights that follow a norm with its gamma
    folded in (tp_fold_norm_weight): qkv (input norm), gate_up (post-attention
    norm), the LM head (final norm)."""
    if R.layers and "qkv_f" in R.layers[0]:
        return
    for L in R.layers:
        L["qkv_f"] = lib.tp_fold_norm_weight(L["qkv"], L["g_in"], torch_empty_like(L["qkv"]))
        L["gate_up_f"] = lib.tp_fold_norm_weight(L["gate_up"], L["g_post"], torch_empty_like(L["gate_up"]))
    if R.vocab:
        R.lm_f = lib.tp_fold_norm_weight(R.lm, R.g_final, torch_empty_like(R.lm))


def torch_empty_like(t):
    import torch
    return torch.empty_like(t)


def build_fused_norm_ops(R, lib, eps=1e-5):
    """The norm step (build_norm_ops, same arithmetic) in four launches per
    layer: each norm runs inside the next column linear's staging of X
    (tp_rmsnorm_column_linear, _swiglu) and each sum over ranks adds into the
    residual as the row-parallel linear's epilogue (tp_row_linear_reduce_add);
    the final norm feeds the LM head the same way."""
    w = R.w
    ops = []
    res = R.x
    if R.vocab:
        ops.append(("embed", lib.tp_vocab_embed, (R.ids, R.embed, w.vocab, w.t, 0, R.ze)))
        ops.append(("embed_reduce", lib.tp_reduce_partials, ([R.ze] + R.peers_e, R.h)))
        res = R.h
    fold_norm_weights(R, lib)
    for L in R.layers:
        ops.append(("qkv", lib.tp_rmsnorm_column_linear, (res, eps, L["qkv_f"], R.qkv)))
        ops.append(("o", lib.tp_row_linear_reduce_add, (L["ctx"], L["o"], [None] + L["peers_o"], 0, res)))
        ops.append(("gate_up_swiglu", lib.tp_rmsnorm_column_linear_swiglu, (res, eps, L["gate_up_f"], R.act)))
        ops.append(("down", lib.tp_row_linear_reduce_add, (R.act, L["down"], [None] + L["peers_d"], 0, res)))
    if R.vocab:
        hs = res[res.shape[0] - R.hs_rows:]
        ops.append(("lm_head", lib.tp_rmsnorm_column_linear, (hs, eps, R.lm_f, R.logits)))
        ops.append(("concat", lib.tp_concat_logits, ([R.logits] + R.peer_logits, w.vocab, R.full_logits)))
    return ops


def build_layer_ops(R, lib, fused_norm, eps=1e-5):
    """The decode step of whole layers minus the rotary embedding: the norm
    step (build_fused_norm_ops or build_norm_ops) with o_proj reading the
    rank's attention over its KV caches (tp_decode_attention, which also
    appends the new token) instead of a synthetic context."""
    ops = []
    for name, fn, args in (build_fused_norm_ops if fused_norm else build_norm_ops)(R, lib, eps):
        if name == "o":
            L = next(Ld for Ld in R.layers if Ld["o"] is args[1])
            ops.append(("attention", lib.tp_decode_attention,
                        (R.qkv, L["k_cache"], L["v_cache"], R.kv_lens, R.nq_r, R.ctx_attn)))
            ops.append(("o", fn, (R.ctx_attn,) + tuple(args[1:])))
        else:
            ops.append((name, fn, args))
    return ops


GEMM_OPS = ("qkv", "o", "gate_up", "down", "lm_head", "o_reduce", "gate_up_swiglu", "down_reduce")
# (M, N, K) of each GEMM op's product, for the vendor-GEMM comparison
GEMM_SHAPES = {
    "qkv": lambda R: (R.w.tokens,) + tuple(R.shapes["qkv"]),
    "o": lambda R: (R.w.tokens,) + tuple(R.shapes["o"]),
    "o_reduce": lambda R: (R.w.tokens,) + tuple(R.shapes["o"]),
    "gate_up": lambda R: (R.w.tokens,) + tuple(R.shapes["gate_up"]),
    "gate_up_swiglu": lambda R: (R.w.tokens,) + tuple(R.shapes["gate_up"]),
    "down": lambda R: (R.w.tokens,) + tuple(R.shapes["down"]),
    "down_reduce": lambda R: (R.w.tokens,) + tuple(R.shapes["down"]),
    "lm_head": lambda R: (R.hs_rows, R.vs, R.w.hidden),
}
KV_LEN = 2048      # tokens cached per sequence before the decode step (the pages' prefill chunk)
KV_CAP = 2304      # cache capacity per sequence


def time_step(torch, ops, steps, warmup):
    """K replays of the captured step between HIP events: (ms per step, wall s)."""
    g_step = capture(torch, ops)
    for _ in range(warmup):
        g_step.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        g_step.replay()
    end.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall0
    del g_step
    return start.elapsed_time(end) / steps, wall_s


def run_ops(ops, only=None):
    for name, fn, args in ops:
        if only is None or name == only:
            fn(*args)


def capture(torch, ops, only=None, repeat=1):
    """HIP graph of the step's launches (or of one op's launches, `repeat`
    times over)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_ops(ops, only)            # per-stream workspace is allocated before capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for _ in range(repeat):
                run_ops(ops, only)
    torch.cuda.synchronize()
    return g


ROTATE_BYTES = 512 << 20    # distinct memory a per-op graph streams: twice the 256 MiB last-level cache


def _tensors(args):
    import torch
    for a in args:
        if isinstance(a, torch.Tensor):
            yield a
        elif isinstance(a, (list, tuple)):
            yield from _tensors(a)


def _clone_args(args):
    import torch

    def c(a):
        if isinstance(a, torch.Tensor):
            return a.clone()
        if isinstance(a, list):
            return [c(x) for x in a]
        return a
    return tuple(c(a) for a in args)


def rotated_launches(ops, name, min_launches=8):
    """The op's launches of one step, then the same launches on clones of
    every operand, repeated until the launches touch at least ROTATE_BYTES of
    distinct memory (and number at least `min_launches`): replayed back to
    back, no launch finds its operands in a cache from the one before."""
    base = [op for op in ops if op[0] == name]
    out, seen = list(base), {}
    for _, _, a in base:
        for x in _tensors(a):
            seen[x.data_ptr()] = x.numel() * x.element_size()
    while sum(seen.values()) < ROTATE_BYTES or len(out) < min_launches:
        for n, f, a in base:
            ca = _clone_args(a)
            for x in _tensors(ca):
                seen[x.data_ptr()] = x.numel() * x.element_size()
            out.append((n, f, ca))
    return out, sum(seen.values())


def time_rotated(torch, ops, name, reps, spread=None):
    """Microseconds per launch of op `name`: its rotated launches
    (rotated_launches) captured into one graph, replayed `reps` times between
    events on the replaying stream. Returns (us, distinct bytes); `spread`, a
    dict, receives the 10th, 50th and 90th percentiles of the per-replay
    figure (each replay bracketed by its own events)."""
    launches, distinct = rotated_launches(ops, name)
    g = capture(torch, launches)
    ms = time_graph(torch, g, reps, 2)
    n = len(launches)
    if spread is not None:
        per = []
        for _ in range(max(reps, 10)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            b.synchronize()
            per.append(a.elapsed_time(b) * 1e3 / n)
        per.sort()
        q = lambda f: per[min(len(per) - 1, int(f * len(per)))]
        spread.update({"us_p10": round(q(0.1), 3), "us_p50": round(q(0.5), 3), "us_p90": round(q(0.9), 3)})
    del g, launches
    torch.cuda.empty_cache()
    return ms * 1e3 / n, distinct


def vendor_mm_us(torch, M, N, K, reps):
    """The same product as a plain bf16 GEMM through torch.mm (hipBLASLt on
    ROCm), Y = X W^T with W rotated over at least ROTATE_BYTES of distinct
    weights like the per-op timings: context for the shard GEMMs (the
    library's calls add the epilogues)."""
    n = max(8, -(-ROTATE_BYTES // (N * K * 2)))
    x = torch.randn((M, K), device="cuda").to(torch.bfloat16)
    ws = [(torch.randn((N, K), device="cuda") * 0.02).to(torch.bfloat16) for _ in range(n)]
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ops = [("mm", lambda w: torch.mm(x, w.t(), out=y), (w,)) for w in ws]
    g = capture(torch, ops)
    ms = time_graph(torch, g, reps, 2)
    del g, ws, ops
    torch.cuda.empty_cache()
    return ms * 1e3 / n


def time_graph(torch, g, reps, warmup):
    """Events around `reps` replays on the replaying (current) stream; ms per replay."""
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def measure_copy(torch, lib, I, w, reps=10):
    """HBM bandwidth of a plain streaming copy on this device: the shard copy
    at t = 1 over the full gate_up weight, a few distinct buffers captured in
    one graph so that no cache holds them. Context for the roofline fractions
    (the 8 TB/s peak is the vendor's figure)."""
    cfg = w.cfg()
    full = lib.tp_full_shape(cfg, "gate_up")
    nbytes = full[0] * full[1] * 2
    n = max(2, min(8, (2 << 30) // (2 * nbytes)))
    src = [I.device_normal_bf16(full, 1.0, 90 + i, "cuda") for i in range(n)]
    dst = [torch.empty_like(x) for x in src]
    ops = [("copy", lib.tp_shard_weights, (cfg, 1, 0, "gate_up", src[i], dst[i])) for i in range(n)]
    g = capture(torch, ops)
    ms = time_graph(torch, g, reps, 2)
    del g, src, dst
    gbps = 2 * nbytes * n / (ms * 1e-3) / 1e9
    return {"kernel": "shard_copy_kernel (t = 1, 16-byte vectors)", "bytes_per_launch": 2 * nbytes,
            "launches": n, "GBps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}


def pages_context(w):
    """The traffic the pages estimate for this workload's all-reduces and
    logits all-gather (arithmetic only; the pages measure nothing)."""
    from megatron_sharded_linears_amd import traffic as T
    one, total = T.per_step(w.tokens, w.hidden, w.layers)
    ctx = {"all_reduces_per_forward": T.all_reduces_per_forward(w.layers),
           "all_reduce_payload_KiB": one / T.KIB, "all_reduce_payload_per_forward_MiB": round(total / T.MIB, 2),
           "ring_sent_per_rank_per_token_KiB": T.ring_sent_per_rank_per_token(w.hidden, w.layers, w.t) / T.KIB}
    if w.has_vocab:
        ctx["logits_gather_received_per_sampled_token_KiB"] = round(
            T.logits_gather_received_per_token(w.vocab, w.t) / T.KIB, 1)
    return ctx


# ----------------------------------------------------------- CPU baseline

def cpu_baseline(w, seconds):
    """The float64 oracle on this host, on a bounded sample of the same
    per-rank work: the shard GEMMs, SwiGLU and reduces of two layers, looped
    until `seconds` have passed. Returns shard-GEMM TFLOP/s."""
    import numpy as np
    import oracle
    from megatron_sharded_linears_amd import inputs as I
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        cores = os.cpu_count()
    from megatron_sharded_linears_amd import lib
    cfg, t, M, H = w.cfg(), w.t, w.tokens, w.hidden
    sh = {k: lib.tp_shard_shape(cfg, t, k) for k in ("qkv", "o", "gate_up", "down")}
    f64 = I.to_f64
    layers = []
    for l in range(2):
        layers.append({k: f64(I.normal_bf16((w.index, l, 50 + j), sh[k], 0.02))
                       for j, k in enumerate(sh)})
        layers[-1]["ctx"] = f64(I.normal_bf16((w.index, l, 60), (M, sh["o"][1])))
        layers[-1]["peers"] = [f64(I.normal_bf16((w.index, l, 70 + j), (M, H), 0.5)) for j in range(t - 1)]
    x = f64(I.normal_bf16((w.index, 99), (M, H)))
    flops_layer = sum(gemm_flops(M, sh[k][0], sh[k][1]) for k in sh)
    n = 0
    t0 = time.perf_counter()
    while True:
        for L in layers:
            oracle.linear(x, L["qkv"])
            po = oracle.linear(L["ctx"], L["o"])
            y1 = oracle.round_bf16(oracle.all_reduce_sum([po] + L["peers"]))
            gu = oracle.round_bf16(oracle.linear(y1, L["gate_up"]))
            i_s = gu.shape[1] // 2
            act = oracle.round_bf16(oracle.swiglu(gu[:, :i_s], gu[:, i_s:]))
            pd = oracle.linear(act, L["down"])
            x = oracle.round_bf16(oracle.all_reduce_sum([pd] + L["peers"]))
            n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    # the unsharded layer's four products once, for scale (one rank's share
    # is 1/t of them); decode sizes only (at prefill sizes it would take
    # minutes of float64)
    unsharded_s = None
    if M <= 64:
        full = {k: lib.tp_full_shape(cfg, k) for k in ("qkv", "o", "gate_up", "down")}
        rng = np.random.default_rng(w.index)
        t1 = time.perf_counter()
        for k in full:
            Wf = rng.standard_normal(full[k]) * 0.02
            oracle.linear(rng.standard_normal((M, full[k][1])), Wf)
        unsharded_s = round(time.perf_counter() - t1, 3)
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"value": flops_layer * n / el / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} layer passes (qkv, o, reduce, gate_up, SwiGLU, down, reduce at this workload's "
                      f"rank-share shapes, float64 NumPy) over 2 seeded layers in {el:.1f} s",
            "affinity_cpus": affinity, "os_cpu_count": os.cpu_count(), "blas_threads": int(cores),
            "unsharded_layer_products_s": unsharded_s}


# ------------------------------------------------------------------- main

GEMM_SOURCES = ("gemm_skinny.hip", "gemm_tiled.hip", "common.h", "kernels.h")


def code_digest(text):
    """SHA-256 of C++ source text with comments removed and whitespace
    collapsed: changes to comments or layout do not change it."""
    import hashlib
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def gemm_source_sha256():
    """Digest of the GEMM kernels' code: a stored counter summary speaks for
    the kernels only while this is unchanged."""
    texts = []
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "megatron_sharded_linears_amd", "csrc", f)) as fh:
            texts.append(fh.read())
    return code_digest("\n".join(texts))


def traffic_file(workload):
    return os.path.join(ROOT, "profiles", f"gemm_traffic_{workload}.json")


def stored_traffic(workload):
    """HBM bytes per step of the GEMM launches, from the committed counter
    summary of this workload, or None when there is none or the kernels'
    sources have changed since it was taken."""
    try:
        with open(traffic_file(workload)) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_sha256") != gemm_source_sha256():
        return None
    return d


# every kernel a GEMM call launches (a K split over 64-row tiles finishes in
# skinny_split_finish; a prefill call may split its token rows over two
# tiled launches)
GEMM_KERNELS = ("skinny_kernel", "skinny_split_finish", "tiled_dma_kernel", "tiled_dma64_kernel", "tiled_reg_kernel")


# the library's other kernels (the step's sums, embedding, concatenation,
# norms, attention), whose traffic the counter summary lists per launch
LIBRARY_KERNELS = ("reduce_kernel", "vocab_embed_kernel", "concat_", "add_rmsnorm_kernel", "swiglu_kernel",
                   "attn_chunk_kernel", "attn_merge_kernel", "fold_norm_weight_kernel")


def is_gemm_kernel(name):
    return any(k in name for k in GEMM_KERNELS)


def summarize_counters(fetch_csv, write_csv, run_json, out=None):
    """HBM traffic of the step's GEMM launches from two rocprofv3 --pmc runs
    of `bench.py --counters` (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).
    Each counter is scaled by what it reads for the plain copy of known size
    (shard_copy_kernel at t = 1: reads and writes exactly `copy_bytes`)."""
    import csv
    import re
    with open(run_json) as f:
        run = json.loads([ln for ln in f if ln.startswith("{")][-1])

    def load(path, counter):
        per = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                m = re.search(r"(\w+_kernel)(<[^>]*>)?", r["Kernel_Name"])
                short = (m.group(1) + (m.group(2) or "")) if m else r["Kernel_Name"][:60]
                if r.get("Grid_Size"):
                    short += f" grid={r['Grid_Size']}"
                per.setdefault(short, []).append(float(r["Counter_Value"]) * 1024.0)
        return per

    fetch, write = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    nb = run["copy_bytes"]
    cf = [v for k, vs in fetch.items() if k.startswith("shard_copy_kernel") for v in vs]
    cw = [v for k, vs in write.items() if k.startswith("shard_copy_kernel") for v in vs]
    if len(cf) != run["copy_launches"] or len(cw) != run["copy_launches"]:
        raise SystemExit(f"expected {run['copy_launches']} copy dispatches, found {len(cf)} / {len(cw)}")
    f_fetch = nb / (sum(cf) / len(cf))
    f_write = nb / (sum(cw) / len(cw))
    steps = run["steps"]
    rows, fetch_step, write_step, launches = [], 0.0, 0.0, 0
    for k in sorted(set(fetch) | set(write)):
        if not is_gemm_kernel(k):
            continue
        fv, wv = fetch.get(k, []), write.get(k, [])
        if len(fv) != len(wv) or len(fv) % steps:
            raise SystemExit(f"{k}: {len(fv)} fetch / {len(wv)} write dispatches over {steps} steps")
        fetch_step += sum(fv) * f_fetch / steps
        write_step += sum(wv) * f_write / steps
        launches += len(fv) // steps
        rows.append((k, len(fv) // steps, sum(fv) / len(fv) * f_fetch, sum(wv) / len(wv) * f_write))
    if launches < run["gemm_launches_per_step"]:
        raise SystemExit(f"found {launches} GEMM launches per step, fewer than the {run['gemm_launches_per_step']} calls")
    alg = run["gemm_algorithmic_bytes_per_step"]
    other = []
    for k in sorted(set(fetch) | set(write)):
        if is_gemm_kernel(k) or "at::" in k or not any(k.startswith(n) for n in LIBRARY_KERNELS):
            continue
        fv, wv = fetch.get(k, []), write.get(k, [])
        if fv and wv:
            other.append({"kernel": k, "launches": len(fv), "fetch_bytes_per_launch": round(sum(fv) / len(fv) * f_fetch),
                          "write_bytes_per_launch": round(sum(wv) / len(wv) * f_write)})
    d = {"workload": run["workload"], "source_sha256": run["source_sha256"],
         "copy_bytes": nb, "fetch_scale": round(f_fetch, 5), "write_scale": round(f_write, 5),
         "gemm_calls_per_step": run["gemm_launches_per_step"],
         "gemm_launches_per_step": launches, "fetch_bytes_per_step": round(fetch_step),
         "write_bytes_per_step": round(write_step), "traffic_bytes_per_step": round(fetch_step + write_step),
         "algorithmic_bytes_per_step": alg, "traffic_over_algorithmic": round((fetch_step + write_step) / alg, 4),
         "per_kernel": [{"kernel": k, "launches_per_step": n, "fetch_bytes_per_launch": round(fb),
                         "write_bytes_per_launch": round(wb)} for k, n, fb, wb in rows],
         "other_kernels": other}
    print(f"copy of {nb} B: FETCH_SIZE scale {f_fetch:.4f}, WRITE_SIZE scale {f_write:.4f}")
    print(f"{'kernel':56s} {'launches/step':>13s} {'fetch_MiB/launch':>16s} {'write_MiB/launch':>16s}")
    for k, n, fb, wb in rows:
        print(f"{k[:56]:56s} {n:13d} {fb / 2**20:16.3f} {wb / 2**20:16.3f}")
    for o in other:
        print(f"{o['kernel'][:56]:56s} {o['launches']:13d} {o['fetch_bytes_per_launch'] / 2**20:16.3f} "
              f"{o['write_bytes_per_launch'] / 2**20:16.3f}  (all launches of the run)")
    print(f"per step: traffic {(fetch_step + write_step) / 2**20:.2f} MiB, algorithmic {alg / 2**20:.2f} MiB, "
          f"ratio {(fetch_step + write_step) / alg:.4f}")
    if out:
        with open(out, "w") as f:
            json.dump(d, f, indent=1)
            f.write("\n")
    return d



MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "GRBM_GUI_ACTIVE")
NUM_SIMDS = 1024                # 256 CUs x 4 SIMDs
NUM_XCDS = 8                    # GRBM_GUI_ACTIVE comes summed over the XCDs' instances


def summarize_mfma(pmc_csv, trace_csv, run_json, out=None):
    """Matrix-core use of the step's GEMM launches from one rocprofv3 --pmc
    pass of `bench.py --counters` with MFMA_COUNTERS and a --kernel-trace
    pass of the same command (durations), per kernel shape: the MFMA busy
    fraction (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x 1024 SIMDs),
    the busy-CU fraction, the shader clock the dispatch ran at
    (GRBM_GUI_ACTIVE over its duration) and the bf16 MFMA rate (512 flop per
    SQ_INSTS_VALU_MFMA_MOPS_BF16 over the duration). GRBM_GUI_ACTIVE is
    reported summed over its 8 per-XCD instances: one XCD's busy cycles are
    that over 8. The counter window spans a little more than the kernel
    (setup and drain around each serialised dispatch), so the clock of short
    dispatches reads high."""
    import csv
    import re
    with open(run_json) as f:
        run = json.loads([ln for ln in f if ln.startswith("{")][-1])

    def short(r):
        m = re.search(r"(\w+_kernel)(<[^>]*>)?", r["Kernel_Name"])
        name = (m.group(1) + (m.group(2) or "")) if m else r["Kernel_Name"][:60]
        return f"{name} grid={r['Grid_Size']}" if r.get("Grid_Size") else name

    cnt = {}
    with open(pmc_csv) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] in MFMA_COUNTERS:
                d = cnt.setdefault(short(r), {})
                d.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    dur = {}
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            m = re.search(r"(\w+_kernel)(<[^>]*>)?", r["Kernel_Name"])
            name = (m.group(1) + (m.group(2) or "")) if m else r["Kernel_Name"][:60]
            g = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            dur.setdefault(f"{name} grid={g}", []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    steps = run["steps"]
    lines = [f"workload {run['workload']}: GEMM launches of {steps} eager steps",
             "", "| kernel | per step | avg us | GUI_ACTIVE cycles | clock GHz | MFMA busy | CUs busy | bf16 MFMA TFLOP/s |",
             "|---|---:|---:|---:|---:|---:|---:|---:|"]
    tot = {"busy": 0.0, "gui": 0.0, "flop": 0.0, "ns": 0.0}
    for k in sorted(cnt, key=lambda k: -sum(dur.get(k, [0]))):
        if not is_gemm_kernel(k) or k not in dur:
            continue
        c = cnt[k]
        n = len(c["GRBM_GUI_ACTIVE"])
        avg = {name: sum(v) / len(v) for name, v in c.items()}
        ns = sum(dur[k]) / len(dur[k])
        gui = avg["GRBM_GUI_ACTIVE"] / NUM_XCDS
        busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * NUM_SIMDS)
        cu = avg["SQ_BUSY_CU_CYCLES"] / (gui * 256)
        flop = avg["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        lines.append(f"| `{k}` | {n // steps} | {ns / 1e3:.2f} | {gui:.0f} | {gui / ns:.2f} | {busy:.3f} | "
                     f"{cu:.3f} | {flop / ns / 1e3:.1f} |")
        tot["busy"] += avg["SQ_VALU_MFMA_BUSY_CYCLES"] * n
        tot["gui"] += gui * n
        tot["flop"] += flop * n
        tot["ns"] += ns * n
    if tot["gui"]:
        lines += ["", f"- over all GEMM launches: MFMA busy {tot['busy'] / (tot['gui'] * NUM_SIMDS):.3f} of the "
                      f"SIMD-cycles, {tot['flop'] / tot['ns'] / 1e3:.1f} TFLOP/s of bf16 MFMA work over their "
                      f"summed durations ({tot['flop'] / tot['ns'] / 1e3 / BF16_PEAK_TFLOPS:.3f} of "
                      f"{BF16_PEAK_TFLOPS:.0f})"]
    text = "\n".join(lines)
    print(text)
    if out:
        with open(out, "w") as f:
            f.write(text + "\n")


def summarize_trace(path, top=30):
    """Per (kernel, workgroups) duration stats from a rocprofv3
    --kernel-trace --output-format csv trace: a row per distinct launch shape,
    so each op of the step can be matched to its kernel."""
    import csv
    import re
    groups = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            m = re.search(r"(\w+_kernel)(<[^>]*>)?", name)
            short = (m.group(1) + (m.group(2) or "")) if m else name[:60]
            wg = int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"])
            wgs = (int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]), int(r["Grid_Size_Y"]) // int(r["Workgroup_Size_Y"]))
            d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            groups.setdefault((short, wgs, wg), []).append(d)
    rows = sorted(groups.items(), key=lambda kv: -sum(kv[1]))[:top]
    print(f"{'kernel':44s} {'workgroups':>12s} {'threads':>7s} {'calls':>6s} {'avg_us':>8s} {'min_us':>8s} {'max_us':>8s} {'total_ms':>9s}")
    for (short, wgs, wg), ds in rows:
        print(f"{short[:44]:44s} {str(wgs):>12s} {wg:7d} {len(ds):6d} {sum(ds) / len(ds) / 1e3:8.2f} "
              f"{min(ds) / 1e3:8.2f} {max(ds) / 1e3:8.2f} {sum(ds) / 1e6:9.2f}")


def summarize_step_trace(trace_csv, run_log, out=None):
    """Kernel time per step from a rocprofv3 --kernel-trace (csv) of
    `bench.py --step-only`: the dispatches of the last K (timed) replays,
    per kernel and summed, against the step time the same run measured, and
    the GEMM launches' algorithmic bytes over their summed durations."""
    import csv
    import re
    with open(run_log) as f:
        run = json.loads([ln for ln in f if ln.startswith("{")][-1])
    rows = []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            m = re.search(r"(\w+_kernel)(<[^>]*>)?", r["Kernel_Name"])
            short = (m.group(1) + (m.group(2) or "")) if m else r["Kernel_Name"][:60]
            wgs = int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"])
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), f"{short} x{wgs}"))
    rows.sort()
    n_steps_trace, K = run["steps_in_trace"], run["steps"]
    # The timed replays are the trace's last dispatches (set-up kernels such
    # as the seeded generators come first): the step's length is the
    # smallest period of the kernel sequence over its last K repeats.
    # A step of identical layers repeats with the layer's period too, and a
    # call may launch more than one kernel: the step's period is the multiple
    # of the smallest one, covering at least the step's calls, whose K
    # repeats span the time the run measured for K steps.
    names = [k for _, _, k in rows]
    q = next((p for p in range(1, len(names) // K + 1)
              if all(names[-1 - i] == names[-1 - i - p] for i in range(p * (K - 1)))), None)
    if q is None:
        raise SystemExit("no step period found in the trace")

    def span_ms_of(per):
        t = rows[-K * per:]
        return (t[-1][1] - t[0][0]) / 1e6 / K

    cands = [q * j for j in range(-(-run["launches_per_step"] // q), 4 * run["launches_per_step"] // q + 2)
             if K * q * j <= len(rows) and
             all(names[-1 - i] == names[-1 - i - q * j] for i in range(q * j * (K - 1)))]
    if not cands:
        raise SystemExit(f"the trace does not repeat with a period of {q} dispatches over {K} steps")
    per = min(cands, key=lambda p: abs(span_ms_of(p) - run["ms_per_step"]))
    timed = rows[-K * per:]
    span_ms = (timed[-1][1] - timed[0][0]) / 1e6 / K
    groups = {}
    for a, b, k in timed:
        groups.setdefault(k, []).append(b - a)
    total_us = sum(b - a for a, b, _ in timed) / 1e3 / K
    gemm_us = sum(b - a for a, b, k in timed if is_gemm_kernel(k)) / 1e3 / K
    gemm_n = sum(1 for _, _, k in timed if is_gemm_kernel(k)) // K
    alg = run["gemm_algorithmic_bytes_per_step"]
    gbps = alg / (gemm_us * 1e-6) / 1e9
    tflops = run["gemm_flops_per_step"] / (gemm_us * 1e-6) / 1e12
    lines = [f"workload {run['workload']}: {per} dispatches per step; the last {K} of "
             f"{n_steps_trace} passes (the timed graph replays)",
             "", "| kernel x workgroups | per step | avg us | us per step |", "|---|---:|---:|---:|"]
    for k, ds in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{k}` | {len(ds) // K} | {sum(ds) / len(ds) / 1e3:.2f} | {sum(ds) / 1e3 / K:.2f} |")
    lines += ["",
              f"- sum of dispatch durations per step: {total_us:.1f} us",
              f"- span of a traced step (first start to last end, averaged): {span_ms * 1e3:.1f} us",
              f"- step time the traced run measured with events (ms_per_step): {run['ms_per_step'] * 1e3:.1f} us",
              f"- GEMM dispatches per step: {gemm_n} ({run['gemm_launches_per_step']} GEMM calls), "
              f"summed {gemm_us:.1f} us",
              f"- GEMM algorithmic bytes per step: {alg} -> {gbps:.1f} GB/s over their summed durations, "
              f"{gbps / HBM_PEAK_GBPS:.4f} of {HBM_PEAK_GBPS:.0f} GB/s",
              f"- GEMM flops per step: {run['gemm_flops_per_step']} -> {tflops:.1f} TFLOP/s over their summed "
              f"durations, {tflops / BF16_PEAK_TFLOPS:.4f} of {BF16_PEAK_TFLOPS:.0f} TFLOP/s"]
    text = "\n".join(lines)
    print(text)
    if out:
        with open(out, "w") as f:
            f.write(text + "\n")


def layer_linears(work, per_op, gemm_ops):
    """TFLOP/s and GB/s of the step's per-layer linears (qkv, o, gate_up,
    down and their fused forms) from their per-op durations."""
    ops = [k for k in gemm_ops if k != "lm_head"]
    us = sum(per_op[k]["us_per_launch"] * work[k][0] for k in ops)
    fl = sum(work[k][0] * work[k][1] for k in ops)
    by = sum(work[k][0] * work[k][2] for k in ops)
    layers = work[ops[0]][0]
    return {"ops": ops, "us_per_layer": round(us / layers, 3), "TFLOPs": round(fl / (us * 1e-6) / 1e12, 3),
            "GBps": round(by / (us * 1e-6) / 1e9, 1), "frac_of_hbm": round(by / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "frac_of_bf16": round(fl / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)}


def main():
    if len(sys.argv) in (4, 5) and sys.argv[1] == "--summarize-step-trace":
        summarize_step_trace(*sys.argv[2:])
        return
    if len(sys.argv) == 3 and sys.argv[1] == "--summarize-trace":
        summarize_trace(sys.argv[2])
        return
    if len(sys.argv) in (5, 6) and sys.argv[1] == "--summarize-mfma":
        summarize_mfma(*sys.argv[2:])
        return
    if len(sys.argv) in (5, 6) and sys.argv[1] == "--summarize-counters":
        summarize_counters(*sys.argv[2:])
        return
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: every shard of the t-way split is computed on that one "
              "device and there is no cross-GPU path to scale. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from megatron_sharded_linears_amd import inputs as I
    from megatron_sharded_linears_amd import lib
    from megatron_sharded_linears_amd.workloads import BY_NAME

    w = BY_NAME[args.workload]
    if args.steps is None:
        args.steps = 1000 if w.tokens <= 64 else 50
    if args.warmup is None:
        args.warmup = 50 if w.tokens <= 64 else 5
    torch.cuda.set_device(0)
    R = Rank(w, lib, I, torch)
    torch.cuda.synchronize()
    work = R.work()

    # The step: fused calls where they are one launch (SwiGLU always; the
    # reduce at decode sizes, where the linear's epilogue sums the partials).
    fused = not args.separate
    # the sum over ranks fused into the row-parallel linear wherever the
    # library fuses it: every decode size, and prefill sizes at t <= 2
    fuse_sum = w.tokens <= 64 or w.t <= 2
    fused_reduce = fused and fuse_sum
    ops = build_ops(R, lib, fused_swiglu=fused, fused_reduce=fused_reduce)
    alt_ops = build_ops(R, lib, fused_swiglu=not fused, fused_reduce=(not fused) and fuse_sum)
    names = []
    for n, _, _ in ops:
        if n not in names:
            names.append(n)

    gemm_ops = [k for k in GEMM_OPS if k in names]
    if args.counters:
        # A plain copy of known size (the counters' scale), then W+K eager steps.
        cfg = w.cfg()
        full = lib.tp_full_shape(cfg, "gate_up")
        src = I.device_normal_bf16(full, 1.0, 5, "cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            lib.tp_shard_weights(cfg, 1, 0, "gate_up", src, dst)
        torch.cuda.synchronize()
        if not torch.equal(src, dst):
            raise SystemExit("calibration copy mismatch")
        del src, dst
        for _ in range(args.warmup + args.steps):
            run_ops(ops)
        # and the sums over ranks of the separate-call path (their traffic is
        # reported per launch, beside the step's GEMMs)
        for _ in range(args.warmup + args.steps):
            run_ops([op for op in alt_ops if op[0] == "reduce"])
        torch.cuda.synchronize()
        print(json.dumps({"workload": w.name, "copy_bytes": full[0] * full[1] * 2, "copy_launches": 3,
                          "steps": args.warmup + args.steps,
                          "gemm_launches_per_step": sum(work[k][0] for k in gemm_ops),
                          "gemm_algorithmic_bytes_per_step": sum(work[k][0] * work[k][2] for k in gemm_ops),
                          "source_sha256": gemm_source_sha256()}), flush=True)
        return

    flops_step = sum(work[k][0] * work[k][1] for k in gemm_ops)
    gemm_bytes_step = sum(work[k][0] * work[k][2] for k in gemm_ops)
    if args.step_only:
        # one eager pass (before capture), W warm-up replays, K timed replays
        ms_step, wall_s = time_step(torch, ops, args.steps, args.warmup)
        print(json.dumps({"workload": w.name, "ms_per_step": round(ms_step, 4), "steps": args.steps,
                          "warmup": args.warmup, "steps_in_trace": 1 + args.warmup + args.steps,
                          "value": round(flops_step / (ms_step * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
                          "gemm_launches_per_step": sum(work[k][0] for k in gemm_ops),
                          "gemm_algorithmic_bytes_per_step": gemm_bytes_step,
                          "gemm_flops_per_step": flops_step,
                          "launches_per_step": len(ops)}), flush=True)
        return

    t_start = time.perf_counter()

    def note(what):
        # progress on stderr (the JSON line alone goes to stdout)
        print(f"bench: {what} done at {time.perf_counter() - t_start:.0f} s", file=sys.stderr, flush=True)

    # --- eager: the same calls issued one by one from Python
    for _ in range(args.warmup):
        run_ops(ops)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        run_ops(ops)
    b.record()
    torch.cuda.synchronize()
    ms_eager = a.elapsed_time(b) / args.steps
    note("eager step")

    # --- timed region: exactly K steps, each the replay of the captured step
    ms_step, wall_s = time_step(torch, ops, args.steps, args.warmup)
    if args.eager:
        ms_step = ms_eager
    # the same step through the other set of calls, for comparison
    ms_alt, _ = time_step(torch, alt_ops, args.steps, args.warmup)
    note("graph step and the other calls' step")
    # partial sums stored in bf16 or fp32, the sum over ranks through the
    # fused call (tp_row_linear_reduce) or a call of its own (where the
    # library fuses the sum: decode sizes, and bf16 partials at prefill
    # sizes at t <= 2)
    partials = {}
    for p32 in (False, True):
        d = {}
        for fr in ((True, False) if fuse_sum and (w.tokens <= 64 or not p32) else (False,)):
            ms_p = time_step(torch, build_ops(R, lib, fused_swiglu=fused, fused_reduce=fr, fp32_partials=p32),
                             args.steps, args.warmup)[0]
            d["reduce_fused" if fr else "reduce_separate"] = round(ms_p, 4)
        partials["fp32" if p32 else "bf16"] = d
    partials["default"] = "bf16"
    note("partial storage steps")
    # and with the residual stream and the RMSNorms of a real layer
    norm_ops = build_norm_ops(R, lib)
    ms_norm, _ = time_step(torch, norm_ops, args.steps, args.warmup)
    # decode: the same step with the norms folded into the linears
    ms_norm_fused = time_step(torch, build_fused_norm_ops(R, lib), args.steps, args.warmup)[0] if R.attn else None
    # and (decode) whole layers: norms and the rank's attention over its KV
    # caches, on whichever norm step measured faster
    fused_norm = ms_norm_fused is not None and ms_norm_fused < ms_norm
    layer_ops = build_layer_ops(R, lib, fused_norm) if R.attn else None
    ms_layer = time_step(torch, layer_ops, args.steps, args.warmup)[0] if layer_ops else None
    note("norm and layer steps")

    # --- per kernel: each op's launches of one step, captured and replayed K times
    per_op = {}
    op_names = names + [n for n in ("reduce",) if n not in names]
    for name in op_names:
        n_per_step, flops, byts = work[name]
        spread = {}
        us, distinct = time_rotated(torch, ops if name in names else alt_ops, name, args.steps, spread)
        per_op[name] = {"launches_per_step": n_per_step, "us_per_launch": round(us, 3),
                        "GBps": round(byts / (us * 1e-6) / 1e9, 1),
                        "TFLOPs": round(flops / (us * 1e-6) / 1e12, 2) if flops else None,
                        "bytes_per_launch": byts, "distinct_MiB": round(distinct / 2**20), **spread}
        if name in GEMM_SHAPES:
            Mv, Nv, Kv = GEMM_SHAPES[name](R)
            per_op[name]["vendor_mm_us"] = round(vendor_mm_us(torch, Mv, Nv, Kv, args.steps), 3)
        note(f"per-op {name}")

    attn = None
    if layer_ops:
        us_at, _ = time_rotated(torch, layer_ops, "attention", args.steps)
        attn = {"us_per_call": round(us_at, 3), "GBps": round(work["attention"][2] / (us_at * 1e-6) / 1e9, 1),
                "frac_of_hbm": round(work["attention"][2] / (us_at * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                "bytes_per_call": work["attention"][2], "kv_len": KV_LEN, "kv_capacity": KV_CAP,
                "q_heads": R.nq_r, "kv_heads": R.nkv_r}
    us_norm, _ = time_rotated(torch, norm_ops, "reduce_norm", args.steps)

    copy = measure_copy(torch, lib, I, w)
    note("attention, norm call and copy")

    # the step's sums over ranks alone, back to back (the separate-call
    # path's 2 per layer): launched one by one from Python, and replayed as
    # a captured graph (the count problem of the decode all-reduces)
    red_ops = [op for op in alt_ops if op[0] == "reduce"]
    for _ in range(3):
        run_ops(red_ops)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        run_ops(red_ops)
    b.record()
    torch.cuda.synchronize()
    red_eager_us = a.elapsed_time(b) * 1e3 / (args.steps * len(red_ops))
    g = capture(torch, red_ops)
    red_graph_us = time_graph(torch, g, args.steps, 2) * 1e3 / len(red_ops)
    del g

    value = flops_step / (ms_step * 1e-3) / 1e12
    gemm_us = sum(per_op[k]["us_per_launch"] * work[k][0] for k in gemm_ops)
    achieved = gemm_bytes_step / (gemm_us * 1e-6) / 1e9
    red = per_op["reduce"]
    st = stored_traffic(w.name)
    traffic = st["traffic_bytes_per_step"] if st else None
    if w.tokens <= 64:
        roofline = {"bound": "hbm", "kernel": "decode linear (skinny_kernel), all GEMM launches of a step",
                    "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                    "launches_per_step": sum(work[k][0] for k in gemm_ops), "us_per_step": round(gemm_us, 2)}
    else:
        tflops = flops_step / (gemm_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "kernel": "prefill linear (tiled_dma64_kernel / tiled_dma_kernel), all GEMM launches of a step",
                    "achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                    "launches_per_step": sum(work[k][0] for k in gemm_ops), "us_per_step": round(gemm_us, 2)}
    roofline["algorithmic_bytes_per_step"] = gemm_bytes_step
    roofline["traffic_unit"] = "HBM bytes over the launches of one step (rocprofv3 FETCH_SIZE + WRITE_SIZE, " \
                               "scaled by a plain copy of known size)"
    if st:
        roofline["traffic_over_algorithmic"] = st["traffic_over_algorithmic"]

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "t": w.t, "rank": 0, "tokens": w.tokens, "layers": w.layers,
                   "hidden": w.hidden, "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "intermediate": w.intermediate,
                   "vocab": w.vocab if w.has_vocab else None, "lm_positions": w.lm_positions if w.has_vocab else 0,
                   "parallelism": f"tp{w.t} rank share on 1 GPU",
                   "execution": "eager launches" if args.eager else "HIP graph of the step",
                   "calls": ("fused SwiGLU and reduce epilogues" if fused_reduce else
                             "fused SwiGLU epilogue" if fused else "separate calls")},
        "roofline": roofline,
        "reduce": {"GBps": red["GBps"], "frac": round(red["GBps"] / HBM_PEAK_GBPS, 4),
                   "us_per_call": red["us_per_launch"], "calls_per_step": work["reduce"][0],
                   "bytes_per_call": work["reduce"][2],
                   "sequence": {"calls": len(red_ops), "eager_us_per_call": round(red_eager_us, 3),
                                "graph_us_per_call": round(red_graph_us, 3)},
                   "note": ("latency-bound at this size: a launch and one memory round trip "
                            f"({work['reduce'][2] / 8e12 * 1e6:.2f} us of HBM time per call)")
                   if work["reduce"][2] < (8 << 20) else "bandwidth-bound"},
        "eager_ms_per_step": round(ms_eager, 4),
        "gemm_only_TFLOPs": round(flops_step / (gemm_us * 1e-6) / 1e12, 2),
        # the four per-layer linears alone (no embedding, LM head or
        # concatenation): the workload's shard-GEMM figure proper
        "layer_linears": layer_linears(work, per_op, gemm_ops),
        "step_GBps": round(sum(work[k][0] * work[k][2] for k in names) / (ms_step * 1e-3) / 1e9, 1),
        "partial_storage_ms_per_step": partials,
        "alt_path": {"calls": "separate" if fused else "fused", "ms_per_step": round(ms_alt, 4),
                     "value": round(flops_step / (ms_alt * 1e-3) / 1e12, 3)},
        "with_norms": {"calls": "input norm; per layer qkv, o partial, sum + residual add + RMSNorm "
                                "(tp_reduce_add_rmsnorm), gate_up + SwiGLU, down partial, sum + add + norm",
                       "ms_per_step": round(ms_norm, 4), "value": round(flops_step / (ms_norm * 1e-3) / 1e12, 3),
                       "reduce_norm_us_per_call": round(us_norm, 3),
                       "reduce_norm_GBps": round(work["reduce_norm"][2] / (us_norm * 1e-6) / 1e9, 1),
                       "fused": None if ms_norm_fused is None else {
                           "calls": "per layer tp_rmsnorm_column_linear (qkv), tp_row_linear_reduce_add (o), "
                                    "tp_rmsnorm_column_linear_swiglu (gate_up), tp_row_linear_reduce_add (down); "
                                    "the final norm inside the LM head's linear",
                           "ms_per_step": round(ms_norm_fused, 4),
                           "value": round(flops_step / (ms_norm_fused * 1e-3) / 1e12, 3)}},
        "full_layer": None if not layer_ops else {
            "calls": ("with_norms' fused calls" if fused_norm else "with_norms' calls") +
                     " plus tp_decode_attention (KV append + attention) feeding o_proj; no rotary embedding",
            "ms_per_step": round(ms_layer, 4), "value": round(flops_step / (ms_layer * 1e-3) / 1e12, 3),
            "attention": attn},
        "per_op": per_op,
        "hbm_copy": copy,
        "wall_s_timed": round(wall_s, 3),
        "pages_context": pages_context(w),
    }

    if not args.no_cpu:
        note("GPU measurements")
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
