"""The decode step captured into a HIP graph and replayed: every replay gives
the bits of the same calls issued eagerly.

The step is the benchmark's call sequence at the Llama-3.1-8B t = 8 rank
shapes (16 tokens, two layers): the embedding shard and its sum over ranks,
then per layer qkv (K split across workgroups: arrival counters in the
workspace, which every launch must leave zero), o_proj with the sum over ranks
as its epilogue, gate_up with SwiGLU, down_proj with the sum, then the LM-head
shard and the concatenation of the vocabulary shards. A second sequence adds
what a whole layer does: the folded RMSNorms, the residual updated in place,
and the decode attention over the KV caches (its new token appended). The
graph is replayed several times with eager calls on the same workspace and
host synchronisations in between (a node that left a counter or a flag
behind, or a memset recorded into the graph, would show up as a replay that
differs). A replay starts from the same state: the residual is copied back
from a pristine buffer by a copy node at the start of the graph."""

import numpy as np
import pytest
import torch

from megatron_sharded_linears_amd import inputs as I
from megatron_sharded_linears_amd import lib

pytestmark = pytest.mark.gpu

DEV = "cuda"
CFG = {"hidden": 4096, "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128, "intermediate": 14336,
       "vocab": 128256}
T, M, LAYERS = 8, 16, 2
KV_LEN, KV_CAP = 300, 320


def _bits(t):
    return t.detach().view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else \
        t.detach().view(torch.int32).cpu().numpy()


def _state(seed):
    sh = {k: lib.tp_shard_shape(CFG, T, k) for k in lib.KIND}
    H = CFG["hidden"]
    n = lambda shape, std, s: I.device_normal_bf16(shape, std, seed + s, DEV)
    S = {"x": n((M, H), 1.0, 1), "ids": torch.randint(0, CFG["vocab"], (M,), dtype=torch.int32,
                                                       generator=torch.Generator().manual_seed(seed)).to(DEV),
         "embed": n(sh["embed"], 0.02, 2), "lm": n(sh["lm_head"], 0.02, 3),
         "peers_e": [n((M, H), 0.02, 4 + j) for j in range(T - 1)],
         "peer_logits": [n((M, sh["lm_head"][0]), 1.0, 20 + j) for j in range(T - 1)], "layers": []}
    d = CFG["head_dim"]
    nq = sh["o"][1] // d
    nkv = (sh["qkv"][0] // d - nq) // 2
    for l in range(LAYERS):
        s = 100 * (l + 1)
        S["layers"].append({
            "qkv": n(sh["qkv"], 0.02, s + 1), "o": n(sh["o"], 0.02, s + 2),
            "gate_up": n(sh["gate_up"], 0.02, s + 3), "down": n(sh["down"], 0.02, s + 4),
            "ctx": n((M, sh["o"][1]), 1.0, s + 5),
            "peers_o": [n((M, H), 0.5, s + 10 + j) for j in range(T - 1)],
            "peers_d": [n((M, H), 0.5, s + 30 + j) for j in range(T - 1)],
            "g_in": (1.0 + n((H,), 0.1, s + 6).float()).to(torch.bfloat16),
            "g_post": (1.0 + n((H,), 0.1, s + 7).float()).to(torch.bfloat16),
            "k": n((M, nkv, KV_CAP, d), 1.0, s + 8), "v": n((M, nkv, KV_CAP, d), 1.0, s + 9)})
    S["nq"] = nq
    S["lens"] = torch.full((M,), KV_LEN, dtype=torch.int32, device=DEV)
    bf = torch.bfloat16
    e = lambda *shape: torch.empty(shape, dtype=bf, device=DEV)
    S["out"] = {"ze": e(M, H), "h": e(M, H), "qkv": e(M, sh["qkv"][0]), "y1": e(M, H),
                "act": e(M, sh["gate_up"][0] // 2), "logits": e(M, sh["lm_head"][0]),
                "full": e(M, CFG["vocab"]), "ctx": e(M, sh["o"][1]), "res": e(M, H)}
    return S


def _fused_step(S):
    o = S["out"]
    lib.tp_vocab_embed(S["ids"], S["embed"], CFG["vocab"], T, 0, o["ze"])
    lib.tp_reduce_partials([o["ze"]] + S["peers_e"], o["h"])
    cur = S["x"]
    for L in S["layers"]:
        lib.tp_column_linear(cur, L["qkv"], o["qkv"])
        lib.tp_row_linear_reduce(L["ctx"], L["o"], [None] + L["peers_o"], 0, o["y1"])
        lib.tp_column_linear_swiglu(o["y1"], L["gate_up"], o["act"])
        lib.tp_row_linear_reduce(o["act"], L["down"], [None] + L["peers_d"], 0, o["h"])
        cur = o["h"]
    lib.tp_lm_head_shard(o["h"], S["lm"], o["logits"])
    lib.tp_concat_logits([o["logits"]] + S["peer_logits"], CFG["vocab"], o["full"])


def _layer_step(S, pristine_res, folded):
    """Whole layers: norms folded into the linears, the residual in place,
    attention over the caches feeding o_proj."""
    o = S["out"]
    o["res"].copy_(pristine_res)
    for L, (wq, wgu) in zip(S["layers"], folded):
        lib.tp_rmsnorm_column_linear(o["res"], 1e-5, wq, o["qkv"])
        lib.tp_decode_attention(o["qkv"], L["k"], L["v"], S["lens"], S["nq"], o["ctx"])
        lib.tp_row_linear_reduce_add(o["ctx"], L["o"], [None] + L["peers_o"], 0, o["res"])
        lib.tp_rmsnorm_column_linear_swiglu(o["res"], 1e-5, wgu, o["act"])
        lib.tp_row_linear_reduce_add(o["act"], L["down"], [None] + L["peers_d"], 0, o["res"])


def _snapshot(S, keys):
    return {k: _bits(S["out"][k]) for k in keys}


def _spoil(S, keys):
    for k in keys:
        S["out"][k].fill_(float("nan"))


def _replays_match(S, step, keys, n_replays=4):
    """`keys`: the outputs the step writes."""
    step()                                  # eager: the reference bits
    torch.cuda.synchronize()
    want = _snapshot(S, keys)
    _spoil(S, keys)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    x = I.device_normal_bf16((M, CFG["hidden"]), 1.0, 999, DEV)
    w = S["layers"][0]["qkv"]
    y = torch.empty((M, w.shape[0]), dtype=torch.bfloat16, device=DEV)
    for r in range(n_replays):
        _spoil(S, keys)
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(S, keys)
        for k in want:
            assert np.array_equal(got[k], want[k]), f"replay {r}: {k} differs from the eager call"
        # eager work on the same default workspace between replays (its split-K
        # counters must be zero for the next replay as well)
        lib.tp_column_linear(x, w, y)
        torch.cuda.synchronize()
    del g


def test_fused_decode_step_graph_replays_give_the_eager_bits():
    S = _state(7100)
    _replays_match(S, lambda: _fused_step(S), ("ze", "h", "qkv", "y1", "act", "logits", "full"))


def test_whole_layer_step_with_attention_graph_replays_give_the_eager_bits():
    S = _state(7200)
    folded = [(lib.tp_fold_norm_weight(L["qkv"], L["g_in"], torch.empty_like(L["qkv"])),
               lib.tp_fold_norm_weight(L["gate_up"], L["g_post"], torch.empty_like(L["gate_up"])))
              for L in S["layers"]]
    pristine = I.device_normal_bf16((M, CFG["hidden"]), 1.0, 7299, DEV)
    # the attention appends the new token at lens[b] in place: appending the
    # same K/V rows again is idempotent, so every replay sees the same caches
    _replays_match(S, lambda: _layer_step(S, pristine, folded), ("qkv", "ctx", "res", "act"))
