"""Full-size parity: every call of the benchmark's step at each workload's
full shapes (Llama-3.1-8B t = 8 decode of 16 tokens, t = 2 prefill of 2048,
t = 16 decode of 64 with KV heads replicated, Qwen2.5-32B t = 8 prefill of
4096), through the same calls, the same workspace size and so the same
automatic kernel choice the benchmark times, with every output element
compared against the oracle:

* tp_shard_weights on full weights of every kind, bit for bit against the
  oracle's shard of the same full weight (every rank for QKV, so every KV
  replica of the t = 16 split);
* exact-integer mode, on every rank of the split. Activations and weights in
  {-1, 0, 1} make every fp32 sum an exact integer below 2^24, whatever the
  summation order, tile or K split, so each bf16 result is that integer
  rounded once and has unique bits. The pages' invariants then hold exactly
  at full size: the column-parallel outputs of all ranks, gathered in the
  oracle's head order, are the unsharded X W^T ([P3 线性层怎么切]: Y_i = X A_i);
  the row-parallel partials of all t ranks, summed in rank order, are the
  unsharded product ([P1 3.1] All-Reduce; [P2 前向执行的实际流程]:
  output_partial then AllReduce); the LM-head shards concatenated are the
  full logits ([P1 3.1] All-Gather). SwiGLU, the one inexact step (an
  exponential), is held to one bf16 unit of the exact value's rounding;
* the vocab-parallel embedding over the full vocabulary: each shard's masked
  rows and their sum over all shards bit for bit against the oracle's
  per-shard contribution and direct lookup;
* random data of the benchmark's distributions (weights N(0, 0.02),
  activations N(0, 1)), every element within the linear bar (max|d| <= 2e-2
  max|ref|, L1 ratio <= 5e-3): every layer of the decode workloads, layer 0
  of the prefill ones.
"""

import numpy as np
import pytest
import torch

import oracle
from megatron_sharded_linears_amd import inputs as I
from megatron_sharded_linears_amd.workloads import WORKLOADS
from parity import assert_close, assert_within_bf16_ulps, bits, f64

pytestmark = pytest.mark.gpu

from megatron_sharded_linears_amd import lib  # noqa: E402

DEV = "cuda"
FULL = [w for w in WORKLOADS if w.layers > 1]
VOCAB = [w for w in FULL if w.has_vocab]
IDS = [w.name for w in FULL]


def ints(shape, seed):
    return I.device_small_int_bf16(shape, seed, device=DEV)


def normal(shape, std, seed):
    return I.device_normal_bf16(shape, std, seed, DEV)


def empty(shape, dtype=torch.bfloat16):
    t = torch.empty(shape, dtype=dtype, device=DEV)
    t.fill_(float("nan"))                     # every element must be written
    return t


def shard(cfg, t, r, kind, full):
    s = torch.empty(lib.tp_shard_shape(cfg, t, kind), dtype=torch.bfloat16, device=DEV)
    lib.tp_shard_weights(cfg, t, r, kind, full, s)
    return s


def u16(x):
    """uint16 bit patterns of a bf16 tensor, on the host."""
    return bits(x)


def rounded_bits(ref):
    return oracle.bf16_bits(oracle.round_bf16(ref))


def o_cols(w, r):
    return oracle.o_shard_cols(w.num_q_heads, w.head_dim, w.t, r)


def down_cols(w, r):
    return oracle.down_shard_cols(w.intermediate, w.t, r)


# --------------------------------------------------------------- S1 shards

@pytest.mark.parametrize("w", FULL, ids=IDS)
def test_shard_weights_full_size_bitexact(w):
    cfg, t = w.cfg(), w.t
    seed = 20000 + 100 * w.index
    kinds = [("qkv", range(t)), ("o", sorted({0, t // 2, t - 1})), ("gate_up", sorted({0, t // 2, t - 1})),
             ("down", sorted({0, t // 2, t - 1}))]
    if w.has_vocab:
        kinds += [("lm_head", [0, t - 1]), ("embed", [t // 2])]
    for j, (kind, ranks) in enumerate(kinds):
        full = normal(lib.tp_full_shape(cfg, kind), 0.02, seed + j)
        fb = u16(full)
        for r in ranks:
            got = u16(shard(cfg, t, r, kind, full))
            want = oracle.shard_weight(kind, fb, cfg, t, r)
            assert np.array_equal(got.astype(np.float64), np.asarray(want, dtype=np.float64)), (w.name, kind, r)
        del full, fb
        torch.cuda.empty_cache()


# ------------------------------------------- column-parallel, exact integers

@pytest.mark.parametrize("w", FULL, ids=IDS)
def test_qkv_all_ranks_exact_integer_full_size(w):
    """Every rank's qkv output (KV heads replicated at t = 16) equals the
    columns of the unsharded product for its heads, rounded once."""
    cfg, t, M, H = w.cfg(), w.t, w.tokens, w.hidden
    seed = 21000 + 100 * w.index
    X = ints((M, H), seed)
    Wq = ints(lib.tp_full_shape(cfg, "qkv"), seed + 1)
    Xh, Wh = f64(X), f64(Wq)
    for r in range(t):
        sq = shard(cfg, t, r, "qkv", Wq)
        y = empty((M, sq.shape[0]))
        lib.tp_column_linear(X, sq, y)
        rows = oracle.qkv_shard_rows(w.num_q_heads, w.num_kv_heads, w.head_dim, t, r)
        ref = oracle.linear(Xh, Wh[rows])
        assert np.array_equal(u16(y), rounded_bits(ref)), (w.name, r)


@pytest.mark.parametrize("w", FULL, ids=IDS)
def test_gate_up_swiglu_all_ranks_exact_integer_full_size(w):
    """Every rank's fused gate_up + SwiGLU output: gate and up are exact
    integers rounded once to bf16, so the only inexact step is SwiGLU's own;
    within one bf16 unit of the exact value's rounding. Where exp(-g)
    overflows fp32 (g < -88) the kernel's SiLU is -0 and the exact value is
    below 1e-30; that is the absolute slack."""
    cfg, t, M, H = w.cfg(), w.t, w.tokens, w.hidden
    seed = 22000 + 100 * w.index
    X = ints((M, H), seed)
    Wgu = ints(lib.tp_full_shape(cfg, "gate_up"), seed + 1)
    Xh = f64(X)
    Is = w.intermediate // t
    for r in range(t):
        s = shard(cfg, t, r, "gate_up", Wgu)
        act = empty((M, Is))
        lib.tp_column_linear_swiglu(X, s, act)
        rows = oracle.gate_up_shard_rows(w.intermediate, t, r)
        gu = oracle.linear(Xh, f64(Wgu[torch.as_tensor(rows, device=DEV)]))
        g, u = oracle.round_bf16(gu[:, :Is]), oracle.round_bf16(gu[:, Is:])
        assert_within_bf16_ulps(f64(act), oracle.swiglu(g, u), 1, f"{w.name} rank {r}", slack=1e-30)


# ---------------------------------------------- row-parallel, exact integers

def row_parallel_exact(w, kind, seed):
    cfg, t, M, H = w.cfg(), w.t, w.tokens, w.hidden
    K_full = lib.tp_full_shape(cfg, kind)[1]
    cols = o_cols if kind == "o" else down_cols
    X = ints((M, K_full), seed)
    Wf = ints(lib.tp_full_shape(cfg, kind), seed + 1)
    Xh, Wh = f64(X), f64(Wf)
    full_ref = oracle.linear(Xh, Wh)
    p32, p16, own_refs, xs, shards = [], [], [], [], []
    for r in range(t):
        cr = cols(w, r)
        xr = X[:, cr[0]:cr[-1] + 1].contiguous()
        sr = shard(cfg, t, r, kind, Wf)
        a, b = empty((M, H), torch.float32), empty((M, H))
        lib.tp_row_linear_partial(xr, sr, a)
        lib.tp_row_linear_partial(xr, sr, b)
        own = oracle.row_linear_rank_partial(Xh, Wh, cr)
        assert np.array_equal(f64(a), own), (w.name, kind, "fp32 partial", r)
        assert np.array_equal(u16(b), rounded_bits(own)), (w.name, kind, "bf16 partial", r)
        p32.append(a)
        p16.append(b)
        own_refs.append(own)
        xs.append(xr)
        shards.append(sr)
    # the sum of the t fp32 partials is the unsharded product, exactly
    s32 = empty((M, H), torch.float32)
    lib.tp_reduce_partials(p32, s32)
    assert np.array_equal(f64(s32), full_ref), (w.name, kind, "sum of fp32 partials")
    # bf16 partials: each rounded once, the in-order fp32 sum rounded once
    want16 = rounded_bits(oracle.all_reduce_sum([oracle.round_bf16(p) for p in own_refs]))
    s16 = empty((M, H))
    lib.tp_reduce_partials(p16, s16)
    assert np.array_equal(u16(s16), want16), (w.name, kind, "sum of bf16 partials")
    # the benchmark's call for this workload, from the first and last rank;
    # with fp32 partials beyond one launch's reach the rank's own partial is
    # staged in the workspace, which must then hold M H floats
    ws32 = None if M <= 64 else lib.make_workspace(lib.tp_workspace_bytes() + M * H * 4)
    for r in sorted({0, t - 1}):
        out = empty((M, H))
        lib.tp_row_linear_reduce(xs[r], shards[r], [None if i == r else p for i, p in enumerate(p16)], r, out)
        assert np.array_equal(u16(out), want16), (w.name, kind, "tp_row_linear_reduce, bf16 partials", r)
        out32 = empty((M, H))
        lib.tp_row_linear_reduce(xs[r], shards[r], [None if i == r else p for i, p in enumerate(p32)], r, out32,
                                 workspace=ws32)
        assert np.array_equal(u16(out32), rounded_bits(full_ref)), (w.name, kind, "fp32 partials", r)


@pytest.mark.parametrize("w", FULL, ids=IDS)
def test_o_proj_all_ranks_sum_to_unsharded_product_full_size(w):
    row_parallel_exact(w, "o", 23000 + 100 * w.index)


@pytest.mark.parametrize("w", FULL, ids=IDS)
def test_down_proj_all_ranks_sum_to_unsharded_product_full_size(w):
    row_parallel_exact(w, "down", 24000 + 100 * w.index)


# ------------------------------------------------------ vocab: embed, LM head

@pytest.mark.parametrize("w", VOCAB, ids=[w.name for w in VOCAB])
def test_vocab_embedding_all_shards_full_size_bitexact(w):
    """Every shard's masked lookup over the full vocabulary, and their sum,
    against the oracle (per-shard contribution and direct lookup). The host
    copy of the table holds only the rows the ids select (np.zeros pages
    that are never written are never allocated): the oracle reads no other."""
    cfg, t, M, H, V = w.cfg(), w.t, w.tokens, w.hidden, w.vocab
    seed = 25000 + 100 * w.index
    E = normal((V, H), 0.02, seed)
    Vs = lib.tp_vocab_shard_rows(V, t)
    ids = I.uniform_ids((seed, 1), M, V).numpy()
    edge = [0, Vs - 1, Vs, V - 1, (t - 1) * Vs, (t - 1) * Vs - 1]
    ids[:len(edge)] = edge[:M]
    table = np.zeros((V, H))
    uniq = np.unique(ids)
    table[uniq] = f64(E[torch.as_tensor(uniq, device=DEV)])
    ids_d = torch.from_numpy(ids.astype(np.int32)).to(DEV)
    parts = []
    for r in range(t):
        z = empty((M, H))
        lib.tp_vocab_embed(ids_d, shard(cfg, t, r, "embed", E), V, t, r, z)
        assert np.array_equal(u16(z), oracle.bf16_bits(oracle.vocab_embed_shard(table, ids, t, r))), (w.name, r)
        parts.append(z)
    out = empty((M, H))
    lib.tp_reduce_partials(parts, out)
    assert np.array_equal(u16(out), oracle.bf16_bits(oracle.embedding_lookup(table, ids))), w.name


@pytest.mark.parametrize("w", VOCAB, ids=[w.name for w in VOCAB])
def test_lm_head_all_shards_concat_exact_integer_full_size(w):
    """Every rank's LM-head shard on the sampled positions, concatenated in
    vocab order, equals the unsharded logits rounded once (exact integers);
    the oracle's product is taken over blocks of vocab rows (each logit
    depends on its own row only)."""
    cfg, t, H, V = w.cfg(), w.t, w.hidden, w.vocab
    Ms = w.lm_positions
    seed = 26000 + 100 * w.index
    Hs = ints((Ms, H), seed)
    Wlm = ints((V, H), seed + 1)
    Vs = lib.tp_vocab_shard_rows(V, t)
    logits = []
    for r in range(t):
        lg = empty((Ms, Vs))
        lib.tp_lm_head_shard(Hs, shard(cfg, t, r, "lm_head", Wlm), lg)
        logits.append(lg)
    full = empty((Ms, V))
    lib.tp_concat_logits(logits, V, full)
    got = u16(full)
    Hh = f64(Hs)
    for a in range(0, V, 16384):
        b = min(V, a + 16384)
        ref = oracle.linear(Hh, f64(Wlm[a:b]))
        assert np.array_equal(got[:, a:b], rounded_bits(ref)), (w.name, a)


# --------------------------------------------- random data, every element

def step_layer_random(w, layer, seed):
    """One layer of the benchmark's step on rank 0's shards with random data
    of the benchmark's distributions; every output element against the
    oracle within the linear bar."""
    cfg, t, M, H = w.cfg(), w.t, w.tokens, w.hidden
    sh = {k: lib.tp_shard_shape(cfg, t, k) for k in ("qkv", "o", "gate_up", "down")}
    fused_reduce = M <= 64                      # as the benchmark's step
    s = seed + 1000 * layer
    X = normal((M, H), 1.0, s + 1)
    Wq = normal(sh["qkv"], 0.02, s + 2)
    qkv = empty((M, sh["qkv"][0]))
    lib.tp_column_linear(X, Wq, qkv)
    Xh = f64(X)
    assert_close(f64(qkv), oracle.round_bf16(oracle.linear(Xh, f64(Wq))), f"{w.name} L{layer} qkv")

    def row_parallel(x, wt, peer_seed, what):
        peers = [normal((M, H), 0.5, peer_seed + j) for j in range(t - 1)]
        y = empty((M, H))
        if fused_reduce:
            lib.tp_row_linear_reduce(x, wt, [None] + peers, 0, y)
        else:
            p = empty((M, H))
            lib.tp_row_linear_partial(x, wt, p)
            lib.tp_reduce_partials([p] + peers, y)
        own = oracle.round_bf16(oracle.linear(f64(x), f64(wt)))
        ref = oracle.round_bf16(oracle.all_reduce_sum([own] + [f64(q) for q in peers]))
        assert_close(f64(y), ref, f"{w.name} L{layer} {what}")
        return y

    C = normal((M, sh["o"][1]), 1.0, s + 3)
    y1 = row_parallel(C, normal(sh["o"], 0.02, s + 4), s + 10, "o + sum over ranks")
    Wgu = normal(sh["gate_up"], 0.02, s + 5)
    Is = sh["gate_up"][0] // 2
    act = empty((M, Is))
    lib.tp_column_linear_swiglu(y1, Wgu, act)
    gu = oracle.round_bf16(oracle.linear(f64(y1), f64(Wgu)))
    assert_close(f64(act), oracle.round_bf16(oracle.swiglu(gu[:, :Is], gu[:, Is:])), f"{w.name} L{layer} gate_up + SwiGLU")
    row_parallel(act, normal(sh["down"], 0.02, s + 6), s + 40, "down + sum over ranks")


@pytest.mark.parametrize("w", FULL, ids=IDS)
def test_step_random_every_element(w):
    layers = range(w.layers) if w.tokens <= 64 else [0]
    for layer in layers:
        step_layer_random(w, layer, 27000 + 100 * w.index)


@pytest.mark.parametrize("w", VOCAB, ids=[w.name for w in VOCAB])
def test_lm_head_random_every_element(w):
    cfg, t, H = w.cfg(), w.t, w.hidden
    Ms = w.lm_positions
    seed = 28000 + 100 * w.index
    Hs = normal((Ms, H), 1.0, seed)
    Wlm = normal(lib.tp_shard_shape(cfg, t, "lm_head"), 0.02, seed + 1)
    lg = empty((Ms, Wlm.shape[0]))
    lib.tp_lm_head_shard(Hs, Wlm, lg)
    assert_close(f64(lg), oracle.round_bf16(oracle.linear(f64(Hs), f64(Wlm))), f"{w.name} lm_head")
