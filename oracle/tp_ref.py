"""Unsharded reference for one tensor-parallel rank's share of a Llama-style
decoder layer's linear path.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does, and this
module imports nothing from the product package.

Pages cited (by title and section):
  [P1] "第 9 章 多进程与张量并行" (zero-to-sglang), sections 2.2, 3.1, 3.2.
  [P2] "Tensor Parallelism 执行路径" (SGLang internals), the weight-split
       diagram, "前向执行的实际流程" and "KV Cache 在 TP 下怎样分布".
  [P3] "张量、流水线与数据并行", sections "线性层怎么切",
       "每 token 的通信量（估算）" and "流水线并行".

Everything is plain NumPy in float64. Inputs are arrays of any float type
(bf16 values upcast exactly); results are float64 and are not rounded unless a
function says so. Where the path stores an activation in bf16 the caller (or
``layer_linear_path``) applies ``round_bf16`` explicitly.

Layout convention: a weight is stored [out, in] and a linear computes
Y = X W^T. [P1 3.2] calls the output dimension a "row"; the column-parallel
split is therefore a split of the output (first) axis and the row-parallel
split a split of the input (second) axis.
"""

import math

import numpy as np

from .bf16 import round_bf16


# ---------------------------------------------------------------------------
# The unsharded operations
# ---------------------------------------------------------------------------

def linear(x, w, bias=None):
    """Y = X W^T (+ b) in float64.

    [P1 2.2]: one GPU computes the whole product Y = XW. [P3 线性层怎么切]: a
    column shard computes Y_i = X A_i. With W stored [out, in] the product is
    X W^T. ``bias`` (length out) is added to every row, [P1 3.2] (bias is split
    with the weight along the output dimension).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError(f"linear: x {x.shape} and w {w.shape} do not contract")
    y = x @ w.T
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y


def silu(g):
    """silu(g) = g * sigmoid(g) = g / (1 + exp(-g)), float64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(gate, up):
    """SiLU(gate) x up, elementwise. [P3 线性层怎么切], layer diagram: the
    gate_up projection is followed by "SiLU × up" before down_proj."""
    gate = np.asarray(gate, dtype=np.float64)
    up = np.asarray(up, dtype=np.float64)
    if gate.shape != up.shape:
        raise ValueError("swiglu: gate and up differ in shape")
    return silu(gate) * up


def all_reduce_sum(partials):
    """Y = Y_0 + Y_1 + ... + Y_{p-1}, summed in float64 in rank order.

    [P1 3.1]: the row-parallel layer's All-Reduce sums the ranks' tensors.
    [P2 前向执行的实际流程] Step 3: the all-reduce adds the ranks' partial
    outputs [batch, seq, d_model] into the full output."""
    acc = np.array(np.asarray(partials[0], dtype=np.float64), copy=True)
    for p in partials[1:]:
        acc = acc + np.asarray(p, dtype=np.float64)
    return acc


def all_gather_concat(shards, vocab):
    """Y = cat(Y_0, ..., Y_{p-1}) along the vocab (last) axis, cut to ``vocab``
    columns. [P1 3.1] (All-Gather concatenates logits in vocab order);
    [P3 线性层怎么切] (the lm_head shards' V/t logits are gathered into the full
    V). Columns past ``vocab`` are the padding of the last shard."""
    cat = np.concatenate([np.asarray(s) for s in shards], axis=-1)
    if cat.shape[-1] < vocab:
        raise ValueError("all_gather_concat: shards cover fewer than vocab columns")
    return cat[..., :vocab]


def embedding_lookup(table, ids):
    """Direct lookup E[id] of the unsharded table.

    Ids outside [0, V) are not defined by the pages. Reading taken: such an id
    yields a row of zeros, and the zero is -0.0, because a vocab-parallel lookup
    masks the id in every shard and the sum of masked rows is the sum of zeros
    written by each shard (see ``vocab_embed_shard``)."""
    table = np.asarray(table, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    V, H = table.shape
    out = np.full((ids.shape[0], H), -0.0, dtype=np.float64)
    ok = (ids >= 0) & (ids < V)
    out[ok] = table[ids[ok]]
    return out


def rms_norm(x, gamma, eps):
    """RMSNorm of each row, float64: y[m, j] = x[m, j] / sqrt(mean_k x[m, k]^2
    + eps) * gamma[j].

    [P1 3.2]: RMSNorm is not split; every rank keeps the whole norm and
    applies it to the whole (replicated) hidden row. The pages name the norm
    but do not write it out; the reading taken is the usual root-mean-square
    definition, mean over the hidden axis, eps inside the square root, the
    per-column weight gamma applied after the scaling."""
    x = np.asarray(x, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    if x.ndim != 2 or gamma.shape != (x.shape[1],):
        raise ValueError(f"rms_norm: x {x.shape} and gamma {gamma.shape} do not match")
    if not (eps >= 0.0 and math.isfinite(eps)):
        raise ValueError("rms_norm: eps must be finite and >= 0")
    ms = np.mean(x * x, axis=1, keepdims=True)
    return x / np.sqrt(ms + eps) * gamma[None, :]


def add_rms_norm(x, residual, gamma, eps):
    """Residual add, then RMSNorm, as a rank applies them after the all-reduce
    of a row-parallel output ([P1 3.2]: the norm replicated on every rank;
    [P3 流水线并行]: the residual is carried beside hidden_states).

    h = bf16(residual + x): the residual stream is a stored activation and is
    held in bf16 like every activation on this path. Returns (h, rms_norm(h))
    in float64, the second not rounded. ``x`` may be None (no add: h =
    residual)."""
    residual = np.asarray(residual, dtype=np.float64)
    h = residual if x is None else round_bf16(residual + np.asarray(x, dtype=np.float64))
    return h, rms_norm(h, gamma, eps)


def gqa_decode_attention(q, k_cache, v_cache, lens, num_q_heads, num_kv_heads):
    """One decode step of grouped-query attention for the heads a rank holds,
    float64.

    [P2 前向执行的实际流程] Step 2 and [P2 KV Cache 在 TP 下怎样分布]: a rank
    computes attention for its own Q heads against the K and V of its own KV
    heads, with no exchange; [P3 线性层怎么切]: with fewer KV heads than ranks a
    KV head is replicated, so the rank's Q heads all read it. The pages do not
    write the attention itself; the reading taken is scaled dot-product
    attention, softmax over positions of q . k / sqrt(d), no rotary
    embedding, no mask beyond the sequence's length.

    q: [B, num_q_heads, d]; k_cache, v_cache: [B, num_kv_heads, L, d]; lens:
    [B] — sequence b attends to positions 0 .. lens[b] - 1 (lens[b] >= 1).
    Q head h reads KV head h // (num_q_heads // num_kv_heads).
    Returns [B, num_q_heads, d]."""
    q = np.asarray(q, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    B, nq, d = q.shape
    if nq != num_q_heads or num_q_heads % num_kv_heads != 0 or k_cache.shape[1] != num_kv_heads:
        raise ValueError("gqa_decode_attention: head counts do not match")
    group = num_q_heads // num_kv_heads
    out = np.zeros((B, nq, d))
    for b in range(B):
        n = int(lens[b])
        if n < 1 or n > k_cache.shape[2]:
            raise ValueError("gqa_decode_attention: lens[b] outside [1, L]")
        for h in range(nq):
            kv = h // group
            s = k_cache[b, kv, :n] @ q[b, h] / math.sqrt(d)
            p = np.exp(s - s.max())
            out[b, h] = (p / p.sum()) @ v_cache[b, kv, :n]
    return out


def append_kv(k_cache, v_cache, k_new, v_new, lens):
    """The decode step's cache write: the new token's K and V of sequence b go
    to position lens[b] (the cache grows by one; [P2 KV Cache 在 TP 下怎样分布]:
    each rank writes only its own KV heads). Returns new arrays.
    k_new, v_new: [B, num_kv_heads, d]."""
    k = np.array(np.asarray(k_cache, dtype=np.float64), copy=True)
    v = np.array(np.asarray(v_cache, dtype=np.float64), copy=True)
    for b in range(k.shape[0]):
        k[b, :, int(lens[b])] = np.asarray(k_new, dtype=np.float64)[b]
        v[b, :, int(lens[b])] = np.asarray(v_new, dtype=np.float64)[b]
    return k, v


# ---------------------------------------------------------------------------
# How each weight is split: the oracle's own head and vocab maps
# ---------------------------------------------------------------------------

def q_heads_of_rank(num_q_heads, t, rank):
    """Query heads held by ``rank``: an even split by head.

    [P1 3.2] (attention heads): query heads are split along the head dimension
    and num_attention_heads % tp_size == 0 is required. [P2 前向执行的实际流程]
    Step 2: rank 0 computes heads 0..H/4-1, rank 1 the next H/4, and so on."""
    if num_q_heads % t:
        raise ValueError("num_q_heads must be divisible by t")
    per = num_q_heads // t
    return list(range(rank * per, (rank + 1) * per))


def kv_heads_of_rank(num_kv_heads, t, rank):
    """Key/value heads held by ``rank``.

    [P1 3.2]: with num_kv_heads >= tp_size the KV heads are split by head,
    num_kv_heads // tp_size per rank; with num_kv_heads < tp_size a head cannot
    be split and is replicated so that several ranks share one. [P3 线性层怎么切]:
    below t KV heads the per-card KV stops shrinking (num_kv_head_replicas).

    Readings taken where the pages are silent: the split case needs
    num_kv_heads % t == 0; the replicated case needs t % num_kv_heads == 0, and
    consecutive ranks share a head, so that every query head of a rank keeps
    the KV head of its GQA group (see ``gqa_group``)."""
    if num_kv_heads >= t:
        if num_kv_heads % t:
            raise ValueError("num_kv_heads must be divisible by t when >= t")
        per = num_kv_heads // t
        return list(range(rank * per, (rank + 1) * per))
    if t % num_kv_heads:
        raise ValueError("t must be a multiple of num_kv_heads when num_kv_heads < t")
    ranks_per_head = t // num_kv_heads
    return [rank // ranks_per_head]


def gqa_group(q_head, num_q_heads, num_kv_heads):
    """KV head that query head ``q_head`` attends with under grouped-query
    attention: query heads are grouped in consecutive runs of n_h / n_kv."""
    return q_head // (num_q_heads // num_kv_heads)


def vocab_shard_rows(vocab, t):
    """Rows per vocab shard. [P1 3.2] (Vocab Parallel): the vocab is padded
    up to a multiple of tp_size and split evenly, so each shard has ceil(V/t)
    rows and the padded vocab is t * ceil(V/t)."""
    return -(-vocab // t)


def vocab_range_of_rank(vocab, t, rank):
    """[lo, hi) of real vocab ids held by ``rank`` (hi <= V; may be empty for
    the last ranks when the padding exceeds a shard)."""
    vs = vocab_shard_rows(vocab, t)
    lo = rank * vs
    return lo, min(lo + vs, vocab)


# ---------------------------------------------------------------------------
# Expected shards of each full weight (index gathers with explicit row lists)
# ---------------------------------------------------------------------------

def qkv_shard_rows(num_q_heads, num_kv_heads, head_dim, t, rank):
    """Row indices of the fused QKV weight [(n_h + 2 n_kv) d, H] that make up
    rank ``rank``'s shard, in the order Q heads, then K heads, then V heads.
    [P1 3.2]; [P3 线性层怎么切] (each card holds n_h/t Q heads and n_kv/t KV
    heads)."""
    rows = []
    for h in q_heads_of_rank(num_q_heads, t, rank):
        rows.extend(range(h * head_dim, (h + 1) * head_dim))
    k_base = num_q_heads * head_dim
    v_base = (num_q_heads + num_kv_heads) * head_dim
    kv = kv_heads_of_rank(num_kv_heads, t, rank)
    for g in kv:
        rows.extend(range(k_base + g * head_dim, k_base + (g + 1) * head_dim))
    for g in kv:
        rows.extend(range(v_base + g * head_dim, v_base + (g + 1) * head_dim))
    return rows


def gate_up_shard_rows(intermediate, t, rank):
    """Row indices of the fused [gate (I); up (I)] weight held by ``rank``:
    its slice of the gate rows followed by the matching slice of the up rows,
    so that SiLU(gate) x up is local to the rank ([P3 线性层怎么切], the
    activation sits between the column-split gate_up and the row-split down
    with no communication). Needs I % t == 0 (reading)."""
    if intermediate % t:
        raise ValueError("intermediate must be divisible by t")
    per = intermediate // t
    gate = list(range(rank * per, (rank + 1) * per))
    return gate + [intermediate + i for i in gate]


def o_shard_cols(num_q_heads, head_dim, t, rank):
    """Input columns of o_proj [H, n_h d] held by ``rank``: the context
    columns of its own query heads. [P1 3.2] (Row Parallel: the input is the
    previous layer's local result)."""
    cols = []
    for h in q_heads_of_rank(num_q_heads, t, rank):
        cols.extend(range(h * head_dim, (h + 1) * head_dim))
    return cols


def down_shard_cols(intermediate, t, rank):
    """Input columns of down_proj [H, I] held by ``rank``: the same slice of
    the intermediate dimension that its gate_up shard produces."""
    per = intermediate // t
    return list(range(rank * per, (rank + 1) * per))


def vocab_shard(table, t, rank):
    """Rank ``rank``'s rows of a [V, H] vocab table (embedding or LM head),
    ceil(V/t) of them, the padding past V filled with zeros (reading: the pages
    pad the vocab but do not say with what)."""
    table = np.asarray(table, dtype=np.float64)
    V, H = table.shape
    vs = vocab_shard_rows(V, t)
    lo, hi = vocab_range_of_rank(V, t, rank)
    out = np.zeros((vs, H), dtype=np.float64)
    if hi > lo:
        out[: hi - lo] = table[lo:hi]
    return out


def shard_weight(kind, full, cfg, t, rank):
    """Expected shard of a full weight. ``kind`` is one of 'qkv', 'o',
    'gate_up', 'down', 'embed', 'lm_head'; ``cfg`` is a mapping with hidden,
    num_q_heads, num_kv_heads, head_dim, intermediate, vocab."""
    full = np.asarray(full)
    if kind == "qkv":
        rows = qkv_shard_rows(cfg["num_q_heads"], cfg["num_kv_heads"], cfg["head_dim"], t, rank)
        return full[rows, :]
    if kind == "gate_up":
        return full[gate_up_shard_rows(cfg["intermediate"], t, rank), :]
    if kind == "o":
        return full[:, o_shard_cols(cfg["num_q_heads"], cfg["head_dim"], t, rank)]
    if kind == "down":
        return full[:, down_shard_cols(cfg["intermediate"], t, rank)]
    if kind in ("embed", "lm_head"):
        return vocab_shard(full, t, rank)
    raise ValueError(f"unknown weight kind {kind!r}")


# ---------------------------------------------------------------------------
# Per-rank operations, defined from the unsharded ones
# ---------------------------------------------------------------------------

def vocab_embed_shard(table, ids, t, rank):
    """What shard ``rank`` contributes to the vocab-parallel embedding: the
    row of the full table for ids inside its range, a zero row otherwise.
    [P1 3.2] (each rank can look up only its own vocab range);
    [P3 线性层怎么切] (look up, then one all-reduce).

    Reading: the zero is written as -0.0. It is an exact additive identity
    for every value including +0.0 and -0.0, so the sum over shards reproduces
    the owning shard's bits exactly; a +0.0 would turn an owned -0.0 into +0.0.
    Ids outside [0, V) are masked in every shard, so padded rows are never
    read."""
    table = np.asarray(table, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    V, H = table.shape
    lo, hi = vocab_range_of_rank(V, t, rank)
    out = np.full((ids.shape[0], H), -0.0, dtype=np.float64)
    own = (ids >= lo) & (ids < hi)
    out[own] = table[ids[own]]
    return out


def vocab_embed_from_shard(shard_table, ids, vocab, t, rank):
    """The same contribution computed from the rank's own padded shard table
    [ceil(V/t), H] (what a rank holds after loading): local row id - lo for
    the ids it owns, -0.0 rows otherwise. Padded rows of the shard table are
    never read, because ownership is bounded by min(hi, V)."""
    shard_table = np.asarray(shard_table, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    lo, hi = vocab_range_of_rank(vocab, t, rank)
    out = np.full((ids.shape[0], shard_table.shape[1]), -0.0, dtype=np.float64)
    own = (ids >= lo) & (ids < hi)
    out[own] = shard_table[ids[own] - lo]
    return out


def column_linear_rank(x, w_full, rows, bias_full=None):
    """Rank output of a column-parallel linear: the columns ``rows`` of the
    full product X W^T. [P3 线性层怎么切] (Y_i = X A_i, no communication,
    output stays sharded)."""
    y = linear(x, w_full, bias_full)
    return y[:, rows]


def row_linear_rank_partial(x_full, w_full, cols):
    """Rank partial of a row-parallel linear: X[:, cols] W[:, cols]^T.
    [P1 3.2] (Row Parallel); [P2 前向执行的实际流程] Step 3 (output_partial)."""
    x_full = np.asarray(x_full, dtype=np.float64)
    w_full = np.asarray(w_full, dtype=np.float64)
    return linear(x_full[:, cols], w_full[:, cols])


# ---------------------------------------------------------------------------
# The whole linear path of one decoder layer (unsharded)
# ---------------------------------------------------------------------------

def layer_linear_path(x, context, w_qkv, w_o, w_gate_up, w_down, intermediate):
    """The four linears of one Llama decoder layer and the activation between
    them, unsharded, with every activation the path stores held in bf16.

    [P3 线性层怎么切], layer diagram: hidden -> qkv_proj (column) -> attention
    -> o_proj (row) -> all-reduce 1 -> gate_up (column) -> SiLU x up ->
    down_proj (row) -> all-reduce 2.

    Attention is not on this path: ``context`` stands in for its output
    [M, n_h d]. gate_up reads the same hidden ``x`` as qkv (no norm or residual
    on this path). Returns a dict of float64 arrays:
      qkv     = bf16(X Wqkv^T)
      o       = bf16(C Wo^T)                  (value after all-reduce 1)
      gate_up = bf16(X Wgu^T)
      act     = bf16(silu(gate) * up) of the stored gate_up
      down    = bf16(act Wd^T)                (value after all-reduce 2)
    """
    qkv = round_bf16(linear(x, w_qkv))
    o = round_bf16(linear(context, w_o))
    gu = round_bf16(linear(x, w_gate_up))
    act = round_bf16(swiglu(gu[:, :intermediate], gu[:, intermediate:]))
    down = round_bf16(linear(act, w_down))
    return {"qkv": qkv, "o": o, "gate_up": gu, "act": act, "down": down}
