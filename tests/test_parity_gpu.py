"""GPU parity of every device call against the oracle, on seeded inputs, at
sizes the oracle finishes in seconds that span several tiles and ragged
tails. Bit-exact for copies, indexing and exact-integer inputs; within the
linear tolerance (max|d| <= 2e-2 max|ref|, L1 ratio <= 5e-3) for random data.
"""

import numpy as np
import pytest
import torch

import oracle
from megatron_sharded_linears_amd import inputs as I
from megatron_sharded_linears_amd.workloads import WORKLOADS
from parity import assert_close, assert_within_bf16_ulps, bits, f64

pytestmark = pytest.mark.gpu

from megatron_sharded_linears_amd import lib  # noqa: E402  (fails loudly if the library is not built)
DEV = "cuda"
SEED = 9000


def dev(t):
    return t.to(DEV)


def empty(shape, dtype=torch.bfloat16):
    return torch.empty(shape, dtype=dtype, device=DEV)


# ------------------------------------------------------------ S1 shard copy

SHARD_CFGS = [
    # (cfg, t): tiny workload; KV replication (n_kv < t); MQA; padded vocab
    ({"hidden": 256, "num_q_heads": 8, "num_kv_heads": 2, "head_dim": 32, "intermediate": 1024, "vocab": 1000}, 2),
    ({"hidden": 64, "num_q_heads": 8, "num_kv_heads": 2, "head_dim": 16, "intermediate": 128, "vocab": 1001}, 4),
    ({"hidden": 64, "num_q_heads": 16, "num_kv_heads": 8, "head_dim": 8, "intermediate": 256, "vocab": 7}, 16),
    ({"hidden": 32, "num_q_heads": 4, "num_kv_heads": 1, "head_dim": 8, "intermediate": 64, "vocab": 5}, 4),
    ({"hidden": 128, "num_q_heads": 4, "num_kv_heads": 4, "head_dim": 16, "intermediate": 96, "vocab": 1000}, 1),
]


@pytest.mark.parametrize("ci", range(len(SHARD_CFGS)))
def test_shard_weights_bitexact(ci):
    cfg, t = SHARD_CFGS[ci]
    for kind in lib.KIND:
        full = I.normal_bf16((SEED, ci, lib.KIND[kind]), lib.tp_full_shape(cfg, kind), 0.02)
        full_d = dev(full)
        full64 = f64(full)
        for r in range(t):
            shard = empty(lib.tp_shard_shape(cfg, t, kind))
            shard.fill_(float("nan"))           # every element must be written
            lib.tp_shard_weights(cfg, t, r, kind, full_d, shard)
            want = oracle.shard_weight(kind, full64, cfg, t, r)
            got = shard.cpu()
            assert np.array_equal(bits(got), oracle.bf16_bits(want)), (kind, r)


# ------------------------------------------------- linears, exact integers

LIN_SHAPES = [
    # (M, N, K): decode path (M <= 64) and tiled path (M > 64), ragged tails
    (1, 7, 8), (5, 64, 40), (16, 100, 264), (16, 771, 1032), (17, 33, 72),
    (33, 200, 520), (64, 64, 4104), (64, 129, 136),
    (65, 70, 64), (130, 257, 200), (300, 128, 1032), (256, 384, 4096),
    # 17-32 tokens on a weight of LM-head size: the 64 x 64 tiled kernel
    (24, 8200, 2048), (32, 8192, 2112),
    # 17-32 tokens on the decode kernel: the 64-token plans (K split in two
    # launches), and the 32-token tiles for long rows with K in (1024, 2048]
    (24, 768, 4096), (29, 1800, 4104), (32, 2100, 1792),
]


@pytest.mark.parametrize("M,N,K", LIN_SHAPES)
def test_linear_exact_integer_mode(M, N, K):
    """Inputs in {-1, 0, 1}: every partial sum is an integer below 2^24, so
    the fp32 result is exact whatever the summation order and split."""
    x = I.small_int_bf16((SEED, 1, M, N, K), (M, K))
    w = I.small_int_bf16((SEED, 2, M, N, K), (N, K))
    ref = oracle.linear(f64(x), f64(w))
    y32 = empty((M, N), torch.float32)
    lib.tp_row_linear_partial(dev(x), dev(w), y32)
    assert np.array_equal(f64(y32), ref)
    yb = empty((M, N))
    lib.tp_column_linear(dev(x), dev(w), yb)
    assert np.array_equal(bits(yb), oracle.bf16_bits(oracle.round_bf16(ref)))


# every decode-kernel variant the library builds: (ksteps, nwn, nwk, x_direct)
SKINNY_VARIANTS = (
    [v + (0,) for v in [(4, 4, 1), (8, 4, 1), (4, 2, 2), (8, 2, 2), (4, 1, 4), (8, 1, 4), (4, 4, 2), (8, 4, 2),
                        (8, 4, 4), (4, 4, 4), (8, 1, 8), (8, 2, 8), (4, 2, 8), (4, 1, 16), (8, 1, 16),
                        (16, 1, 8), (16, 2, 4), (16, 4, 2)]]
    + [v + (1,) for v in [(4, 1, 4), (8, 1, 4), (8, 1, 8), (4, 1, 16), (8, 1, 16), (16, 1, 8), (4, 2, 8)]]
    + [(20, 1, 8, 0), (7, 1, 8, 0), (7, 1, 8, 1)]
    + [(2, 1, 4, 1), (7, 1, 4, 0), (7, 1, 4, 1)])     # these three are built for 33-64 tokens only


@pytest.mark.parametrize("ks,nn,nk,xd", SKINNY_VARIANTS)
def test_every_decode_kernel_variant_exact_and_deterministic(ks, nn, nk, xd):
    plan = {"decode": (ks, nn, nk, xd)}
    for (M, N, K) in [(16, 768, 4096), (64, 200, 1032), (3, 50, 520), (40, 96, 8192)]:
        x = I.small_int_bf16((SEED, 3, M, N, K), (M, K))
        w = I.small_int_bf16((SEED, 4, M, N, K), (N, K))
        ref = oracle.linear(f64(x), f64(w))
        xd_, wd = dev(x), dev(w)
        y1 = empty((M, N), torch.float32)
        y2 = empty((M, N), torch.float32)
        lib.tp_row_linear_partial(xd_, wd, y1, plan=plan)
        lib.tp_row_linear_partial(xd_, wd, y2, plan=plan)
        assert np.array_equal(f64(y1), ref), (M, N, K)
        # random values too: must be bitwise reproducible (fixed split order)
        xr = dev(I.normal_bf16((SEED, 5, M, K), (M, K)))
        wr = dev(I.normal_bf16((SEED, 6, N, K), (N, K), 0.02))
        lib.tp_row_linear_partial(xr, wr, y1, plan=plan)
        lib.tp_row_linear_partial(xr, wr, y2, plan=plan)
        assert torch.equal(y1, y2)
        assert_close(f64(y1), oracle.linear(f64(xr.cpu()), f64(wr.cpu())), f"variant {(ks, nn, nk, xd)} {(M, N, K)}")


@pytest.mark.parametrize("M,N,K", [(16, 6000, 4096), (3, 8008, 4104)])
def test_persistent_decode_grid_with_xcd_tile_order(M, N, K):
    """More 16-row tiles than resident workgroups (K = 4096 keeps one
    LDS-staged workgroup per CU): workgroups loop over tiles in the XCD-
    contiguous order, the last round partly filled. Exact on integers."""
    x = I.small_int_bf16((SEED, 40, M, N, K), (M, K))
    w = I.small_int_bf16((SEED, 41, M, N, K), (N, K))
    y = empty((M, N), torch.float32)
    y.fill_(float("nan"))
    lib.tp_row_linear_partial(dev(x), dev(w), y)
    assert np.array_equal(f64(y), oracle.linear(f64(x), f64(w)))


def test_split_k_partials_are_never_stale():
    """Heavily split variants reuse one workspace call after call: every call
    gets new inputs, so a partial read before its writer's store was visible
    (a stale value from the previous call) would break exactness."""
    for variant in [(4, 4, 1, 0), (4, 2, 2, 0), (8, 4, 2, 0)]:
        for it in range(6):
            M, N, K = (16, 1000, 4096) if it % 2 == 0 else (40, 777, 2056)
            x = I.small_int_bf16((SEED, 30, it) + variant, (M, K))
            w = I.small_int_bf16((SEED, 31, it) + variant, (N, K))
            y = empty((M, N), torch.float32)
            lib.tp_row_linear_partial(dev(x), dev(w), y, plan={"decode": variant})
            assert np.array_equal(f64(y), oracle.linear(f64(x), f64(w))), (variant, it)


@pytest.mark.parametrize("variant", list(range(lib.tp_prefill_tile_count())))
def test_every_prefill_tile_shape_exact(variant):
    """Every tiled kernel shape (an explicit tile plan runs it at any token
    count, decode sizes included)."""
    plan = {"tile": variant}
    for (M, N, K) in [(65, 70, 64), (300, 257, 200), (512, 768, 1032), (2048, 300, 640), (130, 1024, 4096),
                      (700, 520, 96), (257, 4100, 32), (300, 257, 192), (129, 130, 128),
                      (64, 520, 4096), (33, 130, 128), (16, 70, 64), (1, 257, 256)]:
        x = I.small_int_bf16((SEED, 40, M, N, K), (M, K))
        w = I.small_int_bf16((SEED, 41, M, N, K), (N, K))
        y = empty((M, N), torch.float32)
        lib.tp_row_linear_partial(dev(x), dev(w), y, plan=plan)
        assert np.array_equal(f64(y), oracle.linear(f64(x), f64(w))), (variant, M, N, K)
        b = I.normal_bf16((SEED, 42, N), (N,))
        yb = empty((M, N))
        xr, wr = I.normal_bf16((SEED, 43, M, K), (M, K)), I.normal_bf16((SEED, 44, N, K), (N, K), 0.02)
        lib.tp_column_linear(dev(xr), dev(wr), yb, bias=dev(b), plan=plan)
        assert_close(f64(yb), oracle.linear(f64(xr), f64(wr), f64(b)), f"tile {variant} {(M, N, K)}")


@pytest.mark.parametrize("N", [12008, 14336])
def test_weight_row_split_exact(N):
    """2048 tokens and between one and two waves of 256 x 256 tiles: the
    planner runs one whole wave of them on the first weight rows and 192 x 256
    tiles on the rest (a ragged last tile at N = 12008). Exact-integer inputs
    (|sums| <= 64, exact in bf16 too): the fp32 row partial and the bf16
    column linear with bias against the oracle, every element, and one launch
    of 256 x 256 tiles over the whole product gives the same bits."""
    M, K = 2048, 64
    x = dev(I.small_int_bf16((SEED, 60, N), (M, K)))
    w = dev(I.small_int_bf16((SEED, 61, N), (N, K)))
    b = dev(I.small_int_bf16((SEED, 62, N), (N,)))
    ref = oracle.linear(f64(x), f64(w))
    y = empty((M, N), torch.float32)
    y.fill_(float("nan"))
    lib.tp_row_linear_partial(x, w, y)
    assert np.array_equal(f64(y), ref), N
    yb = empty((M, N))
    yb.fill_(float("nan"))
    lib.tp_column_linear(x, w, yb, bias=b)
    assert np.array_equal(f64(yb), ref + f64(b)[None, :]), N
    y8 = empty((M, N))
    lib.tp_column_linear(x, w, y8, bias=b, plan={"tile": 8})
    assert torch.equal(yb.view(torch.int16), y8.view(torch.int16)), N


# ------------------------------------------------ linears, random tolerance

@pytest.mark.parametrize("M,N,K", [(16, 768, 4096), (64, 1792, 4096), (1, 1000, 256), (200, 300, 512), (2048, 256, 1024)])
def test_column_linear_random_with_bias(M, N, K):
    x = I.normal_bf16((SEED, 7, M, N, K), (M, K))
    w = I.normal_bf16((SEED, 8, M, N, K), (N, K), 0.02)
    b = I.normal_bf16((SEED, 9, N), (N,))
    y = empty((M, N))
    lib.tp_column_linear(dev(x), dev(w), y, bias=dev(b))
    ref = oracle.linear(f64(x), f64(w), f64(b))
    assert_close(f64(y), ref, "column_linear")


def test_lm_head_fp32_logits_and_zero_padded_rows():
    cfg = {"hidden": 256, "num_q_heads": 8, "num_kv_heads": 2, "head_dim": 32, "intermediate": 1024, "vocab": 1001}
    t, M = 2, 16
    W = I.normal_bf16((SEED, 10), (1001, 256), 0.02)
    h = I.normal_bf16((SEED, 11), (M, 256))
    full = oracle.linear(f64(h), f64(W))
    shards = []
    for r in range(t):
        ws = empty(lib.tp_shard_shape(cfg, t, "lm_head"))
        lib.tp_shard_weights(cfg, t, r, "lm_head", dev(W), ws)
        lg = empty((M, ws.shape[0]), torch.float32)
        lib.tp_lm_head_shard(dev(h), ws, lg)
        shards.append(lg)
    out = empty((M, 1001), torch.float32)
    lib.tp_concat_logits(shards, 1001, out)
    assert_close(f64(out), full, "lm_head")
    assert np.all(f64(shards[1])[:, 500] == 0.0)       # the padded row of the last shard


@pytest.mark.parametrize("V,t", [(1000, 2), (1001, 4), (7, 4)])
def test_tied_embedding_and_lm_head_share_one_shard(V, t):
    """Tied input embedding and LM head (one [V, H] table): the vocab split
    gives both the same rows, so one shard buffer serves tp_vocab_embed and
    tp_lm_head_shard. The embed and lm_head shard copies are bit-identical,
    the summed lookups equal E[ids] and the concatenated logits equal h E^T."""
    H, M = 64, 16
    cfg = {"hidden": H, "num_q_heads": t, "num_kv_heads": 1, "head_dim": 8, "intermediate": 8 * t, "vocab": V}
    E = I.normal_bf16((SEED, 40, V, t), (V, H), 0.02)
    ids = I.uniform_ids((SEED, 41, V, t), M, V)
    h = I.normal_bf16((SEED, 42, V, t), (M, H))
    parts, logits = [], []
    for r in range(t):
        es = empty(lib.tp_shard_shape(cfg, t, "embed"))
        lib.tp_shard_weights(cfg, t, r, "embed", dev(E), es)
        ls = empty(lib.tp_shard_shape(cfg, t, "lm_head"))
        lib.tp_shard_weights(cfg, t, r, "lm_head", dev(E), ls)
        assert np.array_equal(bits(es), bits(ls)), r
        z = empty((M, H))
        lib.tp_vocab_embed(dev(ids), es, V, t, r, z)
        parts.append(z)
        lg = empty((M, es.shape[0]))
        lib.tp_lm_head_shard(dev(h), es, lg)
        logits.append(lg)
    total = empty((M, H))
    lib.tp_reduce_partials(parts, total)
    assert np.array_equal(bits(total), oracle.bf16_bits(oracle.embedding_lookup(f64(E), ids.numpy())))
    out = empty((M, V))
    lib.tp_concat_logits(logits, V, out)
    assert_close(f64(out), oracle.linear(f64(h), f64(E)), "tied lm_head")


# ------------------------------------------------------------------ S4 swiglu

@pytest.mark.parametrize("M,Is", [(16, 512), (3, 8), (64, 896), (2048, 1792)])
def test_swiglu(M, Is):
    gu = I.normal_bf16((SEED, 12, M, Is), (M, 2 * Is), 3.0)
    g64 = f64(gu)
    out = empty((M, Is))
    lib.tp_swiglu(dev(gu), out)
    ref = oracle.swiglu(g64[:, :Is], g64[:, Is:])
    assert_within_bf16_ulps(f64(out), ref, 1, "swiglu")


def test_swiglu_special_values():
    g = torch.tensor([0.0, 1.0, -1.0, 80.0, -80.0, -0.0, 1e-30, 20.0], dtype=torch.float32)
    u = torch.tensor([1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1.0, -2.0], dtype=torch.float32)
    gu = torch.cat([g, u]).view(1, 16).to(torch.bfloat16)
    out = empty((1, 8))
    lib.tp_swiglu(dev(gu), out)
    ref = oracle.swiglu(f64(gu)[:, :8], f64(gu)[:, 8:])
    assert_within_bf16_ulps(f64(out), ref, 1, "swiglu special")
    assert f64(out)[0, 0] == 0.0


# ------------------------------------------------------------------ reduce

@pytest.mark.parametrize("t", [1, 2, 3, 8, 16, 64])
@pytest.mark.parametrize("numel", [8, 13, 4096 * 16, 100003])
def test_reduce_integer_exact_and_random(t, numel):
    parts = [I.small_int_bf16((SEED, 13, t, numel, i), (numel,), -8, 8) for i in range(t)]
    out = empty((numel,))
    lib.tp_reduce_partials([dev(p) for p in parts], out)
    ref = oracle.all_reduce_sum([f64(p) for p in parts])
    assert np.array_equal(f64(out), ref)
    parts = [I.normal_bf16((SEED, 14, t, numel, i), (numel,)) for i in range(t)]
    outf = empty((numel,), torch.float32)
    lib.tp_reduce_partials([dev(p) for p in parts], outf)
    assert_close(f64(outf), oracle.all_reduce_sum([f64(p) for p in parts]), "reduce fp32 out")
    if t == 1:
        lib.tp_reduce_partials([dev(parts[0])], out)
        assert np.array_equal(bits(out), bits(parts[0]))


@pytest.mark.parametrize("t", [2, 3, 8])
def test_reduce_wide_launch_ragged(t):
    """Sums of at least 65536 vectors run the wide launch (512 threads, two
    vectors per thread): a length whose last block is partly empty and whose
    last 5 elements fall outside the 8-element vectors."""
    numel = 65536 * 8 + 8 * 1023 + 5
    parts = [I.small_int_bf16((SEED, 18, t, i), (numel,), -8, 8) for i in range(t)]
    out = empty((numel,))
    lib.tp_reduce_partials([dev(p) for p in parts], out)
    assert np.array_equal(f64(out), oracle.all_reduce_sum([f64(p) for p in parts]))


def test_reduce_fp32_partials_in_place_and_signed_zero():
    t, n = 4, 4096 + 5
    parts = [dev(I.normal_bf16((SEED, 15, i), (n,)).float()) for i in range(t)]
    ref = oracle.all_reduce_sum([f64(p) for p in parts])
    out = empty((n,))
    lib.tp_reduce_partials(parts, out)
    assert_within_bf16_ulps(f64(out), ref, 1, "reduce fp32->bf16")
    lib.tp_reduce_partials(parts, parts[0])             # in place, like an in-place all-reduce
    assert_close(f64(parts[0]), ref, "reduce in place")
    z = [dev(torch.full((16,), -0.0, dtype=torch.bfloat16)) for _ in range(3)]
    out = empty((16,))
    lib.tp_reduce_partials(z, out)
    assert np.all(bits(out) == 0x8000)


# ----------------------------------------------------- S9 vocab embedding

EMBED_CASES = [(1000, 2, 256), (1001, 2, 64), (1000, 3, 64), (7, 4, 32), (5, 4, 16), (128256, 16, 64)]


@pytest.mark.parametrize("V,t,H", EMBED_CASES)
def test_vocab_embed_bitexact(V, t, H):
    cfg = {"hidden": H, "num_q_heads": t, "num_kv_heads": 1, "head_dim": 8, "intermediate": 8 * t, "vocab": V}
    E = I.normal_bf16((SEED, 16, V, t), (V, H), 0.02)
    E[min(2, V - 1), 1] = -0.0
    E[min(3, V - 1), 2] = 2.0 ** -130                      # bf16 subnormal
    ids = I.uniform_ids((SEED, 17, V, t), 64, V)
    ids[:6] = torch.tensor([0, V - 1, min(V - 1, (V + t - 1) // t), -1, V, 2 ** 30], dtype=torch.int32)
    vs = lib.tp_vocab_shard_rows(V, t)
    parts = []
    for r in range(t):
        es = empty((vs, H))
        lib.tp_shard_weights(cfg, t, r, "embed", dev(E), es)
        es[max(0, min(V - r * vs, vs)):] = float("nan")    # padded rows: NaN sentinels, never read
        z = empty((64, H))
        lib.tp_vocab_embed(dev(ids), es, V, t, r, z)
        want = oracle.vocab_embed_shard(f64(E), ids.numpy(), t, r)
        assert np.array_equal(bits(z), oracle.bf16_bits(want)), r
        parts.append(z)
    total = empty((64, H))
    lib.tp_reduce_partials(parts, total)
    direct = oracle.embedding_lookup(f64(E), ids.numpy())
    assert np.array_equal(bits(total), oracle.bf16_bits(direct))


# --------------------------------------------------------- S11 concat

@pytest.mark.parametrize("V,t,dt", [(1000, 2, torch.bfloat16), (1001, 2, torch.float32), (7, 4, torch.bfloat16),
                                    (128256, 16, torch.bfloat16), (152064, 8, torch.float32), (5, 4, torch.float32)])
def test_concat_logits_bitexact(V, t, dt):
    M = 5
    vs = -(-V // t)
    shards = [I.normal_bf16((SEED, 18, V, t, r), (M, vs)).to(dt) for r in range(t)]
    out = empty((M, V), dt)
    lib.tp_concat_logits([dev(s) for s in shards], V, out)
    want = oracle.all_gather_concat([s.float().numpy() for s in shards], V)
    assert np.array_equal(out.cpu().float().numpy(), want)


# ------------------------------------------------ tiny workload, whole chain

def test_tiny_workload_layer_chain():
    w = WORKLOADS[0]
    cfg, t, M, H, I_ = w.cfg(), w.t, w.tokens, w.hidden, w.intermediate
    key = (SEED, 19)
    X = I.normal_bf16(key + (I.T_X,), (M, H))
    Cx = I.normal_bf16(key + (I.T_CTX,), (M, w.num_q_heads * w.head_dim))
    Wf = {k: I.normal_bf16(key + (j,), lib.tp_full_shape(cfg, k), 0.02)
          for j, k in ((I.T_QKV, "qkv"), (I.T_O, "o"), (I.T_GATE_UP, "gate_up"), (I.T_DOWN, "down"))}
    ref = oracle.layer_linear_path(f64(X), f64(Cx), f64(Wf["qkv"]), f64(Wf["o"]), f64(Wf["gate_up"]),
                                   f64(Wf["down"]), I_)
    Xd, Cd = dev(X), dev(Cx)
    o_parts, d_parts, acts = [], [], []
    for r in range(t):
        sh = {}
        for k in Wf:
            sh[k] = empty(lib.tp_shard_shape(cfg, t, k))
            lib.tp_shard_weights(cfg, t, r, k, dev(Wf[k]), sh[k])
        qkv = empty((M, sh["qkv"].shape[0]))
        lib.tp_column_linear(Xd, sh["qkv"], qkv)
        rows = oracle.qkv_shard_rows(w.num_q_heads, w.num_kv_heads, w.head_dim, t, r)
        assert_close(f64(qkv), ref["qkv"][:, rows], f"qkv rank {r}")
        c_r = Cd[:, r * sh["o"].shape[1]:(r + 1) * sh["o"].shape[1]].contiguous()
        po = empty((M, H))
        lib.tp_row_linear_partial(c_r, sh["o"], po)
        o_parts.append(po)
        gu = empty((M, sh["gate_up"].shape[0]))
        lib.tp_column_linear(Xd, sh["gate_up"], gu)
        assert_close(f64(gu), ref["gate_up"][:, oracle.gate_up_shard_rows(I_, t, r)], f"gate_up rank {r}")
        a = empty((M, I_ // t))
        lib.tp_swiglu(gu, a)
        assert_close(f64(a), ref["act"][:, oracle.down_shard_cols(I_, t, r)], f"act rank {r}")
        pd = empty((M, H))
        lib.tp_row_linear_partial(a, sh["down"], pd)
        d_parts.append(pd)
    o = empty((M, H))
    lib.tp_reduce_partials(o_parts, o)
    assert_close(f64(o), ref["o"], "o after reduce")
    d = empty((M, H))
    lib.tp_reduce_partials(d_parts, d)
    assert_close(f64(d), ref["down"], "down after reduce")


def test_one_hip_runtime_in_process():
    torch.zeros(1, device=DEV)
    maps = open("/proc/self/maps").read()
    libs = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(libs) == 1, libs
    assert any("libtpshard.so" in l for l in maps.splitlines())
