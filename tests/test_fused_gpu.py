"""The fused calls: tp_column_linear_swiglu (gate_up linear with SwiGLU as
its epilogue) and tp_row_linear_reduce (row-parallel linear with the sum over
ranks as its epilogue). Each must give the same bits as the two separate
calls it replaces — for every decode-kernel variant, both tiled shapes, split
and unsplit K — and match the oracle on exact-integer and random inputs."""

import numpy as np
import pytest
import torch

import oracle
from megatron_sharded_linears_amd import inputs as I
from parity import assert_close, assert_within_bf16_ulps, bits, f64

pytestmark = pytest.mark.gpu

from megatron_sharded_linears_amd import lib  # noqa: E402
from test_parity_gpu import SKINNY_VARIANTS  # noqa: E402

DEV = "cuda"
SEED = 9100


def dev(t):
    return t.to(DEV)


def empty(shape, dtype=torch.bfloat16):
    return torch.empty(shape, dtype=dtype, device=DEV)


def separate_swiglu(x, w, i_s, plan=None):
    gu = empty((x.shape[0], 2 * i_s))
    lib.tp_column_linear(x, w, gu, plan=plan)
    act = empty((x.shape[0], i_s))
    lib.tp_swiglu(gu, act)
    return act


def fused_swiglu(x, w, i_s, plan=None):
    act = empty((x.shape[0], i_s))
    act.fill_(float("nan"))                      # every element must be written
    lib.tp_column_linear_swiglu(x, w, act, plan=plan)
    return act


# (M, I_shard, K): Llama-8B t=8 decode (16, 1792, 4096) and t=16 (64, 896,
# 4096), ragged tails, the tiled path (M > 64) with 256- and 128-row tiles
SWIGLU_SHAPES = [(16, 1792, 4096), (64, 896, 4096), (1, 8, 64), (7, 904, 520), (33, 96, 1032),
                 (65, 136, 200), (300, 520, 256), (256, 1024, 2048), (130, 64, 4104), (24, 896, 4096)]


@pytest.mark.parametrize("M,Is,K", SWIGLU_SHAPES)
def test_column_linear_swiglu_same_bits_as_separate_calls(M, Is, K):
    x = dev(I.normal_bf16((SEED, 1, M, Is, K), (M, K)))
    w = dev(I.normal_bf16((SEED, 2, M, Is, K), (2 * Is, K), 0.05))
    got = fused_swiglu(x, w, Is)
    assert np.array_equal(bits(got), bits(separate_swiglu(x, w, Is))), (M, Is, K)
    # and the oracle's gate_up -> bf16 -> SwiGLU chain
    gu = oracle.round_bf16(oracle.linear(f64(x.cpu()), f64(w.cpu())))
    assert_close(f64(got), oracle.swiglu(gu[:, :Is], gu[:, Is:]), f"fused swiglu {(M, Is, K)}")


@pytest.mark.parametrize("variant", list(range(lib.tp_prefill_tile_count())))
def test_every_prefill_tile_shape_fused_swiglu(variant):
    """The SwiGLU epilogue pairs gate and up rows inside each tile (first
    and second half of its rows): every tile shape, ragged widths."""
    plan = {"tile": variant}
    for (M, Is, K) in [(300, 520, 256), (130, 200, 1024), (257, 96, 64)]:
        x = dev(I.normal_bf16((SEED, 20, M, Is, K), (M, K)))
        w = dev(I.normal_bf16((SEED, 21, M, Is, K), (2 * Is, K), 0.05))
        assert np.array_equal(bits(fused_swiglu(x, w, Is, plan)), bits(separate_swiglu(x, w, Is, plan))), \
            (variant, M, Is, K)


def test_weight_row_split_swiglu():
    """SwiGLU over the planner's weight-row split (2048 tokens, I_shard = 6008:
    256 x 256 tiles for the first 4096 gate/up row pairs, then 192 x 256 tiles
    with a ragged last one): the fused epilogue against the separate calls,
    bit for bit, every element written."""
    M, Is, K = 2048, 6008, 128
    x = dev(I.normal_bf16((SEED, 70, M, Is, K), (M, K)))
    w = dev(I.normal_bf16((SEED, 71, M, Is, K), (2 * Is, K), 0.05))
    assert np.array_equal(bits(fused_swiglu(x, w, Is)), bits(separate_swiglu(x, w, Is)))


@pytest.mark.parametrize("M,Is,K", [(16, 100, 256), (3, 13, 72), (64, 1, 8), (100, 37, 136)])
def test_column_linear_swiglu_ragged_width_exact_integer(M, Is, K):
    """I_shard not a multiple of 8 (no separate tp_swiglu to compare with):
    inputs in {-1, 0, 1} with K <= 256 make gate and up exact in bf16, so the
    only rounding is SwiGLU's own: within 1 bf16 ulp of the oracle."""
    x = I.small_int_bf16((SEED, 3, M, Is, K), (M, K))
    w = I.small_int_bf16((SEED, 4, M, Is, K), (2 * Is, K))
    got = fused_swiglu(dev(x), dev(w), Is)
    gu = oracle.linear(f64(x), f64(w))
    assert np.array_equal(gu, oracle.round_bf16(gu))
    assert_within_bf16_ulps(f64(got), oracle.swiglu(gu[:, :Is], gu[:, Is:]), 1, "ragged fused swiglu")


@pytest.mark.parametrize("ks,nn,nk,xd", SKINNY_VARIANTS)
def test_every_decode_variant_fused_epilogues(ks, nn, nk, xd):
    plan = {"decode": (ks, nn, nk, xd)}
    for (M, Is, K) in [(16, 136, 1032), (40, 48, 4104)]:
        x = dev(I.normal_bf16((SEED, 5, M, Is, K), (M, K)))
        w = dev(I.normal_bf16((SEED, 6, M, Is, K), (2 * Is, K), 0.05))
        assert np.array_equal(bits(fused_swiglu(x, w, Is, plan)), bits(separate_swiglu(x, w, Is, plan))), (M, Is, K)
    for (M, N, K, t, rank) in [(16, 200, 1032, 8, 3), (33, 64, 4104, 3, 0)]:
        x = dev(I.normal_bf16((SEED, 7, M, N, K), (M, K)))
        w = dev(I.normal_bf16((SEED, 8, M, N, K), (N, K), 0.05))
        for dt in (torch.bfloat16, torch.float32):
            peers = [dev(I.normal_bf16((SEED, 9, M, N, i), (M, N))).to(dt) for i in range(t)]
            summed = fused_reduce(x, w, peers, rank, plan)
            assert np.array_equal(bits(summed), bits(separate_reduce(x, w, peers, rank, plan))), \
                (M, N, K, t, rank, dt)
            # the residual-add epilogue: y = bf16(y + the bf16 sum over ranks)
            res = dev(I.normal_bf16((SEED, 10, M, N), (M, N)))
            want = (res.float() + summed.float()).to(torch.bfloat16)
            parts = [None if i == rank else p for i, p in enumerate(peers)]
            lib.tp_row_linear_reduce_add(x, w, parts, rank, res, plan=plan)
            assert np.array_equal(bits(res), bits(want)), (M, N, K, t, rank, dt, "add")


def separate_reduce(x, w, peers, rank, plan=None):
    """The rank's partial stored in the peers' dtype, then the reducer."""
    parts = list(peers)
    dt = next(p.dtype for i, p in enumerate(peers) if i != rank) if len(peers) > 1 else torch.bfloat16
    parts[rank] = empty((x.shape[0], w.shape[0]), dt)
    lib.tp_row_linear_partial(x, w, parts[rank], plan=plan)
    out = empty((x.shape[0], w.shape[0]))
    lib.tp_reduce_partials(parts, out)
    return out


def fused_reduce(x, w, peers, rank, plan=None):
    out = empty((x.shape[0], w.shape[0]))
    out.fill_(float("nan"))
    parts = list(peers)
    parts[rank] = None
    lib.tp_row_linear_reduce(x, w, parts, rank, out, plan=plan)
    return out


# (M, N, K_shard): Llama-8B t=8 o and down, t=16 o; ragged; tiled (M > 64)
REDUCE_SHAPES = [(16, 4096, 512), (16, 4096, 1792), (64, 4096, 256), (5, 100, 40), (33, 130, 264),
                 (100, 256, 128), (300, 72, 520), (24, 4096, 512), (32, 4096, 1792)]


@pytest.mark.parametrize("M,N,K", REDUCE_SHAPES)
@pytest.mark.parametrize("t", [1, 2, 3, 8, 16, 17])
def test_row_linear_reduce_same_bits_as_separate_calls(M, N, K, t):
    x = dev(I.normal_bf16((SEED, 10, M, N, K), (M, K)))
    w = dev(I.normal_bf16((SEED, 11, M, N, K), (N, K), 0.05))
    peers = [dev(I.normal_bf16((SEED, 12, M, N, t, i), (M, N), 0.5)) for i in range(t)]
    for rank in sorted({0, t // 2, t - 1}):
        got = fused_reduce(x, w, peers, rank)
        assert np.array_equal(bits(got), bits(separate_reduce(x, w, peers, rank))), (M, N, K, t, rank)
    # the oracle: own partial rounded to bf16, then the in-order sum
    own = oracle.round_bf16(oracle.linear(f64(x.cpu()), f64(w.cpu())))
    ps = [f64(p) for p in peers]
    ps[t - 1] = own
    assert_close(f64(got), oracle.all_reduce_sum(ps), f"fused reduce {(M, N, K, t)}")


# prefill sizes at one or two ranks, where the sum over ranks is the tiled
# kernel's epilogue: Llama-3.1-8B t = 2 o and down at 2048 tokens, and ragged
# token counts and widths over several tiles
PREFILL_REDUCE_SHAPES = [(2048, 4096, 2048), (2048, 4096, 7168), (333, 1000, 256), (129, 4100, 512), (65, 264, 64)]


@pytest.mark.parametrize("M,N,K", PREFILL_REDUCE_SHAPES)
@pytest.mark.parametrize("t", [1, 2])
def test_row_linear_reduce_prefill_same_bits_as_separate_calls(M, N, K, t):
    x = I.device_normal_bf16((M, K), 1.0, SEED + 40 + M + K, DEV)
    w = I.device_normal_bf16((N, K), 0.03, SEED + 41 + N + K, DEV)
    peers = [I.device_normal_bf16((M, N), 0.5, SEED + 42 + i, DEV) for i in range(t)]
    for rank in range(t):
        got = fused_reduce(x, w, peers, rank)
        assert np.array_equal(bits(got), bits(separate_reduce(x, w, peers, rank))), (M, N, K, t, rank)
    # the oracle on sampled rows (first, last and a spread between)
    rows = sorted(set(np.linspace(0, M - 1, min(M, 48)).astype(int).tolist()))
    own = oracle.round_bf16(oracle.linear(f64(x[rows].cpu()), f64(w.cpu())))
    ps = [f64(p[rows].cpu()) for p in peers]
    ps[t - 1] = own
    assert_close(f64(got[rows].cpu()), oracle.all_reduce_sum(ps), f"fused prefill reduce {(M, N, K, t)}")


@pytest.mark.parametrize("M,N,K,t", [(16, 4096, 192, 8), (64, 300, 72, 16), (90, 128, 200, 4), (1, 8, 8, 2),
                                     (300, 520, 192, 2), (129, 1000, 128, 1)])
def test_row_linear_reduce_exact_integer(M, N, K, t):
    """Small integers everywhere, sized so that the own partial (|p| <= K)
    and the sum (|s| <= K + 8 (t - 1)) stay within 256, where every integer
    is a bf16 value: the result equals the oracle exactly."""
    x = I.small_int_bf16((SEED, 13, M, N, K), (M, K))
    w = I.small_int_bf16((SEED, 14, M, N, K), (N, K))
    peers = [I.small_int_bf16((SEED, 15, M, N, i), (M, N), -8, 8) for i in range(t)]
    rank = t // 2
    got = fused_reduce(dev(x), dev(w), [dev(p) for p in peers], rank)
    ps = [f64(p) for p in peers]
    ps[rank] = oracle.linear(f64(x), f64(w))
    ref = oracle.all_reduce_sum(ps)
    assert np.all(np.abs(ref) <= 256)
    assert np.array_equal(f64(got), ref)


@pytest.mark.parametrize("M,N,K", REDUCE_SHAPES)
@pytest.mark.parametrize("t", [1, 2, 8, 16, 17])
def test_row_linear_reduce_fp32_partials_same_bits_as_separate_calls(M, N, K, t):
    """fp32 partial storage: the rank's own partial enters the sum as its
    fp32 accumulator (unrounded), as tp_row_linear_partial into an fp32
    buffer followed by tp_reduce_partials gives; one launch up to 16 ranks,
    two beyond (the own partial staged in the workspace)."""
    x = dev(I.normal_bf16((SEED, 30, M, N, K), (M, K)))
    w = dev(I.normal_bf16((SEED, 31, M, N, K), (N, K), 0.05))
    peers = [dev(I.normal_bf16((SEED, 32, M, N, t, i), (M, N), 0.5)).float() for i in range(t)]
    for rank in sorted({0, t - 1}):
        got = fused_reduce(x, w, peers, rank)
        assert np.array_equal(bits(got), bits(separate_reduce(x, w, peers, rank))), (M, N, K, t, rank)
    own = oracle.linear(f64(x.cpu()), f64(w.cpu()))
    ps = [f64(p) for p in peers]
    ps[t - 1] = own
    assert_close(f64(got), oracle.all_reduce_sum(ps), f"fused reduce fp32 {(M, N, K, t)}")


@pytest.mark.parametrize("M,N,K,t", [(16, 4096, 512, 8), (64, 300, 4104, 16), (90, 128, 200, 4), (16, 4096, 1792, 17)])
def test_row_linear_reduce_fp32_partials_exact_integer(M, N, K, t):
    """Integers in {-1, 0, 1} and peers in [-64, 64]: the fp32 own partial
    and the fp32 sum are exact integers (below 2^24), so the one rounding to
    bf16 is of the exact sum: bit-exact against the oracle."""
    x = I.small_int_bf16((SEED, 33, M, N, K), (M, K))
    w = I.small_int_bf16((SEED, 34, M, N, K), (N, K))
    peers = [I.small_int_bf16((SEED, 35, M, N, i), (M, N), -64, 64).float() for i in range(t)]
    rank = t // 2
    got = fused_reduce(dev(x), dev(w), [dev(p) for p in peers], rank)
    ps = [f64(p) for p in peers]
    ps[rank] = oracle.linear(f64(x), f64(w))
    ref = oracle.all_reduce_sum(ps)
    assert np.array_equal(bits(got), oracle.bf16_bits(oracle.round_bf16(ref)))


def test_row_linear_reduce_skipping_a_rank_fails_the_tolerance():
    """A planted mistake (one rank's partial left out of the sum, as a
    dropped all-reduce contribution would) is caught by the parity bar."""
    M, N, K, t, rank = 16, 512, 256, 4, 1
    x = dev(I.normal_bf16((SEED, 16), (M, K)))
    w = dev(I.normal_bf16((SEED, 17), (N, K), 0.05))
    peers = [dev(I.normal_bf16((SEED, 18, i), (M, N), 0.5)) for i in range(t)]
    got = f64(fused_reduce(x, w, peers, rank))
    own = oracle.round_bf16(oracle.linear(f64(x.cpu()), f64(w.cpu())))
    ps = [f64(p) for p in peers]
    ps[rank] = own
    assert_close(got, oracle.all_reduce_sum(ps), "fused reduce")
    with pytest.raises(AssertionError):
        assert_close(got, oracle.all_reduce_sum(ps[:2] + ps[3:]), "missing rank")
