"""Pins of the oracle to things other than itself: closed forms, exact
brute force, library routines in special cases, hand-worked cases from the
pages' split rules (tests/golden) and the sizes the pages print.

CPU only. Each test names the oracle function it pins.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import (
    round_bf16, bf16_bits, linear, silu, swiglu, all_reduce_sum, all_gather_concat,
    embedding_lookup, q_heads_of_rank, kv_heads_of_rank, gqa_group, vocab_shard_rows,
    vocab_range_of_rank, qkv_shard_rows, gate_up_shard_rows, o_shard_cols,
    down_shard_cols, shard_weight, vocab_embed_shard, vocab_embed_from_shard,
    layer_linear_path, rms_norm, add_rms_norm, gqa_decode_attention, append_kv,
)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- round_bf16

def _torch_bf16(x32):
    return torch.from_numpy(np.asarray(x32, dtype=np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


def test_round_bf16_matches_torch_cast_on_float32_inputs():
    rng = np.random.default_rng(1234)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ours = round_bf16(x.astype(np.float64))
    ref = _torch_bf16(x)
    assert np.array_equal(ours, ref)
    # signs of zeros too
    assert np.array_equal(np.signbit(ours), np.signbit(ref))


def test_round_bf16_ties_subnormals_overflow():
    # exact ties between two bf16 neighbours round to the even one
    one = 1.0
    ulp = 2.0 ** -7
    assert round_bf16(one + ulp / 2) == one                 # tie, 1.0 is even
    assert round_bf16(one + ulp + ulp / 2) == one + 2 * ulp  # tie, rounds up to even
    assert round_bf16(one + ulp / 2 + 2.0 ** -40) == one + ulp
    # subnormals: smallest bf16 subnormal is 2**-133
    tiny = 2.0 ** -133
    assert round_bf16(tiny) == tiny
    assert round_bf16(tiny / 2) == 0.0                      # tie to even (zero)
    assert round_bf16(tiny * 0.75) == tiny
    assert round_bf16(3 * tiny / 2) == 2 * tiny             # tie to even
    assert np.signbit(round_bf16(-tiny / 4))
    # largest finite bf16 and overflow
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127
    assert round_bf16(big) == big
    assert np.isinf(round_bf16(big + 2.0 ** 119))            # tie with 2**128: to even -> inf
    assert round_bf16(big + 2.0 ** 118) == big
    assert np.isnan(round_bf16(np.nan))
    assert round_bf16(-np.inf) == -np.inf
    assert bf16_bits(np.array([-0.0, 0.0, 1.0, -2.0])).tolist() == [0x8000, 0x0000, 0x3F80, 0xC000]


def test_round_bf16_float64_inputs_against_exact_rationals():
    # for float64 inputs, compare with an exact rational nearest-even search
    rng = np.random.default_rng(7)
    xs = rng.standard_normal(300) * 10.0 ** rng.integers(-5, 5, 300)
    for x in xs:
        fx = Fraction(float(x))
        e = math.frexp(abs(float(x)))[1] - 1
        ulp = Fraction(2) ** (max(e, -126) - 7)
        q = fx / ulp
        lo = math.floor(q)
        rem = q - lo
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
            lo += 1
        assert Fraction(float(round_bf16(x))) == lo * ulp


# --------------------------------------------------------------------- linear

def test_linear_equals_exact_rational_brute_force():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3, 5))
    w = rng.standard_normal((4, 5))
    b = rng.standard_normal(4)
    y = linear(x, w, b)
    for i in range(3):
        for j in range(4):
            terms = [Fraction(float(x[i, k])) * Fraction(float(w[j, k])) for k in range(5)]
            terms.append(Fraction(float(b[j])))
            exact = sum(terms)
            # floating-point dot product bound: |err| <= n u sum|terms|, u = 2**-53
            bound = len(terms) * Fraction(1, 2**53) * sum(abs(v) for v in terms)
            assert abs(Fraction(float(y[i, j])) - exact) <= bound


def test_linear_integer_inputs_exact_triple_loop():
    rng = np.random.default_rng(12)
    x = rng.integers(-3, 4, (6, 9)).astype(np.float64)
    w = rng.integers(-3, 4, (7, 9)).astype(np.float64)
    y = linear(x, w)
    for i in range(6):
        for j in range(7):
            assert y[i, j] == sum(int(x[i, k]) * int(w[j, k]) for k in range(9))
    # the output is indexed [token, out]: a transposed operand would change it
    assert y.shape == (6, 7)


def test_row_split_partials_sum_to_full_product():
    """[P1 3.1, 3.2] a row-parallel layer's partials, all-reduced, equal the
    unsharded product. Exact on integer inputs."""
    rng = np.random.default_rng(13)
    t = 4
    x = rng.integers(-2, 3, (5, 24)).astype(np.float64)
    w = rng.integers(-2, 3, (6, 24)).astype(np.float64)
    partials = [linear(x[:, r * 6:(r + 1) * 6], w[:, r * 6:(r + 1) * 6]) for r in range(t)]
    assert np.array_equal(all_reduce_sum(partials), linear(x, w))
    # a planted mistake: one partial missing from the sum (the pages: a missing
    # collective gives a badly wrong result) must break the identity
    assert not np.array_equal(all_reduce_sum(partials[:-1]), linear(x, w))


def test_column_split_concat_equals_full_product():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((5, 16))
    w = rng.standard_normal((12, 16))
    cols = [linear(x, w[r * 4:(r + 1) * 4]) for r in range(3)]
    full = linear(x, w)
    assert np.array_equal(np.concatenate(cols, axis=1), full)
    # swapping two shards breaks it
    swapped = np.concatenate([cols[1], cols[0], cols[2]], axis=1)
    assert not np.array_equal(swapped, full)


# --------------------------------------------------------------- silu/swiglu

def test_silu_closed_forms():
    assert silu(0.0) == 0.0
    sig1 = 0.7310585786300049        # 1 / (1 + e^-1)
    assert abs(silu(1.0) - sig1) < 1e-15
    assert abs(silu(-1.0) - (sig1 - 1.0)) < 1e-15   # silu(-x) = silu(x) - x
    assert silu(60.0) == pytest.approx(60.0, rel=1e-15)
    assert abs(silu(-60.0)) < 1e-24
    assert silu(-1e4) == 0.0 and np.signbit(silu(-1e4))


def test_silu_tanh_identity_and_library():
    from scipy.special import expit
    # 1 + tanh(x/2) cancels for very negative x: use it where it is well conditioned
    x = np.linspace(-4, 30, 2001)
    via_tanh = x * (1.0 + np.tanh(x / 2.0)) / 2.0
    assert np.allclose(silu(x), via_tanh, rtol=1e-13, atol=1e-300)
    x = np.linspace(-60, 60, 4001)
    assert np.allclose(silu(x), x * expit(x), rtol=1e-14, atol=1e-300)


def test_swiglu_is_silu_of_gate_times_up_not_the_reverse():
    g = np.array([[2.0, -1.0, 0.5]])
    u = np.array([[3.0, 4.0, -2.0]])
    out = swiglu(g, u)
    sig = 1.0 / (1.0 + np.exp(-g))
    assert np.allclose(out, g * sig * u, rtol=1e-15)
    assert not np.allclose(out, swiglu(u, g))


# ---------------------------------------------------------- reduce / concat

def test_all_reduce_sum_closed_form():
    parts = [np.full((3, 4), float(r + 1)) for r in range(8)]
    assert np.array_equal(all_reduce_sum(parts), np.full((3, 4), 36.0))
    assert np.array_equal(all_reduce_sum(parts[:1]), parts[0])     # t = 1: identity


def test_all_gather_concat_positions():
    shards = [np.array([[10 * r + j for j in range(3)]], dtype=np.float64) for r in range(3)]
    out = all_gather_concat(shards, vocab=8)
    assert out.tolist() == [[0, 1, 2, 10, 11, 12, 20, 21]]


# ----------------------------------------------------------- head/vocab maps

def test_head_maps_against_hand_worked_golden():
    g = _golden("shard_rules_tiny.json")
    for case in g["qkv"]:
        for r, rows in enumerate(case["rows"]):
            assert qkv_shard_rows(case["n_h"], case["n_kv"], case["d"], case["t"], r) == rows
    for case in g["gate_up"]:
        for r, rows in enumerate(case["rows"]):
            assert gate_up_shard_rows(case["I"], case["t"], r) == rows
    for case in g["o_cols"]:
        for r, cols in enumerate(case["cols"]):
            assert o_shard_cols(case["n_h"], case["d"], case["t"], r) == cols
    for case in g["down_cols"]:
        for r, cols in enumerate(case["cols"]):
            assert down_shard_cols(case["I"], case["t"], r) == cols
    for case in g["vocab"]:
        assert vocab_shard_rows(case["V"], case["t"]) == case["rows_per_shard"]
        for r, (lo, hi) in enumerate(case["ranges"]):
            a, b = vocab_range_of_rank(case["V"], case["t"], r)
            assert (a, max(a, b)) == (lo, hi)


def test_kv_per_card_matches_printed_sizes():
    """Page 3 prints the KV cache per token per card for Llama-3.1-8B:
    128 KiB in total, 64 KiB at t=2, 16 KiB at t=8, and no further shrink once
    the KV heads are fewer than t."""
    g = _golden("p3_traffic_estimates.json")
    layers = g["model"]["layers"]
    nkv = g["model"]["num_kv_heads"]
    total = g["kv_cache_per_token_per_card"]["total_KiB"] * 1024
    head_dim = total // (layers * nkv * 2 * 2)       # K and V, 2 bytes each
    assert head_dim == 128

    def per_card(t):
        heads = len(kv_heads_of_rank(nkv, t, 0))
        return layers * heads * head_dim * 2 * 2 // 1024

    for row in g["kv_cache_per_token_per_card"]["per_card_KiB"]:
        assert per_card(row["t"]) == row["KiB"]
    assert per_card(16) == per_card(8) == 16


def test_gqa_grouping_is_preserved_for_every_rank():
    for n_h, n_kv in [(32, 8), (40, 8), (8, 2), (4, 1), (16, 16)]:
        for t in [1, 2, 4, 8, 16, 32]:
            if n_h % t or (n_kv >= t and n_kv % t) or (n_kv < t and t % n_kv):
                continue
            owners = {}
            for r in range(t):
                kv = kv_heads_of_rank(n_kv, t, r)
                for h in q_heads_of_rank(n_h, t, r):
                    assert gqa_group(h, n_h, n_kv) in kv
                for g in kv:
                    owners.setdefault(g, []).append(r)
            # every KV head is held, by max(1, t / n_kv) consecutive ranks
            assert sorted(owners) == list(range(n_kv))
            for g, rs in owners.items():
                assert len(rs) == max(1, t // n_kv)
                assert rs == list(range(rs[0], rs[0] + len(rs)))


def test_split_preconditions_raise():
    with pytest.raises(ValueError):
        q_heads_of_rank(40, 16, 0)
    with pytest.raises(ValueError):
        kv_heads_of_rank(8, 3, 0)       # 3 <= 8 but 8 % 3 != 0
    with pytest.raises(ValueError):
        kv_heads_of_rank(2, 3, 0)       # replication needs t % n_kv == 0
    with pytest.raises(ValueError):
        gate_up_shard_rows(10, 4, 0)


def test_workload_shard_sizes():
    g = _golden("workload_shapes.json")
    for w in g["workloads"]:
        t, d = w["t"], w["head_dim"]
        cfg = {k: w[k] for k in ("hidden", "num_q_heads", "num_kv_heads", "head_dim", "intermediate", "vocab")}
        s = w["stated"]
        if "qkv_shard_cols" in s:
            assert len(qkv_shard_rows(w["num_q_heads"], w["num_kv_heads"], d, t, 0)) == s["qkv_shard_cols"]
        if "gate_up_shard" in s:
            assert len(gate_up_shard_rows(w["intermediate"], t, 0)) == s["gate_up_shard"]
        if "down_shard_in" in s:
            assert len(down_shard_cols(w["intermediate"], t, 0)) == s["down_shard_in"]
        if "vocab_rows_per_shard" in s:
            assert vocab_shard_rows(w["vocab"], t) == s["vocab_rows_per_shard"]
        if "q_heads_per_shard" in s:
            assert len(q_heads_of_rank(w["num_q_heads"], t, 0)) == s["q_heads_per_shard"]
        if "kv_heads_per_shard" in s:
            assert len(kv_heads_of_rank(w["num_kv_heads"], t, 0)) == s["kv_heads_per_shard"]
        if "ranks_per_kv_head" in s:
            shared = [r for r in range(t) if kv_heads_of_rank(w["num_kv_heads"], t, r) == [0]]
            assert len(shared) == s["ranks_per_kv_head"]
        if "reduce_partial_MiB_bf16" in s:
            assert w["tokens"] * w["hidden"] * 2 == s["reduce_partial_MiB_bf16"] * 2**20
        # every rank's shards of a full weight tile the full weight exactly once
        rows = sum((qkv_shard_rows(w["num_q_heads"], w["num_kv_heads"], d, t, r) for r in range(t)), [])
        qrows = [x for x in rows if x < w["num_q_heads"] * d]
        assert sorted(qrows) == list(range(w["num_q_heads"] * d))
        gu = sum((gate_up_shard_rows(w["intermediate"], t, r) for r in range(t)), [])
        assert sorted(gu) == list(range(2 * w["intermediate"]))


# ------------------------------------------------------------------ shards

def test_shard_weight_column_and_row_split_reassemble():
    cfg = {"hidden": 8, "num_q_heads": 4, "num_kv_heads": 2, "head_dim": 2, "intermediate": 6, "vocab": 7}
    t = 2
    rng = np.random.default_rng(21)
    wqkv = rng.integers(-3, 4, ((4 + 2 * 2) * 2, 8)).astype(np.float64)
    wo = rng.integers(-3, 4, (8, 4 * 2)).astype(np.float64)
    x = rng.integers(-3, 4, (3, 8)).astype(np.float64)
    c = rng.integers(-3, 4, (3, 8)).astype(np.float64)
    full_qkv = linear(x, wqkv)
    got = np.concatenate([linear(x, shard_weight("qkv", wqkv, cfg, t, r)) for r in range(t)], axis=1)
    want = np.concatenate([full_qkv[:, qkv_shard_rows(4, 2, 2, t, r)] for r in range(t)], axis=1)
    assert np.array_equal(got, want)
    cs = [c[:, o_shard_cols(4, 2, t, r)] for r in range(t)]
    parts = [linear(cs[r], shard_weight("o", wo, cfg, t, r)) for r in range(t)]
    assert np.array_equal(all_reduce_sum(parts), linear(c, wo))
    wd = rng.integers(-3, 4, (8, 6)).astype(np.float64)
    a = rng.integers(-3, 4, (3, 6)).astype(np.float64)
    parts = [linear(a[:, down_shard_cols(6, t, r)], shard_weight("down", wd, cfg, t, r)) for r in range(t)]
    assert np.array_equal(all_reduce_sum(parts), linear(a, wd))


# ------------------------------------------------------------------- embed

def test_masked_vocab_shards_sum_to_direct_lookup_bitwise():
    """[P1 3.2] each rank looks up only its own range; [P3] then all-reduce.
    The sum of the shards' rows must equal E[ids] bit for bit, including
    planted -0.0 and subnormal entries and NaN-filled padding."""
    V, H = 7, 5
    for t in (1, 2, 3, 4, 8):
        rng = np.random.default_rng(30 + t)
        table = round_bf16(rng.standard_normal((V, H)))
        table[2, 1] = -0.0
        table[3, 4] = 2.0 ** -130          # bf16 subnormal
        table[6, 0] = -(2.0 ** -133)
        ids = np.array([0, 6, 2, 3, 6, 1, 5, 4, 0, -1, 7, 100])
        shards = [vocab_embed_shard(table, ids, t, r) for r in range(t)]
        total = shards[0].copy()
        for s in shards[1:]:
            total = total + s
        direct = embedding_lookup(table, ids)
        assert np.array_equal(bf16_bits(total), bf16_bits(direct))
        assert np.array_equal(direct[:9], table[ids[:9]])
        # padding rows of the shard tables hold NaN sentinels: never read
        vs = vocab_shard_rows(V, t)
        padded = np.full((t * vs, H), np.nan)
        padded[:V] = table
        total_p = None
        for r in range(t):
            shard_tab = shard_weight("embed", table, {"vocab": V}, t, r)
            assert shard_tab.shape == (vs, H)
            lo, hi = vocab_range_of_rank(V, t, r)
            assert np.all(shard_tab[max(0, hi - lo):] == 0.0)        # zero padding
            z = vocab_embed_from_shard(padded[r * vs:(r + 1) * vs], ids, V, t, r)
            assert np.array_equal(bf16_bits(z), bf16_bits(shards[r]))
            total_p = z if total_p is None else total_p + z
        assert not np.isnan(total_p).any()
        assert not np.isnan(total).any()


def test_embedding_out_of_range_ids_give_negative_zero_rows():
    table = np.ones((4, 3))
    out = embedding_lookup(table, np.array([-1, 4, 2]))
    assert bf16_bits(out[:2]).tolist() == [[0x8000] * 3] * 2
    assert out[2].tolist() == [1.0, 1.0, 1.0]


# -------------------------------------------------------------- layer path

def test_layer_linear_path_integer_case_matches_hand_chain():
    rng = np.random.default_rng(40)
    M, H, I = 3, 8, 4
    x = rng.integers(-2, 3, (M, H)).astype(np.float64)
    c = rng.integers(-2, 3, (M, 6)).astype(np.float64)
    wqkv = rng.integers(-1, 2, (10, H)).astype(np.float64)
    wo = rng.integers(-1, 2, (H, 6)).astype(np.float64)
    wgu = rng.integers(-1, 2, (2 * I, H)).astype(np.float64)
    wd = rng.integers(-1, 2, (H, I)).astype(np.float64)
    out = layer_linear_path(x, c, wqkv, wo, wgu, wd, I)
    # integer products are small: bf16 storage is exact for them
    assert np.array_equal(out["qkv"], x @ wqkv.T)
    assert np.array_equal(out["o"], c @ wo.T)
    g = x @ wgu[:I].T
    u = x @ wgu[I:].T
    assert np.array_equal(out["gate_up"], np.concatenate([g, u], axis=1))
    act = round_bf16(g / (1 + np.exp(-g)) * u)
    assert np.array_equal(out["act"], act)
    assert np.array_equal(out["down"], round_bf16(act @ wd.T))


# ------------------------------------------------------- rms_norm / add_rms_norm

def test_rms_norm_closed_forms():
    # hand-worked row: mean(9, 16) = 12.5, so 3 and 4 scale by 1 / sqrt(12.5) = sqrt(2) / 5
    out = rms_norm([[3.0, 4.0]], [1.0, 1.0], 0.0)
    assert np.allclose(out, [[3 * math.sqrt(2) / 5, 4 * math.sqrt(2) / 5]], rtol=1e-15, atol=0)
    # a constant row keeps only its sign (eps = 0), scaled by gamma per column
    g = np.array([0.5, -1.0, 2.0, 3.0, 0.25, 1.0, -7.0])
    assert np.allclose(rms_norm(np.full((1, 7), -2.5), g, 0.0), -g[None, :], rtol=1e-15, atol=0)
    # ... and c / sqrt(c^2 + eps) with eps
    assert np.allclose(rms_norm([[1.0, 1.0]], [1.0, 1.0], 3.0), [[0.5, 0.5]], rtol=1e-15, atol=0)
    # a row whose mean square is 1 is only multiplied by gamma
    x = np.array([[1.0, -1.0, 1.0, -1.0]])
    g4 = np.array([2.0, 3.0, -4.0, 0.5])
    assert np.array_equal(rms_norm(x, g4, 0.0), x * g4)


def test_rms_norm_scale_invariance_rows_and_columns():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 64))
    g = rng.standard_normal(64)
    base = rms_norm(x, g, 0.0)
    for a in (1e-3, 0.37, 12.0, 4096.0):
        assert np.allclose(rms_norm(a * x, g, 0.0), base, rtol=1e-13, atol=0)
    # rows are normalised independently: rows of very different scale stacked
    # together give the same rows as alone (a mean over the wrong axis fails)
    y = np.vstack([x[:1] * 1e3, x[1:2] * 1e-3])
    assert np.allclose(rms_norm(y, g, 0.0)[0], rms_norm(x[:1], g, 0.0)[0], rtol=1e-13, atol=0)
    assert np.allclose(rms_norm(y, g, 0.0)[1], rms_norm(x[1:2], g, 0.0)[0], rtol=1e-13, atol=0)
    # gamma multiplies columns: in a square case the transposed reading differs
    sq = rng.standard_normal((6, 6))
    gs = np.arange(1.0, 7.0)
    out = rms_norm(sq, gs, 0.0)
    assert np.allclose(out / gs[None, :], rms_norm(sq, np.ones(6), 0.0), rtol=1e-13, atol=0)
    # every output row has mean square mean(gamma^2 * (x / rms)^2); with gamma = 1 it is 1
    assert np.allclose(np.mean(rms_norm(x, np.ones(64), 0.0) ** 2, axis=1), 1.0, rtol=1e-13, atol=0)
    # a larger eps shrinks every magnitude
    assert np.all(np.abs(rms_norm(x, g, 1e-1)) <= np.abs(rms_norm(x, g, 1e-6)) + 1e-300)


def test_rms_norm_matches_torch_in_float64():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((9, 40)) * rng.uniform(0.01, 100.0, size=(9, 1))
    g = rng.standard_normal(40)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (40,), torch.from_numpy(g), eps=1e-5).numpy()
    assert np.allclose(rms_norm(x, g, 1e-5), ref, rtol=1e-12, atol=1e-300)


def test_add_rms_norm_rounds_the_add_once():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: to even, 1
    h, _ = add_rms_norm([[2.0 ** -8]], [[1.0]], [1.0], 0.0)
    assert h[0, 0] == 1.0
    h, _ = add_rms_norm([[3 * 2.0 ** -8]], [[1.0]], [1.0], 0.0)
    assert h[0, 0] == 1.0 + 2 * 2.0 ** -7                   # tie again, to even upward
    # against torch's bf16 add (fp32 add of two bf16 values, rounded once)
    rng = np.random.default_rng(3)
    a = torch.from_numpy(rng.standard_normal((4, 256)).astype(np.float32)).to(torch.bfloat16)
    b = torch.from_numpy((rng.standard_normal((4, 256)) * 3).astype(np.float32)).to(torch.bfloat16)
    g = rng.standard_normal(256)
    h, out = add_rms_norm(a.float().numpy(), b.float().numpy(), g, 1e-5)
    assert np.array_equal(h, (a + b).float().numpy().astype(np.float64))
    # the norm reads the rounded sum, not the exact one
    assert np.array_equal(out, rms_norm(h, g, 1e-5))
    # no add: the residual is normalised as it is
    h0, out0 = add_rms_norm(None, b.float().numpy(), g, 1e-5)
    assert np.array_equal(h0, b.float().numpy()) and np.array_equal(out0, rms_norm(h0, g, 1e-5))


# ------------------------------------------------- gqa_decode_attention / append_kv

def test_attention_closed_forms():
    rng = np.random.default_rng(21)
    B, nq, nkv, L, d = 2, 4, 2, 9, 16
    q = rng.standard_normal((B, nq, d))
    v = rng.standard_normal((B, nkv, L, d))
    # identical keys: every position scores the same, the output is the mean of V
    k = np.broadcast_to(rng.standard_normal((1, 1, 1, d)), (B, nkv, L, d)).copy()
    lens = [9, 5]
    out = gqa_decode_attention(q, k, v, lens, nq, nkv)
    for b in range(B):
        for h in range(nq):
            assert np.allclose(out[b, h], v[b, h // 2, :lens[b]].mean(axis=0), rtol=1e-13, atol=1e-15)
    # one key aligned with q and far larger than the others selects its V row
    k = rng.standard_normal((B, nkv, L, d)) * 1e-3
    k[0, 0, 3] = 1e4 * q[0, 0] / np.linalg.norm(q[0, 0])
    out = gqa_decode_attention(q, k, v, [9, 9], nq, nkv)
    assert np.allclose(out[0, 0], v[0, 0, 3], rtol=0, atol=1e-12)
    # a single position: the output is that V row whatever the scores
    out = gqa_decode_attention(q, rng.standard_normal((B, nkv, L, d)), v, [1, 1], nq, nkv)
    assert np.array_equal(out[:, 0], v[:, 0, 0]) and np.array_equal(out[:, 3], v[:, 1, 0])


def test_attention_invariances_and_grouping():
    rng = np.random.default_rng(22)
    B, nq, nkv, L, d = 3, 8, 2, 12, 32
    q = rng.standard_normal((B, nq, d))
    k = rng.standard_normal((B, nkv, L, d))
    v = rng.standard_normal((B, nkv, L, d))
    lens = [12, 7, 1]
    out = gqa_decode_attention(q, k, v, lens, nq, nkv)
    # a joint permutation of the valid positions changes nothing
    perm = rng.permutation(7)
    k2, v2 = k.copy(), v.copy()
    k2[1, :, :7], v2[1, :, :7] = k[1][:, perm], v[1][:, perm]
    assert np.allclose(gqa_decode_attention(q, k2, v2, lens, nq, nkv)[1], out[1], rtol=1e-13, atol=1e-15)
    # positions at or past lens[b] are never read
    k3, v3 = k.copy(), v.copy()
    k3[1, :, 7:], v3[1, :, 7:] = np.nan, np.nan
    assert np.array_equal(gqa_decode_attention(q, k3, v3, lens, nq, nkv), out)
    # Q heads 0-3 read KV head 0, heads 4-7 KV head 1 (not h mod n_kv)
    for h in range(nq):
        one = gqa_decode_attention(q[:, h:h + 1], k[:, h // 4:h // 4 + 1], v[:, h // 4:h // 4 + 1], lens, 1, 1)
        assert np.allclose(one[:, 0], out[:, h], rtol=1e-14, atol=1e-15)
    assert not np.allclose(out[:, 1], gqa_decode_attention(q[:, 1:2], k[:, 1:2], v[:, 1:2], lens, 1, 1)[:, 0])


def test_attention_matches_torch_sdpa_in_float64():
    rng = np.random.default_rng(23)
    B, nq, nkv, L, d = 4, 4, 1, 40, 64
    q = rng.standard_normal((B, nq, d))
    k = rng.standard_normal((B, nkv, L, d))
    v = rng.standard_normal((B, nkv, L, d))
    lens = [40, 17, 2, 33]
    out = gqa_decode_attention(q, k, v, lens, nq, nkv)
    F = torch.nn.functional
    for b in range(B):
        n = lens[b]
        qt = torch.from_numpy(q[b:b + 1, :, None, :])
        kt = torch.from_numpy(k[b:b + 1, :, :n]).repeat_interleave(nq // nkv, dim=1)
        vt = torch.from_numpy(v[b:b + 1, :, :n]).repeat_interleave(nq // nkv, dim=1)
        ref = F.scaled_dot_product_attention(qt, kt, vt)[0, :, 0].numpy()
        assert np.allclose(out[b], ref, rtol=1e-12, atol=1e-14)


def test_append_kv_places_rows():
    k = np.zeros((2, 1, 4, 3))
    v = np.zeros((2, 1, 4, 3))
    kn = np.arange(6.0).reshape(2, 1, 3) + 1
    vn = -kn
    k2, v2 = append_kv(k, v, kn, vn, [0, 3])
    assert np.array_equal(k2[0, 0, 0], [1, 2, 3]) and np.array_equal(k2[1, 0, 3], [4, 5, 6])
    assert np.array_equal(v2[1, 0, 3], [-4, -5, -6]) and np.count_nonzero(k2) == 6
    assert np.count_nonzero(k) == 0                    # inputs untouched
