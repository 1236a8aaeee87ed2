"""The rank's GQA decode attention with its KV-cache append, against the
oracle: the appended cache rows bit for bit (a copy), every other cache row
untouched, and the context within the bf16 bar of the linears (fp32 scores,
exponentials and sums against float64) and within two bf16 units of the exact
value's rounding plus the fp32 summation bound (which matters only where
the weighted sum cancels far below its terms)."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from megatron_sharded_linears_amd import inputs as I
from parity import assert_close, assert_within_bf16_ulps, bits, f64

pytestmark = pytest.mark.gpu

from megatron_sharded_linears_amd import lib  # noqa: E402

DEV = "cuda"
SEED = 9300


def make(key, B, nq, nkv, d, L, lens):
    qkv = I.normal_bf16((SEED, key, 1), (B, (nq + 2 * nkv) * d))
    kc = I.normal_bf16((SEED, key, 2), (B, nkv, L, d))
    vc = I.normal_bf16((SEED, key, 3), (B, nkv, L, d))
    return qkv, kc, vc, torch.tensor(lens, dtype=torch.int32)


def reference(qkv, kc, vc, lens, nq, nkv, d):
    B = qkv.shape[0]
    q = f64(qkv[:, :nq * d]).reshape(B, nq, d)
    k_new = f64(qkv[:, nq * d:(nq + nkv) * d]).reshape(B, nkv, d)
    v_new = f64(qkv[:, (nq + nkv) * d:]).reshape(B, nkv, d)
    k2, v2 = oracle.append_kv(f64(kc), f64(vc), k_new, v_new, lens.numpy())
    ctx = oracle.gqa_decode_attention(q, k2, v2, lens.numpy() + 1, nq, nkv)
    return ctx.reshape(B, nq * d), k2, v2


def fp32_sum_slack(qkv, k2, v2, lens, nq, nkv, d):
    """Error bound of the context's fp32 arithmetic before its bf16
    rounding: a sum of n = lens + 1 terms p v carries up to n 2^-24 sum|p v|
    (recursive summation), plus a few units for the exponentials and the
    normalisation. sum_p p |v| is the attention over |V| (same weights)."""
    B = qkv.shape[0]
    q = f64(qkv[:, :nq * d]).reshape(B, nq, d)
    mag = oracle.gqa_decode_attention(q, k2, np.abs(v2), lens.numpy() + 1, nq, nkv).reshape(B, nq * d)
    n = (lens.numpy().astype(np.float64) + 1 + 8)[:, None]
    return n * 2.0 ** -24 * mag


def run(qkv, kc, vc, lens, nq):
    k, v = kc.to(DEV).contiguous(), vc.to(DEV).contiguous()
    ctx = torch.empty((qkv.shape[0], nq * kc.shape[3]), dtype=torch.bfloat16, device=DEV)
    lib.tp_decode_attention(qkv.to(DEV).contiguous(), k, v, lens.to(DEV), nq, ctx)
    torch.cuda.synchronize()
    return ctx, k, v


# (B, nq, nkv, d, L): the workloads' rank shapes (tiny t=2: 4 Q heads of 32
# over 1 KV head; Llama t=8: 4 of 128 over 1; t=16: 2 over a replicated 1;
# Llama t=2: 16 over 4; Qwen t=8: 5 over 1) and the other head widths
CASES = [(16, 4, 1, 32, 300), (16, 4, 1, 128, 2304), (64, 2, 1, 128, 1100), (4, 16, 4, 128, 520),
         (8, 5, 1, 128, 700), (5, 8, 1, 64, 257), (3, 8, 2, 256, 390), (2, 1, 1, 128, 129)]


@pytest.mark.parametrize("B,nq,nkv,d,L", CASES)
def test_decode_attention_matches_oracle(B, nq, nkv, d, L):
    r = np.random.default_rng(B * 1000 + L)
    # lengths: the new token only, edges of 64- and 192-position chunks, the last slot, random
    special = [0, 63, 64, 191, 192, 383, L - 1]
    lens = [special[i] if i < len(special) and special[i] < L else int(r.integers(0, L)) for i in range(B)]
    qkv, kc, vc, lens_t = make(B * 10 + nq, B, nq, nkv, d, L, lens)
    ctx, k, v = run(qkv, kc, vc, lens_t, nq)
    ref, k2, v2 = reference(qkv, kc, vc, lens_t, nq, nkv, d)
    assert np.array_equal(f64(k), k2) and np.array_equal(f64(v), v2), "cache after the append"
    slack = fp32_sum_slack(qkv, k2, v2, lens_t, nq, nkv, d)
    assert_within_bf16_ulps(f64(ctx), ref, 2, f"ctx {(B, nq, nkv, d, L)}", slack=slack)
    assert_close(f64(ctx), ref, f"ctx {(B, nq, nkv, d, L)}")


def test_out_of_range_lengths_give_zero_rows_and_no_write():
    B, nq, nkv, d, L = 4, 4, 1, 128, 200
    lens = [-1, 50, 200, 1 << 30]
    qkv, kc, vc, lens_t = make(77, B, nq, nkv, d, L, lens)
    ctx, k, v = run(qkv, kc, vc, lens_t, nq)
    for b in (0, 2, 3):
        assert (f64(ctx[b]) == 0.0).all()
        assert np.array_equal(bits(k[b]), bits(kc[b])) and np.array_equal(bits(v[b]), bits(vc[b]))
    q = f64(qkv[1:2, :nq * d]).reshape(1, nq, d)
    k2, v2 = oracle.append_kv(f64(kc[1:2]), f64(vc[1:2]), f64(qkv[1:2, nq * d:(nq + 1) * d]).reshape(1, 1, d),
                              f64(qkv[1:2, (nq + 1) * d:]).reshape(1, 1, d), [50])
    ref = oracle.gqa_decode_attention(q, k2, v2, [51], nq, nkv).reshape(1, nq * d)
    slack = fp32_sum_slack(qkv[1:2], k2, v2, lens_t[1:2], nq, nkv, d)
    assert_within_bf16_ulps(f64(ctx[1:2]), ref, 2, "in-range row beside out-of-range ones", slack=slack)


def test_deterministic_and_independent_of_other_sequences():
    """The same bits on a second call (the chunks are merged in order, not in
    arrival order); a sequence's context does not depend on its neighbours."""
    B, nq, nkv, d, L = 16, 4, 1, 128, 3000
    lens = [2048] * B
    qkv, kc, vc, lens_t = make(88, B, nq, nkv, d, L, lens)
    c1, _, _ = run(qkv, kc, vc, lens_t, nq)
    c2, _, _ = run(qkv, kc, vc, lens_t, nq)
    assert np.array_equal(bits(c1), bits(c2))
    c3, _, _ = run(qkv[5:6], kc[5:6], vc[5:6], lens_t[5:6], nq)
    assert np.array_equal(bits(c3), bits(c1[5:6]))


def test_empty_batch_is_a_no_op():
    d, nq, nkv, L = 128, 4, 1, 64
    qkv = torch.zeros((1, (nq + 2 * nkv) * d), dtype=torch.bfloat16, device=DEV)
    kc = torch.ones((1, nkv, L, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.ones((1, nkv, L, d), dtype=torch.bfloat16, device=DEV)
    lens = torch.zeros(1, dtype=torch.int32, device=DEV)
    ctx = torch.full((1, nq * d), 7.0, dtype=torch.bfloat16, device=DEV)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    S = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib._lib.tp_decode_attention(P(qkv), 0, nq, nkv, d, P(kc), P(vc), L, P(lens), P(ctx), None, 0, S) == 0
    torch.cuda.synchronize()
    assert (f64(ctx) == 7.0).all() and (f64(kc) == 1.0).all()
