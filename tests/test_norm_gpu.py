"""Residual add + RMSNorm and its fusion with the sum over ranks, against the
oracle: the new residual bit for bit (one bf16 rounding of an exact sum of
two bf16 values), the normalised output within one bf16 unit of the exact
value's rounding (the kernel's fp32 mean and scale against float64), and the
fused call bit for bit against the separate calls it replaces."""

import numpy as np
import pytest
import torch

import oracle
from megatron_sharded_linears_amd import inputs as I
from parity import assert_close, assert_within_bf16_ulps, bits, f64

pytestmark = pytest.mark.gpu

from megatron_sharded_linears_amd import lib  # noqa: E402

DEV = "cuda"
SEED = 9100


def dev(t):
    return t.to(DEV).contiguous()


def empty(shape, dtype=torch.bfloat16):
    return torch.empty(shape, dtype=dtype, device=DEV)


def gamma_of(key, H):
    # a norm weight around 1 with spread, as trained RMSNorm weights are
    return (1.0 + 0.25 * I.normal_bf16(tuple(key) + (77,), (H,)).float()).to(torch.bfloat16)


# (M, H): one vector per row, rows shorter and longer than one pass of the
# workgroup (256 threads x 8 values), the model widths, ragged remainders
SHAPES = [(1, 8), (3, 64), (5, 2056), (16, 4096), (7, 5120), (64, 4096), (130, 6152), (2, 16384)]


@pytest.mark.parametrize("M,H", SHAPES)
@pytest.mark.parametrize("eps", [1e-5, 1e-6])
def test_add_rmsnorm_matches_oracle(M, H, eps):
    x = I.normal_bf16((SEED, 1, M, H), (M, H))
    res = I.normal_bf16((SEED, 2, M, H), (M, H), 3.0)
    g = gamma_of((SEED, 3, H), H)
    r = dev(res)
    out = empty((M, H))
    lib.tp_add_rmsnorm(dev(x), r, dev(g), eps, out)
    h_ref, out_ref = oracle.add_rms_norm(f64(x), f64(res), f64(g), eps)
    assert np.array_equal(f64(r), h_ref), "new residual"
    assert_within_bf16_ulps(f64(out), out_ref, 1, f"out {(M, H, eps)}")
    assert_close(f64(out), out_ref, f"out {(M, H, eps)}")


@pytest.mark.parametrize("M,H", [(4, 64), (16, 4096), (9, 2056)])
def test_norm_without_add_leaves_residual_and_matches_oracle(M, H):
    res = I.normal_bf16((SEED, 10, M, H), (M, H), 0.7)
    g = gamma_of((SEED, 11, H), H)
    r = dev(res)
    before = bits(r)
    out = empty((M, H))
    lib.tp_add_rmsnorm(None, r, dev(g), 1e-5, out)
    assert np.array_equal(bits(r), before)
    assert_within_bf16_ulps(f64(out), oracle.rms_norm(f64(res), f64(g), 1e-5), 1, f"norm {(M, H)}")


def test_eps_zero_and_wide_magnitudes():
    """eps = 0 (pure RMS scaling), rows from 1e-6 to 1e15 in scale: the output
    does not depend on the row's scale (up to the bf16 rounding of the input)."""
    M, H = 6, 1024
    base = I.normal_bf16((SEED, 20), (1, H)).float()
    scales = torch.tensor([1e-6, 1e-3, 1.0, 37.0, 1e6, 1e15]).reshape(M, 1)
    res = (base * scales).to(torch.bfloat16)
    g = gamma_of((SEED, 21), H)
    r = dev(res)
    out = empty((M, H))
    lib.tp_add_rmsnorm(None, r, dev(g), 0.0, out)
    assert_within_bf16_ulps(f64(out), oracle.rms_norm(f64(res), f64(g), 0.0), 1, "eps 0")


# H = 4096: all partials loaded at once (1 vector per thread); 6152: 2 per
# thread (16 fp32 partials: loop); 16384 and 32768: 4 and 8 per thread, loop
@pytest.mark.parametrize("t", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("pdt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("H", [4096, 6152, 32768])
def test_reduce_add_rmsnorm_equals_separate_calls_and_oracle(t, pdt, H):
    M = 16 if H <= 8192 else 3
    parts = [dev(I.normal_bf16((SEED, 30, t, i), (M, H), 0.5).to(pdt)) for i in range(t)]
    res = I.normal_bf16((SEED, 31, t), (M, H), 2.0)
    g = dev(gamma_of((SEED, 32, t), H))
    # fused
    r1 = dev(res)
    o1 = empty((M, H))
    lib.tp_reduce_add_rmsnorm(parts, r1, g, 1e-5, o1)
    # separate: reduce to bf16, then add + norm
    s = empty((M, H))
    lib.tp_reduce_partials(parts, s)
    r2 = dev(res)
    o2 = empty((M, H))
    lib.tp_add_rmsnorm(s, r2, g, 1e-5, o2)
    assert np.array_equal(bits(r1), bits(r2)) and np.array_equal(bits(o1), bits(o2)), (t, pdt)
    # oracle: the sum over ranks in rank order, rounded to bf16, then the add and the norm
    summed = oracle.round_bf16(oracle.all_reduce_sum([f64(p) for p in parts]))
    h_ref, out_ref = oracle.add_rms_norm(summed, f64(res), f64(g), 1e-5)
    assert np.array_equal(f64(r1), h_ref)
    assert_within_bf16_ulps(f64(o1), out_ref, 1, f"fused t={t}")


@pytest.mark.parametrize("M,t", [(2048, 2), (4096, 8)])
def test_prefill_sizes_and_determinism(M, t):
    """Prefill-sized rows (Llama-8B t = 2, Qwen-32B t = 8 widths), all rows
    against the oracle, and the same bits on a second call."""
    H = 4096 if t == 2 else 5120
    parts = [dev(I.normal_bf16((SEED, 40, M, i), (M, H), 0.5)) for i in range(t)]
    res = I.normal_bf16((SEED, 41, M), (M, H))
    g = dev(gamma_of((SEED, 42, M), H))
    outs = []
    for _ in range(2):
        r = dev(res)
        o = empty((M, H))
        lib.tp_reduce_add_rmsnorm(parts, r, g, 1e-6, o)
        outs.append((r, o))
    assert np.array_equal(bits(outs[0][0]), bits(outs[1][0])) and np.array_equal(bits(outs[0][1]), bits(outs[1][1]))
    summed = oracle.round_bf16(oracle.all_reduce_sum([f64(p) for p in parts]))
    h_ref, out_ref = oracle.add_rms_norm(summed, f64(res), f64(g), 1e-6)
    assert np.array_equal(f64(outs[0][0]), h_ref)
    assert_within_bf16_ulps(f64(outs[0][1]), out_ref, 1, f"prefill M={M} t={t}")


def test_empty_batch_is_a_no_op():
    """M = 0 through the C ABI with real buffers (torch gives zero-row views a
    NULL data pointer, which the ABI rejects): nothing is read or written."""
    import ctypes
    H = 64
    r = dev(I.normal_bf16((SEED, 50), (1, H)))
    g = dev(gamma_of((SEED, 51), H))
    x = dev(I.normal_bf16((SEED, 52), (1, H)))
    out = empty((1, H)).fill_(7.0)
    before = bits(r)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    S = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib._lib.tp_add_rmsnorm(P(x), 0, H, P(r), P(g), 1e-5, P(out), S) == 0
    arr, keep = lib._ptrs([x])
    assert lib._lib.tp_reduce_add_rmsnorm(arr, 1, 0, 0, H, P(r), P(g), 1e-5, P(out), S) == 0
    torch.cuda.synchronize()
    assert np.array_equal(bits(r), before) and (f64(out) == 7.0).all()
