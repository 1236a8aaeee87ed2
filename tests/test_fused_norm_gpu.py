"""The decode layer's norm folded into its neighbouring linears, against the
oracle and against the separate calls:

* tp_row_linear_reduce_add: the new residual bit for bit against
  tp_row_linear_reduce's sum plus one bf16 rounding of residual + sum (the
  update tp_reduce_add_rmsnorm makes), and within the linear bar of the
  float64 residual + sum of the ranks' products;
* tp_fold_norm_weight: bit for bit against bf16(w * gamma) on the host;
* tp_rmsnorm_column_linear(_swiglu): within the linear bar of the call's
  definition, the oracle's RMSNorm with unit weights followed by the linear
  (and SwiGLU) on the folded weight the call receives; the plain linear also
  within the bar of the unfolded chain (RMSNorm with gamma, then W) and of
  the separate calls.

Shapes: the decode workloads' (one launch: M <= 16, whole rows of K in LDS)
and the two-launch paths (M in (16, 64] and M > 64; t > 16)."""

import numpy as np
import pytest
import torch

import oracle
from megatron_sharded_linears_amd import inputs as I
from parity import assert_close, bits, f64

pytestmark = pytest.mark.gpu

from megatron_sharded_linears_amd import lib  # noqa: E402

DEV = "cuda"
SEED = 9400
EPS = 1e-5


def dev(t):
    return t.to(DEV).contiguous()


def empty(shape, dtype=torch.bfloat16):
    return torch.empty(shape, dtype=dtype, device=DEV)


# (M, K, N, t, rank): o_proj / down_proj rank shares of the decode workloads,
# a ragged token count, 64 tokens, more ranks than the one-launch limit, and
# a prefill-sized M
REDUCE_ADD_CASES = [(16, 512, 4096, 8, 0), (16, 1792, 4096, 8, 3), (16, 128, 256, 2, 1), (5, 256, 4096, 16, 15),
                    (64, 896, 4096, 16, 2), (16, 64, 512, 17, 4), (100, 512, 1024, 4, 1)]


@pytest.mark.parametrize("pdt", [torch.bfloat16, torch.float32], ids=["bf16_partials", "fp32_partials"])
@pytest.mark.parametrize("M,K,N,t,rank", REDUCE_ADD_CASES)
def test_row_linear_reduce_add(M, K, N, t, rank, pdt):
    key = (SEED, 1, M, K, N, t)
    x = I.normal_bf16(key + (0,), (M, K))
    w = I.normal_bf16(key + (1,), (N, K), 0.02)
    res = I.normal_bf16(key + (2,), (M, N))
    peers = [None if r == rank else dev(I.normal_bf16(key + (3, r), (M, N), 0.5)).to(pdt) for r in range(t)]
    # separate: the sum over ranks, then the residual add on the host (one
    # fp32 add of two bf16 values, rounded to nearest even, as the kernels do)
    red = empty((M, N))
    lib.tp_row_linear_reduce(dev(x), dev(w), peers, rank, red)
    want = (res.float() + red.cpu().float()).to(torch.bfloat16)
    got = dev(res)
    lib.tp_row_linear_reduce_add(dev(x), dev(w), peers, rank, got)
    assert np.array_equal(bits(got), bits(want)), (M, K, N, t, rank)
    ref = f64(res) + oracle.linear(f64(x), f64(w)) + sum(f64(p) for p in peers if p is not None)
    assert_close(f64(got), ref, "reduce_add")


# (M, K, N): qkv rank shares of the decode workloads and the tiny one, a
# ragged token count, one token, the two-launch paths (M = 64, M = 200), and
# 33-64 tokens with K <= 1024 (K within one workgroup: the norm in one launch)
NORM_LINEAR_CASES = [(16, 4096, 768), (16, 4096, 512), (16, 256, 192), (5, 2048, 300), (1, 1024, 64),
                     (64, 4096, 512), (40, 4096, 520), (64, 600, 96), (24, 1024, 64), (200, 512, 384),
                     (64, 1024, 192), (48, 1024, 256), (33, 960, 100), (24, 4096, 768), (30, 4096, 520),
                     (17, 1024, 64)]


def row_scaled(h):
    """Rows at scales 2^-3 .. 2^3 (exact in bf16): RMSNorm cancels them, so a
    row normalised with another row's sum of squares is off by up to 64x."""
    sc = torch.tensor([2.0 ** ((m % 7) - 3) for m in range(h.shape[0])], dtype=torch.float32)
    return (h.float() * sc[:, None]).to(torch.bfloat16)


def normed(h, g):
    """The oracle's RMSNorm of h rounded to bf16 (the normalised row as stored)."""
    return oracle.round_bf16(oracle.rms_norm(f64(h), f64(g), EPS))


def gamma(key, K):
    return (1.0 + I.normal_bf16(key, (K,), 0.1).float()).to(torch.bfloat16)


def folded(w, g):
    out = empty(tuple(w.shape))
    lib.tp_fold_norm_weight(dev(w), dev(g), out)
    return out


def unit_normed(h):
    """The oracle's RMSNorm of h with unit weights (gamma is in the folded weight)."""
    return oracle.rms_norm(f64(h), np.ones(h.shape[1]), EPS)


@pytest.mark.parametrize("N,K", [(768, 4096), (7, 8), (1000, 256)])
def test_fold_norm_weight_bitexact(N, K):
    key = (SEED, 6, N, K)
    w = I.normal_bf16(key + (0,), (N, K), 0.02)
    g = gamma(key + (1,), K)
    want = (w.float() * g.float()[None, :]).to(torch.bfloat16)   # one product, rounded to nearest even
    assert np.array_equal(bits(folded(w, g)), bits(want))
    inplace = dev(w)
    lib.tp_fold_norm_weight(inplace, dev(g), inplace)
    assert np.array_equal(bits(inplace), bits(want))


@pytest.mark.parametrize("M,K,N", NORM_LINEAR_CASES)
def test_rmsnorm_column_linear(M, K, N):
    key = (SEED, 2, M, K, N)
    h = row_scaled(I.normal_bf16(key + (0,), (M, K), 3.0))
    g = gamma(key + (1,), K)
    w = I.normal_bf16(key + (2,), (N, K), 0.02)
    b = I.normal_bf16(key + (3,), (N,))
    y = empty((M, N))
    hd = dev(h)
    wf = folded(w, g)
    lib.tp_rmsnorm_column_linear(hd, EPS, wf, y, bias=dev(b))
    assert np.array_equal(bits(hd), bits(h)), "h is read only"
    assert_close(f64(y), oracle.linear(unit_normed(h), f64(wf), f64(b)), f"rmsnorm_column_linear {(M, K, N)}")
    ref = oracle.linear(normed(h, g), f64(w), f64(b))
    assert_close(f64(y), ref, f"rmsnorm_column_linear vs unfolded chain {(M, K, N)}")
    # against the separate calls: the norm, then the plain linear
    xn, res = empty((M, K)), dev(h)
    lib.tp_add_rmsnorm(None, res, dev(g), EPS, xn)
    y2 = empty((M, N))
    lib.tp_column_linear(xn, dev(w), y2, bias=dev(b))
    assert_close(f64(y), f64(y2), "fused vs separate")


@pytest.mark.parametrize("M,K,Is", [(16, 4096, 1792), (16, 4096, 896), (16, 256, 512), (7, 1024, 200),
                                    (64, 4096, 896), (40, 2048, 300), (130, 256, 512), (64, 1024, 256),
                                    (50, 1024, 120), (24, 4096, 896)])
def test_rmsnorm_column_linear_swiglu(M, K, Is):
    key = (SEED, 3, M, K, Is)
    h = row_scaled(I.normal_bf16(key + (0,), (M, K), 3.0))
    g = gamma(key + (1,), K)
    w = I.normal_bf16(key + (2,), (2 * Is, K), 0.02)
    act = empty((M, Is))
    wf = folded(w, g)
    lib.tp_rmsnorm_column_linear_swiglu(dev(h), EPS, wf, act)
    x = unit_normed(h)
    gate = oracle.round_bf16(oracle.linear(x, f64(wf[:Is])))
    up = oracle.round_bf16(oracle.linear(x, f64(wf[Is:])))
    assert_close(f64(act), oracle.swiglu(gate, up), f"rmsnorm_column_linear_swiglu {(M, K, Is)}")


@pytest.mark.parametrize("M,K,N,row", [(16, 4096, 768, 3), (40, 4096, 520, 37), (64, 4096, 512, 63),
                                       (64, 4096, 512, 17), (64, 1024, 192, 50), (24, 4096, 768, 23)])
def test_norm_linear_scale_invariance_and_per_row(M, K, N, row):
    """RMSNorm is invariant to scaling a row (up to eps) and rows are
    independent: scaling one row by 2^3 (exact in bf16) leaves every output
    row's value within the bar, and the other rows' bits unchanged (16 tokens:
    one launch; 40 and 64: K split over two launches, the scaled row in the
    ragged last token tile or an inner one)."""
    key = (SEED, 4, M, K, N)
    h = I.normal_bf16(key + (0,), (M, K))
    g = gamma(key + (1,), K)
    w = folded(I.normal_bf16(key + (2,), (N, K), 0.02), g)
    y1, y2 = empty((M, N)), empty((M, N))
    lib.tp_rmsnorm_column_linear(dev(h), EPS, w, y1)
    h2 = h.clone()
    h2[row] = h2[row] * 8.0
    lib.tp_rmsnorm_column_linear(dev(h2), EPS, w, y2)
    other = [m for m in range(M) if m != row]
    assert np.array_equal(bits(y1[other]), bits(y2[other]))
    assert_close(f64(y2[row:row + 1]), f64(y1[row:row + 1]), "scaled row")


def test_fused_norm_step_matches_oracle_chain():
    """One decode layer through the four fused calls against the oracle's
    chain (input norm, qkv; o + sum + residual add; post norm, gate_up,
    SwiGLU; down + sum + residual add) on the same (folded) weights, at the
    tiny workload's rank shapes."""
    t, rank, M, H, Is, nq = 2, 0, 16, 256, 512, 128
    key = (SEED, 5)
    h = I.normal_bf16(key + (0,), (M, H))
    g_in, g_post = gamma(key + (1,), H), gamma(key + (2,), H)
    w_qkv = I.normal_bf16(key + (3,), (192, H), 0.02)
    w_o = I.normal_bf16(key + (4,), (H, nq), 0.02)
    w_gu = I.normal_bf16(key + (5,), (2 * Is, H), 0.02)
    w_d = I.normal_bf16(key + (6,), (H, Is), 0.02)
    ctx = I.normal_bf16(key + (7,), (M, nq))
    peer_o = I.normal_bf16(key + (8,), (M, H), 0.5)
    peer_d = I.normal_bf16(key + (9,), (M, H), 0.5)
    res = dev(h)
    qkv, act = empty((M, 192)), empty((M, Is))
    wq_f, wgu_f = folded(w_qkv, g_in), folded(w_gu, g_post)
    lib.tp_rmsnorm_column_linear(res, EPS, wq_f, qkv)
    lib.tp_row_linear_reduce_add(dev(ctx), dev(w_o), [None, dev(peer_o)], rank, res)
    lib.tp_rmsnorm_column_linear_swiglu(res, EPS, wgu_f, act)
    lib.tp_row_linear_reduce_add(act, dev(w_d), [None, dev(peer_d)], rank, res)
    # the oracle's chain on the weights the calls receive (gamma folded into
    # qkv and gate_up), every stored activation rounded to bf16
    r64 = f64(h)
    q_ref = oracle.linear(unit_normed(h), f64(wq_f))
    assert_close(f64(qkv), q_ref, "qkv")
    r64 = oracle.round_bf16(r64 + oracle.round_bf16(oracle.linear(f64(ctx), f64(w_o)) + f64(peer_o)))
    x = oracle.rms_norm(r64, np.ones(H), EPS)
    a = oracle.swiglu(oracle.round_bf16(oracle.linear(x, f64(wgu_f[:Is]))),
                      oracle.round_bf16(oracle.linear(x, f64(wgu_f[Is:]))))
    assert_close(f64(act), a, "act")
    r64 = r64 + oracle.linear(f64(act), f64(w_d)) + f64(peer_d)
    assert_close(f64(res), r64, "residual after the layer")


@pytest.mark.parametrize("M,K,N", [(16, 4096, 16032), (16, 4096, 8016), (16, 4096, 3584), (64, 4096, 8016)])
def test_rmsnorm_lm_head_persistent_grid(M, K, N):
    """The LM head with the final norm (the Llama-8B vocab shards of t = 8
    and t = 16, and gate_up's row count): more row tiles than workgroups, so
    each workgroup loops over tiles and reuses its first tile's row scales;
    at 64 tokens the two-launch path, whose staged rows share the workspace
    with the linear's split-K partials."""
    key = (SEED, 7, M, K, N)
    h = I.normal_bf16(key + (0,), (M, K), 2.0)
    g = gamma(key + (1,), K)
    w = I.normal_bf16(key + (2,), (N, K), 0.02)
    wf = folded(w, g)
    y = empty((M, N))
    lib.tp_rmsnorm_column_linear(dev(h), EPS, wf, y)
    assert_close(f64(y), oracle.linear(unit_normed(h), f64(wf)), f"norm + lm_head {(M, K, N)}")
    # every row tile against the plain linear of the separately normalised rows
    xn, res = empty((M, K)), dev(h)
    lib.tp_add_rmsnorm(None, res, dev(g), EPS, xn)
    y2 = empty((M, N))
    lib.tp_column_linear(xn, dev(w), y2)
    d = (f64(y) - f64(y2)).reshape(M, -1, 16)
    per_tile = np.abs(d).max(axis=(0, 2)) / np.abs(f64(y2)).max()
    assert per_tile.max() <= 2e-2, f"worst row tile {int(per_tile.argmax())}: {per_tile.max():.3g}"
