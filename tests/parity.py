"""Comparison helpers for the GPU parity tests."""

import numpy as np
import torch

import oracle

# Linears: bf16 in, fp32 accumulate. Gate on both the worst element and the
# ratio of L1 norms (elementwise relative error is ill-defined near zero).
MAX_ABS_FRAC = 2e-2
MEAN_REL = 5e-3


def f64(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def bits(t):
    """uint16 bit patterns of a bf16 tensor."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().astype(np.uint16)


def close_stats(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    d = np.abs(got - ref)
    max_ref = float(np.max(np.abs(ref))) if ref.size else 0.0
    l1 = float(np.sum(np.abs(ref)))
    return float(d.max()) if d.size else 0.0, max_ref, (float(d.sum()) / l1 if l1 > 0 else 0.0)


def assert_close(got, ref, what=""):
    """max|d| <= 2e-2 max|ref| and sum|d| / sum|ref| <= 5e-3."""
    mx, mref, rel = close_stats(got, ref)
    assert np.isfinite(np.asarray(got)).all(), f"{what}: non-finite output"
    assert mx <= MAX_ABS_FRAC * mref, f"{what}: max|d|={mx:.4g} > {MAX_ABS_FRAC}*max|ref|={MAX_ABS_FRAC * mref:.4g}"
    assert rel <= MEAN_REL, f"{what}: mean rel err {rel:.4g} > {MEAN_REL}"
    return mx, mref, rel


def assert_within_bf16_ulps(got, ref, ulps=1, what="", slack=0.0):
    """Each element within `ulps` bf16 units of the exact value's bf16
    rounding, plus an absolute `slack` (scalar or per element) where the
    fp32 arithmetic before the rounding has an error bound of its own."""
    got = np.asarray(got, dtype=np.float64)
    r = oracle.round_bf16(ref)
    a = np.abs(r)
    e = np.frexp(np.where(a > 0, a, 1.0))[1] - 1
    ulp = np.ldexp(1.0, np.maximum(e, -126) - 7)
    bad = np.abs(got - r) > ulps * ulp + slack
    assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond {ulps} ulp, e.g. got {got[bad][:4]} ref {r[bad][:4]}"
