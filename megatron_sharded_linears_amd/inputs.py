"""Seeded synthetic inputs, shared by the tests, the smoke check and the
benchmark. This module holds none of the linear path's arithmetic: it only
draws random numbers and stores them as bf16 (torch's float32 -> bfloat16
cast) or int32.

Every stream of random numbers is NumPy's PCG64 seeded from
SeedSequence([workload, layer, tensor]), so any tensor can be regenerated on
its own, on any host.
"""

import numpy as np
import torch

# tensor ids inside a (workload, layer) seed
T_X, T_CTX, T_QKV, T_O, T_GATE_UP, T_DOWN, T_EMBED, T_LM_HEAD, T_IDS, T_HS, T_EXTRA = range(11)

WEIGHT_STD = 0.02
ACT_STD = 1.0


def rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def normal_bf16(key, shape, std=1.0):
    """bf16 tensor (CPU) of N(0, std^2) draws."""
    a = rng(*key).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return torch.from_numpy(a).to(torch.bfloat16)


def small_int_bf16(key, shape, lo=-1, hi=1):
    """bf16 tensor (CPU) of integers drawn uniformly from [lo, hi]: products
    and sums of these are exact in fp32, so results do not depend on the
    summation order."""
    a = rng(*key).integers(lo, hi + 1, size=shape).astype(np.float32)
    return torch.from_numpy(a).to(torch.bfloat16)


def uniform_ids(key, n, vocab):
    """int32 token ids drawn uniformly from [0, vocab)."""
    return torch.from_numpy(rng(*key).integers(0, vocab, size=n).astype(np.int32))


def to_f64(t):
    """Exact float64 copy (NumPy) of a bf16/fp32 tensor, for the oracle."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def device_normal_bf16(shape, std, seed, device="cuda"):
    """bf16 N(0, std^2) tensor drawn on the device with a seeded torch
    generator: for weights too large to draw on the host quickly (timing runs,
    where values do not affect speed)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


def device_small_int_bf16(shape, seed, lo=-1, hi=1, device="cuda"):
    """bf16 tensor of integers drawn uniformly from [lo, hi] on the device with
    a seeded torch generator: exact-integer inputs at sizes too large to draw
    on the host quickly (sums of products of these are exact in fp32 while
    below 2^24)."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randint(lo, hi + 1, shape, generator=g, device=device, dtype=torch.int32).to(torch.bfloat16)
