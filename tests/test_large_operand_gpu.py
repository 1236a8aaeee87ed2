"""A weight shard larger than 4 GiB: the kernels that read through buffer
resources address 32-bit byte offsets, so a launch whose weight (or
activation) extends past 2^32 bytes must run on kernels that do not (the
register-staged prefill tile; the decode kernel's LDS-staged shapes) and still
give every output. Exact-integer inputs ({-1, 0, 1}, sums exact in fp32), so
each bf16 output is the exact sum rounded once; the rows checked sit at the
start, on both sides of the 2^32-byte boundary and at the end of the weight.
"""

import numpy as np
import pytest
import torch

import oracle
from megatron_sharded_linears_amd import inputs as I
from parity import f64

pytestmark = pytest.mark.gpu

from megatron_sharded_linears_amd import lib  # noqa: E402

DEV = "cuda"
SEED = 9700


@pytest.mark.parametrize("M", [128, 16], ids=["prefill", "decode"])
def test_weight_past_4gib_exact_integer(M):
    K = 4096
    boundary = (1 << 32) // (K * 2)             # first row that starts at 2^32 bytes
    N = boundary + 1000                         # 4.3 GB of bf16 weight
    w = I.device_small_int_bf16((N, K), SEED + 1, device=DEV)
    x = I.device_small_int_bf16((M, K), SEED + 2, device=DEV)
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    lib.tp_column_linear(x, w, y)
    torch.cuda.synchronize()
    rows = np.r_[0:64, boundary - 64:boundary + 64, N - 64:N]
    idx = torch.as_tensor(rows, device=DEV)
    got = f64(y.index_select(1, idx).cpu())
    want = oracle.round_bf16(oracle.linear(f64(x.cpu()), f64(w.index_select(0, idx).cpu())))
    assert np.array_equal(got, want), (M, int(np.abs(got - want).max()))
    del w, y
    torch.cuda.empty_cache()
