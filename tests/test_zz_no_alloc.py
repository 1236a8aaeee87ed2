"""tp_column_linear_noalloc (scratch in the library's fixed per-GPU array, no
workspace, no allocation) against tp_column_linear with a workspace of
tp_workspace_bytes(): both take the same kernel plan, so the outputs must have
the same bits. Four calls in a row on one stream: the Llama-3.1-8B t = 8 qkv
shard at 16 tokens (K split 4 ways through the array's counters and
partials), a smaller one with a bias, the first again (the counters must
have been left zero), then 64 tokens of a 4096 x 4096 weight (the prefill
kernel's 64 x 64 tiles: no scratch, so accepted). A size whose plan needs
more than the array holds is rejected with TP_ERR_SHAPE."""

import pytest
import torch

from megatron_sharded_linears_amd import inputs as I
from parity import bits

pytestmark = pytest.mark.gpu

from megatron_sharded_linears_amd import lib  # noqa: E402

DEV = "cuda"


def test_noalloc_column_linear_same_bits_as_workspace_call():
    ws = lib.make_workspace()
    cases = [(16, 768, 4096, False), (5, 256, 2048, True), (16, 768, 4096, False), (64, 4096, 4096, False)]
    for i, (M, N, K, with_bias) in enumerate(cases):
        x = I.device_normal_bf16((M, K), 1.0, 500 + i, DEV)
        w = I.device_normal_bf16((N, K), 0.02, 600 + i, DEV)
        b = I.device_normal_bf16((N,), 1.0, 700 + i, DEV) if with_bias else None
        want = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        lib.tp_column_linear(x, w, want, bias=b, workspace=ws)
        got = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        lib.tp_column_linear_noalloc(x, w, got, bias=b)
        torch.cuda.synchronize()
        assert (bits(got) == bits(want)).all(), (i, M, N, K)


def test_noalloc_rejects_a_plan_beyond_its_array():
    # 64 tokens of a 2816 x 4096 weight: the decode kernel with K split 8
    # ways needs 8 x 64 x 2816 fp32 partials (5.8 MB), beyond the 4 MiB array
    x = torch.zeros((64, 4096), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((2816, 4096), dtype=torch.bfloat16, device=DEV)
    y = torch.zeros((64, 2816), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(lib.TPError) as e:
        lib.tp_column_linear_noalloc(x, w, y)
    assert e.value.status == -2
    torch.cuda.synchronize()
    assert (y == 0).all()
