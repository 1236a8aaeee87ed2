"""Calls from several host threads at once, each on its own stream with its
own workspace, give the bits of the same calls made one at a time.

The library keeps per-device launch state (kernel attributes set on first
use, occupancy and CU counts, the tiled kernels' attribute flags) behind a
mutex or atomics; its split-K partials and arrival counters live in the
caller's workspace, so calls on different workspaces share nothing on the
device. Each thread runs a decode linear with a K split (qkv at the Llama-8B
t = 8 shape), the fused sum over ranks, the SwiGLU epilogue, a prefill-sized
tile GEMM and the decode attention, several times, on its own stream."""

import threading

import numpy as np
import pytest
import torch

from megatron_sharded_linears_amd import inputs as I
from megatron_sharded_linears_amd import lib

pytestmark = pytest.mark.gpu

DEV = "cuda"
THREADS, REPEATS = 4, 5


def _case(seed):
    n = lambda shape, std, s: I.device_normal_bf16(shape, std, seed + s, DEV)
    bf = torch.bfloat16
    c = {"x": n((16, 4096), 1.0, 1), "w_qkv": n((768, 4096), 0.02, 2),
         "ctx": n((16, 512), 1.0, 3), "w_o": n((4096, 512), 0.02, 4),
         "peers": [None] + [n((16, 4096), 0.5, 10 + j) for j in range(7)],
         "w_gu": n((3584, 4096), 0.02, 5),
         "xp": n((300, 1024), 1.0, 6), "wp": n((520, 1024), 0.02, 7),
         "qkv_a": n((4, 6 * 128), 1.0, 8), "k": n((4, 1, 256, 128), 1.0, 9), "v": n((4, 1, 256, 128), 1.0, 20),
         "lens": torch.full((4,), 200, dtype=torch.int32, device=DEV)}
    c["out"] = {"qkv": torch.empty((16, 768), dtype=bf, device=DEV), "y1": torch.empty((16, 4096), dtype=bf, device=DEV),
                "act": torch.empty((16, 1792), dtype=bf, device=DEV), "yp": torch.empty((300, 520), dtype=bf, device=DEV),
                "ctx_a": torch.empty((4, 4 * 128), dtype=bf, device=DEV)}
    return c


def _run(c, ws, stream):
    o = c["out"]
    lib.tp_column_linear(c["x"], c["w_qkv"], o["qkv"], workspace=ws, stream=stream)
    lib.tp_row_linear_reduce(c["ctx"], c["w_o"], c["peers"], 0, o["y1"], workspace=ws, stream=stream)
    lib.tp_column_linear_swiglu(o["y1"], c["w_gu"], o["act"], workspace=ws, stream=stream)
    lib.tp_column_linear(c["xp"], c["wp"], o["yp"], workspace=ws, stream=stream)
    lib.tp_decode_attention(c["qkv_a"], c["k"], c["v"], c["lens"], 4, o["ctx_a"], workspace=ws, stream=stream)


def _bits(c):
    return {k: v.view(torch.int16).cpu().numpy() for k, v in c["out"].items()}


def test_concurrent_host_threads_on_their_own_streams_and_workspaces():
    cases = [_case(8000 + 100 * i) for i in range(THREADS)]
    wss = [lib.make_workspace() for _ in range(THREADS)]
    # one at a time: the reference bits
    want = []
    for c, ws in zip(cases, wss):
        _run(c, ws, None)
        torch.cuda.synchronize()
        want.append(_bits(c))
        for v in c["out"].values():
            v.fill_(float("nan"))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(THREADS)]
    errors = []
    start = threading.Barrier(THREADS)

    def worker(i):
        try:
            torch.cuda.set_device(0)
            start.wait()
            for _ in range(REPEATS):
                _run(cases[i], wss[i], streams[i])
            streams[i].synchronize()
        except Exception as e:        # reported below, with the thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(THREADS)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i, c in enumerate(cases):
        got = _bits(c)
        for k in want[i]:
            assert np.array_equal(got[k], want[i][k]), (i, k)
