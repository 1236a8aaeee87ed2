"""The C ABI on a machine without a GPU: the library loads, exports every
function include/tp_shard.h declares, its host-only shape queries agree with
the oracle's independent head and vocab maps, and argument errors are
reported before any HIP call (so no compute call is made here)."""

import ctypes
import os
import re

import pytest

import oracle
from megatron_sharded_linears_amd import lib
from megatron_sharded_linears_amd.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
C = lib._lib


def _declared_functions():
    names = []
    inc = os.path.join(ROOT, "include")
    for fn in sorted(os.listdir(inc)):
        if not fn.endswith(".h"):
            continue
        text = open(os.path.join(inc, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(tp_[a-z_]+)\s*\(", text, flags=re.M)
    return names


def test_every_declared_function_is_exported_and_bound():
    names = _declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(C, n), n
        assert n in lib.EXPORTED, n
        assert callable(getattr(lib, n)), n
    # the eight device calls of the path
    for n in ["tp_shard_weights", "tp_column_linear", "tp_swiglu", "tp_row_linear_partial",
              "tp_reduce_partials", "tp_vocab_embed", "tp_lm_head_shard", "tp_concat_logits"]:
        assert n in names


def test_library_links_hip_runtime_by_soname():
    import subprocess
    out = subprocess.run(["readelf", "-d", lib.library_path()], capture_output=True, text=True).stdout
    assert "libamdhip64.so.7" in out


@pytest.mark.parametrize("w", WORKLOADS, ids=lambda w: w.name)
def test_shard_shapes_agree_with_oracle_maps(w):
    cfg = w.cfg()
    t = w.t
    d = w.head_dim
    assert lib.tp_shard_shape(cfg, t, "qkv") == (len(oracle.qkv_shard_rows(w.num_q_heads, w.num_kv_heads, d, t, 0)), w.hidden)
    assert lib.tp_shard_shape(cfg, t, "gate_up") == (len(oracle.gate_up_shard_rows(w.intermediate, t, 0)), w.hidden)
    assert lib.tp_shard_shape(cfg, t, "o") == (w.hidden, len(oracle.o_shard_cols(w.num_q_heads, d, t, 0)))
    assert lib.tp_shard_shape(cfg, t, "down") == (w.hidden, len(oracle.down_shard_cols(w.intermediate, t, 0)))
    assert lib.tp_shard_shape(cfg, t, "embed") == (oracle.vocab_shard_rows(w.vocab, t), w.hidden)
    assert lib.tp_vocab_shard_rows(w.vocab, t) == oracle.vocab_shard_rows(w.vocab, t)
    for r in range(t):
        first, count = lib.tp_kv_heads_of_rank(cfg, t, r)
        assert list(range(first, first + count)) == oracle.kv_heads_of_rank(w.num_kv_heads, t, r)
    full = {k: lib.tp_full_shape(cfg, k) for k in lib.KIND}
    assert full["qkv"] == ((w.num_q_heads + 2 * w.num_kv_heads) * d, w.hidden)
    assert full["gate_up"] == (2 * w.intermediate, w.hidden)


def test_kv_replication_and_split_rule_errors():
    base = {"hidden": 64, "num_q_heads": 8, "num_kv_heads": 2, "head_dim": 8, "intermediate": 64, "vocab": 10}
    for t in (1, 2, 4, 8):
        for r in range(t):
            f, c = lib.tp_kv_heads_of_rank(base, t, r)
            assert list(range(f, f + c)) == oracle.kv_heads_of_rank(2, t, r)
    with pytest.raises(lib.TPError) as e:
        lib.tp_shard_shape(base, 3, "qkv")             # 8 % 3
    assert e.value.status == -3
    with pytest.raises(lib.TPError) as e:
        lib.tp_shard_shape(dict(base, num_kv_heads=4, num_q_heads=12), 3, "qkv")  # 4 >= 3, 4 % 3
    assert e.value.status == -3
    with pytest.raises(lib.TPError) as e:
        lib.tp_shard_shape(dict(base, intermediate=60), 8, "gate_up")
    assert e.value.status == -3
    with pytest.raises(lib.TPError) as e:
        lib.tp_shard_shape(base, 65, "qkv")
    assert e.value.status == -6
    with pytest.raises(lib.TPError) as e:
        lib.tp_kv_heads_of_rank(base, 4, 4)
    assert e.value.status == -6
    with pytest.raises(lib.TPError) as e:
        lib.tp_shard_shape(base, 2, 17)
    assert e.value.status == -5
    assert lib.tp_vocab_shard_rows(1001, 2) == 501
    assert lib.tp_vocab_shard_rows(5, 4) == 2
    assert C.tp_vocab_shard_rows(10, 0) == -6
    assert C.tp_status_string(12345) == b"unknown status"


# Fake device addresses: validation must reject (or accept as a no-op) before
# touching them, so nothing is ever dereferenced.
A = ctypes.c_void_p(0x10000)      # 16-byte aligned
B = ctypes.c_void_p(0x20000)
Y = ctypes.c_void_p(0x30000)
MIS = ctypes.c_void_p(0x10008)    # 8-byte aligned only
NULL = ctypes.c_void_p(0)
S = ctypes.c_void_p(0)
NO_WS = (NULL, 0)                 # no workspace
WS = ctypes.c_void_p(0x1000000)   # a fake workspace far from the operands
WSB = lib.tp_workspace_bytes()


def test_workspace_size_query():
    assert lib.tp_workspace_bytes() == lib.TP_WS_COUNTER_BYTES + 16 * 2**20
    assert C.tp_workspace_bytes() == WSB


def test_linear_validation_before_any_hip_call():
    f = C.tp_column_linear
    assert f(NULL, 16, 64, B, 32, NULL, Y, *NO_WS, S) == -1
    assert f(A, 16, 64, NULL, 32, NULL, Y, *NO_WS, S) == -1
    assert f(A, -1, 64, B, 32, NULL, Y, *NO_WS, S) == -2
    assert f(A, 16, 0, B, 32, NULL, Y, *NO_WS, S) == -2
    assert f(A, 16, 60, B, 32, NULL, Y, *NO_WS, S) == -4          # K % 8
    assert f(MIS, 16, 64, B, 32, NULL, Y, *NO_WS, S) == -4
    assert f(A, 16, 64, B, 32, ctypes.c_void_p(0x40001), Y, *NO_WS, S) == -4
    assert f(A, 0, 64, B, 32, NULL, Y, *NO_WS, S) == 0            # M == 0: no-op
    assert f(A, 0, 64, B, 32, NULL, Y, WS, WSB, S) == 0
    g = C.tp_row_linear_partial
    assert g(A, 16, 64, B, 32, Y, 7, *NO_WS, S) == -5
    assert g(A, 0, 64, B, 32, Y, 1, *NO_WS, S) == 0
    h = C.tp_lm_head_shard
    assert h(A, 4, 64, B, 32, Y, 2, *NO_WS, S) == -5
    assert h(A, 0, 64, B, 32, Y, 0, *NO_WS, S) == 0


def test_linear_rejects_overlapping_buffers():
    """Outputs may not overlap any input (x 16 x 64 bf16 = 2 KiB at A, w
    32 x 64 bf16 = 4 KiB at B, y 16 x 32 bf16 = 1 KiB)."""
    f = C.tp_column_linear
    assert f(A, 16, 64, B, 32, NULL, ctypes.c_void_p(0x10000 + 1024), *NO_WS, S) == -2   # y inside x
    assert f(A, 16, 64, B, 32, NULL, ctypes.c_void_p(0x20000 - 512), *NO_WS, S) == -2    # y runs into w
    assert f(A, 16, 64, B, 32, ctypes.c_void_p(0x30000 + 32), Y, *NO_WS, S) == -2        # bias inside y
    assert f(A, 16, 64, B, 32, NULL, Y, ctypes.c_void_p(0x30000 - 256), WSB, S) == -2    # workspace over y
    g = C.tp_row_linear_partial
    assert g(A, 16, 64, B, 32, ctypes.c_void_p(0x20000 + 4096 - 16), 1, *NO_WS, S) == -2  # fp32 y into w's tail
    s = C.tp_swiglu
    assert s(A, 4, 16, ctypes.c_void_p(0x10000 + 64), S) == -2          # out inside gu
    r = C.tp_reduce_partials
    arr = (ctypes.c_void_p * 2)(0x10000, 0x20000)
    pp = ctypes.cast(arr, lib._ptr_array)
    assert r(pp, 2, 64, 0, ctypes.c_void_p(0x20000 + 64), 0, S) == -2   # out overlaps partial 1
    assert r(pp, 2, 64, 0, ctypes.c_void_p(0x10000 + 16), 0, S) == -2   # overlaps partial 0, not equal
    assert r(pp, 2, 64, 1, A, 0, S) == -2                               # in place needs one element size
    assert C.tp_concat_logits(pp, 2, 4, 8, 16, 0, ctypes.c_void_p(0x20000 + 16), S) == -2
    assert C.tp_vocab_embed(A, 4, B, 1000, 2, 0, 64, ctypes.c_void_p(0x20000 + 64), S) == -2  # out in the table


def test_workspace_argument_validation():
    f = C.tp_column_linear
    assert f(A, 16, 64, B, 32, NULL, Y, NULL, 4096, S) == -1          # size without a buffer
    assert f(A, 16, 64, B, 32, NULL, Y, WS, -1, S) == -2
    assert f(A, 16, 64, B, 32, NULL, Y, ctypes.c_void_p(0x1000008), WSB, S) == -4
    at = C.tp_decode_attention
    KC, VC, LN, CT = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), ctypes.c_void_p(0x300000), \
        ctypes.c_void_p(0x400000)
    # the records of 4 sequences x 1 KV head x 1 chunk x 4 heads x 130 floats need scratch
    assert at(A, 4, 4, 1, 128, KC, VC, 64, LN, CT, *NO_WS, S) == -2
    assert at(A, 4, 4, 1, 128, KC, VC, 64, LN, CT, WS, lib.TP_WS_COUNTER_BYTES + 1024, S) == -2


def test_elementwise_validation_before_any_hip_call():
    assert C.tp_swiglu(A, 4, 12, Y, S) == -4               # i_shard % 8
    assert C.tp_swiglu(NULL, 4, 16, Y, S) == -1
    assert C.tp_swiglu(A, 0, 16, Y, S) == 0
    arr = (ctypes.c_void_p * 3)(0x10000, 0x20000, 0x30008)
    pp = ctypes.cast(arr, lib._ptr_array)
    assert C.tp_reduce_partials(pp, 3, 64, 0, Y, 0, S) == -4  # third partial misaligned
    assert C.tp_reduce_partials(pp, 0, 64, 0, Y, 0, S) == -6
    assert C.tp_reduce_partials(pp, 65, 64, 0, Y, 0, S) == -6
    assert C.tp_reduce_partials(pp, 2, 64, 3, Y, 0, S) == -5
    assert C.tp_reduce_partials(pp, 2, 0, 0, Y, 0, S) == 0
    assert C.tp_reduce_partials(pp, 2, 0, 0, A, 0, S) == 0    # in place on partial 0
    assert C.tp_vocab_embed(A, 4, B, 1000, 2, 2, 64, Y, S) == -6      # rank == t
    assert C.tp_vocab_embed(A, 4, B, 1000, 2, 0, 60, Y, S) == -4      # H % 8
    assert C.tp_vocab_embed(A, 0, B, 1000, 2, 0, 64, Y, S) == 0
    arr2 = (ctypes.c_void_p * 2)(0x10000, 0x20000)
    pp2 = ctypes.cast(arr2, lib._ptr_array)
    assert C.tp_concat_logits(pp2, 2, 4, 499, 1000, 0, Y, S) == -2    # v_shard != ceil(V/t)
    assert C.tp_concat_logits(pp2, 2, 0, 500, 1000, 0, Y, S) == 0
    cfg = lib._cfg({"hidden": 64, "num_q_heads": 8, "num_kv_heads": 2, "head_dim": 8,
                    "intermediate": 64, "vocab": 10})
    assert C.tp_shard_weights(ctypes.byref(cfg), 2, 2, 0, A, B, S) == -6
    assert C.tp_shard_weights(ctypes.byref(cfg), 3, 0, 0, A, B, S) == -3
    assert C.tp_shard_weights(ctypes.byref(cfg), 2, 0, 0, MIS, B, S) == -4
    assert C.tp_shard_weights(ctypes.byref(cfg), 2, 0, 9, A, B, S) == -5
    assert C.tp_shard_weights(ctypes.byref(cfg), 2, 0, 0, A, ctypes.c_void_p(0x10000 + 256), S) == -2  # shard in full


def test_fused_calls_validate_before_any_hip_call():
    f = C.tp_column_linear_swiglu
    assert f(NULL, 16, 64, B, 32, Y, *NO_WS, S) == -1
    assert f(A, 16, 64, B, 0, Y, *NO_WS, S) == -2                    # i_shard 0
    assert f(A, 16, 60, B, 32, Y, *NO_WS, S) == -4                   # K % 8
    assert f(A, 16, 64, MIS, 32, Y, *NO_WS, S) == -4
    assert f(A, 0, 64, B, 12, Y, *NO_WS, S) == 0                     # any i_shard; M == 0 no-op
    assert f(A, 16, 64, B, 32, ctypes.c_void_p(0x20000 + 6000), *NO_WS, S) == -2   # act inside w's 2 x 32 rows
    g = C.tp_row_linear_reduce         # x, M, K, w, N, partials, dtype, t, rank, out, ws, ws_bytes, stream
    arr = (ctypes.c_void_p * 4)(0x50000, 0, 0x60000, 0x70000)   # entry 1 is the calling rank
    pp = ctypes.cast(arr, lib._ptr_array)
    assert g(A, 0, 64, B, 32, pp, 0, 4, 1, Y, *NO_WS, S) == 0             # own entry may be NULL
    assert g(A, 0, 64, B, 32, pp, 1, 4, 1, Y, *NO_WS, S) == 0             # fp32 peers
    assert g(A, 0, 64, B, 32, pp, 2, 4, 1, Y, *NO_WS, S) == -5            # peer dtype
    assert g(A, 0, 64, B, 32, pp, 0, 4, 2, Y, *NO_WS, S) == -1            # another rank's entry NULL
    assert g(A, 0, 64, B, 32, pp, 0, 4, 4, Y, *NO_WS, S) == -6            # rank == t
    assert g(A, 0, 64, B, 32, pp, 0, 0, 0, Y, *NO_WS, S) == -6
    assert g(A, 0, 64, B, 32, pp, 0, 65, 0, Y, *NO_WS, S) == -6
    assert g(A, 0, 64, B, 32, None, 0, 4, 1, Y, *NO_WS, S) == -1
    assert g(A, 16, 60, B, 32, pp, 0, 4, 1, Y, *NO_WS, S) == -4           # K % 8
    assert g(A, 4, 64, B, 32, pp, 0, 4, 1, ctypes.c_void_p(0x60000), *NO_WS, S) == -2   # out is a peer's partial
    assert g(A, 4, 64, B, 32, pp, 0, 4, 1, ctypes.c_void_p(0x60000 - 64), *NO_WS, S) == -2  # out runs into one
    assert g(A, 4, 64, B, 32, pp, 0, 4, 1, ctypes.c_void_p(0x10000 + 64), *NO_WS, S) == -2  # out inside x
    mis = (ctypes.c_void_p * 2)(0, 0x60008)
    assert g(A, 0, 64, B, 32, ctypes.cast(mis, lib._ptr_array), 0, 2, 0, Y, *NO_WS, S) == -4


def _call(**kw):
    c = lib.tp_linear_call()
    c.x, c.M, c.K, c.w, c.N, c.y = 0x10000, 16, 64, 0x20000, 32, 0x30000
    c.out_dtype, c.epilogue = 0, 0
    for k, v in kw.items():
        if k == "plan":
            c.plan = lib._plan(v)
        else:
            setattr(c, k, v)
    return c


def test_linear_ex_validates_call_and_plan():
    f = C.tp_linear_ex
    assert f(None, S) == -1
    assert f(ctypes.byref(_call(M=0)), S) == 0
    assert f(ctypes.byref(_call(M=0, epilogue=4)), S) == -5                  # unknown epilogue
    nt = C.tp_prefill_tile_count()
    assert nt == lib.tp_prefill_tile_count() == 18
    assert f(ctypes.byref(_call(M=0, plan={"tile": nt})), S) == -6           # tile kernels 0 .. nt - 1
    assert f(ctypes.byref(_call(M=0, plan={"tile": nt - 1})), S) == 0
    assert f(ctypes.byref(_call(M=0, plan={"tile": 11})), S) == 0
    assert f(ctypes.byref(_call(M=0, plan={"decode": (3, 4, 2, 0)})), S) == -6   # no such decode kernel
    assert f(ctypes.byref(_call(M=0, plan={"decode": (8, 4, 2, 0)})), S) == 0
    assert f(ctypes.byref(_call(M=0, plan={"decode": (8, 1, 16, 1)})), S) == 0
    assert f(ctypes.byref(_call(M=0, epilogue=1, bias=0x40000)), S) == -2     # bias only with a plain store
    assert f(ctypes.byref(_call(M=0, epilogue=1, out_dtype=1)), S) == -5      # SwiGLU output is bf16
    arr = (ctypes.c_void_p * 2)(0, 0x60000)
    assert f(ctypes.byref(_call(M=0, epilogue=2, norm=1, partials=ctypes.cast(arr, lib._ptr_array), t=2)), S) == -2
    assert f(ctypes.byref(_call(M=0, epilogue=2, t=2)), S) == -1              # reduce needs partials
    assert f(ctypes.byref(_call(M=0, norm=1, eps=-1.0)), S) == -6
    assert f(ctypes.byref(_call(M=4, y=0x10000)), S) == -2                    # y == x


def test_library_has_no_tuning_state_or_allocations():
    """The C ABI exports no process-wide tuning hooks, and the library's
    sources allocate no device memory (scratch is the caller's workspace)."""
    assert not hasattr(C, "tp_tune_skinny") and not hasattr(C, "tp_tune_tiled")
    csrc = os.path.join(ROOT, "megatron_sharded_linears_amd", "csrc")
    for fn in os.listdir(csrc):
        text = open(os.path.join(csrc, fn)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        for call in ("hipMalloc", "hipFree", "hipMemset(", "hipHostMalloc"):
            assert call not in text, (fn, call)


def test_norm_calls_validate_before_any_hip_call():
    f = C.tp_add_rmsnorm
    R, G = ctypes.c_void_p(0x90000), ctypes.c_void_p(0xA0000)
    eps = ctypes.c_float(1e-5)
    assert f(A, 4, 64, NULL, G, eps, Y, S) == -1                      # residual NULL
    assert f(A, 4, 64, R, NULL, eps, Y, S) == -1
    assert f(A, 4, 60, R, G, eps, Y, S) == -4                         # H % 8
    assert f(A, 4, 64, R, G, ctypes.c_float(-1.0), Y, S) == -6        # eps < 0
    assert f(A, 4, 64, R, G, ctypes.c_float(float("nan")), Y, S) == -6
    assert f(A, 4, 64, R, G, ctypes.c_float(float("inf")), Y, S) == -6
    assert f(A, -1, 64, R, G, eps, Y, S) == -2
    assert f(A, 4, 0, R, G, eps, Y, S) == -2
    assert f(A, 4, 32776, R, G, eps, Y, S) == -2                      # H > 32768
    assert f(A, 0, 32768, R, G, eps, Y, S) == 0
    assert f(MIS, 4, 64, R, G, eps, Y, S) == -4
    assert f(A, 4, 64, R, G, eps, ctypes.c_void_p(0x90000 + 64), S) == -2   # out overlaps residual
    assert f(ctypes.c_void_p(0x90000 + 128), 4, 64, R, G, eps, Y, S) == -2  # x overlaps residual
    assert f(A, 0, 64, R, G, eps, Y, S) == 0                          # M == 0: no-op
    assert f(NULL, 0, 64, R, G, eps, Y, S) == 0                       # x may be NULL
    g = C.tp_reduce_add_rmsnorm
    arr = (ctypes.c_void_p * 3)(0x10000, 0x20000, 0x30000)
    pp = ctypes.cast(arr, lib._ptr_array)
    assert g(pp, 0, 0, 0, 64, R, G, eps, Y, S) == -6                  # t >= 1
    assert g(pp, 65, 0, 0, 64, R, G, eps, Y, S) == -6
    assert g(None, 3, 0, 0, 64, R, G, eps, Y, S) == -1
    assert g(pp, 3, 7, 0, 64, R, G, eps, Y, S) == -5                  # dtype
    bad = (ctypes.c_void_p * 2)(0x10000, 0x30008)
    assert g(ctypes.cast(bad, lib._ptr_array), 2, 0, 4, 64, R, G, eps, Y, S) == -4
    same = (ctypes.c_void_p * 2)(0x10000, 0x90000)
    assert g(ctypes.cast(same, lib._ptr_array), 2, 0, 4, 64, R, G, eps, Y, S) == -2   # partial is residual
    assert g(pp, 3, 1, 0, 64, R, G, eps, Y, S) == 0                   # fp32 partials, M == 0


def test_attention_validates_before_any_hip_call():
    f = C.tp_decode_attention
    KC, VC, LN, CT = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), ctypes.c_void_p(0x300000), \
        ctypes.c_void_p(0x400000)
    W = (WS, WSB)
    assert f(NULL, 4, 4, 1, 128, KC, VC, 64, LN, CT, *W, S) == -1
    assert f(A, 4, 4, 1, 128, KC, VC, 64, NULL, CT, *W, S) == -1
    assert f(A, 4, 4, 1, 96, KC, VC, 64, LN, CT, *W, S) == -2            # head_dim not 32/64/128/256
    assert f(A, 4, 6, 4, 128, KC, VC, 64, LN, CT, *W, S) == -2           # nq % nkv
    assert f(A, 4, 18, 2, 128, KC, VC, 64, LN, CT, *W, S) == -2          # group of 9 > 8
    assert f(A, 4, 4, 1, 128, KC, VC, 0, LN, CT, *W, S) == -2            # L >= 1
    assert f(A, 4, 4, 1, 128, KC, VC, 32769, LN, CT, *W, S) == -2        # L <= 32768
    assert f(A, -1, 4, 1, 128, KC, VC, 64, LN, CT, *W, S) == -2
    assert f(A, 65536, 4, 1, 128, KC, VC, 64, LN, CT, *W, S) == -2
    assert f(MIS, 4, 4, 1, 128, KC, VC, 64, LN, CT, *W, S) == -4
    assert f(A, 4, 4, 1, 128, KC, VC, 64, ctypes.c_void_p(0x300002), CT, *W, S) == -4   # lens 4-byte aligned
    assert f(A, 4, 4, 1, 128, KC, KC, 64, LN, CT, *W, S) == -2           # caches overlap
    assert f(A, 4, 4, 1, 128, KC, VC, 64, LN, ctypes.c_void_p(0x100000 + 256), *W, S) == -2   # ctx in the K cache
    assert f(A, 4, 4, 1, 128, KC, VC, 64, LN, CT, ctypes.c_void_p(0x400000 - 4096), WSB, S) == -2  # ws over ctx
    assert f(A, 0, 4, 1, 128, KC, VC, 64, LN, CT, *W, S) == 0            # B == 0: no-op


def test_folded_norm_calls_validate_before_any_hip_call():
    """The norm-folded decode calls: argument errors before any HIP call;
    M = 0 is a no-op."""
    eps = ctypes.c_float(1e-5)
    f = C.tp_rmsnorm_column_linear          # h, eps, M, K, w_folded, N, bias, y, ws, ws_bytes, stream
    assert f(NULL, eps, 4, 64, B, 32, NULL, Y, *NO_WS, S) == -1
    assert f(A, eps, 4, 60, B, 32, NULL, Y, *NO_WS, S) == -4                          # K % 8
    assert f(MIS, eps, 4, 64, B, 32, NULL, Y, *NO_WS, S) == -4
    assert f(A, ctypes.c_float(-1.0), 4, 64, B, 32, NULL, Y, *NO_WS, S) == -6         # eps < 0
    assert f(A, ctypes.c_float(float("nan")), 4, 64, B, 32, NULL, Y, *NO_WS, S) == -6
    assert f(A, eps, 4, 40000, B, 32, NULL, ctypes.c_void_p(0x800000), *NO_WS, S) == -2   # row wider than 32768
    assert f(A, eps, 4, 64, B, 32, NULL, ctypes.c_void_p(0x10000 + 64), *NO_WS, S) == -2   # y overlaps h
    assert f(A, eps, 0, 64, B, 32, NULL, Y, *NO_WS, S) == 0
    g = C.tp_rmsnorm_column_linear_swiglu   # h, eps, M, K, w_gate_up_folded, i_shard, act, ws, ws_bytes, stream
    assert g(A, eps, 4, 64, B, 0, Y, *NO_WS, S) == -2                                 # i_shard <= 0
    assert g(A, ctypes.c_float(float("inf")), 4, 64, B, 16, Y, *NO_WS, S) == -6
    assert g(NULL, eps, 4, 64, B, 16, Y, *NO_WS, S) == -1
    assert g(A, eps, 0, 64, B, 16, Y, *NO_WS, S) == 0
    h = C.tp_fold_norm_weight               # w, N, K, gamma, w_folded, stream
    assert h(NULL, 4, 64, B, Y, S) == -1
    assert h(A, 4, 64, NULL, Y, S) == -1
    assert h(A, 0, 64, B, Y, S) == -2
    assert h(A, 4, 60, B, Y, S) == -4
    assert h(MIS, 4, 64, B, Y, S) == -4
    assert h(A, 4, 64, B, ctypes.c_void_p(0x10000 + 16), S) == -2             # out overlaps w partly
    assert h(A, 4, 64, ctypes.c_void_p(0x30000 + 16), Y, S) == -2             # gamma inside out
    r = C.tp_row_linear_reduce_add          # x, M, K, w, N, partials, dtype, t, rank, residual, ws, ws_bytes, stream
    arr = (ctypes.c_void_p * 2)(0, 0x60000)
    pp = ctypes.cast(arr, lib._ptr_array)
    assert r(A, 4, 64, B, 32, None, 0, 2, 0, Y, *NO_WS, S) == -1
    assert r(A, 4, 64, B, 32, pp, 0, 0, 0, Y, *NO_WS, S) == -6                           # t < 1
    assert r(A, 4, 64, B, 32, pp, 0, 2, 2, Y, *NO_WS, S) == -6                           # rank >= t
    assert r(A, 4, 64, B, 32, pp, 0, 2, 0, ctypes.c_void_p(0x60000), *NO_WS, S) == -2    # residual is a peer's partial
    assert r(ctypes.c_void_p(0x30000 + 64), 4, 64, B, 32, pp, 0, 2, 0, Y, *NO_WS, S) == -2   # x overlaps the residual
    mis = (ctypes.c_void_p * 2)(0, 0x60008)
    assert r(A, 4, 64, B, 32, ctypes.cast(mis, lib._ptr_array), 0, 2, 0, Y, *NO_WS, S) == -4
    null_peer = (ctypes.c_void_p * 2)(0, 0)
    assert r(A, 4, 64, B, 32, ctypes.cast(null_peer, lib._ptr_array), 0, 2, 0, Y, *NO_WS, S) == -1
    assert r(A, 0, 64, B, 32, pp, 0, 2, 0, Y, *NO_WS, S) == 0


def test_sanitized_build_is_the_one_loaded():
    """Under the sanitizer run (tests/test_abi_sanitized.py) this process must
    have loaded the ASan runtime and the sanitized library."""
    if os.environ.get("TPSHARD_EXPECT_SANITIZED") != "1":
        pytest.skip("not the sanitized run")
    maps = open("/proc/self/maps").read()
    assert "libasan" in maps
    assert lib.library_path().endswith("libtpshard_asan.so") and lib.library_path() in maps


def test_noalloc_linear_validates_and_rejects_large_plans_before_any_hip_call():
    """tp_column_linear_noalloc checks its arguments, and that the plan
    tp_column_linear would take fits its fixed 4 MiB of partials, on the host
    before its first HIP call."""
    f = C.tp_column_linear_noalloc
    assert f(NULL, 16, 64, B, 32, NULL, Y, S) == -1
    assert f(A, 16, 60, B, 32, NULL, Y, S) == -4
    assert f(A, 16, 64, B, 32, NULL, ctypes.c_void_p(0x10000 + 256), S) == -2   # y inside x
    assert f(A, 0, 64, B, 32, NULL, Y, S) == 0
    X, W, Yb = ctypes.c_void_p(0x1000000), ctypes.c_void_p(0x3000000), ctypes.c_void_p(0x8000000)
    # 64 tokens of a 2816 x 4096 weight (44 tiles of 64 rows: the decode
    # kernel): K split 8 ways, 8 x 64 x 2816 fp32 partials (5.8 MB) do not
    # fit: rejected, nothing launched
    assert f(X, 64, 4096, W, 2816, NULL, Yb, S) == -2
