"""ctypes binding of libtpshard, with the names of its C entry points.

Argument marshalling only: each wrapper takes torch tensors, checks that their
shapes, dtypes and devices agree with one another, and passes data pointers,
sizes and the current HIP stream to the C function of the same name. Every
step of the computation runs in the library's gfx950 kernels; there is no
fallback of any kind. If the shared library is missing, importing this module
fails with an ImportError.

torch is imported before the library is loaded so that the process uses
torch's HIP runtime (the library links libamdhip64.so.7 by soname and binds to
the already-loaded copy); stream handles from torch are then valid here.
"""

import ctypes
import os

import torch

# TPSHARD_LIB may name another build of the same library (e.g. a tuning build).
_LIB_PATH = os.environ.get("TPSHARD_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                          "libtpshard.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is not built; run `python -m megatron_sharded_linears_amd.build` "
        "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(_LIB_PATH)

# ----------------------------------------------------------------- constants

TP_OK = 0
TP_BF16, TP_F32 = 0, 1
TP_W_QKV, TP_W_O, TP_W_GATE_UP, TP_W_DOWN, TP_W_EMBED, TP_W_LM_HEAD = range(6)
TP_MAX_SHARDS = 64

KIND = {"qkv": TP_W_QKV, "o": TP_W_O, "gate_up": TP_W_GATE_UP, "down": TP_W_DOWN,
        "embed": TP_W_EMBED, "lm_head": TP_W_LM_HEAD}

STATUS_NAMES = {0: "TP_OK", -1: "TP_ERR_NULL", -2: "TP_ERR_SHAPE", -3: "TP_ERR_DIVISIBILITY",
                -4: "TP_ERR_ALIGNMENT", -5: "TP_ERR_DTYPE", -6: "TP_ERR_RANGE", -7: "TP_ERR_HIP"}

TP_EPI_STORE, TP_EPI_SWIGLU, TP_EPI_REDUCE, TP_EPI_REDUCE_ADD = range(4)
TP_WS_COUNTER_BYTES = 262144


class tp_model_cfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("intermediate", ctypes.c_int32), ("vocab", ctypes.c_int32)]


class tp_linear_plan(ctypes.Structure):
    _fields_ = [("decode_ksteps", ctypes.c_int32), ("decode_nwn", ctypes.c_int32), ("decode_nwk", ctypes.c_int32),
                ("decode_x_direct", ctypes.c_int32), ("prefill_tile", ctypes.c_int32)]


class tp_linear_call(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("M", ctypes.c_int64), ("K", ctypes.c_int64), ("w", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("bias", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("out_dtype", ctypes.c_int32), ("epilogue", ctypes.c_int32),
                ("partials", ctypes.POINTER(ctypes.c_void_p)), ("partial_dtype", ctypes.c_int32),
                ("t", ctypes.c_int32), ("rank", ctypes.c_int32), ("norm", ctypes.c_int32), ("eps", ctypes.c_float),
                ("plan", tp_linear_plan), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64)]


class TPError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib.tp_status_string(status).decode()
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({msg})")


# --------------------------------------------------------------- prototypes

_vp, _i64, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
_cfgp = ctypes.POINTER(tp_model_cfg)
_ptr_array = ctypes.POINTER(ctypes.c_void_p)

_ws = [_vp, _i64]           # workspace, workspace_bytes

_PROTOS = {
    "tp_status_string": (ctypes.c_char_p, [_int]),
    "tp_full_shape": (_int, [_cfgp, _int, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "tp_shard_shape": (_int, [_cfgp, _int, _int, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "tp_vocab_shard_rows": (_i64, [_i64, _int]),
    "tp_kv_heads_of_rank": (_int, [_cfgp, _int, _int, ctypes.POINTER(_int), ctypes.POINTER(_int)]),
    "tp_workspace_bytes": (_i64, []),
    "tp_prefill_tile_count": (ctypes.c_int, []),
    "tp_shard_weights": (_int, [_cfgp, _int, _int, _int, _vp, _vp, _vp]),
    "tp_column_linear": (_int, [_vp, _i64, _i64, _vp, _i64, _vp, _vp] + _ws + [_vp]),
    "tp_swiglu": (_int, [_vp, _i64, _i64, _vp, _vp]),
    "tp_column_linear_swiglu": (_int, [_vp, _i64, _i64, _vp, _i64, _vp] + _ws + [_vp]),
    "tp_row_linear_reduce": (_int, [_vp, _i64, _i64, _vp, _i64, _ptr_array, _int, _int, _int, _vp] + _ws + [_vp]),
    "tp_row_linear_reduce_add": (_int, [_vp, _i64, _i64, _vp, _i64, _ptr_array, _int, _int, _int, _vp] + _ws + [_vp]),
    "tp_fold_norm_weight": (_int, [_vp, _i64, _i64, _vp, _vp, _vp]),
    "tp_rmsnorm_column_linear": (_int, [_vp, ctypes.c_float, _i64, _i64, _vp, _i64, _vp, _vp] + _ws + [_vp]),
    "tp_rmsnorm_column_linear_swiglu": (_int, [_vp, ctypes.c_float, _i64, _i64, _vp, _i64, _vp] + _ws + [_vp]),
    "tp_row_linear_partial": (_int, [_vp, _i64, _i64, _vp, _i64, _vp, _int] + _ws + [_vp]),
    "tp_reduce_partials": (_int, [_ptr_array, _int, _i64, _int, _vp, _int, _vp]),
    "tp_vocab_embed": (_int, [_vp, _i64, _vp, _i64, _int, _int, _i64, _vp, _vp]),
    "tp_lm_head_shard": (_int, [_vp, _i64, _i64, _vp, _i64, _vp, _int] + _ws + [_vp]),
    "tp_concat_logits": (_int, [_ptr_array, _int, _i64, _i64, _i64, _int, _vp, _vp]),
    "tp_add_rmsnorm": (_int, [_vp, _i64, _i64, _vp, _vp, ctypes.c_float, _vp, _vp]),
    "tp_reduce_add_rmsnorm": (_int, [_ptr_array, _int, _int, _i64, _i64, _vp, _vp, ctypes.c_float, _vp, _vp]),
    "tp_decode_attention": (_int, [_vp, _i64, _int, _int, _int, _vp, _vp, _i64, _vp, _vp] + _ws + [_vp]),
    "tp_linear_ex": (_int, [ctypes.POINTER(tp_linear_call), _vp]),
    "tp_column_linear_noalloc": (_int, [_vp, _i64, _i64, _vp, _i64, _vp, _vp, _vp]),
}
for _name, (_res, _args) in _PROTOS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_PROTOS)


def library_path():
    return _LIB_PATH


# ------------------------------------------------------------------ helpers

def _check(status, where):
    if status != TP_OK:
        raise TPError(status, where)


def _cfg(cfg):
    if isinstance(cfg, tp_model_cfg):
        return cfg
    return tp_model_cfg(cfg["hidden"], cfg["num_q_heads"], cfg["num_kv_heads"], cfg["head_dim"],
                        cfg["intermediate"], cfg["vocab"])


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev(t, name, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    return ctypes.c_void_p(t.data_ptr())


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return TP_BF16
    if dt == torch.float32:
        return TP_F32
    raise ValueError(f"unsupported dtype {dt}")


def _ptrs(tensors):
    arr = (ctypes.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])
    return ctypes.cast(arr, _ptr_array), arr


# ------------------------------------------------------------ host queries

def tp_status_string(status):
    return _lib.tp_status_string(status).decode()


def tp_full_shape(cfg, kind):
    r, c = _i64(), _i64()
    _check(_lib.tp_full_shape(ctypes.byref(_cfg(cfg)), KIND.get(kind, kind), ctypes.byref(r), ctypes.byref(c)),
           "tp_full_shape")
    return r.value, c.value


def tp_shard_shape(cfg, t, kind):
    r, c = _i64(), _i64()
    _check(_lib.tp_shard_shape(ctypes.byref(_cfg(cfg)), t, KIND.get(kind, kind), ctypes.byref(r), ctypes.byref(c)),
           "tp_shard_shape")
    return r.value, c.value


def tp_vocab_shard_rows(vocab, t):
    v = _lib.tp_vocab_shard_rows(vocab, t)
    if v < 0:
        raise TPError(int(v), "tp_vocab_shard_rows")
    return v


def tp_kv_heads_of_rank(cfg, t, rank):
    f, c = _int(), _int()
    _check(_lib.tp_kv_heads_of_rank(ctypes.byref(_cfg(cfg)), t, rank, ctypes.byref(f), ctypes.byref(c)),
           "tp_kv_heads_of_rank")
    return f.value, c.value


def tp_workspace_bytes():
    return int(_lib.tp_workspace_bytes())


def tp_prefill_tile_count():
    """Tiled kernel shapes a plan's "tile" may name (0 .. count - 1)."""
    return int(_lib.tp_prefill_tile_count())


# --------------------------------------------------------------- workspace

_default_ws = {}


def make_workspace(nbytes=None, device=None):
    """A zero-filled device buffer to pass as `workspace=` (the counters at its
    front must start at zero; every call leaves them zero). Calls that share
    one workspace must be ordered on one stream."""
    n = tp_workspace_bytes() if nbytes is None else int(nbytes)
    return torch.zeros(n, dtype=torch.uint8, device=device if device is not None else "cuda")


def default_workspace(device=None):
    """The workspace the wrappers use when none is passed: one per device,
    made on first use (outside any graph capture). For calls on one stream;
    callers on several streams pass workspaces of their own."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    if dev.index is None:
        dev = torch.device("cuda", torch.cuda.current_device())
    ws = _default_ws.get(dev.index)
    if ws is None:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("no default workspace yet on this device: make one call (or default_workspace()) "
                               "before capturing a graph, or pass workspace=")
        ws = make_workspace(device=dev)
        torch.cuda.synchronize(dev)
        _default_ws[dev.index] = ws
    return ws


def _ws_args(workspace, like):
    """(pointer, bytes) of a workspace: a uint8 device tensor, None for the
    device's default, or 0 for none at all."""
    if isinstance(workspace, int) and workspace == 0:
        return None, 0
    ws = default_workspace(like.device) if workspace is None else workspace
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


def _plan(plan):
    """tp_linear_plan from a dict: decode=(ksteps, nwn, nwk, x_direct) and/or
    tile=<prefill kernel index>."""
    p = tp_linear_plan(0, 0, 0, 0, 0)
    if plan is None:
        return p
    if "decode" in plan and plan["decode"] is not None:
        p.decode_ksteps, p.decode_nwn, p.decode_nwk, p.decode_x_direct = (int(v) for v in plan["decode"])
    if "tile" in plan and plan["tile"] is not None:
        p.prefill_tile = int(plan["tile"]) + 1
    return p


def _linear_ex(x, M, K, w, N, y, out_dtype, epilogue, bias=None, partials=None, partial_dtype=TP_BF16, t=0, rank=0,
               norm_eps=None, plan=None, workspace=None, stream=None, where="tp_linear_ex"):
    """Any linear through tp_linear_ex with an explicit kernel plan."""
    c = tp_linear_call()
    c.x, c.M, c.K, c.w, c.N = x, M, K, w, N
    c.bias = bias
    c.y = y
    c.out_dtype, c.epilogue = out_dtype, epilogue
    keep = None
    if partials is not None:
        keep = (ctypes.c_void_p * len(partials))(*partials)
        c.partials = ctypes.cast(keep, _ptr_array)
    c.partial_dtype, c.t, c.rank = partial_dtype, t, rank
    c.norm = 0 if norm_eps is None else 1
    c.eps = 0.0 if norm_eps is None else float(norm_eps)
    c.plan = _plan(plan)
    c.workspace, c.workspace_bytes = workspace
    _check(_lib.tp_linear_ex(ctypes.byref(c), _stream(stream)), where)
    del keep


# ------------------------------------------------------------ device calls

def tp_shard_weights(cfg, t, rank, kind, full_w, shard_w, stream=None):
    c = _cfg(cfg)
    k = KIND.get(kind, kind)
    if tuple(full_w.shape) != tp_full_shape(c, k):
        raise ValueError(f"full weight shape {tuple(full_w.shape)} != {tp_full_shape(c, k)}")
    if tuple(shard_w.shape) != tp_shard_shape(c, t, k):
        raise ValueError(f"shard shape {tuple(shard_w.shape)} != {tp_shard_shape(c, t, k)}")
    _check(_lib.tp_shard_weights(ctypes.byref(c), t, rank, k, _dev(full_w, "full_w", torch.bfloat16, 2),
                                 _dev(shard_w, "shard_w", torch.bfloat16, 2), _stream(stream)),
           "tp_shard_weights")
    return shard_w


def _linear_shapes(x, w, y, name):
    M, K = x.shape
    N, K2 = w.shape
    if K != K2:
        raise ValueError(f"{name}: x has K={K}, weight has K={K2}")
    if tuple(y.shape) != (M, N):
        raise ValueError(f"{name}: output shape {tuple(y.shape)} != {(M, N)}")
    return M, K, N


def tp_column_linear(x, w_shard, y, bias=None, workspace=None, plan=None, stream=None):
    """y = x w_shard^T (+ bias). `workspace`: a uint8 device tensor (None: the
    device's default, 0: none); `plan`: an explicit kernel shape
    ({"decode": (ksteps, nwn, nwk, x_direct)} or {"tile": index}) run through
    tp_linear_ex, for sweeps and variant tests."""
    M, K, N = _linear_shapes(x, w_shard, y, "tp_column_linear")
    b = None
    if bias is not None:
        b = _dev(bias, "bias", torch.bfloat16, 1)
        if bias.shape[0] != N:
            raise ValueError("bias length != N")
    xp, wp, yp = _dev(x, "x", torch.bfloat16, 2), _dev(w_shard, "w_shard", torch.bfloat16, 2), _dev(y, "y", torch.bfloat16, 2)
    ws = _ws_args(workspace, x)
    if plan is not None:
        _linear_ex(xp, M, K, wp, N, yp, TP_BF16, TP_EPI_STORE, bias=b, plan=plan, workspace=ws, stream=stream)
        return y
    _check(_lib.tp_column_linear(xp, M, K, wp, N, b, yp, *ws, _stream(stream)), "tp_column_linear")
    return y


def tp_column_linear_noalloc(x, w_shard, y, bias=None, stream=None):
    """tp_column_linear with its scratch in the library's fixed per-GPU array
    (no workspace, no allocation); TPError TP_ERR_SHAPE when the plan's split
    partials exceed that array."""
    M, K, N = _linear_shapes(x, w_shard, y, "tp_column_linear_noalloc")
    b = None
    if bias is not None:
        b = _dev(bias, "bias", torch.bfloat16, 1)
        if bias.shape[0] != N:
            raise ValueError("bias length != N")
    _check(_lib.tp_column_linear_noalloc(_dev(x, "x", torch.bfloat16, 2), M, K,
                                         _dev(w_shard, "w_shard", torch.bfloat16, 2), N, b,
                                         _dev(y, "y", torch.bfloat16, 2), _stream(stream)),
           "tp_column_linear_noalloc")
    return y


def tp_swiglu(gu, out, stream=None):
    M, two_i = gu.shape
    if two_i % 2 or tuple(out.shape) != (M, two_i // 2):
        raise ValueError("tp_swiglu: out must be [M, gu.shape[1] / 2]")
    _check(_lib.tp_swiglu(_dev(gu, "gu", torch.bfloat16, 2), M, two_i // 2, _dev(out, "out", torch.bfloat16, 2),
                          _stream(stream)), "tp_swiglu")
    return out


def _swiglu_shapes(x, w, act, name):
    M, K = x.shape
    two_i, K2 = w.shape
    if K != K2 or two_i % 2 or tuple(act.shape) != (M, two_i // 2):
        raise ValueError(f"{name}: need x [M, K], w_gate_up [2 I, K], act [M, I]")
    return M, K, two_i // 2


def tp_column_linear_swiglu(x, w_gate_up, act, workspace=None, plan=None, stream=None):
    M, K, Is = _swiglu_shapes(x, w_gate_up, act, "tp_column_linear_swiglu")
    xp, wp, ap = _dev(x, "x", torch.bfloat16, 2), _dev(w_gate_up, "w_gate_up", torch.bfloat16, 2), _dev(act, "act", torch.bfloat16, 2)
    ws = _ws_args(workspace, x)
    if plan is not None:
        _linear_ex(xp, M, K, wp, Is, ap, TP_BF16, TP_EPI_SWIGLU, plan=plan, workspace=ws, stream=stream)
        return act
    _check(_lib.tp_column_linear_swiglu(xp, M, K, wp, Is, ap, *ws, _stream(stream)), "tp_column_linear_swiglu")
    return act


def _peer_ptrs(partials, rank, M, N):
    """Device pointers of the other ranks' partials (slot `rank` ignored, None
    allowed) and their common dtype code."""
    t = len(partials)
    if t < 1 or t > TP_MAX_SHARDS:
        raise ValueError("need 1..64 partials")
    dts = {p.dtype for i, p in enumerate(partials) if i != rank and p is not None}
    if len(dts) > 1:
        raise ValueError("partials differ in dtype")
    dt = dts.pop() if dts else torch.bfloat16
    ptrs = []
    for i, p in enumerate(partials):
        if i == rank:
            ptrs.append(0)
            continue
        _dev(p, f"partials[{i}]", dt, 2)
        if tuple(p.shape) != (M, N):
            raise ValueError(f"partials[{i}] must be [M, N]")
        ptrs.append(p.data_ptr())
    return ptrs, _dtype_code(dt)


def _row_reduce(name, epilogue, x_shard, w_shard, partials, rank, y, workspace, plan, stream):
    M, K, N = _linear_shapes(x_shard, w_shard, y, name)
    ptrs, pdt = _peer_ptrs(partials, rank, M, N)
    t = len(partials)
    xp, wp, yp = _dev(x_shard, "x_shard", torch.bfloat16, 2), _dev(w_shard, "w_shard", torch.bfloat16, 2), \
        _dev(y, "out" if epilogue == TP_EPI_REDUCE else "residual", torch.bfloat16, 2)
    ws = _ws_args(workspace, x_shard)
    if plan is not None:
        _linear_ex(xp, M, K, wp, N, yp, TP_BF16, epilogue, partials=ptrs, partial_dtype=pdt, t=t, rank=rank,
                   plan=plan, workspace=ws, stream=stream, where=name)
        return y
    arr = (ctypes.c_void_p * t)(*ptrs)
    _check(getattr(_lib, name)(xp, M, K, wp, N, ctypes.cast(arr, _ptr_array), pdt, t, rank, yp, *ws, _stream(stream)),
           name)
    return y


def tp_row_linear_reduce(x_shard, w_shard, partials, rank, out, workspace=None, plan=None, stream=None):
    """`partials`: t entries; entry `rank` is ignored (None allowed), the others
    are the other ranks' [M, N] partials, all bf16 or all fp32 (the rank's own
    partial then enters the sum as that dtype stores it)."""
    return _row_reduce("tp_row_linear_reduce", TP_EPI_REDUCE, x_shard, w_shard, partials, rank, out, workspace, plan,
                       stream)


def tp_row_linear_reduce_add(x_shard, w_shard, partials, rank, residual, workspace=None, plan=None, stream=None):
    """residual <- bf16(residual + bf16(sum over ranks in order)), the rank's
    own partial being x_shard W^T; `partials` as in tp_row_linear_reduce."""
    return _row_reduce("tp_row_linear_reduce_add", TP_EPI_REDUCE_ADD, x_shard, w_shard, partials, rank, residual,
                       workspace, plan, stream)


def tp_fold_norm_weight(w, gamma, w_folded, stream=None):
    """w_folded = bf16(w * gamma) column by column: the RMSNorm weight folded
    into the next linear (load time). w_folded may be w."""
    N, K = w.shape
    _dev(gamma, "gamma", torch.bfloat16, 1)
    if gamma.shape[0] != K or tuple(w_folded.shape) != (N, K):
        raise ValueError("tp_fold_norm_weight: need w [N, K], gamma [K], w_folded [N, K]")
    _check(_lib.tp_fold_norm_weight(_dev(w, "w", torch.bfloat16, 2), N, K, gamma.data_ptr(),
                                    _dev(w_folded, "w_folded", torch.bfloat16, 2), _stream(stream)),
           "tp_fold_norm_weight")
    return w_folded


def tp_rmsnorm_column_linear(h, eps, w_folded, y, bias=None, workspace=None, plan=None, stream=None):
    """y = RMSNorm(h) W^T (+ bias) with the norm's gamma folded into w_folded
    (tp_fold_norm_weight); the normalised rows are not written."""
    M, K, N = _linear_shapes(h, w_folded, y, "tp_rmsnorm_column_linear")
    b = None
    if bias is not None:
        b = _dev(bias, "bias", torch.bfloat16, 1)
        if bias.shape[0] != N:
            raise ValueError("bias length != N")
    hp, wp, yp = _dev(h, "h", torch.bfloat16, 2), _dev(w_folded, "w_folded", torch.bfloat16, 2), _dev(y, "y", torch.bfloat16, 2)
    ws = _ws_args(workspace, h)
    if plan is not None:
        _linear_ex(hp, M, K, wp, N, yp, TP_BF16, TP_EPI_STORE, bias=b, norm_eps=eps, plan=plan, workspace=ws,
                   stream=stream)
        return y
    _check(_lib.tp_rmsnorm_column_linear(hp, float(eps), M, K, wp, N, b, yp, *ws, _stream(stream)),
           "tp_rmsnorm_column_linear")
    return y


def tp_rmsnorm_column_linear_swiglu(h, eps, w_gate_up_folded, act, workspace=None, plan=None, stream=None):
    """act = SwiGLU of RMSNorm(h) W_gate_up^T, gamma folded into the weight."""
    M, K, Is = _swiglu_shapes(h, w_gate_up_folded, act, "tp_rmsnorm_column_linear_swiglu")
    hp, wp, ap = (_dev(h, "h", torch.bfloat16, 2), _dev(w_gate_up_folded, "w_gate_up_folded", torch.bfloat16, 2),
                  _dev(act, "act", torch.bfloat16, 2))
    ws = _ws_args(workspace, h)
    if plan is not None:
        _linear_ex(hp, M, K, wp, Is, ap, TP_BF16, TP_EPI_SWIGLU, norm_eps=eps, plan=plan, workspace=ws, stream=stream)
        return act
    _check(_lib.tp_rmsnorm_column_linear_swiglu(hp, float(eps), M, K, wp, Is, ap, *ws, _stream(stream)),
           "tp_rmsnorm_column_linear_swiglu")
    return act


def tp_row_linear_partial(x_shard, w_shard, partial, workspace=None, plan=None, stream=None):
    M, K, N = _linear_shapes(x_shard, w_shard, partial, "tp_row_linear_partial")
    xp, wp = _dev(x_shard, "x_shard", torch.bfloat16, 2), _dev(w_shard, "w_shard", torch.bfloat16, 2)
    pp, dt = _dev(partial, "partial", partial.dtype, 2), _dtype_code(partial.dtype)
    ws = _ws_args(workspace, x_shard)
    if plan is not None:
        _linear_ex(xp, M, K, wp, N, pp, dt, TP_EPI_STORE, plan=plan, workspace=ws, stream=stream)
        return partial
    _check(_lib.tp_row_linear_partial(xp, M, K, wp, N, pp, dt, *ws, _stream(stream)), "tp_row_linear_partial")
    return partial


_EPI = {"store": TP_EPI_STORE, "swiglu": TP_EPI_SWIGLU, "reduce": TP_EPI_REDUCE, "reduce_add": TP_EPI_REDUCE_ADD}


def tp_linear_ex(x, w, y, epilogue="store", bias=None, partials=None, rank=0, eps=None, plan=None,
                 workspace=None, stream=None):
    """Any linear through the C call tp_linear_ex: `epilogue` "store" (y = x
    w^T (+ bias), bf16 or fp32 y), "swiglu" (w [2 I, K], y [M, I]), "reduce"
    or "reduce_add" (`partials` and `rank` as in tp_row_linear_reduce); `eps`
    given: the rows of x RMS-normalised (gamma folded into w); `plan`: the
    kernel shape, as in tp_column_linear."""
    e = _EPI[epilogue]
    M, K = x.shape
    if e == TP_EPI_SWIGLU:
        M, K, N = _swiglu_shapes(x, w, y, "tp_linear_ex")
    else:
        M, K, N = _linear_shapes(x, w, y, "tp_linear_ex")
    xp, wp = _dev(x, "x", torch.bfloat16, 2), _dev(w, "w", torch.bfloat16, 2)
    yp, dt = _dev(y, "y", y.dtype, 2), _dtype_code(y.dtype)
    b = None if bias is None else _dev(bias, "bias", torch.bfloat16, 1)
    ptrs, pdt, t = None, TP_BF16, 0
    if e in (TP_EPI_REDUCE, TP_EPI_REDUCE_ADD):
        ptrs, pdt = _peer_ptrs(partials, rank, M, N)
        t = len(partials)
    _linear_ex(xp, M, K, wp, N, yp, dt, e, bias=b, partials=ptrs, partial_dtype=pdt, t=t, rank=rank, norm_eps=eps,
               plan=plan, workspace=_ws_args(workspace, x), stream=stream)
    return y


def tp_reduce_partials(partials, out, stream=None):
    t = len(partials)
    if t < 1 or t > TP_MAX_SHARDS:
        raise ValueError("need 1..64 partials")
    numel = partials[0].numel()
    in_dt = partials[0].dtype
    for i, p in enumerate(partials):
        _dev(p, f"partials[{i}]", in_dt)
        if p.numel() != numel:
            raise ValueError("partials differ in size")
    _dev(out, "out", out.dtype)
    if out.numel() != numel:
        raise ValueError("out size != partial size")
    arr, keep = _ptrs(partials)
    _check(_lib.tp_reduce_partials(arr, t, numel, _dtype_code(in_dt), ctypes.c_void_p(out.data_ptr()),
                                   _dtype_code(out.dtype), _stream(stream)), "tp_reduce_partials")
    del keep
    return out


def _norm_operands(residual, gamma, out):
    _dev(residual, "residual", torch.bfloat16, 2)
    M, H = residual.shape
    _dev(gamma, "gamma", torch.bfloat16, 1)
    if gamma.shape[0] != H:
        raise ValueError("gamma length != hidden size")
    _dev(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (M, H):
        raise ValueError("out shape != residual shape")
    return M, H


def tp_add_rmsnorm(x, residual, gamma, eps, out, stream=None):
    """residual <- bf16(residual + x) (x None: unchanged); out <- RMSNorm of
    the new residual times gamma."""
    M, H = _norm_operands(residual, gamma, out)
    if x is not None:
        _dev(x, "x", torch.bfloat16, 2)
        if tuple(x.shape) != (M, H):
            raise ValueError("x shape != residual shape")
    _check(_lib.tp_add_rmsnorm(None if x is None else ctypes.c_void_p(x.data_ptr()), M, H,
                               ctypes.c_void_p(residual.data_ptr()), ctypes.c_void_p(gamma.data_ptr()),
                               float(eps), ctypes.c_void_p(out.data_ptr()), _stream(stream)), "tp_add_rmsnorm")
    return out


def tp_reduce_add_rmsnorm(partials, residual, gamma, eps, out, stream=None):
    """residual <- bf16(residual + bf16(sum of partials in rank order)); out <-
    RMSNorm of the new residual times gamma."""
    M, H = _norm_operands(residual, gamma, out)
    t = len(partials)
    if t < 1 or t > TP_MAX_SHARDS:
        raise ValueError("need 1..64 partials")
    in_dt = partials[0].dtype
    for i, p in enumerate(partials):
        _dev(p, f"partials[{i}]", in_dt, 2)
        if tuple(p.shape) != (M, H):
            raise ValueError("partial shape != residual shape")
    arr, keep = _ptrs(partials)
    _check(_lib.tp_reduce_add_rmsnorm(arr, t, _dtype_code(in_dt), M, H, ctypes.c_void_p(residual.data_ptr()),
                                      ctypes.c_void_p(gamma.data_ptr()), float(eps),
                                      ctypes.c_void_p(out.data_ptr()), _stream(stream)), "tp_reduce_add_rmsnorm")
    del keep
    return out


def tp_decode_attention(qkv, k_cache, v_cache, lens, nq, ctx, workspace=None, stream=None):
    """One decode step of the rank's GQA attention: the new K, V of each
    sequence go to position lens[b] of the caches, then ctx = attention of
    its nq query heads over positions 0..lens[b]. Caches [B, nkv, L, d]."""
    _dev(k_cache, "k_cache", torch.bfloat16, 4)
    _dev(v_cache, "v_cache", torch.bfloat16, 4)
    B, nkv, L, d = k_cache.shape
    if tuple(v_cache.shape) != (B, nkv, L, d):
        raise ValueError("v_cache shape != k_cache shape")
    _dev(qkv, "qkv", torch.bfloat16, 2)
    if tuple(qkv.shape) != (B, (nq + 2 * nkv) * d):
        raise ValueError("qkv must be [B, (nq + 2 nkv) d]")
    _dev(lens, "lens", torch.int32, 1)
    if lens.shape[0] != B:
        raise ValueError("lens must have B entries")
    _dev(ctx, "ctx", torch.bfloat16, 2)
    if tuple(ctx.shape) != (B, nq * d):
        raise ValueError("ctx must be [B, nq d]")
    _check(_lib.tp_decode_attention(ctypes.c_void_p(qkv.data_ptr()), B, nq, nkv, d,
                                    ctypes.c_void_p(k_cache.data_ptr()), ctypes.c_void_p(v_cache.data_ptr()), L,
                                    ctypes.c_void_p(lens.data_ptr()), ctypes.c_void_p(ctx.data_ptr()),
                                    *_ws_args(workspace, qkv), _stream(stream)), "tp_decode_attention")
    return ctx


def tp_vocab_embed(ids, e_shard, vocab, t, rank, out_partial, stream=None):
    M = ids.shape[0]
    Vs, H = e_shard.shape
    if Vs != tp_vocab_shard_rows(vocab, t):
        raise ValueError("e_shard rows != ceil(vocab / t)")
    if tuple(out_partial.shape) != (M, H):
        raise ValueError("out_partial must be [M, H]")
    _check(_lib.tp_vocab_embed(_dev(ids, "ids", torch.int32, 1), M, _dev(e_shard, "e_shard", torch.bfloat16, 2),
                               vocab, t, rank, H, _dev(out_partial, "out_partial", torch.bfloat16, 2),
                               _stream(stream)), "tp_vocab_embed")
    return out_partial


def tp_lm_head_shard(h, w_lm_shard, logits_shard, workspace=None, plan=None, stream=None):
    M, K, N = _linear_shapes(h, w_lm_shard, logits_shard, "tp_lm_head_shard")
    hp, wp = _dev(h, "h", torch.bfloat16, 2), _dev(w_lm_shard, "w_lm_shard", torch.bfloat16, 2)
    lp, dt = _dev(logits_shard, "logits_shard", logits_shard.dtype, 2), _dtype_code(logits_shard.dtype)
    ws = _ws_args(workspace, h)
    if plan is not None:
        _linear_ex(hp, M, K, wp, N, lp, dt, TP_EPI_STORE, plan=plan, workspace=ws, stream=stream)
        return logits_shard
    _check(_lib.tp_lm_head_shard(hp, M, K, wp, N, lp, dt, *ws, _stream(stream)), "tp_lm_head_shard")
    return logits_shard


def tp_concat_logits(shard_logits, vocab, out, stream=None):
    t = len(shard_logits)
    M, v_shard = shard_logits[0].shape
    dt = shard_logits[0].dtype
    for i, s in enumerate(shard_logits):
        _dev(s, f"shard_logits[{i}]", dt, 2)
        if tuple(s.shape) != (M, v_shard):
            raise ValueError("shard logits differ in shape")
    _dev(out, "out", dt, 2)
    if tuple(out.shape) != (M, vocab):
        raise ValueError("out must be [M, vocab]")
    arr, keep = _ptrs(shard_logits)
    _check(_lib.tp_concat_logits(arr, t, M, v_shard, vocab, _dtype_code(dt), ctypes.c_void_p(out.data_ptr()),
                                 _stream(stream)), "tp_concat_logits")
    del keep
    return out
