"""Thin ctypes binding of libmoe_mi355x.so (the C ABI in include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch supplies device memory and the current stream.  There is no
fallback: if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_mi355x.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_ERR_SCRATCH_LIMIT = -5
NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_NOALLOC_SCRATCH_BYTES

MOE_F32 = 0
MOE_BF16 = 1
MOE_FP8_E4M3 = 2
MOE_TOPK_THEN_SOFTMAX = 0
MOE_SOFTMAX_THEN_TOPK = 1

# every entry point declared in include/moe.h
SYMBOLS = ("moe_capacity", "moe_rows_bound", "moe_route_workspace_bytes",
           "moe_permute_workspace_bytes",
           "moe_grouped_ffn_workspace_bytes", "moe_workspace_bytes",
           "moe_route", "moe_permute", "moe_grouped_ffn", "moe_grouped_ffn_rows",
           "moe_combine",
           "moe_forward", "moe_forward_noalloc", "moe_route_stats_workspace_bytes", "moe_route_stats",
           "moe_forward_stats_workspace_bytes", "moe_forward_stats",
           "moe_forward_shared_workspace_bytes", "moe_forward_shared",
           "moe_grouped_ffn_scaled", "moe_forward_scaled",
           "moe_train_state_bytes", "moe_forward_train",
           "moe_backward_workspace_bytes", "moe_backward", "moe_status_string")


class MoeError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class Problem(ctypes.Structure):
    """moe_problem_t."""
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("E", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("capacity_factor", ctypes.c_float),
                ("act_dtype", ctypes.c_int), ("w_dtype", ctypes.c_int),
                ("gating", ctypes.c_int), ("out_dtype", ctypes.c_int)]


_lib = None


def load(path: str = LIB_PATH):
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with "
            "`python -m mixture_experts_layer_wavefront_amd.build`")
    # torch first: the library then binds to the HIP runtime torch has loaded
    # (loaded the other way round, a second runtime would own the library's
    # launches and see none of torch's memory or streams)
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(Problem)
    vp, sz, st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p
    i64 = ctypes.c_int64
    sig = {
        "moe_capacity": (i64, [P]),
        "moe_rows_bound": (i64, [P]),
        "moe_route_workspace_bytes": (sz, [P]),
        "moe_permute_workspace_bytes": (sz, [P]),
        "moe_grouped_ffn_workspace_bytes": (sz, [P]),
        "moe_workspace_bytes": (sz, [P]),
        "moe_route": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, sz, st]),
        "moe_permute": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       sz, st]),
        "moe_grouped_ffn": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, sz,
                                           st]),
        "moe_grouped_ffn_rows": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp,
                                                vp, vp, sz, st]),
        "moe_combine": (ctypes.c_int, [P, vp, vp, vp, vp, st]),
        "moe_forward": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       sz, st]),
        "moe_forward_noalloc": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, vp, st]),
        "moe_route_stats_workspace_bytes": (sz, [P]),
        "moe_route_stats": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, sz, st]),
        "moe_forward_stats_workspace_bytes": (sz, [P]),
        "moe_forward_stats": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                             vp, sz, st]),
        "moe_forward_shared_workspace_bytes": (sz, [P, ctypes.c_int32]),
        "moe_forward_shared": (ctypes.c_int, [P, ctypes.c_int32, vp, vp, vp, vp,
                                              vp, vp, vp, vp, vp, vp, vp, vp,
                                              sz, st, st]),
        "moe_grouped_ffn_scaled": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp,
                                                  vp, sz, st]),
        "moe_forward_scaled": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, vp,
                                              vp, vp, sz, st]),
        "moe_train_state_bytes": (sz, [P]),
        "moe_forward_train": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp, vp,
                                             vp, sz, vp, sz, st]),
        "moe_backward_workspace_bytes": (sz, [P]),
        "moe_backward": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, sz, vp, vp,
                                        vp, vp, vp, vp, vp, vp, sz, st]),
        "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().moe_status_string(int(status)).decode()


def _dt(x):
    return {"bf16": MOE_BF16, "f32": MOE_F32, "fp8": MOE_FP8_E4M3}[x] \
        if isinstance(x, str) else int(x)


def problem(T, d_model, E, top_k, d_ff, capacity_factor=0.0, dtype="bf16",
            gating=MOE_TOPK_THEN_SOFTMAX, out_dtype="f32", w_dtype=None) -> Problem:
    """moe_problem_t; `dtype` is the activation dtype and, unless `w_dtype`
    is given ("fp8": FP8 E4M3 expert weights), the expert-weight dtype;
    `out_dtype` the dtype of the layer output (fp32 by default)."""
    dt = _dt(dtype)
    return Problem(int(T), int(d_model), int(E), int(top_k), int(d_ff),
                   float(capacity_factor or 0.0), dt,
                   dt if w_dtype is None else _dt(w_dtype), int(gating),
                   _dt(out_dtype))


def capacity(p: Problem) -> int:
    return load().moe_capacity(ctypes.byref(p))


def rows_bound(p: Problem) -> int:
    return load().moe_rows_bound(ctypes.byref(p))


def route_workspace_bytes(p: Problem) -> int:
    return load().moe_route_workspace_bytes(ctypes.byref(p))


def permute_workspace_bytes(p: Problem) -> int:
    return load().moe_permute_workspace_bytes(ctypes.byref(p))


def grouped_ffn_workspace_bytes(p: Problem) -> int:
    return load().moe_grouped_ffn_workspace_bytes(ctypes.byref(p))


def workspace_bytes(p: Problem) -> int:
    return load().moe_workspace_bytes(ctypes.byref(p))


# ---------------------------------------------------------------- torch side
def _torch():
    import torch
    return torch


def _act_dtype(p: Problem):
    torch = _torch()
    return torch.bfloat16 if p.act_dtype == MOE_BF16 else torch.float32


def _out_dtype(p: Problem):
    torch = _torch()
    return torch.bfloat16 if p.out_dtype == MOE_BF16 else torch.float32


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status, where):
    if status != MOE_OK:
        raise MoeError(status, where)


def _workspace(nbytes, device, workspace):
    torch = _torch()
    if workspace is not None:
        return workspace
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def moe_route(p, X, W_r, bias=None, topk_idx=None, topk_w=None,
              workspace=None, stream=None):
    """Router logits, top-k ids and gate weights.  Returns (topk_idx, topk_w)."""
    torch = _torch()
    dev = X.device
    if topk_idx is None:
        topk_idx = torch.empty((p.T, p.top_k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((p.T, p.top_k), dtype=torch.float32, device=dev)
    ws = _workspace(route_workspace_bytes(p), dev, workspace)
    _check(load().moe_route(
        ctypes.byref(p), _ptr(X, _act_dtype(p), "X"),
        _ptr(W_r, torch.float32, "W_r"), _ptr(bias, torch.float32, "bias"),
        _ptr(topk_idx, torch.int32, "topk_idx"),
        _ptr(topk_w, torch.float32, "topk_w"), _ptr(ws), ws.numel(),
        _stream(stream)), "moe_route")
    return topk_idx, topk_w


def moe_permute(p, X, topk_idx, workspace=None, stream=None, out=None,
                copy_rows=True):
    """Counts, offsets, drops, dest rows, inverse map and X_perm (dict).
    copy_rows=False: no X_perm (None), for moe_grouped_ffn_rows."""
    torch = _torch()
    dev = X.device
    R = rows_bound(p)
    o = out if out is not None else dict(
        counts=torch.empty(p.E, dtype=torch.int32, device=dev),
        offsets=torch.empty(p.E + 1, dtype=torch.int32, device=dev),
        dropped=torch.empty(1, dtype=torch.int32, device=dev),
        dest_row=torch.empty((p.T, p.top_k), dtype=torch.int32, device=dev),
        row_token=torch.empty(max(R, 1), dtype=torch.int32, device=dev),
        X_perm=(torch.empty((max(R, 1), p.d_model), dtype=_act_dtype(p),
                            device=dev) if copy_rows else None))
    ws = _workspace(permute_workspace_bytes(p), dev, workspace)
    _check(load().moe_permute(
        ctypes.byref(p), _ptr(X, _act_dtype(p), "X"),
        _ptr(topk_idx, torch.int32, "topk_idx"),
        _ptr(o["counts"], torch.int32), _ptr(o["offsets"], torch.int32),
        _ptr(o["dropped"], torch.int32), _ptr(o["dest_row"], torch.int32),
        _ptr(o["row_token"], torch.int32), _ptr(o["X_perm"], _act_dtype(p)),
        _ptr(ws), ws.numel(), _stream(stream)), "moe_permute")
    return o


def moe_grouped_ffn(p, X_perm, offsets, W_gate, W_up, W_down, Y_perm=None,
                    workspace=None, stream=None):
    """Every expert's SwiGLU FFN over its rows.  Returns Y_perm (fp32)."""
    torch = _torch()
    dev = X_perm.device
    R = rows_bound(p)
    if Y_perm is None:
        Y_perm = torch.empty((max(R, 1), p.d_model), dtype=torch.float32,
                             device=dev)
    ws = _workspace(grouped_ffn_workspace_bytes(p), dev, workspace)
    wt = _act_dtype(p)
    _check(load().moe_grouped_ffn(
        ctypes.byref(p), _ptr(X_perm, wt, "X_perm"),
        _ptr(offsets, torch.int32, "offsets"), _ptr(W_gate, wt, "W_gate"),
        _ptr(W_up, wt, "W_up"), _ptr(W_down, wt, "W_down"),
        _ptr(Y_perm, torch.float32, "Y_perm"), _ptr(ws), ws.numel(),
        _stream(stream)), "moe_grouped_ffn")
    return Y_perm


def moe_grouped_ffn_rows(p, X, row_token, offsets, W_gate, W_up, W_down,
                         Y_perm=None, workspace=None, stream=None, w_scales=None):
    """moe_grouped_ffn with row r of X_perm read as X[row_token[r]] (bf16
    activations): no permuted copy of X.  FP8 expert weights (uint8 codes)
    take their scales [E, 3] in `w_scales`.  Returns Y_perm (fp32)."""
    torch = _torch()
    dev = X.device
    R = rows_bound(p)
    if Y_perm is None:
        Y_perm = torch.empty((max(R, 1), p.d_model), dtype=torch.float32,
                             device=dev)
    ws = _workspace(grouped_ffn_workspace_bytes(p), dev, workspace)
    wt = _act_dtype(p)
    qt = torch.uint8 if w_scales is not None else wt
    _check(load().moe_grouped_ffn_rows(
        ctypes.byref(p), _ptr(X, wt, "X"), _ptr(row_token, torch.int32, "row_token"),
        _ptr(offsets, torch.int32, "offsets"), _ptr(W_gate, qt, "W_gate"),
        _ptr(W_up, qt, "W_up"), _ptr(W_down, qt, "W_down"),
        _ptr(w_scales, torch.float32, "w_scales"),
        _ptr(Y_perm, torch.float32, "Y_perm"), _ptr(ws), ws.numel(),
        _stream(stream)), "moe_grouped_ffn_rows")
    return Y_perm


def moe_combine(p, Y_perm, dest_row, topk_w, out=None, stream=None):
    """Gate-weighted gather back to token order.  Returns out."""
    torch = _torch()
    if out is None:
        out = torch.empty((p.T, p.d_model), dtype=_out_dtype(p),
                          device=Y_perm.device)
    _check(load().moe_combine(
        ctypes.byref(p), _ptr(Y_perm, torch.float32, "Y_perm"),
        _ptr(dest_row, torch.int32, "dest_row"),
        _ptr(topk_w, torch.float32, "topk_w"),
        _ptr(out, _out_dtype(p), "out"), _stream(stream)), "moe_combine")
    return out


def moe_forward(p, X, W_r, bias, W_gate, W_up, W_down, out=None, stats=None,
                workspace=None, stream=None):
    """The whole layer.  Returns out; `stats` (int32 [2E+2]) if given is
    filled with counts | offsets | dropped."""
    torch = _torch()
    dev = X.device
    if out is None:
        out = torch.empty((p.T, p.d_model), dtype=_out_dtype(p), device=dev)
    ws = _workspace(workspace_bytes(p), dev, workspace)
    wt = _act_dtype(p)
    _check(load().moe_forward(
        ctypes.byref(p), _ptr(X, wt, "X"), _ptr(W_r, torch.float32, "W_r"),
        _ptr(bias, torch.float32, "bias"), _ptr(W_gate, wt, "W_gate"),
        _ptr(W_up, wt, "W_up"), _ptr(W_down, wt, "W_down"),
        _ptr(out, _out_dtype(p), "out"), _ptr(stats, torch.int32, "stats"),
        _ptr(ws),
        ws.numel(), _stream(stream)), "moe_forward")
    return out


def moe_forward_noalloc(p, X, W_r, bias, W_gate, W_up, W_down, out=None, stats=None,
                        stream=None):
    """moe_forward with the library's own fixed scratch instead of a
    workspace (the call allocates no device memory; `out` and `stats` are
    allocated here only when not given).  Returns out."""
    torch = _torch()
    if out is None:
        out = torch.empty((p.T, p.d_model), dtype=_out_dtype(p), device=X.device)
    wt = _act_dtype(p)
    _check(load().moe_forward_noalloc(
        ctypes.byref(p), _ptr(X, wt, "X"), _ptr(W_r, torch.float32, "W_r"),
        _ptr(bias, torch.float32, "bias"), _ptr(W_gate, wt, "W_gate"),
        _ptr(W_up, wt, "W_up"), _ptr(W_down, wt, "W_down"),
        _ptr(out, _out_dtype(p), "out"), _ptr(stats, torch.int32, "stats"),
        _stream(stream)), "moe_forward_noalloc")
    return out


def forward_shared_workspace_bytes(p: Problem, shared_d_ff: int) -> int:
    return load().moe_forward_shared_workspace_bytes(ctypes.byref(p),
                                                     int(shared_d_ff))


_side_streams = {}


def _side_stream(device):
    """One extra stream per device (default priority) for the shared expert."""
    torch = _torch()
    key = torch.device(device).index
    if key not in _side_streams:
        _side_streams[key] = torch.cuda.Stream(device=device)
    return _side_streams[key]


def moe_forward_shared(p, shared_d_ff, X, W_r, bias, W_gate, W_up, W_down,
                       Ws_gate, Ws_up, Ws_down, out=None, stats=None,
                       workspace=None, stream=None, side_stream="auto"):
    """The layer plus a shared expert (Ws_gate/Ws_up [shared_d_ff, d],
    Ws_down [d, shared_d_ff]).  side_stream: "auto" (a per-device extra
    stream), None (everything on `stream`) or a torch stream."""
    torch = _torch()
    dev = X.device
    if out is None:
        out = torch.empty((p.T, p.d_model), dtype=_out_dtype(p), device=dev)
    ws = _workspace(forward_shared_workspace_bytes(p, shared_d_ff), dev, workspace)
    wt = _act_dtype(p)
    if isinstance(side_stream, str):
        side_stream = _side_stream(dev)
    side = None if side_stream is None else ctypes.c_void_p(side_stream.cuda_stream)
    _check(load().moe_forward_shared(
        ctypes.byref(p), int(shared_d_ff), _ptr(X, wt, "X"),
        _ptr(W_r, torch.float32, "W_r"), _ptr(bias, torch.float32, "bias"),
        _ptr(W_gate, wt, "W_gate"), _ptr(W_up, wt, "W_up"),
        _ptr(W_down, wt, "W_down"), _ptr(Ws_gate, wt, "Ws_gate"),
        _ptr(Ws_up, wt, "Ws_up"), _ptr(Ws_down, wt, "Ws_down"),
        _ptr(out, _out_dtype(p), "out"), _ptr(stats, torch.int32, "stats"),
        _ptr(ws), ws.numel(), _stream(stream), side), "moe_forward_shared")
    return out


def route_stats_workspace_bytes(p: Problem) -> int:
    return load().moe_route_stats_workspace_bytes(ctypes.byref(p))


def forward_stats_workspace_bytes(p: Problem) -> int:
    return load().moe_forward_stats_workspace_bytes(ctypes.byref(p))


def moe_route_stats(p, X, W_r, bias=None, topk_idx=None, topk_w=None,
                    router_stats=None, workspace=None, stream=None):
    """moe_route plus the router statistics.  Returns (topk_idx, topk_w,
    router_stats [2E+2]: importance | mean_prob | aux_loss | z_loss)."""
    torch = _torch()
    dev = X.device
    if topk_idx is None:
        topk_idx = torch.empty((p.T, p.top_k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((p.T, p.top_k), dtype=torch.float32, device=dev)
    if router_stats is None:
        router_stats = torch.empty(2 * p.E + 2, dtype=torch.float32, device=dev)
    ws = _workspace(route_stats_workspace_bytes(p), dev, workspace)
    _check(load().moe_route_stats(
        ctypes.byref(p), _ptr(X, _act_dtype(p), "X"), _ptr(W_r, torch.float32, "W_r"),
        _ptr(bias, torch.float32, "bias"), _ptr(topk_idx, torch.int32, "topk_idx"),
        _ptr(topk_w, torch.float32, "topk_w"),
        _ptr(router_stats, torch.float32, "router_stats"), _ptr(ws), ws.numel(),
        _stream(stream)), "moe_route_stats")
    return topk_idx, topk_w, router_stats


def moe_forward_stats(p, X, W_r, bias, W_gate, W_up, W_down, out=None,
                      stats=None, router_stats=None, workspace=None, stream=None):
    """moe_forward plus the router statistics.  Returns (out, router_stats)."""
    torch = _torch()
    dev = X.device
    if out is None:
        out = torch.empty((p.T, p.d_model), dtype=_out_dtype(p), device=dev)
    if router_stats is None:
        router_stats = torch.empty(2 * p.E + 2, dtype=torch.float32, device=dev)
    ws = _workspace(forward_stats_workspace_bytes(p), dev, workspace)
    wt = _act_dtype(p)
    _check(load().moe_forward_stats(
        ctypes.byref(p), _ptr(X, wt, "X"), _ptr(W_r, torch.float32, "W_r"),
        _ptr(bias, torch.float32, "bias"), _ptr(W_gate, wt, "W_gate"),
        _ptr(W_up, wt, "W_up"), _ptr(W_down, wt, "W_down"),
        _ptr(out, _out_dtype(p), "out"), _ptr(stats, torch.int32, "stats"),
        _ptr(router_stats, torch.float32, "router_stats"), _ptr(ws), ws.numel(),
        _stream(stream)), "moe_forward_stats")
    return out, router_stats


def moe_grouped_ffn_scaled(p, X_perm, offsets, W_gate, W_up, W_down, w_scales,
                           Y_perm=None, workspace=None, stream=None):
    """moe_grouped_ffn with FP8 E4M3 expert weights (uint8 codes) and scales
    [E, 3] (gate, up, down).  Returns Y_perm (fp32)."""
    torch = _torch()
    dev = X_perm.device
    R = rows_bound(p)
    if Y_perm is None:
        Y_perm = torch.empty((max(R, 1), p.d_model), dtype=torch.float32, device=dev)
    ws = _workspace(grouped_ffn_workspace_bytes(p), dev, workspace)
    u8 = torch.uint8
    _check(load().moe_grouped_ffn_scaled(
        ctypes.byref(p), _ptr(X_perm, torch.bfloat16, "X_perm"),
        _ptr(offsets, torch.int32, "offsets"), _ptr(W_gate, u8, "W_gate"),
        _ptr(W_up, u8, "W_up"), _ptr(W_down, u8, "W_down"),
        _ptr(w_scales, torch.float32, "w_scales"),
        _ptr(Y_perm, torch.float32, "Y_perm"), _ptr(ws), ws.numel(),
        _stream(stream)), "moe_grouped_ffn_scaled")
    return Y_perm


def moe_forward_scaled(p, X, W_r, bias, W_gate, W_up, W_down, w_scales,
                       out=None, stats=None, workspace=None, stream=None):
    """moe_forward with FP8 E4M3 expert weights and scales [E, 3]."""
    torch = _torch()
    dev = X.device
    if out is None:
        out = torch.empty((p.T, p.d_model), dtype=_out_dtype(p), device=dev)
    ws = _workspace(workspace_bytes(p), dev, workspace)
    u8 = torch.uint8
    _check(load().moe_forward_scaled(
        ctypes.byref(p), _ptr(X, torch.bfloat16, "X"), _ptr(W_r, torch.float32, "W_r"),
        _ptr(bias, torch.float32, "bias"), _ptr(W_gate, u8, "W_gate"),
        _ptr(W_up, u8, "W_up"), _ptr(W_down, u8, "W_down"),
        _ptr(w_scales, torch.float32, "w_scales"), _ptr(out, _out_dtype(p), "out"),
        _ptr(stats, torch.int32, "stats"), _ptr(ws), ws.numel(), _stream(stream)),
        "moe_forward_scaled")
    return out


def train_state_bytes(p: Problem) -> int:
    return int(load().moe_train_state_bytes(ctypes.byref(p)))


def backward_workspace_bytes(p: Problem) -> int:
    return int(load().moe_backward_workspace_bytes(ctypes.byref(p)))


def moe_forward_train(p, X, W_r, bias, W_gate, W_up, W_down, out=None,
                      stats=None, state=None, workspace=None, stream=None):
    """moe_forward that also fills the state moe_backward needs.
    Returns (out, state)."""
    torch = _torch()
    dev = X.device
    if out is None:
        out = torch.empty((p.T, p.d_model), dtype=_out_dtype(p), device=dev)
    if state is None:
        state = torch.empty(max(train_state_bytes(p), 1), dtype=torch.uint8,
                            device=dev)
    ws = _workspace(workspace_bytes(p), dev, workspace)
    wt = _act_dtype(p)
    _check(load().moe_forward_train(
        ctypes.byref(p), _ptr(X, wt, "X"), _ptr(W_r, torch.float32, "W_r"),
        _ptr(bias, torch.float32, "bias"), _ptr(W_gate, wt, "W_gate"),
        _ptr(W_up, wt, "W_up"), _ptr(W_down, wt, "W_down"),
        _ptr(out, _out_dtype(p), "out"), _ptr(stats, torch.int32, "stats"),
        _ptr(state, torch.uint8, "state"), state.numel(), _ptr(ws), ws.numel(),
        _stream(stream)), "moe_forward_train")
    return out, state


def moe_backward(p, X, W_r, W_gate, W_up, W_down, state, dout, grads=None,
                 with_dbias=True, workspace=None, stream=None):
    """Gradients of the layer given dout [T, d_model] fp32 and the state of
    moe_forward_train.  Returns a dict dX, dW_r, dbias (None without
    with_dbias), dW_gate, dW_up, dW_down (fp32), reusing ``grads`` when
    given."""
    torch = _torch()
    dev = X.device
    f32 = torch.float32
    shapes = dict(dX=(p.T, p.d_model), dW_r=(p.E, p.d_model), dbias=(p.E,),
                  dW_gate=(p.E, p.d_ff, p.d_model), dW_up=(p.E, p.d_ff, p.d_model),
                  dW_down=(p.E, p.d_model, p.d_ff))
    g = dict(grads) if grads is not None else {}
    for name, shp in shapes.items():
        if name == "dbias" and not with_dbias:
            g[name] = None
        elif g.get(name) is None:
            g[name] = torch.empty(shp, dtype=f32, device=dev)
    ws = _workspace(backward_workspace_bytes(p), dev, workspace)
    wt = _act_dtype(p)
    _check(load().moe_backward(
        ctypes.byref(p), _ptr(X, wt, "X"), _ptr(W_r, f32, "W_r"),
        _ptr(W_gate, wt, "W_gate"), _ptr(W_up, wt, "W_up"),
        _ptr(W_down, wt, "W_down"), _ptr(state, torch.uint8, "state"),
        state.numel(), _ptr(dout, f32, "dout"), _ptr(g["dX"], f32, "dX"),
        _ptr(g["dW_r"], f32, "dW_r"), _ptr(g["dbias"], f32, "dbias"),
        _ptr(g["dW_gate"], f32, "dW_gate"), _ptr(g["dW_up"], f32, "dW_up"),
        _ptr(g["dW_down"], f32, "dW_down"), _ptr(ws), ws.numel(),
        _stream(stream)), "moe_backward")
    return g
