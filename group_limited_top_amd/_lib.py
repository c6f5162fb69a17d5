"""ctypes binding of libmoe (include/moe.h).

Argument marshalling only: every function takes torch tensors, checks that
their device, dtype, shape and contiguity match the layer description (the C
ABI takes bare pointers, so a wrong-sized tensor would be read out of bounds),
and passes ``data_ptr()`` plus the current HIP stream.  All computation happens
in the HIP kernels of libmoe.so; there is no fallback of any kind, and a
missing library raises at import.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_F_WRITE_LOGITS, MOE_F_CHECK_FINITE = 1, 2
MOE_STATUS_NONFINITE, MOE_STATUS_BAD_INDEX = 1, 2

EXPORTS = (
    "moe_workspace_size", "moe_route", "moe_permute", "moe_experts", "moe_layer_forward",
    "moe_residual_rmsnorm", "moe_status", "moe_sigmoid32", "moe_strerror",
    "moe_layer_forward_timed", "moe_stage_kernel", "moe_expert_stats", "moe_bias_update",
    "moe_aux_loss_workspace_size", "moe_aux_loss", "moe_backward_workspace_size",
    "moe_layer_backward", "moe_layer_forward_noalloc",
)
MOE_ERR_SCRATCH = -6
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20  # the static buffer of moe_layer_forward_noalloc
MOE_NSTAT = 8
STAT_NAMES = ("hits", "max_load", "min_load", "cv", "idle", "hottest", "coldest",
              "max_group_load")
# kernel stages (moe_stage_t), in launch order
STAGES = ("router_split", "logits", "select", "hist", "scan", "scatter", "tiles", "gate_up",
          "down", "combine")


class MoeDesc(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
        ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("I", ctypes.c_int32), ("I_shared", ctypes.c_int32),
        ("routed_scaling_factor", ctypes.c_float), ("dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_router", "expert_bias", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")]


class MoeError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: libmoe error {code}: {strerror(code)}")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m group_limited_top_amd.build` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    P, S = ctypes.c_void_p, ctypes.c_size_t
    D = ctypes.POINTER(MoeDesc)
    W = ctypes.POINTER(MoeWeights)
    i = ctypes.c_int
    lib.moe_workspace_size.argtypes = [D]
    lib.moe_workspace_size.restype = S
    lib.moe_route.argtypes = [D, P, P, P, P, P, P, P, S, P]
    lib.moe_route.restype = i
    lib.moe_permute.argtypes = [D, P, P, P, P, P, P, P, S, P]
    lib.moe_permute.restype = i
    lib.moe_experts.argtypes = [D, P, P, P, P, P, W, P, P, S, P]
    lib.moe_experts.restype = i
    lib.moe_layer_forward.argtypes = [D, P, W, P, P, P, P, P, P, P, S, P]
    lib.moe_layer_forward.restype = i
    lib.moe_layer_forward_noalloc.argtypes = [D, P, W, P, P, P, P, P, P, P]
    lib.moe_layer_forward_noalloc.restype = i
    lib.moe_layer_forward_timed.argtypes = [D, P, W, P, P, P, P, P, P, P, S, P, i, P, P]
    lib.moe_layer_forward_timed.restype = i
    lib.moe_residual_rmsnorm.argtypes = [D, P, P, P, P, ctypes.c_float, P]
    lib.moe_residual_rmsnorm.restype = i
    lib.moe_status.argtypes = [P, S, P, ctypes.POINTER(ctypes.c_uint32)]
    lib.moe_status.restype = i
    lib.moe_sigmoid32.argtypes = [P, P, ctypes.c_int64, P]
    lib.moe_sigmoid32.restype = i
    lib.moe_stage_kernel.argtypes = [D, i]
    lib.moe_stage_kernel.restype = ctypes.c_char_p
    i32 = ctypes.c_int32
    lib.moe_expert_stats.argtypes = [i32, i32, i32, P, P, P, P]
    lib.moe_expert_stats.restype = i
    lib.moe_bias_update.argtypes = [i32, P, P, P, ctypes.c_double, P]
    lib.moe_bias_update.restype = i
    lib.moe_aux_loss_workspace_size.argtypes = [i32, i32]
    lib.moe_aux_loss_workspace_size.restype = S
    lib.moe_aux_loss.argtypes = [i32, i32, P, P, P, P, P, P, S, P]
    lib.moe_aux_loss.restype = i
    lib.moe_backward_workspace_size.argtypes = [D]
    lib.moe_backward_workspace_size.restype = S
    lib.moe_layer_backward.argtypes = [D, P, W, P, P, P, P, P, P, P, P, P, P, P, P, S, P]
    lib.moe_layer_backward.restype = i
    lib.moe_strerror.argtypes = [i]
    lib.moe_strerror.restype = ctypes.c_char_p
    return lib


LIB = _load()


def strerror(code: int) -> str:
    return LIB.moe_strerror(code).decode()


# ---------------------------------------------------------------------------- helpers

def make_desc(T: int, H: int, *, E: int = 256, n_group: int = 8, topk_group: int = 4,
              top_k: int = 8, I: int = 512, I_shared: int = 512, scale: float = 2.5,
              dtype: str = "bf16", flags: int = 0) -> MoeDesc:
    return MoeDesc(T, H, E, n_group, topk_group, top_k, I, I_shared, scale,
                   MOE_BF16 if dtype == "bf16" else MOE_F32, flags)


def desc_from_shape(shape, flags: int = 0, T: int | None = None) -> MoeDesc:
    """MoeDesc for a group_limited_top_amd.synth.LayerShape."""
    return make_desc(shape.T if T is None else T, shape.H, E=shape.E, n_group=shape.n_group,
                     topk_group=shape.topk_group, top_k=shape.top_k, I=shape.I,
                     I_shared=shape.I_shared, scale=shape.scale, dtype=shape.dtype, flags=flags)


def _act_dtype(d: MoeDesc):
    return torch.bfloat16 if d.dtype == MOE_BF16 else torch.float32


def workspace_size(d: MoeDesc) -> int:
    n = LIB.moe_workspace_size(ctypes.byref(d))
    if n == 0:
        raise MoeError(-1, "moe_workspace_size (invalid or unsupported desc)")
    return n


def alloc_workspace(d: MoeDesc, device="cuda") -> torch.Tensor:
    """Zeroed workspace (the status word must start at zero)."""
    return torch.zeros(workspace_size(d), dtype=torch.uint8, device=device)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(t, name, shape, dtype, device, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _ws(d, ws):
    if ws is None or ws.dtype != torch.uint8 or not ws.is_contiguous() or ws.device.type != "cuda":
        raise ValueError("ws must be a contiguous cuda uint8 tensor (see alloc_workspace)")
    return ctypes.c_void_p(ws.data_ptr()), ws.numel()


def _rc(code, where):
    if code != 0:
        raise MoeError(code, where)


def _weights(d: MoeDesc, w: dict, device, need_router: bool) -> MoeWeights:
    dt = _act_dtype(d)
    E, I, H, Is = d.E, d.I, d.H, d.I_shared
    out = MoeWeights()
    out.w_router = _check(w.get("w_router"), "w_router", (E, H), torch.float32, device,
                          optional=not need_router)
    out.expert_bias = _check(w.get("expert_bias"), "expert_bias", (E,), torch.float32, device,
                             optional=True)
    out.w_gate = _check(w["w_gate"], "w_gate", (E, I, H), dt, device)
    out.w_up = _check(w["w_up"], "w_up", (E, I, H), dt, device)
    out.w_down = _check(w["w_down"], "w_down", (E, I, H), dt, device)
    opt = Is == 0
    out.ws_gate = _check(w.get("ws_gate"), "ws_gate", (Is, H), dt, device, optional=opt)
    out.ws_up = _check(w.get("ws_up"), "ws_up", (Is, H), dt, device, optional=opt)
    out.ws_down = _check(w.get("ws_down"), "ws_down", (Is, H), dt, device, optional=opt)
    return out


# ---------------------------------------------------------------------------- entry points

def moe_route(d: MoeDesc, x, w_router, expert_bias, logits, topk_idx, topk_w, ws, stream=None):
    dev = x.device
    T, H, E, K = d.T, d.H, d.E, d.top_k
    args = (
        _check(x, "x", (T, H), _act_dtype(d), dev),
        _check(w_router, "w_router", (E, H), torch.float32, dev),
        _check(expert_bias, "expert_bias", (E,), torch.float32, dev, optional=True),
        _check(logits, "logits", (T, E), torch.float32, dev, optional=True),
        _check(topk_idx, "topk_idx", (T, K), torch.int32, dev),
        _check(topk_w, "topk_w", (T, K), torch.float32, dev),
    )
    p, n = _ws(d, ws)
    _rc(LIB.moe_route(ctypes.byref(d), *args, p, n, _stream(stream)), "moe_route")


def moe_permute(d: MoeDesc, topk_idx, counts, offsets, sorted_pair, pair_slot, tracking, ws,
                stream=None):
    dev = topk_idx.device
    T, E, K = d.T, d.E, d.top_k
    args = (
        _check(topk_idx, "topk_idx", (T, K), torch.int32, dev),
        _check(counts, "counts", (E,), torch.int32, dev),
        _check(offsets, "offsets", (E + 1,), torch.int32, dev),
        _check(sorted_pair, "sorted_pair", (T * K,), torch.int32, dev),
        _check(pair_slot, "pair_slot", (T * K,), torch.int32, dev),
        _check(tracking, "tracking", (E,), torch.int64, dev, optional=True),
    )
    p, n = _ws(d, ws)
    _rc(LIB.moe_permute(ctypes.byref(d), *args, p, n, _stream(stream)), "moe_permute")


def moe_experts(d: MoeDesc, x, topk_w, offsets, sorted_pair, pair_slot, weights: dict, y, ws,
                stream=None):
    dev = x.device
    T, H, E, K = d.T, d.H, d.E, d.top_k
    dt = _act_dtype(d)
    args = (
        _check(x, "x", (T, H), dt, dev),
        _check(topk_w, "topk_w", (T, K), torch.float32, dev),
        _check(offsets, "offsets", (E + 1,), torch.int32, dev),
        _check(sorted_pair, "sorted_pair", (T * K,), torch.int32, dev),
        _check(pair_slot, "pair_slot", (T * K,), torch.int32, dev),
    )
    W = _weights(d, weights, dev, need_router=False)
    yp = _check(y, "y", (T, H), dt, dev)
    p, n = _ws(d, ws)
    _rc(LIB.moe_experts(ctypes.byref(d), *args, ctypes.byref(W), yp, p, n, _stream(stream)),
        "moe_experts")


def moe_layer_forward(d: MoeDesc, x, weights: dict, y, topk_idx_out=None, topk_w_out=None,
                      logits_out=None, counts_out=None, tracking=None, ws=None, stream=None,
                      timed_stage=None, events=None):
    """Whole layer.  With timed_stage (a name from STAGES) and events (a pair
    of torch.cuda.Event(enable_timing=True)), the pair is recorded around that
    stage's kernel on the same stream (moe_layer_forward_timed); raw hipEvent_t
    handles (ints) are accepted as well."""
    dev = x.device
    T, H, E, K = d.T, d.H, d.E, d.top_k
    dt = _act_dtype(d)
    xp = _check(x, "x", (T, H), dt, dev)
    W = _weights(d, weights, dev, need_router=True)
    args = (
        _check(y, "y", (T, H), dt, dev),
        _check(topk_idx_out, "topk_idx_out", (T, K), torch.int32, dev, optional=True),
        _check(topk_w_out, "topk_w_out", (T, K), torch.float32, dev, optional=True),
        _check(logits_out, "logits_out", (T, E), torch.float32, dev, optional=True),
        _check(counts_out, "counts_out", (E,), torch.int32, dev, optional=True),
        _check(tracking, "tracking", (E,), torch.int64, dev, optional=True),
    )
    p, n = _ws(d, ws)
    if timed_stage is None:
        _rc(LIB.moe_layer_forward(ctypes.byref(d), xp, ctypes.byref(W), *args, p, n,
                                  _stream(stream)), "moe_layer_forward")
        return
    ev0, ev1 = (e if isinstance(e, int) else e.cuda_event for e in events)
    _rc(LIB.moe_layer_forward_timed(ctypes.byref(d), xp, ctypes.byref(W), *args, p, n,
                                    _stream(stream), STAGES.index(timed_stage),
                                    ctypes.c_void_p(ev0), ctypes.c_void_p(ev1)),
        "moe_layer_forward_timed")


def moe_layer_forward_noalloc(d: MoeDesc, x, weights: dict, y, topk_idx_out=None,
                              topk_w_out=None, logits_out=None, counts_out=None, tracking=None,
                              stream=None):
    """The whole layer with the library's static per-device scratch buffer
    instead of a workspace (no device allocation anywhere in the call)."""
    dev = x.device
    T, H, E, K = d.T, d.H, d.E, d.top_k
    dt = _act_dtype(d)
    xp = _check(x, "x", (T, H), dt, dev)
    W = _weights(d, weights, dev, need_router=True)
    args = (
        _check(y, "y", (T, H), dt, dev),
        _check(topk_idx_out, "topk_idx_out", (T, K), torch.int32, dev, optional=True),
        _check(topk_w_out, "topk_w_out", (T, K), torch.float32, dev, optional=True),
        _check(logits_out, "logits_out", (T, E), torch.float32, dev, optional=True),
        _check(counts_out, "counts_out", (E,), torch.int32, dev, optional=True),
        _check(tracking, "tracking", (E,), torch.int64, dev, optional=True),
    )
    _rc(LIB.moe_layer_forward_noalloc(ctypes.byref(d), xp, ctypes.byref(W), *args,
                                      _stream(stream)), "moe_layer_forward_noalloc")


def moe_residual_rmsnorm(d: MoeDesc, x_in, y, x_out, r_out, eps: float = 1e-6, stream=None):
    dev = x_in.device
    dt = _act_dtype(d)
    shp = (d.T, d.H)
    args = (
        _check(x_in, "x_in", shp, dt, dev),
        _check(y, "y", shp, dt, dev, optional=True),
        _check(x_out, "x_out", shp, dt, dev),
        _check(r_out, "r_out", shp, dt, dev),
    )
    _rc(LIB.moe_residual_rmsnorm(ctypes.byref(d), *args, ctypes.c_float(eps), _stream(stream)),
        "moe_residual_rmsnorm")


def moe_stage_kernel(d: MoeDesc, stage: str):
    """Name of the kernel moe_layer_forward launches for an expert stage
    ("gate_up", "down", "combine") with this desc, or None."""
    r = LIB.moe_stage_kernel(ctypes.byref(d), STAGES.index(stage))
    return None if r is None else r.decode()


def moe_status(ws, stream=None) -> int:
    v = ctypes.c_uint32(0)
    _rc(LIB.moe_status(ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(stream),
                       ctypes.byref(v)), "moe_status")
    return v.value


def moe_sigmoid32(z, s, stream=None):
    dev = z.device
    zp = _check(z, "z", tuple(z.shape), torch.float32, dev)
    sp = _check(s, "s", tuple(z.shape), torch.float32, dev)
    _rc(LIB.moe_sigmoid32(zp, sp, z.numel(), _stream(stream)), "moe_sigmoid32")


# ---------------------------------------------------------------------------- load balancing

def moe_expert_stats(tracking, n_group: int, load=None, summary=None, stream=None):
    """Load statistics of tracked hits [L, E] int64 (one row per layer):
    returns (load fp32 [L, E], summary fp64 [L, MOE_NSTAT]) (see STAT_NAMES)."""
    if tracking.dim() == 1:
        tracking = tracking.view(1, -1)
    Lr, E = tracking.shape
    dev = tracking.device
    if load is None:
        load = torch.empty(Lr, E, dtype=torch.float32, device=dev)
    if summary is None:
        summary = torch.empty(Lr, MOE_NSTAT, dtype=torch.float64, device=dev)
    tp = _check(tracking, "tracking", (Lr, E), torch.int64, dev)
    lp = _check(load, "load", (Lr, E), torch.float32, dev)
    sp = _check(summary, "summary", (Lr, MOE_NSTAT), torch.float64, dev)
    _rc(LIB.moe_expert_stats(Lr, E, n_group, tp, lp, sp, _stream(stream)), "moe_expert_stats")
    return load, summary


def moe_bias_update(counts, bias_in, bias_out, rate: float, stream=None):
    """bias_out = bias_in moved against each expert's hit excess (bias_in may
    be None = zeros, or the same tensor as bias_out)."""
    E = counts.numel()
    dev = counts.device
    cp = _check(counts, "counts", (E,), torch.int32, dev)
    bi = _check(bias_in, "bias_in", (E,), torch.float32, dev, optional=True)
    bo = _check(bias_out, "bias_out", (E,), torch.float32, dev)
    _rc(LIB.moe_bias_update(E, cp, bi, bo, float(rate), _stream(stream)), "moe_bias_update")


def aux_loss_workspace(T: int, E: int, device="cuda") -> torch.Tensor:
    n = LIB.moe_aux_loss_workspace_size(T, E)
    if n == 0:
        raise MoeError(-1, "moe_aux_loss_workspace_size (invalid sizes)")
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_aux_loss(logits, counts, ws=None, out=None, stream=None):
    """(f fp64 [E], P fp64 [E], loss fp64 [1]) of the load-balancing loss
    E * sum_i f_i * P_i from router logits [T, E] fp32 and counts [E] int32;
    `out` may supply the three result tensors."""
    T, E = logits.shape
    dev = logits.device
    if ws is None:
        ws = aux_loss_workspace(T, E, dev)
    if out is None:
        out = (torch.empty(E, dtype=torch.float64, device=dev),
               torch.empty(E, dtype=torch.float64, device=dev),
               torch.empty(1, dtype=torch.float64, device=dev))
    f, P, loss = out
    lp = _check(logits, "logits", (T, E), torch.float32, dev)
    cp = _check(counts, "counts", (E,), torch.int32, dev)
    fp = _check(f, "f", (E,), torch.float64, dev)
    pp = _check(P, "P", (E,), torch.float64, dev)
    sp = _check(loss, "loss", (1,), torch.float64, dev)
    wp, wn = _ws(None, ws)
    _rc(LIB.moe_aux_loss(T, E, lp, cp, fp, pp, sp, wp, wn, _stream(stream)), "moe_aux_loss")
    return f, P, loss


# ---------------------------------------------------------------------------- backward

def backward_workspace(d: MoeDesc, device="cuda") -> torch.Tensor:
    n = LIB.moe_backward_workspace_size(ctypes.byref(d))
    if n == 0:
        raise MoeError(-2, "moe_backward_workspace_size (invalid or unsupported desc)")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def moe_layer_backward(d: MoeDesc, x, weights: dict, topk_idx, logits, dy, ws=None, out=None,
                       stream=None):
    """Gradients of sum(dy * y) for the routing topk_idx: returns dict(dx bf16
    [T, H], dw_router fp32 [E, H], dw_gate / dw_up / dw_down fp32 [E, I, H],
    dws_gate / dws_up / dws_down fp32 [I_shared, H] or None).  `out` may
    supply those tensors."""
    dev = x.device
    T, H, E, K, I, Is = d.T, d.H, d.E, d.top_k, d.I, d.I_shared
    dt = _act_dtype(d)
    if out is None:
        f32 = dict(dtype=torch.float32, device=dev)
        out = dict(dx=torch.empty(T, H, dtype=dt, device=dev),
                   dw_router=torch.empty(E, H, **f32), dw_gate=torch.empty(E, I, H, **f32),
                   dw_up=torch.empty(E, I, H, **f32), dw_down=torch.empty(E, I, H, **f32),
                   dws_gate=torch.empty(Is, H, **f32) if Is else None,
                   dws_up=torch.empty(Is, H, **f32) if Is else None,
                   dws_down=torch.empty(Is, H, **f32) if Is else None)
    if ws is None:
        ws = backward_workspace(d, dev)
    W = _weights(d, weights, dev, need_router=True)
    args = [
        _check(x, "x", (T, H), dt, dev), ctypes.byref(W),
        _check(topk_idx, "topk_idx", (T, K), torch.int32, dev),
        _check(logits, "logits", (T, E), torch.float32, dev),
        _check(dy, "dy", (T, H), dt, dev),
        _check(out["dx"], "dx", (T, H), dt, dev),
        _check(out["dw_router"], "dw_router", (E, H), torch.float32, dev),
        _check(out["dw_gate"], "dw_gate", (E, I, H), torch.float32, dev),
        _check(out["dw_up"], "dw_up", (E, I, H), torch.float32, dev),
        _check(out["dw_down"], "dw_down", (E, I, H), torch.float32, dev),
        _check(out["dws_gate"], "dws_gate", (Is, H), torch.float32, dev, optional=True),
        _check(out["dws_up"], "dws_up", (Is, H), torch.float32, dev, optional=True),
        _check(out["dws_down"], "dws_down", (Is, H), torch.float32, dev, optional=True),
    ]
    wp, wn = _ws(d, ws)
    _rc(LIB.moe_layer_backward(ctypes.byref(d), *args, wp, wn, _stream(stream)),
        "moe_layer_backward")
    return out


def moe_stack_forward(d: MoeDesc, x, layers, ws, eps: float = 1e-6, tracking=None,
                      idx_out=None, counts_out=None, on_layer=None, stream=None):
    """A residual stack of MoE layers, each x <- RN(x + layer(RN(RMSNorm(x)))).

    `x` [T][H] is updated in place; `layers` is a list of weight dicts;
    tracking (optional, [L][E] int64) accumulates per-layer counts; idx_out /
    counts_out (optional, [L][T][k] int32 / [L][E] int32) receive each
    layer's routing.  on_layer(l, x) is called after layer l (for inspection).
    Every step runs in libmoe kernels (moe_residual_rmsnorm, moe_layer_forward)."""
    r = torch.empty_like(x)
    y = torch.empty_like(x)
    moe_residual_rmsnorm(d, x, None, x, r, eps, stream)
    for l, w in enumerate(layers):
        moe_layer_forward(d, r, w, y,
                          topk_idx_out=None if idx_out is None else idx_out[l],
                          counts_out=None if counts_out is None else counts_out[l],
                          tracking=None if tracking is None else tracking[l], ws=ws, stream=stream)
        moe_residual_rmsnorm(d, x, y, x, r, eps, stream)
        if on_layer is not None:
            on_layer(l, x)
    return x
