"""CPU oracle of the group-limited top-k MoE layer (forward, load balancing and
the backward for a fixed routing) -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never calls it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, loops per token and per
expert); this module only marshals numpy arrays.  Activations and expert
weights are passed either as ``np.float32`` arrays or as bf16 bit patterns in
``np.uint16`` arrays (numpy has no bf16 type); the backward's functions also
take ``np.float64`` arrays (the finite-difference pins perturb in fp64).

Method source: the page "InternLumina-U2中256个专家的路由秘密：分组受限Top-K、
Expert Bias与Fused MoE详解", sections 二 (sigmoid router, group-limited top-k,
weight normalisation), 三 (selection-only expert bias, and its use for load
balancing), 四 (stacked SwiGLU experts, eager per-expert loop and
sort-by-expert inference), 五 (shared expert added unweighted), 六 (per-expert
hit counts and their statistics); and the page at m.lqnn.cn/news/279712,
section "MoE 负载均衡 Loss 别忘加" (the auxiliary loss E * sum_i f_i * P_i).

The backward (chain rule written out in ``oracle.c``) is pinned by central
finite differences of every input and weight, by torch.autograd applied to
the same forward written with torch ops, and by identities of the forward's
form (``tests/test_oracle_backward.py``).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
except the layer output's numeric value at full size, which no page prints
("parity unpinned" beyond the invariants and special cases those tests check).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_SO lets the mutation test load a deliberately broken copy
_SO = os.environ.get("ORACLE_SO") or os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

F32, BF16, F64 = 0, 1, 2
_lib = None


def build() -> str:
    """Compile oracle.c with contraction and fast-math off (sigma32 needs it)."""
    cmd = [
        "gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
        "-pthread", "-o", _SO + ".tmp", _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(_SO + ".tmp", _SO)
    return _SO


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO):
        build()
    lib = ctypes.CDLL(_SO)
    P = ctypes.c_void_p
    i32, i64, u64 = ctypes.c_int, ctypes.c_int64, ctypes.c_uint64
    lib.orc_sigmoid32.argtypes = [ctypes.c_float]
    lib.orc_sigmoid32.restype = ctypes.c_float
    lib.orc_sigmoid32_array.argtypes = [P, P, i64]
    lib.orc_sigmoid32_scan.argtypes = [u64, u64, u64, i32, P]
    lib.orc_sigmoid32_compare.argtypes = [u64, u64, P, i32, P]
    lib.orc_logits.argtypes = [i32, i32, i32, P, i32, P, P, i32]
    lib.orc_select.argtypes = [i32, i32, i32, i32, i32, ctypes.c_float, P, P, P, P, P]
    lib.orc_select.restype = i32
    lib.orc_route_intervals.argtypes = [i32, i32, i32, i32, i32, P, ctypes.c_double,
                                        ctypes.c_double, P, P, P, P, P, P, P]
    lib.orc_route_intervals.restype = i32
    lib.orc_permute.argtypes = [i32, i32, i32, P, P, P, P, P]
    lib.orc_experts_path_a.argtypes = [P, P, i32, P, P, P, i32, P, i32]
    lib.orc_experts_path_b.argtypes = [P, i32, P, i32, P, P, P, i32]
    lib.orc_rmsnorm.argtypes = [i32, i32, P, i32, ctypes.c_double, P]
    lib.orc_track.argtypes = [i32, i32, i32, P, P]
    lib.orc_expert_stats.argtypes = [i32, i32, i32, P, P, P]
    lib.orc_bias_update.argtypes = [i32, P, P, P, ctypes.c_double]
    lib.orc_aux_loss.argtypes = [i32, i32, P, P, P, P, P]
    d = ctypes.c_double
    lib.orc_backward_tokens.argtypes = [P, i32, i32, P, i32, P, i32, P, P, d, P, P, i32,
                                        P, P, P, P, i32]
    lib.orc_backward_expert_weights.argtypes = [P, i32, i32, P, i32, P, P, d, P, i32, P, P, P,
                                                i32]
    lib.orc_router_weight_grad.argtypes = [i32, i32, i32, P, i32, P, P]
    lib.orc_logits_any.argtypes = [i32, i32, i32, P, i32, P, i32, P]
    _lib = lib
    return lib


class _Experts(ctypes.Structure):
    _fields_ = [
        ("H", ctypes.c_int), ("I", ctypes.c_int), ("I_shared", ctypes.c_int),
        ("E", ctypes.c_int), ("K", ctypes.c_int), ("wdt", ctypes.c_int),
        ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
        ("ws_gate", ctypes.c_void_p), ("ws_up", ctypes.c_void_p), ("ws_down", ctypes.c_void_p),
    ]


def default_threads() -> int:
    n = int(os.environ.get("ORACLE_THREADS", "0"))
    if n > 0:
        return n
    return max(1, min(16, os.cpu_count() or 1))


def _ptr(a):
    return None if a is None else a.ctypes.data


def _act(a: np.ndarray):
    """(contiguous array, dtype code) for an fp32 or bf16-bits array."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    if a.dtype == np.float64:
        return a, F64
    raise TypeError(f"expected float32 or uint16 (bf16 bits), got {a.dtype}")


# --------------------------------------------------------------------------- sigma32

def sigmoid32(z) -> np.ndarray:
    z = np.ascontiguousarray(np.asarray(z, dtype=np.float32))
    out = np.empty_like(z)
    _load().orc_sigmoid32_array(_ptr(z), _ptr(out), z.size)
    return out


def sigmoid32_compare(start: int, other: np.ndarray, nthreads: int | None = None):
    """(mismatches, first mismatching index or -1) of sigma32 over the fp32 bit
    patterns start .. start + len(other) - 1 against ``other`` (another
    implementation's results for those patterns; NaN matches any NaN)."""
    other = np.ascontiguousarray(other, dtype=np.float32)
    out = np.zeros(2, dtype=np.int64)
    _load().orc_sigmoid32_compare(start, other.size, _ptr(other), nthreads or default_threads(),
                                  _ptr(out))
    return int(out[0]), int(out[1])


def sigmoid32_scan(start: int, stop: int, stride: int, nthreads: int | None = None):
    """(checked, not correctly rounded, more than 1 ulp off, non-monotone)."""
    out = np.zeros(4, dtype=np.int64)
    _load().orc_sigmoid32_scan(start, stop, stride, nthreads or default_threads(), _ptr(out))
    return tuple(int(v) for v in out)


# --------------------------------------------------------------------------- routing

def logits(x: np.ndarray, w_router: np.ndarray, nthreads: int | None = None) -> np.ndarray:
    """R1: fp64 router logits [T, E]."""
    x, xdt = _act(x)
    w = np.ascontiguousarray(w_router, dtype=np.float32)
    T, H = x.shape
    E = w.shape[0]
    assert w.shape[1] == H
    out = np.empty((T, E), dtype=np.float64)
    _load().orc_logits(T, H, E, _ptr(x), xdt, _ptr(w), _ptr(out), nthreads or default_threads())
    return out


def select(lam: np.ndarray, bias, n_group: int, topk_group: int, top_k: int,
           scale: float):
    """R2..R8 from fp32 logits.  Returns (idx int32 [T,K], w fp32 [T,K], flag uint8 [T])."""
    lam = np.ascontiguousarray(lam, dtype=np.float32)
    T, E = lam.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    idx = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float32)
    flag = np.empty(T, dtype=np.uint8)
    rc = _load().orc_select(T, E, n_group, topk_group, top_k, scale, _ptr(lam), _ptr(b),
                            _ptr(idx), _ptr(w), _ptr(flag))
    if rc < 0:
        raise ValueError("invalid routing shape")
    return idx, w, flag


def route(x, w_router, bias, n_group, topk_group, top_k, scale, nthreads=None):
    """Own-mode routing: lam = RN32(fp64 logits).  Returns (idx, w, flag, l64)."""
    l64 = logits(x, w_router, nthreads)
    idx, w, flag = select(l64.astype(np.float32), bias, n_group, topk_group, top_k, scale)
    return idx, w, flag, l64


def route_intervals(l64: np.ndarray, tau: float, bias, n_group, topk_group, top_k,
                    idx_ref: np.ndarray, want_bounds: bool = False, tau_rel: float = 0.0):
    """Decidedness of each token's selection when every fp32 logit may lie
    anywhere within tau + tau_rel*|l| of the fp64 logit l."""
    l64 = np.ascontiguousarray(l64, dtype=np.float64)
    T, E = l64.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    ref = np.ascontiguousarray(idx_ref, dtype=np.int32)
    dec = np.empty(T, dtype=np.uint8)
    bounds = None
    if want_bounds:
        bounds = dict(sb_lo=np.empty((T, E), np.float32), sb_hi=np.empty((T, E), np.float32),
                      gs_lo=np.empty((T, n_group), np.float32),
                      gs_hi=np.empty((T, n_group), np.float32))
    g = (lambda k: _ptr(bounds[k]) if bounds else None)
    rc = _load().orc_route_intervals(T, E, n_group, topk_group, top_k, _ptr(l64), tau, tau_rel,
                                     _ptr(b),
                                     _ptr(ref), _ptr(dec), g("sb_lo"), g("sb_hi"), g("gs_lo"),
                                     g("gs_hi"))
    if rc < 0:
        raise ValueError("invalid routing shape")
    return dec, bounds


def permute(idx: np.ndarray, E: int):
    """a5: (counts [E], offsets [E+1], sorted_pair [P], pair_slot [P]) int32."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, K = idx.shape
    P = T * K
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sp = np.empty(max(P, 1), np.int32)
    ps = np.empty(max(P, 1), np.int32)
    _load().orc_permute(T, K, E, _ptr(idx), _ptr(counts), _ptr(offsets), _ptr(sp), _ptr(ps))
    return counts, offsets, sp[:P], ps[:P]


# --------------------------------------------------------------------------- experts

def _experts_struct(H, K, w_gate, w_up, w_down, ws_gate, ws_up, ws_down):
    wg, wdt = _act(w_gate)
    wu, wdt2 = _act(w_up)
    wd, wdt3 = _act(w_down)
    assert wdt == wdt2 == wdt3
    E, I, H2 = wg.shape
    assert H2 == H and wu.shape == wg.shape and wd.shape == wg.shape
    keep = [wg, wu, wd]
    Is = 0
    sg = su = sd = None
    if ws_gate is not None:
        sg, d1 = _act(ws_gate)
        su, d2 = _act(ws_up)
        sd, d3 = _act(ws_down)
        assert d1 == d2 == d3 == wdt
        Is = sg.shape[0]
        assert sg.shape == (Is, H) and su.shape == (Is, H) and sd.shape == (Is, H)
        keep += [sg, su, sd]
    st = _Experts(H, I, Is, E, K, wdt, _ptr(wg), _ptr(wu), _ptr(wd), _ptr(sg), _ptr(su),
                  _ptr(sd))
    return st, keep


def experts(x, idx, w, w_gate, w_up, w_down, ws_gate=None, ws_up=None, ws_down=None,
            tokens=None, path: str = "A", nthreads=None) -> np.ndarray:
    """a6..a8: y = shared(x) + sum_j w_j * expert_{idx_j}(x), fp64.

    Path "A" loops tokens then their K experts (optionally only ``tokens``);
    path "B" buckets pairs by expert first and always returns all T rows."""
    x, xdt = _act(x)
    T, H = x.shape
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    K = idx.shape[1]
    st, keep = _experts_struct(H, K, w_gate, w_up, w_down, ws_gate, ws_up, ws_down)
    nt = nthreads or default_threads()
    if path == "A":
        tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
        n = T if tok is None else tok.size
        y = np.empty((n, H), np.float64)
        _load().orc_experts_path_a(ctypes.byref(st), _ptr(x), xdt, _ptr(idx), _ptr(w), _ptr(tok),
                                   n, _ptr(y), nt)
    elif path == "B":
        assert tokens is None
        y = np.empty((T, H), np.float64)
        _load().orc_experts_path_b(ctypes.byref(st), T, _ptr(x), xdt, _ptr(idx), _ptr(w),
                                   _ptr(y), nt)
    else:
        raise ValueError(path)
    del keep
    return y


def layer(x, w_router, bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, *, n_group,
          topk_group, top_k, scale, tokens=None, nthreads=None):
    """Whole layer in own mode.  Returns dict(idx, w, flag, l64, y) where y holds
    the rows ``tokens`` (all rows when None)."""
    idx, w, flag, l64 = route(x, w_router, bias, n_group, topk_group, top_k, scale, nthreads)
    y = experts(x, idx, w, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, tokens=tokens,
                path="A", nthreads=nthreads)
    return dict(idx=idx, w=w, flag=flag, l64=l64, y=y)


def rmsnorm(x, eps: float = 1e-6) -> np.ndarray:
    x, xdt = _act(x)
    T, H = x.shape
    r = np.empty((T, H), np.float64)
    _load().orc_rmsnorm(T, H, _ptr(x), xdt, eps, _ptr(r))
    return r


# --------------------------------------------------------------------------- dtype helpers

def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (nearest, ties to even) in one step and return
    the bit patterns.  Used by the layer-stack reference for its bf16 storage
    of activations.  Values below the bf16 normal range are flushed to zero."""
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)                       # a = m * 2^e, 0.5 <= |m| < 1
    q = np.rint(m * 256.0) / 256.0           # keep 8 significant bits, RNE
    r = np.ldexp(q, e).astype(np.float32)    # exact: 8-bit significand
    r[np.abs(r) < np.float32(2.0 ** -126)] = 0.0
    out = (r.view(np.uint32) >> 16).astype(np.uint16)
    out[np.isnan(a)] = 0x7FC0
    return out


# --------------------------------------------------------------------------- load balancing

NSTAT = 8
STAT_NAMES = ("hits", "max_load", "min_load", "cv", "idle", "hottest", "coldest",
              "max_group_load")


def track(idx: np.ndarray, E: int, tracking: np.ndarray | None = None) -> np.ndarray:
    """tracking[e] += hits of expert e in idx [T, K] (int64 [E], updated in place)."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, K = idx.shape
    if tracking is None:
        tracking = np.zeros(E, np.int64)
    assert tracking.dtype == np.int64 and tracking.flags.c_contiguous and tracking.size == E
    _load().orc_track(T, K, E, _ptr(idx), _ptr(tracking))
    return tracking


def expert_stats(tracking: np.ndarray, n_group: int):
    """(load fp32 [L, E], summary fp64 [L, NSTAT]) from tracked hits [L, E]."""
    tr = np.ascontiguousarray(np.atleast_2d(tracking), dtype=np.int64)
    L, E = tr.shape
    load = np.empty((L, E), np.float32)
    summ = np.empty((L, NSTAT), np.float64)
    _load().orc_expert_stats(L, E, n_group, _ptr(tr), _ptr(load), _ptr(summ))
    return load, summ


def bias_update(counts: np.ndarray, bias: np.ndarray | None, rate: float) -> np.ndarray:
    """The expert-bias update from one routing's counts; returns the new bias (fp32)."""
    c = np.ascontiguousarray(counts, dtype=np.int32)
    E = c.size
    b = np.zeros(E, np.float32) if bias is None else np.ascontiguousarray(bias, np.float32)
    out = np.empty(E, np.float32)
    _load().orc_bias_update(E, _ptr(c), _ptr(b), _ptr(out), float(rate))
    return out


def aux_loss(lam: np.ndarray, counts: np.ndarray):
    """(f fp64 [E], P fp64 [E], loss float) from fp32 logits [T, E] and counts [E]."""
    lam = np.ascontiguousarray(lam, dtype=np.float32)
    T, E = lam.shape
    if T < 1:
        raise ValueError("the auxiliary loss needs at least one token")
    c = np.ascontiguousarray(counts, dtype=np.int32)
    assert c.size == E
    f = np.empty(E, np.float64)
    P = np.empty(E, np.float64)
    loss = np.empty(1, np.float64)
    _load().orc_aux_loss(T, E, _ptr(lam), _ptr(c), _ptr(f), _ptr(P), _ptr(loss))
    return f, P, float(loss[0])


# --------------------------------------------------------------------------- backward

def logits_any(x, w_router) -> np.ndarray:
    """fp64 router logits from x and W_r of any dtype (fp32, bf16 bits, fp64)."""
    x, xdt = _act(x)
    wr, rdt = _act(w_router)
    T, H = x.shape
    E = wr.shape[0]
    lam = np.empty((T, E), np.float64)
    _load().orc_logits_any(T, H, E, _ptr(x), xdt, _ptr(wr), rdt, _ptr(lam))
    return lam


def backward_tokens(x, w_router, lam, idx, scale, dy, w_gate, w_up, w_down, ws_gate=None,
                    ws_up=None, ws_down=None, tokens=None, want_y=False, nthreads=None):
    """Per-token backward for a fixed routing: dict(dx, dweight, dlogit[, y])
    for the rows ``tokens`` (all rows when None).  fp64, exact sigmoid."""
    x, xdt = _act(x)
    wr, rdt = _act(w_router)
    T, H = x.shape
    E = wr.shape[0]
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    K = idx.shape[1]
    lam = np.ascontiguousarray(lam, dtype=np.float64)
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    assert lam.shape == (T, E) and dy.shape == (T, H)
    st, keep = _experts_struct(H, K, w_gate, w_up, w_down, ws_gate, ws_up, ws_down)
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    n = T if tok is None else tok.size
    dx = np.empty((n, H), np.float64)
    dw = np.empty((n, K), np.float64)
    dl = np.empty((n, E), np.float64)
    y = np.empty((n, H), np.float64) if want_y else None
    _load().orc_backward_tokens(ctypes.byref(st), T, E, _ptr(x), xdt, _ptr(wr), rdt, _ptr(lam),
                                _ptr(idx), float(scale), _ptr(dy), _ptr(tok), n, _ptr(dx),
                                _ptr(dw), _ptr(dl), _ptr(y), nthreads or default_threads())
    del keep
    out = dict(dx=dx, dweight=dw, dlogit=dl)
    if want_y:
        out["y"] = y
    return out


def backward_expert_weights(x, lam, idx, scale, dy, e, w_gate, w_up, w_down, ws_gate=None,
                            ws_up=None, ws_down=None, nthreads=None):
    """(dW_gate, dW_up, dW_down) of expert e ([I][H] each; e == E: the shared
    expert, [I_shared][H]) for a fixed routing, fp64."""
    x, xdt = _act(x)
    T, H = x.shape
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    K = idx.shape[1]
    lam = np.ascontiguousarray(lam, dtype=np.float64)
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    st, keep = _experts_struct(H, K, w_gate, w_up, w_down, ws_gate, ws_up, ws_down)
    E = st.E
    I = st.I_shared if e >= E else st.I
    assert I > 0
    out = [np.empty((I, H), np.float64) for _ in range(3)]
    _load().orc_backward_expert_weights(ctypes.byref(st), T, E, _ptr(x), xdt, _ptr(lam),
                                        _ptr(idx), float(scale), _ptr(dy), int(e),
                                        *[_ptr(o) for o in out], nthreads or default_threads())
    del keep
    return tuple(out)


def router_weight_grad(x, dlogit) -> np.ndarray:
    """dW_r [E][H] = dlogit^T x, fp64, summed over tokens in order."""
    x, xdt = _act(x)
    T, H = x.shape
    dl = np.ascontiguousarray(dlogit, dtype=np.float64)
    E = dl.shape[1]
    out = np.empty((E, H), np.float64)
    _load().orc_router_weight_grad(T, E, H, _ptr(x), xdt, _ptr(dl), _ptr(out))
    return out
