"""GPU parity of the layer backward (moe_layer_backward, through the C ABI)
against the oracle's fp64 backward for the same fixed routing.

Data flows oracle -> GPU only: the routing (chosen experts) and the fp32
logits the GPU backward takes are the oracle's own (its routing of the
inputs, its fp64 logits rounded to fp32); GPU results are only compared.
Bar: relative L2 error <= 1e-2 per gradient tensor (bf16 operands, fp32
accumulation), the same bar as the bf16 forward; experts no token chose get
exactly zero weight gradients; results are bit-reproducible.
"""
import numpy as np
import pytest
import torch

import oracle
from group_limited_top_amd import synth

from gpu_helpers import DEV, L, make_layer, nb, oracle_weights, rel_l2, to_f64

pytestmark = pytest.mark.gpu
TOL = 1e-2


def say(*a):
    print("[gpu-case]", *a, flush=True)


def _routing(shape, dev):
    """The oracle's routing of the layer's inputs: idx, fp64 logits."""
    bias = None if dev["expert_bias"] is None else nb(dev["expert_bias"])
    idx, _, flag, l64 = oracle.route(nb(dev["x"]), nb(dev["w_router"]), bias, shape.n_group,
                                     shape.topk_group, shape.top_k, shape.scale)
    assert not flag.any()
    return idx, l64


def _dy(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape.T, shape.H, generator=g).to(torch.bfloat16)


def _gpu_backward(shape, dev, idx, l64, dy):
    d = L().desc_from_shape(shape)
    weights = {k: dev[k] for k in ("w_router", "expert_bias", "w_gate", "w_up", "w_down",
                                   "ws_gate", "ws_up", "ws_down")}
    out = L().moe_layer_backward(d, dev["x"], weights, torch.from_numpy(idx).to(DEV),
                                 torch.from_numpy(l64.astype(np.float32)).to(DEV), dy.to(DEV))
    torch.cuda.synchronize()
    return out


def _check_tokens(shape, dev, idx, l64, dy, gpu, tokens):
    ref = oracle.backward_tokens(nb(dev["x"]), nb(dev["w_router"]), l64, idx, shape.scale,
                                 dy.double().numpy(), *oracle_weights(dev), tokens=tokens)
    got = to_f64(gpu["dx"]) if tokens is None else to_f64(gpu["dx"])[tokens]
    r = rel_l2(got, ref["dx"])
    say("dx rel_l2", r)
    assert r <= TOL
    return ref


def _check_expert(shape, dev, idx, l64, dy, gpu, e):
    E = shape.E
    ref = oracle.backward_expert_weights(nb(dev["x"]), l64, idx, shape.scale, dy.double().numpy(),
                                         e, *oracle_weights(dev))
    names = ("dws_gate", "dws_up", "dws_down") if e >= E else ("dw_gate", "dw_up", "dw_down")
    for name, rv in zip(names, ref):
        gv = gpu[name] if e >= E else gpu[name][e]
        got = gv.double().cpu().numpy()
        if not np.any(rv):
            np.testing.assert_array_equal(got, 0.0)
            continue
        r = rel_l2(got, rv)
        say("expert", e, name, "rel_l2", r)
        assert r <= TOL, (e, name, r)


# (T, I_shared, extra shape): token counts below and above one router-gradient
# chunk (1024 tokens, ragged tails), no shared expert, E = 64 (a partial tile
# of 256 experts) and 512 (two tiles), I = 320 (64-wide column tiles)
@pytest.mark.parametrize("T,Is,kw", [
    (200, 64, {}), (77, 0, {}), (1, 64, {}), (33, 64, {}),
    (2500, 64, {}),
    (300, 0, dict(E=64, n_group=4, topk_group=2, top_k=6)),
    (1100, 64, dict(E=512, n_group=8, topk_group=4, top_k=16)),
    (150, 320, dict(I=320)),
])
def test_backward_small_all_gradients(T, Is, kw):
    kw = dict(kw)
    I = kw.pop("I", 64)
    shape = synth.small_shape(T, H=256, I=I, I_shared=Is, bias="normal", seed=500 + T, **kw)
    say("backward small", T, Is, I, kw)
    dev = make_layer(shape)
    idx, l64 = _routing(shape, dev)
    dy = _dy(shape, 7 + T)
    gpu = _gpu_backward(shape, dev, idx, l64, dy)
    ref = _check_tokens(shape, dev, idx, l64, dy, gpu, None)
    # the router weight gradient from the oracle's dlogit of every token
    dwr = oracle.router_weight_grad(nb(dev["x"]), ref["dlogit"])
    r = rel_l2(gpu["dw_router"].double().cpu().numpy(), dwr)
    say("dw_router rel_l2", r)
    assert r <= TOL
    counts = np.bincount(idx.ravel(), minlength=shape.E)
    hot = [int(np.argmax(counts)), int(np.argsort(counts)[len(counts) // 2])]
    cold = [int(e) for e in np.nonzero(counts == 0)[0][:1]]
    for e in hot + cold + ([shape.E] if Is else []):
        _check_expert(shape, dev, idx, l64, dy, gpu, e)
    # experts no token chose: exactly zero, all of them
    unused = counts == 0
    for name in ("dw_gate", "dw_up", "dw_down"):
        assert torch.count_nonzero(gpu[name][torch.from_numpy(unused).to(DEV)]) == 0


def test_backward_deterministic():
    shape = synth.small_shape(300, H=256, I=64, I_shared=64, bias="normal", seed=901)
    say("backward determinism")
    dev = make_layer(shape)
    idx, l64 = _routing(shape, dev)
    dy = _dy(shape, 3)
    a = _gpu_backward(shape, dev, idx, l64, dy)
    b = _gpu_backward(shape, dev, idx, l64, dy)
    for k, v in a.items():
        if v is not None:
            assert torch.equal(v, b[k]), k


def test_backward_full_size_sampled():
    """The full-size layer at 16384 tokens (with expert bias): dx on sampled
    tokens, the weight gradients of sampled experts."""
    shape = synth.WORKLOADS["full_t16k_bias"]
    say("backward full_t16k_bias")
    dev = make_layer(shape)
    idx, l64 = _routing(shape, dev)
    dy = _dy(shape, 11)
    gpu = _gpu_backward(shape, dev, idx, l64, dy)
    rng = np.random.default_rng(5)
    tok = np.sort(rng.choice(shape.T, 48, replace=False)).astype(np.int32)
    _check_tokens(shape, dev, idx, l64, dy, gpu, tok)
    counts = np.bincount(idx.ravel(), minlength=shape.E)
    for e in (int(np.argmax(counts)), int(np.argmin(counts)), 17):
        _check_expert(shape, dev, idx, l64, dy, gpu, e)
    # a router weight gradient row of an expert about 64 tokens chose (spread
    # over the token chunks): only the tokens that chose it contribute, so the
    # oracle's backward of those tokens alone gives the row exactly
    e = int(np.argmin(np.abs(counts - 64)))
    toks = np.nonzero((idx == e).any(axis=1))[0].astype(np.int32)
    say("router gradient row", e, "from", len(toks), "tokens")
    ref = oracle.backward_tokens(nb(dev["x"]), nb(dev["w_router"]), l64, idx, shape.scale,
                                 dy.double().numpy(), *oracle_weights(dev), tokens=toks)
    want = oracle.router_weight_grad(nb(dev["x"])[toks], ref["dlogit"])[e]
    r = rel_l2(gpu["dw_router"][e].double().cpu().numpy(), want)
    say("dw_router row rel_l2", r)
    assert r <= TOL


def _takes_expert_gemm(shape):
    """The backward runs its row products on the forward's expert GEMM
    (256-row tiles) when a routed expert averages at least 128 rows, the
    shared expert is as wide as the routed ones, and I is a multiple of 256
    and H of 256."""
    return (shape.T * shape.top_k // shape.E >= 128 and shape.I_shared == shape.I
            and shape.I % 256 == 0 and shape.H % 256 == 0)


# the expert-GEMM path: 256 experts at 128 rows each (the threshold), 64
# experts with I = 512 (two r slices, ragged tiles), a skew in which one
# expert owns every token (many row tiles of one expert), and 512 experts
# with top_k = 16 (the combine's router term over 16 pairs)
@pytest.mark.parametrize("T,H,I,kw,skew", [
    (4096, 512, 256, {}, False),
    (2304, 512, 512, dict(E=64, n_group=4, topk_group=2, top_k=6), False),
    (3000, 768, 256, dict(E=64, n_group=4, topk_group=2), True),
    (4100, 512, 256, dict(E=512, n_group=8, topk_group=4, top_k=16), False),
])
def test_backward_expert_gemm_path(T, H, I, kw, skew):
    shape = synth.small_shape(T, H=H, I=I, I_shared=I, bias="normal", seed=700 + T, **kw)
    assert _takes_expert_gemm(shape)
    say("backward expert-GEMM path", T, H, I, kw, "skew" if skew else "")
    dev = make_layer(shape)
    if skew:
        rng = np.random.default_rng(5)
        idx = np.empty((T, shape.top_k), np.int32)
        idx[:, 0] = 0
        for t in range(T):
            idx[t, 1:] = 1 + rng.choice(40, shape.top_k - 1, replace=False)
        l64 = oracle.logits_any(nb(dev["x"]), nb(dev["w_router"]))
    else:
        idx, l64 = _routing(shape, dev)
    dy = _dy(shape, 23 + T)
    gpu = _gpu_backward(shape, dev, idx, l64, dy)
    rng = np.random.default_rng(T)
    tok = np.sort(rng.choice(T, 64, replace=False)).astype(np.int32)
    tok[-1] = T - 1  # the last token: the shared expert's last, partial tile
    tok = np.unique(tok)
    ref = _check_tokens(shape, dev, idx, l64, dy, gpu, tok)
    counts = np.bincount(idx.ravel(), minlength=shape.E)
    for e in (int(np.argmax(counts)), int(np.argsort(counts)[len(counts) // 2]), shape.E):
        _check_expert(shape, dev, idx, l64, dy, gpu, e)
    # a router weight gradient row from the tokens that chose that expert
    e = int(np.argmin(np.abs(counts - 40))) if not skew else 3
    toks = np.nonzero((idx == e).any(axis=1))[0].astype(np.int32)
    ref = oracle.backward_tokens(nb(dev["x"]), nb(dev["w_router"]), l64, idx, shape.scale,
                                 dy.double().numpy(), *oracle_weights(dev), tokens=toks)
    want = oracle.router_weight_grad(nb(dev["x"])[toks], ref["dlogit"])[e]
    r = rel_l2(gpu["dw_router"][e].double().cpu().numpy(), want)
    say("dw_router row", e, "rel_l2", r)
    assert r <= TOL


def test_backward_expert_gemm_path_deterministic():
    shape = synth.small_shape(4096, H=512, I=256, I_shared=256, bias="normal", seed=931)
    assert _takes_expert_gemm(shape)
    say("backward expert-GEMM path determinism")
    dev = make_layer(shape)
    idx, l64 = _routing(shape, dev)
    dy = _dy(shape, 4)
    a = _gpu_backward(shape, dev, idx, l64, dy)
    b = _gpu_backward(shape, dev, idx, l64, dy)
    for k, v in a.items():
        if v is not None:
            assert torch.equal(v, b[k]), k


def test_backward_skewed_routing():
    """Every token picks expert 0 and seven of experts 1..32: expert 0's rows
    are all the tokens (many row tiles of one expert, long weight-gradient
    sums), experts past 32 get none.  Any routing is a valid point of the
    fixed-routing backward, so the choice is given, not computed."""
    T = 1500
    shape = synth.small_shape(T, H=256, I=64, I_shared=64, bias="normal", seed=77)
    say("backward skewed routing", T)
    dev = make_layer(shape)
    rng = np.random.default_rng(3)
    idx = np.empty((T, shape.top_k), np.int32)
    idx[:, 0] = 0
    for t in range(T):
        idx[t, 1:] = 1 + rng.choice(32, shape.top_k - 1, replace=False)
    l64 = oracle.logits_any(nb(dev["x"]), nb(dev["w_router"]))
    dy = _dy(shape, 19)
    gpu = _gpu_backward(shape, dev, idx, l64, dy)
    ref = _check_tokens(shape, dev, idx, l64, dy, gpu, None)
    dwr = oracle.router_weight_grad(nb(dev["x"]), ref["dlogit"])
    r = rel_l2(gpu["dw_router"].double().cpu().numpy(), dwr)
    say("dw_router rel_l2", r)
    assert r <= TOL
    for e in (0, 5, 32, 100, shape.E):
        _check_expert(shape, dev, idx, l64, dy, gpu, e)
    assert torch.count_nonzero(gpu["dw_gate"][33:]) == 0
    assert torch.count_nonzero(gpu["dw_down"][33:]) == 0
