"""GPU parity of the HIP path (called through the C ABI) against the oracle.

Each case prints what it runs before the GPU step (so a failing run names
its case).  Bars: indices, counts and permutations bit-exact; fp32 layers
rel-L2 <= 1e-5, bf16 layers rel-L2 <= 1e-2 (per row <= 2e-2); routing on
random inputs: every token bit-exact (indices in order, weights, counts)
against the oracle's selection from the GPU's fp32 logits, the logits within
a forward-error band of the oracle's fp64 logits, and bit-exact against the
oracle's own logits on every token whose choice is unique within that band
(see gpu_helpers.check_routing_random).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from group_limited_top_amd import synth

from gpu_helpers import (DEV, L, TAU, TAU_REL, check_routing_random, gpu_layer, make_layer, nb,
                         oracle_weights, printable, rel_l2, row_rel, to_f64)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "routing_hand_examples.json")


def say(*a):
    print("[gpu-case]", *a, flush=True)


# --------------------------------------------------------------------------- sigma32

def test_sigmoid32_bit_exact_sampled():
    """The device sigma32 equals the oracle's on every 251st fp32 bit pattern
    and on dense runs around the values routing compares."""
    say("sigmoid32 sampled")
    bits = np.arange(0, 2 ** 32, 251, dtype=np.uint64).astype(np.uint32)
    dense = [np.arange(b, b + 2 ** 20, dtype=np.uint32) for b in
             (0x3F000000, 0xBF000000, 0x40000000, 0xC0000000, 0x42B00000, 0xC2B00000, 0xC2D00000)]
    z = np.concatenate([bits] + dense).view(np.float32)
    ref = oracle.sigmoid32(z)
    zt = torch.from_numpy(z).to(DEV)
    st = torch.empty_like(zt)
    L().moe_sigmoid32(zt, st)
    torch.cuda.synchronize()
    got = st.cpu().numpy()
    same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), f"{(~same).sum()} mismatches, first at z={z[~same][:4]}"


SIG_CHUNK = 1 << 28


@pytest.mark.parametrize("chunk", range(16))
def test_sigmoid32_exhaustive(chunk):
    """Every fp32 bit pattern, in 16 chunks of 2^28: the device sigma32 equals
    the oracle's bit for bit (NaN inputs: NaN on both sides)."""
    start = chunk * SIG_CHUNK
    say("sigmoid32 exhaustive, patterns", hex(start), "..", hex(start + SIG_CHUNK - 1))
    # the chunk's bit patterns as int32 (two's complement for patterns >= 2^31)
    off = start if start < 2 ** 31 else start - 2 ** 32
    bits = torch.arange(SIG_CHUNK, dtype=torch.int32, device=DEV) + off
    z = bits.view(torch.float32)
    s = torch.empty_like(z)
    L().moe_sigmoid32(z, s)
    torch.cuda.synchronize()
    del bits
    got = s.cpu().numpy()
    del s
    n_bad, first = oracle.sigmoid32_compare(start, got)
    assert n_bad == 0, f"{n_bad} mismatches, first at pattern {hex(start + first)}"


# --------------------------------------------------------------------------- routing, exact logits

def _route_exact(lam, bias, n_group, topk_group, top_k, scale, dtype="bf16"):
    """Route through moe_route with one-hot x, so that every fp32 logit equals
    lam exactly (a single non-zero product per dot product)."""
    T, E = lam.shape
    H = 256 * ((T + 255) // 256)
    x = torch.zeros(T, H, dtype=torch.float32)
    x[torch.arange(T), torch.arange(T)] = 1.0
    wr = torch.zeros(E, H, dtype=torch.float32)
    wr[:, :T] = torch.from_numpy(lam.T.copy())
    d = L().make_desc(T, H, E=E, n_group=n_group, topk_group=topk_group, top_k=top_k, I=64,
                      I_shared=0, scale=scale, dtype=dtype)
    xt = x.to(torch.bfloat16 if dtype == "bf16" else torch.float32).to(DEV)
    idx = torch.empty(T, top_k, dtype=torch.int32, device=DEV)
    w = torch.empty(T, top_k, dtype=torch.float32, device=DEV)
    lg = torch.empty(T, E, dtype=torch.float32, device=DEV)
    ws = L().alloc_workspace(d, DEV)
    b = None if bias is None else torch.from_numpy(bias).to(DEV)
    L().moe_route(d, xt, wr.to(DEV), b, lg, idx, w, ws)
    torch.cuda.synchronize()
    return lg.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("ex", _golden(), ids=lambda e: e["name"])
def test_route_hand_examples(ex, dtype):
    say("route hand example", ex["name"], dtype)
    E = ex["E"]
    if "logits" in ex:
        lam = np.array([ex["logits"]], np.float32)
    else:
        lam = np.full((1, E), ex["logits_default"], np.float32)
        for k, v in ex["logits_set"].items():
            lam[0, int(k)] = v
    bias = None if ex["bias"] is None else np.array(ex["bias"], np.float32)
    lg, idx, w = _route_exact(lam, bias, ex["n_group"], ex["topk_group"], ex["top_k"],
                              ex["scale"], dtype)
    np.testing.assert_array_equal(lg, lam)
    assert idx[0].tolist() == ex["expected_idx"]
    ri, rw, _ = oracle.select(lam, bias, ex["n_group"], ex["topk_group"], ex["top_k"], ex["scale"])
    np.testing.assert_array_equal(w.view(np.uint32), rw.view(np.uint32))


@pytest.mark.parametrize("kind", ["normal", "coarse", "wide", "underflow"])
@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_route_exact_logits_bit_exact(kind, with_bias, dtype):
    """Random logits (including heavy ties) fed exactly: indices AND weights
    bit-exact against the oracle's selection."""
    say("route exact logits", kind, with_bias, dtype)
    rng = np.random.default_rng(100 + 3 * with_bias + (dtype == "f32"))
    T, E = 300, 256
    if kind == "normal":
        lam = rng.normal(0, 1, (T, E)).astype(np.float32)
    elif kind == "coarse":
        lam = (rng.integers(-3, 4, (T, E)) * 0.5).astype(np.float32)
    elif kind == "wide":
        lam = rng.normal(0, 8, (T, E)).astype(np.float32)
    else:  # scores in the subnormal range and exact zeros
        lam = rng.uniform(-110, -80, (T, E)).astype(np.float32)
    bias = None
    if with_bias:
        bias = (rng.integers(-2, 3, E) * 0.125).astype(np.float32) if kind == "coarse" else \
            rng.normal(0, 0.05, E).astype(np.float32)
    lg, idx, w = _route_exact(lam, bias, 8, 4, 8, 2.5, dtype)
    np.testing.assert_array_equal(lg, lam)
    ri, rw, rf = oracle.select(lam, bias, 8, 4, 8, 2.5)
    assert not rf.any()
    np.testing.assert_array_equal(idx, ri)
    np.testing.assert_array_equal(w.view(np.uint32), rw.view(np.uint32))


@pytest.mark.parametrize("shape", [(16, 4, 2, 4), (64, 8, 3, 5), (512, 16, 4, 16), (96, 3, 2, 6)])
def test_route_exact_other_shapes(shape):
    E, G, KG, K = shape
    say("route exact other shape", shape)
    rng = np.random.default_rng(E + G)
    lam = (rng.integers(-3, 4, (200, E)) * 0.5).astype(np.float32)
    lg, idx, w = _route_exact(lam, None, G, KG, K, 2.5)
    ri, rw, _ = oracle.select(lam, None, G, KG, K, 2.5)
    np.testing.assert_array_equal(idx, ri)
    np.testing.assert_array_equal(w.view(np.uint32), rw.view(np.uint32))


def test_route_nonfinite_flag():
    """A NaN or Inf in x makes that token's logits non-finite (and only that
    token's): the status bit is raised, its indices stay in range, every other
    token is routed as usual."""
    say("route non-finite")
    Lb = L()
    rng = np.random.default_rng(7)
    T, E, H = 6, 256, 256
    lam = rng.normal(0, 1, (T, E)).astype(np.float32)
    x = torch.zeros(T, H)
    x[torch.arange(T), torch.arange(T)] = 1.0
    x[2, 100] = float("nan")
    x[4, 101] = float("inf")
    wr = torch.zeros(E, H)
    wr[:, :T] = torch.from_numpy(lam.T.copy())
    wr[:, 100:102] = 1.0  # inf * 1 stays infinite; other tokens multiply these by 0
    d = Lb.make_desc(T, H, I=64, I_shared=0, flags=Lb.MOE_F_CHECK_FINITE)
    idx = torch.empty(T, 8, dtype=torch.int32, device=DEV)
    w = torch.empty(T, 8, dtype=torch.float32, device=DEV)
    lg = torch.empty(T, E, dtype=torch.float32, device=DEV)
    ws = Lb.alloc_workspace(d, DEV)
    Lb.moe_route(d, x.to(torch.bfloat16).to(DEV), wr.to(DEV), None, lg, idx, w, ws)
    st = Lb.moe_status(ws)
    assert st & Lb.MOE_STATUS_NONFINITE
    assert Lb.moe_status(ws) == 0  # cleared by the read
    gl = lg.cpu().numpy()
    assert not np.isfinite(gl[2]).any() and not np.isfinite(gl[4]).any()
    ok = np.array([1, 1, 0, 1, 0, 1], bool)
    np.testing.assert_array_equal(gl[ok], lam[ok])
    gi = idx.cpu().numpy()
    assert gi.min() >= 0 and gi.max() < E
    assert gi[2].tolist() == list(range(8)) and (w.cpu().numpy()[[2, 4]] == 0).all()
    lam_nf = lam.copy()
    lam_nf[2, :] = np.nan
    lam_nf[4, :] = np.inf
    ri, rw, rf = oracle.select(lam_nf, None, 8, 4, 8, 2.5)
    assert rf.tolist() == [0, 0, 1, 0, 1, 0]
    np.testing.assert_array_equal(gi[ok], ri[ok])
    np.testing.assert_array_equal(w.cpu().numpy()[ok].view(np.uint32), rw[ok].view(np.uint32))


# --------------------------------------------------------------------------- routing, random inputs

@pytest.mark.parametrize("name", ["full_t512", "full_t16k_bias"])
def test_route_random_full_size(name):
    shape = synth.WORKLOADS[name]
    say("route random", name)
    x, wr, b = synth.router_inputs(shape)
    d = L().desc_from_shape(shape, flags=L().MOE_F_WRITE_LOGITS)
    T, E = shape.T, shape.E
    idx = torch.empty(T, 8, dtype=torch.int32, device=DEV)
    w = torch.empty(T, 8, dtype=torch.float32, device=DEV)
    lg = torch.empty(T, E, dtype=torch.float32, device=DEV)
    ws = L().alloc_workspace(d, DEV)
    L().moe_route(d, x.to(DEV), wr.to(DEV), None if b is None else b.to(DEV), lg, idx, w, ws)
    torch.cuda.synchronize()
    l64 = oracle.logits(nb(x), wr.numpy())
    dev = {"expert_bias": None if b is None else b}
    stats = check_routing_random(d, {"expert_bias": None if b is None else b},
                                 {"logits": lg, "idx": idx, "w": w}, l64)
    say("route stats", name, printable(stats))
    assert stats["decided"] >= 0.9 * T


@pytest.mark.parametrize("T", [1025, 2999])
def test_route_random_ragged_large(T):
    """Token counts past the small-batch router path that end in a partial
    token tile (the large-batch logits kernel covers 256 tokens per block)."""
    shape = synth.small_shape(T, H=2048, I=64, I_shared=0, bias="normal", seed=900 + T)
    say("route random ragged", T)
    x, wr, b = synth.router_inputs(shape)
    d = L().desc_from_shape(shape, flags=L().MOE_F_WRITE_LOGITS)
    E = shape.E
    idx = torch.empty(T, 8, dtype=torch.int32, device=DEV)
    w = torch.empty(T, 8, dtype=torch.float32, device=DEV)
    lg = torch.empty(T, E, dtype=torch.float32, device=DEV)
    ws = L().alloc_workspace(d, DEV)
    L().moe_route(d, x.to(DEV), wr.to(DEV), b.to(DEV), lg, idx, w, ws)
    torch.cuda.synchronize()
    l64 = oracle.logits(nb(x), wr.numpy())
    stats = check_routing_random(d, {"expert_bias": b}, {"logits": lg, "idx": idx, "w": w}, l64)
    assert stats["decided"] >= 0.9 * T


@pytest.mark.parametrize("T,H,E,G,KG,K", [(37, 320, 96, 3, 2, 6), (256, 512, 256, 8, 4, 8),
                                            (9, 1088, 160, 5, 2, 8), (300, 64, 64, 4, 2, 4)])
def test_route_random_f32_shapes(T, H, E, G, KG, K):
    """fp32 activations: logits from random inputs within the band of the
    oracle's fp64 logits for token counts that end in a partial 8-token block,
    expert counts that end in a partial 32-expert block (E = 96, 160) and
    hidden sizes that end in a partial 512-float chunk (H = 320, 1088); the
    routing then as for the other random inputs."""
    say("route random f32", T, H, E, G, KG, K)
    shape = synth.small_shape(T, H=H, I=64, I_shared=0, E=E, n_group=G, topk_group=KG, top_k=K,
                              dtype="f32", bias="normal", seed=1300 + T)
    x, wr, b = synth.router_inputs(shape)
    d = L().desc_from_shape(shape, flags=L().MOE_F_WRITE_LOGITS)
    idx = torch.empty(T, K, dtype=torch.int32, device=DEV)
    w = torch.empty(T, K, dtype=torch.float32, device=DEV)
    lg = torch.empty(T, E, dtype=torch.float32, device=DEV)
    ws = L().alloc_workspace(d, DEV)
    L().moe_route(d, x.to(DEV), wr.to(DEV), b.to(DEV), lg, idx, w, ws)
    torch.cuda.synchronize()
    l64 = oracle.logits(nb(x), wr.numpy())
    stats = check_routing_random(d, {"expert_bias": b}, {"logits": lg, "idx": idx, "w": w}, l64)
    assert stats["decided"] >= 0.9 * T


# --------------------------------------------------------------------------- permute

@pytest.mark.parametrize("T,kind", [(1, "uniform"), (77, "uniform"), (512, "uniform"),
                                    (4096, "skew"), (3000, "one_expert"), (16384, "uniform")])
def test_permute_bit_exact(T, kind):
    say("permute", T, kind)
    Lb = L()
    rng = np.random.default_rng(T)
    E, K = 256, 8
    if kind == "uniform":
        idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    elif kind == "skew":
        idx = rng.zipf(1.3, (T, K)).astype(np.int64) % E
        idx = idx.astype(np.int32)
    else:
        idx = np.full((T, K), 37, np.int32)
    d = Lb.make_desc(T, 2048)
    it = torch.from_numpy(idx).to(DEV)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    sp = torch.empty(T * K, dtype=torch.int32, device=DEV)
    ps = torch.empty(T * K, dtype=torch.int32, device=DEV)
    tracking = torch.zeros(E, dtype=torch.int64, device=DEV)
    ws = Lb.alloc_workspace(d, DEV)
    for _ in range(2):
        Lb.moe_permute(d, it, counts, offsets, sp, ps, tracking, ws)
    torch.cuda.synchronize()
    c, o, s, p = oracle.permute(idx, E)
    np.testing.assert_array_equal(counts.cpu().numpy(), c)
    np.testing.assert_array_equal(offsets.cpu().numpy(), o)
    np.testing.assert_array_equal(sp.cpu().numpy(), s)
    np.testing.assert_array_equal(ps.cpu().numpy(), p)
    np.testing.assert_array_equal(tracking.cpu().numpy(), 2 * c.astype(np.int64))
    assert Lb.moe_status(ws) == 0


@pytest.mark.parametrize("T,E,n_group,kind", [(65536, 256, 8, "skew"), (20000, 192, 6, "uniform"),
                                              (40000, 512, 8, "uniform"),
                                              (2100, 384, 6, "uniform")])
def test_permute_bit_exact_chunked(T, E, n_group, kind):
    """The chunked path (more than 16384 pairs) at up to 256 chunks of up to
    2048 pairs, and expert counts that are not a power of two (the chunk scan
    splits each expert's chunks over 1024 / E-rounded-up threads)."""
    say("permute chunked", T, E, kind)
    Lb = L()
    rng = np.random.default_rng(T + E)
    K = 8
    if kind == "uniform":
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    else:
        idx = (rng.zipf(1.3, (T, K)).astype(np.int64) % E).astype(np.int32)
    d = Lb.make_desc(T, 2048, E=E, n_group=n_group)
    it = torch.from_numpy(idx).to(DEV)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    sp = torch.empty(T * K, dtype=torch.int32, device=DEV)
    ps = torch.empty(T * K, dtype=torch.int32, device=DEV)
    ws = Lb.alloc_workspace(d, DEV)
    Lb.moe_permute(d, it, counts, offsets, sp, ps, None, ws)
    torch.cuda.synchronize()
    c, o, s, p = oracle.permute(idx, E)
    np.testing.assert_array_equal(counts.cpu().numpy(), c)
    np.testing.assert_array_equal(offsets.cpu().numpy(), o)
    np.testing.assert_array_equal(sp.cpu().numpy(), s)
    np.testing.assert_array_equal(ps.cpu().numpy(), p)
    assert Lb.moe_status(ws) == 0


# --------------------------------------------------------------------------- experts

def _random_routing(rng, T, E, K):
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 0.6, (T, K)).astype(np.float32)
    return idx, w


def _gpu_experts(d, dev, idx, w):
    """moe_experts fed with the oracle's permutation of the given routing."""
    Lb = L()
    E = d.E
    c, o, s, p = oracle.permute(idx, E)
    y = torch.empty(d.T, d.H, dtype=dev["x"].dtype, device=DEV)
    ws = Lb.alloc_workspace(d, DEV)
    weights = {k: dev[k] for k in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")}
    Lb.moe_experts(d, dev["x"], torch.from_numpy(w).to(DEV), torch.from_numpy(o).to(DEV),
                   torch.from_numpy(s).to(DEV), torch.from_numpy(p).to(DEV), weights, y, ws)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("T,dtype,Is", [(100, "bf16", 64), (100, "bf16", 0), (37, "bf16", 128),
                                        (100, "f32", 64), (5, "f32", 0), (1, "bf16", 64)])
def test_experts_small(T, dtype, Is):
    say("experts small", T, dtype, Is)
    shape = synth.small_shape(T, H=256, I=64, I_shared=Is, dtype=dtype, seed=300 + T)
    dev = make_layer(shape)
    rng = np.random.default_rng(T)
    idx, w = _random_routing(rng, T, shape.E, shape.top_k)
    d = L().desc_from_shape(shape)
    y = _gpu_experts(d, dev, idx, w)
    ref = oracle.experts(nb(dev["x"]), idx, w, *oracle_weights(dev))
    got = to_f64(y)
    tol = 1e-2 if dtype == "bf16" else 1e-5
    assert rel_l2(got, ref) <= tol / 2
    assert row_rel(got, ref).max() <= tol


@pytest.mark.parametrize("T,H,I,Is,hot", [(300, 320, 192, 192, 0), (200, 512, 320, 64, 0),
                                           (150, 256, 64, 128, 70), (40, 1088, 128, 0, 40)])
def test_experts_f32_shapes(T, H, I, Is, hot):
    """fp32 expert kernels: odd counts of 64-feature slices (I = 192, 320),
    K chunks of 256 with a partial last one (H = 320, 1088),
    I chunks of 256 with a partial last one (I = 320), a shared expert of
    another width, and `hot` tokens all choosing expert 3 (several 32-row
    tiles of one expert, the last partial)."""
    say("experts f32", T, H, I, Is, hot)
    shape = synth.small_shape(T, H=H, I=I, I_shared=Is, dtype="f32", seed=700 + T)
    dev = make_layer(shape)
    rng = np.random.default_rng(T + H)
    idx, w = _random_routing(rng, T, shape.E, shape.top_k)
    for t in range(hot):
        if 3 not in idx[t]:
            idx[t, 0] = 3
    d = L().desc_from_shape(shape)
    y = _gpu_experts(d, dev, idx, w)
    ref = oracle.experts(nb(dev["x"]), idx, w, *oracle_weights(dev))
    got = to_f64(y)
    assert rel_l2(got, ref) <= 5e-6
    assert row_rel(got, ref).max() <= 1e-5


@pytest.mark.parametrize("T,H,I,Is,hot", [(300, 384, 192, 192, 0), (150, 256, 64, 64, 70),
                                           (1000, 512, 128, 0, 200), (33, 1024, 256, 256, 0)])
def test_experts_f32_stream_shapes(T, H, I, Is, hot):
    """fp32 weight-streaming path (H a multiple of 128, I of 64, the shared
    expert as wide as the routed ones): three gate/up slices (I = 192),
    one-stage down items (I = 64), three down column slices (H = 384), no
    shared expert, and `hot` tokens all choosing expert 3 (many 32-row
    tiles of one expert, the last partial)."""
    say("experts f32 stream", T, H, I, Is, hot)
    shape = synth.small_shape(T, H=H, I=I, I_shared=Is, dtype="f32", seed=720 + T)
    dev = make_layer(shape)
    rng = np.random.default_rng(T + 3 * H)
    idx, w = _random_routing(rng, T, shape.E, shape.top_k)
    for t in range(hot):
        if 3 not in idx[t]:
            idx[t, 0] = 3
    d = L().desc_from_shape(shape)
    assert L().moe_stage_kernel(d, "gate_up") == "k_gateup_stream_f32"
    assert L().moe_stage_kernel(d, "down") == "k_down_stream_f32"
    y = _gpu_experts(d, dev, idx, w)
    ref = oracle.experts(nb(dev["x"]), idx, w, *oracle_weights(dev))
    got = to_f64(y)
    assert rel_l2(got, ref) <= 5e-6
    assert row_rel(got, ref).max() <= 1e-5


@pytest.mark.parametrize("T,H,I,Is,hot", [(200, 1024, 640, 640, 0), (64, 512, 1024, 0, 0),
                                           (300, 2048, 512, 0, 120), (150, 768, 256, 256, 60),
                                           (90, 1280, 192, 192, 0)])
def test_experts_bf16_stream_shapes(T, H, I, Is, hot):
    """bf16 weight-streaming path at other widths: down items of 4 to 16
    stages (I = 256 .. 1024), 2 to 8 down column slices of 256 (H = 512 ..
    2048, 1280), no shared expert, a hot expert with several tiles, and
    I = 192 (the register-streaming down kernel next to the gate/up
    stream)."""
    say("experts bf16 stream", T, H, I, Is, hot)
    shape = synth.small_shape(T, H=H, I=I, I_shared=Is, dtype="bf16", seed=740 + T)
    dev = make_layer(shape)
    rng = np.random.default_rng(T + 5 * H)
    idx, w = _random_routing(rng, T, shape.E, shape.top_k)
    for t in range(hot):
        if 3 not in idx[t]:
            idx[t, 0] = 3
    d = L().desc_from_shape(shape)
    assert L().moe_stage_kernel(d, "gate_up") == "k_gateup_stream"
    assert L().moe_stage_kernel(d, "down") == ("k_down_stream" if I >= 256 else "k_down_bf16")
    y = _gpu_experts(d, dev, idx, w)
    ref = oracle.experts(nb(dev["x"]), idx, w, *oracle_weights(dev))
    got = to_f64(y)
    assert rel_l2(got, ref) <= 5e-3
    assert row_rel(got, ref).max() <= 1e-2


def test_experts_full_size_sampled_rows():
    """Full-size shapes (H 2048, I 512), uneven buckets including one expert
    with many rows: every row of a sample of tokens against the oracle."""
    shape = synth.WORKLOADS["full_t512"]
    say("experts full size sampled", shape.T)
    dev = make_layer(shape)
    rng = np.random.default_rng(5)
    idx, w = _random_routing(rng, shape.T, shape.E, shape.top_k)
    idx[:100, 0] = 5  # expert 5 gets >100 rows: several tiles
    for t in range(100):
        if 5 in idx[t, 1:]:
            idx[t, 1 + list(idx[t, 1:]).index(5)] = 6 if 6 not in idx[t] else 7
    d = L().desc_from_shape(shape)
    y = _gpu_experts(d, dev, idx, w)
    tok = np.array(sorted(set(rng.choice(shape.T, 48, replace=False).tolist()) | {0, 99, 511}),
                   np.int32)
    ref = oracle.experts(nb(dev["x"]), idx, w, *oracle_weights(dev), tokens=tok)
    got = to_f64(y)[tok]
    assert rel_l2(got, ref) <= 5e-3
    assert row_rel(got, ref).max() <= 1e-2


# --------------------------------------------------------------------------- whole layer

def test_layer_tiny_f32():
    shape = synth.WORKLOADS["tiny_f32"]
    say("layer", shape.name)
    dev = make_layer(shape)
    d = L().desc_from_shape(shape)
    gpu = gpu_layer(d, dev)
    out = oracle.layer(nb(dev["x"]), nb(dev["w_router"]), None, *oracle_weights(dev),
                       n_group=8, topk_group=4, top_k=8, scale=2.5)
    stats = check_routing_random(d, dev, gpu, out["l64"])
    say("routing", printable(stats))
    got = to_f64(gpu["y"])
    assert rel_l2(got, out["y"]) <= 1e-5
    # every row, for the routing the oracle derives from the GPU's logits
    ref = oracle.experts(nb(dev["x"]), stats["idx"], stats["w"], *oracle_weights(dev))
    assert rel_l2(got, ref) <= 1e-5
    assert row_rel(got, ref).max() <= 2e-5
    dec, _ = oracle.route_intervals(out["l64"], TAU, None, 8, 4, 8, out["idx"], tau_rel=TAU_REL)
    ok = (dec & 2) != 0
    assert row_rel(got[ok], out["y"][ok]).max() <= 1e-5


def test_layer_full_t512():
    shape = synth.WORKLOADS["full_t512"]
    say("layer", shape.name)
    dev = make_layer(shape)
    d = L().desc_from_shape(shape)
    tracking = torch.zeros(shape.E, dtype=torch.int64, device=DEV)
    gpu = gpu_layer(d, dev, tracking=tracking)
    out = oracle.layer(nb(dev["x"]), nb(dev["w_router"]), None, *oracle_weights(dev),
                       n_group=8, topk_group=4, top_k=8, scale=2.5)
    # routing: every token and the counts bit-exact given the GPU's logits
    stats = check_routing_random(d, dev, gpu, out["l64"])
    say("routing", printable(stats))
    got = to_f64(gpu["y"])
    # every row against the oracle's experts for that routing
    ref = oracle.experts(nb(dev["x"]), stats["idx"], stats["w"], *oracle_weights(dev))
    r = rel_l2(got, ref)
    say("rel_l2 all rows", r, "worst row", row_rel(got, ref).max())
    assert r <= 1e-2
    assert row_rel(got, ref).max() <= 2e-2
    # the oracle on its own (no GPU value in its input): the whole layer, and
    # each row whose routing is decided within the logit band
    assert rel_l2(got, out["y"]) <= 1e-2
    dec, _ = oracle.route_intervals(out["l64"], TAU, None, 8, 4, 8, out["idx"], tau_rel=TAU_REL)
    ok = (dec & 2) != 0
    assert row_rel(got[ok], out["y"][ok]).max() <= 2e-2
    gc = gpu["counts"].cpu().numpy()
    oc = np.bincount(out["idx"].reshape(-1), minlength=256)
    assert np.abs(gc - oc).sum() <= 2 * 8 * int((~ok).sum())
    np.testing.assert_array_equal(tracking.cpu().numpy(), gc)
    # determinism: a second call is bit-identical
    gpu2 = gpu_layer(d, dev, tracking=tracking)
    assert torch.equal(gpu["y"], gpu2["y"]) and torch.equal(gpu["idx"], gpu2["idx"])
    assert torch.equal(gpu["w"], gpu2["w"])
    np.testing.assert_array_equal(tracking.cpu().numpy(), 2 * gc)


def test_layer_token_independence():
    shape = synth.small_shape(64, H=256, I=64, I_shared=64, seed=9)
    say("layer token independence")
    dev = make_layer(shape)
    d = L().desc_from_shape(shape)
    a = gpu_layer(d, dev)
    dev2 = dict(dev)
    dev2["x"] = dev["x"].clone()
    dev2["x"][10] = -dev2["x"][10]
    b = gpu_layer(d, dev2)
    keep = torch.ones(64, dtype=torch.bool)
    keep[10] = False
    assert torch.equal(a["y"][keep.to(DEV)], b["y"][keep.to(DEV)])
    assert not torch.equal(a["y"][10], b["y"][10])


@pytest.mark.parametrize("T", [1, 3, 33, 200])
def test_layer_ragged_small(T):
    shape = synth.small_shape(T, H=512, I=128, I_shared=64, bias="none", seed=40 + T)
    say("layer ragged", T)
    dev = make_layer(shape)
    d = L().desc_from_shape(shape)
    gpu = gpu_layer(d, dev)
    out = oracle.layer(nb(dev["x"]), nb(dev["w_router"]), None, *oracle_weights(dev),
                       n_group=8, topk_group=4, top_k=8, scale=2.5)
    check_routing_random(d, dev, gpu, out["l64"])
    dec, _ = oracle.route_intervals(out["l64"], TAU, None, 8, 4, 8, out["idx"], tau_rel=TAU_REL)
    ok = (dec & 2) != 0
    got = to_f64(gpu["y"])
    assert row_rel(got[ok], out["y"][ok]).max() <= 2e-2


def test_layer_nonfinite_row_isolated():
    shape = synth.small_shape(16, H=256, I=64, I_shared=64, seed=11)
    say("layer non-finite row")
    Lb = L()
    dev = make_layer(shape)
    d = Lb.desc_from_shape(shape, flags=Lb.MOE_F_CHECK_FINITE)
    a = gpu_layer(d, dev)
    assert Lb.moe_status(a["ws"]) == 0
    dev2 = dict(dev)
    dev2["x"] = dev["x"].clone()
    dev2["x"][3, 7] = float("nan")
    b = gpu_layer(d, dev2)
    assert Lb.moe_status(b["ws"]) & Lb.MOE_STATUS_NONFINITE
    gi = b["idx"].cpu().numpy()
    assert gi.min() >= 0 and gi.max() < shape.E
    keep = torch.ones(16, dtype=torch.bool, device=DEV)
    keep[3] = False
    assert torch.equal(a["y"][keep], b["y"][keep])


def test_layer_t16k_bias_all_rows():
    """16384 tokens with a per-expert bias that changes most tokens' choice:
    routing and counts of every token bit-exact given the GPU's logits, and
    every output row against the oracle's experts for that routing (the
    400+-row buckets run the 256-row MFMA GEMM path)."""
    shape = synth.WORKLOADS["full_t16k_bias"]
    say("layer", shape.name)
    dev = make_layer(shape)
    d = L().desc_from_shape(shape)
    gpu = gpu_layer(d, dev)
    assert L().moe_stage_kernel(d, "gate_up") == "k_expert_gemm<0>"
    xb = nb(dev["x"])
    l64 = oracle.logits(xb, nb(dev["w_router"]))
    stats = check_routing_random(d, dev, gpu, l64)
    say("routing", printable(stats))
    bias = nb(dev["expert_bias"])
    # the bias changes most tokens' choice, the weights stay unbiased
    idx0, _, _ = oracle.select(l64.astype(np.float32), None, 8, 4, 8, 2.5)
    assert (np.sort(stats["idx"], 1) != np.sort(idx0, 1)).any(1).mean() > 0.5
    ref = oracle.experts(xb, stats["idx"], stats["w"], *oracle_weights(dev))
    got = to_f64(gpu["y"])
    r = rel_l2(got, ref)
    say("rel_l2 all rows", r, "worst row", row_rel(got, ref).max())
    assert r <= 1e-2
    assert row_rel(got, ref).max() <= 2e-2
    # the oracle on its own: rows whose routing is decided within the band
    idx, w, _ = oracle.select(l64.astype(np.float32), bias, 8, 4, 8, 2.5)
    dec, _ = oracle.route_intervals(l64, TAU, bias, 8, 4, 8, idx, tau_rel=TAU_REL)
    ok = np.nonzero(dec & 2)[0][::16].astype(np.int32)
    own = oracle.experts(xb, idx, w, *oracle_weights(dev), tokens=ok)
    assert row_rel(got[ok], own).max() <= 2e-2


# --------------------------------------------------------------------------- skewed layer

def test_layer_skew_t64k_every_8th_row():
    """65536 tokens with Zipf-skewed routing (one expert takes almost every
    token) and the bias of the oracle's first pass: routing and counts of
    every token bit-exact given the GPU's logits; output rows t = 0 mod 8
    against the oracle's experts for that routing."""
    shape = synth.WORKLOADS["skew_t64k"]
    say("layer", shape.name)
    bias = np.loadtxt(os.path.join(os.path.dirname(__file__), "golden",
                                   "skew_t64k_expert_bias.txt"), dtype=np.float32)
    dev = make_layer(shape, bias=torch.from_numpy(bias))
    d = L().desc_from_shape(shape)
    xb = nb(dev["x"])
    l64 = oracle.logits(xb, nb(dev["w_router"]))
    # the stored bias is the oracle's bias update (rate 0.1, from zero) of its
    # own unbiased routing counts
    idx0, _, _ = oracle.select(l64.astype(np.float32), None, 8, 4, 8, 2.5)
    c0 = np.bincount(idx0.reshape(-1), minlength=256).astype(np.int32)
    np.testing.assert_array_equal(oracle.bias_update(c0, None, 0.1), bias)
    gpu = gpu_layer(d, dev)
    stats = check_routing_random(d, dev, gpu, l64)
    say("routing", printable(stats))
    assert stats["decided"] >= 0.9 * shape.T
    gc = gpu["counts"].cpu().numpy()
    assert gc.max() > shape.T // 2  # still heavily skewed after the bias
    tok = np.arange(0, shape.T, 8, dtype=np.int32)
    ref = oracle.experts(xb, stats["idx"], stats["w"], *oracle_weights(dev), tokens=tok)
    got = to_f64(gpu["y"])[tok]
    r = rel_l2(got, ref)
    say("rel_l2 rows t = 0 mod 8", r, "worst row", row_rel(got, ref).max())
    assert r <= 1e-2
    assert row_rel(got, ref).max() <= 2e-2


# --------------------------------------------------------------------------- residual + RMSNorm

@pytest.mark.parametrize("dtype,H", [("bf16", 2048), ("bf16", 256), ("bf16", 6144),
                                     ("bf16", 40960), ("fp32", 512), ("fp32", 16384)])
def test_residual_rmsnorm(dtype, H):
    """x_out = RN(x + y) (bf16: at most a rare 1-ulp double-rounding
    difference from the fp32 add; fp32: exact) and r_out = RN(RMSNorm(x_out))
    within one ulp-scale of the fp64 oracle.  Widths cover one to sixteen
    16-byte chunks per thread, a partial last round, and rows too wide for
    registers (the two-pass kernel)."""
    say("residual rmsnorm", dtype, H)
    Lb = L()
    T = 37
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(5 + H)
    x = torch.randn(T, H, generator=g).to(tdt)
    y = (0.3 * torch.randn(T, H, generator=g)).to(tdt)
    d = Lb.make_desc(T, H, dtype=dtype)
    xo = torch.empty(T, H, dtype=tdt, device=DEV)
    ro = torch.empty_like(xo)
    Lb.moe_residual_rmsnorm(d, x.to(DEV), y.to(DEV), xo, ro, 1e-6)
    torch.cuda.synchronize()
    rtol = 2.0 ** -7 if dtype == "bf16" else 2e-6
    if dtype == "bf16":
        ref_x = oracle.f64_to_bf16_bits(x.double().numpy() + y.double().numpy())
        got_x = nb(xo)
        diff = got_x != ref_x
        assert diff.mean() <= 1e-4
        assert np.all(np.abs(got_x.astype(np.int32) - ref_x.astype(np.int32))[diff] <= 1)
        got_r = oracle.bf16_bits_to_f32(nb(ro)).astype(np.float64)
    else:
        got_x = xo.cpu().numpy()
        np.testing.assert_array_equal(got_x, x.numpy() + y.numpy())
        got_r = ro.cpu().numpy().astype(np.float64)
    ref_r = oracle.rmsnorm(got_x, 1e-6)
    assert np.all(np.abs(got_r - ref_r) <= rtol * np.abs(ref_r) + 1e-30)
    # in place, and without the residual
    x2 = x.to(DEV)
    Lb.moe_residual_rmsnorm(d, x2, None, x2, ro, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(x2.cpu(), x)
    got_r = (oracle.bf16_bits_to_f32(nb(ro)) if dtype == "bf16" else ro.cpu().numpy()).astype(np.float64)
    ref_r = oracle.rmsnorm(nb(x) if dtype == "bf16" else x.numpy(), 1e-6)
    assert np.all(np.abs(got_r - ref_r) <= rtol * np.abs(ref_r) + 1e-30)


# --------------------------------------------------------------------------- 19-layer stack

def test_stack19_t8k():
    """19 residual MoE layers on 8192 tokens, every layer checked at its own
    size (the 256-row MFMA GEMM path the stack runs, with its partial tiles).

    (a) The stack as moe_stack_forward runs it; the same stack is then run
        layer by layer through the same C-ABI calls, writing logits as well,
        and must reproduce (a)'s indices and counts bit for bit.
    (b) Teacher-forced per layer from the GPU's own layer input r_l (all 8192
        tokens): logits within the band of the oracle's fp64 logits of r_l;
        indices, weights and counts bit-exact against the oracle's selection
        from the GPU's logits; tracking == counts; output rows t = 0 mod 8
        against the oracle's experts (rel-L2 <= 1e-2); the residual + RMSNorm
        step against the oracle's from the GPU's x and y.
    (c) Oracle-fed rows through the full-size path: in each layer's batch,
        256 sampled rows are replaced by the free-running oracle's own layer
        input (data oracle -> GPU); those rows are checked like (b).
    (d) End to end on the 256 sampled tokens: the free-running oracle's final
        activations against the GPU stack's on the tokens whose routing
        agreed at every layer (routing is discontinuous: bf16 roundings make
        a share of tokens pick a different expert somewhere in 19 layers,
        after which the two trajectories are unrelated), bar sqrt(19)*1e-2/2
        (independent per-layer differences add up roughly as sqrt(L))."""
    shape = synth.WORKLOADS["stack19_t8k"]
    say("stack", shape.name)
    Lb = L()
    nl = shape.layers
    layers = []
    for l in range(nl):
        dv = make_layer(shape, layer=l)
        layers.append({k: dv[k] for k in ("w_router", "expert_bias", "w_gate", "w_up", "w_down",
                                          "ws_gate", "ws_up", "ws_down")})
    x0 = synth.router_inputs(shape, 0)[0].to(DEV)
    d = Lb.desc_from_shape(shape)
    ws = Lb.alloc_workspace(d, DEV)
    T, E, H = shape.T, shape.E, shape.H
    assert Lb.moe_stage_kernel(d, "gate_up") == "k_expert_gemm<0>"
    # (a)
    idx_out = torch.empty(nl, T, 8, dtype=torch.int32, device=DEV)
    counts_out = torch.empty(nl, E, dtype=torch.int32, device=DEV)
    tracking = torch.zeros(nl, E, dtype=torch.int64, device=DEV)
    x = x0.clone()
    Lb.moe_stack_forward(d, x, layers, ws, tracking=tracking, idx_out=idx_out,
                         counts_out=counts_out)
    torch.cuda.synchronize()
    gidx_stack = idx_out.cpu().numpy()
    np.testing.assert_array_equal(tracking.cpu().numpy(), counts_out.cpu().numpy().astype(np.int64))
    rng = np.random.default_rng(19)
    n_s = 256
    free = np.sort(rng.choice(T, n_s, replace=False)).astype(np.int32)
    free_t = torch.from_numpy(free).to(DEV).long()
    x_final = nb(x[free_t])
    every8 = np.arange(0, T, 8, dtype=np.int32)

    dl = Lb.desc_from_shape(shape)
    xg = x0.clone()
    r = torch.empty_like(xg)
    Lb.moe_residual_rmsnorm(dl, xg, None, xg, r, 1e-6)
    xo = nb(x0)[free]  # the free-running oracle's state on the sampled tokens
    agree = np.ones(n_s, bool)
    for l in range(nl):
        ow = oracle_weights(layers[l])
        wr = nb(layers[l]["w_router"])
        say("stack layer", l)
        # (b) teacher-forced from the GPU's own layer input
        rb = nb(r)
        gl = gpu_layer(dl, dict(layers[l], x=r), ws=ws)
        np.testing.assert_array_equal(gl["idx"].cpu().numpy(), gidx_stack[l])
        l64 = oracle.logits(rb, wr)
        st = check_routing_random(dl, layers[l], gl, l64)
        ref = oracle.experts(rb, st["idx"], st["w"], *ow, tokens=every8)
        got = to_f64(gl["y"])[every8]
        rl = rel_l2(got, ref)
        assert rl <= 1e-2, (l, rl)
        assert row_rel(got, ref).max() <= 2e-2, l
        x_prev = nb(xg)
        y_l = nb(gl["y"])
        Lb.moe_residual_rmsnorm(dl, xg, gl["y"], xg, r, 1e-6)
        torch.cuda.synchronize()
        ref_x = oracle.f64_to_bf16_bits(oracle.bf16_bits_to_f32(x_prev).astype(np.float64)
                                        + oracle.bf16_bits_to_f32(y_l).astype(np.float64))
        got_x = nb(xg)
        diff = got_x != ref_x
        assert diff.mean() <= 1e-4, l  # a rare 1-ulp double rounding (fp32 add, then bf16)
        assert np.all(np.abs(got_x.astype(np.int32) - ref_x.astype(np.int32))[diff] <= 1), l
        ref_r = oracle.rmsnorm(got_x[every8], 1e-6)
        got_r = oracle.bf16_bits_to_f32(nb(r)[every8]).astype(np.float64)
        assert np.all(np.abs(got_r - ref_r) <= 2.0 ** -7 * np.abs(ref_r) + 1e-30), l
        # (c) the free-running oracle's own layer input in the sampled rows
        ro = oracle.f64_to_bf16_bits(oracle.rmsnorm(xo, 1e-6))
        mix = torch.from_numpy(rb.view(np.int16).copy())
        mix[torch.from_numpy(free).long()] = torch.from_numpy(ro.view(np.int16))
        gm = gpu_layer(dl, dict(layers[l], x=mix.view(torch.bfloat16).to(DEV)), ws=ws)
        l64o = oracle.logits(ro, wr)
        sub = {k: (gm[k][free_t] if k in ("logits", "idx", "w", "y") else None)
               for k in ("logits", "idx", "w", "y")}
        dso = Lb.desc_from_shape(shape, T=n_s)
        sto = check_routing_random(dso, layers[l], sub, l64o)
        refo = oracle.experts(ro, sto["idx"], sto["w"], *ow)
        goto = to_f64(sub["y"])
        assert rel_l2(goto, refo) <= 1e-2, l
        assert row_rel(goto, refo).max() <= 2e-2, l
        # (d) the free-running oracle's own step
        idx_o, w_o, _ = oracle.select(l64o.astype(np.float32), None, 8, 4, 8, 2.5)
        y_o = oracle.experts(ro, idx_o, w_o, *ow)
        agree &= (np.sort(idx_o, 1) == np.sort(gidx_stack[l][free], 1)).all(1)
        yb = oracle.bf16_bits_to_f32(oracle.f64_to_bf16_bits(y_o)).astype(np.float64)
        xo = oracle.f64_to_bf16_bits(oracle.bf16_bits_to_f32(xo).astype(np.float64) + yb)
    # the step-by-step run ends where the stack did
    np.testing.assert_array_equal(nb(xg)[free], x_final)
    say("stack: sampled tokens with identical routing at all layers", int(agree.sum()), "/", n_s)
    assert agree.sum() >= 32  # 63 of 256 agreed when this bar was set
    got = oracle.bf16_bits_to_f32(x_final).astype(np.float64)
    ref = oracle.bf16_bits_to_f32(xo).astype(np.float64)
    r_end = rel_l2(got[agree], ref[agree])
    say("stack final rel_l2 on agreeing tokens", r_end)
    bar = math.sqrt(nl) * 1e-2 / 2
    assert r_end <= bar
    assert row_rel(got[agree], ref[agree]).max() <= 2 * bar
