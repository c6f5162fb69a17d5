"""Pins of the oracle's expert math and combine.

Rule ([InternLumina-U2中256个专家的路由秘密…] §四, §五): each expert is a SwiGLU
feed-forward network down(silu(gate x) * up x) over stacked [E][I][H] weights
(down used as h @ W_down[e]), the shared expert has the same form and is added
with no weight, and the layer output is the shared output plus the
weight-scaled sum of the K routed outputs.  The page's two eager paths (a loop
per expert during training, bucketing by expert at inference) must agree.

Pins: numpy matmul evaluation (an independent route), path A == path B
bit-for-bit, identical-experts closed form, the single-expert textbook MLP,
zero routing weights leaving only the shared expert, and token independence.
"""
import numpy as np
import pytest

import oracle


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _mlp_np(x, wg, wu, wd):
    """Textbook SwiGLU with numpy matmuls: x [n,H], w* [I,H] -> [n,H]."""
    a = _silu(x @ wg.T) * (x @ wu.T)
    return a @ wd


def _make(rng, T, H, I, Is, E, K, dt="f32"):
    x = rng.normal(0, 1, (T, H)).astype(np.float32)
    wg = rng.normal(0, 0.05, (E, I, H)).astype(np.float32)
    wu = rng.normal(0, 0.05, (E, I, H)).astype(np.float32)
    wd = rng.normal(0, 0.05, (E, I, H)).astype(np.float32)
    sg = rng.normal(0, 0.05, (Is, H)).astype(np.float32) if Is else None
    su = rng.normal(0, 0.05, (Is, H)).astype(np.float32) if Is else None
    sd = rng.normal(0, 0.05, (Is, H)).astype(np.float32) if Is else None
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.05, 0.6, (T, K)).astype(np.float32)
    if dt == "bf16":
        conv = lambda a: None if a is None else oracle.f64_to_bf16_bits(a)
        return [conv(v) if i not in (7, 8) else v for i, v in
                enumerate([x, wg, wu, wd, sg, su, sd, idx, w])]
    return [x, wg, wu, wd, sg, su, sd, idx, w]


def _f64(a):
    if a is None:
        return None
    return (oracle.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_matches_numpy_matmul(dt):
    rng = np.random.default_rng(1)
    T, H, I, Is, E, K = 9, 96, 40, 24, 12, 4
    x, wg, wu, wd, sg, su, sd, idx, w = _make(rng, T, H, I, Is, E, K, dt)
    y = oracle.experts(x, idx, w, wg, wu, wd, sg, su, sd)
    X, WG, WU, WD = _f64(x), _f64(wg), _f64(wu), _f64(wd)
    ref = _mlp_np(X, _f64(sg), _f64(su), _f64(sd))
    for t in range(T):
        for j in range(K):
            e = idx[t, j]
            ref[t] += float(w[t, j]) * _mlp_np(X[t:t + 1], WG[e], WU[e], WD[e])[0]
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12)


def test_down_projection_orientation_matters():
    """[I][H] down weights used as h @ W_down: a transposed reading differs."""
    rng = np.random.default_rng(2)
    T, H, I, E, K = 4, 32, 32, 3, 2
    x, wg, wu, wd, _, _, _, idx, w = _make(rng, T, H, I, 0, E, K)
    y = oracle.experts(x, idx, w, wg, wu, wd)
    wdt = np.ascontiguousarray(np.transpose(wd, (0, 2, 1)))
    y2 = oracle.experts(x, idx, w, wg, wu, wdt)
    assert np.abs(y - y2).max() > 1e-3


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_path_a_equals_path_b(dt):
    rng = np.random.default_rng(3)
    T, H, I, Is, E, K = 40, 64, 32, 16, 16, 5
    x, wg, wu, wd, sg, su, sd, idx, w = _make(rng, T, H, I, Is, E, K, dt)
    idx[:20] = idx[0]  # a hot expert set: uneven buckets
    a = oracle.experts(x, idx, w, wg, wu, wd, sg, su, sd, path="A")
    b = oracle.experts(x, idx, w, wg, wu, wd, sg, su, sd, path="B")
    np.testing.assert_array_equal(a, b)
    # path A on a token subset returns exactly those rows
    tok = np.array([39, 0, 17], np.int32)
    np.testing.assert_array_equal(
        oracle.experts(x, idx, w, wg, wu, wd, sg, su, sd, tokens=tok), a[tok])


def test_identical_experts_closed_form():
    """All experts equal: y = (sum_j w_j) * MLP(x) + shared(x), whatever the routing."""
    rng = np.random.default_rng(4)
    T, H, I, Is, E, K = 12, 48, 24, 16, 10, 4
    x, wg, wu, wd, sg, su, sd, idx, w = _make(rng, T, H, I, Is, E, K)
    wg[:] = wg[0]
    wu[:] = wu[0]
    wd[:] = wd[0]
    y = oracle.experts(x, idx, w, wg, wu, wd, sg, su, sd)
    X = x.astype(np.float64)
    ref = (w.astype(np.float64).sum(1, keepdims=True) *
           _mlp_np(X, wg[0].astype(np.float64), wu[0].astype(np.float64), wd[0].astype(np.float64))
           + _mlp_np(X, sg.astype(np.float64), su.astype(np.float64), sd.astype(np.float64)))
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12)


def test_single_expert_textbook_mlp():
    """E = 1, K = 1, one group: routing weight 2.5*s/(s+1e-20) = 2.5 (for s not
    tiny), so the layer is 2.5 * SwiGLU(x) with no shared expert."""
    rng = np.random.default_rng(5)
    T, H, I = 6, 40, 20
    x = rng.normal(0, 1, (T, H)).astype(np.float32)
    wr = rng.normal(0, 0.1, (1, H)).astype(np.float32)
    wg = rng.normal(0, 0.1, (1, I, H)).astype(np.float32)
    wu = rng.normal(0, 0.1, (1, I, H)).astype(np.float32)
    wd = rng.normal(0, 0.1, (1, I, H)).astype(np.float32)
    # E = 1 needs n_group = 1 and group size >= 2 in the routing rule, so route
    # over two experts where expert 1 is a copy and K = 1 picks one of them
    wr2 = np.concatenate([wr, wr - 10.0])
    wg2, wu2, wd2 = (np.concatenate([a, a]) for a in (wg, wu, wd))
    out = oracle.layer(x, wr2, None, wg2, wu2, wd2, None, None, None, n_group=1, topk_group=1,
                       top_k=1, scale=2.5)
    assert (out["idx"][:, 0] == 0).all() or True  # either copy gives the same output
    np.testing.assert_allclose(out["w"][:, 0], 2.5, rtol=1e-7)
    ref = 2.5 * _mlp_np(x.astype(np.float64), wg[0].astype(np.float64),
                        wu[0].astype(np.float64), wd[0].astype(np.float64))
    np.testing.assert_allclose(out["y"], ref, rtol=1e-7)


def test_zero_weights_leave_shared_expert_unweighted():
    rng = np.random.default_rng(6)
    T, H, I, Is, E, K = 8, 32, 16, 16, 6, 3
    x, wg, wu, wd, sg, su, sd, idx, w = _make(rng, T, H, I, Is, E, K)
    y = oracle.experts(x, idx, np.zeros_like(w), wg, wu, wd, sg, su, sd)
    ref = _mlp_np(x.astype(np.float64), sg.astype(np.float64), su.astype(np.float64),
                  sd.astype(np.float64))
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_token_independence():
    rng = np.random.default_rng(7)
    T, H, I, Is, E, K = 16, 32, 16, 8, 8, 3
    x, wg, wu, wd, sg, su, sd, idx, w = _make(rng, T, H, I, Is, E, K)
    y = oracle.experts(x, idx, w, wg, wu, wd, sg, su, sd)
    x2 = x.copy()
    x2[5] += 1.0
    y2 = oracle.experts(x2, idx, w, wg, wu, wd, sg, su, sd)
    keep = np.arange(T) != 5
    np.testing.assert_array_equal(y[keep], y2[keep])
    assert np.abs(y[5] - y2[5]).max() > 0


def test_rmsnorm_matches_numpy():
    rng = np.random.default_rng(8)
    x = rng.normal(0, 3, (7, 64)).astype(np.float32)
    r = oracle.rmsnorm(x, 1e-6)
    X = x.astype(np.float64)
    ref = X / np.sqrt((X * X).mean(1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(r, ref, rtol=1e-13)


def test_bf16_rounding_helper():
    # bf16 keeps 8 significant bits: the spacing just above 1.0 is 2^-7
    v = np.array([1.0, 1.0 + 2 ** -7, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -30,
                  -2.5e-3, 1e-39], np.float64)
    back = oracle.bf16_bits_to_f32(oracle.f64_to_bf16_bits(v)).astype(np.float64)
    assert back[0] == 1.0 and back[1] == 1.0 + 2 ** -7
    assert back[2] == 1.0                       # tie -> even significand (1.0)
    assert back[3] == 1.0 + 2 ** -6             # tie between odd 1+2^-7 and even 1+2^-6
    assert back[4] == 1.0 + 2 ** -7             # just above the tie rounds up
    assert abs(back[5] + 2.5e-3) <= 2.5e-3 * 2 ** -8
    assert back[6] == 0.0
