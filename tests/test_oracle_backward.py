"""Pins of the oracle's backward of the layer (fixed routing): every gradient
against central finite differences of the fp64 forward, against
torch.autograd (float64, CPU) applied to the forward written with torch ops,
and against identities that follow from the forward's form.

Definition being differentiated (the oracle's header states it): router
logits lam = x W_r^T, scores s = sigmoid(lam), routing weights w_j =
scale * s_j / (sum s + 1e-20) over the chosen experts ([Routing §二 steps 1-3]),
y = shared(x) + sum_j w_j expert_j(x) ([Routing §四, §五]); L = <dy, y>.  The
choice of experts is held fixed (it is piecewise constant).
"""
import numpy as np
import pytest
import torch

import oracle


def tiny_layer(seed, T=4, H=8, E=8, I=4, Is=3, K=3):
    rng = np.random.default_rng(seed)
    p = dict(
        x=rng.standard_normal((T, H)),
        w_router=rng.standard_normal((E, H)) * 0.5,
        w_gate=rng.standard_normal((E, I, H)) * 0.4,
        w_up=rng.standard_normal((E, I, H)) * 0.4,
        w_down=rng.standard_normal((E, I, H)) * 0.4,
        ws_gate=rng.standard_normal((Is, H)) * 0.4 if Is else None,
        ws_up=rng.standard_normal((Is, H)) * 0.4 if Is else None,
        ws_down=rng.standard_normal((Is, H)) * 0.4 if Is else None,
    )
    lam = oracle.logits_any(p["x"], p["w_router"])
    # a fixed choice of K distinct experts per token (any choice is a valid
    # point of the piecewise-smooth layer; take the K largest logits)
    idx = np.argsort(-lam, axis=1, kind="stable")[:, :K].astype(np.int32)
    dy = rng.standard_normal((T, H))
    return p, idx, dy


def weights_of(p):
    return [p[k] for k in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")]


def loss(p, idx, dy, scale):
    lam = oracle.logits_any(p["x"], p["w_router"])
    out = oracle.backward_tokens(p["x"], p["w_router"], lam, idx, scale, dy, *weights_of(p),
                                 want_y=True, nthreads=1)
    return float((out["y"] * dy).sum())


def analytic(p, idx, dy, scale):
    lam = oracle.logits_any(p["x"], p["w_router"])
    tok = oracle.backward_tokens(p["x"], p["w_router"], lam, idx, scale, dy, *weights_of(p),
                                 want_y=True, nthreads=1)
    E = p["w_router"].shape[0]
    g = {"x": tok["dx"], "w_router": oracle.router_weight_grad(p["x"], tok["dlogit"])}
    for k in ("w_gate", "w_up", "w_down"):
        g[k] = np.zeros_like(p[k])
    for e in range(E):
        dg, du, dd = oracle.backward_expert_weights(p["x"], lam, idx, scale, dy, e,
                                                    *weights_of(p), nthreads=1)
        g["w_gate"][e], g["w_up"][e], g["w_down"][e] = dg, du, dd
    if p["ws_gate"] is not None:
        g["ws_gate"], g["ws_up"], g["ws_down"] = oracle.backward_expert_weights(
            p["x"], lam, idx, scale, dy, E, *weights_of(p), nthreads=1)
    return g, tok


# --------------------------------------------------------------------------- finite differences

@pytest.mark.parametrize("seed,scale", [(0, 2.5), (1, 1.0)])
def test_every_gradient_matches_central_differences(seed, scale):
    p, idx, dy = tiny_layer(seed)
    g, _ = analytic(p, idx, dy, scale)
    h = 1e-5
    for name, arr in p.items():
        if arr is None:
            continue
        flat = arr.reshape(-1)
        num = np.empty_like(flat)
        for i in range(flat.size):
            v = flat[i]
            flat[i] = v + h
            lp = loss(p, idx, dy, scale)
            flat[i] = v - h
            lm = loss(p, idx, dy, scale)
            flat[i] = v
            num[i] = (lp - lm) / (2 * h)
        ana = g[name].reshape(-1)
        # central differences are exact to O(h^2) ~ 1e-10 here, plus
        # cancellation of the loss (~1e0) at ~1e-16 / h ~ 1e-11
        np.testing.assert_allclose(ana, num, rtol=1e-6, atol=1e-8, err_msg=name)


def test_unchosen_experts_get_no_gradient():
    p, idx, dy = tiny_layer(3)
    g, tok = analytic(p, idx, dy, 2.5)
    chosen = np.zeros(p["w_router"].shape[0], bool)
    chosen[np.unique(idx)] = True
    for k in ("w_gate", "w_up", "w_down"):
        assert np.all(g[k][~chosen] == 0)
    mask = np.zeros_like(tok["dlogit"], bool)
    np.put_along_axis(mask, idx, True, axis=1)
    assert np.all(tok["dlogit"][~mask] == 0)


# --------------------------------------------------------------------------- torch.autograd

def torch_forward(t, idx, scale):
    """The same forward written with torch ops (float64), for autograd."""
    lam = t["x"] @ t["w_router"].T
    s = torch.sigmoid(lam)
    idx_t = torch.from_numpy(idx).long()
    sc = torch.gather(s, 1, idx_t)
    w = scale * sc / (sc.sum(1, keepdim=True) + 1e-20)

    def mlp(xr, wg, wu, wd):
        gg = xr @ wg.T
        uu = xr @ wu.T
        return (torch.nn.functional.silu(gg) * uu) @ wd

    y = torch.zeros_like(t["x"])
    if t.get("ws_gate") is not None:
        y = y + mlp(t["x"], t["ws_gate"], t["ws_up"], t["ws_down"])
    T, K = idx.shape
    rows = []
    for tt in range(T):
        acc = y[tt]
        for j in range(K):
            e = int(idx[tt, j])
            acc = acc + w[tt, j] * mlp(t["x"][tt:tt + 1], t["w_gate"][e], t["w_up"][e],
                                       t["w_down"][e])[0]
        rows.append(acc)
    return torch.stack(rows)


@pytest.mark.parametrize("shape", [(16, 24, 16, 8, 6, 4), (9, 16, 32, 12, 0, 8)])
def test_matches_torch_autograd(shape):
    T, H, E, I, Is, K = shape
    p, idx, dy = tiny_layer(7 + T, T=T, H=H, E=E, I=I, Is=Is, K=K)
    g, tok = analytic(p, idx, dy, 2.5)
    t = {k: (None if v is None else torch.tensor(v, dtype=torch.float64, requires_grad=True))
         for k, v in p.items()}
    y = torch_forward(t, idx, 2.5)
    np.testing.assert_allclose(tok["y"], y.detach().numpy(), rtol=1e-12, atol=1e-12)
    (y * torch.from_numpy(dy)).sum().backward()
    for k, v in t.items():
        if v is None:
            continue
        np.testing.assert_allclose(g[k], v.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=k)


# --------------------------------------------------------------------------- identities

def test_weight_gradient_identity_and_linearity():
    """y - shared(x) = sum_j w_j expert_j(x) and dL/dw_j = <dy, expert_j(x)>,
    so sum_j w_j dL/dw_j = <dy, y - shared(x)>; the backward is linear in dy."""
    p, idx, dy = tiny_layer(11, T=6, H=8, E=8, I=4, Is=3, K=3)
    lam = oracle.logits_any(p["x"], p["w_router"])
    tok = oracle.backward_tokens(p["x"], p["w_router"], lam, idx, 2.5, dy, *weights_of(p),
                                 want_y=True)
    p0 = dict(p, ws_down=np.zeros_like(p["ws_down"]))   # shared(x) = 0
    tok0 = oracle.backward_tokens(p["x"], p["w_router"], lam, idx, 2.5, dy, *weights_of(p0),
                                  want_y=True)
    s = 1 / (1 + np.exp(-np.take_along_axis(lam, idx, 1)))
    w = 2.5 * s / (s.sum(1, keepdims=True) + 1e-20)
    lhs = (w * tok["dweight"]).sum(1)
    rhs = (dy * tok0["y"]).sum(1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12)
    tok2 = oracle.backward_tokens(p["x"], p["w_router"], lam, idx, 2.5, 2 * dy, *weights_of(p))
    for k in ("dx", "dweight", "dlogit"):
        np.testing.assert_array_equal(tok2[k], 2 * tok[k])


def test_routing_weights_are_scale_invariant_in_the_scores():
    """w_j = scale s_j / (sum s + 1e-20) does not change when every chosen score
    is multiplied by the same factor (while the 1e-20 is negligible), so the
    score gradient is orthogonal to the scores: sum_m s_m dL/ds_m = 0, i.e.
    sum_m dlogit_m / (1 - s_m) = 0 over the chosen experts."""
    p, idx, dy = tiny_layer(13, T=8, H=8, E=8, I=4, Is=3, K=4)
    lam = oracle.logits_any(p["x"], p["w_router"])
    tok = oracle.backward_tokens(p["x"], p["w_router"], lam, idx, 2.5, dy, *weights_of(p))
    s = 1 / (1 + np.exp(-np.take_along_axis(lam, idx, 1)))
    dl = np.take_along_axis(tok["dlogit"], idx, 1)
    ortho = (dl / (1 - s)).sum(1)
    scale_ref = np.abs(dl / (1 - s)).sum(1)
    assert np.all(np.abs(ortho) <= 1e-12 * scale_ref)
    # with one chosen expert the weight is the constant scale: no router gradient
    p1, idx1, dy1 = tiny_layer(13, T=8, H=8, E=8, I=4, Is=3, K=1)
    tok1 = oracle.backward_tokens(p1["x"], p1["w_router"], oracle.logits_any(p1["x"], p1["w_router"]),
                                  idx1, 2.5, dy1, *weights_of(p1))
    assert np.abs(tok1["dlogit"]).max() < 1e-15


def test_token_subset_matches_full_rows():
    p, idx, dy = tiny_layer(17, T=10, H=8, E=8, I=4, Is=3, K=3)
    lam = oracle.logits_any(p["x"], p["w_router"])
    full = oracle.backward_tokens(p["x"], p["w_router"], lam, idx, 2.5, dy, *weights_of(p))
    sub = oracle.backward_tokens(p["x"], p["w_router"], lam, idx, 2.5, dy, *weights_of(p),
                                 tokens=np.array([7, 2, 9]))
    for k in ("dx", "dweight", "dlogit"):
        np.testing.assert_array_equal(sub[k], full[k][[7, 2, 9]])
