"""Pins of the oracle's load-balancing functions: hit tracking and its
statistics ([Routing §六]), the expert-bias update ([Routing §三]) and the
auxiliary loss E * sum_i f_i * P_i ([Pitfalls, MoE 负载均衡 Loss 别忘加]).

Each expected value here is a hand-worked example, a closed form, an invariant
or a property the pages state (the bias steers tokens toward idle experts);
none is computed by re-running the oracle's own formula.
"""
import math

import numpy as np
import pytest

import oracle
from group_limited_top_amd import synth


# --------------------------------------------------------------------------- tracking

def test_track_hand_example_and_accumulation():
    idx = np.array([[0, 3], [3, 1], [3, 0]], np.int32)       # T=3, K=2, E=5
    tr = oracle.track(idx, 5)
    np.testing.assert_array_equal(tr, [2, 1, 0, 3, 0])
    oracle.track(idx[:1], 5, tr)                               # accumulates
    np.testing.assert_array_equal(tr, [3, 1, 0, 4, 0])


def test_track_equals_bincount_of_a_routing():
    rng = np.random.default_rng(5)
    lam = rng.standard_normal((300, 64)).astype(np.float32)
    idx, _, _ = oracle.select(lam, None, 8, 4, 6, 2.5)
    tr = oracle.track(idx, 64)
    np.testing.assert_array_equal(tr, np.bincount(idx.ravel(), minlength=64))
    assert tr.sum() == 300 * 6


# --------------------------------------------------------------------------- statistics

def test_stats_hand_example():
    # hits [1, 2, 3, 6]: N = 12, balanced share 3, loads 1/3, 2/3, 1, 2;
    # cv = sqrt(((1-3)^2 + (2-3)^2 + 0 + (6-3)^2) / 4) / 3 = sqrt(3.5) / 3;
    # groups of two: {1, 2} = 3, {3, 6} = 9 -> largest group load 9 * 2 / 12
    load, s = oracle.expert_stats(np.array([1, 2, 3, 6]), n_group=2)
    np.testing.assert_array_equal(load[0], np.float32([1 / 3, 2 / 3, 1.0, 2.0]))
    assert s[0, 0] == 12 and s[0, 1] == 2.0 and s[0, 2] == 1 / 3
    assert s[0, 3] == pytest.approx(math.sqrt(3.5) / 3, rel=1e-15)
    assert s[0, 4] == 0 and s[0, 5] == 3 and s[0, 6] == 0 and s[0, 7] == 1.5


def test_stats_closed_forms():
    E, G = 256, 8
    tr = np.zeros((3, E), np.int64)
    tr[0] = 7                      # balanced
    tr[1, 40] = 1000               # every hit on one expert
    load, s = oracle.expert_stats(tr, G)   # layer 2: no hits at all
    assert np.all(load[0] == 1.0)
    assert list(s[0]) == [7 * E, 1.0, 1.0, 0.0, 0, 0, 0, 1.0]
    assert load[1, 40] == E and np.count_nonzero(load[1]) == 1
    assert s[1, 1] == E and s[1, 2] == 0 and s[1, 4] == E - 1
    assert s[1, 3] == pytest.approx(math.sqrt(E - 1), rel=1e-14)
    assert s[1, 5] == 40 and s[1, 6] == 0 and s[1, 7] == G
    assert np.all(load[2] == 0) and list(s[2]) == [0, 0, 0, 0, E, 0, 0, 0]


def test_stats_ties_take_the_lowest_index():
    _, s = oracle.expert_stats(np.array([4, 9, 9, 1, 1, 4]), n_group=3)
    assert s[0, 5] == 1 and s[0, 6] == 3


# --------------------------------------------------------------------------- bias update

def test_bias_update_hand_example():
    # counts [5, 1, 1, 1]: mean 2, excess [3, -1, -1, -1], largest 3;
    # rate 0.1 from zero: [-0.1, 0.1/3, 0.1/3, 0.1/3]
    b = oracle.bias_update(np.array([5, 1, 1, 1]), None, 0.1)
    np.testing.assert_array_equal(b, np.float32([-0.1, 0.1 / 3, 0.1 / 3, 0.1 / 3]))
    # from a non-zero bias the step adds to it
    b2 = oracle.bias_update(np.array([5, 1, 1, 1]), np.float32([1, 2, 3, 4]), 0.3)
    np.testing.assert_array_equal(b2, np.float32([1 - 0.3, 2 + 0.1, 3 + 0.1, 4 + 0.1]))


def test_bias_update_invariants():
    rng = np.random.default_rng(11)
    E = 256
    c = rng.integers(0, 400, E).astype(np.int32)
    b0 = (rng.standard_normal(E) * 0.05).astype(np.float32)
    b1 = oracle.bias_update(c, b0, 0.02)
    d = b1.astype(np.float64) - b0
    mean = c.sum() / E
    # hot experts go down, cold ones up, by at most the rate; the most
    # unbalanced expert moves by exactly the rate (up to the fp32 rounding)
    assert np.all(d[c > mean] < 0) and np.all(d[c < mean] > 0)
    assert np.all(np.abs(d) <= 0.02 + 1e-8)
    worst = np.argmax(np.abs(c - mean))
    assert abs(abs(d[worst]) - 0.02) < 1e-8
    # the steps sum to zero (up to the rounding of each bias to fp32)
    assert abs(d.sum()) < E * 2 ** -24
    # from a zero bias, the step is monotone in the count (rounding to fp32
    # keeps the order)
    order = np.argsort(c, kind="stable")
    assert np.all(np.diff(oracle.bias_update(c, None, 0.02)[order]) <= 0)
    # balanced counts and all-zero counts leave the bias unchanged
    np.testing.assert_array_equal(oracle.bias_update(np.full(E, 9, np.int32), b0, 0.5), b0)
    np.testing.assert_array_equal(oracle.bias_update(np.zeros(E, np.int32), b0, 0.5), b0)


def test_bias_update_from_zero_is_the_skewed_workload_bias():
    """The skewed workload's bias recipe, -0.1 (c_e - m) / max_e |c_e - m| with
    m = T k / E (evaluated here in numpy fp64, one rounding to fp32), is the
    oracle's update from a zero bias at rate 0.1."""
    rng = np.random.default_rng(3)
    c = rng.integers(0, 5000, 256).astype(np.int32)
    T = int(c.sum()) // 8
    c[0] += T * 8 - int(c.sum())
    ex = c.astype(np.float64) - T * 8 / 256
    recipe = ((-0.1 * ex) / max(np.abs(ex).max(), 1.0)).astype(np.float32)
    np.testing.assert_array_equal(oracle.bias_update(c, None, 0.1), recipe)


def test_balancing_loop_spreads_a_skewed_routing():
    """[Routing §三]: adding to cold experts and subtracting from hot ones
    drives tokens to idle experts.  Route a Zipf-skewed set of logits, update
    the bias from the counts, and repeat: the load evens out."""
    T, E = 4096, 256
    rng = np.random.default_rng(0)
    lam = (rng.standard_normal((T, E)) + synth.skew_offsets(E, 8, 7).numpy()).astype(np.float32)
    b = np.zeros(E, np.float32)
    first = None
    for it in range(40):
        idx, w, _ = oracle.select(lam, b, 8, 4, 8, 2.5)
        tr = oracle.track(idx, E)
        _, s = oracle.expert_stats(tr, 8)
        if first is None:
            first = s[0]
            w0 = w
        b = oracle.bias_update(tr.astype(np.int32), b, 0.01)
    assert first[1] > 20 and first[3] > 3          # heavily skewed at the start
    # the step never shrinks below the rate for the most unbalanced expert, so
    # the loads settle into a small oscillation instead of converging exactly
    assert s[0, 1] < 3.5 and s[0, 3] < 0.15 and s[0, 4] == 0
    # the bias changed the selection, and so the weights are those of the
    # unbiased scores of other experts, still summing to the scale
    assert not np.array_equal(idx, oracle.select(lam, None, 8, 4, 8, 2.5)[0])
    np.testing.assert_allclose(w.sum(1), 2.5, rtol=1e-6)
    np.testing.assert_allclose(w0.sum(1), 2.5, rtol=1e-6)


# --------------------------------------------------------------------------- auxiliary loss

def test_aux_loss_balanced_is_k():
    # equal logits: every P_i = 1/E; balanced counts: f_i = K/E; loss = K
    T, E, K = 64, 256, 8
    f, P, loss = oracle.aux_loss(np.zeros((T, E), np.float32), np.full(E, T * K // E, np.int32))
    assert np.all(P == 1 / E) and np.all(f == K / E) and loss == K


def test_aux_loss_closed_form_one_large_logit():
    # every token: logit a on expert 0, 0 elsewhere -> P_0 = e^a / (e^a + E - 1),
    # P_i = 1 / (e^a + E - 1) for the others; f = counts / T
    T, E, a = 10, 16, 2.0
    lam = np.zeros((T, E), np.float32)
    lam[:, 0] = a
    counts = np.array([10, 3, 0, 7] + [0] * 12, np.int32)
    f, P, loss = oracle.aux_loss(lam, counts)
    z = math.exp(a) + E - 1
    assert P[0] == pytest.approx(math.exp(a) / z, rel=1e-14)
    assert np.allclose(P[1:], 1 / z, rtol=1e-14, atol=0)
    want = E * (1.0 * math.exp(a) / z + 0.3 / z + 0.7 / z)
    assert loss == pytest.approx(want, rel=1e-14)
    np.testing.assert_array_equal(f, counts / T)


def test_aux_loss_invariants():
    rng = np.random.default_rng(9)
    T, E = 200, 64
    # logits on a grid of 2^-10, so that adding 5 is exact in fp32
    lam = (np.round(rng.standard_normal((T, E)) * 3 * 1024) / 1024).astype(np.float32)
    idx, _, _ = oracle.select(lam, None, 8, 4, 6, 2.5)
    c = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
    f, P, loss = oracle.aux_loss(lam, c)
    assert P.sum() == pytest.approx(1.0, abs=1e-14) and f.sum() == pytest.approx(6.0, abs=1e-14)
    assert np.all(P > 0)
    # a shift of a token's logits leaves its probabilities unchanged
    sh = lam + np.float32(5.0)
    assert np.all(sh - np.float32(5.0) == lam)
    _, P2, loss2 = oracle.aux_loss(sh, c)
    np.testing.assert_allclose(P2, P, rtol=1e-13)
    assert loss2 == pytest.approx(loss, rel=1e-13)
    # brute force in another order, over every (token, routed pair):
    # E / T^2 * sum_t sum_{t', j} softmax(lam_t)[idx[t', j]]
    p = np.exp(lam.astype(np.float64) - lam.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    bf = E / T ** 2 * float(p[:, idx.ravel()].sum())
    assert loss == pytest.approx(bf, rel=1e-12)
    # sending every token to the experts of highest mean probability raises the loss
    top = np.argsort(-P, kind="stable")[:6]
    c2 = np.zeros(E, np.int32)
    c2[top] = T
    assert oracle.aux_loss(lam, c2)[2] > loss
