"""Pins of the Linear Relation oracle (oracle/linear.py) against facts the pages
and the mathematics fix, not against its own formulas:

* The two statements the pages give, the recurrent step (Sec. 5.2) and the
  unrolled historical Exchange (App. A.4.5), must agree.
* Closed forms: without retention loss and with every coordinate along one
  direction, E_t = S_t sum_{j<t} S_j I_j; with a constant retention r on
  that direction, E_t = S_t sum_{j<t} r^(t-j) S_j I_j; total loss (alpha = 0)
  leaves Y = I; orthogonal read and write directions give E = 0; a single
  token has no history (Y = I).
* Strict history (Sec. 5.2: the state is read before the token is written):
  I_t never reaches E_t or any earlier row.
* State hand-off: running two segments with the first's final state as the
  second's initial state equals one pass.
* RoPE (App. A.4.1): it leaves S unchanged (same rotation on p1_t and p2_t);
  with retention equal across channels only relative positions matter.
* The decode step reproduces the forward token by token.
* Gradients (p1, p2, I, g, C0) against central finite differences in fp64.
"""
import math

import numpy as np
import pytest

import oracle


@pytest.fixture
def rng():
    return np.random.default_rng(31415)


def sig(x):
    return 1.0 / (1.0 + math.exp(-x))


def rand_inputs(rng, lead, T, D, gmax=1.5):
    p1, p2, I = (rng.standard_normal((*lead, T, D)) for _ in range(3))
    g = -rng.uniform(0.0, gmax, (*lead, T, D))
    return p1, p2, I, g


@pytest.mark.parametrize("use_rope", [False, True])
def test_recurrence_equals_unrolled_exchange(rng, use_rope):
    B, H, T, D = 2, 2, 9, 6
    p1, p2, I, g = rand_inputs(rng, (B, H), T, D)
    cs, sn = oracle.rope_tables(T, D) if use_rope else (None, None)
    f = oracle.linear_relation_forward(p1, p2, I, g, 0.4, 2.0, cs, sn)
    E = oracle.linear_relation_unrolled(p1, p2, I, g, 0.4, 2.0, cs, sn)
    assert np.allclose(f["E"], E, atol=1e-13, rtol=0)
    assert np.array_equal(f["Y"], I + f["E"])
    assert np.abs(E).max() > 0.1  # not trivially zero


def test_one_direction_no_retention_loss_is_a_cumulative_sum(rng):
    T, D = 7, 4
    c, d = rng.uniform(0.5, 2.0, T), rng.uniform(0.5, 2.0, T)
    p1 = np.zeros((T, D))
    p2 = np.zeros((T, D))
    p1[:, 2], p2[:, 2] = c, d
    I = rng.standard_normal((T, D))
    s, tau = 0.3, 2.0
    f = oracle.linear_relation_forward(p1, p2, I, np.zeros((T, D)), s, tau)
    S = np.array([sig(s * c[t] * d[t] / tau) for t in range(T)])
    assert np.allclose(f["S"], S, atol=1e-15)
    for t in range(T):
        want = S[t] * sum(S[j] * I[j] for j in range(t)) if t else np.zeros(D)
        assert np.allclose(f["E"][t], want, atol=1e-14)


def test_constant_retention_on_one_direction_is_geometric(rng):
    T, D, r = 8, 5, 0.7
    p1 = np.zeros((T, D))
    p2 = np.zeros((T, D))
    p1[:, 1] = rng.uniform(0.5, 2.0, T)
    p2[:, 1] = rng.uniform(0.5, 2.0, T)
    g = -rng.uniform(0.0, 3.0, (T, D))  # other channels carry nothing
    g[:, 1] = math.log(r)
    I = rng.standard_normal((T, D))
    f = oracle.linear_relation_forward(p1, p2, I, g, 1.0, 2.0)
    S = f["S"]
    for t in range(T):
        want = S[t] * sum(r ** (t - j) * S[j] * I[j] for j in range(t)) if t else 0 * I[0]
        assert np.allclose(f["E"][t], want, atol=1e-14)


def test_total_retention_loss_and_orthogonal_directions_give_no_exchange(rng):
    T, D = 6, 4
    p1, p2, I, _ = rand_inputs(rng, (2,), T, D)
    f = oracle.linear_relation_forward(p1, p2, I, np.full((2, T, D), -1.0e4), 0.5, 2.0)
    assert np.array_equal(f["Y"], I)
    # the last write is all that is left in the state
    h2, _ = oracle.linear_normalize(p2[:, -1])
    want = f["S"][:, -1, None, None] * h2[:, :, None] * I[:, -1, None, :]
    assert np.allclose(f["C"], want, atol=1e-15)
    # read along channel 0, write along channel 1: nothing is read back
    a, b = np.zeros((T, D)), np.zeros((T, D))
    a[:, 0], b[:, 1] = 1.0 + np.arange(T), 2.0
    f = oracle.linear_relation_forward(a, b, I[0], np.zeros((T, D)), 0.5, 2.0)
    assert np.array_equal(f["E"], np.zeros((T, D)))
    assert np.allclose(f["S"], 0.5)


def test_single_token_and_zero_rows(rng):
    p1, p2, I, g = rand_inputs(rng, (3,), 1, 5)
    f = oracle.linear_relation_forward(p1, p2, I, g, 0.5, 2.0)
    assert np.array_equal(f["Y"], I)
    # a zero coordinate row reads nothing (and writes nothing) without NaN
    p1, p2, I, g = rand_inputs(rng, (), 6, 4)
    p1[3] = 0.0
    p2[2] = 0.0
    f = oracle.linear_relation_forward(p1, p2, I, g, 0.5, 2.0)
    assert np.isfinite(f["Y"]).all()
    assert np.array_equal(f["E"][3], np.zeros(4))
    E = oracle.linear_relation_unrolled(p1, p2, I, g, 0.5, 2.0)
    assert np.allclose(f["E"], E, atol=1e-14)


def test_strict_history(rng):
    T, D, t0 = 9, 5, 4
    p1, p2, I, g = rand_inputs(rng, (), T, D)
    base = oracle.linear_relation_forward(p1, p2, I, g, 0.5, 2.0)
    I2 = I.copy()
    I2[t0] += 10.0
    pert = oracle.linear_relation_forward(p1, p2, I2, g, 0.5, 2.0)
    assert np.array_equal(pert["E"][:t0 + 1], base["E"][:t0 + 1])
    assert np.allclose(pert["Y"][t0] - base["Y"][t0], 10.0, atol=1e-13)
    assert np.abs(pert["E"][t0 + 1:] - base["E"][t0 + 1:]).max() > 1e-3


def test_state_handoff_equals_one_pass(rng):
    T, D, T1 = 11, 6, 4
    p1, p2, I, g = rand_inputs(rng, (2, 3), T, D)
    cs, sn = oracle.rope_tables(T, D)
    whole = oracle.linear_relation_forward(p1, p2, I, g, 0.4, 2.0, cs, sn)
    a = oracle.linear_relation_forward(p1[..., :T1, :], p2[..., :T1, :], I[..., :T1, :],
                                       g[..., :T1, :], 0.4, 2.0, cs[:T1], sn[:T1])
    b = oracle.linear_relation_forward(p1[..., T1:, :], p2[..., T1:, :], I[..., T1:, :],
                                       g[..., T1:, :], 0.4, 2.0, cs[T1:], sn[T1:], C0=a["C"])
    assert np.allclose(np.concatenate([a["Y"], b["Y"]], axis=-2), whole["Y"], atol=1e-13)
    assert np.allclose(b["C"], whole["C"], atol=1e-13)


def test_rope_keeps_self_and_only_relative_positions_matter_with_uniform_retention(rng):
    T, D = 8, 6
    p1, p2, I, _ = rand_inputs(rng, (), T, D)
    cs, sn = oracle.rope_tables(T + 5, D)
    gu = np.repeat(-rng.uniform(0, 1, (T, 1)), D, axis=1)  # the same on every channel
    f0 = oracle.linear_relation_forward(p1, p2, I, gu, 0.5, 2.0, cs[:T], sn[:T])
    f5 = oracle.linear_relation_forward(p1, p2, I, gu, 0.5, 2.0, cs[5:], sn[5:])
    plain = oracle.linear_relation_forward(p1, p2, I, gu, 0.5, 2.0)
    assert np.allclose(f0["S"], plain["S"], atol=1e-15)
    assert np.allclose(f0["Y"], f5["Y"], atol=1e-13)
    assert np.abs(f0["Y"] - plain["Y"]).max() > 1e-3  # RoPE does act
    # per-channel retention breaks the shift invariance
    g = -rng.uniform(0, 1, (T, D))
    a = oracle.linear_relation_forward(p1, p2, I, g, 0.5, 2.0, cs[:T], sn[:T])
    b = oracle.linear_relation_forward(p1, p2, I, g, 0.5, 2.0, cs[5:], sn[5:])
    assert np.abs(a["Y"] - b["Y"]).max() > 1e-4


def test_decode_steps_reproduce_the_forward(rng):
    T, D = 7, 4
    p1, p2, I, g = rand_inputs(rng, (2, 2), T, D)
    cs, sn = oracle.rope_tables(T, D)
    f = oracle.linear_relation_forward(p1, p2, I, g, 0.5, 2.0, cs, sn)
    C = np.zeros((2, 2, D, D))
    for t in range(T):
        y, C = oracle.linear_relation_step(p1[..., t, :], p2[..., t, :], I[..., t, :],
                                           g[..., t, :], C, 0.5, 2.0, cs[t], sn[t])
        assert np.allclose(y, f["Y"][..., t, :], atol=1e-14)
    assert np.allclose(C, f["C"], atol=1e-14)


@pytest.mark.parametrize("use_rope", [False, True])
def test_backward_matches_finite_differences(rng, use_rope):
    T, D = 6, 4
    p1, p2, I, g = rand_inputs(rng, (2,), T, D)
    C0 = rng.standard_normal((2, D, D))
    W = rng.standard_normal((2, T, D))
    WC = rng.standard_normal((2, D, D))
    cs, sn = oracle.rope_tables(T, D) if use_rope else (None, None)
    s, tau = 0.6, 2.0

    def loss(a, b, c, d, e):
        f = oracle.linear_relation_forward(a, b, c, d, s, tau, cs, sn, C0=e)
        return float((f["Y"] * W).sum() + (f["C"] * WC).sum())

    grads = oracle.linear_relation_backward(p1, p2, I, g, W, s, tau, cs, sn, C0=C0, dC_T=WC)
    args = [p1, p2, I, g, C0]
    h = 1e-6
    for which, grad in enumerate(grads):
        x = args[which]
        idxs = [(0, 0, 0), (1, 3, 2), (0, T - 1, 3) if which < 4 else (0, 2, 3), (1, 2, 1)]
        for idx in idxs:
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap = list(args)
            am = list(args)
            ap[which], am[which] = xp, xm
            num = (loss(*ap) - loss(*am)) / (2 * h)
            assert abs(num - grad[idx]) < 1e-6 * max(1.0, abs(num)), (which, idx, num, grad[idx])
