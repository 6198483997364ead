"""Pins of the CPU oracle's RoPE and Givens maps and of the Multi-Head Relation
backward built from them (oracle/mhr.py), against facts the pages and the
mathematics fix rather than against the oracle's own formulas:

* RoPE (Sec. 3.1; App. B.3): a rotation per pair, so norms are kept,
  position 0 is the identity, and q.k depends on the two positions only
  through their difference; pair 0 turns by exactly t radians at position t
  (base^0 = 1) and the last pair by t * base^(-(D-2)/D); the transpose is the
  inverse.
* Givens (Sec. 3.2; App. A.2.2-A.2.3): the pairings are the pages' M_A and
  M_B lists; theta = 0 is the identity and theta = pi/2 maps
  [I_a; I_b] -> [I_b; -I_a] as G(theta) prescribes; the mixing is
  orthogonal.
* The full chain's gradients (p1, p2, I, lambda, theta) against central
  finite differences of the forward in fp64.
"""
import math

import numpy as np
import pytest

import oracle


@pytest.fixture
def rng():
    return np.random.default_rng(20260)


def test_rope_tables_pair0_turns_one_radian_per_position_and_last_pair_slowest():
    T, D = 9, 8
    c, s = oracle.rope_tables(T, D)
    for t in range(T):
        x = np.zeros((T, D))
        x[t, 0] = 1.0  # unit vector in pair 0 (elements 0 and D/2)
        y = oracle.rope_rotate(x, c, s)
        assert abs(y[t, 0] - math.cos(t)) < 1e-15 and abs(y[t, D // 2] - math.sin(t)) < 1e-15
        x = np.zeros((T, D))
        x[t, D // 2 - 1] = 1.0  # last pair: frequency 1e4^(-(D-2)/D)
        w = t * 1.0e4 ** (-(D - 2) / D)
        y = oracle.rope_rotate(x, c, s)
        assert abs(y[t, D // 2 - 1] - math.cos(w)) < 1e-15
        assert abs(y[t, D - 1] - math.sin(w)) < 1e-15


def test_rope_is_a_rotation_with_identity_at_position_0(rng):
    T, D = 7, 16
    c, s = oracle.rope_tables(T, D)
    x = rng.standard_normal((2, 3, T, D))
    y = oracle.rope_rotate(x, c, s)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), atol=1e-13)
    assert np.array_equal(y[..., 0, :], x[..., 0, :])
    assert np.allclose(oracle.rope_rotate_transpose(y, c, s), x, atol=1e-13)


def test_rope_scores_depend_only_on_relative_position(rng):
    T, D = 12, 8
    c, s = oracle.rope_tables(T, D)
    qv, kv = rng.standard_normal(D), rng.standard_normal(D)

    def score(m, n):
        Q = np.zeros((T, D))
        K = np.zeros((T, D))
        Q[m], K[n] = qv, kv
        return oracle.rope_rotate(Q, c, s)[m] @ oracle.rope_rotate(K, c, s)[n]

    for m, n, sh in ((5, 2, 3), (7, 7, 4), (3, 0, 8)):
        assert abs(score(m, n) - score(m + sh, n + sh)) < 1e-12
    assert abs(score(5, 2) - score(5, 3)) > 1e-6  # but it does depend on m - n


def test_rope_transpose_is_the_adjoint(rng):
    T, D = 6, 10
    c, s = oracle.rope_tables(T, D)
    x, g = rng.standard_normal((T, D)), rng.standard_normal((T, D))
    lhs = (oracle.rope_rotate(x, c, s) * g).sum()
    rhs = (x * oracle.rope_rotate_transpose(g, c, s)).sum()
    assert abs(lhs - rhs) < 1e-12


def test_givens_pairings_are_the_pages_lists():
    # App. A.2.3, 1-based: M_A = {(1,2),(3,4),...,(H-1,H)}, M_B = {(2,3),...,(H,1)}
    ma = [(a + 1, b + 1) for a, b in oracle.givens_pairs(8, 0)]
    mb = [(a + 1, b + 1) for a, b in oracle.givens_pairs(8, 1)]
    assert ma == [(1, 2), (3, 4), (5, 6), (7, 8)]
    assert mb == [(2, 3), (4, 5), (6, 7), (8, 1)]
    with pytest.raises(ValueError):
        oracle.givens_pairs(5, 0)


@pytest.mark.parametrize("pairing", [0, 1])
def test_givens_special_angles_and_orthogonality(rng, pairing):
    B, H, T, D = 2, 6, 3, 4
    I = rng.standard_normal((B, H, T, D))
    assert np.array_equal(oracle.givens_mix(I, np.zeros(H // 2), pairing), I)
    out = oracle.givens_mix(I, np.full(H // 2, math.pi / 2), pairing)
    for a, b in oracle.givens_pairs(H, pairing):
        # G(pi/2) = [[0, 1], [-1, 0]]
        assert np.allclose(out[:, a], I[:, b], atol=1e-15)
        assert np.allclose(out[:, b], -I[:, a], atol=1e-15)
    th = rng.uniform(-3, 3, H // 2)
    out = oracle.givens_mix(I, th, pairing)
    assert np.allclose((out ** 2).sum(axis=1), (I ** 2).sum(axis=1), atol=1e-12)
    g = rng.standard_normal(I.shape)
    dI, _ = oracle.givens_mix_transpose(g, out, th, pairing)
    assert abs((out * g).sum() - (I * dI).sum()) < 1e-11  # adjoint


@pytest.mark.parametrize("pairing", [0, 1])
def test_mhr_backward_matches_finite_differences(rng, pairing):
    B, H, T, D = 1, 4, 6, 4
    scale, tau, lam = 0.7, 2.0, 0.4
    p1, p2, I = (rng.standard_normal((B, H, T, D)) for _ in range(3))
    W = rng.standard_normal((B, H, T, D))
    c, s = oracle.rope_tables(T, D)
    th = rng.uniform(-1.5, 1.5, H // 2)

    def loss(p1_, p2_, I_, lam_, th_):
        f = oracle.relation_mhr_forward(p1_, p2_, I_, c, s, th_, pairing, scale, tau, lam_)
        return float((f["Y"] * W).sum())

    dp1, dp2, dI, dlam, dth = oracle.relation_mhr_backward(p1, p2, I, W, c, s, th, pairing,
                                                           scale, tau, lam)
    h = 1e-6
    for name, x, grad in (("p1", p1, dp1), ("p2", p2, dp2), ("I", I, dI)):
        for idx in [(0, 0, 0, 0), (0, 1, 3, 2), (0, 3, 5, 1), (0, 2, 1, 3)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"p1": (xp, p2, I), "p2": (p1, xp, I), "I": (p1, p2, xp)}[name]
            args_m = {"p1": (xm, p2, I), "p2": (p1, xm, I), "I": (p1, p2, xm)}[name]
            num = (loss(*args_p, lam, th) - loss(*args_m, lam, th)) / (2 * h)
            assert abs(num - grad[idx]) < 1e-7 * max(1.0, abs(num)), (name, idx, num, grad[idx])
    num = (loss(p1, p2, I, lam + h, th) - loss(p1, p2, I, lam - h, th)) / (2 * h)
    assert abs(num - dlam) < 1e-7 * max(1.0, abs(num))
    for p in range(H // 2):
        tp, tm = th.copy(), th.copy()
        tp[p] += h
        tm[p] -= h
        num = (loss(p1, p2, I, lam, tp) - loss(p1, p2, I, lam, tm)) / (2 * h)
        assert abs(num - dth[p]) < 1e-7 * max(1.0, abs(num)), (p, num, dth[p])


def test_mhr_without_rope_and_mixing_is_the_plain_operator(rng):
    B, H, T, D = 1, 2, 5, 3
    p1, p2, I = (rng.standard_normal((B, H, T, D)) for _ in range(3))
    f = oracle.relation_mhr_forward(p1, p2, I, None, None, None, 0, 0.5, 2.0, 0.3)
    Y, LSE, g = oracle.relation_forward(p1, p2, I, 0.5, 2.0, 0.3)
    assert np.array_equal(f["Y"], Y) and np.array_equal(f["LSE"], LSE)


def test_input_generator_tables_are_the_rope_definition_in_fp32():
    # the tables both sides consume are the oracle's fp64 tables rounded once
    import torch  # noqa: F401  (the generator returns torch tensors)
    from workloads import make_mhr_maps
    T, D, H = 300, 64, 8
    cs, sn, th = make_mhr_maps(T, D, H, seed=1)
    c64, s64 = oracle.rope_tables(T, D)
    assert np.array_equal(cs.numpy(), c64.astype(np.float32))
    assert np.array_equal(sn.numpy(), s64.astype(np.float32))
    assert th.shape == (H // 2,) and np.all(np.abs(th.numpy()) <= math.pi)
