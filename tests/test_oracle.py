"""Pins of the fp64 CPU oracle (no GPU): brute force, the pages' invariants,
closed forms, finite differences, the tiled scan, decode and causality."""
import math

import numpy as np
import pytest

import oracle
from tests import oracle_pins as P


@pytest.fixture
def rng():
    return np.random.default_rng(1234)


@pytest.mark.parametrize("T,D,scale,lam", [(1, 2, 0.5, 0.3), (2, 1, 1.0, 0.0), (5, 3, 0.6, 0.37),
                                           (8, 4, 1 / math.sqrt(4), -0.5), (8, 2, 1.7, 1.0)])
def test_brute_force_matches_vectorised(rng, T, D, scale, lam):
    err = P.check_brute_force(oracle.relation_forward_head, oracle.brute_force_forward_head,
                              rng, T=T, D=D, scale=scale, lam=lam)
    assert err < 1e-13


@pytest.mark.parametrize("lam", [0.0, 0.6, 1.0, -0.5])
@pytest.mark.parametrize("scale", [1 / math.sqrt(4), 1 / 4])
def test_flow_invariants(rng, lam, scale):
    assert P.check_invariants(oracle.relation_forward_head, rng, scale=scale, lam=lam) < 1e-13


def test_lambda_leaves_allocation_unchanged(rng):
    err, g_moves = P.check_lambda_allocation(oracle.relation_forward_head, rng)
    assert err < 1e-14
    assert g_moves > 1e-3


@pytest.mark.parametrize("which", ["q", "k"])
def test_closed_form_zero_evidence(rng, which):
    assert P.check_closed_form_zero_evidence(oracle.relation_forward_head, rng, which=which) < 1e-14


def test_closed_form_two_tokens():
    assert P.check_closed_form_T2(oracle.relation_forward_head) < 1e-15


def test_single_token_is_all_self(rng):
    q, k, v = P.rand_head(rng, 1, 5)
    r = oracle.relation_forward_head(q, k, v, 0.4, 2.0, 0.7)
    assert np.array_equal(r["Y"], v)
    assert r["g"][0] == 0.0
    S = 1 / (1 + math.exp(-0.4 * float(q[0] @ k[0]) / 2.0))
    assert abs(r["LSE"][0] - S) < 1e-16


def test_extreme_lambda_limits(rng):
    q, k, v = P.rand_head(rng, 6, 3)
    big = oracle.relation_forward_head(q, k, v, 0.5, 2.0, 60.0)
    assert np.abs(big["Y"] - v).max() < 1e-12       # history suppressed: all Self
    neg = oracle.relation_forward_head(q, k, v, 0.5, 2.0, -60.0)
    assert np.abs(neg["g"][1:] - 1.0).max() < 1e-12  # history dominates


def test_causality_exact(rng):
    assert P.check_causality(oracle.relation_forward_head, rng) == 0.0


@pytest.mark.parametrize("tile", [1, 2, 3, 16, 64])
def test_tiled_scan_is_exact(rng, tile):
    q, k, v = P.rand_head(rng, 70, 4)
    r = oracle.relation_forward_head(q, k, v, 0.5, 2.0, 0.42)
    Y, LSE, g = oracle.tiled_forward_head(q, k, v, 0.5, 2.0, 0.42, tile)
    assert np.abs(Y - r["Y"]).max() < 1e-13
    assert np.abs(LSE - r["LSE"]).max() < 1e-13
    assert np.abs(g - r["g"]).max() < 1e-13


def test_rows_match_materialised(rng):
    q, k, v = P.rand_head(rng, 40, 6)
    r = oracle.relation_forward_head(q, k, v, 0.4, 2.0, 0.3)
    rows = [1, 2, 17, 39, 40]
    Y, LSE, g = oracle.relation_forward_rows(q, k, v, rows, 0.4, 2.0, 0.3)
    idx = np.array(rows) - 1
    assert np.abs(Y - r["Y"][idx]).max() < 1e-14
    assert np.abs(LSE - r["LSE"][idx]).max() < 1e-14
    assert np.abs(g - r["g"][idx]).max() < 1e-14


def test_multihead_is_headwise(rng):
    q = rng.standard_normal((2, 3, 12, 4))
    k = rng.standard_normal((2, 3, 12, 4))
    v = rng.standard_normal((2, 3, 12, 4))
    Y, LSE, g = oracle.relation_forward(q, k, v, 0.5, 2.0, 0.2)
    for b in range(2):
        for h in range(3):
            r = oracle.relation_forward_head(q[b, h], k[b, h], v[b, h], 0.5, 2.0, 0.2)
            assert np.array_equal(Y[b, h], r["Y"])
    q2 = q.copy()
    q2[0, 1] += 1.0
    Y2, _, _ = oracle.relation_forward(q2, k, v, 0.5, 2.0, 0.2)
    assert np.array_equal(Y2[0, 0], Y[0, 0]) and np.array_equal(Y2[1], Y[1])
    assert not np.array_equal(Y2[0, 1], Y[0, 1])


@pytest.mark.parametrize("lam", [0.55, 0.0, -0.5])
def test_backward_finite_differences(rng, lam):
    err = P.check_backward_fd(oracle.relation_forward_head, oracle.relation_backward_head,
                              rng, lam=lam)
    assert err < 1e-8


def test_backward_identities(rng):
    assert P.check_backward_identities(oracle.relation_backward_head, rng) < 1e-14


def test_self_derivative(rng):
    """dS/dU_ii = S(1 - S)/tau_S (App. A.1.7), by central difference."""
    tau = 2.0
    for u in (-3.0, -0.2, 0.0, 1.4, 5.0):
        S = lambda x: 1 / (1 + math.exp(-x / tau))  # noqa: E731
        h = 1e-6
        fd = (S(u + h) - S(u - h)) / (2 * h)
        s = S(u)
        assert abs(fd - s * (1 - s) / tau) < 1e-9


def test_multihead_backward_sums_lambda(rng):
    q = rng.standard_normal((1, 2, 6, 3))
    k = rng.standard_normal((1, 2, 6, 3))
    v = rng.standard_normal((1, 2, 6, 3))
    dY = rng.standard_normal((1, 2, 6, 3))
    dq, dk, dv, dlam = oracle.relation_backward(q, k, v, dY, 0.5, 2.0, 0.3)
    tot = 0.0
    for h in range(2):
        r = oracle.relation_backward_head(q[0, h], k[0, h], v[0, h], dY[0, h], 0.5, 2.0, 0.3)
        tot += r["dlam"]
        assert np.array_equal(dq[0, h], r["dq"])
    assert dlam == tot


def test_decode_is_last_row_of_forward(rng):
    B, H, D, n, cap = 2, 3, 4, 9, 12
    kc = rng.standard_normal((B, H, cap, D))
    vc = rng.standard_normal((B, H, cap, D))
    q = rng.standard_normal((B, H, D))
    kn = rng.standard_normal((B, H, D))
    vn = rng.standard_normal((B, H, D))
    y, g, kc2, vc2 = oracle.relation_decode_step(q, kn, vn, kc, vc, n, 0.5, 2.0, 0.35)
    for b in range(B):
        for h in range(H):
            K = np.concatenate([kc[b, h, :n], kn[b, h][None]], 0)
            V = np.concatenate([vc[b, h, :n], vn[b, h][None]], 0)
            Q = rng.standard_normal((n + 1, D))
            Q[n] = q[b, h]
            r = oracle.relation_forward_head(Q, K, V, 0.5, 2.0, 0.35)
            assert np.abs(y[b, h] - r["Y"][n]).max() < 1e-14
            assert abs(g[b, h] - r["g"][n]) < 1e-14
            assert np.array_equal(kc2[b, h, : n + 1], K)
            assert np.array_equal(vc2[b, h, : n + 1], V)
    assert np.array_equal(kc2[:, :, n + 1:], kc[:, :, n + 1:])
    assert np.array_equal(vc2[:, :, n + 1:], vc[:, :, n + 1:])


def test_decode_ragged_rows_are_last_rows_of_their_forwards(rng):
    # each sequence's output is the last row of the forward over its own
    # history + new token, whatever the other sequences' lengths
    B, H, D, cap = 4, 2, 3, 11
    ns = [0, 10, 3, 7]
    kc = rng.standard_normal((B, H, cap, D))
    vc = rng.standard_normal((B, H, cap, D))
    q, kn, vn = (rng.standard_normal((B, H, D)) for _ in range(3))
    y, g, kc2, vc2 = oracle.relation_decode_step_ragged(q, kn, vn, kc, vc, ns, 0.5, 2.0, 0.35)
    for b, n in enumerate(ns):
        for h in range(H):
            K = np.concatenate([kc[b, h, :n], kn[b, h][None]], 0)
            V = np.concatenate([vc[b, h, :n], vn[b, h][None]], 0)
            Q = np.zeros((n + 1, D))
            Q[n] = q[b, h]
            r = oracle.relation_forward_head(Q, K, V, 0.5, 2.0, 0.35)
            assert np.abs(y[b, h] - r["Y"][n]).max() < 1e-14
            assert abs(g[b, h] - r["g"][n]) < 1e-14
            assert np.array_equal(kc2[b, h, : n + 1], K)
            assert np.array_equal(kc2[b, h, n + 1:], kc[b, h, n + 1:])
            assert np.array_equal(vc2[b, h, n + 1:], vc[b, h, n + 1:])


def test_prefill_rows_are_the_forwards_last_rows_and_m1_is_decode(rng):
    B, H, D, cap, m = 2, 2, 3, 14, 4
    ns = [5, 0]
    kc = rng.standard_normal((B, H, cap, D))
    vc = rng.standard_normal((B, H, cap, D))
    q, kn, vn = (rng.standard_normal((B, H, m, D)) for _ in range(3))
    y, lse, g, kc2, vc2 = oracle.relation_prefill_rows(q, kn, vn, kc, vc, ns, 0.5, 2.0, 0.35)
    for b, n in enumerate(ns):
        for h in range(H):
            K = np.concatenate([kc[b, h, :n], kn[b, h]], 0)
            V = np.concatenate([vc[b, h, :n], vn[b, h]], 0)
            Q = np.concatenate([rng.standard_normal((n, D)), q[b, h]], 0)
            r = oracle.relation_forward_head(Q, K, V, 0.5, 2.0, 0.35)
            assert np.abs(y[b, h] - r["Y"][n:]).max() < 1e-13
            assert np.abs(lse[b, h] - r["LSE"][n:]).max() < 1e-13
            assert np.abs(g[b, h] - r["g"][n:]).max() < 1e-13
            assert np.array_equal(kc2[b, h, :n + m], K)
            assert np.array_equal(kc2[b, h, n + m:], kc[b, h, n + m:])
    # one token at a time is the decode step
    y1, _, g1, _, _ = oracle.relation_prefill_rows(q[:, :, :1], kn[:, :, :1], vn[:, :, :1], kc,
                                                   vc, ns, 0.5, 2.0, 0.35)
    yd, gd, _, _ = oracle.relation_decode_step_ragged(q[:, :, 0], kn[:, :, 0], vn[:, :, 0], kc,
                                                      vc, ns, 0.5, 2.0, 0.35)
    assert np.abs(y1[:, :, 0] - yd).max() < 1e-14 and np.abs(g1[:, :, 0] - gd).max() < 1e-14


def test_decode_empty_history(rng):
    B, H, D = 1, 2, 3
    kc = rng.standard_normal((B, H, 4, D))
    vc = rng.standard_normal((B, H, 4, D))
    q, kn, vn = (rng.standard_normal((B, H, D)) for _ in range(3))
    y, g, _, _ = oracle.relation_decode_step(q, kn, vn, kc, vc, 0, 0.5, 2.0, 0.35)
    assert np.array_equal(y, vn) and np.all(g == 0.0)
