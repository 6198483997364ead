"""The Linear Relation pins can see plausible mistakes.

A copy of the oracle's recurrence (forward and reverse-mode backward) with
switchable planted mistakes replaces oracle.linear_relation_forward /
_backward while the independent pins of tests/test_oracle_linear.py run
(closed forms, strict history, state hand-off, RoPE invariants, finite
differences; not the comparison with the unrolled sum or the decode step,
which are the oracle's own second implementations). Unmutated, the copy
equals the oracle; each mutation must fail at least one pin.
"""
import numpy as np
import pytest

import oracle
from tests import test_oracle_linear as pins


def _sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def _coords(p1, p2, cos, sin, mut):
    x1 = np.asarray(p1, np.float64) if cos is None else oracle.rope_rotate(p1, cos, sin)
    x2 = np.asarray(p2, np.float64) if cos is None else oracle.rope_rotate(p2, cos, sin)
    return x1, x2


def _norm(x, mut):
    if mut == "no_normalise":
        return np.asarray(x, np.float64), np.ones(x.shape[:-1] + (1,))
    return oracle.linear_normalize(x)


def mutable_forward(mut):
    def fwd(p1, p2, I, g, scale, tau, cos=None, sin=None, C0=None):
        x1, x2 = _coords(p1, p2, cos, sin, mut)
        I, g = np.asarray(I, np.float64), np.asarray(g, np.float64)
        *lead, T, D = I.shape
        C = np.zeros((*lead, D, D)) if C0 is None else np.asarray(C0, np.float64).copy()
        S = _sig(scale * (x1 * x2).sum(-1) / (tau if mut != "drop_tau" else 1.0))
        h1, _ = _norm(x1, mut)
        h2, _ = _norm(x2, mut)
        E = np.zeros_like(I)
        for t in range(T):
            a = np.exp(g[..., t, :])
            if mut == "retention_on_value_channel":
                Cr = a[..., None, :] * C
            else:
                Cr = a[..., :, None] * C
            read = C if mut == "read_before_retention" else Cr
            if mut == "transposed_read":
                r = np.einsum("...kv,...v->...k", read, h1[..., t, :])
            else:
                r = np.einsum("...kv,...k->...v", read, h1[..., t, :])
            wS = S[..., t, None, None] if mut != "no_self_on_write" else 1.0
            Cn = Cr + wS * h2[..., t, :, None] * I[..., t, None, :]
            if mut == "read_after_write":
                r = np.einsum("...kv,...k->...v", Cn, h1[..., t, :])
            E[..., t, :] = S[..., t, None] * r
            C = Cn
        return {"Y": I + E, "E": E, "S": S, "C": C, "x1": x1, "x2": x2}
    return fwd


def mutable_backward(mut):
    def bwd(p1, p2, I, g, dY, scale, tau, cos=None, sin=None, C0=None, dC_T=None):
        x1, x2 = _coords(p1, p2, cos, sin, None)
        I, g, dY = (np.asarray(a, np.float64) for a in (I, g, dY))
        *lead, T, D = I.shape
        S = _sig(scale * (x1 * x2).sum(-1) / tau)
        h1, n1 = oracle.linear_normalize(x1)
        h2, n2 = oracle.linear_normalize(x2)
        al = np.exp(g)
        Cp = np.zeros((T, *lead, D, D))
        C = np.zeros((*lead, D, D)) if C0 is None else np.asarray(C0, np.float64).copy()
        for t in range(T):
            Cp[t] = C
            C = al[..., t, :, None] * C + S[..., t, None, None] * h2[..., t, :, None] * I[..., t, None, :]
        dC = np.zeros((*lead, D, D)) if dC_T is None else np.asarray(dC_T, np.float64).copy()
        dh1, dh2, dS, dI, dg = (np.zeros_like(h1), np.zeros_like(h2), np.zeros_like(S),
                                dY.copy(), np.zeros_like(g))
        for t in range(T - 1, -1, -1):
            St = S[..., t]
            Cr = al[..., t, :, None] * Cp[t]
            dCr = dC.copy()
            if mut != "drop_write_dS":
                dS[..., t] += np.einsum("...kv,...k,...v->...", dC, h2[..., t, :], I[..., t, :])
            dh2[..., t, :] = St[..., None] * np.einsum("...kv,...v->...k", dC, I[..., t, :])
            dI[..., t, :] += St[..., None] * np.einsum("...kv,...k->...v", dC, h2[..., t, :])
            dE = dY[..., t, :]
            dS[..., t] += (dE * np.einsum("...kv,...k->...v", Cr, h1[..., t, :])).sum(-1)
            dh1[..., t, :] = St[..., None] * np.einsum("...kv,...v->...k", Cr, dE)
            dCr += St[..., None, None] * h1[..., t, :, None] * dE[..., None, :]
            da = (dCr * Cp[t]).sum(-1)
            dg[..., t, :] = da * (al[..., t, :] if mut != "dg_without_alpha" else 1.0)
            dC = al[..., t, :, None] * dCr if mut != "state_grad_not_retained" else dCr
        dA = dS * S * (1 - S) * scale / tau

        def thr(dh, h, n):
            safe = np.where(n > 0, n, 1.0)
            if mut == "norm_grad_no_projection":
                return np.where(n > 0, dh / safe, 0.0)
            return np.where(n > 0, (dh - h * (h * dh).sum(-1, keepdims=True)) / safe, 0.0)

        dx1 = thr(dh1, h1, n1) + dA[..., None] * x2
        dx2 = thr(dh2, h2, n2) + dA[..., None] * x1
        if cos is not None:
            dx1 = oracle.rope_rotate_transpose(dx1, cos, sin)
            dx2 = oracle.rope_rotate_transpose(dx2, cos, sin)
        return dx1, dx2, dI, dg, dC
    return bwd


FWD_PINS = [
    pins.test_one_direction_no_retention_loss_is_a_cumulative_sum,
    pins.test_constant_retention_on_one_direction_is_geometric,
    pins.test_total_retention_loss_and_orthogonal_directions_give_no_exchange,
    pins.test_strict_history,
    pins.test_state_handoff_equals_one_pass,
    pins.test_rope_keeps_self_and_only_relative_positions_matter_with_uniform_retention,
]
FWD_MUTATIONS = ["drop_tau", "no_normalise", "retention_on_value_channel",
                 "read_before_retention", "transposed_read", "no_self_on_write",
                 "read_after_write"]
BWD_MUTATIONS = ["drop_write_dS", "dg_without_alpha", "state_grad_not_retained",
                 "norm_grad_no_projection"]


def _failures(fns):
    bad = 0
    for fn in fns:
        try:
            fn(np.random.default_rng(31415))
        except AssertionError:
            bad += 1
    return bad


def test_unmutated_copy_equals_oracle():
    rng = np.random.default_rng(5)
    p1, p2, I, g = pins.rand_inputs(rng, (2,), 7, 4)
    cs, sn = oracle.rope_tables(7, 4)
    C0 = rng.standard_normal((2, 4, 4))
    a = oracle.linear_relation_forward(p1, p2, I, g, 0.5, 2.0, cs, sn, C0=C0)
    b = mutable_forward(None)(p1, p2, I, g, 0.5, 2.0, cs, sn, C0=C0)
    assert np.array_equal(a["Y"], b["Y"]) and np.array_equal(a["C"], b["C"])
    W = rng.standard_normal(I.shape)
    ga = oracle.linear_relation_backward(p1, p2, I, g, W, 0.5, 2.0, cs, sn, C0=C0, dC_T=C0)
    gb = mutable_backward(None)(p1, p2, I, g, W, 0.5, 2.0, cs, sn, C0=C0, dC_T=C0)
    for x, y in zip(ga, gb):
        assert np.array_equal(x, y)


def test_unmutated_copy_passes_every_pin(monkeypatch):
    monkeypatch.setattr(oracle, "linear_relation_forward", mutable_forward(None))
    monkeypatch.setattr(oracle, "linear_relation_backward", mutable_backward(None))
    assert _failures(FWD_PINS) == 0
    for rope in (False, True):
        pins.test_backward_matches_finite_differences(np.random.default_rng(31415), rope)


@pytest.mark.parametrize("mut", FWD_MUTATIONS)
def test_forward_mutation_is_caught(mut, monkeypatch):
    monkeypatch.setattr(oracle, "linear_relation_forward", mutable_forward(mut))
    assert _failures(FWD_PINS) >= 1


@pytest.mark.parametrize("mut", BWD_MUTATIONS)
def test_backward_mutation_is_caught(mut, monkeypatch):
    monkeypatch.setattr(oracle, "linear_relation_backward", mutable_backward(mut))
    bad = 0
    for rope in (False, True):
        try:
            pins.test_backward_matches_finite_differences(np.random.default_rng(31415), rope)
        except AssertionError:
            bad += 1
    assert bad >= 1
