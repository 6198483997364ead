"""The oracle's pins can see plausible mistakes.

A copy of the oracle's forward / backward with switchable planted mistakes is
run through the independent pins of tests/oracle_pins.py (invariants, closed
forms, causality, lambda-invariance of the allocation, finite differences,
App. A.1.7 identities; not the brute-force comparison, which is the oracle's
own second implementation). Unmutated, the copy equals the oracle exactly;
each mutation must fail at least one pin.
"""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as P


def _sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def mutable_forward(mut):
    def fwd(q, k, v, scale, tau, lam):
        q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
        T = q.shape[0]
        U = scale * (q @ k.T) if mut != "transposed_U" else scale * (k @ q.T)
        d = np.arange(T)
        strict = np.tril(np.ones((T, T), bool), -1)
        rows = np.arange(1, T + 1, dtype=np.float64)
        if mut == "log_off_by_one":
            rows = rows + 1.0
        S = _sig(U[d, d] / (tau if mut != "drop_tau" else 1.0))
        if mut == "self_is_silu":
            S = U[d, d] * _sig(U[d, d])
        E = U * _sig(U) if mut != "exchange_identity" else U.copy()
        sign = -1.0 if mut != "correction_sign" else 1.0
        R = np.full((T, T), -np.inf)
        R[strict] = (E + sign * lam * np.log(rows)[:, None])[strict]
        R[d, d] = S if mut != "lambda_on_self" else S - lam * np.log(rows)
        if mut == "non_strict_mask":
            R[0, 1] = E[0, 1]
        W = np.exp(R - R.max(1, keepdims=True))
        F = W / W.sum(1, keepdims=True)
        Y = F @ v if mut != "transposed_F" else F.T @ v
        LSE = R.max(1) + np.log(W.sum(1))
        g = np.where(strict, F, 0.0).sum(1)
        return {"U": U, "S": S, "E": E, "R": R, "F": F, "Y": Y, "LSE": LSE, "g": g}
    return fwd


def mutable_backward(mut):
    fwd = mutable_forward(None)

    def bwd(q, k, v, dY, scale, tau, lam):
        fw = fwd(q, k, v, scale, tau, lam)
        U, F, S = fw["U"], fw["F"], fw["S"]
        T = U.shape[0]
        strict = np.tril(np.ones((T, T), bool), -1)
        d = np.arange(T)
        Hm = dY @ v.T
        dv = F.T @ dY if mut != "dv_untransposed" else F @ dY
        dR = F * (Hm - (F * Hm).sum(1, keepdims=True))
        sg = _sig(U)
        dsilu = sg * (1 + U * (1 - sg)) if mut != "silu_grad_drop_term" else sg
        dU = np.zeros((T, T))
        dU[strict] = (dR * dsilu)[strict]
        dU[d, d] = dR[d, d] * S * (1 - S) / (tau if mut != "self_grad_drop_tau" else 1.0)
        dq = scale * dU @ k
        dk = scale * dU.T @ q if mut != "dk_untransposed" else scale * dU @ q
        logi = np.log(np.arange(1, T + 1, dtype=np.float64))[:, None]
        sgn = -1.0 if mut != "dlam_sign" else 1.0
        dlam = float(sgn * (np.where(strict, dR, 0.0) * logi).sum())
        return {"dq": dq, "dk": dk, "dv": dv, "dlam": dlam, "dR": dR, "fwd": fw}
    return bwd


FWD_MUTATIONS = ["transposed_U", "log_off_by_one", "drop_tau", "self_is_silu",
                 "exchange_identity", "correction_sign", "lambda_on_self",
                 "non_strict_mask", "transposed_F"]
BWD_MUTATIONS = ["dv_untransposed", "silu_grad_drop_term", "self_grad_drop_tau",
                 "dk_untransposed", "dlam_sign"]


def _forward_pin_failures(fwd):
    rng = np.random.default_rng(7)
    fails = []
    if P.check_invariants(fwd, rng) > 1e-10:
        fails.append("invariants")
    err, moves = P.check_lambda_allocation(fwd, rng)
    if err > 1e-10 or moves < 1e-6:
        fails.append("lambda_allocation")
    for which in ("q", "k"):
        if P.check_closed_form_zero_evidence(fwd, rng, which=which) > 1e-10:
            fails.append("closed_form_" + which)
    if P.check_closed_form_T2(fwd) > 1e-12:
        fails.append("closed_form_T2")
    if P.check_causality(fwd, rng) != 0.0:
        fails.append("causality")
    return fails


def test_unmutated_copy_equals_oracle():
    rng = np.random.default_rng(3)
    q, k, v = P.rand_head(rng, 9, 4)
    a = mutable_forward(None)(q, k, v, 0.5, 2.0, 0.3)
    b = oracle.relation_forward_head(q, k, v, 0.5, 2.0, 0.3)
    assert np.abs(a["Y"] - b["Y"]).max() < 1e-15
    assert _forward_pin_failures(mutable_forward(None)) == []
    dY = rng.standard_normal((9, 4))
    c = mutable_backward(None)(q, k, v, dY, 0.5, 2.0, 0.3)
    d = oracle.relation_backward_head(q, k, v, dY, 0.5, 2.0, 0.3)
    assert np.abs(c["dq"] - d["dq"]).max() < 1e-14
    assert abs(c["dlam"] - d["dlam"]) < 1e-13


@pytest.mark.parametrize("mut", FWD_MUTATIONS)
def test_forward_mutation_is_caught(mut):
    assert _forward_pin_failures(mutable_forward(mut)), f"no pin catches {mut}"


@pytest.mark.parametrize("mut", BWD_MUTATIONS)
def test_backward_mutation_is_caught(mut):
    rng = np.random.default_rng(11)
    fwd = mutable_forward(None)
    bwd = mutable_backward(mut)
    fd = P.check_backward_fd(fwd, bwd, rng)
    ident = P.check_backward_identities(bwd, rng)
    assert fd > 1e-6 or ident > 1e-10, f"no pin catches {mut}"
