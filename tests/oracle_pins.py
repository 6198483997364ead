"""Checks that pin the fp64 oracle to facts other than itself.

Each check takes the forward (and, where needed, the backward) as a function
argument so the same check can be run against the oracle (it must pass) and
against deliberately broken copies of it (tests/test_oracle_mutations.py: at
least one check must fail), which shows the checks can see the mistakes.

Sources (arXiv 2608.20172, "Ask Self, Ask Others: Relation Is All You Need"):
  Sec. 3.1   definitions of U, S, E, R, F, Y
  Sec. 4.2   F_ii + g_i = 1, F_ii = sigmoid(S_i - A_i), F_ij = g_i pi_ij,
             Y_i = I_i + g_i Delta_i with 0 <= g_i <= 1
  Sec. 4.3   log(g_i / F_ii) = A_i - S_i; lambda leaves pi unchanged
  App. A.1.2 Z_i = e^{S_i} + i^{-lambda} sum_{j<i} e^{E_ij}
  App. A.1.7 dL/dS_i = -g_i (1 - g_i) c_i, dS_i/dU_ii = S_i (1 - S_i) / tau_S
  App. A.1.8 row 1: A_1 = -inf
"""
import math

import numpy as np
from scipy.special import logsumexp, softmax


def rand_head(rng, T, D, Dv=None, std=1.0):
    Dv = D if Dv is None else Dv
    q = rng.standard_normal((T, D)) * std
    k = rng.standard_normal((T, D)) * std
    v = rng.standard_normal((T, Dv))
    return q, k, v


def check_brute_force(fwd, brute, rng, T=7, D=3, scale=0.6, tau=2.0, lam=0.37):
    """Vectorised forward == scalar-loop forward entry by entry."""
    q, k, v = rand_head(rng, T, D)
    r = fwd(q, k, v, scale, tau, lam)
    Yb, Lb, gb = brute(q.tolist(), k.tolist(), v.tolist(), scale, tau, lam)
    return max(np.abs(r["Y"] - np.array(Yb)).max(),
               np.abs(r["LSE"] - np.array(Lb)).max(),
               np.abs(r["g"] - np.array(gb)).max())


def check_invariants(fwd, rng, T=9, D=4, scale=0.5, tau=2.0, lam=0.6):
    """Largest violation of the pages' exact identities of Flow (Sec. 4.2,
    Sec. 4.3, App. A.1.2), each evaluated with library routines (scipy's
    logsumexp / softmax) independent of the oracle's own arithmetic."""
    q, k, v = rand_head(rng, T, D)
    r = fwd(q, k, v, scale, tau, lam)
    F, Y, g, LSE = r["F"], r["Y"], r["g"], r["LSE"]
    U = scale * (q @ k.T)
    S = 1.0 / (1.0 + np.exp(-np.diag(U) / tau))
    E = U / (1.0 + np.exp(-U))
    errs = []
    errs.append(np.abs(F.sum(axis=1) - 1.0).max())                 # rows of F sum to 1
    errs.append(np.abs(np.triu(F, 1)).max())                        # causal
    errs.append(np.abs(np.diag(F) + g - 1.0).max())                 # F_ii + g_i = 1
    i1 = np.arange(1, T + 1)
    for i in range(2, T + 1):
        hist = E[i - 1, : i - 1]
        A = logsumexp(hist) - lam * math.log(i)
        Fii = 1.0 / (1.0 + math.exp(-(S[i - 1] - A)))               # sigmoid(S - A)
        errs.append(abs(F[i - 1, i - 1] - Fii))
        errs.append(abs(math.log(g[i - 1] / F[i - 1, i - 1]) - (A - S[i - 1])))
        Z = math.exp(S[i - 1]) + i ** (-lam) * np.exp(hist).sum()  # App. A.1.2
        errs.append(abs(LSE[i - 1] - math.log(Z)))
        pi = softmax(hist)                                          # allocation
        errs.append(np.abs(F[i - 1, : i - 1] - g[i - 1] * pi).max())
        Ibar = pi @ v[: i - 1]
        errs.append(np.abs(Y[i - 1] - (v[i - 1] + g[i - 1] * (Ibar - v[i - 1]))).max())
    errs.append(abs(F[0, 0] - 1.0))                                 # row 1 is all Self
    errs.append(abs(g[0]))
    errs.append(np.abs(Y[0] - v[0]).max())
    errs.append(abs(LSE[0] - S[0]))
    bad_range = float(((g < 0) | (g > 1)).any())
    errs.append(bad_range)
    del i1
    return max(errs)


def check_lambda_allocation(fwd, rng, T=8, D=3, scale=0.7, tau=2.0):
    """pi_ij = F_ij / g_i does not depend on lambda (Sec. 4.3), while g does."""
    q, k, v = rand_head(rng, T, D)
    pis = []
    gs = []
    for lam in (0.0, 0.8, -0.5, 2.0):
        r = fwd(q, k, v, scale, tau, lam)
        F, g = r["F"], r["g"]
        pi = np.zeros_like(F)
        for i in range(1, T):
            pi[i, :i] = F[i, :i] / g[i]
        pis.append(pi)
        gs.append(g)
    err = max(np.abs(p - pis[0]).max() for p in pis[1:])
    g_moves = min(np.abs(gg[1:] - gs[0][1:]).max() for gg in gs[1:])
    return err, g_moves


def check_closed_form_zero_evidence(fwd, rng, T=11, D=4, tau=2.0, lam=0.45, which="q"):
    """q = 0 (or k = 0) makes U = 0, so S_i = sigmoid(0) = 1/2, E_ij = 0 and
    R_ij = -lambda log i. Then
      g_i = (i-1) i^-lambda / (e^{1/2} + (i-1) i^-lambda),
      Y_i = (1 - g_i) v_i + g_i * mean_{j<i} v_j,
    LSE_i = log(e^{1/2} + (i-1) i^-lambda) (derived from Sec. 3.1)."""
    q, k, v = rand_head(rng, T, D)
    if which == "q":
        q[:] = 0.0
    else:
        k[:] = 0.0
    r = fwd(q, k, v, 0.9, tau, lam)
    errs = []
    for i in range(1, T + 1):
        hist = (i - 1) * i ** (-lam)
        Z = math.exp(0.5) + hist
        gi = hist / Z
        ybar = v[: i - 1].mean(axis=0) if i > 1 else np.zeros(D)
        yi = (1 - gi) * v[i - 1] + gi * ybar
        errs.append(abs(r["g"][i - 1] - gi))
        errs.append(np.abs(r["Y"][i - 1] - yi).max())
        errs.append(abs(r["LSE"][i - 1] - math.log(Z)))
    return max(errs)


def check_closed_form_T2(fwd, scale=1.0, tau=2.0, lam=0.3):
    """T = 2, D = 1 by hand: U = [[a*c, a*d], [b*c, b*d]] for q = (a, b),
    k = (c, d). Row 2 has one historical entry, so
      g_2 = e^{E21 - lam log 2} / (e^{S_2} + e^{E21 - lam log 2}),
      Y_2 = (1 - g_2) v_2 + g_2 v_1, with S_2 = 1/(1+e^{-b d / tau}) and
      E21 = b c / (1 + e^{-b c})."""
    a, b, c, d = 0.7, -1.3, 2.1, 0.4
    v1, v2 = 1.5, -0.25
    q = np.array([[a], [b]])
    k = np.array([[c], [d]])
    v = np.array([[v1], [v2]])
    r = fwd(q, k, v, scale, tau, lam)
    S1 = 1 / (1 + math.exp(-scale * a * c / tau))
    S2 = 1 / (1 + math.exp(-scale * b * d / tau))
    u21 = scale * b * c
    E21 = u21 / (1 + math.exp(-u21))
    R21 = E21 - lam * math.log(2)
    g2 = math.exp(R21) / (math.exp(S2) + math.exp(R21))
    y2 = (1 - g2) * v2 + g2 * v1
    return max(abs(r["Y"][0, 0] - v1), abs(r["g"][0]), abs(r["LSE"][0] - S1),
               abs(r["Y"][1, 0] - y2), abs(r["g"][1] - g2),
               abs(r["LSE"][1] - math.log(math.exp(S2) + math.exp(R21))))


def check_causality(fwd, rng, T=10, D=3):
    """Changing token t (q, k or v) leaves rows < t bit-identical."""
    q, k, v = rand_head(rng, T, D)
    base = fwd(q, k, v, 0.5, 2.0, 0.3)
    worst = 0.0
    for t in (3, 6, 9):
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        q2[t] += 1.0
        k2[t] -= 2.0
        v2[t] *= 3.0
        r = fwd(q2, k2, v2, 0.5, 2.0, 0.3)
        worst = max(worst, np.abs(r["Y"][:t] - base["Y"][:t]).max(),
                    np.abs(r["LSE"][:t] - base["LSE"][:t]).max())
        if np.abs(r["Y"][t] - base["Y"][t]).max() == 0.0:
            worst = max(worst, 1.0)  # row t itself must move
    return worst


def finite_difference_grads(fwd, q, k, v, dY, scale, tau, lam, h=1e-6):
    """Central differences of L = sum(Y * dY) w.r.t. every entry of q, k, v
    and lambda, through the forward alone."""
    def loss(q_, k_, v_, lam_):
        return float((fwd(q_, k_, v_, scale, tau, lam_)["Y"] * dY).sum())

    grads = []
    for which in range(3):
        base = [q, k, v][which]
        gr = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            gr[idx] = (loss(*args_p, lam) - loss(*args_m, lam)) / (2 * h)
        grads.append(gr)
    dlam = (loss(q, k, v, lam + h) - loss(q, k, v, lam - h)) / (2 * h)
    return grads[0], grads[1], grads[2], dlam


def check_backward_fd(fwd, bwd, rng, T=6, D=3, scale=0.8, tau=2.0, lam=0.55):
    q, k, v = rand_head(rng, T, D)
    dY = rng.standard_normal((T, D))
    r = bwd(q, k, v, dY, scale, tau, lam)
    fq, fk, fv, flam = finite_difference_grads(fwd, q, k, v, dY, scale, tau, lam)
    return max(np.abs(r["dq"] - fq).max(), np.abs(r["dk"] - fk).max(),
               np.abs(r["dv"] - fv).max(), abs(r["dlam"] - flam))


def check_backward_identities(bwd, rng, T=9, D=4, scale=0.6, tau=2.0, lam=0.4):
    """App. A.1.7: dL/dS_i = -g_i(1-g_i) c_i with c_i = G_i . Delta_i, and
    the rows of dL/dR sum to zero."""
    q, k, v = rand_head(rng, T, D)
    dY = rng.standard_normal((T, D))
    r = bwd(q, k, v, dY, scale, tau, lam)
    dR, fw = r["dR"], r["fwd"]
    F, g = fw["F"], fw["g"]
    errs = [np.abs(dR.sum(axis=1)).max()]
    for i in range(2, T + 1):
        pi = F[i - 1, : i - 1] / g[i - 1]
        delta = pi @ v[: i - 1] - v[i - 1]
        c = dY[i - 1] @ delta
        errs.append(abs(dR[i - 1, i - 1] - (-g[i - 1] * (1 - g[i - 1]) * c)))
    return max(errs)
