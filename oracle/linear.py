"""Plain fp64 CPU oracle of Linear Relation: the recurrent form of Relation in
which historical Others are compressed into a state with channel-wise
retention.

TEST INFRASTRUCTURE, like oracle/relation.py: only the test suite, the smoke
check and the benchmark's CPU-baseline leg may use it; it shares no code with
the HIP library.

Source: "Ask Self, Ask Others: Relation Is All You Need" (arXiv 2608.20172).
  - Sec. 5.2 (Change Exchange: Linear and Hybrid Relation): the Self map
    S_t = sigma(p1_t . p2_t / tau_S), the normalised coordinates
    p^_1 = p1 / ||p1||, p^_2 = p2 / ||p2||, the channel-wise retention
    alpha_t = exp(g_t) in (0, 1]^D, and the recurrent step
        E_t = S_t (Diag(alpha_t) C_{t-1})^T p^_{1,t}     (ask Others)
        Y_t = I_t + E_t                                  (answer)
        C_t = Diag(alpha_t) C_{t-1} + S_t p^_{2,t} I_t^T  (become Others)
    with C_0 = 0; the state is read before the current token is written, so
    Exchange is strictly historical.
  - App. A.4.1: RoPE is applied to p1 and p2 before S and the normalisation.
  - App. A.4.4-A.4.5: unrolled, the Exchange of row t is
        E_t = sum_{j<t} S_t S_j (p^_{1,t}^T (prod_{u=j+1..t} D_u) p^_{2,j}) I_j.
  - Sec. 5.2: the retention itself (g = -exp(A_log) * softplus(r + dt_bias),
    following KDA) is produced upstream from the token; the operator receives
    g = log alpha, one value per key channel per token.

Readings where the pages are silent or garbled (stated again where used):
  * The Self evidence is printed as p1 . p2 / (tau_S d_h); as for the Full
    Relation score, the page converter drops square roots, so the scale is an
    explicit argument (1/sqrt(d_h) in the callers):
    S_t = sigma(scale * p1_t . p2_t / tau_S).
  * A zero coordinate row has no direction: its normalised row is taken as
    zero (and passes no gradient through the normalisation).
  * The state is D x D with rows indexed by the key channel (the channel the
    retention acts on) and columns by the value channel.
  * RoPE is the rotate-half map of oracle/mhr.py with tables [T, D/2]; rows
    are positions 0..T-1 of the given tables.

Arithmetic is numpy float64; inputs are upcast from whatever exact values the
caller holds.
"""
import numpy as np

from .mhr import rope_rotate, rope_rotate_transpose

__all__ = [
    "linear_normalize",
    "linear_relation_forward",
    "linear_relation_unrolled",
    "linear_relation_step",
    "linear_relation_backward",
]


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def linear_normalize(x):
    """Rows of x [..., D] divided by their Euclidean norm (Sec. 5.2); a zero
    row stays zero (reading: it has no direction). Returns (x^, norm)."""
    x = _as64(x)
    n = np.sqrt((x * x).sum(axis=-1, keepdims=True))
    safe = np.where(n > 0, n, 1.0)
    return np.where(n > 0, x / safe, 0.0), n


def _coords(p1, p2, cos, sin):
    """RoPE (App. A.4.1) when tables are given, then Self and the
    normalised coordinates."""
    x1 = _as64(p1) if cos is None else rope_rotate(p1, cos, sin)
    x2 = _as64(p2) if cos is None else rope_rotate(p2, cos, sin)
    return x1, x2


def linear_relation_forward(p1, p2, I, g, scale, tau_s, cos=None, sin=None, C0=None):
    """Linear Relation by its recurrent step (Sec. 5.2), one token at a time.

    p1, p2, I, g: [..., T, D] (g = log alpha <= 0); C0: [..., D, D] initial
    state (None = 0). Returns dict(Y, E, S, C) with C the state after the
    last token, plus the rotated coordinates x1, x2."""
    x1, x2 = _coords(p1, p2, cos, sin)
    I, g = _as64(I), _as64(g)
    *lead, T, D = I.shape
    C = np.zeros((*lead, D, D)) if C0 is None else _as64(C0).copy()
    S = _sigmoid(scale * (x1 * x2).sum(axis=-1) / tau_s)  # [..., T]
    h1, _ = linear_normalize(x1)
    h2, _ = linear_normalize(x2)
    E = np.zeros_like(I)
    for t in range(T):
        alpha = np.exp(g[..., t, :])
        Cr = alpha[..., :, None] * C  # Diag(alpha_t) C_{t-1}
        E[..., t, :] = S[..., t, None] * np.einsum("...kv,...k->...v", Cr, h1[..., t, :])
        C = Cr + S[..., t, None, None] * h2[..., t, :, None] * I[..., t, None, :]
    return {"Y": I + E, "E": E, "S": S, "C": C, "x1": x1, "x2": x2}


def linear_relation_unrolled(p1, p2, I, g, scale, tau_s, cos=None, sin=None):
    """Exchange by the unrolled sum of App. A.4.5 (zero initial state): every
    historical token j < t contributes S_t S_j (p^_1t^T prod D_u p^_2j) I_j,
    the retention product taken over u = j+1..t as a product of alphas.
    Returns E [..., T, D]. O(T^2 D) per head: small inputs only."""
    x1, x2 = _coords(p1, p2, cos, sin)
    I, g = _as64(I), _as64(g)
    T = I.shape[-2]
    S = _sigmoid(scale * (x1 * x2).sum(axis=-1) / tau_s)
    h1, _ = linear_normalize(x1)
    h2, _ = linear_normalize(x2)
    alpha = np.exp(g)
    E = np.zeros_like(I)
    for t in range(T):
        for j in range(t):
            ret = np.prod(alpha[..., j + 1:t + 1, :], axis=-2)  # prod_{u=j+1..t} alpha_u
            w = S[..., t] * S[..., j] * (h1[..., t, :] * ret * h2[..., j, :]).sum(axis=-1)
            E[..., t, :] += w[..., None] * I[..., j, :]
    return E


def linear_relation_step(p1, p2, I, g, C, scale, tau_s, cos=None, sin=None):
    """One recurrent (decode) step of Sec. 5.2 for a single new token:
    p1, p2, I, g [..., D]; C [..., D, D] the state before it; cos, sin [D/2]
    the table row of the token's position (None = no RoPE).
    Returns (Y [..., D], C_new [..., D, D])."""
    x1 = _as64(p1)[..., None, :]
    x2 = _as64(p2)[..., None, :]
    if cos is not None:
        x1 = rope_rotate(x1, _as64(cos)[None, :], _as64(sin)[None, :])
        x2 = rope_rotate(x2, _as64(cos)[None, :], _as64(sin)[None, :])
    x1, x2 = x1[..., 0, :], x2[..., 0, :]
    S = _sigmoid(scale * (x1 * x2).sum(axis=-1) / tau_s)
    h1, _ = linear_normalize(x1)
    h2, _ = linear_normalize(x2)
    Cr = np.exp(_as64(g))[..., :, None] * _as64(C)
    E = S[..., None] * np.einsum("...kv,...k->...v", Cr, h1)
    I = _as64(I)
    return I + E, Cr + S[..., None, None] * h2[..., :, None] * I[..., None, :]


def linear_relation_backward(p1, p2, I, g, dY, scale, tau_s, cos=None, sin=None, C0=None,
                             dC_T=None):
    """Gradients of linear_relation_forward by reverse-mode through its
    recurrence, one token at a time from the last (the pages give no
    backward; this is the chain rule of the Sec. 5.2 step).

    dY: [..., T, D] gradient of Y; dC_T: [..., D, D] gradient of the final
    state (None = 0). Returns (dp1, dp2, dI, dg, dC0)."""
    x1, x2 = _coords(p1, p2, cos, sin)
    I, g, dY = _as64(I), _as64(g), _as64(dY)
    *lead, T, D = I.shape
    S = _sigmoid(scale * (x1 * x2).sum(axis=-1) / tau_s)
    h1, n1 = linear_normalize(x1)
    h2, n2 = linear_normalize(x2)
    alpha = np.exp(g)
    # the state before every token, C_{t-1}
    Cprev = np.zeros((T, *lead, D, D))
    C = np.zeros((*lead, D, D)) if C0 is None else _as64(C0).copy()
    for t in range(T):
        Cprev[t] = C
        C = alpha[..., t, :, None] * C + S[..., t, None, None] * h2[..., t, :, None] * I[..., t, None, :]
    dC = np.zeros((*lead, D, D)) if dC_T is None else _as64(dC_T).copy()
    dh1, dh2 = np.zeros_like(h1), np.zeros_like(h2)
    dS = np.zeros_like(S)
    dI = dY.copy()  # Y_t = I_t + E_t
    dg = np.zeros_like(g)
    for t in range(T - 1, -1, -1):
        St = S[..., t]
        Cr = alpha[..., t, :, None] * Cprev[t]
        # C_t = Cr + S_t p^_2t I_t^T
        dCr = dC.copy()
        dS[..., t] += np.einsum("...kv,...k,...v->...", dC, h2[..., t, :], I[..., t, :])
        dh2[..., t, :] = St[..., None] * np.einsum("...kv,...v->...k", dC, I[..., t, :])
        dI[..., t, :] += St[..., None] * np.einsum("...kv,...k->...v", dC, h2[..., t, :])
        # E_t = S_t Cr^T p^_1t
        dE = dY[..., t, :]
        dS[..., t] += (dE * np.einsum("...kv,...k->...v", Cr, h1[..., t, :])).sum(axis=-1)
        dh1[..., t, :] = St[..., None] * np.einsum("...kv,...v->...k", Cr, dE)
        dCr += St[..., None, None] * h1[..., t, :, None] * dE[..., None, :]
        # Cr = Diag(alpha_t) C_{t-1}, alpha_t = exp(g_t)
        dalpha = (dCr * Cprev[t]).sum(axis=-1)
        dg[..., t, :] = dalpha * alpha[..., t, :]
        dC = alpha[..., t, :, None] * dCr
    # S_t = sigma(scale * x1_t . x2_t / tau)
    da = dS * S * (1.0 - S) * scale / tau_s
    # x^ = x / ||x||: dx = (dx^ - x^ (x^ . dx^)) / ||x||, zero for a zero row
    def through_norm(dh, h, n):
        safe = np.where(n > 0, n, 1.0)
        return np.where(n > 0, (dh - h * (h * dh).sum(axis=-1, keepdims=True)) / safe, 0.0)

    dx1 = through_norm(dh1, h1, n1) + da[..., None] * x2
    dx2 = through_norm(dh2, h2, n2) + da[..., None] * x1
    if cos is not None:
        dx1 = rope_rotate_transpose(dx1, cos, sin)
        dx2 = rope_rotate_transpose(dx2, cos, sin)
    return dx1, dx2, dI, dg, dC
