"""Plain fp64 CPU oracle of the Multi-Head Relation token-mixing core with its
two upstream maps: rotary position encoding of p1 and p2, and the alternating
Givens mixing of the information slices.

TEST INFRASTRUCTURE, like oracle/relation.py: only the test suite, the smoke
check and the benchmark's CPU-baseline leg may use it; it shares no code with
the HIP library.

Source: "Ask Self, Ask Others: Relation Is All You Need" (arXiv 2608.20172).
  - Sec. 3.1: p1 and p2 are rotated by RoPE before the pairwise evidence U;
    the information state I is not rotated.
  - App. B.3 (training setup): RoPE covers the full head dimension with base
    1e4 and no scaling.
  - Sec. 3.2 and App. A.2.2-A.2.3: the head-wise information slices are mixed
    pairwise by Givens rotations G(theta) = [[cos, sin], [-sin, cos]] acting
    on [I^(a); I^(b)], with the pairing M_A = {(1,2), (3,4), ...} or
    M_B = {(2,3), ..., (H,1)} alternating between layers; each head's
    transport then uses its mixed slice, Y^(h) = F^(h) I^(h).

Readings where the pages are silent (stated again in the functions):
  * RoPE pairs element d with element d + D/2 (rotate-half) and uses the
    frequency base^(-2j/D) for pair j; the row at 1-based position i has
    position index i - 1. The tables cos, sin [T, D/2] are arguments, so
    callers can offset or extend positions.
  * One angle per pair per layer; theta[p] belongs to the p-th pair in the
    listed order of M_A or M_B. H must be even.
  * The mixed slice enters both the Exchange transport and the Self term
    (Y_i = (1 - g_i) I'_i + g_i Ibar_i): it is the only I the head sees.

Arithmetic is numpy float64.
"""
import numpy as np

from .relation import relation_backward, relation_forward

__all__ = [
    "rope_tables",
    "rope_rotate",
    "rope_rotate_transpose",
    "givens_pairs",
    "givens_mix",
    "givens_mix_transpose",
    "relation_mhr_forward",
    "relation_mhr_backward",
]


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def rope_tables(T, D, base=1.0e4):
    """cos / sin [T, D/2] of angle (position t) * base^(-2j/D), t = 0..T-1
    (App. B.3: full head, base 1e4, no scaling)."""
    j = np.arange(D // 2, dtype=np.float64)
    ang = np.arange(T, dtype=np.float64)[:, None] * base ** (-2.0 * j / D)[None, :]
    return np.cos(ang), np.sin(ang)


def rope_rotate(x, cos, sin):
    """RoPE applied to x [..., T, D] with tables [T, D/2] (Sec. 3.1): each
    pair (x_d, x_{d+D/2}) is rotated by the angle of its row and index d."""
    x, c, s = _as64(x), _as64(cos), _as64(sin)
    h = x.shape[-1] // 2
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def rope_rotate_transpose(g, cos, sin):
    """The transpose (inverse) of rope_rotate: maps a gradient with respect
    to the rotated tensor to the gradient with respect to its input."""
    g, c, s = _as64(g), _as64(cos), _as64(sin)
    h = g.shape[-1] // 2
    a, b = g[..., :h], g[..., h:]
    return np.concatenate([a * c + b * s, -a * s + b * c], axis=-1)


def givens_pairs(H, pairing):
    """0-based head pairs of App. A.2.3: pairing 0 is M_A = (1,2), (3,4), ...,
    pairing 1 is M_B = (2,3), (4,5), ..., (H,1)."""
    if H % 2:
        raise ValueError("Givens pairing needs an even head count")
    if pairing == 0:
        return [(2 * p, 2 * p + 1) for p in range(H // 2)]
    return [(2 * p + 1, (2 * p + 2) % H) for p in range(H // 2)]


def givens_mix(I, theta, pairing):
    """Mixed information slices (Sec. 3.2; App. A.2.2): for every pair (a, b)
    with angle theta_p, I'^(a) = cos I^(a) + sin I^(b) and
    I'^(b) = -sin I^(a) + cos I^(b). I: [B, H, T, D]."""
    I = _as64(I)
    out = I.copy()
    for p, (a, b) in enumerate(givens_pairs(I.shape[1], pairing)):
        c, s = np.cos(theta[p]), np.sin(theta[p])
        out[:, a] = c * I[:, a] + s * I[:, b]
        out[:, b] = -s * I[:, a] + c * I[:, b]
    return out


def givens_mix_transpose(dIm, Im, theta, pairing):
    """Chain rule through givens_mix: from dL/dI' (and the mixed I') returns
    (dL/dI, dL/dtheta). The rotation's transpose undoes the mixing of the
    gradient; d I'^(a)/d theta = I'^(b) and d I'^(b)/d theta = -I'^(a), so
    dL/dtheta_p = sum(dI'^(a) I'^(b) - dI'^(b) I'^(a))."""
    dIm, Im = _as64(dIm), _as64(Im)
    dI = dIm.copy()
    dth = np.zeros(len(theta))
    for p, (a, b) in enumerate(givens_pairs(dIm.shape[1], pairing)):
        c, s = np.cos(theta[p]), np.sin(theta[p])
        dI[:, a] = c * dIm[:, a] - s * dIm[:, b]
        dI[:, b] = s * dIm[:, a] + c * dIm[:, b]
        dth[p] = float((dIm[:, a] * Im[:, b]).sum() - (dIm[:, b] * Im[:, a]).sum())
    return dI, dth


def relation_mhr_forward(p1, p2, I, cos, sin, theta, pairing, scale, tau_s, lam):
    """Multi-Head Relation with its upstream maps: q = RoPE(p1), k = RoPE(p2),
    I' = Givens(I), then the Relation operator per head (Sec. 3.1-3.2).
    theta None skips the mixing; cos None skips RoPE.
    Returns dict(Y, LSE, g, q, k, v) with the rotated / mixed tensors."""
    q = _as64(p1) if cos is None else rope_rotate(p1, cos, sin)
    k = _as64(p2) if cos is None else rope_rotate(p2, cos, sin)
    v = _as64(I) if theta is None else givens_mix(I, theta, pairing)
    Y, LSE, g = relation_forward(q, k, v, scale, tau_s, lam)
    return {"Y": Y, "LSE": LSE, "g": g, "q": q, "k": k, "v": v}


def relation_mhr_backward(p1, p2, I, dY, cos, sin, theta, pairing, scale, tau_s, lam):
    """Gradients of relation_mhr_forward: the Relation backward (App. A.1.7)
    on the rotated / mixed tensors, then the transposes of RoPE and of the
    Givens mixing. Returns (dp1, dp2, dI, dlambda, dtheta or None)."""
    f = relation_mhr_forward(p1, p2, I, cos, sin, theta, pairing, scale, tau_s, lam)
    dq, dk, dv, dlam = relation_backward(f["q"], f["k"], f["v"], dY, scale, tau_s, lam)
    dp1 = dq if cos is None else rope_rotate_transpose(dq, cos, sin)
    dp2 = dk if cos is None else rope_rotate_transpose(dk, cos, sin)
    if theta is None:
        return dp1, dp2, dv, dlam, None
    dI, dth = givens_mix_transpose(dv, f["v"], theta, pairing)
    return dp1, dp2, dI, dlam, dth
