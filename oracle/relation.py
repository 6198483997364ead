"""Plain fp64 CPU oracle of the exact causal Full / Multi-Head Relation operator.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module. The product path (the HIP library and
its Python binding) never calls it, and it shares no code with that path.

Source: "Ask Self, Ask Others: Relation Is All You Need" (arXiv 2608.20172).
Every function cites the passage it follows:
  - Sec. 3.1 (Self-Exchange Relation): U, the Self map S, the Exchange map E,
    the count correction -lambda*log i, the causal Relation matrix R, the Flow
    F = Softmax(R) and the transport Y = F I.
  - Sec. 3.2 / App. A.2: every head builds its own R and F independently.
  - Sec. 4.2 / App. A.1.2-A.1.6: L^E, A, Z, F_ii, g, pi^E, Ibar^E, Delta^E.
  - Sec. 5.1 / App. A.3: the FlashRelation (m, l, z) scan.
  - App. A.1.7: backward credit decomposition.
  - App. A.1.8: the empty-history boundary of row 1.

Readings where the pages are silent or garbled (each is stated again where it
is used):
  * The extracted text prints the pairwise evidence as q.k / d_h; the page
    converter drops square roots, so the scale is an explicit argument
    (default 1/sqrt(d_h) in the callers).
  * Rows are 1-based in the maths (i = 1..T); log is the natural log.
  * -lambda*log i is added to historical entries j < i only, never to Self.
  * Row 1 has no history: A_1 = -inf, so g_1 = 0 and Y_1 = I_1.

Arithmetic is numpy float64 throughout; inputs are upcast to float64 from
whatever exact values the caller holds (e.g. bf16-rounded tensors).
"""
import math

import numpy as np

__all__ = [
    "sigmoid",
    "silu",
    "relation_forward_head",
    "relation_forward",
    "relation_forward_rows",
    "relation_backward_head",
    "relation_backward",
    "relation_decode_step",
    "relation_decode_step_ragged",
    "relation_prefill_rows",
    "brute_force_forward_head",
    "tiled_forward_head",
]


def sigmoid(x):
    """Logistic function, evaluated without overflow for either sign of x."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def silu(x):
    """SiLU(u) = u * sigmoid(u): the Exchange map of Sec. 3.1."""
    x = np.asarray(x, dtype=np.float64)
    return x * sigmoid(x)


def _as64(a):
    return np.asarray(a, dtype=np.float64)


def relation_forward_head(q, k, v, scale, tau_s, lam):
    """Materialised forward of one head (Sec. 3.1; Sec. 4.2).

    q, k, v: [T, D] (p_1, p_2 and I of the pages, already RoPE'd / mixed).
    Returns a dict with the T x T matrices U, E, R, F, the per-row S, LSE
    (= log Z_i), g (Exchange mass), and the output Y [T, D].
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    T = q.shape[0]
    # Pairwise evidence U_ij = scale * p1_i . p2_j (Sec. 3.1).
    U = scale * (q @ k.T)
    rows = np.arange(1, T + 1, dtype=np.float64)          # 1-based i
    diag = np.arange(T)
    strict = np.tril(np.ones((T, T), dtype=bool), k=-1)   # j < i
    # Self S_i = sigmoid(U_ii / tau_S); Exchange E_ij = SiLU(U_ij) (Sec. 3.1).
    S = sigmoid(U[diag, diag] / tau_s)
    E = silu(U)
    # Causal Relation matrix: S_i on the diagonal, E_ij - lambda log i below,
    # -inf above (Sec. 3.1, the piecewise definition of R).
    R = np.full((T, T), -np.inf)
    corr = lam * np.log(rows)[:, None]
    R[strict] = (E - corr)[strict]
    R[diag, diag] = S
    # Flow F_i = Softmax(R_i) (Sec. 3.1), with the usual max shift.
    rmax = R.max(axis=1, keepdims=True)
    W = np.exp(R - rmax)
    Z = W.sum(axis=1, keepdims=True)
    F = W / Z
    # Transport Y_i = sum_{j<=i} F_ij I_j (Sec. 3.1).
    Y = F @ v
    LSE = rmax[:, 0] + np.log(Z[:, 0])
    # Exchange mass g_i = sum_{j<i} F_ij (Sec. 4.2).
    g = np.where(strict, F, 0.0).sum(axis=1)
    return {"U": U, "S": S, "E": E, "R": R, "F": F, "Y": Y, "LSE": LSE, "g": g}


def relation_forward(q, k, v, scale, tau_s, lam):
    """Multi-Head Relation forward over [B, H, T, D] inputs (Sec. 3.2, App.
    A.2.1: each head independently).  Returns (Y, LSE, g) as float64 arrays
    of shapes [B,H,T,D], [B,H,T], [B,H,T]."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, T, D = q.shape
    Y = np.empty((B, H, T, v.shape[-1]))
    LSE = np.empty((B, H, T))
    g = np.empty((B, H, T))
    for b in range(B):
        for h in range(H):
            r = relation_forward_head(q[b, h], k[b, h], v[b, h], scale, tau_s, lam)
            Y[b, h], LSE[b, h], g[b, h] = r["Y"], r["LSE"], r["g"]
    return Y, LSE, g


def relation_forward_rows(q, k, v, rows, scale, tau_s, lam):
    """Selected rows of one head's forward, each straight from the definition
    (Sec. 3.1): row i (1-based) needs only p1_i and p2_j, I_j for j <= i.

    q, k, v: [T, D]; rows: iterable of 1-based row indices.
    Returns (Y [len(rows), D], LSE [len(rows)], g [len(rows)]).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    ys, lses, gs = [], [], []
    for i in rows:
        i = int(i)
        u = scale * (k[:i] @ q[i - 1])                     # U_ij, j = 1..i
        s_self = float(sigmoid(np.array([u[i - 1] / tau_s]))[0])
        r = np.empty(i)
        r[: i - 1] = silu(u[: i - 1]) - lam * math.log(i)   # historical entries
        r[i - 1] = s_self                                   # Self entry
        rmax = r.max()
        w = np.exp(r - rmax)
        z = w.sum()
        f = w / z
        ys.append(f @ v[:i])
        lses.append(rmax + math.log(z))
        gs.append(f[: i - 1].sum())
    return np.array(ys), np.array(lses), np.array(gs)


def relation_backward_head(q, k, v, dY, scale, tau_s, lam):
    """Materialised backward of one head: the chain rule through the
    definitions of Sec. 3.1, organised as in App. A.1.7.

    G_i = dL/dY_i; H_ij = G_i . I_j is dL/dF_ij; the softmax Jacobian gives
    dL/dR_ij = F_ij (H_ij - sum_k F_ik H_ik); then
      j < i : dL/dU_ij = dL/dR_ij * SiLU'(U_ij),
              SiLU'(u) = sigmoid(u) (1 + u (1 - sigmoid(u)))
      j = i : dL/dU_ii = dL/dR_ii * S_i (1 - S_i) / tau_S  (App. A.1.7)
      dL/dlambda = sum_{j<i} dL/dR_ij * (-log i)
    and U = scale * q k^T, Y = F I give dq, dk, dv.
    Returns dict(dq, dk, dv, dlam, dR, fwd).
    """
    q, k, v, dY = _as64(q), _as64(k), _as64(v), _as64(dY)
    T = q.shape[0]
    fw = relation_forward_head(q, k, v, scale, tau_s, lam)
    U, F, S = fw["U"], fw["F"], fw["S"]
    strict = np.tril(np.ones((T, T), dtype=bool), k=-1)
    diag = np.arange(T)
    Hm = dY @ v.T                       # H_ij = G_i . I_j (App. A.1.7)
    dv = F.T @ dY
    rowterm = (F * Hm).sum(axis=1, keepdims=True)
    dR = F * (Hm - rowterm)             # zero above the diagonal (F = 0 there)
    sg = sigmoid(U)
    dU = np.zeros((T, T))
    dU[strict] = (dR * sg * (1.0 + U * (1.0 - sg)))[strict]
    dU[diag, diag] = dR[diag, diag] * S * (1.0 - S) / tau_s
    dq = scale * (dU @ k)
    dk = scale * (dU.T @ q)
    logi = np.log(np.arange(1, T + 1, dtype=np.float64))[:, None]
    dlam = float(-(np.where(strict, dR, 0.0) * logi).sum())
    return {"dq": dq, "dk": dk, "dv": dv, "dlam": dlam, "dR": dR, "fwd": fw}


def relation_backward(q, k, v, dY, scale, tau_s, lam):
    """Backward over [B, H, T, D]; lambda is one scalar per layer shared by
    all heads (Sec. 3.1 calls it layer-wise), so dlambda sums every head.
    Returns (dq, dk, dv, dlam)."""
    q, k, v, dY = _as64(q), _as64(k), _as64(v), _as64(dY)
    B, H = q.shape[:2]
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    dlam = 0.0
    for b in range(B):
        for h in range(H):
            r = relation_backward_head(q[b, h], k[b, h], v[b, h], dY[b, h], scale, tau_s, lam)
            dq[b, h], dk[b, h], dv[b, h] = r["dq"], r["dk"], r["dv"]
            dlam += r["dlam"]
    return dq, dk, dv, dlam


def relation_decode_step(q, k_new, v_new, k_cache, v_cache, n_hist, scale, tau_s, lam):
    """One autoregressive step over a KV-style Relation Cache.

    The cache holds the history's p2 (keys) and I (values) per head. The new
    token sits at 1-based position i = n_hist + 1; its Relation row is the
    last row of the forward on the concatenated sequence (Sec. 3.1), so only
    that row is evaluated. Afterwards the new k and v occupy slot n_hist.

    q, k_new, v_new: [B, H, D]; k_cache, v_cache: [B, H, capacity, D].
    Returns (y [B,H,D], g [B,H], k_cache', v_cache') with new arrays for the
    caches (the inputs are not modified).
    """
    q, k_new, v_new = _as64(q), _as64(k_new), _as64(v_new)
    B, H, D = q.shape
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    kc[:, :, n_hist] = k_new
    vc[:, :, n_hist] = v_new
    i = n_hist + 1
    y = np.empty((B, H, v_new.shape[-1]))
    g = np.empty((B, H))
    for b in range(B):
        for h in range(H):
            kk = _as64(kc[b, h, :i])
            vv = _as64(vc[b, h, :i])
            qq = np.zeros((i, D))
            qq[i - 1] = q[b, h]
            yy, _, gg = relation_forward_rows(qq, kk, vv, [i], scale, tau_s, lam)
            y[b, h] = yy[0]
            g[b, h] = gg[0]
    return y, g, kc, vc


def relation_decode_step_ragged(q, k_new, v_new, k_cache, v_cache, n_hist, scale, tau_s, lam):
    """The decode step for a batch whose sequences have different history
    lengths: sequence b is advanced exactly as relation_decode_step advances
    a batch of one with n_hist = n_hist[b] (each sequence is its own Relation
    row; Sec. 3.1). Returns (y, g, k_cache', v_cache') like that function."""
    B = len(n_hist)
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    y = np.empty((B,) + tuple(np.shape(v_new)[1:]))
    g = np.empty(np.shape(q)[:2])
    for b in range(B):
        yb, gb, kcb, vcb = relation_decode_step(q[b:b + 1], k_new[b:b + 1], v_new[b:b + 1],
                                                kc[b:b + 1], vc[b:b + 1], int(n_hist[b]),
                                                scale, tau_s, lam)
        y[b], g[b], kc[b], vc[b] = yb[0], gb[0], kcb[0], vcb[0]
    return y, g, kc, vc


def relation_prefill_rows(q, k_new, v_new, k_cache, v_cache, n_hist, scale, tau_s, lam):
    """Chunked prefill into the Relation Cache: sequence b's m new tokens
    take cache slots n_hist[b] .. n_hist[b] + m - 1 and their rows are rows
    n_hist[b] + 1 .. n_hist[b] + m (1-based) of the forward over the whole
    sequence (Sec. 3.1), each straight from the definition.

    q, k_new, v_new: [B, H, m, D]; caches [B, H, capacity, D]; n_hist: a
    length per sequence. Returns (y [B,H,m,D], LSE [B,H,m], g [B,H,m],
    k_cache', v_cache')."""
    q, k_new, v_new = _as64(q), _as64(k_new), _as64(v_new)
    B, H, m, D = q.shape
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    y = np.empty((B, H, m, v_new.shape[-1]))
    lse = np.empty((B, H, m))
    g = np.empty((B, H, m))
    for b in range(B):
        n = int(n_hist[b])
        kc[b, :, n:n + m] = k_new[b]
        vc[b, :, n:n + m] = v_new[b]
        for h in range(H):
            kk = _as64(kc[b, h, :n + m])
            vv = _as64(vc[b, h, :n + m])
            qq = np.zeros((n + m, D))
            qq[n:] = q[b, h]
            y[b, h], lse[b, h], g[b, h] = relation_forward_rows(
                qq, kk, vv, range(n + 1, n + m + 1), scale, tau_s, lam)
    return y, lse, g, kc, vc


def brute_force_forward_head(q, k, v, scale, tau_s, lam):
    """Entry-by-entry evaluation with scalar Python loops (Sec. 3.1), for tiny
    T. No array arithmetic: every U_ij, S_i, E_ij, R_ij, F_ij is formed from
    its definition. Returns (Y, LSE, g) as nested lists."""
    T = len(q)
    D = len(q[0])
    Dv = len(v[0])

    def sig(x):
        if x >= 0:
            return 1.0 / (1.0 + math.exp(-x))
        e = math.exp(x)
        return e / (1.0 + e)

    Y, LSE, G = [], [], []
    for i in range(1, T + 1):
        r = []
        for j in range(1, T + 1):
            u = 0.0
            for d in range(D):
                u += float(q[i - 1][d]) * float(k[j - 1][d])
            u *= scale
            if j == i:
                r.append(sig(u / tau_s))
            elif j < i:
                r.append(u * sig(u) - lam * math.log(i))
            else:
                r.append(-math.inf)
        mx = max(r)
        w = [math.exp(x - mx) if x != -math.inf else 0.0 for x in r]
        z = sum(w)
        f = [x / z for x in w]
        y = []
        for d in range(Dv):
            acc = 0.0
            for j in range(T):
                acc += f[j] * float(v[j][d])
            y.append(acc)
        Y.append(y)
        LSE.append(mx + math.log(z))
        G.append(sum(f[: i - 1]))
    return Y, LSE, G


def tiled_forward_head(q, k, v, scale, tau_s, lam, tile):
    """FlashRelation's exact tiled evaluation (Sec. 5.1; App. A.3), in fp64.

    For each row i the strictly historical Exchange entries are scanned tile
    by tile with running (m, l, z); the terminal accumulators give
    L^E = m + log l and Ibar^E = z / l, then A = L^E - lambda log i,
    g = sigmoid(A - S) and Y = (1 - g) I_i + g Ibar^E (App. A.3.5). Row 1 has
    no history, A_1 = -inf (App. A.1.8), so g_1 = 0 and Y_1 = I_1.
    Returns (Y, LSE, g) with LSE = log(e^S + e^A) (App. A.1.2).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    T = q.shape[0]
    Y = np.empty((T, v.shape[1]))
    LSE = np.empty(T)
    g = np.empty(T)
    for i in range(1, T + 1):
        qi = q[i - 1]
        S = float(sigmoid(np.array([scale * (qi @ k[i - 1]) / tau_s]))[0])
        m, l, z = -math.inf, 0.0, np.zeros(v.shape[1])
        for start in range(0, i - 1, tile):
            idx = np.arange(start, min(start + tile, i - 1))
            Eb = silu(scale * (k[idx] @ qi))
            m_new = max(m, float(Eb.max()))
            alpha = math.exp(m - m_new) if m != -math.inf else 0.0
            p = np.exp(Eb - m_new)
            l = alpha * l + p.sum()
            z = alpha * z + p @ v[idx]
            m = m_new
        if i == 1:
            A = -math.inf
            gi = 0.0
            y = v[0].copy()
            lse = S
        else:
            A = m + math.log(l) - lam * math.log(i)
            gi = float(sigmoid(np.array([A - S]))[0])
            y = (1.0 - gi) * v[i - 1] + gi * (z / l)
            top = max(S, A)
            lse = top + math.log(math.exp(S - top) + math.exp(A - top))
        Y[i - 1], LSE[i - 1], g[i - 1] = y, lse, gi
    return Y, LSE, g
