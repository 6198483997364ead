"""GPU parity: librelation (through its C ABI) vs the fp64 CPU oracle on the
same seeded inputs.

Tolerances (stated for the operator's outputs Y, dq, dk, dv and used also for
the fp32 row statistics LSE and g):
  fp32 path: max-abs <= 1e-5;
  bf16 path: max-abs <= 2e-2 and mean-abs <= 3e-3.
dL/dlambda is a scalar sum over every row of every head: fp32 within
1e-5 * max(1, |oracle|); bf16 within 2e-2 * max(1, |oracle|) plus the
worst-case effect of the bf16 rounding of the stored Y that the backward
reads (dlambda_rounding_bound).
The full-size forward + backward workloads are checked on every head, and
their dL/dlambda as launched (one scalar over all heads); the cache decode
workload on every head at its first and last step and on sampled heads in
between, with the cache contents compared bit for bit.
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import exchange_relation_amd as rel
import oracle
from workloads import WORKLOADS, make_decode_inputs, make_inputs, ragged_decode_lengths

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
F32_MAX = 1e-5
BF16_MAX, BF16_MEAN = 2e-2, 3e-3


def f64(t):
    return t.detach().cpu().double().numpy()


def check(name, got, ref, dtype):
    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    mx, mean = float(err.max()), float(err.mean())
    print(f"  {name}: max-abs {mx:.3e} mean-abs {mean:.3e}")
    if dtype == "f32":
        assert mx <= F32_MAX, f"{name}: max-abs {mx:.3e} > {F32_MAX}"
    else:
        assert mx <= BF16_MAX, f"{name}: max-abs {mx:.3e} > {BF16_MAX}"
        assert mean <= BF16_MEAN, f"{name}: mean-abs {mean:.3e} > {BF16_MEAN}"


def check_rel(name, got, ref, tol, extra=0.0):
    """|got - ref| <= tol * max(1, |ref|) + extra."""
    err = abs(got - ref)
    bound = tol * max(1.0, abs(ref)) + extra
    print(f"  {name}: {got:.6g} vs {ref:.6g} abs err {err:.3e} (bound {bound:.3e})")
    assert err <= bound, f"{name}: abs err {err:.3e} > {bound:.3e}"


def dlambda_rounding_bound(inp, heads, scale, tau, lam):
    """Worst-case effect on dL/dlambda of the bf16 rounding of Y.

    dL/dlambda = sum_i ln(i) F_ii (G_i . v_i - G_i . Y_i); the backward reads
    the stored (bf16, round-to-nearest-even) Y, whose every element is off by
    at most 2^-9 |Y| relative, so the sum moves by at most
    2^-9 sum_i ln(i) F_ii sum_d |G_id Y_id|. F, Y from the fp64 oracle."""
    tot = 0.0
    for b, h in heads:
        r = oracle.relation_forward_head(f64(inp["q"][b, h]), f64(inp["k"][b, h]),
                                         f64(inp["v"][b, h]), scale, tau, lam)
        G = f64(inp["dy"][b, h])
        T = G.shape[0]
        Fii = np.diag(r["F"])
        logi = np.log(np.arange(1, T + 1, dtype=np.float64))
        tot += float((logi * Fii * np.abs(G * r["Y"]).sum(axis=1)).sum())
    return tot * 2.0 ** -9


def run_fwd(inp, dtype, scale, tau=2.0, lam=None):
    lam = inp["lam"] if lam is None else lam
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    y, lse, gate = rel.relation_fwd(q, k, v, lam=lam, scale=scale, tau_s=tau, want_gate=True)
    torch.cuda.synchronize()
    return y, lse, gate


def oracle_heads(inp, heads, scale, tau, lam):
    out = []
    for b, h in heads:
        r = oracle.relation_forward_head(f64(inp["q"][b, h]), f64(inp["k"][b, h]),
                                         f64(inp["v"][b, h]), scale, tau, lam)
        out.append(r)
    return out


# ----------------------------------------------------------------- forward
@pytest.mark.parametrize("seed", [42, 43, 44])
def test_fwd_f32_mhr_workload(seed):
    w = WORKLOADS["mhr_fwd_f32"]
    inp = make_inputs(w.B, w.H, w.T, w.D, "f32", seed)
    scale = 1 / math.sqrt(w.D)
    y, lse, gate = run_fwd(inp, "f32", scale)
    Y, L, G = oracle.relation_forward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), scale, 2.0,
                                      inp["lam"])
    check("y", f64(y), Y, "f32")
    check("lse", f64(lse), L, "f32")
    check("gate", f64(gate), G, "f32")


@pytest.mark.parametrize("D", [32, 64])
@pytest.mark.parametrize("T", [1, 2, 63, 65, 129])
@pytest.mark.parametrize("lam,scale_kind", [(0.0, "sqrt"), (1.0, "lin"), (-0.5, "sqrt")])
def test_fwd_f32_shapes_params(D, T, lam, scale_kind):
    inp = make_inputs(2, 2, T, D, "f32", seed=7 + T)
    scale = 1 / math.sqrt(D) if scale_kind == "sqrt" else 1 / D
    y, lse, gate = run_fwd(inp, "f32", scale, lam=lam)
    Y, L, G = oracle.relation_forward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), scale, 2.0, lam)
    check("y", f64(y), Y, "f32")
    check("lse", f64(lse), L, "f32")
    check("gate", f64(gate), G, "f32")


BF16_SHAPES = [(1, 1, 1), (1, 2, 2), (2, 1, 31), (1, 2, 32), (1, 1, 33), (1, 2, 63), (2, 1, 64),
               (1, 1, 65), (2, 2, 127), (1, 2, 128), (1, 1, 129), (1, 2, 191), (1, 1, 192),
               (2, 1, 193), (1, 3, 300), (1, 1, 513)]


@pytest.mark.parametrize("B,H,T", BF16_SHAPES)
def test_fwd_bf16_shapes(B, H, T):
    inp = make_inputs(B, H, T, 64, "bf16", seed=100 + T)
    scale = 1 / 8
    y, lse, gate = run_fwd(inp, "bf16", scale)
    Y, L, G = oracle.relation_forward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), scale, 2.0,
                                      inp["lam"])
    check("y", f64(y), Y, "bf16")
    check("lse", f64(lse), L, "bf16")
    check("gate", f64(gate), G, "bf16")


@pytest.mark.parametrize("T", [1, 65, 129])
def test_fwd_bf16_many_heads_short_rows(T):
    """Short rows on 1024 heads: a grid too large for the 64-row split-key
    blocks, so the 128-row blocks run their ragged and single-row cases
    (small grids take the split-key blocks); sampled heads vs the oracle."""
    B, H, scale = 16, 64, 1 / 8
    inp = make_inputs(B, H, T, 64, "bf16", seed=700 + T)
    y, lse, gate = run_fwd(inp, "bf16", scale)
    heads = [(b, h) for b in range(0, B, 5) for h in range(0, H, 13)]
    refs = oracle_heads(inp, heads, scale, 2.0, inp["lam"])
    check("y", np.stack([f64(y[b, h]) for b, h in heads]), np.stack([r["Y"] for r in refs]), "bf16")
    check("lse", np.stack([f64(lse[b, h]) for b, h in heads]), np.stack([r["LSE"] for r in refs]),
          "bf16")
    check("gate", np.stack([f64(gate[b, h]) for b, h in heads]), np.stack([r["g"] for r in refs]),
          "bf16")


@pytest.mark.parametrize("D", [48, 64, 80])
def test_fwd_bf16_split_key_blocks_match_full_blocks(D):
    """The same heads through both block shapes: inside a 1024-head call
    (128-row blocks) and as a 2-head call (64-row blocks whose key tiles two
    waves split, merged before the completion). Each wave rounds P against
    its own stabiliser, so the two agree to the split-over-keys bound."""
    B, H, T = 16, 64, 300
    inp = make_inputs(B, H, T, D, "bf16", seed=800 + D)
    scale = 1 / math.sqrt(D)
    y, lse, gate = run_fwd(inp, "bf16", scale)
    sub = {n: inp[n][3:4, 10:12].contiguous() for n in ("q", "k", "v")}
    y2, l2, g2 = run_fwd({**inp, **sub}, "bf16", scale)
    vmax = float(sub["v"].float().abs().max())
    close_to_unsplit("y", y2, y[3:4, 10:12], vmax)
    close_to_unsplit("lse", l2, lse[3:4, 10:12], vmax)
    close_to_unsplit("gate", g2, gate[3:4, 10:12], vmax)


@pytest.mark.parametrize("H,D", [(48, 64), (49, 64), (32, 80), (33, 80), (48, 48), (49, 48)])
def test_fwd_bf16_block_form_boundary(H, D):
    """Grids on either side of the limit for 64-row split-key blocks (768 of
    them at d_h <= 64, 512 at 80, at one workgroup slot per block): B=1, T=1024
    with H = 48 / 32 heads take split-key blocks, one more head 128-row
    blocks. First, middle and last heads, every row, against the oracle."""
    B, T = 1, 1024
    inp = make_inputs(B, H, T, D, "bf16", seed=860 + H + D)
    scale = 1 / math.sqrt(D)
    y, lse, gate = run_fwd(inp, "bf16", scale)
    heads = [(0, 0), (0, H // 2), (0, H - 1)]
    refs = oracle_heads(inp, heads, scale, 2.0, inp["lam"])
    check("y", np.stack([f64(y[b, h]) for b, h in heads]), np.stack([r["Y"] for r in refs]),
          "bf16")
    check("lse", np.stack([f64(lse[b, h]) for b, h in heads]), np.stack([r["LSE"] for r in refs]),
          "bf16")
    check("gate", np.stack([f64(gate[b, h]) for b, h in heads]), np.stack([r["g"] for r in refs]),
          "bf16")


@pytest.mark.parametrize("lam", [0.0, 1.0, -0.5, 4.0])
@pytest.mark.parametrize("scale", [1 / 8, 1 / 64, 0.5])
def test_fwd_bf16_params(lam, scale):
    inp = make_inputs(1, 2, 257, 64, "bf16", seed=5)
    y, lse, gate = run_fwd(inp, "bf16", scale, lam=lam)
    Y, L, G = oracle.relation_forward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), scale, 2.0, lam)
    check("y", f64(y), Y, "bf16")
    check("gate", f64(gate), G, "bf16")
    check("lse", f64(lse), L, "bf16")


@pytest.mark.parametrize("D", [48, 64, 80])
def test_fwd_bf16_large_scores_rescale(D):
    """Scores far above the lazy-rescale slack force the running stabiliser
    to move several times inside a row (a small grid: the split-key blocks,
    whose two key halves then merge scans with different stabilisers)."""
    inp = make_inputs(1, 2, 384, D, "bf16", seed=9)
    scale = 2.0 * 8 / math.sqrt(D)  # U std ~ 16
    y, lse, gate = run_fwd(inp, "bf16", scale)
    Y, L, G = oracle.relation_forward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), scale, 2.0,
                                      inp["lam"])
    err = np.abs(f64(y) - Y)
    print(f"  y: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert np.isfinite(f64(y)).all()
    check("y", f64(y), Y, "bf16")


def close_to_unsplit(name, a, b, vmax):
    """Split and unsplit runs round every P = exp(E - m) to bf16 against their
    own stabiliser m (each piece has its own), so single terms differ by up to
    2^-9 relative and the rows by at most 2^-8 max|v| (y, plus one bf16 unit
    in the last place of the output) and 2^-8 (lse, gate)."""
    a, b = a.float(), b.float()
    d = (a - b).abs()
    frac = float((d > 0).float().mean())
    print(f"  {name}: max diff {d.max().item():.3e}, differing {frac:.2e}")
    if name == "y":
        bound = 2.0 ** -8 * vmax + torch.clamp(b.abs(), min=2.0 ** -126) * 2.0 ** -7
    else:
        bound = torch.full_like(b, 2.0 ** -8)
    assert bool((d <= bound).all()), name
    assert frac < 0.05, name


@pytest.mark.parametrize("B,H,T,D", [(1, 2, 1300, 64), (1, 1, 2500, 64), (2, 1, 1800, 64),
                                     (1, 1, 2100, 48), (1, 1, 2100, 80)])
def test_fwd_bf16_split_over_keys(B, H, T, D):
    """A grid too small to fill the GPU splits its long query blocks over the
    keys; the pieces are merged by App. A.3.2's rule in a second kernel (at
    every head width: the partial rows are D + 4 floats)."""
    assert rel.relation_fwd_workspace_bytes(torch.bfloat16, B, H, T, D) > 0
    inp = make_inputs(B, H, T, D, "bf16", seed=700 + T)
    scale = 1 / math.sqrt(D)
    y, lse, gate = run_fwd(inp, "bf16", scale)
    Y, L, G = oracle.relation_forward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), scale, 2.0,
                                      inp["lam"])
    check("y", f64(y), Y, "bf16")
    check("lse", f64(lse), L, "bf16")
    check("gate", f64(gate), G, "bf16")
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    y1, l1, g1 = rel.relation_fwd(q, k, v, lam=inp["lam"], scale=scale, want_gate=True,
                                  split=False)
    y2, l2, g2 = run_fwd(inp, "bf16", scale)
    torch.cuda.synchronize()
    vmax = float(inp["v"].float().abs().max())
    close_to_unsplit("y", y, y1, vmax)
    close_to_unsplit("lse", lse, l1, vmax)
    close_to_unsplit("gate", gate, g1, vmax)
    assert torch.equal(y, y2) and torch.equal(lse, l2) and torch.equal(gate, g2)  # deterministic


@pytest.mark.parametrize("key,heads", [
    ("layer10m_fwd_bf16", "all"),
])
def test_fwd_bf16_full_size(key, heads):
    w = WORKLOADS[key]
    inp = make_inputs(w.B, w.H, w.T, w.D, "bf16", seed=42, rope=w.rope)
    scale = 1 / math.sqrt(w.D)
    y, lse, gate = run_fwd(inp, "bf16", scale)
    if heads == "all":
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    refs = oracle_heads(inp, heads, scale, 2.0, inp["lam"])
    Yg = np.stack([f64(y[b, h]) for b, h in heads])
    Lg = np.stack([f64(lse[b, h]) for b, h in heads])
    Gg = np.stack([f64(gate[b, h]) for b, h in heads])
    check("y", Yg, np.stack([r["Y"] for r in refs]), "bf16")
    check("lse", Lg, np.stack([r["LSE"] for r in refs]), "bf16")
    check("gate", Gg, np.stack([r["g"] for r in refs]), "bf16")


# ---------------------------------------------------------------- backward
def run_bwd(inp, scale, tau=2.0, lam=None):
    lam = inp["lam"] if lam is None else lam
    q, k, v, dy = (inp[n].to(DEV) for n in ("q", "k", "v", "dy"))
    y, lse, _ = rel.relation_fwd(q, k, v, lam=lam, scale=scale, tau_s=tau)
    dq, dk, dv, dl = rel.relation_bwd(q, k, v, y, dy, lse, lam=lam, scale=scale, tau_s=tau)
    torch.cuda.synchronize()
    return dq, dk, dv, float(dl.item())


@pytest.mark.parametrize("lam,T", [(None, 128), (0.0, 65), (-0.5, 1), (1.0, 200)])
def test_bwd_f32(lam, T):
    inp = make_inputs(1, 2, T, 32, "f32", seed=42, with_dy=True)
    lam = inp["lam"] if lam is None else lam
    scale = 1 / math.sqrt(32)
    dq, dk, dv, dl = run_bwd(inp, scale, lam=lam)
    gq, gk, gv, gl = oracle.relation_backward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]),
                                              f64(inp["dy"]), scale, 2.0, lam)
    check("dq", f64(dq), gq, "f32")
    check("dk", f64(dk), gk, "f32")
    check("dv", f64(dv), gv, "f32")
    check_rel("dlambda", dl, gl, 1e-5)


@pytest.mark.parametrize("B,H,T", [(1, 1, 1), (1, 2, 33), (2, 1, 64), (1, 2, 127), (1, 1, 130),
                                   (2, 2, 256), (1, 1, 300)])
def test_bwd_bf16_shapes(B, H, T):
    inp = make_inputs(B, H, T, 64, "bf16", seed=200 + T, with_dy=True)
    scale = 1 / 8
    dq, dk, dv, dl = run_bwd(inp, scale)
    gq, gk, gv, gl = oracle.relation_backward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]),
                                              f64(inp["dy"]), scale, 2.0, inp["lam"])
    check("dq", f64(dq), gq, "bf16")
    check("dk", f64(dk), gk, "bf16")
    check("dv", f64(dv), gv, "bf16")
    heads = [(b, h) for b in range(B) for h in range(H)]
    check_rel("dlambda", dl, gl, 2e-2, dlambda_rounding_bound(inp, heads, scale, 2.0, inp["lam"]))


@pytest.mark.parametrize("lam", [0.0, 1.0, -0.5])
def test_bwd_bf16_params(lam):
    inp = make_inputs(1, 2, 193, 64, "bf16", seed=11, with_dy=True)
    scale = 1 / 8
    dq, dk, dv, dl = run_bwd(inp, scale, lam=lam)
    gq, gk, gv, gl = oracle.relation_backward(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]),
                                              f64(inp["dy"]), scale, 2.0, lam)
    check("dq", f64(dq), gq, "bf16")
    check("dk", f64(dk), gk, "bf16")
    check("dv", f64(dv), gv, "bf16")
    check_rel("dlambda", dl, gl, 2e-2,
              dlambda_rounding_bound(inp, [(0, 0), (0, 1)], scale, 2.0, lam))


def _oracle_threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_backward_heads(inp, heads, scale, tau, lam):
    """fp64 oracle forward + backward of whole heads, several heads at a time
    on the host's cores (numpy releases the interpreter lock in its array
    work). Per head: Y, LSE, g, dq, dk, dv, dlam and the head's term of
    dlambda_rounding_bound (before the 2^-9 factor)."""
    def one(bh):
        b, h = bh
        G = f64(inp["dy"][b, h])
        r = oracle.relation_backward_head(f64(inp["q"][b, h]), f64(inp["k"][b, h]),
                                          f64(inp["v"][b, h]), G, scale, tau, lam)
        fw = r["fwd"]
        T = G.shape[0]
        logi = np.log(np.arange(1, T + 1, dtype=np.float64))
        rb = float((logi * np.diag(fw["F"]) * np.abs(G * fw["Y"]).sum(axis=1)).sum())
        return {"Y": fw["Y"], "LSE": fw["LSE"], "g": fw["g"], "dq": r["dq"], "dk": r["dk"],
                "dv": r["dv"], "dlam": r["dlam"], "rbound": rb}
    with ThreadPoolExecutor(_oracle_threads()) as ex:
        return list(ex.map(one, heads))


@pytest.mark.parametrize("key", ["layer30m_fwdbwd_bf16", "layer100m_fwdbwd_bf16"])
def test_fwdbwd_bf16_full_size_every_head(key):
    """The whole workload in the benchmark's launch shape (one forward and
    one backward call over every head): y, LSE, g, dq, dk and dv of EVERY
    head element by element against the fp64 oracle, and the launch's
    dL/dlambda (one scalar summed over all B*H heads, since lambda is one
    layer-wise parameter, Sec. 3.1) against the oracle's sum over the same
    heads."""
    w = WORKLOADS[key]
    inp = make_inputs(w.B, w.H, w.T, w.D, "bf16", seed=42, with_dy=True)
    scale, lam = 1 / math.sqrt(w.D), inp["lam"]
    q, k, v, dy = (inp[n].to(DEV) for n in ("q", "k", "v", "dy"))
    y, lse, gate = rel.relation_fwd(q, k, v, lam=lam, scale=scale, tau_s=2.0, want_gate=True)
    dq, dk, dv, dl = rel.relation_bwd(q, k, v, y, dy, lse, lam=lam, scale=scale, tau_s=2.0)
    torch.cuda.synchronize()
    got = {n: f64(t).reshape(w.B * w.H, *t.shape[2:])
           for n, t in (("Y", y), ("LSE", lse), ("g", gate), ("dq", dq), ("dk", dk), ("dv", dv))}
    dl = float(dl.item())
    del q, k, v, dy, y, lse, gate, dq, dk, dv
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    print(f"  {key}: {len(heads)} heads, oracle on {_oracle_threads()} threads")
    refs = oracle_backward_heads(inp, heads, scale, 2.0, lam)
    for n in ("Y", "LSE", "g", "dq", "dk", "dv"):
        check(n, got[n], np.stack([r[n] for r in refs]), "bf16")
    check_rel("dlambda(full launch)", dl, float(sum(r["dlam"] for r in refs)), 2e-2,
              2.0 ** -9 * sum(r["rbound"] for r in refs))


# ------------------------------------------------------------------ decode
def run_decode_steps(d, n0, steps, scale, dtype_t=None):
    kc, vc = d["k_cache"].to(DEV), d["v_cache"].to(DEV)
    ys, gs = [], []
    B, H, cap, D = kc.shape
    ws = torch.empty(rel.relation_decode_workspace_bytes(kc.dtype, B, H, D, cap), device=DEV,
                     dtype=torch.uint8)
    for s in range(steps):
        y, g = rel.relation_cache_decode(d["q"][s].to(DEV), d["k_new"][s].to(DEV),
                                         d["v_new"][s].to(DEV), kc, vc, n0 + s, lam=d["lam"],
                                         scale=scale, tau_s=2.0, want_gate=True, workspace=ws)
        ys.append(y.cpu())
        gs.append(g.cpu())
    torch.cuda.synchronize()
    return ys, gs, kc.cpu(), vc.cpu()


def oracle_decode_rows(d, s, n, heads, scale, lam):
    """Last row of the forward over [cache[:n]; k_new] for each (b, h)."""
    ys, gs = [], []
    for b, h in heads:
        K = np.concatenate([f64(d["k_cache"][b, h, :n]), f64(d["k_new"][s, b, h])[None]], 0)
        V = np.concatenate([f64(d["v_cache"][b, h, :n]), f64(d["v_new"][s, b, h])[None]], 0)
        Q = np.zeros_like(K)
        Q[n] = f64(d["q"][s, b, h])
        y, _, g = oracle.relation_forward_rows(Q, K, V, [n + 1], scale, 2.0, lam)
        ys.append(y[0])
        gs.append(g[0])
    return np.stack(ys), np.array(gs)


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("f32", 64), ("f32", 32)])
@pytest.mark.parametrize("n0", [0, 1, 31, 33, 511, 512, 513, 1500])
def test_decode_small(dtype, D, n0):
    B, H, steps = 2, 3, 3
    d = make_decode_inputs(B, H, D, n0, steps, n0 + steps + 5, dtype, seed=300 + n0)
    scale = 1 / math.sqrt(D)
    ys, gs, kc, vc = run_decode_steps(d, n0, steps, scale)
    heads = [(b, h) for b in range(B) for h in range(H)]
    # later steps see the earlier steps' appended tokens
    kfull, vfull = d["k_cache"].clone(), d["v_cache"].clone()
    for s in range(steps):
        dd = dict(d, k_cache=kfull, v_cache=vfull)
        Y, G = oracle_decode_rows(dd, s, n0 + s, heads, scale, d["lam"])
        check(f"y step {s}", np.stack([f64(ys[s][b, h]) for b, h in heads]), Y, dtype)
        check(f"gate step {s}", np.stack([f64(gs[s][b, h]) for b, h in heads]), G, dtype)
        kfull[:, :, n0 + s] = d["k_new"][s]
        vfull[:, :, n0 + s] = d["v_new"][s]
    assert torch.equal(kc, kfull) and torch.equal(vc, vfull)  # bit-exact append, rest untouched


def test_decode_full_size_cache_workload():
    w = WORKLOADS["cache_decode_bf16"]
    d = make_decode_inputs(w.B, w.H, w.D, w.n_hist, w.steps, w.capacity, "bf16", seed=42)
    scale = 1 / math.sqrt(w.D)
    ys, gs, kc, vc = run_decode_steps(d, w.n_hist, w.steps, scale)
    # bit-exact cache: history untouched, slots n..n+steps-1 = the new tokens,
    # slots past them untouched
    exp_k, exp_v = d["k_cache"].clone(), d["v_cache"].clone()
    exp_k[:, :, w.n_hist:w.n_hist + w.steps] = d["k_new"].permute(1, 2, 0, 3)
    exp_v[:, :, w.n_hist:w.n_hist + w.steps] = d["v_new"].permute(1, 2, 0, 3)
    assert torch.equal(kc, exp_k) and torch.equal(vc, exp_v)
    dd = dict(d, k_cache=exp_k, v_cache=exp_v)
    all_heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    for s in (0, 1, 128, 255):
        heads = all_heads if s in (0, 255) else all_heads[::17]
        Y, G = oracle_decode_rows(dd, s, w.n_hist + s, heads, scale, d["lam"])
        check(f"y step {s}", np.stack([f64(ys[s][b, h]) for b, h in heads]), Y, "bf16")
        check(f"gate step {s}", np.stack([f64(gs[s][b, h]) for b, h in heads]), G, "bf16")


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 48), ("bf16", 80), ("f32", 64),
                                     ("f32", 32)])
@pytest.mark.parametrize("n0", [1, 33, 700])
def test_decode_whole_history_mode(dtype, D, n0):
    """B * H >= 256: one workgroup per head scans the whole history and
    completes the row in the same launch. Every head against the oracle over
    two steps, and the cache bit for bit."""
    B, H, steps = 32, 8, 2
    d = make_decode_inputs(B, H, D, n0, steps, n0 + steps + 3, dtype, seed=350 + n0 + D)
    scale = 1 / math.sqrt(D)
    ys, gs, kc, vc = run_decode_steps(d, n0, steps, scale)
    heads = [(b, h) for b in range(B) for h in range(H)]
    kfull, vfull = d["k_cache"].clone(), d["v_cache"].clone()
    for s in range(steps):
        dd = dict(d, k_cache=kfull, v_cache=vfull)
        Y, G = oracle_decode_rows(dd, s, n0 + s, heads, scale, d["lam"])
        check(f"y step {s}", np.stack([f64(ys[s][b, h]) for b, h in heads]), Y, dtype)
        check(f"gate step {s}", np.stack([f64(gs[s][b, h]) for b, h in heads]), G, dtype)
        kfull[:, :, n0 + s] = d["k_new"][s]
        vfull[:, :, n0 + s] = d["v_new"][s]
    assert torch.equal(kc, kfull) and torch.equal(vc, vfull)


# ------------------------------------------------------------ ragged decode
def ragged_lengths_inputs(B, H, D, lengths, capacity, steps, dtype, seed):
    """Decode inputs with every cache slot filled (so untouched slots can be
    checked) and per-sequence history lengths."""
    d = make_decode_inputs(B, H, D, capacity - steps, steps, capacity, dtype, seed=seed)
    return d, torch.tensor(lengths, dtype=torch.int32)


def run_ragged_steps(d, lengths, steps, scale, bound):
    kc, vc = d["k_cache"].to(DEV), d["v_cache"].to(DEV)
    B, H, cap, D = kc.shape
    nh = lengths.to(DEV)
    ws = torch.empty(rel.relation_decode_workspace_bytes(kc.dtype, B, H, D, cap), device=DEV,
                     dtype=torch.uint8)
    ys, gs = [], []
    for s in range(steps):
        y, g = rel.relation_cache_decode_ragged(d["q"][s].to(DEV), d["k_new"][s].to(DEV),
                                                d["v_new"][s].to(DEV), kc, vc, nh, bound + s,
                                                lam=d["lam"], scale=scale, tau_s=2.0,
                                                want_gate=True, workspace=ws)
        ys.append(y.cpu())
        gs.append(g.cpu())
        nh += 1  # the caller advances the lengths
    torch.cuda.synchronize()
    return ys, gs, kc.cpu(), vc.cpu()


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("f32", 64), ("f32", 32)])
def test_decode_ragged_vs_oracle(dtype, D):
    lengths = [0, 1, 31, 512, 513, 700]
    B, H, cap, steps = len(lengths), 3, 720, 2
    d, nh = ragged_lengths_inputs(B, H, D, lengths, cap, steps, dtype, seed=410 + D)
    scale = 1 / math.sqrt(D)
    ys, gs, kc, vc = run_ragged_steps(d, nh, steps, scale, max(lengths))
    kfull, vfull = d["k_cache"].clone(), d["v_cache"].clone()
    for s in range(steps):
        ns = [n + s for n in lengths]
        Y, G, kexp, vexp = oracle.relation_decode_step_ragged(
            f64(d["q"][s]), f64(d["k_new"][s]), f64(d["v_new"][s]), f64(kfull), f64(vfull), ns,
            scale, 2.0, d["lam"])
        check(f"ragged y step {s}", f64(ys[s]), Y, dtype)
        check(f"ragged gate step {s}", f64(gs[s]), G, dtype)
        for b, n in enumerate(ns):
            kfull[b, :, n] = d["k_new"][s, b]
            vfull[b, :, n] = d["v_new"][s, b]
    assert torch.equal(kc, kfull) and torch.equal(vc, vfull)  # bit-exact appends, rest untouched


def test_decode_ragged_equal_lengths_match_uniform_bit_exact():
    B, H, D, n, cap = 3, 4, 64, 1030, 1040
    d = make_decode_inputs(B, H, D, n, 1, cap, "bf16", seed=421)
    scale = 1 / 8
    yu, gu, kcu, vcu = run_decode_steps(d, n, 1, scale)
    yr, gr_, kcr, vcr = run_ragged_steps(d, torch.full((B,), n, dtype=torch.int32), 1, scale, n)
    assert torch.equal(yu[0], yr[0]) and torch.equal(gu[0], gr_[0])
    assert torch.equal(kcu, kcr) and torch.equal(vcu, vcr)


def test_decode_ragged_out_of_range_lengths_give_nan_and_no_write():
    lengths = [5, 40, -1, 9]  # the bound passed is 20: sequence 1 is above it, 2 negative
    B, H, D, cap = len(lengths), 2, 64, 64
    d, nh = ragged_lengths_inputs(B, H, D, lengths, cap, 1, "bf16", seed=433)
    ys, gs, kc, vc = run_ragged_steps(d, nh, 1, 1 / 8, 20)
    y, g = f64(ys[0]), f64(gs[0])
    assert np.isnan(y[1]).all() and np.isnan(y[2]).all() and np.isnan(g[1]).all()
    assert torch.equal(kc[1], d["k_cache"][1]) and torch.equal(kc[2], d["k_cache"][2])
    assert torch.equal(vc[1], d["v_cache"][1]) and torch.equal(vc[2], d["v_cache"][2])
    for b in (0, 3):
        n = lengths[b]
        Y, G, _, _ = oracle.relation_decode_step_ragged(
            f64(d["q"][0, b:b + 1]), f64(d["k_new"][0, b:b + 1]), f64(d["v_new"][0, b:b + 1]),
            f64(d["k_cache"][b:b + 1]), f64(d["v_cache"][b:b + 1]), [n], 1 / 8, 2.0, d["lam"])
        check(f"valid row {b}", y[b:b + 1], Y, "bf16")
        assert torch.equal(kc[b, :, n], d["k_new"][0, b])


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 80), ("f32", 32)])
def test_decode_ragged_many_heads(dtype, D):
    """Ragged lengths on a batch of B * H >= 256 heads (where uniform
    batches take the one-workgroup-per-head mode; ragged ones keep the
    split): lengths 0, 1, 31, 512, 513, 700 and two out of range (above the
    bound, negative); valid rows against the oracle, invalid rows NaN with
    their cache rows untouched, appends bit for bit."""
    base = [0, 1, 31, 512, 513, 700, 900, -3]  # bound 720: 900 above it, -3 negative
    lengths = base * 4
    B, H, cap = len(lengths), 8, 730
    d, nh = ragged_lengths_inputs(B, H, D, lengths, cap, 1, dtype, seed=470 + D)
    scale = 1 / math.sqrt(D)
    ys, gs, kc, vc = run_ragged_steps(d, nh, 1, scale, 720)
    y, g = f64(ys[0]), f64(gs[0])
    ok = [b for b, n in enumerate(lengths) if 0 <= n <= 720]
    bad = [b for b in range(B) if b not in ok]
    assert np.isnan(y[bad]).all() and np.isnan(g[bad]).all()
    for b in bad:
        assert torch.equal(kc[b], d["k_cache"][b]) and torch.equal(vc[b], d["v_cache"][b])
    Y, G, kexp, vexp = oracle.relation_decode_step_ragged(
        f64(d["q"][0, ok]), f64(d["k_new"][0, ok]), f64(d["v_new"][0, ok]),
        f64(d["k_cache"][ok]), f64(d["v_cache"][ok]), [lengths[b] for b in ok], scale, 2.0,
        d["lam"])
    check("ragged whole y", y[ok], Y, dtype)
    check("ragged whole gate", g[ok], G, dtype)
    for b in ok:
        n = lengths[b]
        assert torch.equal(kc[b, :, n], d["k_new"][0, b])
        assert torch.equal(vc[b, :, n], d["v_new"][0, b])


def test_decode_ragged_full_size_workload():
    w = WORKLOADS["cache_decode_bf16"]
    lengths = ragged_decode_lengths(w.B, w.n_hist, seed=42)
    steps = 3
    d, nh = ragged_lengths_inputs(w.B, w.H, w.D, lengths, w.capacity, steps, "bf16", seed=42)
    scale = 1 / math.sqrt(w.D)
    ys, gs, kc, vc = run_ragged_steps(d, nh, steps, scale, w.n_hist)
    kfull, vfull = d["k_cache"].clone(), d["v_cache"].clone()
    for s in range(steps):
        ns = [n + s for n in lengths]
        bs = list(range(0, w.B, 5)) if s < steps - 1 else list(range(w.B))
        for b in bs:
            Y, G, _, _ = oracle.relation_decode_step_ragged(
                f64(d["q"][s, b:b + 1]), f64(d["k_new"][s, b:b + 1]), f64(d["v_new"][s, b:b + 1]),
                f64(kfull[b:b + 1]), f64(vfull[b:b + 1]), [ns[b]], scale, 2.0, d["lam"])
            check(f"ragged full y step {s} seq {b}", f64(ys[s][b:b + 1]), Y, "bf16")
        for b, n in enumerate(ns):
            kfull[b, :, n] = d["k_new"][s, b]
            vfull[b, :, n] = d["v_new"][s, b]
    assert torch.equal(kc, kfull) and torch.equal(vc, vfull)


# ------------------------------------------------------ bit-exact properties
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fwd_causality_bit_exact(dtype):
    D = 64
    inp = make_inputs(1, 2, 300, D, dtype, seed=17)
    scale = 1 / 8
    y0, l0, g0 = run_fwd(inp, dtype, scale)
    for t in (0, 77, 128, 255):
        pert = {n: inp[n].clone() for n in ("q", "k", "v")}
        pert["lam"] = inp["lam"]
        for n in ("q", "k", "v"):
            pert[n][:, :, t] = pert[n][:, :, t] * -2 + 1
        y1, l1, g1 = run_fwd(pert, dtype, scale)
        assert torch.equal(y1[:, :, :t], y0[:, :, :t]), t
        assert torch.equal(l1[:, :, :t], l0[:, :, :t]) and torch.equal(g1[:, :, :t], g0[:, :, :t])
        assert not torch.equal(y1[:, :, t], y0[:, :, t])


def test_fwd_deterministic():
    inp = make_inputs(2, 3, 517, 64, "bf16", seed=3)
    a = run_fwd(inp, "bf16", 1 / 8)
    b = run_fwd(inp, "bf16", 1 / 8)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_dk_dv_deterministic():
    inp = make_inputs(1, 2, 300, 64, "bf16", seed=4, with_dy=True)
    a = run_bwd(inp, 1 / 8)
    b = run_bwd(inp, 1 / 8)
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    assert a[3] == b[3]  # dlambda is reduced in a fixed order


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 80), ("f32", 64)])
def test_bwd_events_entry_point_matches_bwd(dtype, D):
    """relation_bwd_events gives relation_bwd's results (dk, dv and dlambda bit
    for bit; dq, accumulated by fp32 atomics in no fixed order, within the
    tolerance) and its events bracket a non-empty part of the call."""
    inp = make_inputs(2, 4, 700, D, dtype, seed=21, with_dy=True)
    scale = 1 / math.sqrt(D)
    q, k, v, dy = (inp[n].to(DEV) for n in ("q", "k", "v", "dy"))
    y, lse, _ = rel.relation_fwd(q, k, v, lam=inp["lam"], scale=scale)
    a = rel.relation_bwd(q, k, v, y, dy, lse, lam=inp["lam"], scale=scale)
    stream = torch.cuda.current_stream(DEV)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    b = rel.relation_bwd(q, k, v, y, dy, lse, lam=inp["lam"], scale=scale, main_events=(m0, m1))
    c1.record(stream)
    torch.cuda.synchronize()
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    assert float(a[3].item()) == float(b[3].item())
    check("dq", f64(b[0]), f64(a[0]), dtype)
    t_main, t_call = m0.elapsed_time(m1), c0.elapsed_time(c1)
    print(f"  main kernel(s) {t_main * 1e3:.1f} us of the call's {t_call * 1e3:.1f} us")
    assert 0.0 < t_main <= t_call


def test_decode_matches_forward_last_row():
    """The decode step's output equals the GPU forward's row at the same
    position (within bf16 tolerance)."""
    B, H, D, n = 2, 2, 64, 700
    inp = make_inputs(B, H, n + 1, D, "bf16", seed=21)
    y, _, gate = run_fwd(inp, "bf16", 1 / 8)
    cap = n + 8
    kc = torch.zeros((B, H, cap, D), dtype=torch.bfloat16)
    vc = torch.zeros((B, H, cap, D), dtype=torch.bfloat16)
    kc[:, :, :n] = inp["k"][:, :, :n]
    vc[:, :, :n] = inp["v"][:, :, :n]
    d = {"k_cache": kc, "v_cache": vc, "q": inp["q"][:, :, n][None], "k_new": inp["k"][:, :, n][None],
         "v_new": inp["v"][:, :, n][None], "lam": inp["lam"]}
    ys, gs, _, _ = run_decode_steps(d, n, 1, 1 / 8)
    check("decode vs fwd row", f64(ys[0]), f64(y[:, :, n]), "bf16")
    check("gate", f64(gs[0]), f64(gate[:, :, n]), "bf16")
