"""GPU parity of Multi-Head Relation with its upstream maps (RoPE of p1, p2;
alternating Givens mixing of I; Sec. 3.1-3.2 and App. A.2.2-A.2.3 of the
Relation paper): relation_mhr_fwd / relation_mhr_bwd through the C ABI
against the fp64 oracle (oracle/mhr.py) on the same seeded inputs and the
same fp32 RoPE tables and angles.

Tolerances as for the plain operator (see test_parity_gpu.py): fp32 max-abs
<= 1e-5; bf16 max-abs <= 2e-2 and mean-abs <= 3e-3 for y, lse, gate, dp1,
dp2, dI. dL/dlambda as there, with the Y-rounding bound evaluated on the
rotated and mixed tensors. dL/dtheta_p = sum(dI'_a I'_b - dI'_b I'_a) is a
sum of products whose factors each carry the path's rounding: it must be
within 1e-5 (fp32) or 2e-2 (bf16) * max(1, |oracle|) plus 1e-6 (fp32) or
2^-7 (bf16) times the sum of the terms' magnitudes.
"""
import math

import numpy as np
import pytest
import torch

import exchange_relation_amd as rel
import oracle
from workloads import make_inputs, make_mhr_maps

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
    err = abs(got - ref)
    bound = tol * max(1.0, abs(ref)) + extra
    print(f"  {name}: {got:.6g} vs {ref:.6g} abs err {err:.3e} (bound {bound:.3e})")
    assert err <= bound, f"{name}: abs err {err:.3e} > {bound:.3e}"


def maps(T, D, H, seed, use_rope, use_mix):
    cs, sn, th = make_mhr_maps(T, D, H, seed)
    return (cs if use_rope else None, sn if use_rope else None, th if use_mix else None)


def to_dev(*ts):
    return [None if t is None else t.to(DEV) for t in ts]


def oracle_fwd(inp, cs, sn, th, pairing, scale, lam):
    return oracle.relation_mhr_forward(
        f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), None if cs is None else f64(cs),
        None if sn is None else f64(sn), None if th is None else f64(th), pairing, scale, 2.0,
        lam)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("pairing", [0, 1])
@pytest.mark.parametrize("T", [1, 33, 130, 300])
def test_mhr_fwd_vs_oracle(dtype, pairing, T):
    B, H, D = 2, 4, 64
    inp = make_inputs(B, H, T, D, dtype, seed=500 + T + pairing)
    cs, sn, th = maps(T, D, H, 500 + T, True, True)
    scale = 1 / math.sqrt(D)
    dcs, dsn, dth = to_dev(cs, sn, th)
    y, lse, g = rel.relation_mhr_fwd(*(inp[n].to(DEV) for n in ("q", "k", "v")), dcs, dsn, dth,
                                     pairing, lam=inp["lam"], scale=scale, want_gate=True)
    torch.cuda.synchronize()
    r = oracle_fwd(inp, cs, sn, th, pairing, scale, inp["lam"])
    check("y", f64(y), r["Y"], dtype)
    check("lse", f64(lse), r["LSE"], dtype)
    check("gate", f64(g), r["g"], dtype)


@pytest.mark.parametrize("use_rope,use_mix", [(True, False), (False, True)])
def test_mhr_fwd_single_map(use_rope, use_mix):
    B, H, T, D = 1, 6, 97, 64
    inp = make_inputs(B, H, T, D, "bf16", seed=611)
    cs, sn, th = maps(T, D, H, 611, use_rope, use_mix)
    dcs, dsn, dth = to_dev(cs, sn, th)
    y, lse, _ = rel.relation_mhr_fwd(*(inp[n].to(DEV) for n in ("q", "k", "v")), dcs, dsn, dth, 1,
                                     lam=inp["lam"], scale=0.125)
    torch.cuda.synchronize()
    r = oracle_fwd(inp, cs, sn, th, 1, 0.125, inp["lam"])
    check("y", f64(y), r["Y"], "bf16")
    check("lse", f64(lse), r["LSE"], "bf16")


def test_mhr_fwd_without_maps_is_relation_fwd_bit_exact():
    inp = make_inputs(2, 2, 200, 64, "bf16", seed=617)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    y1, l1, _ = rel.relation_mhr_fwd(q, k, v, lam=inp["lam"], scale=0.125)
    y2, l2, _ = rel.relation_fwd(q, k, v, lam=inp["lam"], scale=0.125)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(l1, l2)


def dlam_bound(f, dY):
    """2^-9 sum ln(i) F_ii sum_d |G_id Y_id| on the rotated / mixed tensors."""
    tot = 0.0
    B, H = f["q"].shape[:2]
    for b in range(B):
        for h in range(H):
            r = oracle.relation_forward_head(f["q"][b, h], f["k"][b, h], f["v"][b, h],
                                             f["scale"], 2.0, f["lam"])
            T = r["Y"].shape[0]
            logi = np.log(np.arange(1, T + 1, dtype=np.float64))
            tot += float((logi * np.diag(r["F"]) * np.abs(dY[b, h] * r["Y"]).sum(axis=1)).sum())
    return tot * 2.0 ** -9


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("pairing", [0, 1])
@pytest.mark.parametrize("T", [33, 300])
def test_mhr_bwd_vs_oracle(dtype, pairing, T):
    B, H, D = 2, 4, 64
    inp = make_inputs(B, H, T, D, dtype, seed=700 + T + pairing, with_dy=True)
    cs, sn, th = maps(T, D, H, 700 + T, True, True)
    scale, lam = 1 / math.sqrt(D), inp["lam"]
    p1, p2, I, dy = (inp[n].to(DEV) for n in ("q", "k", "v", "dy"))
    dcs, dsn, dth = to_dev(cs, sn, th)
    y, lse, _ = rel.relation_mhr_fwd(p1, p2, I, dcs, dsn, dth, pairing, lam=lam, scale=scale)
    dp1, dp2, dI, dl, dtheta = rel.relation_mhr_bwd(p1, p2, I, y, dy, lse, dcs, dsn, dth, pairing,
                                                    lam=lam, scale=scale)
    torch.cuda.synchronize()
    args = (f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["dy"]), f64(cs), f64(sn),
            f64(th), pairing, scale, 2.0, lam)
    r1, r2, rI, rl, rth = oracle.relation_mhr_backward(*args)
    check("dp1", f64(dp1), r1, dtype)
    check("dp2", f64(dp2), r2, dtype)
    check("dI", f64(dI), rI, dtype)
    f = oracle_fwd(inp, cs, sn, th, pairing, scale, lam)
    if dtype == "f32":
        check_rel("dlambda", float(dl.item()), rl, 1e-5)
    else:
        f.update(scale=scale, lam=lam)
        check_rel("dlambda", float(dl.item()), rl, 2e-2, dlam_bound(f, f64(inp["dy"])))
    # dI' (gradient w.r.t. the mixed values) from the oracle, for the terms' magnitude
    _, _, dv_mixed, _ = oracle.relation_backward(f["q"], f["k"], f["v"], f64(inp["dy"]), scale,
                                                 2.0, lam)
    for p, (a, b) in enumerate(oracle.givens_pairs(H, pairing)):
        mag = float(np.abs(dv_mixed[:, a] * f["v"][:, b]).sum()
                    + np.abs(dv_mixed[:, b] * f["v"][:, a]).sum())
        if dtype == "f32":
            check_rel(f"dtheta[{p}]", float(dtheta[p].item()), rth[p], 1e-5, 1e-6 * mag)
        else:
            check_rel(f"dtheta[{p}]", float(dtheta[p].item()), rth[p], 2e-2, 2.0 ** -7 * mag)


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 48), ("f32", 64)])
@pytest.mark.parametrize("use_rope,use_mix", [(True, True), (True, False), (False, True)])
def test_mhr_bwd_reuses_forward_workspace(dtype, D, use_rope, use_mix):
    """Gradients computed with the forward's workspace (its rotated keys and
    mixed values, and its rotated queries where it stores them) equal those
    that form them again, bit for bit."""
    B, H, T = 1, 4, 200
    inp = make_inputs(B, H, T, D, dtype, seed=760 + D, with_dy=True)
    cs, sn, th = to_dev(*maps(T, D, H, 760, use_rope, use_mix))
    p1, p2, I, dy = (inp[n].to(DEV) for n in ("q", "k", "v", "dy"))
    lib = rel.load_library()
    code = rel.REL_BF16 if dtype == "bf16" else rel.REL_F32
    fws = torch.empty((lib.relation_mhr_fwd_workspace_bytes(code, B, H, T, D),), device=DEV,
                      dtype=torch.uint8)
    y, lse, _ = rel.relation_mhr_fwd(p1, p2, I, cs, sn, th, 1, lam=inp["lam"], scale=0.125,
                                     workspace=fws)
    a = rel.relation_mhr_bwd(p1, p2, I, y, dy, lse, cs, sn, th, 1, lam=inp["lam"], scale=0.125)
    b = rel.relation_mhr_bwd(p1, p2, I, y, dy, lse, cs, sn, th, 1, lam=inp["lam"], scale=0.125,
                             fwd_workspace=fws)
    torch.cuda.synchronize()
    for x, x1 in zip(a, b):
        assert (x is None and x1 is None) or torch.equal(x, x1)


def test_mhr_layer30m_shape_sampled_pairs():
    """The 30M layer's head geometry (H=8, D=64) at T=2048 with both maps; one
    sequence, every head computed by the oracle for the forward and two head
    pairs' gradients."""
    B, H, T, D = 1, 8, 2048, 64
    inp = make_inputs(B, H, T, D, "bf16", seed=42, with_dy=True)
    cs, sn, th = maps(T, D, H, 42, True, True)
    scale, lam = 1 / 8, inp["lam"]
    p1, p2, I, dy = (inp[n].to(DEV) for n in ("q", "k", "v", "dy"))
    dcs, dsn, dth = to_dev(cs, sn, th)
    y, lse, _ = rel.relation_mhr_fwd(p1, p2, I, dcs, dsn, dth, 1, lam=lam, scale=scale)
    dp1, dp2, dI, dl, dtheta = rel.relation_mhr_bwd(p1, p2, I, y, dy, lse, dcs, dsn, dth, 1,
                                                    lam=lam, scale=scale)
    torch.cuda.synchronize()
    f = oracle_fwd(inp, cs, sn, th, 1, scale, lam)
    check("y", f64(y), f["Y"], "bf16")
    check("lse", f64(lse), f["LSE"], "bf16")
    r1, r2, rI, rl, rth = oracle.relation_mhr_backward(
        f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["dy"]), f64(cs), f64(sn), f64(th),
        1, scale, 2.0, lam)
    check("dp1", f64(dp1), r1, "bf16")
    check("dp2", f64(dp2), r2, "bf16")
    check("dI", f64(dI), rI, "bf16")
    check_rel("dlambda", float(dl.item()), rl, 2e-2,
              dlam_bound(dict(f, scale=scale, lam=lam), f64(inp["dy"])))
