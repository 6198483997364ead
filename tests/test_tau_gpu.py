"""GPU parity away from the default Self temperature tau_S = 2 (Sec. 3.1
defines S_i = sigma(U_ii / tau_S); every other GPU test uses 2): tau_S in
{0.5, 7} for the forward and backward (bf16, fp32), decode, prefill, Multi-
Head Relation and Linear Relation, against the fp64 oracle with the same
tolerances as the rest of the suite (bf16 max-abs 2e-2 / mean-abs 3e-3, fp32
max-abs 1e-5; dL/dlambda as in test_parity_gpu)."""
import math

import numpy as np
import pytest
import torch

import exchange_relation_amd as rel
import oracle
from tests.test_parity_gpu import check, check_rel, dlambda_rounding_bound
from workloads import make_decode_inputs, make_inputs, make_linear_inputs, make_mhr_maps

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TAUS = [0.5, 7.0]


def f64(t):
    return t.detach().cpu().double().numpy()


@pytest.mark.parametrize("tau", TAUS)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fwd_bwd_tau(dtype, tau):
    B, H, T, D = 1, 2, 257, 64
    inp = make_inputs(B, H, T, D, dtype, seed=1300 + int(tau * 10), with_dy=True)
    q, k, v, dy = (inp[n].to(DEV) for n in ("q", "k", "v", "dy"))
    scale, lam = 1 / 8, inp["lam"]
    y, lse, gate = rel.relation_fwd(q, k, v, lam=lam, scale=scale, tau_s=tau, want_gate=True)
    dq, dk, dv, dl = rel.relation_bwd(q, k, v, y, dy, lse, lam=lam, scale=scale, tau_s=tau)
    torch.cuda.synchronize()
    args = [f64(inp[n]) for n in ("q", "k", "v")]
    Y, L, G = oracle.relation_forward(*args, scale, tau, lam)
    check("y", f64(y), Y, dtype)
    check("lse", f64(lse), L, dtype)
    check("gate", f64(gate), G, dtype)
    gq, gk, gv, gl = oracle.relation_backward(*args, f64(inp["dy"]), scale, tau, lam)
    check("dq", f64(dq), gq, dtype)
    check("dk", f64(dk), gk, dtype)
    check("dv", f64(dv), gv, dtype)
    if dtype == "f32":
        check_rel("dlambda", float(dl.item()), gl, 1e-5)
    else:
        heads = [(0, 0), (0, 1)]
        check_rel("dlambda", float(dl.item()), gl, 2e-2,
                  dlambda_rounding_bound(inp, heads, scale, tau, lam))


@pytest.mark.parametrize("tau", TAUS)
def test_decode_tau(tau):
    B, H, D, n = 2, 3, 64, 300
    d = make_decode_inputs(B, H, D, n, 1, n + 8, "bf16", seed=1310)
    kc, vc = d["k_cache"].to(DEV), d["v_cache"].to(DEV)
    y, g = rel.relation_cache_decode(d["q"][0].to(DEV), d["k_new"][0].to(DEV),
                                     d["v_new"][0].to(DEV), kc, vc, n, lam=d["lam"], scale=1 / 8,
                                     tau_s=tau, want_gate=True)
    torch.cuda.synchronize()
    Y, G, _, _ = oracle.relation_decode_step(f64(d["q"][0]), f64(d["k_new"][0]),
                                             f64(d["v_new"][0]), f64(d["k_cache"]),
                                             f64(d["v_cache"]), n, 1 / 8, tau, d["lam"])
    check("y", f64(y), Y, "bf16")
    check("gate", f64(g), G, "bf16")


@pytest.mark.parametrize("tau", TAUS)
def test_prefill_tau(tau):
    B, H, D, m, n = 2, 2, 64, 70, 200
    d = make_decode_inputs(B, H, D, n, m, n + m + 4, "bf16", seed=1320)
    new = {k_: d[k_].permute(1, 2, 0, 3).contiguous() for k_ in ("q", "k_new", "v_new")}
    kc, vc = d["k_cache"].to(DEV), d["v_cache"].to(DEV)
    y, lse, g = rel.relation_cache_prefill(new["q"].to(DEV), new["k_new"].to(DEV),
                                           new["v_new"].to(DEV), kc, vc, n, lam=d["lam"],
                                           scale=1 / 8, tau_s=tau, want_stats=True)
    torch.cuda.synchronize()
    Y, L, G, _, _ = oracle.relation_prefill_rows(f64(new["q"]), f64(new["k_new"]),
                                                 f64(new["v_new"]), f64(d["k_cache"]),
                                                 f64(d["v_cache"]), [n] * B, 1 / 8, tau, d["lam"])
    check("y", f64(y), Y, "bf16")
    check("lse", f64(lse), L, "bf16")
    check("gate", f64(g), G, "bf16")


@pytest.mark.parametrize("tau", TAUS)
def test_mhr_tau(tau):
    B, H, T, D = 1, 4, 150, 64
    inp = make_inputs(B, H, T, D, "bf16", seed=1330, with_dy=True)
    cs, sn, th = make_mhr_maps(T, D, H, 1330)
    p1, p2, I, dy = (inp[n].to(DEV) for n in ("q", "k", "v", "dy"))
    dcs, dsn, dth = cs.to(DEV), sn.to(DEV), th.to(DEV)
    scale, lam = 1 / 8, inp["lam"]
    y, lse, _ = rel.relation_mhr_fwd(p1, p2, I, dcs, dsn, dth, 0, lam=lam, scale=scale, tau_s=tau)
    dp1, dp2, dI, _, _ = rel.relation_mhr_bwd(p1, p2, I, y, dy, lse, dcs, dsn, dth, 0, lam=lam,
                                              scale=scale, tau_s=tau)
    torch.cuda.synchronize()
    args = (f64(inp["q"]), f64(inp["k"]), f64(inp["v"]))
    f = oracle.relation_mhr_forward(*args, f64(cs), f64(sn), f64(th), 0, scale, tau, lam)
    check("y", f64(y), f["Y"], "bf16")
    r1, r2, rI, _, _ = oracle.relation_mhr_backward(*args, f64(inp["dy"]), f64(cs), f64(sn),
                                                    f64(th), 0, scale, tau, lam)
    check("dp1", f64(dp1), r1, "bf16")
    check("dp2", f64(dp2), r2, "bf16")
    check("dI", f64(dI), rI, "bf16")


@pytest.mark.parametrize("tau", TAUS)
def test_linear_tau(tau):
    d = make_linear_inputs(1, 2, 200, 64, seed=1340)
    y, c = rel.relation_linear_fwd(*(d[n].to(DEV) for n in ("p1", "p2", "I", "g")),
                                   want_state=True, scale=1 / 8, tau_s=tau)
    torch.cuda.synchronize()
    r = oracle.linear_relation_forward(f64(d["p1"]), f64(d["p2"]), f64(d["I"]), f64(d["g"]),
                                       1 / 8, tau)
    err = np.abs(f64(y) - r["Y"])
    assert float((err / (2e-2 * np.maximum(1.0, np.abs(r["Y"]) / 4.0))).max()) <= 1.0
    assert float(err.mean()) <= 3e-3
