"""GPU parity over seeded random shapes: the bf16 forward and backward (and
the fp32 forward) on every head of a launch against the fp64 oracle, and the
chunked cache prefill on ragged histories (its caches bit for bit).

The shapes are drawn so that one sweep reaches every forward launch form:
* the 64-row split-key blocks of grids that fit the GPU at once;
* the 128-row blocks of larger grids;
* the pieces split over keys of long, few-head launches.
Row counts are ragged, and the bf16 head widths are 48, 64 and 80 (the paper's
three widths, App. B, Table 6); the fp32 path runs 32 and 64.

Tolerances are the same as in the other parity tests. bf16: max-abs 2e-2 and
mean-abs 3e-3 on y, lse, gate, dq, dk and dv. An output of magnitude >= 4
loses up to 2^-8 |ref| (1.56e-2) to its bf16 rounding alone, so the
largest errors of the sweep sit there (dv 1.95e-2 at |ref| = 4.43). dL/dlambda (one scalar over all heads; Sec. 3.1,
App. A.1.7) must be within 2e-2 relative, plus the bound that the bf16
rounding of the stored Y allows. fp32: max-abs 1e-5.
"""
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import exchange_relation_amd as rel
import oracle
from workloads import make_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
BF16_MAX, BF16_MEAN = 2e-2, 3e-3
F32_MAX = 1e-5
NCASE = 12


def f64(t):
    return t.detach().cpu().double().numpy()


def case(i):
    """Shape (B, H, T, D) of case i, by i % 3:
    0: long rows on 1-3 heads (the launch may split over keys);
    1: a grid of at most 512 64-row blocks (split-key blocks);
    2: more than 768 64-row blocks (128-row blocks)."""
    rng = np.random.default_rng(9100 + i)
    D = int(rng.choice([48, 64, 80]))
    kind = i % 3
    if kind == 0:
        B, H, T = 1, int(rng.integers(1, 4)), int(rng.integers(1000, 1500))
    elif kind == 1:
        B, H, T = int(rng.integers(1, 4)), int(rng.integers(1, 17)), int(rng.integers(1, 601))
        while B * H * ((T + 63) // 64) > 512:
            H = max(1, H // 2)
    else:
        B, H, T = int(rng.integers(3, 5)), int(rng.integers(32, 49)), int(rng.integers(520, 701))
    return B, H, T, D


def check(name, got, ref, dtype):
    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    mx, mean = float(err.max()), float(err.mean())
    at = np.unravel_index(int(err.argmax()), err.shape)
    print(f"  {name}: max-abs {mx:.3e} (|ref| there {abs(float(ref[at])):.3g}) mean-abs {mean:.3e}")
    if dtype == "f32":
        assert mx <= F32_MAX, f"{name}: max-abs {mx:.3e} > {F32_MAX}"
        return
    assert mx <= BF16_MAX, f"{name}: max-abs {mx:.3e} > {BF16_MAX}"
    assert mean <= BF16_MEAN, f"{name}: mean-abs {mean:.3e} > {BF16_MEAN}"


def oracle_heads(inp, B, H, scale, tau, lam, backward=True):
    """fp64 oracle of every head, several heads at a time (numpy releases the
    interpreter lock in its array work)."""
    def one(bh):
        b, h = bh
        q, k, v = f64(inp["q"][b, h]), f64(inp["k"][b, h]), f64(inp["v"][b, h])
        if not backward:
            return oracle.relation_forward_head(q, k, v, scale, tau, lam)
        G = f64(inp["dy"][b, h])
        r = oracle.relation_backward_head(q, k, v, G, scale, tau, lam)
        fw = r["fwd"]
        T = G.shape[0]
        logi = np.log(np.arange(1, T + 1, dtype=np.float64))
        # this head's term of the bound on dL/dlambda from the bf16 rounding of
        # the stored Y (before its 2^-9 factor)
        r["rbound"] = float((logi * np.diag(fw["F"]) * np.abs(G * fw["Y"]).sum(axis=1)).sum())
        return r
    heads = [(b, h) for b in range(B) for h in range(H)]
    nthr = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(nthr) as ex:
        return list(ex.map(one, heads))


@pytest.mark.parametrize("i", range(NCASE))
def test_sweep_bf16_fwd_bwd_every_head(i):
    B, H, T, D = case(i)
    print(f"case {i}: B={B} H={H} T={T} D={D}", flush=True)
    inp = make_inputs(B, H, T, D, "bf16", seed=9200 + i, with_dy=True)
    scale, tau, lam = 1 / math.sqrt(D), 2.0, inp["lam"]
    q, k, v, dy = (inp[n].to(DEV) for n in ("q", "k", "v", "dy"))
    y, lse, gate = rel.relation_fwd(q, k, v, lam=lam, scale=scale, tau_s=tau, want_gate=True)
    dq, dk, dv, dl = rel.relation_bwd(q, k, v, y, dy, lse, lam=lam, scale=scale, tau_s=tau)
    torch.cuda.synchronize()
    ref = oracle_heads(inp, B, H, scale, tau, lam)

    def stack(vals, *shape):
        return np.stack(vals).reshape(B, H, T, *shape)

    check("y", f64(y), stack([r["fwd"]["Y"] for r in ref], D), "bf16")
    check("lse", f64(lse), stack([r["fwd"]["LSE"] for r in ref]), "bf16")
    check("gate", f64(gate), stack([r["fwd"]["g"] for r in ref]), "bf16")
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        check(name, f64(t), stack([r[name] for r in ref], D), "bf16")
    gl = float(sum(r["dlam"] for r in ref))
    extra = 2.0 ** -9 * sum(r["rbound"] for r in ref)
    got = float(dl.item())
    bound = 2e-2 * max(1.0, abs(gl)) + extra
    print(f"  dlambda: {got:.6g} vs {gl:.6g} (bound {bound:.3e})")
    assert abs(got - gl) <= bound


@pytest.mark.parametrize("i", [0, 2, 4, 6, 9, 11])
def test_sweep_f32_fwd_every_head(i):
    B, H, T, D = case(i)
    D = 32 if D < 64 else 64  # the fp32 path's widths
    print(f"case {i}: B={B} H={H} T={T} D={D}", flush=True)
    inp = make_inputs(B, H, T, D, "f32", seed=9300 + i)
    scale, tau, lam = 1 / math.sqrt(D), 2.0, inp["lam"]
    y, lse, gate = rel.relation_fwd(*(inp[n].to(DEV) for n in ("q", "k", "v")), lam=lam,
                                    scale=scale, tau_s=tau, want_gate=True)
    torch.cuda.synchronize()
    ref = oracle_heads(inp, B, H, scale, tau, lam, backward=False)
    check("y", f64(y), np.stack([r["Y"] for r in ref]).reshape(B, H, T, D), "f32")
    check("lse", f64(lse), np.stack([r["LSE"] for r in ref]).reshape(B, H, T), "f32")
    check("gate", f64(gate), np.stack([r["g"] for r in ref]).reshape(B, H, T), "f32")


def prefill_case(i):
    """(B, H, D, m, ns, cap) of prefill case i: m new tokens per sequence
    after ragged histories ns (some long enough to split over keys)."""
    rng = np.random.default_rng(9400 + i)
    D = int(rng.choice([48, 64, 80]))
    B, H, m = int(rng.integers(1, 5)), int(rng.integers(1, 7)), int(rng.integers(1, 301))
    ns = [int(x) for x in rng.integers(0, 1800, size=B)]
    if B > 1:
        ns[0] = 0  # one sequence with no history
    cap = max(ns) + m + int(rng.integers(0, 40))
    return B, H, D, m, ns, cap


@pytest.mark.parametrize("i", range(6))
def test_sweep_prefill_ragged_every_head(i):
    """Chunked prefill (relation_cache_prefill) on ragged histories: every row
    of every head against the oracle's rows of the whole sequence, and the
    caches bit for bit."""
    from workloads import make_decode_inputs
    B, H, D, m, ns, cap = prefill_case(i)
    print(f"prefill case {i}: B={B} H={H} D={D} m={m} histories={ns} capacity={cap}", flush=True)
    d = make_decode_inputs(B, H, D, cap - m, m, cap, "bf16", seed=9500 + i)
    new = {n: d[n].permute(1, 2, 0, 3).contiguous() for n in ("q", "k_new", "v_new")}
    scale = 1 / math.sqrt(D)
    kc, vc = d["k_cache"].to(DEV), d["v_cache"].to(DEV)
    y, lse, g = rel.relation_cache_prefill(
        new["q"].to(DEV), new["k_new"].to(DEV), new["v_new"].to(DEV), kc, vc,
        torch.tensor(ns, dtype=torch.int32, device=DEV), max_n_hist=max(ns), lam=d["lam"],
        scale=scale, want_stats=True)
    torch.cuda.synchronize()
    Y, L, G, KC, VC = oracle.relation_prefill_rows(f64(new["q"]), f64(new["k_new"]),
                                                   f64(new["v_new"]), f64(d["k_cache"]),
                                                   f64(d["v_cache"]), ns, scale, 2.0, d["lam"])
    check("y", f64(y), Y, "bf16")
    check("lse", f64(lse), L, "bf16")
    check("gate", f64(g), G, "bf16")
    assert np.array_equal(f64(kc), KC) and np.array_equal(f64(vc), VC)
