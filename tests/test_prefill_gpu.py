"""GPU parity of the chunked Relation Cache prefill (relation_cache_prefill):
m new tokens per sequence appended at slot n_b and their rows computed
against the cache, uniform and ragged history lengths, against the fp64
oracle (oracle.relation_prefill_rows). bf16 tolerances as everywhere
(max-abs <= 2e-2, mean-abs <= 3e-3); the cache must match bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import exchange_relation_amd as rel
import oracle
from workloads import make_decode_inputs, make_inputs, ragged_decode_lengths

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
BF16_MAX, BF16_MEAN = 2e-2, 3e-3


def f64(t):
    return t.detach().cpu().double().numpy()


def check(name, got, ref):
    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    mx, mean = float(err.max()), float(err.mean())
    print(f"  {name}: max-abs {mx:.3e} mean-abs {mean:.3e}")
    assert mx <= BF16_MAX, f"{name}: max-abs {mx:.3e} > {BF16_MAX}"
    assert mean <= BF16_MEAN, f"{name}: mean-abs {mean:.3e} > {BF16_MEAN}"


def prefill_inputs(B, H, D, m, cap, seed):
    """Caches with every slot filled and m new tokens per sequence as
    [B, H, m, D]."""
    d = make_decode_inputs(B, H, D, cap - m, m, cap, "bf16", seed=seed)
    new = {n: d[n].permute(1, 2, 0, 3).contiguous() for n in ("q", "k_new", "v_new")}
    return d, new


def run(d, new, n, bound=None, split=True):
    kc, vc = d["k_cache"].to(DEV), d["v_cache"].to(DEV)
    nh = torch.tensor(n, dtype=torch.int32, device=DEV) if isinstance(n, list) else n
    y, lse, g = rel.relation_cache_prefill(new["q"].to(DEV), new["k_new"].to(DEV),
                                           new["v_new"].to(DEV), kc, vc, nh, max_n_hist=bound,
                                           lam=d["lam"], scale=1 / 8, want_stats=True,
                                           split=split)
    torch.cuda.synchronize()
    return y.cpu(), lse.cpu(), g.cpu(), kc.cpu(), vc.cpu()


def oracle_rows(d, new, ns):
    return oracle.relation_prefill_rows(f64(new["q"]), f64(new["k_new"]), f64(new["v_new"]),
                                        f64(d["k_cache"]), f64(d["v_cache"]), ns, 1 / 8, 2.0,
                                        d["lam"])


@pytest.mark.parametrize("n,m", [(0, 1), (0, 130), (1, 7), (31, 64), (64, 64), (100, 257),
                                 (500, 33), (777, 128)])
def test_prefill_uniform_vs_oracle(n, m):
    B, H, D = 2, 3, 64
    d, new = prefill_inputs(B, H, D, m, n + m + 9, seed=900 + n + m)
    y, lse, g, kc, vc = run(d, new, n)
    Y, L, G, KC, VC = oracle_rows(d, new, [n] * B)
    check("y", f64(y), Y)
    check("lse", f64(lse), L)
    check("gate", f64(g), G)
    assert np.array_equal(f64(kc), KC) and np.array_equal(f64(vc), VC)


def test_prefill_ragged_vs_oracle():
    B, H, D, m, cap = 6, 2, 64, 100, 800
    ns = [0, 1, 33, 129, 500, 700]
    d, new = prefill_inputs(B, H, D, m, cap, seed=931)
    y, lse, g, kc, vc = run(d, new, ns, bound=max(ns))
    Y, L, G, KC, VC = oracle_rows(d, new, ns)
    check("y", f64(y), Y)
    check("lse", f64(lse), L)
    assert np.array_equal(f64(kc), KC) and np.array_equal(f64(vc), VC)


@pytest.mark.parametrize("ns,bound", [([0, 1, 33, 900, 1700, 2200], 2200), ([2200] * 6, None)])
def test_prefill_split_over_keys_matches_unsplit(ns, bound):
    """Long histories split over several workgroups (merged by App. A.3.2's
    rule) give the unsplit rows up to the bf16 rounding of P = exp(E - m),
    which each piece takes against its own stabiliser m: y within 2^-8 max|v|
    plus one bf16 unit in the last place, lse and gate within 2^-8; the
    cache bit for bit."""
    B, H, D, m, cap = 6, 2, 64, 100, 2400
    per_seq = bound is not None
    n = max(ns) if per_seq else ns[0]
    assert rel.relation_prefill_workspace_bytes(torch.bfloat16, B, H, D, m, n, per_seq) > 0
    d, new = prefill_inputs(B, H, D, m, cap, seed=933)
    arg = ns if per_seq else ns[0]
    y, lse, g, kc, vc = run(d, new, arg, bound=bound)
    y1, l1, g1, kc1, vc1 = run(d, new, arg, bound=bound, split=False)
    vmax = max(float(d["v_cache"].float().abs().max()), float(new["v_new"].float().abs().max()))
    d_y = (y.float() - y1.float()).abs()
    bound = 2.0 ** -8 * vmax + torch.clamp(y1.float().abs(), min=2.0 ** -126) * 2.0 ** -7
    print(f"  y: max diff {d_y.max().item():.3e}, differing {(d_y > 0).float().mean().item():.2e}")
    assert bool((d_y <= bound).all()) and float((d_y > 0).float().mean()) < 0.05
    assert bool(((lse - l1).abs() <= 2.0 ** -8).all())
    assert bool(((g - g1).abs() <= 2.0 ** -8).all())
    assert torch.equal(kc, kc1) and torch.equal(vc, vc1)
    Y, L, G, _, _ = oracle_rows(d, new, ns)
    check("y", f64(y), Y)
    check("lse", f64(lse), L)


def test_prefill_split_with_out_of_range_sequence():
    """Split over keys with a sequence whose length is above the bound: its
    rows are NaN and its cache rows untouched; the others match the oracle."""
    B, H, D, m, cap = 3, 2, 64, 100, 2400
    ns = [500, 2290, 2200]  # bound 2200: sequence 1 is above it
    assert rel.relation_prefill_workspace_bytes(torch.bfloat16, B, H, D, m, 2200, True) > 0
    d, new = prefill_inputs(B, H, D, m, cap, seed=939)
    y, lse, g, kc, vc = run(d, new, ns, bound=2200)
    assert np.isnan(f64(y[1])).all() and np.isnan(f64(lse[1])).all()
    assert torch.equal(kc[1], d["k_cache"][1]) and torch.equal(vc[1], d["v_cache"][1])
    Y, L, _, _, _ = oracle_rows(
        {**d, "k_cache": d["k_cache"][[0, 2]], "v_cache": d["v_cache"][[0, 2]]},
        {k: t[[0, 2]] for k, t in new.items()}, [500, 2200])
    check("valid rows", f64(y[[0, 2]]), Y)
    check("valid lse", f64(lse[[0, 2]]), L)


def test_prefill_ragged_out_of_range_nan_and_no_write():
    B, H, D, m, cap = 3, 2, 64, 16, 96
    ns = [10, 90, 20]  # bound 40: sequence 1 is above it (and would not fit)
    d, new = prefill_inputs(B, H, D, m, cap, seed=937)
    y, lse, g, kc, vc = run(d, new, ns, bound=40)
    assert np.isnan(f64(y[1])).all() and np.isnan(f64(lse[1])).all()
    assert torch.equal(kc[1], d["k_cache"][1]) and torch.equal(vc[1], d["v_cache"][1])
    Y, L, _, _, _ = oracle_rows(
        {**d, "k_cache": d["k_cache"][[0, 2]], "v_cache": d["v_cache"][[0, 2]]},
        {k: t[[0, 2]] for k, t in new.items()}, [10, 20])
    check("valid rows", f64(y[[0, 2]]), Y)


def test_prefill_from_empty_history_is_the_forward_bit_exact():
    # 192 heads: the forward runs 128-row blocks, as the prefill always does
    # (a small grid would take its 64-row split-key blocks instead)
    B, H, T, D = 4, 48, 300, 64
    inp = make_inputs(B, H, T, D, "bf16", seed=941)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    yf, lf, gf = rel.relation_fwd(q, k, v, lam=inp["lam"], scale=1 / 8, want_gate=True)
    kc = torch.zeros((B, H, T + 4, D), device=DEV, dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    yp, lp, gp = rel.relation_cache_prefill(q, k, v, kc, vc, 0, lam=inp["lam"], scale=1 / 8,
                                            want_stats=True)
    torch.cuda.synchronize()
    assert torch.equal(yf, yp) and torch.equal(lf, lp) and torch.equal(gf, gp)


def test_prefill_cache_workload_shape_ragged():
    """The cache workload's shape (B=32, H=12, capacity 4352) with 256 new
    tokens per sequence at ragged offsets; sampled sequences vs the oracle."""
    B, H, D, m, cap = 32, 12, 64, 256, 4352
    ns = ragged_decode_lengths(B, cap - m, seed=42)
    d, new = prefill_inputs(B, H, D, m, cap, seed=42)
    y, lse, g, kc, vc = run(d, new, ns, bound=cap - m)
    for b in (0, 1, 7, 19):
        sub = {"k_cache": d["k_cache"][b:b + 1], "v_cache": d["v_cache"][b:b + 1],
               "lam": d["lam"]}
        Y, L, _, KC, VC = oracle_rows(sub, {k: t[b:b + 1] for k, t in new.items()}, [ns[b]])
        check(f"y seq {b}", f64(y[b:b + 1]), Y)
        check(f"lse seq {b}", f64(lse[b:b + 1]), L)
        assert np.array_equal(f64(kc[b:b + 1]), KC)
