"""The autograd wrappers (exchange_relation_amd.relation, .mhr_relation):
forward and backward through torch.autograd give the direct C-ABI calls'
results (y, lse-based gradients) bit for bit, except dq / dp1, which the
backward accumulates with fp32 atomics in an unspecified order and which is
therefore compared within the bf16 tolerance (max-abs 2e-2, mean-abs 3e-3)
against the direct call and the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import exchange_relation_amd as rel
import oracle
from workloads import make_inputs, make_mhr_maps

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def close(a, b):
    d = (a.float() - b.float()).abs()
    assert float(d.max()) <= 2e-2 and float(d.mean()) <= 3e-3


def test_relation_autograd_matches_direct_calls_and_oracle():
    B, H, T, D = 1, 2, 300, 64
    inp = make_inputs(B, H, T, D, "bf16", seed=1200, with_dy=True)
    q, k, v, dy = (inp[n].to(DEV) for n in ("q", "k", "v", "dy"))
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    lam = torch.tensor([inp["lam"]], device=DEV, requires_grad=True)
    y = rel.relation(qa, ka, va, lam, scale=1 / 8)
    y.backward(dy)
    y0, lse0, _ = rel.relation_fwd(q, k, v, lam=inp["lam"], scale=1 / 8)
    dq0, dk0, dv0, dl0 = rel.relation_bwd(q, k, v, y0, dy, lse0, lam=inp["lam"], scale=1 / 8)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    assert torch.equal(ka.grad, dk0) and torch.equal(va.grad, dv0)
    assert lam.grad.shape == lam.shape and torch.equal(lam.grad, dl0.reshape(lam.shape))
    close(qa.grad, dq0)
    gq = oracle.relation_backward(*(inp[n].double().numpy() for n in ("q", "k", "v", "dy")),
                                  1 / 8, 2.0, inp["lam"])[0]
    err = np.abs(qa.grad.detach().cpu().double().numpy() - gq)
    assert err.max() <= 2e-2 and err.mean() <= 3e-3


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mhr_relation_autograd_matches_direct_calls(dtype):
    B, H, T, D = 1, 4, 200, 64
    inp = make_inputs(B, H, T, D, dtype, seed=1210, with_dy=True)
    cs, sn, th = (t.to(DEV) for t in make_mhr_maps(T, D, H, 1210))
    p1, p2, I, dy = (inp[n].to(DEV) for n in ("q", "k", "v", "dy"))
    pa, pb, ia = (x.clone().requires_grad_(True) for x in (p1, p2, I))
    tha = th.clone().requires_grad_(True)
    lam = torch.tensor(inp["lam"], device=DEV, requires_grad=True)
    scale = 1 / math.sqrt(D)
    y = rel.mhr_relation(pa, pb, ia, lam, tha, cs, sn, 1, scale=scale)
    y.backward(dy)
    y0, lse0, _ = rel.relation_mhr_fwd(p1, p2, I, cs, sn, th, 1, lam=inp["lam"], scale=scale)
    g0 = rel.relation_mhr_bwd(p1, p2, I, y0, dy, lse0, cs, sn, th, 1, lam=inp["lam"], scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(y, y0)
    assert torch.equal(pb.grad, g0[1]) and torch.equal(ia.grad, g0[2])
    assert torch.equal(lam.grad, g0[3].reshape(())) and torch.equal(tha.grad, g0[4])
    if dtype == "f32":  # the fp32 path has no atomics
        assert torch.equal(pa.grad, g0[0])
    else:
        close(pa.grad, g0[0])


def test_linear_relation_autograd_matches_direct_calls_and_oracle():
    """exchange_relation_amd.linear_relation: y and the final state from the
    forward, and through autograd (with gradients on both outputs) the same
    gradients as the direct three-pass relation_linear_bwd, bit for bit (the
    wrapper's backward reuses the forward's per-chunk states); dp1 also
    against the fp64 oracle."""
    from workloads import make_linear_inputs
    B, H, T, D = 2, 2, 260, 64
    d = make_linear_inputs(B, H, T, D, seed=1300, with_dy=True)
    p1, p2, I, g, dy = (d[n].to(DEV) for n in ("p1", "p2", "I", "g", "dy"))
    cs, sn, _ = (t.to(DEV) for t in make_mhr_maps(T, D, 2, 1300))
    gen = torch.Generator().manual_seed(1301)
    C0 = (0.1 * torch.randn(B, H, D, D, generator=gen)).to(DEV)
    dCT = torch.randn(B, H, D, D, generator=gen).to(DEV)
    scale = 1 / math.sqrt(D)
    leaves = [x.clone().requires_grad_(True) for x in (p1, p2, I, g, C0)]
    y, cT = rel.linear_relation(*leaves, rope_cos=cs, rope_sin=sn, scale=scale)
    ((y.float() * dy.float()).sum() + (cT * dCT).sum()).backward()
    y0, c0 = rel.relation_linear_fwd(p1, p2, I, g, cs, sn, C0, want_state=True, scale=scale)
    ref = rel.relation_linear_bwd(p1, p2, I, g, dy, cs, sn, C0, dstate_out=dCT,
                                  want_dstate_in=True, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), y0) and torch.equal(cT.detach(), c0)
    for name, leaf, r in zip(("dp1", "dp2", "dI", "dg", "dstate_in"), leaves, ref):
        assert torch.equal(leaf.grad, r), name
    o = oracle.linear_relation_backward(
        *(d[n].double().numpy() for n in ("p1", "p2", "I", "g", "dy")), scale, 2.0,
        cs.cpu().double().numpy(), sn.cpu().double().numpy(), C0=C0.cpu().double().numpy(),
        dC_T=dCT.cpu().double().numpy())
    ref_dp1 = o["dp1"] if isinstance(o, dict) else o[0]
    err = np.abs(leaves[0].grad.cpu().double().numpy() - ref_dp1)
    assert float(err.max()) <= 2e-2 * max(1.0, float(np.abs(ref_dp1).max()) / 4)


# ------------------------------------------------- lambda read on the device
def _lam_t(x):
    return torch.tensor([x], device=DEV, dtype=torch.float32)


@pytest.mark.parametrize("dtype,D,T,split", [("bf16", 64, 300, False), ("bf16", 48, 257, False),
                                             ("bf16", 80, 200, False), ("f32", 32, 130, False),
                                             ("bf16", 64, 2100, True)])
def test_device_lambda_forward_bit_identical(dtype, D, T, split):
    """relation_fwd with lambda as a device scalar (read by the kernels when
    they run) equals the call with lambda by value, bit for bit, including
    the split-over-keys path and its combine kernel."""
    B, H = (1, 2) if not split else (1, 4)
    inp = make_inputs(B, H, T, D, dtype, seed=1300 + D + T, lam=0.731)
    q, k, v = (inp[n].to(DEV) for n in ("q", "k", "v"))
    kw = dict(scale=1 / math.sqrt(D), want_gate=True, split=split)
    a = rel.relation_fwd(q, k, v, lam=0.731, **kw)
    b = rel.relation_fwd(q, k, v, lam=_lam_t(0.731), **kw)
    torch.cuda.synchronize()
    for x, y_ in zip(a, b):
        assert torch.equal(x, y_)


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 48), ("bf16", 80), ("f32", 32)])
def test_device_lambda_backward(dtype, D):
    """relation_bwd with a device lambda: dk, dv and dL/dlambda bit for bit
    against lambda by value; dq (fp32 atomics, unspecified order) within
    1e-6 of its magnitude."""
    B, H, T = 1, 2, 200
    inp = make_inputs(B, H, T, D, dtype, seed=1400 + D, with_dy=True, lam=-0.37)
    q, k, v, dy = (inp[n].to(DEV) for n in ("q", "k", "v", "dy"))
    s = 1 / math.sqrt(D)
    y, lse, _ = rel.relation_fwd(q, k, v, lam=-0.37, scale=s)
    a = rel.relation_bwd(q, k, v, y, dy, lse, lam=-0.37, scale=s)
    b = rel.relation_bwd(q, k, v, y, dy, lse, lam=_lam_t(-0.37), scale=s)
    torch.cuda.synchronize()
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2]) and torch.equal(a[3], b[3])
    d = (a[0].float() - b[0].float()).abs().max()
    assert float(d) <= 1e-6 * max(1.0, float(a[0].float().abs().max())) + (
        0.0 if dtype == "f32" else 2.0 ** -7 * float(a[0].float().abs().max()))


def test_device_lambda_mhr_bit_identical():
    B, H, T, D = 1, 4, 150, 64
    inp = make_inputs(B, H, T, D, "bf16", seed=1500, with_dy=True, lam=1.25)
    cs, sn, th = (t.to(DEV) for t in make_mhr_maps(T, D, H, 1500))
    p1, p2, I, dy = (inp[n].to(DEV) for n in ("q", "k", "v", "dy"))
    a = rel.relation_mhr_fwd(p1, p2, I, cs, sn, th, 0, lam=1.25, scale=1 / 8)
    b = rel.relation_mhr_fwd(p1, p2, I, cs, sn, th, 0, lam=_lam_t(1.25), scale=1 / 8)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    ga = rel.relation_mhr_bwd(p1, p2, I, a[0], dy, a[1], cs, sn, th, 0, lam=1.25, scale=1 / 8)
    gb = rel.relation_mhr_bwd(p1, p2, I, a[0], dy, a[1], cs, sn, th, 0, lam=_lam_t(1.25),
                              scale=1 / 8)
    torch.cuda.synchronize()
    assert torch.equal(ga[1], gb[1]) and torch.equal(ga[2], gb[2]) and torch.equal(ga[3], gb[3])


def test_autograd_step_needs_no_host_synchronisation():
    """A forward + backward through the autograd wrappers with a learnable
    lambda on the device runs with torch's synchronisation debugging set to
    raise: lambda is never copied to the host."""
    B, H, T, D = 1, 2, 256, 64
    inp = make_inputs(B, H, T, D, "bf16", seed=1600, with_dy=True)
    q, k, v, dy = (inp[n].to(DEV) for n in ("q", "k", "v", "dy"))
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    lam = torch.tensor([inp["lam"]], device=DEV, requires_grad=True)
    cs, sn, th = (t.to(DEV) for t in make_mhr_maps(T, D, H, 1600))
    tha = th.clone().requires_grad_(True)
    torch.cuda.synchronize()
    torch.cuda.set_sync_debug_mode("error")
    try:
        y = rel.relation(qa, ka, va, lam, scale=1 / 8)
        y.backward(dy)
        y2 = rel.mhr_relation(qa, ka, va, lam, tha, cs, sn, 0, scale=1 / 8)
        y2.backward(dy)
    finally:
        torch.cuda.set_sync_debug_mode("default")
    torch.cuda.synchronize()
    assert lam.grad is not None and bool(torch.isfinite(lam.grad).all())
