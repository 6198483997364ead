"""The library's calls under HIP graph capture: every entry point only
enqueues kernels on the caller's stream (no allocation, no host
synchronisation, no memset nodes), so a captured training step (relation_fwd
+ relation_bwd with lambda as a device scalar) and a captured decode step
(relation_cache_decode_noalloc) replay to the eager results. Each graph is
replayed several times with eager work of the program in between, and every
replay is checked: bit for bit, except dq, whose fp32 partials from the key
blocks are added by atomics in an order that varies from run to run (the
results then differ by a few bf16 ulps at most)."""
import math

import pytest
import torch

import exchange_relation_amd as rel
from workloads import make_decode_inputs, make_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _close_dq(a, b):
    a, b = a.float(), b.float()
    tol = 2.0 ** -6 * b.abs() + 2.0 ** -10 * float(b.abs().max())
    return bool(((a - b).abs() <= tol).all())


@pytest.mark.parametrize("B,H,T", [(2, 4, 520), (1, 3, 1)])
def test_graph_replay_training_step(B, H, T):
    D = 64
    inp = make_inputs(B, H, T, D, "bf16", seed=11, with_dy=True)
    q, k, v, dy = (inp[n].to(DEV) for n in ("q", "k", "v", "dy"))
    lam = torch.tensor([inp["lam"]], device=DEV, dtype=torch.float32)
    scale = 1 / math.sqrt(D)
    y, lse = torch.empty_like(q), torch.empty((B, H, T), device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dl = torch.empty((1,), device=DEV)
    wsf = torch.empty((max(rel.relation_fwd_workspace_bytes(torch.bfloat16, B, H, T, D), 1),),
                      device=DEV, dtype=torch.uint8)
    wsb = torch.empty((rel.relation_bwd_workspace_bytes(torch.bfloat16, B, H, T, D),),
                      device=DEV, dtype=torch.uint8)

    def step():
        rel.relation_fwd(q, k, v, lam=lam, scale=scale, y=y, lse=lse, workspace=wsf)
        rel.relation_bwd(q, k, v, y, dy, lse, lam=lam, scale=scale, dq=dq, dk=dk, dv=dv,
                         dlambda=dl, workspace=wsb)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (y, lse, dq, dk, dv, dl)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream's side, as torch asks
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (y, lse, dq, dk, dv, dl):  # eager work between replays
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"  B={B} H={H} T={T} replay {rep}")
        assert torch.equal(y, ref[0]) and torch.equal(lse, ref[1])
        assert torch.equal(dk, ref[3]) and torch.equal(dv, ref[4]) and torch.equal(dl, ref[5])
        assert _close_dq(dq, ref[2])


def test_graph_replay_decode_noalloc():
    B, H, D, n, cap = 4, 6, 64, 700, 720
    d = make_decode_inputs(B, H, D, n, 1, cap, "bf16", seed=13)
    q, kn, vn = (d[x][0].to(DEV) for x in ("q", "k_new", "v_new"))
    kc, vc = d["k_cache"].to(DEV), d["v_cache"].to(DEV)
    y, gate = torch.empty_like(q), torch.empty((B, H), device=DEV)
    scale = 1 / math.sqrt(D)

    def step():  # appends the same row at the same slot: replays are idempotent
        rel.relation_cache_decode_noalloc(q, kn, vn, kc, vc, n, y, lam=d["lam"], scale=scale,
                                          gate=gate)

    step()
    torch.cuda.synchronize()
    ref_y, ref_g, ref_k, ref_v = y.clone(), gate.clone(), kc.clone(), vc.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        y.fill_(float("nan"))
        gate.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"  decode replay {rep}")
        assert torch.equal(y, ref_y) and torch.equal(gate, ref_g)
        assert torch.equal(kc, ref_k) and torch.equal(vc, ref_v)
