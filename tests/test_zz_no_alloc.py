"""The allocation-free decode entry point (relation_cache_decode_noalloc,
for callers that cannot allocate device memory) against
relation_cache_decode through the C ABI: the same kernels on the same
inputs, so outputs and caches must agree bit for bit. Two calls in a row,
the second on a smaller input (the static scratch keeps the first call's
contents), on the cache workload's shape (one workgroup per head) and then
on a small batch whose history is split over workgroups through the
scratch; a third call at history 0."""
import math

import pytest
import torch

import exchange_relation_amd as rel
from workloads import make_decode_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def one_pair(B, H, D, n, cap, dtype, seed):
    d = make_decode_inputs(B, H, D, n, 1, cap, dtype, seed=seed)
    q, kn, vn = (d[k][0].to(DEV) for k in ("q", "k_new", "v_new"))
    kc1, vc1 = d["k_cache"].to(DEV), d["v_cache"].to(DEV)
    kc2, vc2 = kc1.clone(), vc1.clone()
    scale = 1 / math.sqrt(D)
    y1, g1 = rel.relation_cache_decode(q, kn, vn, kc1, vc1, n, lam=d["lam"], scale=scale,
                                       want_gate=True)
    y2 = torch.full_like(q, float("nan"))
    g2 = torch.full((B, H), float("nan"), device=DEV)
    rel.relation_cache_decode_noalloc(q, kn, vn, kc2, vc2, n, y2, lam=d["lam"], scale=scale,
                                      gate=g2)
    torch.cuda.synchronize()
    print(f"  B={B} H={H} D={D} n={n} cap={cap} {dtype}: max |y diff| "
          f"{float((y1.float() - y2.float()).abs().max()):.3e}")
    assert torch.equal(y1, y2)
    assert torch.equal(g1, g2)
    assert torch.equal(kc1, kc2) and torch.equal(vc1, vc2)


def test_noalloc_decode_matches_workspace_decode_two_calls():
    one_pair(32, 12, 64, 4096, 4352, "bf16", seed=42)   # the cache workload's shape
    one_pair(2, 3, 64, 1500, 1600, "bf16", seed=7)      # smaller, split over the scratch
    one_pair(2, 3, 64, 0, 8, "bf16", seed=8)            # empty history


def test_noalloc_decode_fp32_and_widths():
    one_pair(1, 4, 32, 700, 720, "f32", seed=9)
    one_pair(3, 2, 80, 999, 1024, "bf16", seed=10)
    one_pair(3, 2, 48, 513, 520, "bf16", seed=11)


def test_noalloc_many_heads_need_no_scratch():
    """From 256 heads on, the uniform step runs one workgroup per head and
    uses no scratch, so a batch whose capacity-sized workspace is larger
    than the 8 MiB array (4096 heads at capacity 2048) is still served, bit
    for bit equal to relation_cache_decode; then a small split call reuses
    the scratch."""
    B, H, D, n, cap = 32, 128, 64, 1000, 2048
    assert rel.relation_decode_workspace_bytes(torch.bfloat16, B, H, D, cap) > 8 << 20
    g = torch.Generator(device=DEV).manual_seed(5)

    def rnd(*shape):
        return torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16)
    q, kn, vn = rnd(B, H, D), rnd(B, H, D), rnd(B, H, D)
    kc1, vc1 = rnd(B, H, cap, D), rnd(B, H, cap, D)
    kc2, vc2 = kc1.clone(), vc1.clone()
    scale = 1 / math.sqrt(D)
    y1, g1 = rel.relation_cache_decode(q, kn, vn, kc1, vc1, n, lam=0.3, scale=scale,
                                       want_gate=True)
    y2 = torch.full_like(q, float("nan"))
    g2 = torch.full((B, H), float("nan"), device=DEV)
    rel.relation_cache_decode_noalloc(q, kn, vn, kc2, vc2, n, y2, lam=0.3, scale=scale, gate=g2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(g1, g2)
    assert torch.equal(kc1, kc2) and torch.equal(vc1, vc2)
    del kc1, vc1, kc2, vc2
    one_pair(2, 3, 64, 1500, 1600, "bf16", seed=12)
