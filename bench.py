"""Benchmark of librelation on one MI355X.

A step is one pass of the Relation hot path over one batch: relation_fwd then
relation_bwd on the 30M-model-shaped layer (B=16, H=8, T=2048, D=64, bf16,
causal). The JSON line's `value` is that step's algorithmic throughput in
TFLOP/s (fwd = 2*B*H*T^2*D flops, bwd = 2.5x fwd). The same run also measures
the forward alone on the 10M / 30M / 100M layer shapes, forward+backward on
the 100M shape beside torch's causal scaled-dot-product attention of the same
shape, and 256 Relation Cache decode steps (B=32, H=12, D=64, history 4096) in
GB/s, plus the fp64 CPU oracle on a bounded sample of every workload
(cpu_baseline). Before the W warm-up steps, untimed steps run for
--prewarm-ms of wall time so that the timed window starts at steady clocks
(reported as prewarm_ms / prewarm_steps). The extra
lines cover ragged decode, chunked prefill, Multi-Head Relation and Linear
Relation (forward, backward, decode step); `roofline*` objects price the
dominant kernel of each against MI355X's published peaks.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--prewarm-ms MS]
                       [--no-cpu-baseline] [--no-extra]
                       [--only {step,fwd,fwd10m,fwd100m,decode,ragged,mhr,prefill,
                                attn,linear,copy,cpu}]
--only runs one workload and prints its raw numbers (one workload per run, so
that a profile of it holds that workload alone).
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
METRIC = "Full Relation fwd / fwd+bwd TFLOP/s and % bf16 MFMA peak; decode GB/s"


def fwd_flops(B, H, T, D):
    return 2.0 * B * H * T * T * D


def decode_bytes(B, H, D, n):
    """Algorithmic bytes of one decode step at history n (bf16): read K and V
    history (4 B H n D) + q, k_new, v_new reads, cache-slot writes, y write."""
    return 4.0 * B * H * n * D + 10.0 * B * H * D


class EventTimer:
    """HIP events recorded on the stream the library launches on."""

    def __init__(self, torch, stream):
        self.torch, self.stream, self.pairs = torch, stream, []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        return e

    def stop(self, s):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record(self.stream)
        self.pairs.append((s, e))

    def mean_ms(self):
        self.torch.cuda.synchronize()
        v = [a.elapsed_time(b) for a, b in self.pairs]
        return sum(v) / len(v) if v else float("nan")


def prewarm(torch, fn, ms):
    """Clock ramp: call fn() back to back until `ms` milliseconds of wall time
    have passed (synchronising every few calls), so that the timed window
    starts at the GPU's steady clocks whatever the untimed step count is.
    Returns (wall ms spent, calls)."""
    t0, n = time.perf_counter(), 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(4):
            fn()
        n += 4
        torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3, n


def bench_step(rel, torch, dev, steps, warmup, B=16, H=8, T=2048, D=64, seed=42,
               prewarm_ms=0.0):
    from workloads import make_inputs
    inp = make_inputs(B, H, T, D, "bf16", seed=seed, with_dy=True)
    lam, scale = inp["lam"], 1.0 / math.sqrt(D)
    q, k, v, dy = (inp[n].to(dev) for n in ("q", "k", "v", "dy"))
    y = torch.empty_like(q)
    lse = torch.empty((B, H, T), device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dl = torch.empty((1,), device=dev, dtype=torch.float32)
    ws = torch.empty((rel.relation_bwd_workspace_bytes(torch.bfloat16, B, H, T, D),),
                     device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev)
    tf, tb = EventTimer(torch, stream), EventTimer(torch, stream)
    tk = []  # event pairs the library records around the main backward kernel

    def step(timed):
        s = tf.start() if timed else None
        rel.relation_fwd(q, k, v, lam=lam, scale=scale, y=y, lse=lse, want_gate=False)
        ev = None
        if timed:
            tf.stop(s)
            s = tb.start()
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            tk.append(ev)
        rel.relation_bwd(q, k, v, y, dy, lse, lam=lam, scale=scale, dq=dq, dk=dk, dv=dv,
                         dlambda=dl, workspace=ws, main_events=ev)
        if timed:
            tb.stop(s)

    pw_ms, pw_n = prewarm(torch, lambda: step(False), prewarm_ms)
    for _ in range(warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):  # the timed steps: nothing but the two calls
        step(False)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(steps):  # the same steps again with events around each call
        step(True)
    torch.cuda.synchronize()
    # The same step captured once as a HIP graph and replayed: the launch path
    # of a training loop whose shapes do not change. Reported beside the
    # value, which is the eager step above.
    graph = {}
    try:
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step(False)
        stream.wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(False)
        for _ in range(max(warmup, 3)):
            g.replay()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        graph = {"ms_per_step": (time.perf_counter() - t2) * 1e3 / steps}
    except RuntimeError as e:  # reported, never fatal to the value
        graph = {"error": str(e)[:200]}
    torch.cuda.synchronize()
    bwd_kernel_ms = sum(a.elapsed_time(b) for a, b in tk) / len(tk) if tk else float("nan")
    return {"ms_per_step": (t1 - t0) * 1e3 / steps, "fwd_ms": tf.mean_ms(),
            "bwd_ms": tb.mean_ms(), "bwd_kernel_ms": bwd_kernel_ms,
            "flops_fwd": fwd_flops(B, H, T, D),
            "prewarm_ms": pw_ms, "prewarm_steps": pw_n, "graph": graph}


def bench_fwd(rel, torch, dev, B, H, T, D, reps, rope=False, seed=42, prewarm_ms=100.0):
    from workloads import make_inputs
    inp = make_inputs(B, H, T, D, "bf16", seed=seed, rope=rope)
    q, k, v = (inp[n].to(dev) for n in ("q", "k", "v"))
    y = torch.empty_like(q)
    lse = torch.empty((B, H, T), device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream(dev)
    t = EventTimer(torch, stream)
    nws = rel.relation_fwd_workspace_bytes(torch.bfloat16, B, H, T, D)
    ws = torch.empty((nws,), device=dev, dtype=torch.uint8) if nws else None
    prewarm(torch, lambda: rel.relation_fwd(q, k, v, lam=inp["lam"], scale=1 / math.sqrt(D),
                                            y=y, lse=lse, workspace=ws), prewarm_ms)
    # back-to-back calls between one pair of events: a short call (the 10M
    # layer's is ~20 us) would otherwise also time the host's launch path
    s = t.start()
    for _ in range(reps):
        rel.relation_fwd(q, k, v, lam=inp["lam"], scale=1 / math.sqrt(D), y=y, lse=lse,
                         workspace=ws)
    t.stop(s)
    ms = t.mean_ms() / reps
    tf = fwd_flops(B, H, T, D) / (ms * 1e-3) / 1e12
    return {"ms": ms, "tflops": tf, "frac_peak": tf / PEAK_BF16_TFLOPS,
            "timing": f"{reps} back-to-back calls", "split_over_keys": nws > 0}


def bench_fwdbwd_vs_attention(rel, torch, dev, reps, B=8, H=12, T=4096, D=64, seed=42,
                              prewarm_ms=200.0):
    from workloads import make_inputs
    inp = make_inputs(B, H, T, D, "bf16", seed=seed, with_dy=True)
    q, k, v, dy = (inp[n].to(dev) for n in ("q", "k", "v", "dy"))
    lam, scale = inp["lam"], 1 / math.sqrt(D)
    y = torch.empty_like(q)
    lse = torch.empty((B, H, T), device=dev, dtype=torch.float32)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dl = torch.empty((1,), device=dev, dtype=torch.float32)
    ws = torch.empty((rel.relation_bwd_workspace_bytes(torch.bfloat16, B, H, T, D),),
                     device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev)
    tf_, tfb = EventTimer(torch, stream), EventTimer(torch, stream)

    def rel_step():
        rel.relation_fwd(q, k, v, lam=lam, scale=scale, y=y, lse=lse)
        rel.relation_bwd(q, k, v, y, dy, lse, lam=lam, scale=scale, dq=dq, dk=dk, dv=dv,
                         dlambda=dl, workspace=ws)
    prewarm(torch, rel_step, prewarm_ms)
    for i in range(reps + 2):
        s = tf_.start() if i >= 2 else None
        rel.relation_fwd(q, k, v, lam=lam, scale=scale, y=y, lse=lse)
        if i >= 2:
            tf_.stop(s)
        s2 = tfb.start() if i >= 2 else None
        rel.relation_bwd(q, k, v, y, dy, lse, lam=lam, scale=scale, dq=dq, dk=dk, dv=dv,
                         dlambda=dl, workspace=ws)
        if i >= 2:
            tfb.stop(s2)
    f = fwd_flops(B, H, T, D)
    fwd_ms, bwd_ms = tf_.mean_ms(), tfb.mean_ms()
    out = {"relation_fwd_ms": fwd_ms, "relation_bwd_ms": bwd_ms,
           "relation_fwd_tflops": f / (fwd_ms * 1e-3) / 1e12,
           "relation_fwdbwd_tflops": 3.5 * f / ((fwd_ms + bwd_ms) * 1e-3) / 1e12}
    # reference point: torch's causal softmax attention (SDPA) on the same tensors
    try:
        import torch.nn.functional as Fn
        qa, ka, va = (x.detach().clone().requires_grad_(True) for x in (q, k, v))
        ta, tab = EventTimer(torch, stream), EventTimer(torch, stream)

        def attn_step():
            Fn.scaled_dot_product_attention(qa, ka, va, is_causal=True, scale=scale).backward(dy)
            qa.grad = ka.grad = va.grad = None
        prewarm(torch, attn_step, prewarm_ms)
        for i in range(reps + 2):
            s = ta.start() if i >= 2 else None
            o = Fn.scaled_dot_product_attention(qa, ka, va, is_causal=True, scale=scale)
            if i >= 2:
                ta.stop(s)
            s2 = tab.start() if i >= 2 else None
            o.backward(dy)
            if i >= 2:
                tab.stop(s2)
            qa.grad = ka.grad = va.grad = None
        afwd, abwd = ta.mean_ms(), tab.mean_ms()
        out.update({"attention": "torch.nn.functional.scaled_dot_product_attention(is_causal=True)",
                    "attention_fwd_ms": afwd, "attention_bwd_ms": abwd,
                    "attention_fwd_tflops": f / (afwd * 1e-3) / 1e12,
                    "attention_fwdbwd_tflops": 3.5 * f / ((afwd + abwd) * 1e-3) / 1e12,
                    "relation_over_attention_fwd": afwd / fwd_ms,
                    "relation_over_attention_fwdbwd": (afwd + abwd) / (fwd_ms + bwd_ms)})
    except Exception as e:  # reference point only; report why it is missing
        out["attention_error"] = repr(e)[:200]
    return out


def bench_decode(rel, torch, dev, B=32, H=12, D=64, n0=4096, steps=256, cap=4352, seed=42,
                 prewarm_ms=200.0):
    from workloads import make_decode_inputs
    d = make_decode_inputs(B, H, D, n0, steps, cap, "bf16", seed=seed)
    kc, vc = d["k_cache"].to(dev), d["v_cache"].to(dev)
    qs, kn, vn = d["q"].to(dev), d["k_new"].to(dev), d["v_new"].to(dev)
    y = torch.empty((B, H, D), device=dev, dtype=torch.bfloat16)
    ws = torch.empty((rel.relation_decode_workspace_bytes(torch.bfloat16, B, H, D, cap),),
                     device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev)
    kc0, vc0 = kc.clone(), vc.clone()
    args = [(qs[s], kn[s], vn[s], n0 + s) for s in range(steps)]  # views made before timing

    def call(a):
        rel.relation_cache_decode(a[0], a[1], a[2], kc, vc, a[3], lam=d["lam"],
                                  scale=1 / math.sqrt(D), y=y, workspace=ws)
    # warm-up (clock ramp) on the first step's slot, then restore the cache
    prewarm(torch, lambda: call(args[0]), prewarm_ms)
    kc.copy_(kc0)
    vc.copy_(vc0)
    # the 256 consecutive steps, timed as a whole (events at both ends: the
    # GPU time of the sequence, launch gaps included)
    tw = EventTimer(torch, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e = tw.start()
    for a in args:
        call(a)
    tw.stop(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = tw.mean_ms()
    # the same steps again with events around every call (per-call time)
    kc.copy_(kc0)
    vc.copy_(vc0)
    t = EventTimer(torch, stream)
    for a in args:
        e = t.start()
        call(a)
        t.stop(e)
    call_ms = t.mean_ms()
    del kc0, vc0
    byts = sum(decode_bytes(B, H, D, n0 + s) for s in range(steps))
    return {"steps": steps, "total_ms": total_ms, "GBps": byts / (total_ms * 1e-3) / 1e9,
            "frac_hbm_peak": byts / (total_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "host_wall_ms": wall * 1e3, "call_ms": call_ms,
            "call_GBps": byts / steps / (call_ms * 1e-3) / 1e9, "bytes": byts}


def bench_decode_ragged(rel, torch, dev, B=32, H=12, D=64, nmax=4096, steps=64, cap=4352,
                        seed=42, prewarm_ms=200.0):
    """Ragged Relation Cache decode: per-sequence history lengths drawn
    uniformly in [0, nmax] (one sequence at nmax, one at 0), all advanced by
    one slot per step, over `steps` steps on the decode workload's cache
    shape. Each step's length array is prepared on the device beforehand (a
    serving loop advances it alongside its own state), so the timed sequence
    holds only the library's calls. Bytes are the algorithmic ones of each
    sequence's own length."""
    from workloads import make_decode_inputs, ragged_decode_lengths
    lengths = ragged_decode_lengths(B, nmax, seed)
    d = make_decode_inputs(B, H, D, nmax, steps, cap, "bf16", seed=seed)
    kc, vc = d["k_cache"].to(dev), d["v_cache"].to(dev)
    qs, kn, vn = d["q"].to(dev), d["k_new"].to(dev), d["v_new"].to(dev)
    y = torch.empty((B, H, D), device=dev, dtype=torch.bfloat16)
    ws = torch.empty((rel.relation_decode_workspace_bytes(torch.bfloat16, B, H, D, cap),),
                     device=dev, dtype=torch.uint8)
    nh_steps = (torch.tensor(lengths, dtype=torch.int32).unsqueeze(0) +
                torch.arange(steps, dtype=torch.int32).unsqueeze(1)).to(dev)  # [steps, B]
    stream = torch.cuda.current_stream(dev)
    kc0, vc0 = kc.clone(), vc.clone()
    args = [(qs[s], kn[s], vn[s], nh_steps[s], nmax + s) for s in range(steps)]

    def call(a):
        rel.relation_cache_decode_ragged(a[0], a[1], a[2], kc, vc, a[3], a[4], lam=d["lam"],
                                         scale=1 / math.sqrt(D), y=y, workspace=ws)
    prewarm(torch, lambda: call(args[0]), prewarm_ms)
    kc.copy_(kc0)
    vc.copy_(vc0)
    # the consecutive steps, timed as a whole (launch gaps included)
    tw = EventTimer(torch, stream)
    torch.cuda.synchronize()
    e = tw.start()
    for a in args:
        call(a)
    tw.stop(e)
    torch.cuda.synchronize()
    total_ms = tw.mean_ms()
    # the same steps with events around every call
    kc.copy_(kc0)
    vc.copy_(vc0)
    t = EventTimer(torch, stream)
    for a in args:
        e = t.start()
        call(a)
        t.stop(e)
    call_ms = t.mean_ms()
    del kc0, vc0
    per_seq = [decode_bytes(1, H, D, n + s) for s in range(steps) for n in lengths]
    byts = float(sum(per_seq))
    return {"steps": steps, "B": B, "lengths": f"uniform in [0, {nmax}] (seeded), mean "
            f"{sum(lengths) / B:.0f}", "total_ms": total_ms,
            "GBps": byts / (total_ms * 1e-3) / 1e9,
            "frac_hbm_peak": byts / (total_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "call_ms": call_ms, "call_GBps": byts / steps / (call_ms * 1e-3) / 1e9,
            "bytes": byts}


def bench_prefill(rel, torch, dev, reps, B=32, H=12, D=64, m=256, cap=4352, seed=42,
                  prewarm_ms=200.0):
    """Chunked prefill into the Relation Cache on the decode workload's cache
    shape: m new tokens per sequence at ragged history lengths (uniform in
    [0, cap - m], seeded). Flops count the causal entries of the new rows,
    4 D per entry (both contractions), as for the forward."""
    from workloads import make_decode_inputs, ragged_decode_lengths
    ns = ragged_decode_lengths(B, cap - m, seed)
    d = make_decode_inputs(B, H, D, cap - m, m, cap, "bf16", seed=seed)
    q, kn, vn = (d[n].permute(1, 2, 0, 3).contiguous().to(dev) for n in ("q", "k_new", "v_new"))
    kc, vc = d["k_cache"].to(dev), d["v_cache"].to(dev)
    nh = torch.tensor(ns, dtype=torch.int32, device=dev)
    y = torch.empty_like(q)
    nws = rel.relation_prefill_workspace_bytes(torch.bfloat16, B, H, D, m, cap - m, True)
    ws = torch.empty((nws,), device=dev, dtype=torch.uint8) if nws else None
    stream = torch.cuda.current_stream(dev)

    def call():  # the same new rows at the same slots every call
        rel.relation_cache_prefill(q, kn, vn, kc, vc, nh, cap - m, lam=d["lam"],
                                   scale=1 / math.sqrt(D), y=y, workspace=ws)
    prewarm(torch, call, prewarm_ms)
    t = EventTimer(torch, stream)
    s0 = t.start()  # back-to-back calls between one pair of events
    for _ in range(reps):
        call()
    t.stop(s0)
    ms = t.mean_ms() / reps
    entries = sum(m * n + m * (m + 1) / 2 for n in ns) * H
    tf = 4 * D * entries / (ms * 1e-3) / 1e12
    return {"workload": f"prefill {m} tokens x {B} sequences x {H} heads, ragged history "
            f"(mean {sum(ns) / B:.0f})", "ms": ms, "tflops": tf,
            "frac_peak": tf / PEAK_BF16_TFLOPS, "split_over_keys": nws > 0}


def bench_mhr(rel, torch, dev, reps, B=16, H=8, T=2048, D=64, seed=42, prewarm_ms=200.0):
    """Multi-Head Relation with its upstream maps (RoPE of p1 / p2 from
    [T, D/2] tables, Givens mixing of I, pairing M_B) on the 30M layer shape:
    forward and forward+backward, next to the plain operator on the same
    tensors. Flops are the operator's (the maps are O(T D) per head). The
    backward reads the forward's rotated keys and mixed values from its
    workspace, as a training step that keeps the forward's buffers does."""
    from workloads import make_inputs, make_mhr_maps
    inp = make_inputs(B, H, T, D, "bf16", seed=seed, with_dy=True)
    p1, p2, I, dy = (inp[n].to(dev) for n in ("q", "k", "v", "dy"))
    cs, sn, th = (t.to(dev) for t in make_mhr_maps(T, D, H, seed))
    lam, scale = inp["lam"], 1 / math.sqrt(D)
    lib = rel.load_library()
    wsf = torch.empty((lib.relation_mhr_fwd_workspace_bytes(1, B, H, T, D),), device=dev,
                      dtype=torch.uint8)
    wsb = torch.empty((lib.relation_mhr_bwd_workspace_bytes(1, B, H, T, D),), device=dev,
                      dtype=torch.uint8)
    y = torch.empty_like(I)
    lse = torch.empty((B, H, T), device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream(dev)

    def fwd():
        rel.relation_mhr_fwd(p1, p2, I, cs, sn, th, 1, lam=lam, scale=scale, y=y, lse=lse,
                             workspace=wsf)

    def bwd():
        rel.relation_mhr_bwd(p1, p2, I, y, dy, lse, cs, sn, th, 1, lam=lam, scale=scale,
                             workspace=wsb, fwd_workspace=wsf)
    prewarm(torch, lambda: (fwd(), bwd()), prewarm_ms)
    tf, tb = EventTimer(torch, stream), EventTimer(torch, stream)
    s0 = tf.start()  # back-to-back calls between one pair of events
    for _ in range(reps):
        fwd()
    tf.stop(s0)
    s1 = tb.start()  # the backward reads the last forward's y, lse and maps
    for _ in range(reps):
        bwd()
    tb.stop(s1)
    f = fwd_flops(B, H, T, D)
    fm, bm = tf.mean_ms() / reps, tb.mean_ms() / reps
    return {"workload": "layer30m MHR (RoPE + Givens M_B), backward reusing the forward's maps",
            "fwd_ms": fm, "bwd_ms": bm,
            "fwd_tflops": f / (fm * 1e-3) / 1e12,
            "fwdbwd_tflops": 3.5 * f / ((fm + bm) * 1e-3) / 1e12}


def bench_linear(rel, torch, dev, reps, B=32, H=8, T=1024, D=64, seed=42, prewarm_ms=200.0):
    """Linear Relation forward with RoPE on the 30M-class layer at the pages'
    steady-state micro-batch (B=32, H=8, T=1024, d_h=64; App. H, Table 16).
    Algorithmic HBM bytes per token and head: p1, p2, I, y in bf16 and the
    fp32 log retention g, 12 D."""
    from workloads import make_linear_inputs, make_mhr_maps
    d = make_linear_inputs(B, H, T, D, seed)
    p1, p2, I, g = (d[n].to(dev) for n in ("p1", "p2", "I", "g"))
    cs, sn, _ = (t.to(dev) for t in make_mhr_maps(T, D, 2, seed))
    y = torch.empty_like(I)
    stream = torch.cuda.current_stream(dev)
    tf = EventTimer(torch, stream)
    prewarm(torch, lambda: rel.relation_linear_fwd(p1, p2, I, g, cs, sn, scale=1 / math.sqrt(D),
                                                   y=y), prewarm_ms)
    # back-to-back calls between one pair of events (a ~65 us call would
    # otherwise also time the host's launch path)
    s0 = tf.start()
    for _ in range(reps):
        rel.relation_linear_fwd(p1, p2, I, g, cs, sn, scale=1 / math.sqrt(D), y=y)
    tf.stop(s0)
    fm = tf.mean_ms() / reps
    nbytes = 12 * D * B * H * T
    # backward: reads p1, p2, I, dY (bf16) and g, writes dp1, dp2, dI (bf16)
    # and dg: 22 D bytes per token and head (the state pass is overhead)
    dy = torch.randn_like(I)
    lib = rel.load_library()
    ws = torch.empty((lib.relation_linear_bwd_workspace_bytes(1, B, H, T, D),), device=dev,
                     dtype=torch.uint8)
    tb = EventTimer(torch, stream)
    for _ in range(20):
        rel.relation_linear_bwd(p1, p2, I, g, dy, cs, sn, scale=1 / math.sqrt(D), workspace=ws)
    torch.cuda.synchronize()
    nb = max(1, reps // 2)
    s0 = tb.start()
    for _ in range(nb):
        rel.relation_linear_bwd(p1, p2, I, g, dy, cs, sn, scale=1 / math.sqrt(D), workspace=ws)
    tb.stop(s0)
    bm = tb.mean_ms() / nb
    bbytes = 22 * D * B * H * T
    # a training step: the forward stores the state before every chunk and the
    # backward reuses them instead of running its own state pass
    states = torch.empty(rel.linear_states_shape(B, H, T, D), device=dev, dtype=torch.float32)
    t1, t2 = EventTimer(torch, stream), EventTimer(torch, stream)
    for _ in range(10):
        rel.relation_linear_fwd(p1, p2, I, g, cs, sn, scale=1 / math.sqrt(D), y=y, states=states)
        rel.relation_linear_bwd(p1, p2, I, g, dy, cs, sn, scale=1 / math.sqrt(D), workspace=ws,
                                fwd_states=states)
    torch.cuda.synchronize()
    s1 = t1.start()
    for _ in range(nb):
        rel.relation_linear_fwd(p1, p2, I, g, cs, sn, scale=1 / math.sqrt(D), y=y, states=states)
    t1.stop(s1)
    s2 = t2.start()
    for _ in range(nb):
        rel.relation_linear_bwd(p1, p2, I, g, dy, cs, sn, scale=1 / math.sqrt(D), workspace=ws,
                                fwd_states=states)
    t2.stop(s2)
    tfm, tbm = t1.mean_ms() / nb, t2.mean_ms() / nb
    return {"workload": f"linear relation fwd + bwd, RoPE, B={B} H={H} T={T} D={D}",
            "fwd_ms": fm, "tokens_per_s": B * T / (fm * 1e-3),
            "fwd_GBps": nbytes / (fm * 1e-3) / 1e9,
            "frac_hbm": nbytes / (fm * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "bwd_ms": bm, "bwd_GBps": bbytes / (bm * 1e-3) / 1e9,
            "bwd_frac_hbm": bbytes / (bm * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "fwdbwd_tokens_per_s": B * T / ((fm + bm) * 1e-3),
            "train_fwd_ms": tfm, "train_bwd_ms": tbm,
            "train_fwdbwd_tokens_per_s": B * T / ((tfm + tbm) * 1e-3),
            "train_note": "forward stores the per-chunk states, backward reuses them"}


def bench_linear_step(rel, torch, dev, reps=200, B=32, H=12, D=64, seed=42):
    """One Linear Relation decode step per sequence on the cache workload's
    batch (32 sequences x 12 heads): the fp32 D x D state is read and
    written once; bytes per head 8 D^2 + 10 D."""
    from workloads import make_linear_inputs
    d = make_linear_inputs(B, H, 1, D, seed)
    p1, p2, I, g = (d[n][:, :, 0].contiguous().to(dev) for n in ("p1", "p2", "I", "g"))
    state = torch.zeros((B, H, D, D), device=dev, dtype=torch.float32)
    y = torch.empty_like(I)
    stream = torch.cuda.current_stream(dev)
    t = EventTimer(torch, stream)
    for _ in range(10):
        rel.relation_linear_step(p1, p2, I, g, state, scale=1 / math.sqrt(D), y=y)
    torch.cuda.synchronize()
    # back-to-back steps (each reads and rewrites the state) between one pair
    # of events: a single ~5 us step is far shorter than the host's launch path
    s0 = t.start()
    for _ in range(reps):
        rel.relation_linear_step(p1, p2, I, g, state, scale=1 / math.sqrt(D), y=y)
    t.stop(s0)
    ms = t.mean_ms() / reps
    nbytes = (8 * D * D + 10 * D) * B * H
    return {"workload": f"linear relation decode step, B={B} H={H} D={D}", "ms": ms,
            "GBps": nbytes / (ms * 1e-3) / 1e9}


def bench_copy(torch, dev, nbytes=1 << 30, reps=5):
    """A plain device-to-device copy of known size (torch's copy kernel): the
    calibration for the FETCH_SIZE / WRITE_SIZE counters (reads nbytes and
    writes nbytes per launch)."""
    src = torch.ones(nbytes // 2, device=dev, dtype=torch.bfloat16)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream(dev)
    t = EventTimer(torch, stream)
    for i in range(reps + 1):
        s = t.start() if i >= 1 else None
        dst.copy_(src)
        if i >= 1:
            t.stop(s)
    ms = t.mean_ms()
    return {"bytes_read": nbytes, "bytes_written": nbytes, "ms": ms,
            "GBps_rw": 2 * nbytes / (ms * 1e-3) / 1e9}


def kernel_traffic(name):
    """HBM bytes per launch of one kernel from the committed counter summary
    (profiles/traffic.json), or None when the kernel's source has changed
    since the counters were taken (the summary stores a hash of the source)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)[name]
        src = os.path.join(ROOT, "exchange_relation_amd", "csrc", rec["source"])
        with open(src, "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
                return None
        return rec["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline():
    """The fp64 oracle, as it stands, timed on this host on a bounded sample
    of every workload (about 20 s of CPU work in all), each scaled to the
    workload's unit with the same algorithmic count as the GPU lines:
      * single Multi-Head Relation forward, fp32, B=1 H=2 T=128 D=32: whole;
      * 10M layer forward (B=8 H=8 T=1024 D=64, RoPE'd q / k): 8 of 64 heads;
      * 30M layer (B=16 H=8 T=2048 D=64): forward on 4 heads, forward +
        backward on 8 heads (of 128);
      * 100M layer (B=8 H=12 T=4096 D=64): forward on 1 head, forward +
        backward on 1 head (of 96);
      * Relation Cache decode (B=32 H=12 D=64, history 4096): the first 2 of
        the 256 steps, whole batch, in GB/s of the step's algorithmic bytes.
    Heads are whole (each head's rows are independent of the others), so
    the per-head time scales exactly to the full workload's count.
    `value` is the 30M layer's forward + backward (the step's metric)."""
    import oracle
    from workloads import make_decode_inputs, make_inputs

    def f64(t):
        return t.double().numpy()

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    per = {}

    def heads_run(key, B, H, T, D, dtype, nh, kind, rope=False):
        inp = make_inputs(B, H, T, D, dtype, seed=42, rope=rope, with_dy=(kind == "fwdbwd"))
        a = {n: f64(inp[n].reshape(B * H, T, D)[:nh]) for n in inp if n != "lam"}
        s = 1 / math.sqrt(D)
        if kind == "fwd":
            dt = timed(lambda: [oracle.relation_forward_head(a["q"][i], a["k"][i], a["v"][i], s,
                                                             2.0, inp["lam"]) for i in range(nh)])
            fl = fwd_flops(1, nh, T, D)
        else:
            dt = timed(lambda: [oracle.relation_backward_head(a["q"][i], a["k"][i], a["v"][i],
                                                              a["dy"][i], s, 2.0, inp["lam"])
                                for i in range(nh)])
            fl = 3.5 * fwd_flops(1, nh, T, D)
        per[key] = {"kind": kind, "sample": f"{nh} of {B * H} heads", "seconds": dt,
                    "value": fl / dt / 1e12, "unit": "TFLOP/s",
                    "full_workload_seconds_est": dt * B * H / nh}

    heads_run("mhr_fwd_f32", 1, 2, 128, 32, "f32", 2, "fwd")
    heads_run("layer10m_fwd_bf16", 8, 8, 1024, 64, "bf16", 8, "fwd", rope=True)
    heads_run("layer30m_fwd_bf16", 16, 8, 2048, 64, "bf16", 4, "fwd")
    heads_run("layer30m_fwdbwd_bf16", 16, 8, 2048, 64, "bf16", 8, "fwdbwd")
    heads_run("layer100m_fwd_bf16", 8, 12, 4096, 64, "bf16", 1, "fwd")
    heads_run("layer100m_fwdbwd_bf16", 8, 12, 4096, 64, "bf16", 1, "fwdbwd")
    B, H, D, n0, cap, nst = 32, 12, 64, 4096, 4352, 2
    d = make_decode_inputs(B, H, D, n0, nst, cap, "bf16", seed=42)
    kc, vc = f64(d["k_cache"]), f64(d["v_cache"])
    dt = 0.0
    for st in range(nst):
        t0 = time.perf_counter()
        _, _, kc, vc = oracle.relation_decode_step(f64(d["q"][st]), f64(d["k_new"][st]),
                                                   f64(d["v_new"][st]), kc, vc, n0 + st,
                                                   1 / math.sqrt(D), 2.0, d["lam"])
        dt += time.perf_counter() - t0
    byts = sum(decode_bytes(B, H, D, n0 + st) for st in range(nst))
    per["cache_decode_bf16"] = {"kind": "decode", "sample": f"steps 0..{nst - 1} of 256, whole "
                                "batch", "seconds": dt, "value": byts / dt / 1e9, "unit": "GB/s",
                                "full_workload_seconds_est": dt * 256 / nst}
    head = per["layer30m_fwdbwd_bf16"]
    return {"value": head["value"], "unit": "TFLOP/s", "cores": _oracle_threads(),
            "kind": "oracle",
            "sample": "30M layer (B=16,H=8,T=2048,D=64) fwd+bwd on 8 whole heads of 128, "
                      f"materialised fp64 numpy, {head['seconds']:.1f} s; per_config holds "
                      "every workload's sample",
            "host": {"cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
                     "cpu_model": _cpu_model()},
            "per_config": per}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    # the GPU's clocks take on the order of 0.1 s of sustained work to ramp:
    # a time-based phase of untimed steps comes before the W warm-up steps
    ap.add_argument("--prewarm-ms", type=float, default=500.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--only", choices=["step", "fwd", "fwd10m", "fwd100m", "decode", "ragged",
                                       "mhr", "prefill", "attn", "linear", "copy", "cpu"],
                    default=None,
                    help="run one measurement and print its raw numbers ('copy': a plain "
                         "device copy of known size, the HBM-counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(heads are independent: see DESIGN.md for how the operator shards)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import exchange_relation_amd as rel
    rel.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    torch.manual_seed(0)

    if args.only == "copy":
        print(json.dumps(bench_copy(torch, dev)))
        return
    if args.only == "cpu":
        print(json.dumps(cpu_baseline()))
        return
    if args.only == "step":
        print(json.dumps(bench_step(rel, torch, dev, args.steps, args.warmup,
                                    prewarm_ms=args.prewarm_ms)))
        return
    if args.only == "fwd":
        print(json.dumps(bench_fwd(rel, torch, dev, 16, 8, 2048, 64, args.steps,
                                   prewarm_ms=args.prewarm_ms)))
        return
    if args.only == "fwd10m":
        print(json.dumps(bench_fwd(rel, torch, dev, 8, 8, 1024, 64, args.steps, rope=True,
                                   prewarm_ms=args.prewarm_ms)))
        return
    if args.only == "fwd100m":
        print(json.dumps(bench_fwd(rel, torch, dev, 8, 12, 4096, 64, args.steps,
                                   prewarm_ms=args.prewarm_ms)))
        return
    if args.only == "decode":
        print(json.dumps(bench_decode(rel, torch, dev, prewarm_ms=args.prewarm_ms)))
        return
    if args.only == "ragged":
        print(json.dumps(bench_decode_ragged(rel, torch, dev, prewarm_ms=args.prewarm_ms)))
        return
    if args.only == "mhr":
        print(json.dumps(bench_mhr(rel, torch, dev, args.steps, prewarm_ms=args.prewarm_ms)))
        return
    if args.only == "prefill":
        print(json.dumps(bench_prefill(rel, torch, dev, args.steps, prewarm_ms=args.prewarm_ms)))
        return
    if args.only == "linear":
        print(json.dumps({"fwd": bench_linear(rel, torch, dev, args.steps,
                                              prewarm_ms=args.prewarm_ms),
                          "step": bench_linear_step(rel, torch, dev)}))
        return
    if args.only == "attn":
        print(json.dumps(bench_fwdbwd_vs_attention(rel, torch, dev, args.steps,
                                                   prewarm_ms=args.prewarm_ms)))
        return

    st = bench_step(rel, torch, dev, args.steps, args.warmup, prewarm_ms=args.prewarm_ms)
    f = st["flops_fwd"]
    value = 3.5 * f / (st["ms_per_step"] * 1e-3) / 1e12
    bwd_tf = 2.5 * f / (st["bwd_ms"] * 1e-3) / 1e12
    bwdk_tf = 2.5 * f / (st["bwd_kernel_ms"] * 1e-3) / 1e12
    fwd_tf = f / (st["fwd_ms"] * 1e-3) / 1e12
    rec = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": st["ms_per_step"],
        "prewarm_ms": round(st["prewarm_ms"], 1), "prewarm_steps": st["prewarm_steps"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Gaussian q, k, v, dY; no dataset)",
        "config": {"workload": "layer30m_fwdbwd_bf16", "B": 16, "H": 8, "T": 2048, "D": 64,
                   "causal": True, "step": "relation_fwd + relation_bwd",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "bwd_bf16_kernel (HIP events that relation_bwd "
                     "records around its launch)",
                     "achieved": bwdk_tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": bwdk_tf / PEAK_BF16_TFLOPS,
                     "traffic": kernel_traffic("bwd_bf16_kernel@layer30m")},
        "roofline_bwd_call": {"bound": "mfma", "kernel": "relation_bwd call (preprocess with the "
                              "dq accumulator clear + bwd_bf16_kernel + dq finalize)",
                              "achieved": bwd_tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                              "frac": bwd_tf / PEAK_BF16_TFLOPS},
        "roofline_fwd": {"bound": "mfma", "kernel": "fwd_bf16_kernel (one launch per call)",
                         "achieved": fwd_tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": fwd_tf / PEAK_BF16_TFLOPS,
                         "traffic": kernel_traffic("fwd_bf16_kernel@layer30m")},
        "fwd_ms": st["fwd_ms"], "bwd_ms": st["bwd_ms"], "bwd_kernel_ms": st["bwd_kernel_ms"],
        "step_graph_replay": dict(st["graph"], **({"tflops": 3.5 * f / (st["graph"]["ms_per_step"]
                                                                       * 1e-3) / 1e12}
                                                  if "ms_per_step" in st["graph"] else {})),
    }
    if not args.no_extra:
        rec["fwd_layer10m"] = bench_fwd(rel, torch, dev, 8, 8, 1024, 64, 50, rope=True)
        rec["fwd_layer100m"] = bench_fwd(rel, torch, dev, 8, 12, 4096, 64, 10)
        rec["layer100m_vs_attention"] = bench_fwdbwd_vs_attention(rel, torch, dev, 5)
        dec = bench_decode(rel, torch, dev)
        rec["decode"] = dec
        rec["roofline_decode"] = {"bound": "hbm", "kernel": "relation_cache_decode call "
                                  "(split scan + combine)", "achieved": dec["call_GBps"],
                                  "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": dec["call_GBps"] / PEAK_HBM_GBS,
                                  "traffic": kernel_traffic("decode_split_kernel@cache4096")}
        torch.cuda.empty_cache()
        rec["mhr_layer30m"] = bench_mhr(rel, torch, dev, 10)
        rec["prefill_cache"] = bench_prefill(rel, torch, dev, 10)
        rec["decode_ragged"] = bench_decode_ragged(rel, torch, dev)
        torch.cuda.empty_cache()
        lin = bench_linear(rel, torch, dev, 20)
        rec["linear_layer30m"] = lin
        rec["roofline_linear_fwd"] = {
            "bound": "hbm", "kernel": "linear_fwd_kernel (one launch per call)",
            "achieved": lin["fwd_GBps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": lin["fwd_GBps"] / PEAK_HBM_GBS,
            "traffic": kernel_traffic("linear_fwd_kernel@linear30m")}
        rec["linear_decode_step"] = bench_linear_step(rel, torch, dev)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline()
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
