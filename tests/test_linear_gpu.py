"""GPU parity of Linear Relation (Sec. 5.2; App. A.4): relation_linear_fwd and
relation_linear_step through the C ABI against the fp64 oracle
(oracle/linear.py) on the same seeded inputs (workloads.make_linear_inputs).

Tolerances. y = I + E is not a convex combination of values, so unlike the
Full Relation output its magnitude is not bounded by max|I|; rounding y to
bf16 alone costs up to 2^-9 |y| (0.016 at |y| = 8). Each element must be
within 2e-2 * max(1, |Y|/4) of the oracle (2e-2 absolute up to |Y| = 4,
then 5e-3 relative, 2.5 times the half-ulp), and the mean-abs error within
3e-3. The fp32 state (read through a bf16 hi + lo split, updated with bf16
operands) must be within 2e-2 * max(1, max|C|). Total retention loss
(g = -1e4, alpha = 0) must give y = I bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import exchange_relation_amd as rel
import oracle
from workloads import make_linear_inputs, make_mhr_maps

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
BF16_MAX, BF16_MEAN = 2e-2, 3e-3
SCALE, TAU = 1 / 8, 2.0


def f64(t):
    return t.detach().cpu().double().numpy()


def check(name, got, ref):
    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    bound = BF16_MAX * np.maximum(1.0, np.abs(ref) / 4.0)
    worst = float((err / bound).max())
    mx, mean = float(err.max()), float(err.mean())
    print(f"  {name}: max-abs {mx:.3e} mean-abs {mean:.3e} worst err/bound {worst:.3f}")
    assert worst <= 1.0, f"{name}: error {worst:.3f} x the bound"
    assert mean <= BF16_MEAN, f"{name}: mean-abs {mean:.3e} > {BF16_MEAN}"


def check_state(name, got, ref):
    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    tol = BF16_MAX * max(1.0, float(np.abs(ref).max()))
    print(f"  {name}: max-abs {float(err.max()):.3e} (bound {tol:.3e})")
    assert float(err.max()) <= tol


def tables(T, D=64):
    cs, sn, _ = make_mhr_maps(T, D, 2, 0)
    return cs, sn


def run_fwd(d, rope=None, state_in=None):
    cs, sn = rope if rope is not None else (None, None)
    y, c = rel.relation_linear_fwd(
        *(d[n].to(DEV) for n in ("p1", "p2", "I", "g")),
        rope_cos=None if cs is None else cs.to(DEV), rope_sin=None if sn is None else sn.to(DEV),
        state_in=None if state_in is None else state_in.to(DEV), want_state=True, scale=SCALE,
        tau_s=TAU)
    torch.cuda.synchronize()
    return y.cpu(), c.cpu()


def oracle_fwd(d, rope=None, C0=None):
    cs, sn = (None, None) if rope is None else (f64(rope[0]), f64(rope[1]))
    return oracle.linear_relation_forward(f64(d["p1"]), f64(d["p2"]), f64(d["I"]), f64(d["g"]),
                                          SCALE, TAU, cs, sn,
                                          C0=None if C0 is None else f64(C0))


@pytest.mark.parametrize("use_rope", [False, True])
@pytest.mark.parametrize("T", [1, 17, 128, 129, 300, 520])
def test_linear_fwd_vs_oracle(T, use_rope):
    d = make_linear_inputs(2, 2, T, 64, seed=2000 + T)
    rope = tables(T) if use_rope else None
    y, c = run_fwd(d, rope)
    r = oracle_fwd(d, rope)
    check("y", f64(y), r["Y"])
    check_state("state", f64(c), r["C"])


@pytest.mark.parametrize("resets,keep", [(True, False), (False, True), (True, True)])
def test_linear_fwd_extreme_retention(resets, keep):
    """Near-total resets (g = -60 on 1 % of entries: sub-chunks with two
    resets on one channel take the per-pair path of the diagonal blocks) and
    channels without loss (g = 0)."""
    d = make_linear_inputs(2, 3, 400, 64, seed=2100, resets=resets, keep=keep)
    y, c = run_fwd(d)
    r = oracle_fwd(d)
    check("y", f64(y), r["Y"])
    check_state("state", f64(c), r["C"])


def test_linear_fwd_diagonal_span_limits():
    """The diagonal block's ratio form is used while a sub-chunk's retention
    span stays within 2^120 on every channel, the per-pair path beyond it.
    Sub-chunks with a span just inside (2^-118) and just beyond (2^-122) that
    limit on one channel, and one with a single token of g = -400, against
    the oracle."""
    d = make_linear_inputs(1, 2, 200, 64, seed=2150)
    g = d["g"].clone()
    ln2 = math.log(2.0)
    g[..., 16:32, 5] = -118.0 * ln2 / 16  # sub-chunk 1: ratio form at its limit
    g[..., 48:64, 40] = -122.0 * ln2 / 16  # sub-chunk 3: per-pair path
    g[..., 90, 7] = -400.0  # sub-chunk 5: per-pair path
    g[..., 130:146, :] = -118.0 * ln2 / 16  # a whole chunk-crossing run at the limit
    d["g"] = g
    y, c = run_fwd(d, tables(200))
    r = oracle_fwd(d, tables(200))
    check("y", f64(y), r["Y"])
    check_state("state", f64(c), r["C"])


def test_linear_total_retention_loss_is_identity():
    d = make_linear_inputs(1, 2, 260, 64, seed=2200)
    d["g"] = torch.full_like(d["g"], -1.0e4)
    y, c = run_fwd(d)
    assert torch.equal(y, d["I"])
    r = oracle_fwd(d)
    check_state("state", f64(c), r["C"])


def test_linear_state_in_and_handoff():
    B, H, T, T1 = 2, 2, 300, 128 + 37
    d = make_linear_inputs(B, H, T, 64, seed=2300)
    rope = tables(T)
    C0 = torch.from_numpy(np.random.default_rng(1).standard_normal((B, H, 64, 64)).astype(np.float32))
    y, c = run_fwd(d, rope, state_in=C0)
    r = oracle_fwd(d, rope, C0=C0)
    check("y with C0", f64(y), r["Y"])
    check_state("state with C0", f64(c), r["C"])
    # two calls chained through the state equal one call
    a = {k: v[:, :, :T1].contiguous() for k, v in d.items()}
    b = {k: v[:, :, T1:].contiguous() for k, v in d.items()}
    ya, ca = run_fwd(a, (rope[0][:T1].contiguous(), rope[1][:T1].contiguous()), state_in=C0)
    yb, cb = run_fwd(b, (rope[0][T1:].contiguous(), rope[1][T1:].contiguous()), state_in=ca)
    check("y chained", f64(torch.cat([ya, yb], dim=2)), r["Y"])
    check_state("state chained", f64(cb), r["C"])


@pytest.mark.parametrize("use_rope", [False, True])
def test_linear_step_vs_oracle_and_forward(use_rope):
    B, H, T = 3, 4, 40
    d = make_linear_inputs(B, H, T, 64, seed=2400, with_dy=False)
    rope = tables(T) if use_rope else None
    state = torch.zeros((B, H, 64, 64), device=DEV, dtype=torch.float32)
    C = np.zeros((B, H, 64, 64))
    ys = []
    for t in range(T):
        args = [d[n][:, :, t].contiguous().to(DEV) for n in ("p1", "p2", "I", "g")]
        kw = {}
        if rope is not None:
            kw = {"rope_cos": rope[0][t].contiguous().to(DEV),
                  "rope_sin": rope[1][t].contiguous().to(DEV)}
        y = rel.relation_linear_step(*args, state, scale=SCALE, tau_s=TAU, **kw)
        ys.append(y.cpu())
        yo, C = oracle.linear_relation_step(
            f64(d["p1"][:, :, t]), f64(d["p2"][:, :, t]), f64(d["I"][:, :, t]),
            f64(d["g"][:, :, t]), C, SCALE, TAU,
            None if rope is None else f64(rope[0][t]), None if rope is None else f64(rope[1][t]))
        check(f"step {t} y", f64(ys[-1]), yo)
    torch.cuda.synchronize()
    check_state("step state", f64(state), C)
    yf, cf = run_fwd(d, rope)
    check("steps vs forward", f64(torch.stack(ys, dim=2)), f64(yf).astype(np.float64))


def test_linear_fwd_30m_layer_shape_sampled_heads():
    """The 30M-class Linear Relation layer at its steady-state micro-batch
    (B=32, H=8, T=1024, d_h=64; paper App. H, Table 16) in the benchmark's
    launch shape, with RoPE; sampled heads from the oracle."""
    B, H, T = 32, 8, 1024
    d = make_linear_inputs(B, H, T, 64, seed=42)
    rope = tables(T)
    y, c = run_fwd(d, rope)
    for b, h in ((0, 0), (31, 7), (13, 4)):
        sub = {k: v[b:b + 1, h:h + 1] for k, v in d.items()}
        r = oracle_fwd(sub, rope)
        check(f"y[{b},{h}]", f64(y[b:b + 1, h:h + 1]), r["Y"])
        check_state(f"state[{b},{h}]", f64(c[b:b + 1, h:h + 1]), r["C"])


# ---------------------------------------------------------------- backward
@pytest.fixture(params=["fused", "chunked"])
def bwd_form(request, monkeypatch):
    """Forces the backward's form: the fused per-head pass (chunks walked from
    the last, dC in registers) or the state-gradient pass + chunk-parallel
    gradient pass. Without the variable the library picks by batch size."""
    monkeypatch.setenv("RELATION_LINEAR_BWD", request.param)
    return request.param


def run_bwd(d, rope=None, C0=None, dCT=None):
    cs, sn = rope if rope is not None else (None, None)
    out = rel.relation_linear_bwd(
        *(d[n].to(DEV) for n in ("p1", "p2", "I", "g", "dy")),
        rope_cos=None if cs is None else cs.to(DEV), rope_sin=None if sn is None else sn.to(DEV),
        state_in=None if C0 is None else C0.to(DEV), dstate_out=None if dCT is None else dCT.to(DEV),
        want_dstate_in=True, scale=SCALE, tau_s=TAU)
    torch.cuda.synchronize()
    return [t.cpu() for t in out]


def test_linear_bwd_reuses_forward_states(bwd_form):
    """The forward can store the state before every chunk (and the final
    state); the backward given them skips its own state pass. y and the final
    state are unchanged bit for bit, the last stored state is state_out, and
    every gradient equals the three-pass backward's bit for bit (both sides
    run the same state recurrence)."""
    B, H, T = 2, 3, 300
    d = make_linear_inputs(B, H, T, 64, seed=77, with_dy=True)
    cs, sn = (t.to(DEV) for t in tables(T))
    C0 = (0.1 * torch.randn(B, H, 64, 64, generator=torch.Generator().manual_seed(5))).to(DEV)
    dCT = torch.randn(B, H, 64, 64, generator=torch.Generator().manual_seed(6)).to(DEV)
    p1, p2, I, g, dy = (d[n].to(DEV) for n in ("p1", "p2", "I", "g", "dy"))
    kw = dict(rope_cos=cs, rope_sin=sn, state_in=C0, scale=SCALE, tau_s=TAU)
    states = torch.full(rel.linear_states_shape(B, H, T), float("nan"), device=DEV)
    assert states.shape[2] == 4  # ceil(300 / 128) chunks, then the final state
    y0, c0 = rel.relation_linear_fwd(p1, p2, I, g, want_state=True, **kw)
    y1, c1 = rel.relation_linear_fwd(p1, p2, I, g, want_state=True, states=states, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(c0, c1)
    assert torch.equal(states[:, :, -1], c1)
    assert torch.equal(states[:, :, 0], C0)  # the state before the first chunk
    ref = rel.relation_linear_bwd(p1, p2, I, g, dy, dstate_out=dCT, want_dstate_in=True, **kw)
    # with the forward's states the workspace holds only the state gradients:
    # exactly the size the library asks for, filled with NaN bytes first
    need = rel.load_library().relation_linear_bwd_reuse_workspace_bytes(1, B, H, T, 64)
    assert need == B * H * 3 * 64 * 64 * 4
    ws = torch.full((need,), 0xFF, device=DEV, dtype=torch.uint8)
    got = rel.relation_linear_bwd(p1, p2, I, g, dy, dstate_out=dCT, want_dstate_in=True,
                                  fwd_states=states, workspace=ws, **kw)
    torch.cuda.synchronize()
    for name, a, b in zip(("dp1", "dp2", "dI", "dg", "dstate_in"), got, ref):
        assert torch.equal(a, b), name


def oracle_bwd(d, rope=None, C0=None, dCT=None):
    cs, sn = (None, None) if rope is None else (f64(rope[0]), f64(rope[1]))
    return oracle.linear_relation_backward(
        f64(d["p1"]), f64(d["p2"]), f64(d["I"]), f64(d["g"]), f64(d["dy"]), SCALE, TAU, cs, sn,
        C0=None if C0 is None else f64(C0), dC_T=None if dCT is None else f64(dCT))


def check_dg(got, ref):
    """dg_t = sum_{t' >= t} dB_t': each dB carries the bf16 operands' relative
    error (about 2^-8 of its terms), and those add up over the suffix like a
    random walk, so element t must be within 2e-2 + 2^-7 sqrt(sum_{t'>=t}
    dB_t'^2) (dB from the oracle's dg), and on average within a quarter of
    that bound."""
    dB = ref - np.concatenate([ref[..., 1:, :], np.zeros_like(ref[..., :1, :])], axis=-2)
    walk = np.sqrt(np.flip(np.cumsum(np.flip(dB ** 2, axis=-2), axis=-2), axis=-2))
    err = np.abs(got - ref)
    bound = 2e-2 + 2.0 ** -7 * walk
    worst, mean = float((err / bound).max()), float((err / bound).mean())
    print(f"  dg: max-abs {float(err.max()):.3e} mean-abs {float(err.mean()):.3e} "
          f"err/bound worst {worst:.3f} mean {mean:.3f}")
    assert worst <= 1.0
    assert mean <= 0.25


def check_grads(got, ref):
    for name, a, b in zip(("dp1", "dp2", "dI"), got[:3], ref[:3]):
        check(name, f64(a), b)
    check_dg(f64(got[3]), ref[3])
    check_state("dstate_in", f64(got[4]), ref[4])


@pytest.mark.parametrize("use_rope", [False, True])
@pytest.mark.parametrize("T", [1, 17, 128, 129, 300])
def test_linear_bwd_vs_oracle(T, use_rope, bwd_form):
    d = make_linear_inputs(2, 2, T, 64, seed=2500 + T, with_dy=True)
    rope = tables(T) if use_rope else None
    got = run_bwd(d, rope)
    ref = oracle_bwd(d, rope)
    check_grads(got, ref)


def test_linear_bwd_with_states_and_extreme_retention(bwd_form):
    B, H, T = 2, 2, 300
    d = make_linear_inputs(B, H, T, 64, seed=2600, with_dy=True, resets=True, keep=True)
    rng = np.random.default_rng(3)
    C0 = torch.from_numpy(rng.standard_normal((B, H, 64, 64)).astype(np.float32))
    dCT = torch.from_numpy(rng.standard_normal((B, H, 64, 64)).astype(np.float32))
    got = run_bwd(d, tables(T), C0, dCT)
    ref = oracle_bwd(d, tables(T), C0, dCT)
    check_grads(got, ref)


def test_linear_bwd_30m_layer_shape_sampled_heads():
    """The 30M-class layer (B=32, H=8, T=1024, d_h=64) in the benchmark's
    launch shape, with RoPE; two heads' gradients from the oracle."""
    B, H, T = 32, 8, 1024
    d = make_linear_inputs(B, H, T, 64, seed=42, with_dy=True)
    rope = tables(T)
    got = run_bwd(d, rope)
    for b, h in ((0, 0), (29, 6)):
        sub = {k: v[b:b + 1, h:h + 1] for k, v in d.items()}
        ref = oracle_bwd(sub, rope)
        check_grads([t[b:b + 1, h:h + 1] for t in got], ref)


def test_linear_bwd_fused_matches_chunked_at_30m_layer_shape(monkeypatch):
    """The 30M-class layer (B=32, H=8, T=1024, 256 heads: the fused form by
    default) with RoPE and an initial state, in both backward forms (a
    final-state gradient is covered at T = 300 by the tests above, in both
    forms). They run the same dC recurrence and the same per-chunk
    arithmetic, so dp1, dp2, dI and dstate_in agree bit for bit. dg differs
    only in how the sum of dB over the tokens after a chunk reads the state
    after the chunk (the fused form from its bf16 hi + lo tile in LDS, the
    chunked form in fp32): both must meet the oracle's dg bound on sampled
    heads, and agree with each other within twice that bound on every head."""
    B, H, T = 32, 8, 1024
    d = make_linear_inputs(B, H, T, 64, seed=4242, with_dy=True)
    rope = tables(T)
    rng = np.random.default_rng(11)
    C0 = torch.from_numpy((0.1 * rng.standard_normal((B, H, 64, 64))).astype(np.float32))
    dCT = None
    outs = {}
    for form in ("fused", "chunked"):
        monkeypatch.setenv("RELATION_LINEAR_BWD", form)
        outs[form] = run_bwd(d, rope, C0, dCT)
    monkeypatch.delenv("RELATION_LINEAR_BWD")
    outs["auto"] = run_bwd(d, rope, C0, dCT)
    for i, name in enumerate(("dp1", "dp2", "dI", "dg", "dstate_in")):
        assert torch.equal(outs["auto"][i], outs["fused"][i]), name
    for i, name in ((0, "dp1"), (1, "dp2"), (2, "dI"), (4, "dstate_in")):
        assert torch.equal(outs["fused"][i], outs["chunked"][i]), name
    # every head: each form is within check_dg's bound of the exact dg, so
    # the two are within twice that bound of each other (the walk taken from
    # the chunked form's dB)
    gf, gc = f64(outs["fused"][3]), f64(outs["chunked"][3])
    dB = gc - np.concatenate([gc[..., 1:, :], np.zeros_like(gc[..., :1, :])], axis=-2)
    walk = np.sqrt(np.flip(np.cumsum(np.flip(dB ** 2, axis=-2), axis=-2), axis=-2))
    worst = float((np.abs(gf - gc) / (2 * (2e-2 + 2.0 ** -7 * walk))).max())
    print(f"  dg fused vs chunked, every head: worst diff / (2 x bound) {worst:.3f}")
    assert worst <= 1.0
    for b, h in ((0, 0), (17, 3), (31, 7)):
        sub = {k: v[b:b + 1, h:h + 1] for k, v in d.items()}
        ref = oracle_bwd(sub, rope, C0[b:b + 1, h:h + 1])
        for form in ("fused", "chunked"):
            check_grads([t[b:b + 1, h:h + 1] for t in outs[form]], ref)
