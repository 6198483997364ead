"""Seeded input recipes for the Relation operator's workloads.

Recipe (shared by every test and by the benchmark):
  * numpy.random.default_rng(seed); the draw order is lambda, q, k, v, dY,
    then (decode only) the cache history, the unused cache slots and the
    per-step q, k_new, v_new.
  * lambda ~ U(0, 1): the pages make lambda a learnable layer-wise scalar and
    state no initial value.
  * q, k, v, dY ~ N(0, 1) drawn as float32; the RoPE workload scales q and k
    by 1/sqrt(D) and then applies full-head rotary encoding (base 1e4,
    positions 0..T-1, rotate-half pairing (m, m + D/2)), as the pages apply
    RoPE to p1 and p2 before the pairwise evidence.
  * Tensors of the bf16 workloads are rounded to bf16 (round to nearest even)
    once; the same rounded values feed the GPU and the oracle (which upcasts
    them to float64).

Linear Relation inputs (make_linear_inputs): p1, p2, I, dY ~ N(0, 1) rounded
to bf16 as above, and the log retention g <= 0 (float32) drawn with the
spread that the pages' KDA-style retention map has at initialisation: per
(b, h, channel) a magnitude m = U(1, 16) * exp(U(ln 1e-3, ln 1e-1)), per token
|g| = m * exp(0.5 z), z ~ N(0, 1). The "resets" option sets a random 1 % of
(token, channel) entries to g = -60 (near-total retention loss) and the
"keep" option a random 1/8 of channels to g = 0 (no loss).

Nothing here computes any part of the Relation operator itself.
"""
import math
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "Workload",
    "WORKLOADS",
    "make_inputs",
    "make_decode_inputs",
    "ragged_decode_lengths",
    "make_linear_inputs",
    "make_mhr_maps",
    "apply_rope",
    "to_dtype",
    "default_scale",
]


@dataclass(frozen=True)
class Workload:
    key: str
    kind: str            # "fwd", "fwdbwd" or "decode"
    dtype: str           # "f32" or "bf16"
    B: int
    H: int
    D: int
    T: int = 0           # sequence length (fwd / fwdbwd)
    rope: bool = False
    n_hist: int = 0      # decode: cached history length before the first step
    steps: int = 0       # decode: consecutive steps
    capacity: int = 0    # decode: cache slots per (b, h)
    note: str = field(default="", compare=False)


WORKLOADS = {
    "mhr_fwd_f32": Workload("mhr_fwd_f32", "fwd", "f32", B=1, H=2, D=32, T=128,
                            note="single Multi-Head Relation forward, fp32"),
    "layer10m_fwd_bf16": Workload("layer10m_fwd_bf16", "fwd", "bf16", B=8, H=8, D=64, T=1024,
                                  rope=True, note="10M-model-shaped layer, RoPE'd q/k"),
    "layer30m_fwdbwd_bf16": Workload("layer30m_fwdbwd_bf16", "fwdbwd", "bf16", B=16, H=8, D=64,
                                     T=2048, note="30M-model-shaped layer"),
    "layer100m_fwdbwd_bf16": Workload("layer100m_fwdbwd_bf16", "fwdbwd", "bf16", B=8, H=12,
                                      D=64, T=4096, note="100M-model-shaped layer"),
    "cache_decode_bf16": Workload("cache_decode_bf16", "decode", "bf16", B=32, H=12, D=64,
                                  n_hist=4096, steps=256, capacity=4352,
                                  note="Relation Cache decode, 256 steps from history 4096"),
}


def ragged_decode_lengths(B, max_n, seed):
    """Seeded per-sequence history lengths for a ragged Relation Cache batch:
    uniform integers in [0, max_n], with sequence 0 at max_n and sequence 1
    at 0 so that both extremes are always present."""
    rng = np.random.default_rng(seed + 7919)
    n = rng.integers(0, max_n + 1, size=B)
    n[0] = max_n
    if B > 1:
        n[1] = 0
    return [int(x) for x in n]


def make_mhr_maps(T, D, H, seed, base=1.0e4):
    """Inputs of Multi-Head Relation's upstream maps: RoPE tables cos, sin
    [T, D/2] float32 (angle t * base^(-2j/D) at position t, evaluated in
    float64 and rounded once) and seeded Givens angles theta [H/2] float32,
    uniform in [-pi, pi]. CPU torch tensors."""
    j = np.arange(D // 2, dtype=np.float64)
    ang = np.arange(T, dtype=np.float64)[:, None] * base ** (-2.0 * j / D)[None, :]
    rng = np.random.default_rng(seed + 104729)
    th = rng.uniform(-math.pi, math.pi, size=max(H // 2, 1))
    return (torch.from_numpy(np.cos(ang).astype(np.float32)),
            torch.from_numpy(np.sin(ang).astype(np.float32)),
            torch.from_numpy(th.astype(np.float32)))


def default_scale(D):
    """1/sqrt(d_h): the pages' U = p1.p2 / d_h with the square root that the
    extracted text drops (the textbook scaled dot product)."""
    return 1.0 / math.sqrt(D)


def to_dtype(x, dtype):
    """float32 numpy array -> CPU torch tensor of the workload dtype (bf16 by
    round-to-nearest-even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t.clone()
    raise ValueError(dtype)


def apply_rope(x, base=10000.0):
    """Full-head rotary encoding, rotate-half pairing, positions 0..T-1.
    x: float32 [..., T, D]. Computed in float64, returned as float32."""
    T, D = x.shape[-2], x.shape[-1]
    half = D // 2
    inv = base ** (-(np.arange(half, dtype=np.float64) * 2.0) / D)
    ang = np.arange(T, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x = x.astype(np.float64)
    a, b = x[..., :half], x[..., half:]
    out = np.concatenate([a * c - b * s, a * s + b * c], axis=-1)
    return out.astype(np.float32)


def make_inputs(B, H, T, D, dtype, seed, rope=False, with_dy=False, lam=None):
    """Seeded forward / backward inputs.

    Returns dict(lam, q, k, v[, dy]) where the tensors are CPU torch tensors
    of the workload dtype, shape [B, H, T, D]. lambda is drawn from the seed
    unless given.
    """
    rng = np.random.default_rng(seed)
    lam_draw = float(rng.uniform(0.0, 1.0))
    shape = (B, H, T, D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if rope:
        q = apply_rope(q / math.sqrt(D))
        k = apply_rope(k / math.sqrt(D))
    out = {
        "lam": lam_draw if lam is None else float(lam),
        "q": to_dtype(q, dtype),
        "k": to_dtype(k, dtype),
        "v": to_dtype(v, dtype),
    }
    if with_dy:
        out["dy"] = to_dtype(rng.standard_normal(shape, dtype=np.float32), dtype)
    return out


def make_decode_inputs(B, H, D, n_hist, steps, capacity, dtype, seed, lam=None):
    """Seeded Relation Cache decode inputs.

    Returns dict(lam, k_cache, v_cache [B,H,capacity,D], q, k_new, v_new
    [steps,B,H,D]). Slots [0, n_hist) hold the history; the unused slots are
    filled with other random values so that a test can check they are left
    untouched.
    """
    if n_hist + steps > capacity:
        raise ValueError("capacity too small for n_hist + steps")
    rng = np.random.default_rng(seed)
    lam_draw = float(rng.uniform(0.0, 1.0))
    kc = np.empty((B, H, capacity, D), dtype=np.float32)
    vc = np.empty((B, H, capacity, D), dtype=np.float32)
    kc[:, :, :n_hist] = rng.standard_normal((B, H, n_hist, D), dtype=np.float32)
    vc[:, :, :n_hist] = rng.standard_normal((B, H, n_hist, D), dtype=np.float32)
    kc[:, :, n_hist:] = rng.standard_normal((B, H, capacity - n_hist, D), dtype=np.float32)
    vc[:, :, n_hist:] = rng.standard_normal((B, H, capacity - n_hist, D), dtype=np.float32)
    step_shape = (steps, B, H, D)
    q = rng.standard_normal(step_shape, dtype=np.float32)
    kn = rng.standard_normal(step_shape, dtype=np.float32)
    vn = rng.standard_normal(step_shape, dtype=np.float32)
    return {
        "lam": lam_draw if lam is None else float(lam),
        "k_cache": to_dtype(kc, dtype),
        "v_cache": to_dtype(vc, dtype),
        "q": to_dtype(q, dtype),
        "k_new": to_dtype(kn, dtype),
        "v_new": to_dtype(vn, dtype),
    }


def make_linear_inputs(B, H, T, D, seed, with_dy=False, resets=False, keep=False):
    """Seeded Linear Relation inputs: dict(p1, p2, I[, dy]) bf16 and g float32,
    CPU tensors of shape [B, H, T, D] (recipe in the module docstring)."""
    rng = np.random.default_rng(seed)
    shape = (B, H, T, D)
    p1 = rng.standard_normal(shape, dtype=np.float32)
    p2 = rng.standard_normal(shape, dtype=np.float32)
    iv = rng.standard_normal(shape, dtype=np.float32)
    mag = rng.uniform(1.0, 16.0, (B, H, 1, D)) * np.exp(
        rng.uniform(math.log(1e-3), math.log(1e-1), (B, H, 1, D)))
    z = rng.standard_normal(shape)
    g = -(mag * np.exp(0.5 * z))
    if resets:
        g[rng.uniform(size=shape) < 0.01] = -60.0
    if keep:
        g[np.broadcast_to(rng.uniform(size=(B, H, 1, D)) < 0.125, shape)] = 0.0
    out = {"p1": to_dtype(p1, "bf16"), "p2": to_dtype(p2, "bf16"), "I": to_dtype(iv, "bf16"),
           "g": torch.from_numpy(g.astype(np.float32))}
    if with_dy:
        out["dy"] = to_dtype(rng.standard_normal(shape, dtype=np.float32), "bf16")
    return out
