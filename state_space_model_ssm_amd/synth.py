"""Seeded synthetic inputs for the Mamba-2 SSM core.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the layer's arithmetic. The oracle and the HIP path both
receive exactly these values (the oracle upcasts them to fp64, the GPU path
uploads them in their storage dtype, which represents them exactly).

Distributions (variance reading of N(mu, s)):
  x, z ~ N(0, 1);  B, C ~ N(0, 1) / sqrt(d_state)       (raw, pre-conv xBC)
  A_log = ln U[1, 16];  dt_bias = softplus^-1(logU[1e-3, 0.1])
  dt_raw ~ N(0, 0.5);  D ~ N(0, 1);  conv w ~ N(0, 1/4);  no conv bias
  initial SSM state ~ N(0, 0.1); initial conv state ~ the xBC distribution
  slot ids = permutation(num_slots)[:rows]
Slots that no row uses hold SENTINEL so tests can see that they stay untouched.
All values are drawn as float32 with NumPy's PCG64 and rounded to bf16
(round-to-nearest-even) where the storage dtype is bf16.
"""
from __future__ import annotations

import math

import numpy as np

from .configs import BF16, Dims

SENTINEL = 0.25


def round_to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    """Return float32 values exactly representable in ``dtype`` (RNE for bf16)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype != BF16:
        return a
    bits = a.view(np.uint32)
    # round-to-nearest-even on the upper 16 bits; cannot overflow uint32 for finite inputs
    out = bits + (np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1)))
    out &= np.uint32(0xFFFF0000)
    return out.view(np.float32)


def _normal(rng, shape, std=1.0):
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return v


def _log_uniform(rng, lo, hi, size):
    return np.exp(rng.uniform(math.log(lo), math.log(hi), size=size))


def _softplus_inv(y):
    y = np.asarray(y, dtype=np.float64)
    return y + np.log(-np.expm1(-y))


def layer_params(dims: Dims, rng) -> dict:
    """Per-layer parameters, fp32: conv_w [Cdim, W], A_log/dt_bias/D [H], conv_b None."""
    H = dims.nheads
    conv_w = _normal(rng, (dims.conv_dim, dims.conv_width), std=0.5)
    A_log = np.log(rng.uniform(1.0, 16.0, size=H)).astype(np.float32)
    dt_bias = _softplus_inv(_log_uniform(rng, 1e-3, 0.1, H)).astype(np.float32)
    D = _normal(rng, (H,))
    return {"conv_w": conv_w, "conv_b": None, "A_log": A_log, "dt_bias": dt_bias, "D": D}


def norm_weight(dims: Dims, seed: int) -> np.ndarray:
    """Gated-RMSNorm weight [H*P], fp32: 1 + N(0, 0.1^2), from a stream of its own
    (SeedSequence(seed) spawned child 1) so the other seeded inputs are unchanged."""
    ss = np.random.SeedSequence(seed).spawn(2)[1]
    rng = np.random.Generator(np.random.PCG64(ss))
    return (1.0 + _normal(rng, (dims.d_inner,), std=0.1)).astype(np.float32)


def xbc_values(dims: Dims, rng, rows: int) -> np.ndarray:
    """Raw xBC rows [rows, Cdim]: x ~ N(0,1), B and C ~ N(0,1)/sqrt(d_state)."""
    v = _normal(rng, (rows, dims.conv_dim))
    v[:, dims.d_inner:] *= np.float32(1.0 / math.sqrt(dims.dstate))
    return v


def tokens(dims: Dims, rng, T: int, with_z: bool = True) -> dict:
    """Per-token activations rounded to the activation dtype."""
    xbc = round_to_dtype(xbc_values(dims, rng, T), dims.act_dtype)
    dt_raw = round_to_dtype(_normal(rng, (T, dims.nheads), std=math.sqrt(0.5)), dims.act_dtype)
    out = {"xbc": xbc, "dt_raw": dt_raw, "z": None}
    if with_z:
        out["z"] = round_to_dtype(_normal(rng, (T, dims.d_inner)), dims.act_dtype)
    return out


def pools(dims: Dims, rng, num_slots: int, init_slots) -> dict:
    """SSM pool [slots, H, P, N] and conv pool [slots, W-1, Cdim], float32 values.

    Slots in ``init_slots`` get random contents (state ~ N(0, 0.1), conv state
    ~ xBC distribution); every other slot holds SENTINEL.
    """
    H, P, N, K = dims.nheads, dims.headdim, dims.dstate, dims.conv_width - 1
    ssm = np.full((num_slots, H, P, N), SENTINEL, dtype=np.float32)
    conv = np.full((num_slots, K, dims.conv_dim), SENTINEL, dtype=np.float32)
    for s in np.asarray(init_slots, dtype=np.int64).tolist():
        ssm[s] = round_to_dtype(_normal(rng, (H, P, N), std=math.sqrt(0.1)), dims.state_dtype)
        conv[s] = round_to_dtype(xbc_values(dims, rng, K), dims.state_dtype)
    return {"ssm_pool": ssm, "conv_pool": conv}


def slot_ids(rng, num_slots: int, rows: int) -> np.ndarray:
    return rng.permutation(num_slots)[:rows].astype(np.int32)


# ---------------------------------------------------------------- workloads

def tiny(dims: Dims, seed: int = 0, seqlen: int = 64, decode_steps: int = 8, num_slots: int = 4):
    """One prefill sequence from zero state, then ``decode_steps`` single-token steps."""
    rng = np.random.Generator(np.random.PCG64(seed))
    params = layer_params(dims, rng)
    slots = slot_ids(rng, num_slots, 1)
    pre = tokens(dims, rng, seqlen)
    steps = [tokens(dims, rng, 1) for _ in range(decode_steps)]
    pl = pools(dims, rng, num_slots, [])
    return {"params": params, "slots": slots, "prefill": pre, "decode": steps,
            "cu_seqlens": np.array([0, seqlen], np.int32),
            "has_initial_state": np.zeros(1, np.uint8), **pl}


def decode_batch(dims: Dims, seed: int, rows: int, num_slots: int, with_z: bool = True):
    """One decode step: ``rows`` sequences on random distinct slots, random initial state."""
    rng = np.random.Generator(np.random.PCG64(seed))
    params = layer_params(dims, rng)
    slots = slot_ids(rng, num_slots, rows)
    tok = tokens(dims, rng, rows, with_z=with_z)
    pl = pools(dims, rng, num_slots, slots)
    return {"params": params, "slots": slots, **tok, **pl}


def prefill_batch(dims: Dims, seed: int, seqlens, num_slots: int, with_z: bool = True,
                  initial_state: bool = False):
    """Packed varlen prefill. Zero initial state unless ``initial_state``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    params = layer_params(dims, rng)
    seqlens = np.asarray(seqlens, dtype=np.int64)
    slots = slot_ids(rng, num_slots, len(seqlens))
    cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    tok = tokens(dims, rng, int(cu[-1]), with_z=with_z)
    pl = pools(dims, rng, num_slots, slots if initial_state else [])
    his = np.full(len(seqlens), 1 if initial_state else 0, dtype=np.uint8)
    return {"params": params, "slots": slots, "cu_seqlens": cu, "has_initial_state": his,
            **tok, **pl}


def mixed_batch(dims: Dims, seed: int, num_prefill: int = 8, len_lo: int = 256, len_hi: int = 4096,
                decode_rows: int = 384, num_slots: int = 1024, with_z: bool = False):
    """Varlen prefill sequences (zero initial state) + decode rows (random initial state)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    params = layer_params(dims, rng)
    seqlens = rng.integers(len_lo, len_hi, endpoint=True, size=num_prefill)
    slots = slot_ids(rng, num_slots, num_prefill + decode_rows)
    cu = np.zeros(num_prefill + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    pre = tokens(dims, rng, int(cu[-1]), with_z=with_z)
    dec = tokens(dims, rng, decode_rows, with_z=with_z)
    pl = pools(dims, rng, num_slots, slots[num_prefill:])
    return {"params": params, "prefill_slots": slots[:num_prefill], "decode_slots": slots[num_prefill:],
            "cu_seqlens": cu, "has_initial_state": np.zeros(num_prefill, np.uint8),
            "prefill": pre, "decode": dec, **pl}


def stack_layer(dims: Dims, seed: int, layer: int, concurrency: int, steps: int):
    """Inputs of one layer of the decode stack: per-layer seeded params and an input
    buffer of ``concurrency + steps - 1`` rows; step s uses rows [s, s + concurrency).
    Parameters, xBC rows and dt rows come from separate streams of the layer's seed, so
    the first k rows are the same whatever ``concurrency`` and ``steps`` are."""
    ss = np.random.SeedSequence(seed).spawn(layer + 1)[layer]
    s_par, s_x, s_dt = (np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(3))
    params = layer_params(dims, s_par)
    rows = concurrency + steps - 1
    xbc = round_to_dtype(xbc_values(dims, s_x, rows), dims.act_dtype)
    dt_raw = round_to_dtype(_normal(s_dt, (rows, dims.nheads), std=math.sqrt(0.5)), dims.act_dtype)
    return {"params": params, "xbc": xbc, "dt_raw": dt_raw, "z": None}


def stack_slot(dims: Dims, seed: int, layer: int, slot: int):
    """Initial contents of one slot of one layer's pools in the decode stack (state ~
    N(0, 0.1), conv cache ~ the xBC distribution), from a stream of its own so any subset
    of slots can be drawn alone. Returns (ssm [H, P, N], conv [W-1, Cdim]) float32."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layer, slot, 0x5107])))
    H, P, N, K = dims.nheads, dims.headdim, dims.dstate, dims.conv_width - 1
    ssm = round_to_dtype(_normal(rng, (H, P, N), std=math.sqrt(0.1)), dims.state_dtype)
    conv = round_to_dtype(xbc_values(dims, rng, K), dims.state_dtype)
    return ssm, conv


def mamba1_batch(d, seed: int, seqlens, num_slots: int, with_z: bool = True, initial_state: bool = False):
    """Packed sequences for the Mamba-1 selective scan (``d`` a Mamba1Dims).

    u, z ~ N(0, 1); delta_raw ~ N(0, 0.5); delta_bias = softplus^-1(logU[1e-3, 0.1]) per
    channel; A[c][n] = -(n + 1) * exp(N(0, 0.1^2)) (the S4D-real initialisation of the Mamba
    paper, perturbed per channel); B, C ~ N(0, 1) / sqrt(dstate) per token and group;
    D = 1 + N(0, 0.1^2); initial states ~ N(0, 0.1). Activations are rounded to act_dtype.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    Dc, N, G = d.dim, d.dstate, d.ngroups
    seqlens = np.asarray(seqlens, dtype=np.int64)
    cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    T = int(cu[-1])
    A = (-(np.arange(1, N + 1, dtype=np.float64))[None, :] * np.exp(0.1 * rng.standard_normal((Dc, N)))).astype(np.float32)
    delta_bias = _softplus_inv(_log_uniform(rng, 1e-3, 0.1, Dc)).astype(np.float32)
    Dv = (1.0 + _normal(rng, (Dc,), std=0.1)).astype(np.float32)
    u = round_to_dtype(_normal(rng, (T, Dc)), d.act_dtype)
    delta_raw = round_to_dtype(_normal(rng, (T, Dc), std=math.sqrt(0.5)), d.act_dtype)
    Bm = round_to_dtype(_normal(rng, (T, G, N), std=1.0 / math.sqrt(N)), d.act_dtype)
    Cm = round_to_dtype(_normal(rng, (T, G, N), std=1.0 / math.sqrt(N)), d.act_dtype)
    z = round_to_dtype(_normal(rng, (T, Dc)), d.act_dtype) if with_z else None
    slots = slot_ids(rng, num_slots, len(seqlens))
    pool = np.full((num_slots, Dc, N), SENTINEL, dtype=np.float32)
    if initial_state:
        for sl in slots.tolist():
            pool[sl] = round_to_dtype(_normal(rng, (Dc, N), std=math.sqrt(0.1)), d.state_dtype)
    his = np.full(len(seqlens), 1 if initial_state else 0, dtype=np.uint8)
    return {"u": u, "delta_raw": delta_raw, "A": A, "B": Bm, "C": Cm, "D": Dv, "z": z, "delta_bias": delta_bias,
            "cu_seqlens": cu, "slots": slots, "has_initial_state": his, "ssm_pool": pool}
