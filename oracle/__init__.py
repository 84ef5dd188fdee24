"""Plain fp64 CPU oracle for the Mamba-2 SSM core.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product package.
It shares no code with the HIP library; the two meet only at the seeded
inputs, which both receive from the generator module.

Sources of what it computes (see ``ssm_oracle.c`` for the step list):
  * conv1d + SiLU prefill and single-step forms, and the in-place slot update
    of conv/SSM caches: the vllm.cpp issue "NemotronH runs the PREFILL mamba
    kernels at decode", section "The divergence" (decode ops take
    state/conv-state indices and read+write the cache in place at the slot);
  * the per-head tensors A_log, D, dt_bias and the n_groups=8 grouping: the
    "Nemotron-H-8B-Base-8K" record (mixer tensors, "Recurrent state");
  * the equivalence contract (a T-token chunk scan equals T single steps):
    the vllm.cpp issue, section "Confirm or refute";
  * the gated RMSNorm of the mixer output (``norm.py``): the record's "norm"
    mixer tensor;
  * the Mamba-1 selective scan (diagonal A per channel and state): the
    "selective_scan_fwd" kernel the trace page names for Mamba layers, with the
    recurrence of the Mamba paper that page cites.

Every function here loops over sequences and tokens in order and calls the C
routines, which hold the arithmetic. ``dual`` (the quadratic matrix form) is a
second, independent NumPy formulation used to pin the C loop.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssm_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libssm_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, no fast-math, OpenMP across heads)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            dp = ctypes.POINTER(ctypes.c_double)
            lib.oracle_conv1d_seq.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, dp, dp,
                                              dp, dp, dp]
            lib.oracle_conv1d_seq.restype = None
            lib.oracle_ssm_seq.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, ctypes.c_int32, dp, dp, dp, dp, dp, dp,
                                           dp, dp, ctypes.c_int32]
            lib.oracle_ssm_seq.restype = None
            lib.oracle_selective_scan_seq.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                      ctypes.c_int32, dp, dp, dp, dp, dp, dp, dp, dp,
                                                      ctypes.c_int32, dp, dp]
            lib.oracle_selective_scan_seq.restype = None
            for name in ("oracle_softplus", "oracle_silu", "oracle_round_bf16"):
                getattr(lib, name).argtypes = [ctypes.c_double]
                getattr(lib, name).restype = ctypes.c_double
            _lib = lib
    return _lib


def _ptr(a):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def softplus(v: float) -> float:
    return _load().oracle_softplus(float(v))


def silu(v: float) -> float:
    return _load().oracle_silu(float(v))


def round_bf16(v: float) -> float:
    return _load().oracle_round_bf16(float(v))


def conv1d_seq(u, w, bias, state):
    """One sequence of causal conv1d + SiLU.

    u [T, C] raw inputs; w [C, W]; bias [C] or None; state [W-1, C] cached raw
    inputs (oldest first). Returns (out [T, C], new_state [W-1, C]).
    """
    u = _f64(u)
    w = _f64(w)
    T, C = u.shape
    W = w.shape[1]
    assert w.shape == (C, W) and 1 <= W <= 16
    st = np.array(state, dtype=np.float64, copy=True, order="C").reshape(W - 1, C)
    out = np.empty((T, C), dtype=np.float64)
    _load().oracle_conv1d_seq(T, C, W, _ptr(u), _ptr(w), _ptr(_f64(bias)), _ptr(st), _ptr(out))
    return out, st


def ssm_seq(xbc_post, dt_raw, A_log, dt_bias, D, h0, *, H, P, N, G, z=None, round_state_bf16=False):
    """One sequence of the selective recurrence on post-conv channels.

    xbc_post [T, H*P + 2*G*N]; dt_raw [T, H]; A_log/dt_bias/D [H]; h0 [H, P, N];
    z [T, H*P] or None. Returns (y [T, H*P], h_final [H, P, N]).
    """
    xbc_post = _f64(xbc_post)
    T = xbc_post.shape[0]
    assert xbc_post.shape[1] == H * P + 2 * G * N and H % G == 0
    dt_raw = _f64(dt_raw).reshape(T, H)
    h = np.array(h0, dtype=np.float64, copy=True, order="C").reshape(H, P, N)
    y = np.empty((T, H * P), dtype=np.float64)
    zz = None if z is None else _f64(z).reshape(T, H * P)
    _load().oracle_ssm_seq(T, H, P, N, G, _ptr(xbc_post), _ptr(dt_raw), _ptr(_f64(A_log)),
                           _ptr(_f64(dt_bias)), _ptr(_f64(D)), _ptr(zz), _ptr(h), _ptr(y),
                           1 if round_state_bf16 else 0)
    return y, h


def layer_seq(xbc_raw, dt_raw, params, conv_state, ssm_state, *, H, P, N, G, z=None,
              round_state_bf16=False):
    """conv1d + SiLU then the recurrence, for one sequence.

    params: dict with conv_w [Cdim, W], conv_b (or None), A_log, dt_bias, D.
    Returns (y, xbc_post, new_conv_state, new_ssm_state).
    """
    post, cs = conv1d_seq(xbc_raw, params["conv_w"], params.get("conv_b"), conv_state)
    y, hs = ssm_seq(post, dt_raw, params["A_log"], params["dt_bias"], params["D"], ssm_state,
                    H=H, P=P, N=N, G=G, z=z, round_state_bf16=round_state_bf16)
    return y, post, cs, hs


def prefill(xbc_raw, dt_raw, params, cu_seqlens, state_indices, has_initial_state,
            conv_pool, ssm_pool, *, H, P, N, G, z=None):
    """Varlen prefill over packed sequences; updates fp64 pools in place.

    xbc_raw [T_tot, Cdim]; cu_seqlens [nseq+1]; state_indices [nseq] (slot of
    each sequence); has_initial_state [nseq] or None (all zero: start from zero
    conv and SSM state). conv_pool [slots, W-1, Cdim], ssm_pool [slots, H, P, N]
    (float64, modified in place). Returns (y [T_tot, H*P], xbc_post).
    """
    T_tot, Cdim = xbc_raw.shape
    y = np.zeros((T_tot, H * P), dtype=np.float64)
    post = np.zeros((T_tot, Cdim), dtype=np.float64)
    for i in range(len(cu_seqlens) - 1):
        s, e = int(cu_seqlens[i]), int(cu_seqlens[i + 1])
        slot = int(state_indices[i])
        if slot < 0:
            continue
        init = bool(has_initial_state[i]) if has_initial_state is not None else False
        cs0 = conv_pool[slot] if init else np.zeros_like(conv_pool[slot])
        h0 = ssm_pool[slot] if init else np.zeros_like(ssm_pool[slot])
        zz = None if z is None else z[s:e]
        yy, pp, cs, hs = layer_seq(xbc_raw[s:e], dt_raw[s:e], params, cs0, h0, H=H, P=P, N=N, G=G,
                                   z=zz)
        y[s:e] = yy
        post[s:e] = pp
        conv_pool[slot] = cs
        ssm_pool[slot] = hs
    return y, post


def decode(xbc_raw, dt_raw, params, state_indices, conv_pool, ssm_pool, *, H, P, N, G, z=None,
           round_state_bf16=False):
    """One token per row, reading and writing the pools in place at the slots.

    Rows with a negative slot are padding: y stays zero and no slot is touched.
    Returns (y [B, H*P], xbc_post [B, Cdim]).
    """
    Bd, Cdim = xbc_raw.shape
    y = np.zeros((Bd, H * P), dtype=np.float64)
    post = np.zeros((Bd, Cdim), dtype=np.float64)
    for i in range(Bd):
        slot = int(state_indices[i])
        if slot < 0:
            continue
        zz = None if z is None else z[i:i + 1]
        yy, pp, cs, hs = layer_seq(xbc_raw[i:i + 1], dt_raw[i:i + 1], params, conv_pool[slot],
                                   ssm_pool[slot], H=H, P=P, N=N, G=G, z=zz,
                                   round_state_bf16=round_state_bf16)
        y[i] = yy[0]
        post[i] = pp[0]
        conv_pool[slot] = cs
        ssm_pool[slot] = hs
    return y, post


def selective_scan_seq(u, delta_raw, A, B, C, h0, *, D=None, z=None, delta_bias=None, delta_softplus=True):
    """One sequence of the Mamba-1 selective scan (diagonal A per channel and state).

    u, delta_raw [T, Dc]; A [Dc, N]; B, C [T, G, N]; h0 [Dc, N]; D, delta_bias [Dc] or
    None; z [T, Dc] or None. Returns (y [T, Dc], h_final [Dc, N]).
    """
    u = _f64(u)
    T, Dc = u.shape
    A = _f64(A)
    N = A.shape[1]
    B = _f64(B)
    assert B.ndim == 3 and B.shape[0] == T and B.shape[2] == N, "B must be [T, G, N]"
    G = B.shape[1]
    assert Dc % G == 0
    h = np.array(h0, dtype=np.float64, copy=True, order="C").reshape(Dc, N)
    y = np.empty((T, Dc), dtype=np.float64)
    _load().oracle_selective_scan_seq(T, Dc, N, G, _ptr(u), _ptr(_f64(delta_raw).reshape(T, Dc)), _ptr(A), _ptr(B),
                                      _ptr(_f64(C).reshape(T, G, N)), _ptr(_f64(D)),
                                      _ptr(None if z is None else _f64(z).reshape(T, Dc)), _ptr(_f64(delta_bias)),
                                      1 if delta_softplus else 0, _ptr(h), _ptr(y))
    return y, h


def selective_scan(u, delta_raw, A, B, C, cu_seqlens, state_indices, has_initial_state, ssm_pool, *, D=None, z=None,
                   delta_bias=None, delta_softplus=True):
    """Packed sequences of the selective scan; ssm_pool [slots, Dc, N] fp64, updated in place
    (final state of each sequence to its slot; negative slot = padding, y stays zero)."""
    T, Dc = u.shape
    y = np.zeros((T, Dc), dtype=np.float64)
    for i in range(len(cu_seqlens) - 1):
        s, e = int(cu_seqlens[i]), int(cu_seqlens[i + 1])
        slot = int(state_indices[i])
        if slot < 0:
            continue
        init = bool(has_initial_state[i]) if has_initial_state is not None else False
        h0 = ssm_pool[slot] if init else np.zeros_like(ssm_pool[slot])
        yy, hh = selective_scan_seq(u[s:e], delta_raw[s:e], A, B[s:e], C[s:e], h0, D=D,
                                    z=None if z is None else z[s:e], delta_bias=delta_bias,
                                    delta_softplus=delta_softplus)
        y[s:e] = yy
        ssm_pool[slot] = hh
    return y


def decode_multi(xbc_raw, dt_raw, params, src_indices, dst_indices, conv_pool, ssm_pool, *, H, P, N, G, z=None):
    """T tokens per row (multi-token decode, e.g. verifying drafted tokens).

    xbc_raw [B, T, Cdim]; dt_raw [B, T, H]; z [B, T, H*P] or None. Row i starts from
    slot src_indices[i] and takes its T tokens in order, one step each. After step t
    the conv and SSM state are written to slot dst_indices[i][t] when that is >= 0;
    with dst_indices None only the final state is written, to src_indices[i]. Slots
    are read before any is written. Rows with a negative source slot are padding:
    y stays zero and no slot is touched. Returns (y [B, T, H*P], xbc_post [B, T, Cdim]).
    """
    Bd, T, Cdim = xbc_raw.shape
    y = np.zeros((Bd, T, H * P), dtype=np.float64)
    post = np.zeros((Bd, T, Cdim), dtype=np.float64)
    start_conv = {int(s): conv_pool[int(s)].copy() for s in src_indices if s >= 0}
    start_ssm = {int(s): ssm_pool[int(s)].copy() for s in src_indices if s >= 0}
    writes = []
    for i in range(Bd):
        src = int(src_indices[i])
        if src < 0:
            continue
        cs, hs = start_conv[src], start_ssm[src]
        for t in range(T):
            zz = None if z is None else z[i, t:t + 1]
            yy, pp, cs, hs = layer_seq(xbc_raw[i, t:t + 1], dt_raw[i, t:t + 1], params, cs, hs, H=H, P=P, N=N, G=G,
                                       z=zz)
            y[i, t] = yy[0]
            post[i, t] = pp[0]
            if dst_indices is not None and int(dst_indices[i][t]) >= 0:
                writes.append((int(dst_indices[i][t]), cs.copy(), hs.copy()))
        if dst_indices is None:
            writes.append((src, cs.copy(), hs.copy()))
    for slot, cs, hs in writes:
        conv_pool[slot] = cs
        ssm_pool[slot] = hs
    return y, post


from . import dual  # noqa: E402,F401  (independent quadratic form)
from .norm import gated_rmsnorm  # noqa: E402,F401  (the mixer's gated RMSNorm)
