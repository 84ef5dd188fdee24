"""ctypes binding of libmamba2.so (the gfx950 HIP library), same names as the C ABI.

Argument marshalling only: every function checks tensor devices, dtypes and
shapes, turns torch tensors into device pointers and passes the current HIP
stream. All computation runs in the library's kernels; there is no fallback.
If the library is missing, calls raise immediately.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading
from typing import Optional

import torch

from .configs import BF16, F32, Dims

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmamba2.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "mamba2.h")
HEADER_PATHS = [HEADER_PATH, os.path.join(os.path.dirname(_HERE), "include", "mamba1.h")]

_DT_CODE = {F32: 0, BF16: 1}
_TORCH_DT = {F32: torch.float32, BF16: torch.bfloat16}

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_NO_SLOT = range(6)


class Mamba2Error(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class CDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "nheads", "headdim", "dstate", "ngroups", "conv_width", "chunk_size",
        "act_dtype", "xbc_dtype", "state_dtype", "out_dtype")]


class CDims1(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("dim", "dstate", "ngroups", "act_dtype", "state_dtype", "out_dtype")]


def cdims1(d) -> CDims1:
    return CDims1(d.dim, d.dstate, d.ngroups, _DT_CODE[d.act_dtype], _DT_CODE[d.state_dtype], _DT_CODE[d.out_dtype])


def cdims(d: Dims, xbc_dtype: Optional[str] = None) -> CDims:
    """C struct for ``d``. The post-conv buffer dtype defaults to ``d.post_dtype``."""
    if xbc_dtype is None:
        xbc_dtype = d.post_dtype
    return CDims(d.nheads, d.headdim, d.dstate, d.ngroups, d.conv_width, d.chunk_size,
                 _DT_CODE[d.act_dtype], _DT_CODE[xbc_dtype], _DT_CODE[d.state_dtype], _DT_CODE[d.out_dtype])


_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SIGS = {
    "mamba2_check_dims": (ctypes.c_int, [ctypes.POINTER(CDims)]),
    "mamba2_ssm_slot_bytes": (ctypes.c_size_t, [ctypes.POINTER(CDims)]),
    "mamba2_conv_slot_bytes": (ctypes.c_size_t, [ctypes.POINTER(CDims)]),
    "mamba2_chunk_scan_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(CDims), ctypes.c_int64, ctypes.c_int32,
                                                          ctypes.POINTER(ctypes.c_size_t)]),
    "mamba2_conv1d_fwd": (ctypes.c_int, [ctypes.POINTER(CDims), _P, _P, _P, _P, _P, _I32, _P, _I32,
                                         ctypes.c_int64, _P, _P, _P]),
    "mamba2_conv1d_update": (ctypes.c_int, [ctypes.POINTER(CDims), _P, _P, _P, _P, _P, _I32, _P, _I32, _P]),
    "mamba2_chunk_scan_fwd": (ctypes.c_int, [ctypes.POINTER(CDims), _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P,
                                             _I32, ctypes.c_int64, _P, _P, _P, ctypes.c_size_t, _P]),
    "mamba2_state_update": (ctypes.c_int, [ctypes.POINTER(CDims), _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P,
                                           _I32, _P]),
    "mamba2_mixed_fwd": (ctypes.c_int, [ctypes.POINTER(CDims), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                        _I32, _P, _I32, ctypes.c_int64, _P, _P, _P, _I32, _P,
                                        ctypes.c_size_t, _P]),
    "mamba2_conv1d_update_multi": (ctypes.c_int, [ctypes.POINTER(CDims), _P, _P, _P, _P, _P, _I32, _P, _P,
                                                   _I32, _I32, _P]),
    "mamba2_state_update_multi": (ctypes.c_int, [ctypes.POINTER(CDims), _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P,
                                                  _P, _I32, _I32, _P]),
    "mamba2_prefill_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(CDims), ctypes.c_int64,
                                                       ctypes.POINTER(ctypes.c_size_t)]),
    "mamba2_prefill_fwd": (ctypes.c_int, [ctypes.POINTER(CDims), _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                          _I32, _P, _P, _P, _I32, _P, _I32, ctypes.c_int64, _P, _P, _P,
                                          ctypes.c_size_t, _P]),
    "mamba2_prefill_fwd_noalloc": (ctypes.c_int, [ctypes.POINTER(CDims), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                  ctypes.c_float, _I32, _P, _P, _P, _I32, _P, _I32, ctypes.c_int64,
                                                  _P, _P, _P]),
    "mamba2_gated_rmsnorm": (ctypes.c_int, [ctypes.POINTER(CDims), _P, _P, _P, ctypes.c_float, ctypes.c_int32, _P,
                                            ctypes.c_int64, _P]),
    "mamba1_ssm_slot_bytes": (ctypes.c_size_t, [ctypes.POINTER(CDims1)]),
    "mamba1_selective_scan_fwd": (ctypes.c_int, [ctypes.POINTER(CDims1), _P, _P, _P, _P, _P, _P, _P, _P,
                                                  _I32, _P, _P, _I32, _P, _I32, ctypes.c_int64, _P, _P, _P]),
    "mamba1_selective_state_update": (ctypes.c_int, [ctypes.POINTER(CDims1), _P, _P, _P, _P, _P, _P, _P, _P,
                                                      _I32, _P, _P, _I32, _P, _I32, _P]),
    "mamba2_read_slot_errors": (ctypes.c_int, [_P, _I32, _P]),
    "mamba2_decode_graph_create": (ctypes.c_int, [ctypes.POINTER(CDims), _P, _I32, _I32, _P, ctypes.POINTER(_P)]),
    "mamba2_decode_graph_launch": (ctypes.c_int, [_P, _P]),
    "mamba2_decode_graph_destroy": (None, [_P]),
    "mamba2_decode_graph_last_error": (ctypes.c_char_p, []),
    "mamba2_check_slot_indices": (ctypes.c_int, [_P, _I32, _I32, _P, _P]),
    "mamba2_slots_create": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(_P)]),
    "mamba2_slot_alloc": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_int32)]),
    "mamba2_slot_free": (ctypes.c_int, [_P, ctypes.c_int32]),
    "mamba2_slots_in_use": (ctypes.c_int32, [_P]),
    "mamba2_slots_destroy": (None, [_P]),
    "mamba2_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "mamba2_last_error": (ctypes.c_char_p, []),
    "mamba2_version": (ctypes.c_char_p, []),
}


def lib():
    """Load libmamba2.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m state_space_model_ssm_amd.build` "
                                   "(the HIP library is the only implementation; there is no fallback)")
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGS.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions declared in include/mamba2.h."""
    text = "".join(open(p).read() for p in HEADER_PATHS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mamba[12]_[a-z0-9_]+)\s*\(", text)))


def _check(status: int, fn: str):
    if status != OK:
        raise Mamba2Error(status, fn, lib().mamba2_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _want(t, name, dtype=None, shape=None, device=True, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _xdt(d: Dims, xbc_dtype):
    return _TORCH_DT[xbc_dtype or d.post_dtype]


def _ssm_slots(d: Dims, pool) -> int:
    """Slot count of an SSM pool [slots, H, P, N] (checked)."""
    if pool is None or pool.dim() != 4 or tuple(pool.shape[1:]) != (d.nheads, d.headdim, d.dstate):
        raise ValueError(f"ssm_pool must be [slots, {d.nheads}, {d.headdim}, {d.dstate}], got "
                         f"{None if pool is None else tuple(pool.shape)}")
    _want(pool, "ssm_pool", _TORCH_DT[d.state_dtype])
    return int(pool.shape[0])


def _conv_slots(d: Dims, pool) -> int:
    """Slot count of a conv pool [slots, W-1, Cdim] (checked)."""
    if pool is None or pool.dim() != 3 or tuple(pool.shape[1:]) != (d.conv_width - 1, d.conv_dim):
        raise ValueError(f"conv_pool must be [slots, {d.conv_width - 1}, {d.conv_dim}], got "
                         f"{None if pool is None else tuple(pool.shape)}")
    _want(pool, "conv_pool", _TORCH_DT[d.state_dtype])
    return int(pool.shape[0])


def _both_slots(d: Dims, ssm_pool, conv_pool) -> int:
    n = _ssm_slots(d, ssm_pool)
    if _conv_slots(d, conv_pool) != n:
        raise ValueError("ssm_pool and conv_pool must have the same number of slots")
    return n


def _debug_check(num_slots: int, *index_tensors) -> None:
    """With MAMBA2_CHECK_SLOTS=1 in the environment, every call that indexes a pool first
    checks its index tables on the device (out-of-range and repeated slots; this waits for
    the device) and raises on either."""
    if os.environ.get("MAMBA2_CHECK_SLOTS", "0") in ("", "0"):
        return
    idx = torch.cat([t.reshape(-1) for t in index_tensors if t is not None])
    bad, dup = check_slot_indices(idx, num_slots)
    if bad or dup:
        raise ValueError(f"slot indices: {bad} >= num_slots ({num_slots}), {dup} repeated")


# ------------------------------------------------------------------ queries

def mamba2_check_dims(d: Dims, xbc_dtype=None) -> None:
    c = cdims(d, xbc_dtype)
    _check(lib().mamba2_check_dims(ctypes.byref(c)), "mamba2_check_dims")


def mamba2_ssm_slot_bytes(d: Dims) -> int:
    return int(lib().mamba2_ssm_slot_bytes(ctypes.byref(cdims(d))))


def mamba2_conv_slot_bytes(d: Dims) -> int:
    return int(lib().mamba2_conv_slot_bytes(ctypes.byref(cdims(d))))


def mamba2_chunk_scan_workspace_bytes(d: Dims, total_tokens: int, nseq: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().mamba2_chunk_scan_workspace_bytes(ctypes.byref(cdims(d)), total_tokens, nseq, ctypes.byref(out)),
           "mamba2_chunk_scan_workspace_bytes")
    return int(out.value)


# ------------------------------------------------------------------ compute

def mamba2_conv1d_fwd(d: Dims, xbc, conv_w, conv_b, xbc_out, conv_pool, cu_seqlens, state_indices,
                      has_initial_state=None, *, xbc_dtype=None, stream=None):
    T = xbc.shape[0]
    nseq = state_indices.shape[0]
    _want(xbc, "xbc", _TORCH_DT[d.act_dtype], (T, d.conv_dim))
    _want(conv_w, "conv_w", torch.float32, (d.conv_dim, d.conv_width))
    _want(conv_b, "conv_b", torch.float32, (d.conv_dim,), optional=True)
    _want(xbc_out, "xbc_out", _xdt(d, xbc_dtype), (T, d.conv_dim))
    ns = _conv_slots(d, conv_pool)
    _want(cu_seqlens, "cu_seqlens", torch.int32, (nseq + 1,))
    _want(state_indices, "state_indices", torch.int32, (nseq,))
    _want(has_initial_state, "has_initial_state", torch.uint8, (nseq,), optional=True)
    _debug_check(ns, state_indices)
    c = cdims(d, xbc_dtype)
    _check(lib().mamba2_conv1d_fwd(ctypes.byref(c), _ptr(xbc), _ptr(conv_w), _ptr(conv_b), _ptr(xbc_out),
                                   _ptr(conv_pool), ns, _ptr(cu_seqlens), nseq, T, _ptr(state_indices),
                                   _ptr(has_initial_state), _stream(stream)), "mamba2_conv1d_fwd")


def mamba2_conv1d_update(d: Dims, xbc, conv_w, conv_b, xbc_out, conv_pool, state_indices, *, xbc_dtype=None,
                         stream=None):
    Bd = state_indices.shape[0]
    _want(xbc, "xbc", _TORCH_DT[d.act_dtype], (Bd, d.conv_dim))
    _want(conv_w, "conv_w", torch.float32, (d.conv_dim, d.conv_width))
    _want(conv_b, "conv_b", torch.float32, (d.conv_dim,), optional=True)
    _want(xbc_out, "xbc_out", _xdt(d, xbc_dtype), (Bd, d.conv_dim))
    ns = _conv_slots(d, conv_pool)
    _want(state_indices, "state_indices", torch.int32, (Bd,))
    _debug_check(ns, state_indices)
    c = cdims(d, xbc_dtype)
    _check(lib().mamba2_conv1d_update(ctypes.byref(c), _ptr(xbc), _ptr(conv_w), _ptr(conv_b), _ptr(xbc_out),
                                      _ptr(conv_pool), ns, _ptr(state_indices), Bd, _stream(stream)),
           "mamba2_conv1d_update")


def mamba2_chunk_scan_fwd(d: Dims, xbc, dt_raw, A_log, dt_bias, D, z, y, ssm_pool, cu_seqlens, state_indices,
                          has_initial_state=None, workspace=None, *, xbc_dtype=None, stream=None):
    T = xbc.shape[0]
    nseq = state_indices.shape[0]
    H = d.nheads
    _want(xbc, "xbc", _xdt(d, xbc_dtype), (T, d.conv_dim))
    _want(dt_raw, "dt_raw", _TORCH_DT[d.act_dtype], (T, H))
    for n, t in (("A_log", A_log), ("dt_bias", dt_bias), ("D", D)):
        _want(t, n, torch.float32, (H,))
    _want(z, "z", _TORCH_DT[d.act_dtype], (T, d.d_inner), optional=True)
    _want(y, "y", _TORCH_DT[d.out_dtype], (T, d.d_inner))
    ns = _ssm_slots(d, ssm_pool)
    _want(cu_seqlens, "cu_seqlens", torch.int32, (nseq + 1,))
    _want(state_indices, "state_indices", torch.int32, (nseq,))
    _want(has_initial_state, "has_initial_state", torch.uint8, (nseq,), optional=True)
    _debug_check(ns, state_indices)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    c = cdims(d, xbc_dtype)
    _check(lib().mamba2_chunk_scan_fwd(ctypes.byref(c), _ptr(xbc), _ptr(dt_raw), _ptr(A_log), _ptr(dt_bias),
                                       _ptr(D), _ptr(z), _ptr(y), _ptr(ssm_pool), ns, _ptr(cu_seqlens), nseq, T,
                                       _ptr(state_indices), _ptr(has_initial_state), _ptr(workspace), ws_bytes,
                                       _stream(stream)), "mamba2_chunk_scan_fwd")


def mamba2_state_update(d: Dims, xbc, dt_raw, A_log, dt_bias, D, z, y, ssm_pool, state_indices, *,
                        xbc_dtype=None, stream=None):
    Bd = state_indices.shape[0]
    H = d.nheads
    _want(xbc, "xbc", _xdt(d, xbc_dtype), (Bd, d.conv_dim))
    _want(dt_raw, "dt_raw", _TORCH_DT[d.act_dtype], (Bd, H))
    for n, t in (("A_log", A_log), ("dt_bias", dt_bias), ("D", D)):
        _want(t, n, torch.float32, (H,))
    _want(z, "z", _TORCH_DT[d.act_dtype], (Bd, d.d_inner), optional=True)
    _want(y, "y", _TORCH_DT[d.out_dtype], (Bd, d.d_inner))
    ns = _ssm_slots(d, ssm_pool)
    _want(state_indices, "state_indices", torch.int32, (Bd,))
    _debug_check(ns, state_indices)
    c = cdims(d, xbc_dtype)
    _check(lib().mamba2_state_update(ctypes.byref(c), _ptr(xbc), _ptr(dt_raw), _ptr(A_log), _ptr(dt_bias), _ptr(D),
                                     _ptr(z), _ptr(y), _ptr(ssm_pool), ns, _ptr(state_indices), Bd,
                                     _stream(stream)),
           "mamba2_state_update")


def mamba2_conv1d_update_multi(d: Dims, xbc, conv_w, conv_b, xbc_out, conv_pool, src_indices, dst_indices=None, *,
                               xbc_dtype=None, stream=None):
    """xbc [batch, T, Cdim] raw; xbc_out [batch, T, Cdim]; dst_indices [batch, T] int32 or None."""
    Bd, T = xbc.shape[0], xbc.shape[1]
    _want(xbc, "xbc", _TORCH_DT[d.act_dtype], (Bd, T, d.conv_dim))
    _want(conv_w, "conv_w", torch.float32, (d.conv_dim, d.conv_width))
    _want(conv_b, "conv_b", torch.float32, (d.conv_dim,), optional=True)
    _want(xbc_out, "xbc_out", _xdt(d, xbc_dtype), (Bd, T, d.conv_dim))
    ns = _conv_slots(d, conv_pool)
    _want(src_indices, "src_indices", torch.int32, (Bd,))
    _want(dst_indices, "dst_indices", torch.int32, (Bd, T), optional=True)
    _debug_check(ns, src_indices, dst_indices)
    _check(lib().mamba2_conv1d_update_multi(ctypes.byref(cdims(d, xbc_dtype)), _ptr(xbc), _ptr(conv_w), _ptr(conv_b),
                                            _ptr(xbc_out), _ptr(conv_pool), ns, _ptr(src_indices), _ptr(dst_indices),
                                            Bd, T, _stream(stream)), "mamba2_conv1d_update_multi")


def mamba2_state_update_multi(d: Dims, xbc, dt_raw, A_log, dt_bias, D, z, y, ssm_pool, src_indices, dst_indices=None,
                              *, xbc_dtype=None, stream=None):
    """xbc [batch, T, Cdim] post-conv; dt_raw [batch, T, H]; z/y [batch, T, H*P]; dst_indices [batch, T] or None."""
    Bd, T = xbc.shape[0], xbc.shape[1]
    H = d.nheads
    _want(xbc, "xbc", _xdt(d, xbc_dtype), (Bd, T, d.conv_dim))
    _want(dt_raw, "dt_raw", _TORCH_DT[d.act_dtype], (Bd, T, H))
    for n, t in (("A_log", A_log), ("dt_bias", dt_bias), ("D", D)):
        _want(t, n, torch.float32, (H,))
    _want(z, "z", _TORCH_DT[d.act_dtype], (Bd, T, d.d_inner), optional=True)
    _want(y, "y", _TORCH_DT[d.out_dtype], (Bd, T, d.d_inner))
    ns = _ssm_slots(d, ssm_pool)
    _want(src_indices, "src_indices", torch.int32, (Bd,))
    _want(dst_indices, "dst_indices", torch.int32, (Bd, T), optional=True)
    _debug_check(ns, src_indices, dst_indices)
    _check(lib().mamba2_state_update_multi(ctypes.byref(cdims(d, xbc_dtype)), _ptr(xbc), _ptr(dt_raw), _ptr(A_log),
                                           _ptr(dt_bias), _ptr(D), _ptr(z), _ptr(y), _ptr(ssm_pool), ns,
                                           _ptr(src_indices), _ptr(dst_indices), Bd, T, _stream(stream)),
           "mamba2_state_update_multi")


def mamba2_prefill_workspace_bytes(d: Dims, total_tokens: int, *, xbc_dtype=None) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().mamba2_prefill_workspace_bytes(ctypes.byref(cdims(d, xbc_dtype)), total_tokens, ctypes.byref(out)),
           "mamba2_prefill_workspace_bytes")
    return int(out.value)


def prefill_workspace(d: Dims, total_tokens: int, *, xbc_dtype=None, device="cuda") -> torch.Tensor:
    """A device byte buffer of the size mamba2_prefill_fwd needs (allocate once, reuse)."""
    n = mamba2_prefill_workspace_bytes(d, total_tokens, xbc_dtype=xbc_dtype)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def mamba2_prefill_fwd(d: Dims, xbc, dt_raw, z, conv_w, conv_b, A_log, dt_bias, D, y, ssm_pool, conv_pool,
                       cu_seqlens, state_indices, has_initial_state=None, workspace=None, norm_w=None,
                       norm_eps: float = 1e-5, norm_group: int = 0, *, xbc_dtype=None, stream=None):
    T = xbc.shape[0]
    nseq = state_indices.shape[0]
    H = d.nheads
    _want(xbc, "xbc", _TORCH_DT[d.act_dtype], (T, d.conv_dim))
    _want(dt_raw, "dt_raw", _TORCH_DT[d.act_dtype], (T, H))
    _want(z, "z", _TORCH_DT[d.act_dtype], (T, d.d_inner), optional=True)
    _want(conv_w, "conv_w", torch.float32, (d.conv_dim, d.conv_width))
    _want(conv_b, "conv_b", torch.float32, (d.conv_dim,), optional=True)
    for n, t in (("A_log", A_log), ("dt_bias", dt_bias), ("D", D)):
        _want(t, n, torch.float32, (H,))
    _want(norm_w, "norm_w", torch.float32, (d.d_inner,), optional=True)
    _want(y, "y", _TORCH_DT[d.out_dtype], (T, d.d_inner))
    ns = _both_slots(d, ssm_pool, conv_pool)
    _want(cu_seqlens, "cu_seqlens", torch.int32, (nseq + 1,))
    _want(state_indices, "state_indices", torch.int32, (nseq,))
    _want(has_initial_state, "has_initial_state", torch.uint8, (nseq,), optional=True)
    _want(workspace, "workspace", optional=True)
    _debug_check(ns, state_indices)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    c = cdims(d, xbc_dtype)
    _check(lib().mamba2_prefill_fwd(ctypes.byref(c), _ptr(xbc), _ptr(dt_raw), _ptr(z), _ptr(conv_w), _ptr(conv_b),
                                    _ptr(A_log), _ptr(dt_bias), _ptr(D), _ptr(norm_w), float(norm_eps),
                                    int(norm_group), _ptr(y), _ptr(ssm_pool), _ptr(conv_pool), ns, _ptr(cu_seqlens),
                                    nseq, T, _ptr(state_indices), _ptr(has_initial_state), _ptr(workspace), ws_bytes,
                                    _stream(stream)), "mamba2_prefill_fwd")


STATIC_SCRATCH_BYTES = 64 * 1024 * 1024  # MAMBA2_STATIC_SCRATCH_BYTES in include/mamba2.h


def mamba2_prefill_fwd_noalloc(d: Dims, xbc, dt_raw, z, conv_w, conv_b, A_log, dt_bias, D, y, ssm_pool, conv_pool,
                               cu_seqlens, state_indices, has_initial_state=None, norm_w=None, norm_eps: float = 1e-5,
                               norm_group: int = 0, *, xbc_dtype=None, stream=None):
    """mamba2_prefill_fwd without a workspace argument: the library's fixed per-GPU scratch array
    serves as the workspace (nothing is allocated; calls that overlap on one GPU race)."""
    T = xbc.shape[0]
    nseq = state_indices.shape[0]
    H = d.nheads
    _want(xbc, "xbc", _TORCH_DT[d.act_dtype], (T, d.conv_dim))
    _want(dt_raw, "dt_raw", _TORCH_DT[d.act_dtype], (T, H))
    _want(z, "z", _TORCH_DT[d.act_dtype], (T, d.d_inner), optional=True)
    _want(conv_w, "conv_w", torch.float32, (d.conv_dim, d.conv_width))
    _want(conv_b, "conv_b", torch.float32, (d.conv_dim,), optional=True)
    for n, t in (("A_log", A_log), ("dt_bias", dt_bias), ("D", D)):
        _want(t, n, torch.float32, (H,))
    _want(norm_w, "norm_w", torch.float32, (d.d_inner,), optional=True)
    _want(y, "y", _TORCH_DT[d.out_dtype], (T, d.d_inner))
    ns = _both_slots(d, ssm_pool, conv_pool)
    _want(cu_seqlens, "cu_seqlens", torch.int32, (nseq + 1,))
    _want(state_indices, "state_indices", torch.int32, (nseq,))
    _want(has_initial_state, "has_initial_state", torch.uint8, (nseq,), optional=True)
    _debug_check(ns, state_indices)
    c = cdims(d, xbc_dtype)
    _check(lib().mamba2_prefill_fwd_noalloc(ctypes.byref(c), _ptr(xbc), _ptr(dt_raw), _ptr(z), _ptr(conv_w),
                                            _ptr(conv_b), _ptr(A_log), _ptr(dt_bias), _ptr(D), _ptr(norm_w),
                                            float(norm_eps), int(norm_group), _ptr(y), _ptr(ssm_pool),
                                            _ptr(conv_pool), ns, _ptr(cu_seqlens), nseq, T, _ptr(state_indices),
                                            _ptr(has_initial_state), _stream(stream)), "mamba2_prefill_fwd_noalloc")


def mamba2_gated_rmsnorm(d: Dims, y, z, norm_w, out, eps: float = 1e-5, group_size: int = 0, *, stream=None):
    rows = y.shape[0]
    _want(y, "y", _TORCH_DT[d.out_dtype], (rows, d.d_inner))
    _want(z, "z", _TORCH_DT[d.act_dtype], (rows, d.d_inner), optional=True)
    _want(norm_w, "norm_w", torch.float32, (d.d_inner,))
    _want(out, "out", _TORCH_DT[d.out_dtype], (rows, d.d_inner))
    _check(lib().mamba2_gated_rmsnorm(ctypes.byref(cdims(d)), _ptr(y), _ptr(z), _ptr(norm_w), float(eps),
                                      int(group_size), _ptr(out), rows, _stream(stream)), "mamba2_gated_rmsnorm")


def mamba1_ssm_slot_bytes(d) -> int:
    return int(lib().mamba1_ssm_slot_bytes(ctypes.byref(cdims1(d))))


def mamba1_selective_scan_fwd(d, u, delta_raw, A, B, C, D, z, delta_bias, y, ssm_pool, cu_seqlens, state_indices,
                              has_initial_state=None, delta_softplus: bool = True, *, stream=None):
    """Mamba-1 selective scan over packed sequences. ``d`` is a Mamba1Dims.
    u, delta_raw, z, y [T, dim]; B, C [T, ngroups, dstate]; A [dim, dstate]; ssm_pool [slots, dim, dstate]."""
    T = u.shape[0]
    nseq = state_indices.shape[0]
    act = _TORCH_DT[d.act_dtype]
    _want(u, "u", act, (T, d.dim))
    _want(delta_raw, "delta_raw", act, (T, d.dim))
    _want(A, "A", torch.float32, (d.dim, d.dstate))
    _want(B, "B", act, (T, d.ngroups, d.dstate))
    _want(C, "C", act, (T, d.ngroups, d.dstate))
    _want(D, "D", torch.float32, (d.dim,), optional=True)
    _want(z, "z", act, (T, d.dim), optional=True)
    _want(delta_bias, "delta_bias", torch.float32, (d.dim,), optional=True)
    _want(y, "y", _TORCH_DT[d.out_dtype], (T, d.dim))
    _want(ssm_pool, "ssm_pool", _TORCH_DT[d.state_dtype])
    if ssm_pool.dim() != 3 or tuple(ssm_pool.shape[1:]) != (d.dim, d.dstate):
        raise ValueError("ssm_pool must be [slots, dim, dstate]")
    ns = int(ssm_pool.shape[0])
    _want(cu_seqlens, "cu_seqlens", torch.int32, (nseq + 1,))
    _want(state_indices, "state_indices", torch.int32, (nseq,))
    _want(has_initial_state, "has_initial_state", torch.uint8, (nseq,), optional=True)
    _debug_check(ns, state_indices)
    _check(lib().mamba1_selective_scan_fwd(ctypes.byref(cdims1(d)), _ptr(u), _ptr(delta_raw), _ptr(A), _ptr(B), _ptr(C),
                                           _ptr(D), _ptr(z), _ptr(delta_bias), 1 if delta_softplus else 0, _ptr(y),
                                           _ptr(ssm_pool), ns, _ptr(cu_seqlens), nseq, T, _ptr(state_indices),
                                           _ptr(has_initial_state), _stream(stream)), "mamba1_selective_scan_fwd")


def mamba1_selective_state_update(d, u, delta_raw, A, B, C, D, z, delta_bias, y, ssm_pool, state_indices,
                                  delta_softplus: bool = True, *, stream=None):
    """One token per row of the Mamba-1 selective scan, in place at the slots.
    u, delta_raw, z, y [batch, dim]; B, C [batch, ngroups, dstate]; ssm_pool [slots, dim, dstate]."""
    Bd = state_indices.shape[0]
    act = _TORCH_DT[d.act_dtype]
    _want(u, "u", act, (Bd, d.dim))
    _want(delta_raw, "delta_raw", act, (Bd, d.dim))
    _want(A, "A", torch.float32, (d.dim, d.dstate))
    _want(B, "B", act, (Bd, d.ngroups, d.dstate))
    _want(C, "C", act, (Bd, d.ngroups, d.dstate))
    _want(D, "D", torch.float32, (d.dim,), optional=True)
    _want(z, "z", act, (Bd, d.dim), optional=True)
    _want(delta_bias, "delta_bias", torch.float32, (d.dim,), optional=True)
    _want(y, "y", _TORCH_DT[d.out_dtype], (Bd, d.dim))
    _want(ssm_pool, "ssm_pool", _TORCH_DT[d.state_dtype])
    if ssm_pool.dim() != 3 or tuple(ssm_pool.shape[1:]) != (d.dim, d.dstate):
        raise ValueError("ssm_pool must be [slots, dim, dstate]")
    ns = int(ssm_pool.shape[0])
    _want(state_indices, "state_indices", torch.int32, (Bd,))
    _debug_check(ns, state_indices)
    _check(lib().mamba1_selective_state_update(ctypes.byref(cdims1(d)), _ptr(u), _ptr(delta_raw), _ptr(A), _ptr(B),
                                               _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
                                               1 if delta_softplus else 0, _ptr(y), _ptr(ssm_pool), ns,
                                               _ptr(state_indices), Bd, _stream(stream)),
           "mamba1_selective_state_update")


def mamba2_mixed_fwd(d: Dims, xbc, dt_raw, z, conv_w, conv_b, A_log, dt_bias, D, xbc_post, y, ssm_pool, conv_pool,
                     cu_seqlens, prefill_indices, has_initial_state, decode_indices, workspace=None, *,
                     xbc_dtype=None, stream=None):
    nseq = prefill_indices.shape[0]
    Bd = decode_indices.shape[0]
    rows = xbc.shape[0]
    T = rows - Bd
    H = d.nheads
    _want(xbc, "xbc", _TORCH_DT[d.act_dtype], (rows, d.conv_dim))
    _want(dt_raw, "dt_raw", _TORCH_DT[d.act_dtype], (rows, H))
    _want(z, "z", _TORCH_DT[d.act_dtype], (rows, d.d_inner), optional=True)
    _want(conv_w, "conv_w", torch.float32, (d.conv_dim, d.conv_width))
    _want(conv_b, "conv_b", torch.float32, (d.conv_dim,), optional=True)
    for n, t in (("A_log", A_log), ("dt_bias", dt_bias), ("D", D)):
        _want(t, n, torch.float32, (H,))
    _want(xbc_post, "xbc_post", _xdt(d, xbc_dtype), (rows, d.conv_dim))
    _want(y, "y", _TORCH_DT[d.out_dtype], (rows, d.d_inner))
    ns = _both_slots(d, ssm_pool, conv_pool)
    _want(cu_seqlens, "cu_seqlens", torch.int32, (nseq + 1,))
    _want(prefill_indices, "prefill_indices", torch.int32, (nseq,))
    _want(has_initial_state, "has_initial_state", torch.uint8, (nseq,), optional=True)
    _want(decode_indices, "decode_indices", torch.int32, (Bd,))
    _debug_check(ns, prefill_indices, decode_indices)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    c = cdims(d, xbc_dtype)
    _check(lib().mamba2_mixed_fwd(ctypes.byref(c), _ptr(xbc), _ptr(dt_raw), _ptr(z), _ptr(conv_w), _ptr(conv_b),
                                  _ptr(A_log), _ptr(dt_bias), _ptr(D), _ptr(xbc_post), _ptr(y), _ptr(ssm_pool),
                                  _ptr(conv_pool), ns, _ptr(cu_seqlens), nseq, T, _ptr(prefill_indices),
                                  _ptr(has_initial_state), _ptr(decode_indices), Bd, _ptr(workspace), ws_bytes,
                                  _stream(stream)), "mamba2_mixed_fwd")


# ------------------------------------------------------------------ captured decode step

class CDecodeLayer(ctypes.Structure):
    _fields_ = [("xbc", _P), ("conv_w", _P), ("conv_b", _P), ("xbc_post", _P), ("conv_pool", _P), ("dt_raw", _P),
                ("A_log", _P), ("dt_bias", _P), ("D", _P), ("z", _P), ("y", _P), ("ssm_pool", _P),
                ("num_slots", _I32), ("state_indices", _P)]


class DecodeGraph:
    """mamba2_decode_graph_*: the one-token decode (conv1d_update + state_update) of a list of
    layer entries, captured once as a HIP graph and replayed with one launch.

    Each entry is a dict with the tensors of one layer at one step: xbc [batch, Cdim] raw,
    conv_w, conv_b (or None), xbc_post [batch, Cdim], conv_pool, dt_raw [batch, H], A_log,
    dt_bias, D, z (or None), y [batch, H*P], ssm_pool, state_indices [batch]. The graph keeps
    their addresses (and this object keeps the tensors alive): refill them in place between
    launches."""

    def __init__(self, d: Dims, layers, *, xbc_dtype=None):
        H = d.nheads
        self._keep = [dict(L) for L in layers]
        if not self._keep:
            raise ValueError("no layers")
        batch = int(self._keep[0]["state_indices"].shape[0])
        arr = (CDecodeLayer * len(self._keep))()
        for i, L in enumerate(self._keep):
            _want(L["xbc"], "xbc", _TORCH_DT[d.act_dtype], (batch, d.conv_dim))
            _want(L["conv_w"], "conv_w", torch.float32, (d.conv_dim, d.conv_width))
            _want(L.get("conv_b"), "conv_b", torch.float32, (d.conv_dim,), optional=True)
            _want(L["xbc_post"], "xbc_post", _xdt(d, xbc_dtype), (batch, d.conv_dim))
            _want(L["dt_raw"], "dt_raw", _TORCH_DT[d.act_dtype], (batch, H))
            for n in ("A_log", "dt_bias", "D"):
                _want(L[n], n, torch.float32, (H,))
            _want(L.get("z"), "z", _TORCH_DT[d.act_dtype], (batch, d.d_inner), optional=True)
            _want(L["y"], "y", _TORCH_DT[d.out_dtype], (batch, d.d_inner))
            ns = _both_slots(d, L["ssm_pool"], L["conv_pool"])
            _want(L["state_indices"], "state_indices", torch.int32, (batch,))
            arr[i] = CDecodeLayer(*(_ptr(L.get(k)) for k in ("xbc", "conv_w", "conv_b", "xbc_post", "conv_pool",
                                                              "dt_raw", "A_log", "dt_bias", "D", "z", "y",
                                                              "ssm_pool")),
                                  ns, _ptr(L["state_indices"]))
        self._h = ctypes.c_void_p()
        cap = torch.cuda.Stream()
        st = lib().mamba2_decode_graph_create(ctypes.byref(cdims(d, xbc_dtype)), ctypes.cast(arr, _P),
                                              len(self._keep), batch, ctypes.c_void_p(cap.cuda_stream),
                                              ctypes.byref(self._h))
        if st != OK:
            raise Mamba2Error(st, "mamba2_decode_graph_create",
                              (lib().mamba2_decode_graph_last_error() or lib().mamba2_last_error()).decode())
        self.batch = batch
        self.layers = len(self._keep)

    def launch(self, *, stream=None) -> None:
        st = lib().mamba2_decode_graph_launch(self._h, _stream(stream))
        if st != OK:
            raise Mamba2Error(st, "mamba2_decode_graph_launch", lib().mamba2_decode_graph_last_error().decode())

    def close(self):
        if getattr(self, "_h", None):
            lib().mamba2_decode_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------------ slot index safety

def mamba2_read_slot_errors(reset: bool = False, *, stream=None) -> int:
    """How many times kernels on the current device skipped a row or sequence whose slot
    index was >= its pool's slot count (since the last reset). Waits for the stream."""
    out = torch.empty(4, dtype=torch.int32, device="cuda")
    _check(lib().mamba2_read_slot_errors(_ptr(out), 1 if reset else 0, _stream(stream)), "mamba2_read_slot_errors")
    return int(out[0].item())


def check_slot_indices(indices, num_slots: int, *, stream=None):
    """Debug check of one int32 index table on the device: returns (entries >= num_slots,
    entries in [0, num_slots) that repeat an earlier one). Waits for the stream."""
    _want(indices, "indices", torch.int32)
    res = torch.empty(2, dtype=torch.int32, device=indices.device)
    _check(lib().mamba2_check_slot_indices(_ptr(indices), int(indices.numel()), int(num_slots), _ptr(res),
                                           _stream(stream)), "mamba2_check_slot_indices")
    r = res.cpu()
    return int(r[0]), int(r[1])


# ------------------------------------------------------------------ slot allocator

class SlotAllocator:
    """Host-side O(1) free list of pool slots (``mamba2_slots_*``)."""

    def __init__(self, num_slots: int):
        h = ctypes.c_void_p()
        _check(lib().mamba2_slots_create(num_slots, ctypes.byref(h)), "mamba2_slots_create")
        self._h = h
        self.num_slots = num_slots

    def alloc(self) -> int:
        s = ctypes.c_int32(-1)
        _check(lib().mamba2_slot_alloc(self._h, ctypes.byref(s)), "mamba2_slot_alloc")
        return int(s.value)

    def free(self, slot: int) -> None:
        _check(lib().mamba2_slot_free(self._h, slot), "mamba2_slot_free")

    @property
    def in_use(self) -> int:
        return int(lib().mamba2_slots_in_use(self._h))

    def close(self):
        if self._h:
            lib().mamba2_slots_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
