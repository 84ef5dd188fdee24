"""C-ABI checks that need no GPU: the library loads, exports every declared symbol,
sizes match the pages' arithmetic, invalid arguments are rejected before any HIP
call, the slot allocator works, and the library links no allocator or memset."""
import ctypes
import json
import os
import subprocess

import pytest

from state_space_model_ssm_amd import binding as B
from state_space_model_ssm_amd.configs import BF16, F32, NEMOTRON_H_8B, NEMOTRON_H_8B_MAMBA_LAYERS, TINY, Dims

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from state_space_model_ssm_amd import build
        build.build()
    return B.lib()


def test_every_declared_symbol_is_exported(lib):
    names = B.header_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    assert set(names) <= exported


def test_library_links_no_allocator_or_memset(lib):
    """Decode and scan entry points never allocate or clear device memory (the vllm.cpp issue's
    cost table: 0 alloc/free, 0 memset per layer per token)."""
    out = subprocess.run(["nm", "-D", "--undefined-only", B.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    bad = [ln for ln in out.splitlines() if any(k in ln for k in ("hipMalloc", "hipFree", "hipMemset",
                                                                   "hipDeviceSynchronize", "hipStreamSynchronize"))]
    assert not bad, bad


def test_slot_sizes_match_page_arithmetic(lib):
    g = json.load(open(os.path.join(GOLDEN, "page_sizes.json")))
    d = Dims(g["nheads"], g["headdim"], g["dstate"], g["ngroups"], state_dtype=BF16)
    assert B.mamba2_ssm_slot_bytes(d) == g["ssm_bytes_per_layer_per_seq"]
    assert B.mamba2_ssm_slot_bytes(d) * NEMOTRON_H_8B_MAMBA_LAYERS == g["ssm_bytes_per_seq"]
    assert NEMOTRON_H_8B_MAMBA_LAYERS == g["mamba_layers"]
    assert B.mamba2_ssm_slot_bytes(d.with_(state_dtype=F32)) == 2 * g["ssm_bytes_per_layer_per_seq"]
    assert B.mamba2_conv_slot_bytes(d) == 3 * (128 * 64 + 2 * 8 * 128) * 2
    # the chunk scan's optional workspace: the prefill's B/C planes for P=64, N=128, bf16 act/y; none elsewhere
    assert (B.mamba2_chunk_scan_workspace_bytes(NEMOTRON_H_8B, 32768, 4)
            == B.mamba2_prefill_workspace_bytes(NEMOTRON_H_8B.with_(state_dtype=F32), 32768))
    assert (B.mamba2_chunk_scan_workspace_bytes(NEMOTRON_H_8B, 1000, 3)
            == B.mamba2_prefill_workspace_bytes(NEMOTRON_H_8B.with_(state_dtype=F32), 1000))
    assert B.mamba2_chunk_scan_workspace_bytes(NEMOTRON_H_8B.with_(out_dtype=F32), 32768, 4) == 0
    assert B.mamba2_chunk_scan_workspace_bytes(NEMOTRON_H_8B.with_(act_dtype=F32), 32768, 4) == 0
    assert B.mamba2_chunk_scan_workspace_bytes(TINY, 64, 1) == 0


def test_check_dims(lib):
    B.mamba2_check_dims(NEMOTRON_H_8B)
    B.mamba2_check_dims(TINY)
    with pytest.raises(B.Mamba2Error) as e:
        B.mamba2_check_dims(NEMOTRON_H_8B.with_(ngroups=3))
    assert e.value.status == B.ERR_INVALID_ARG
    with pytest.raises(B.Mamba2Error) as e:
        B.mamba2_check_dims(NEMOTRON_H_8B.with_(chunk_size=256))
    assert e.value.status == B.ERR_UNSUPPORTED
    with pytest.raises(B.Mamba2Error) as e:
        B.mamba2_check_dims(NEMOTRON_H_8B.with_(dstate=48))
    assert e.value.status == B.ERR_UNSUPPORTED
    # the update kernels address rows and state tiles by 32-bit byte offsets: Cdim up to 2^24
    with pytest.raises(B.Mamba2Error) as e:
        B.mamba2_check_dims(NEMOTRON_H_8B.with_(nheads=1 << 18, ngroups=8))
    assert e.value.status == B.ERR_UNSUPPORTED and "2^24" in str(e.value)


def _cd(d=NEMOTRON_H_8B):
    return ctypes.byref(B.cdims(d))


def test_invalid_arguments_rejected_without_gpu(lib):
    P = ctypes.c_void_p
    good = P(0x10000)
    mis = P(0x10004)
    # NULL required pointer
    st = lib.mamba2_state_update(_cd(), None, good, good, good, good, None, good, good, 8, good, 4, None)
    assert st == B.ERR_INVALID_ARG and b"xbc" in lib.mamba2_last_error()
    # misaligned pointer
    st = lib.mamba2_state_update(_cd(), mis, good, good, good, good, None, good, good, 8, good, 4, None)
    assert st == B.ERR_INVALID_ARG and b"aligned" in lib.mamba2_last_error()
    # negative batch
    st = lib.mamba2_state_update(_cd(), good, good, good, good, good, None, good, good, 8, good, -1, None)
    assert st == B.ERR_INVALID_ARG
    # negative pool slot count
    st = lib.mamba2_state_update(_cd(), good, good, good, good, good, None, good, good, -1, good, 4, None)
    assert st == B.ERR_INVALID_ARG and b"num_slots" in lib.mamba2_last_error()
    st = lib.mamba2_conv1d_update(_cd(), good, good, None, good, good, -3, good, 2, None)
    assert st == B.ERR_INVALID_ARG and b"num_slots" in lib.mamba2_last_error()
    # zero rows: valid, nothing enqueued
    assert lib.mamba2_state_update(_cd(), None, None, None, None, None, None, None, None, 0, None, 0, None) == B.OK
    assert lib.mamba2_conv1d_update(_cd(), None, None, None, None, None, 0, None, 0, None) == B.OK
    assert lib.mamba2_conv1d_fwd(_cd(), None, None, None, None, None, 0, None, 0, 0, None, None, None) == B.OK
    # aliasing conv output
    st = lib.mamba2_conv1d_update(_cd(), good, good, None, good, good, 8, good, 2, None)
    assert st == B.ERR_INVALID_ARG and b"alias" in lib.mamba2_last_error()
    # tokens without sequences
    st = lib.mamba2_chunk_scan_fwd(_cd(), good, good, good, good, good, None, good, good, 8, good, 0, 5, good, None,
                                   None, 0, None)
    assert st == B.ERR_INVALID_ARG
    # more packed tokens than int32 cu_seqlens can describe
    st = lib.mamba2_chunk_scan_fwd(_cd(), good, good, good, good, good, None, good, good, 8, good, 1, 2 ** 31, good,
                                   None, None, 0, None)
    assert st == B.ERR_INVALID_ARG and b"int32" in lib.mamba2_last_error()
    st = lib.mamba2_conv1d_fwd(_cd(), good, good, None, good, good, 8, good, 1, 2 ** 31, good, None, None)
    assert st == B.ERR_INVALID_ARG and b"int32" in lib.mamba2_last_error()
    # a multi-token row past the 32-bit byte offsets of its tokens (T x Cdim x 4 >= 2^32)
    st = lib.mamba2_state_update_multi(_cd(), good, good, good, good, good, None, good, good, 8, good, None, 1,
                                       2 ** 17, None)
    assert st == B.ERR_UNSUPPORTED and b"2^32" in lib.mamba2_last_error()
    # a workspace smaller than the block form needs
    st = lib.mamba2_chunk_scan_fwd(_cd(), good, good, good, good, good, None, good, good, 8, good, 1, 64, good, None,
                                   good, 1024, None)
    assert st == B.ERR_WORKSPACE and b"workspace" in lib.mamba2_last_error()
    # unsupported chunk
    st = lib.mamba2_chunk_scan_fwd(_cd(NEMOTRON_H_8B.with_(chunk_size=96)), good, good, good, good, good, None, good,
                                   good, 8, good, 1, 5, good, None, None, 0, None)
    assert st == B.ERR_UNSUPPORTED
    # the slot checks reject bad arguments before any launch
    assert lib.mamba2_check_slot_indices(good, -1, 4, good, None) == B.ERR_INVALID_ARG
    assert lib.mamba2_check_slot_indices(good, 3, 4, None, None) == B.ERR_INVALID_ARG
    assert lib.mamba2_read_slot_errors(None, 0, None) == B.ERR_INVALID_ARG
    assert lib.mamba2_status_string(B.ERR_UNSUPPORTED) == b"unsupported dims or dtype"


def test_slot_allocator(lib):
    a = B.SlotAllocator(3)
    got = [a.alloc(), a.alloc(), a.alloc()]
    assert sorted(got) == [0, 1, 2] and a.in_use == 3
    with pytest.raises(B.Mamba2Error) as e:
        a.alloc()
    assert e.value.status == B.ERR_NO_SLOT
    a.free(1)
    assert a.in_use == 2 and a.alloc() == 1
    with pytest.raises(B.Mamba2Error):
        a.free(7)
    a.free(2)
    with pytest.raises(B.Mamba2Error):
        a.free(2)  # double free
    a.close()


def test_binding_rejects_host_tensors(lib):
    import torch
    d = TINY
    x = torch.zeros(2, d.conv_dim)
    with pytest.raises(ValueError, match="device tensor"):
        B.mamba2_conv1d_update(d, x, torch.zeros(d.conv_dim, 4), None, x.clone(), torch.zeros(4, 3, d.conv_dim),
                               torch.zeros(2, dtype=torch.int32))


def test_binding_checks_pool_shapes(lib):
    """The binding derives num_slots from the pools and refuses pools of the wrong shape
    (a pool that is not [slots, H, P, N] / [slots, W-1, Cdim] would let an index address
    memory outside it)."""
    import torch
    d = TINY
    with pytest.raises(ValueError, match="ssm_pool must be"):
        B._ssm_slots(d, torch.zeros(4, d.nheads * d.headdim, d.dstate))
    with pytest.raises(ValueError, match="conv_pool must be"):
        B._conv_slots(d, torch.zeros(4, d.conv_width, d.conv_dim))
    with pytest.raises(ValueError, match="device tensor"):  # right shape, but host memory
        B._ssm_slots(d, torch.zeros(5, d.nheads, d.headdim, d.dstate))


def test_prefill_workspace_and_validation_without_gpu(lib):
    """Workspace sizing of the fused prefill (B/C operand planes per 32-token block) and of the
    unfused composition (post-conv xBC), and the errors raised before any launch."""
    P = ctypes.c_void_p
    good = P(0x10000)
    d8 = NEMOTRON_H_8B.with_(state_dtype=F32)  # bf16 y: fused shape
    # C, B^T hi/lo (bf16) and C.B^T (fp32 per 32-token block), each region padded to 256 bytes; from
    # 2048 tokens also the small-batch mode's segment records, decays, local states (at most 512 / H
    # segments: 16 MiB of fp32 states at P = 64, N = 128), per-block decays and bf16 initial states
    pad = lambda v: -(-v // 256) * 256
    seg = lambda nv, H, nblk: (pad(nv * 16) + pad(nv * H * 4) + pad(nv * H * 64 * 128 * 4) + pad(nblk * H * 4)
                               + pad(nv * H * 64 * 128 * 2))
    assert (B.mamba2_prefill_workspace_bytes(d8, 32768)
            == 32768 * (3 * 8 * 128 * 2 + 8 * 32 * 4) + seg(4, 128, 1024))
    assert B.mamba2_prefill_workspace_bytes(d8, 2047) == (pad(2047 * 8 * 128 * 2) + pad(64 * 8 * 2 * 128 * 32 * 2)
                                                          + pad(64 * 8 * 32 * 32 * 4))
    assert B.mamba2_prefill_workspace_bytes(d8, 33) == (pad(33 * 8 * 128 * 2) + pad(2 * 8 * 2 * 128 * 32 * 2)
                                                        + pad(2 * 8 * 32 * 32 * 4))
    d8f = d8.with_(out_dtype=F32)  # fp32 y: conv1d_fwd + chunk_scan_fwd through the workspace
    assert B.mamba2_prefill_workspace_bytes(d8f, 100) == 100 * d8f.conv_dim * 4
    assert B.mamba2_prefill_workspace_bytes(TINY, 64) == 64 * TINY.conv_dim * 4
    args = lambda ws, nbytes, norm=None, group=0: (_cd(d8), good, good, None, good, None, good, good, good, norm,
                                                   ctypes.c_float(1e-5), group, good, good, good, 8, good, 1, 64,
                                                   good, None, ws, nbytes, None)
    need = B.mamba2_prefill_workspace_bytes(d8, 64)
    st = lib.mamba2_prefill_fwd(*args(good, need - 16))
    assert st == B.ERR_WORKSPACE and b"workspace" in lib.mamba2_last_error()
    st = lib.mamba2_prefill_fwd(*args(None, need))
    assert st == B.ERR_INVALID_ARG and b"workspace" in lib.mamba2_last_error()
    st = lib.mamba2_prefill_fwd(*args(good, need, norm=good, group=100))
    assert st == B.ERR_UNSUPPORTED
    st = lib.mamba2_gated_rmsnorm(_cd(d8), good, None, good, ctypes.c_float(1e-5), 12, good, 4, None)
    assert st == B.ERR_UNSUPPORTED  # 12 does not divide H*P = 8192
    st = lib.mamba2_gated_rmsnorm(_cd(d8), good, good, good, ctypes.c_float(1e-5), 0, good, 4, None)
    assert st == B.ERR_INVALID_ARG and b"alias" in lib.mamba2_last_error()
    assert lib.mamba2_gated_rmsnorm(_cd(d8), None, None, None, ctypes.c_float(1e-5), 0, None, 0, None) == B.OK
