"""Mamba-2 SSM core on MI355X (gfx950): conv1d + chunked SSD scan + in-place decode state update.

The compute lives in ``libmamba2.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/mamba2.h``); ``binding`` exposes the same entry points on
torch tensors. Import of this package does not load the library; the first
call does, and raises if it has not been built.
"""
from .configs import BF16, F32, NEMOTRON_H_8B, NEMOTRON_H_8B_MAMBA_LAYERS, TINY, WORKLOADS, Dims  # noqa: F401
from .binding import (  # noqa: F401
    Mamba2Error, SlotAllocator, mamba2_check_dims, mamba2_chunk_scan_fwd, mamba2_chunk_scan_workspace_bytes,
    mamba2_conv1d_fwd, mamba2_conv1d_update, mamba2_conv_slot_bytes, mamba2_mixed_fwd, mamba2_ssm_slot_bytes,
    mamba2_state_update,
)
