"""mamba2_prefill_fwd_noalloc (the prefill for callers that cannot allocate: its workspace is
the library's fixed per-GPU scratch array) against mamba2_prefill_fwd with a caller workspace:
two calls in a row, the second smaller than the first, each equal to the existing entry point's
result (the same kernels on the same inputs, so bit for bit, hence within the oracle
tolerances too); a batch whose workspace exceeds the array is refused before any launch."""
import numpy as np
import pytest
import torch

from _helpers import dev, dev_i32, dev_u8, params_dev
from state_space_model_ssm_amd import binding as B
from state_space_model_ssm_amd import synth
from state_space_model_ssm_amd.configs import F32, NEMOTRON_H_8B

pytestmark = pytest.mark.gpu

D8 = NEMOTRON_H_8B.with_(state_dtype=F32)  # bf16 inputs and y, fp32 state: the fused prefill


def run_both(w, has_init):
    d = D8
    T = int(w["cu_seqlens"][-1])
    assert B.mamba2_prefill_workspace_bytes(d, T) <= B.STATIC_SCRATCH_BYTES
    pd = params_dev(w["params"])
    xbc, dt = dev(w["xbc"], d.act_dtype), dev(w["dt_raw"], d.act_dtype)
    z = dev(w["z"], d.act_dtype) if w["z"] is not None else None
    cu, idx, hi = dev_i32(w["cu_seqlens"]), dev_i32(w["slots"]), dev_u8(has_init)
    out = []
    for noalloc in (False, True):
        ssm, conv = dev(w["ssm_pool"], d.state_dtype), dev(w["conv_pool"], d.state_dtype)
        y = torch.full((T, d.d_inner), 3.0, dtype=torch.bfloat16, device="cuda")
        if noalloc:
            B.mamba2_prefill_fwd_noalloc(d, xbc, dt, z, pd["conv_w"], None, pd["A_log"], pd["dt_bias"], pd["D"], y,
                                         ssm, conv, cu, idx, hi)
        else:
            ws = B.prefill_workspace(d, T)
            B.mamba2_prefill_fwd(d, xbc, dt, z, pd["conv_w"], None, pd["A_log"], pd["dt_bias"], pd["D"], y, ssm,
                                 conv, cu, idx, hi, ws)
        torch.cuda.synchronize()
        out.append((y, ssm, conv))
    (y0, s0, c0), (y1, s1, c1) = out
    assert torch.equal(y1, y0), "y differs from mamba2_prefill_fwd"
    assert torch.equal(s1, s0), "SSM pool differs from mamba2_prefill_fwd"
    assert torch.equal(c1, c0), "conv pool differs from mamba2_prefill_fwd"


def test_noalloc_prefill_two_calls_second_smaller():
    # first: 3 varlen sequences at full head count (4,300 tokens), z gate, resumed and fresh
    w = synth.prefill_batch(D8, seed=61, seqlens=[1500, 700, 2100], num_slots=6, initial_state=True)
    run_both(w, np.array([1, 0, 1], np.uint8))
    # second, smaller: 2 short sequences; the array still holds the first call's planes
    w = synth.prefill_batch(D8, seed=62, seqlens=[300, 45], num_slots=3, initial_state=True)
    run_both(w, np.array([0, 1], np.uint8))


def test_noalloc_prefill_segment_mode():
    """One 4,096-token sequence: few sequences, so the segment mode's records, local states and
    decays also live in the scratch array."""
    w = synth.prefill_batch(D8, seed=63, seqlens=[4096], num_slots=2, with_z=False, initial_state=True)
    run_both(w, np.array([1], np.uint8))


def test_noalloc_prefill_refuses_batches_beyond_the_array():
    d = D8
    T = 16384
    assert B.mamba2_prefill_workspace_bytes(d, T) > B.STATIC_SCRATCH_BYTES
    w = synth.prefill_batch(d, seed=64, seqlens=[T], num_slots=1, with_z=False)
    pd = params_dev(w["params"])
    ssm, conv = dev(w["ssm_pool"], d.state_dtype), dev(w["conv_pool"], d.state_dtype)
    y = torch.empty(T, d.d_inner, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.Mamba2Error) as e:
        B.mamba2_prefill_fwd_noalloc(d, dev(w["xbc"], d.act_dtype), dev(w["dt_raw"], d.act_dtype), None, pd["conv_w"],
                                     None, pd["A_log"], pd["dt_bias"], pd["D"], y, ssm, conv,
                                     dev_i32(w["cu_seqlens"]), dev_i32(w["slots"]))
    assert e.value.status == B.ERR_WORKSPACE and "static scratch" in str(e.value)
