"""GPU parity of the prefill path (conv1d_fwd + chunk_scan_fwd), the equivalence
contract (chunk scan == repeated single steps) and mixed batches, against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from _helpers import (assert_close, by_head, by_slot_head, compact_pools, dev, dev_i32, dev_u8, host,
                      oracle_kw, params_dev)
from state_space_model_ssm_amd import binding as B
from state_space_model_ssm_amd import synth
from state_space_model_ssm_amd.configs import BF16, F32, NEMOTRON_H_8B, TINY

pytestmark = pytest.mark.gpu

# Nemotron-H-8B head shape (P=64, N=128) with fewer heads so the oracle stays fast.
D16 = NEMOTRON_H_8B.with_(nheads=16, ngroups=2, chunk_size=64, state_dtype=F32, out_dtype=F32)


def scan_workspace(d, T, nseq):
    """Workspace for chunk_scan_fwd's 32-token-block form (None where the shape has none)."""
    n = B.mamba2_chunk_scan_workspace_bytes(d, T, nseq)
    return torch.empty(n, dtype=torch.uint8, device="cuda") if n > 0 else None


def run_prefill(d, w, has_init=None, slots=None, ws=False):
    pd = params_dev(w["params"])
    T = w["xbc"].shape[0]
    slots = w["slots"] if slots is None else slots
    has_init = w["has_initial_state"] if has_init is None else has_init
    ssm = dev(w["ssm_pool"], d.state_dtype)
    conv = dev(w["conv_pool"], d.state_dtype)
    xbc, dt = dev(w["xbc"], d.act_dtype), dev(w["dt_raw"], d.act_dtype)
    z = None if w["z"] is None else dev(w["z"], d.act_dtype)
    post = torch.empty(T, d.conv_dim, dtype=B._TORCH_DT[d.post_dtype], device="cuda")
    y = torch.empty(T, d.d_inner, dtype=B._TORCH_DT[d.out_dtype], device="cuda")
    cu, idx, hi = dev_i32(w["cu_seqlens"]), dev_i32(slots), dev_u8(has_init)
    B.mamba2_conv1d_fwd(d, xbc, pd["conv_w"], pd["conv_b"], post, conv, cu, idx, hi)
    wsp = scan_workspace(d, T, len(slots)) if ws else None
    B.mamba2_chunk_scan_fwd(d, post, dt, pd["A_log"], pd["dt_bias"], pd["D"], z, y, ssm, cu, idx, hi, wsp)
    torch.cuda.synchronize()
    return y, post, ssm, conv


def oracle_prefill(d, w, has_init=None, slots=None):
    slots = w["slots"] if slots is None else slots
    has_init = w["has_initial_state"] if has_init is None else has_init
    used = [s for s in slots if s >= 0]
    cp, sp = compact_pools(w, used)
    pos = {int(s): i for i, s in enumerate(used)}
    cidx = np.array([pos[int(s)] if s >= 0 else -1 for s in slots])
    y, post = oracle.prefill(w["xbc"], w["dt_raw"], w["params"], w["cu_seqlens"], cidx, has_init, cp, sp, z=w["z"],
                             **oracle_kw(d))
    return y, post, cp, sp, used


def check_prefill(d, w, has_init=None, slots=None, ws=False):
    y, post, ssm, conv = run_prefill(d, w, has_init, slots, ws)
    y_ref, post_ref, cp, sp, used = oracle_prefill(d, w, has_init, slots)
    e_post = assert_close(host(post), post_ref, d.post_dtype, "post-conv xBC")
    e_y = assert_close(host(y), y_ref, d.out_dtype, "y", slices=lambda a: by_head(a, d.nheads))
    u = torch.tensor(used, dtype=torch.long, device="cuda")
    e_h = assert_close(host(ssm[u]), sp, d.state_dtype, "final ssm state", slices=by_slot_head)
    assert np.array_equal(host(conv[u]), cp), "conv cache must hold the exact raw inputs"
    return y, ssm, conv, (e_post, e_y, e_h)


def test_tiny_prefill_then_decode():
    """Tiny fp32 layer: 64-token prefill (chunk 16) then 8 single-token steps."""
    d = TINY
    w = synth.tiny(d, seed=0)
    pre = {**w["prefill"], "params": w["params"], "slots": w["slots"], "cu_seqlens": w["cu_seqlens"],
           "has_initial_state": w["has_initial_state"], "ssm_pool": w["ssm_pool"], "conv_pool": w["conv_pool"]}
    y, post, ssm, conv = run_prefill(d, pre)
    cp, sp = compact_pools(w, w["slots"])
    cp[:] = 0.0
    sp[:] = 0.0
    kw = oracle_kw(d)
    y_ref, _ = oracle.prefill(pre["xbc"], pre["dt_raw"], w["params"], w["cu_seqlens"], [0], None, cp, sp,
                              z=pre["z"], **kw)
    assert_close(host(y), y_ref, F32, "prefill y")
    slot = int(w["slots"][0])
    assert_close(host(ssm[slot:slot + 1]), sp, F32, "state after prefill")
    pd = params_dev(w["params"])
    idx = dev_i32(w["slots"])
    for step in w["decode"]:
        xb, dt, z = dev(step["xbc"], F32), dev(step["dt_raw"], F32), dev(step["z"], F32)
        post1 = torch.empty(1, d.conv_dim, device="cuda")
        y1 = torch.empty(1, d.d_inner, device="cuda")
        B.mamba2_conv1d_update(d, xb, pd["conv_w"], None, post1, conv, idx)
        B.mamba2_state_update(d, post1, dt, pd["A_log"], pd["dt_bias"], pd["D"], z, y1, ssm, idx)
        yr, _ = oracle.decode(step["xbc"], step["dt_raw"], w["params"], [0], cp, sp, z=step["z"], **kw)
        torch.cuda.synchronize()
        assert_close(host(y1), yr, F32, "decode y")
    assert_close(host(ssm[slot:slot + 1]), sp, F32, "state after decode")
    assert np.array_equal(host(conv[slot:slot + 1]), cp)


@pytest.mark.parametrize("ws", [False, True], ids=["chunks", "blocks"])
@pytest.mark.parametrize("out_dtype", [F32, BF16])
@pytest.mark.parametrize("state_dtype", [F32, BF16])
def test_varlen_prefill_matches_oracle(out_dtype, state_dtype, ws):
    """Several chunks per sequence with ragged tails (lengths 1, 37, 130, 200 at chunk 64),
    half of the sequences resuming from a saved state. With a workspace, the bf16-y shapes run
    the scan as 32-token blocks (post-conv xBC in fp32 with an fp32 state, bf16 with a bf16
    state)."""
    d = D16.with_(out_dtype=out_dtype, state_dtype=state_dtype)
    print(f"[prefill parity] out={out_dtype} state={state_dtype} ws={ws}", flush=True)
    if ws and out_dtype == BF16:
        assert B.mamba2_chunk_scan_workspace_bytes(d, 368, 4) > 0
    w = synth.prefill_batch(d, seed=7, seqlens=[1, 37, 130, 200], num_slots=9, initial_state=True)
    has_init = np.array([1, 0, 1, 0], np.uint8)
    check_prefill(d, w, has_init=has_init, ws=ws)


def test_prefill_with_z_gate_and_tiny_dims():
    d = TINY
    w = synth.prefill_batch(d, seed=8, seqlens=[5, 16, 17, 40], num_slots=6, initial_state=True)
    check_prefill(d, w, has_init=np.array([0, 1, 1, 0], np.uint8))


def test_packed_equals_separate_runs_bitwise():
    """Packing sequences with cu_seqlens changes nothing: each sequence's outputs are bit-identical."""
    d = D16
    w = synth.prefill_batch(d, seed=9, seqlens=[70, 3, 129], num_slots=3, initial_state=False)
    y_all, _, ssm_all, _ = run_prefill(d, w)
    cu = w["cu_seqlens"]
    for i in range(3):
        s, e = int(cu[i]), int(cu[i + 1])
        wi = {**w, "xbc": w["xbc"][s:e], "dt_raw": w["dt_raw"][s:e], "z": w["z"][s:e],
              "cu_seqlens": np.array([0, e - s], np.int32), "slots": w["slots"][i:i + 1],
              "has_initial_state": w["has_initial_state"][i:i + 1]}
        yi, _, ssmi, _ = run_prefill(d, wi)
        assert torch.equal(yi, y_all[s:e])
        sl = int(w["slots"][i])
        assert torch.equal(ssmi[sl], ssm_all[sl])


def test_block_scan_packing_invariance():
    """chunk_scan_fwd with a workspace: 32-token blocks at absolute packed positions, so a
    sequence starting at a multiple of 32 is bit-identical packed or alone; elsewhere only the
    rounding order differs."""
    d = D16.with_(out_dtype=BF16)
    w = synth.prefill_batch(d, seed=9, seqlens=[64, 3, 29, 129], num_slots=4, initial_state=True)
    y_all, _, ssm_all, _ = run_prefill(d, w, ws=True)
    cu = w["cu_seqlens"]
    for i in range(4):
        s, e = int(cu[i]), int(cu[i + 1])
        wi = {**w, "xbc": w["xbc"][s:e], "dt_raw": w["dt_raw"][s:e], "z": w["z"][s:e],
              "cu_seqlens": np.array([0, e - s], np.int32), "slots": w["slots"][i:i + 1],
              "has_initial_state": w["has_initial_state"][i:i + 1]}
        yi, _, ssmi, _ = run_prefill(d, wi, ws=True)
        sl = int(w["slots"][i])
        if s % 32 == 0:
            assert torch.equal(yi, y_all[s:e]), f"sequence {i} at offset {s}"
            assert torch.equal(ssmi[sl], ssm_all[sl])
        else:
            assert_close(host(yi), host(y_all[s:e]), BF16, f"y of sequence {i} at offset {s}")
            assert_close(host(ssmi[sl]), host(ssm_all[sl]), d.state_dtype, f"state of sequence {i}")


def test_block_scan_segment_mode_matches_oracle():
    """chunk_scan_fwd with a workspace and few long sequences: the segment mode of the block
    scan (segments scanned in parallel, then the fix-up pass), against the oracle."""
    d = D16.with_(out_dtype=BF16)
    print("[prefill parity] block scan, segment mode", flush=True)
    w = synth.prefill_batch(d, seed=43, seqlens=[4100, 2048, 1], num_slots=4, initial_state=True)
    check_prefill(d, w, has_init=np.array([0, 1, 1], np.uint8), ws=True)


def test_block_scan_equals_chunk_scan():
    """The two forms of chunk_scan_fwd (32-token blocks with a workspace, chunks of 64
    without) agree within the bf16 y / fp32 state tolerances on the same post-conv input."""
    d = D16.with_(out_dtype=BF16)
    w = synth.prefill_batch(d, seed=13, seqlens=[300, 45, 1], num_slots=3, initial_state=True)
    hi = np.array([1, 0, 1], np.uint8)
    y0, post0, s0, _ = run_prefill(d, w, has_init=hi, ws=False)
    y1, post1, s1, _ = run_prefill(d, w, has_init=hi, ws=True)
    assert torch.equal(post0, post1)
    assert_close(host(y1), host(y0), BF16, "y: blocks vs chunks")
    assert_close(host(s1), host(s0), F32, "state: blocks vs chunks")


@pytest.mark.parametrize("dims,qs", [(D16, (64, 128)), (TINY, (16, 32, 64))], ids=["p64n128", "tiny"])
def test_chunk_size_invariance(dims, qs):
    """Every supported chunk length gives the oracle's result (in exact arithmetic the chunk
    length changes nothing) and the same result as the others within the tolerances. The
    32-token blocks of the workspace form are compared with chunks of 64 in
    test_block_scan_equals_chunk_scan; chunks of 256 at headdim 64, dstate 128 would need
    about twice the 120 KB of LDS that chunks of 128 take and are not built."""
    w = synth.prefill_batch(dims, seed=10, seqlens=[150, 77], num_slots=2, initial_state=True)
    hi = np.array([1, 1], np.uint8)
    outs = []
    for q in qs:
        dq = dims.with_(chunk_size=q)
        y, ssm, _, _ = check_prefill(dq, w, has_init=hi)
        outs.append((y, ssm))
    for y, ssm in outs[1:]:
        assert_close(host(y), host(outs[0][0]), dims.out_dtype, "y across chunk sizes")
        assert_close(host(ssm), host(outs[0][1]), dims.state_dtype, "state across chunk sizes")


def test_equivalence_contract_scan_equals_repeated_steps():
    """A T-token chunk scan equals T single-token state updates (GPU vs GPU)."""
    d = D16
    T = 150
    w = synth.prefill_batch(d, seed=11, seqlens=[T], num_slots=1, initial_state=True)
    hi = np.array([1], np.uint8)
    y_scan, _, ssm_scan, conv_scan = run_prefill(d, w, has_init=hi)
    pd = params_dev(w["params"])
    ssm = dev(w["ssm_pool"], d.state_dtype)
    conv = dev(w["conv_pool"], d.state_dtype)
    idx = dev_i32(w["slots"])
    xbc, dt, z = dev(w["xbc"], d.act_dtype), dev(w["dt_raw"], d.act_dtype), dev(w["z"], d.act_dtype)
    ys = torch.empty(T, d.d_inner, device="cuda")
    post = torch.empty(1, d.conv_dim, dtype=B._TORCH_DT[d.post_dtype], device="cuda")
    for t in range(T):
        B.mamba2_conv1d_update(d, xbc[t:t + 1], pd["conv_w"], None, post, conv, idx)
        B.mamba2_state_update(d, post, dt[t:t + 1], pd["A_log"], pd["dt_bias"], pd["D"], z[t:t + 1], ys[t:t + 1],
                              ssm, idx)
    torch.cuda.synchronize()
    assert_close(host(y_scan), host(ys), F32, "y: scan vs steps")
    assert_close(host(ssm_scan), host(ssm), F32, "state: scan vs steps")
    assert torch.equal(conv_scan, conv)


@pytest.mark.parametrize("out_dtype,ws", [(F32, False), (BF16, True)], ids=["chunks", "blocks"])
def test_padding_and_empty_sequences(out_dtype, ws):
    d = D16.with_(out_dtype=out_dtype)
    w = synth.prefill_batch(d, seed=12, seqlens=[40, 0, 33, 0], num_slots=6, initial_state=True)
    slots = w["slots"].copy()
    slots[2] = -1  # padding sequence
    has_init = np.array([1, 1, 0, 0], np.uint8)
    y, post, ssm, conv = run_prefill(d, w, has_init=has_init, slots=slots, ws=ws)
    cu = w["cu_seqlens"]
    assert torch.all(y[int(cu[2]):int(cu[3])] == 0).item()
    pad_slot = int(w["slots"][2])
    assert np.array_equal(host(ssm[pad_slot]), w["ssm_pool"][pad_slot].astype(np.float64))
    # empty sequence with a saved state keeps it; empty sequence without one ends at zero
    assert np.array_equal(host(ssm[int(slots[1])]), w["ssm_pool"][slots[1]].astype(np.float64))
    assert torch.all(ssm[int(slots[3])] == 0).item()
    check_prefill(d, w, has_init=has_init, slots=slots, ws=ws)


def test_mixed_batch_matches_oracle():
    """Varlen prefill sequences and decode rows in one call (fp32 pool)."""
    d = D16
    w = synth.mixed_batch(d, seed=3, num_prefill=3, len_lo=20, len_hi=150, decode_rows=5, num_slots=16,
                          with_z=True)
    pd = params_dev(w["params"])
    T = int(w["cu_seqlens"][-1])
    rows = T + 5
    xbc = dev(np.concatenate([w["prefill"]["xbc"], w["decode"]["xbc"]]), d.act_dtype)
    dt = dev(np.concatenate([w["prefill"]["dt_raw"], w["decode"]["dt_raw"]]), d.act_dtype)
    z = dev(np.concatenate([w["prefill"]["z"], w["decode"]["z"]]), d.act_dtype)
    ssm, conv = dev(w["ssm_pool"], d.state_dtype), dev(w["conv_pool"], d.state_dtype)
    post = torch.empty(rows, d.conv_dim, dtype=B._TORCH_DT[d.post_dtype], device="cuda")
    y = torch.empty(rows, d.d_inner, dtype=B._TORCH_DT[d.out_dtype], device="cuda")
    B.mamba2_mixed_fwd(d, xbc, dt, z, pd["conv_w"], None, pd["A_log"], pd["dt_bias"], pd["D"], post, y, ssm, conv,
                       dev_i32(w["cu_seqlens"]), dev_i32(w["prefill_slots"]), dev_u8(w["has_initial_state"]),
                       dev_i32(w["decode_slots"]))
    torch.cuda.synchronize()
    allslots = np.concatenate([w["prefill_slots"], w["decode_slots"]])
    cp, sp = compact_pools(w, allslots)
    kw = oracle_kw(d)
    yp, _ = oracle.prefill(w["prefill"]["xbc"], w["prefill"]["dt_raw"], w["params"], w["cu_seqlens"],
                           np.arange(3), w["has_initial_state"], cp, sp, z=w["prefill"]["z"], **kw)
    yd, _ = oracle.decode(w["decode"]["xbc"], w["decode"]["dt_raw"], w["params"], np.arange(3, 8), cp, sp,
                          z=w["decode"]["z"], **kw)
    assert_close(host(y), np.concatenate([yp, yd]), d.out_dtype, "mixed y")
    u = torch.from_numpy(allslots.astype(np.int64)).cuda()
    assert_close(host(ssm[u]), sp, d.state_dtype, "mixed states")
    assert np.array_equal(host(conv[u]), cp)
