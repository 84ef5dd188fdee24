"""GPU parity of the decode path (conv1d_update + state_update) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from _helpers import (TOL, assert_close, by_row_head, by_slot_head, compact_pools, dev, dev_i32, host, oracle_kw,
                      params_dev)
from state_space_model_ssm_amd import binding as B
from state_space_model_ssm_amd import synth
from state_space_model_ssm_amd.configs import BF16, F32, NEMOTRON_H_8B, TINY, Dims

pytestmark = pytest.mark.gpu

CASES = {
    # name: (dims, rows, slots, with_z)
    "tiny-f32": (TINY, 3, 4, True),
    "8b-bf16-small": (NEMOTRON_H_8B, 6, 13, True),
    "8b-f32state": (NEMOTRON_H_8B.with_(state_dtype=F32), 5, 9, False),
    "8b-bf16-f32out": (NEMOTRON_H_8B.with_(out_dtype=F32, xbc_dtype=F32), 4, 8, False),
    "mid-n64": (Dims(8, 32, 64, 2, 4, 64, BF16, BF16, BF16), 7, 11, True),
    # the full decode workload: 256 rows from a 512-slot bf16 pool
    "decode-8b": (NEMOTRON_H_8B, 256, 512, False),
    # small batches where a workgroup takes a whole head tile in four passes (bf16: 16 rows;
    # fp32: 12 rows, the tile then split over two workgroups)
    "8b-bf16-16rows": (NEMOTRON_H_8B, 16, 24, True),
    "8b-f32state-12rows": (NEMOTRON_H_8B.with_(state_dtype=F32), 12, 20, False),
}


def run_decode(d, w, slots_override=None):
    pd = params_dev(w["params"])
    idx = w["slots"] if slots_override is None else slots_override
    ssm = dev(w["ssm_pool"], d.state_dtype)
    conv = dev(w["conv_pool"], d.state_dtype)
    xbc = dev(w["xbc"], d.act_dtype)
    dt = dev(w["dt_raw"], d.act_dtype)
    z = None if w["z"] is None else dev(w["z"], d.act_dtype)
    rows = xbc.shape[0]
    post = torch.empty(rows, d.conv_dim, dtype=B._TORCH_DT[d.post_dtype], device="cuda")
    y = torch.empty(rows, d.d_inner, dtype=B._TORCH_DT[d.out_dtype], device="cuda")
    ii = dev_i32(idx)
    B.mamba2_conv1d_update(d, xbc, pd["conv_w"], pd["conv_b"], post, conv, ii)
    B.mamba2_state_update(d, post, dt, pd["A_log"], pd["dt_bias"], pd["D"], z, y, ssm, ii)
    torch.cuda.synchronize()
    return y, post, ssm, conv


@pytest.mark.parametrize("name", list(CASES))
def test_decode_step_matches_oracle(name):
    d, rows, nslots, with_z = CASES[name]
    print(f"[decode parity] {name} rows={rows} slots={nslots}", flush=True)
    w = synth.decode_batch(d, seed=1, rows=rows, num_slots=nslots, with_z=with_z)
    y, post, ssm, conv = run_decode(d, w)
    cp, sp = compact_pools(w, w["slots"])
    y_ref, post_ref = oracle.decode(w["xbc"], w["dt_raw"], w["params"], np.arange(rows), cp, sp, z=w["z"],
                                    **oracle_kw(d))
    assert_close(host(post), post_ref, d.post_dtype, "post-conv xBC")
    assert_close(host(y), y_ref, d.out_dtype, "y", slices=lambda a: by_row_head(a, d.nheads))
    slots = w["slots"].astype(np.int64)
    assert_close(host(ssm[torch.from_numpy(slots).cuda()]), sp, d.state_dtype, "ssm state", slices=by_slot_head)
    # the conv cache holds raw inputs: exact copies
    assert np.array_equal(host(conv[torch.from_numpy(slots).cuda()]), cp)
    # every other slot is bit-identical
    untouched = np.setdiff1d(np.arange(nslots), slots)
    if len(untouched):
        u = torch.from_numpy(untouched).cuda()
        assert torch.all(ssm[u].float() == synth.SENTINEL).item()
        assert torch.all(conv[u].float() == synth.SENTINEL).item()


def test_decode_bf16_state_tracks_rounding_emulation():
    """With a bf16 state the kernel rounds once per step; the oracle's bf16-state
    emulation makes the comparison tight (well inside the 2e-2 bound). The post-conv
    buffer is fp32 here so both sides feed the same x/B/C into the update."""
    d = NEMOTRON_H_8B.with_(xbc_dtype=F32)
    w = synth.decode_batch(d, seed=5, rows=4, num_slots=4, with_z=False)
    _, _, ssm, _ = run_decode(d, w)
    cp, sp = compact_pools(w, w["slots"])
    oracle.decode(w["xbc"], w["dt_raw"], w["params"], np.arange(4), cp, sp, round_state_bf16=True, **oracle_kw(d))
    got = host(ssm[torch.from_numpy(w["slots"].astype(np.int64)).cuda()])
    # at most one bf16 ulp apart where fp32 vs fp64 arithmetic straddles a rounding boundary
    # (plus fp32 rounding of the update itself, relevant only where terms cancel)
    bound = 2.0 ** -7 * np.abs(sp) + 1e-5 * np.max(np.abs(sp))
    bad = np.abs(got - sp) > bound
    assert not bad.any(), f"{int(bad.sum())} of {bad.size} elements beyond one bf16 ulp; " \
                          f"worst ratio {float(np.max(np.abs(got - sp) / bound)):.2f}"


def test_padding_rows_skip_and_zero_y():
    d = NEMOTRON_H_8B
    w = synth.decode_batch(d, seed=2, rows=5, num_slots=8, with_z=False)
    idx = w["slots"].copy()
    idx[[1, 3]] = -1
    y, post, ssm, conv = run_decode(d, w, slots_override=idx)
    assert torch.all(y[[1, 3]] == 0).item() and torch.all(post[[1, 3]] == 0).item()
    for s in w["slots"][[1, 3]]:
        assert np.array_equal(host(ssm[int(s)]), w["ssm_pool"][s].astype(np.float64))
        assert np.array_equal(host(conv[int(s)]), w["conv_pool"][s].astype(np.float64))


def test_decode_makes_no_allocation():
    """The decode entry points allocate nothing (torch's allocator sees no new block)."""
    d = NEMOTRON_H_8B
    w = synth.decode_batch(d, seed=3, rows=8, num_slots=8, with_z=False)
    run_decode(d, w)  # warm
    pd = params_dev(w["params"])
    ssm = dev(w["ssm_pool"], d.state_dtype)
    conv = dev(w["conv_pool"], d.state_dtype)
    xbc, dt = dev(w["xbc"], d.act_dtype), dev(w["dt_raw"], d.act_dtype)
    post = torch.empty(8, d.conv_dim, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(8, d.d_inner, dtype=torch.bfloat16, device="cuda")
    ii = dev_i32(w["slots"])
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats()["allocation.all.allocated"]
    for _ in range(3):
        B.mamba2_conv1d_update(d, xbc, pd["conv_w"], None, post, conv, ii)
        B.mamba2_state_update(d, post, dt, pd["A_log"], pd["dt_bias"], pd["D"], None, y, ssm, ii)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats()["allocation.all.allocated"] == before


@pytest.mark.parametrize("state_dtype,rows,nslots", [(BF16, 1024, 1024), (F32, 384, 1024)],
                         ids=["1024-rows-bf16", "384-rows-f32-1024-slots"])
def test_decode_largest_batches_sampled(state_dtype, rows, nslots):
    """The largest decode batches of the workloads: 1024 concurrent sequences on a full
    1024-slot bf16 pool (the 48-layer stack's top concurrency, per layer) and the mixed batch's
    384 rows on a 1024-slot fp32 pool; 16 sampled rows checked against the oracle, every
    untouched slot bit-identical."""
    d = NEMOTRON_H_8B.with_(state_dtype=state_dtype)
    print(f"[decode parity] {rows} rows, {nslots}-slot {state_dtype} pool (sampled)", flush=True)
    w = synth.decode_batch(d, seed=9, rows=rows, num_slots=nslots, with_z=True)
    y, post, ssm, conv = run_decode(d, w)
    pick = np.sort(np.random.default_rng(9).choice(rows, size=16, replace=False))
    sl = w["slots"][pick]
    cp, sp = compact_pools(w, sl)
    y_ref, post_ref = oracle.decode(w["xbc"][pick], w["dt_raw"][pick], w["params"], np.arange(16), cp, sp,
                                    z=w["z"][pick], **oracle_kw(d))
    ii = torch.from_numpy(pick.astype(np.int64)).cuda()
    assert_close(host(post[ii]), post_ref, d.post_dtype, "post-conv xBC")
    assert_close(host(y[ii]), y_ref, d.out_dtype, "y", slices=lambda a: by_row_head(a, d.nheads))
    s = torch.from_numpy(sl.astype(np.int64)).cuda()
    assert_close(host(ssm[s]), sp, state_dtype, "ssm state", slices=by_slot_head)
    assert np.array_equal(host(conv[s]), cp)
    untouched = np.setdiff1d(np.arange(nslots), w["slots"])
    if len(untouched):
        u = torch.from_numpy(untouched).cuda()
        assert torch.all(ssm[u].float() == synth.SENTINEL).item()
