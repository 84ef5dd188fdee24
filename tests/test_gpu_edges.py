"""Edge cases of the shapes against the oracle: conv widths 2 and 3 (every kernel is built for
widths 2 to 4), one head per group, 80 heads in one group, 12 heads, the largest decode batch (4,096 rows on a full 4,096-slot
pool) and the longest prefill sequence (131,072 tokens, whose packed rows pass 2 GiB of input,
resumed from a saved state)."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from _helpers import (assert_close, by_head, by_row_head, by_slot_head, compact_pools, dev, dev_i32, dev_u8, host,
                      oracle_head_seq, oracle_kw, params_dev)
from state_space_model_ssm_amd import binding as B
from state_space_model_ssm_amd import synth
from state_space_model_ssm_amd.configs import BF16, F32, NEMOTRON_H_8B, TINY

pytestmark = pytest.mark.gpu

D16B = NEMOTRON_H_8B.with_(nheads=16, ngroups=2, chunk_size=64, state_dtype=F32, out_dtype=BF16)


def decode_check(d, w, what):
    rows = w["xbc"].shape[0]
    pd = params_dev(w["params"])
    ssm, conv = dev(w["ssm_pool"], d.state_dtype), dev(w["conv_pool"], d.state_dtype)
    post = torch.empty(rows, d.conv_dim, dtype=B._TORCH_DT[d.post_dtype], device="cuda")
    y = torch.empty(rows, d.d_inner, dtype=B._TORCH_DT[d.out_dtype], device="cuda")
    ii = dev_i32(w["slots"])
    z = None if w["z"] is None else dev(w["z"], d.act_dtype)
    B.mamba2_conv1d_update(d, dev(w["xbc"], d.act_dtype), pd["conv_w"], pd["conv_b"], post, conv, ii)
    B.mamba2_state_update(d, post, dev(w["dt_raw"], d.act_dtype), pd["A_log"], pd["dt_bias"], pd["D"], z, y, ssm, ii)
    torch.cuda.synchronize()
    cp, sp = compact_pools(w, w["slots"])
    yr, pr = oracle.decode(w["xbc"], w["dt_raw"], w["params"], np.arange(rows), cp, sp, z=w["z"], **oracle_kw(d))
    assert_close(host(post), pr, d.post_dtype, f"{what}: post-conv xBC")
    assert_close(host(y), yr, d.out_dtype, f"{what}: y", slices=lambda a: by_row_head(a, d.nheads))
    u = torch.from_numpy(w["slots"].astype(np.int64)).cuda()
    assert_close(host(ssm[u]), sp, d.state_dtype, f"{what}: states", slices=by_slot_head)
    assert np.array_equal(host(conv[u]), cp), f"{what}: conv caches"


def prefill_check(d, w, has_init, fused, what):
    T = w["xbc"].shape[0]
    pd = params_dev(w["params"])
    ssm, conv = dev(w["ssm_pool"], d.state_dtype), dev(w["conv_pool"], d.state_dtype)
    xbc, dt = dev(w["xbc"], d.act_dtype), dev(w["dt_raw"], d.act_dtype)
    z = None if w["z"] is None else dev(w["z"], d.act_dtype)
    cu, ii, hi = dev_i32(w["cu_seqlens"]), dev_i32(w["slots"]), dev_u8(has_init)
    y = torch.empty(T, d.d_inner, dtype=B._TORCH_DT[d.out_dtype], device="cuda")
    if fused:
        B.mamba2_prefill_fwd(d, xbc, dt, z, pd["conv_w"], pd["conv_b"], pd["A_log"], pd["dt_bias"], pd["D"], y, ssm,
                             conv, cu, ii, hi, B.prefill_workspace(d, T))
    else:
        post = torch.empty(T, d.conv_dim, dtype=B._TORCH_DT[d.post_dtype], device="cuda")
        B.mamba2_conv1d_fwd(d, xbc, pd["conv_w"], pd["conv_b"], post, conv, cu, ii, hi)
        B.mamba2_chunk_scan_fwd(d, post, dt, pd["A_log"], pd["dt_bias"], pd["D"], z, y, ssm, cu, ii, hi)
    torch.cuda.synchronize()
    used = list(w["slots"])
    cp, sp = compact_pools(w, used)
    yr, _ = oracle.prefill(w["xbc"], w["dt_raw"], w["params"], w["cu_seqlens"], np.arange(len(used)), has_init, cp,
                           sp, z=w["z"], **oracle_kw(d))
    assert_close(host(y), yr, d.out_dtype, f"{what}: y", slices=lambda a: by_head(a, d.nheads))
    u = torch.tensor(used, dtype=torch.long, device="cuda")
    assert_close(host(ssm[u]), sp, d.state_dtype, f"{what}: states", slices=by_slot_head)
    assert np.array_equal(host(conv[u]), cp), f"{what}: conv caches"


@pytest.mark.parametrize("W", [2, 3])
def test_conv_widths_2_and_3(W):
    """Decode (conv update + state update), the unfused prefill (conv1d_fwd + chunk scan), the
    fused prefill and multi-token decode with conv width W, sequences shorter than W - 1
    included (their new conv cache keeps part of the old one)."""
    print(f"[edges] conv width {W}", flush=True)
    d = D16B.with_(conv_width=W)
    decode_check(d, synth.decode_batch(d, seed=70 + W, rows=5, num_slots=9, with_z=True), f"W={W} decode")
    lens = [1, W - 1, 37, 130]
    w = synth.prefill_batch(d, seed=72 + W, seqlens=lens, num_slots=6, initial_state=True)
    hi = np.array([1, 1, 0, 1], np.uint8)
    prefill_check(d, w, hi, fused=True, what=f"W={W} fused prefill")
    dt = TINY.with_(conv_width=W)
    w = synth.prefill_batch(dt, seed=74 + W, seqlens=lens, num_slots=6, initial_state=True)
    prefill_check(dt, w, hi, fused=False, what=f"W={W} unfused prefill (tiny dims)")
    # multi-token conv update: 2 rows x 3 tokens, final window in place
    w = synth.decode_batch(d, seed=76 + W, rows=2, num_slots=3, with_z=False)
    rng = np.random.default_rng(W)
    xr = synth.round_to_dtype(synth.xbc_values(d, rng, 6), d.act_dtype).reshape(2, 3, d.conv_dim)
    pd = params_dev(w["params"])
    conv = dev(w["conv_pool"], d.state_dtype)
    post = torch.empty(2, 3, d.conv_dim, dtype=B._TORCH_DT[d.post_dtype], device="cuda")
    B.mamba2_conv1d_update_multi(d, dev(xr, d.act_dtype), pd["conv_w"], None, post, conv, dev_i32(w["slots"]))
    torch.cuda.synchronize()
    for r in range(2):
        cs = w["conv_pool"][int(w["slots"][r])].astype(np.float64)
        pr, cs2 = oracle.conv1d_seq(xr[r], w["params"]["conv_w"], None, cs)
        assert_close(host(post[r]), pr, d.post_dtype, f"W={W} multi-token conv row {r}")
        assert np.array_equal(host(conv[int(w["slots"][r])]), cs2)


def test_one_head_per_group():
    """G = H (every head its own B/C group) at the Nemotron head shape: fused prefill and decode."""
    d = D16B.with_(nheads=4, ngroups=4)
    print("[edges] one head per group", flush=True)
    w = synth.prefill_batch(d, seed=78, seqlens=[90, 33], num_slots=3, initial_state=True)
    prefill_check(d, w, np.array([1, 0], np.uint8), fused=True, what="G = H fused prefill")
    decode_check(d.with_(state_dtype=BF16), synth.decode_batch(d.with_(state_dtype=BF16), seed=79, rows=3, num_slots=5),
                 "G = H decode")


def test_decode_largest_batch_4096_rows():
    """4,096 rows on a full 4,096-slot bf16 pool (8 GiB of state, the last slot 8 GiB into it).
    Every slot starts from one shared random state except 32 sampled rows' slots, which get
    their own; those rows and 16 others are checked against the oracle, every y is finite."""
    d = NEMOTRON_H_8B
    rows = 4096
    print(f"[edges] decode {rows} rows", flush=True)
    rng = np.random.Generator(np.random.PCG64(80))
    params = synth.layer_params(d, rng)
    tok = synth.tokens(d, rng, rows, with_z=False)
    slots = synth.slot_ids(rng, rows, rows)  # a permutation of the whole pool
    picked = np.sort(rng.choice(rows, 48, replace=False))
    own, shared = picked[:32], picked[32:]
    hs_base, cs_base = synth.stack_slot(d, 80, 0, rows)  # the shared state (not a pool slot's own seed)
    ssm = dev(hs_base, BF16).unsqueeze(0).repeat(rows, 1, 1, 1)
    conv = dev(cs_base, BF16).unsqueeze(0).repeat(rows, 1, 1)
    init_h = {}
    for r in own:
        hs, cs = synth.stack_slot(d, 80, 0, int(slots[r]))
        ssm[int(slots[r])] = dev(hs, BF16)
        conv[int(slots[r])] = dev(cs, BF16)
        init_h[int(r)] = (hs, cs)
    pd = params_dev(params)
    post = torch.empty(rows, d.conv_dim, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(rows, d.d_inner, dtype=torch.bfloat16, device="cuda")
    ii = dev_i32(slots)
    B.mamba2_conv1d_update(d, dev(tok["xbc"], BF16), pd["conv_w"], None, post, conv, ii)
    B.mamba2_state_update(d, post, dev(tok["dt_raw"], BF16), pd["A_log"], pd["dt_bias"], pd["D"], None, y, ssm, ii)
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all().item()
    sp = np.stack([init_h[int(r)][0] if int(r) in init_h else hs_base for r in picked]).astype(np.float64)
    cp = np.stack([init_h[int(r)][1] if int(r) in init_h else cs_base for r in picked]).astype(np.float64)
    yr, _ = oracle.decode(tok["xbc"][picked], tok["dt_raw"][picked], params, np.arange(len(picked)), cp, sp,
                          **oracle_kw(d))
    pi = torch.from_numpy(picked.astype(np.int64)).cuda()
    assert_close(host(y[pi]), yr, BF16, "y", slices=lambda a: by_row_head(a, d.nheads))
    si = torch.from_numpy(slots[picked].astype(np.int64)).cuda()
    assert_close(host(ssm[si]), sp, BF16, "states", slices=by_slot_head)
    assert np.array_equal(host(conv[si]), cp)


@pytest.mark.timeout(400)
def test_prefill_longest_sequence_131072_tokens():
    """One 131,072-token sequence (2.7 GB of packed bf16 input, past 2^31 bytes; segment mode),
    resumed from a saved conv and SSM state: one head of every group against the oracle (the
    heads' oracle runs in threads: its C loop does not hold the interpreter lock), and the conv
    cache."""
    d = NEMOTRON_H_8B.with_(state_dtype=F32)
    T = 131072
    print(f"[edges] one {T}-token sequence", flush=True)
    w = synth.prefill_batch(d, seed=81, seqlens=[T], num_slots=2, with_z=False, initial_state=True)
    pd = params_dev(w["params"])
    ssm, conv = dev(w["ssm_pool"], F32), dev(w["conv_pool"], F32)
    y = torch.empty(T, d.d_inner, dtype=torch.bfloat16, device="cuda")
    B.mamba2_prefill_fwd(d, dev(w["xbc"], BF16), dev(w["dt_raw"], BF16), None, pd["conv_w"], None, pd["A_log"],
                         pd["dt_bias"], pd["D"], y, ssm, conv, dev_i32(w["cu_seqlens"]), dev_i32(w["slots"]),
                         dev_u8(np.array([1], np.uint8)), B.prefill_workspace(d, T))
    torch.cuda.synchronize()
    sl = int(w["slots"][0])
    cs0, hs0 = w["conv_pool"][sl].astype(np.float64), w["ssm_pool"][sl].astype(np.float64)
    heads = [g * (d.nheads // d.ngroups) + (5 * g) % (d.nheads // d.ngroups) for g in range(d.ngroups)]
    with ThreadPoolExecutor(max_workers=8) as ex:
        refs = list(ex.map(lambda h: oracle_head_seq(d, w["params"], w["xbc"], w["dt_raw"], h, conv_state=cs0,
                                                     ssm_state=hs0), heads))
    for head, (yr, hr) in zip(heads, refs):
        assert_close(host(y[:, head * 64:(head + 1) * 64]), yr, BF16, f"y head {head}",
                     slices=lambda a: a.reshape(-1, 4096, 64))
        assert_close(host(ssm[sl, head]), hr, F32, f"state head {head}")
    assert np.array_equal(host(conv[sl]), w["xbc"][-(d.conv_width - 1):].astype(np.float64))


def test_single_group_80_heads():
    """Mamba-2 2.7B-class head layout at the same head shape: 80 heads sharing one B/C group.
    The fused prefill (a 2,200-token sequence long enough for the segment mode next to a short
    one), the unfused prefill (conv1d_fwd + chunk scan without a workspace) and decode."""
    d = NEMOTRON_H_8B.with_(nheads=80, ngroups=1, state_dtype=F32, out_dtype=BF16)
    print("[edges] 80 heads, one group", flush=True)
    w = synth.prefill_batch(d, seed=82, seqlens=[2200, 300], num_slots=3, initial_state=True)
    hi = np.array([1, 0], np.uint8)
    prefill_check(d, w, hi, fused=True, what="80 heads fused prefill")
    prefill_check(d, w, hi, fused=False, what="80 heads unfused prefill")
    db = d.with_(state_dtype=BF16)
    decode_check(db, synth.decode_batch(db, seed=83, rows=6, num_slots=9, with_z=True), "80 heads decode")


def test_head_count_not_a_multiple_of_eight():
    """12 heads in 3 groups: the head-to-XCD remap needs H divisible by 8 and falls back to
    the identity. Fused prefill and decode."""
    d = D16B.with_(nheads=12, ngroups=3)
    print("[edges] 12 heads, 3 groups", flush=True)
    w = synth.prefill_batch(d, seed=84, seqlens=[150, 1, 77], num_slots=4, initial_state=True)
    prefill_check(d, w, np.array([1, 1, 0], np.uint8), fused=True, what="H = 12 fused prefill")
    decode_check(d, synth.decode_batch(d, seed=85, rows=4, num_slots=6, with_z=True), "H = 12 decode")
