"""Slot index safety: every pool-taking entry point is told the pool's slot count and skips
(like a padding row) any index at or beyond it, counting it in the library's per-device word.

The pools here are allocated with two guard slots past the declared count, in the same
tensor: an index that escaped the bound would write owned memory and show up as a changed
guard slot, never as a fault. Rows with valid indices are checked against the oracle."""

import numpy as np
import pytest
import torch

import oracle
from _helpers import assert_close, by_row_head, by_slot_head, dev, dev_i32, dev_u8, host, oracle_kw, params_dev
from state_space_model_ssm_amd import binding as B
from state_space_model_ssm_amd import synth
from state_space_model_ssm_amd.configs import BF16, F32, MAMBA1_8K, NEMOTRON_H_8B

pytestmark = pytest.mark.gpu

GUARD = 2


def guarded(w, d, n):
    """Device pools of n + GUARD slots (all from the generator: random where used, SENTINEL
    elsewhere) and views of their first n slots."""
    ssm = dev(w["ssm_pool"], d.state_dtype)
    conv = dev(w["conv_pool"], d.state_dtype)
    assert ssm.shape[0] == n + GUARD
    return ssm, conv, ssm[:n], conv[:n]


def assert_guards_untouched(ssm, conv, n):
    assert torch.all(ssm[n:].float() == synth.SENTINEL).item(), "a guard slot of the SSM pool was written"
    assert torch.all(conv[n:].float() == synth.SENTINEL).item(), "a guard slot of the conv pool was written"


def test_decode_skips_indices_past_the_pool():
    d = NEMOTRON_H_8B
    n = 6
    rows = 5
    B.mamba2_read_slot_errors(reset=True)
    w = synth.decode_batch(d, seed=51, rows=rows, num_slots=n + GUARD, with_z=True)
    idx = w["slots"].copy()
    bad = [0, 3]
    idx[bad] = [n, n + 1]  # one index at the bound, one into the second guard slot
    good_rows = [r for r in range(rows) if r not in bad]
    # the good rows' slots must lie inside the declared pool
    for r in good_rows:
        if idx[r] >= n:
            idx[r] = [s for s in range(n) if s not in idx][0]
    w["ssm_pool"][n:] = synth.SENTINEL
    w["conv_pool"][n:] = synth.SENTINEL
    ssm_all, conv_all, ssm, conv = guarded(w, d, n)
    pd = params_dev(w["params"])
    xbc, dt, z = dev(w["xbc"], d.act_dtype), dev(w["dt_raw"], d.act_dtype), dev(w["z"], d.act_dtype)
    post = torch.full((rows, d.conv_dim), 7.0, dtype=torch.float32 if d.post_dtype == F32 else torch.bfloat16,
                      device="cuda")
    y = torch.full((rows, d.d_inner), 7.0, dtype=torch.bfloat16, device="cuda")
    ii = dev_i32(idx)
    B.mamba2_conv1d_update(d, xbc, pd["conv_w"], None, post, conv, ii)
    B.mamba2_state_update(d, post, dt, pd["A_log"], pd["dt_bias"], pd["D"], z, y, ssm, ii)
    torch.cuda.synchronize()
    assert_guards_untouched(ssm_all, conv_all, n)
    assert torch.all(y[bad] == 0).item() and torch.all(post[bad] == 0).item()
    g = np.array(good_rows)
    cp = w["conv_pool"][idx[g]].astype(np.float64)
    sp = w["ssm_pool"][idx[g]].astype(np.float64)
    yr, _ = oracle.decode(w["xbc"][g], w["dt_raw"][g], w["params"], np.arange(len(g)), cp, sp, z=w["z"][g],
                          **oracle_kw(d))
    gi = torch.from_numpy(g).cuda()
    assert_close(host(y[gi]), yr, BF16, "y of the rows with valid slots", slices=lambda a: by_row_head(a, d.nheads))
    si = torch.from_numpy(idx[g].astype(np.int64)).cuda()
    assert_close(host(ssm[si]), sp, d.state_dtype, "their states", slices=by_slot_head)
    assert np.array_equal(host(conv[si]), cp), "their conv caches"
    errs = B.mamba2_read_slot_errors(reset=True)
    assert errs >= len(bad), errs  # each skipping kernel counts the row
    assert B.mamba2_read_slot_errors() == 0


@pytest.mark.parametrize("mode", ["fused", "blocks", "chunks"])
def test_prefill_skips_sequences_past_the_pool(mode):
    d = NEMOTRON_H_8B.with_(nheads=16, ngroups=2, chunk_size=64, state_dtype=F32)
    n = 4
    B.mamba2_read_slot_errors(reset=True)
    w = synth.prefill_batch(d, seed=52, seqlens=[40, 70, 33], num_slots=n + GUARD, initial_state=True)
    slots = np.array([1, n + 1, 3], np.int32)  # the middle sequence points into a guard slot
    w["ssm_pool"][n:] = synth.SENTINEL
    w["conv_pool"][n:] = synth.SENTINEL
    ssm_all, conv_all, ssm, conv = guarded(w, d, n)
    pd = params_dev(w["params"])
    T = int(w["cu_seqlens"][-1])
    xbc, dt = dev(w["xbc"], BF16), dev(w["dt_raw"], BF16)
    cu, ii, hi = dev_i32(w["cu_seqlens"]), dev_i32(slots), dev_u8(np.array([1, 1, 0], np.uint8))
    y = torch.full((T, d.d_inner), 7.0, dtype=torch.bfloat16, device="cuda")
    ws = B.prefill_workspace(d, T)
    if mode == "fused":
        B.mamba2_prefill_fwd(d, xbc, dt, None, pd["conv_w"], None, pd["A_log"], pd["dt_bias"], pd["D"], y, ssm, conv,
                             cu, ii, hi, ws)
    else:
        post = torch.empty(T, d.conv_dim, dtype=torch.float32, device="cuda")
        B.mamba2_conv1d_fwd(d, xbc, pd["conv_w"], None, post, conv, cu, ii, hi)
        B.mamba2_chunk_scan_fwd(d, post, dt, pd["A_log"], pd["dt_bias"], pd["D"], None, y, ssm, cu, ii, hi,
                                ws if mode == "blocks" else None)
    torch.cuda.synchronize()
    assert_guards_untouched(ssm_all, conv_all, n)
    cuh = w["cu_seqlens"]
    assert torch.all(y[int(cuh[1]):int(cuh[2])] == 0).item()
    kw = oracle_kw(d)
    for i in (0, 2):
        s, e, sl = int(cuh[i]), int(cuh[i + 1]), int(slots[i])
        init = i == 0
        cs0 = w["conv_pool"][sl].astype(np.float64) if init else np.zeros((d.conv_width - 1, d.conv_dim))
        hs0 = w["ssm_pool"][sl].astype(np.float64) if init else np.zeros((d.nheads, d.headdim, d.dstate))
        yr, _, cr, hr = oracle.layer_seq(w["xbc"][s:e], w["dt_raw"][s:e], w["params"], cs0, hs0, **kw)
        assert_close(host(y[s:e]), yr, BF16, f"{mode} y of sequence {i}")
        assert_close(host(ssm[sl])[None], hr[None], F32, f"{mode} state of sequence {i}", slices=by_slot_head)
        assert np.array_equal(host(conv[sl]), cr)
    assert B.mamba2_read_slot_errors(reset=True) >= 1


def test_multi_token_skips_destinations_past_the_pool():
    d = NEMOTRON_H_8B
    n, rows, T = 8, 2, 3
    B.mamba2_read_slot_errors(reset=True)
    rng = np.random.default_rng(53)
    w = synth.decode_batch(d, seed=53, rows=rows, num_slots=n + GUARD, with_z=False)
    w["ssm_pool"][n:] = synth.SENTINEL
    w["conv_pool"][n:] = synth.SENTINEL
    src = np.array([0, 1], np.int32)
    w["ssm_pool"][:2] = synth.round_to_dtype(rng.standard_normal((2, d.nheads, d.headdim, d.dstate)) * 0.3, BF16)
    dst = np.array([[2, n, 3], [n + 1, 4, 5]], np.int32)  # two snapshots point past the pool
    ssm_all, conv_all, ssm, conv = guarded(w, d, n)
    pd = params_dev(w["params"])
    tok = synth.tokens(d, rng, rows * T, with_z=False)
    xr = tok["xbc"].reshape(rows, T, d.conv_dim)
    dr = tok["dt_raw"].reshape(rows, T, d.nheads)
    post = torch.empty(rows, T, d.conv_dim, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(rows, T, d.d_inner, dtype=torch.bfloat16, device="cuda")
    B.mamba2_conv1d_update_multi(d, dev(xr, BF16), pd["conv_w"], None, post, conv, dev_i32(src), dev_i32(dst))
    B.mamba2_state_update_multi(d, post, dev(dr, BF16), pd["A_log"], pd["dt_bias"], pd["D"], None, y, ssm,
                                dev_i32(src), dev_i32(dst))
    torch.cuda.synchronize()
    assert_guards_untouched(ssm_all, conv_all, n)
    cp = w["conv_pool"][:n].astype(np.float64)
    sp = w["ssm_pool"][:n].astype(np.float64)
    dst_ok = np.where(dst >= n, -1, dst)
    yr, _ = oracle.decode_multi(xr, dr, w["params"], src, dst_ok, cp, sp, **oracle_kw(d))
    assert_close(host(y).reshape(rows * T, -1), yr.reshape(rows * T, -1), BF16, "multi-token y",
                 slices=lambda a: by_row_head(a, d.nheads))
    written = sorted(int(v) for v in dst_ok.ravel() if v >= 0)
    u = torch.tensor(written, device="cuda")
    assert_close(host(ssm[u]), sp[written], BF16, "snapshots", slices=by_slot_head)
    assert np.array_equal(host(conv[u]), cp[written]), "conv snapshots"
    assert B.mamba2_read_slot_errors(reset=True) >= 2


def test_mamba1_update_skips_indices_past_the_pool():
    d1 = MAMBA1_8K.with_(dim=256)
    n, rows = 3, 3
    B.mamba2_read_slot_errors(reset=True)
    w = synth.mamba1_batch(d1, seed=54, seqlens=[1] * rows, num_slots=n + GUARD, with_z=False, initial_state=True)
    idx = np.array([0, n, 2], np.int32)
    w["ssm_pool"][n:] = synth.SENTINEL
    pool_all = dev(w["ssm_pool"], F32)
    pool = pool_all[:n]
    y = torch.full((rows, d1.dim), 7.0, dtype=torch.bfloat16, device="cuda")
    A, D, db = dev(w["A"], F32), dev(w["D"], F32), dev(w["delta_bias"], F32)
    B.mamba1_selective_state_update(d1, dev(w["u"], BF16), dev(w["delta_raw"], BF16), A, dev(w["B"], BF16),
                                    dev(w["C"], BF16), D, None, db, y, pool, dev_i32(idx))
    torch.cuda.synchronize()
    assert torch.all(pool_all[n:] == synth.SENTINEL).item()
    assert torch.all(y[1] == 0).item()
    for r in (0, 2):
        yr, hr = oracle.selective_scan_seq(w["u"][r:r + 1], w["delta_raw"][r:r + 1], w["A"], w["B"][r:r + 1],
                                           w["C"][r:r + 1], w["ssm_pool"][idx[r]].astype(np.float64), D=w["D"],
                                           delta_bias=w["delta_bias"])
        assert_close(host(y[r:r + 1]), yr, BF16, f"row {r} y")
        assert_close(host(pool[int(idx[r])]), hr, F32, f"row {r} state")
    assert B.mamba2_read_slot_errors(reset=True) >= 1


def test_check_slot_indices_counts_bad_and_repeated():
    idx = torch.tensor([3, -1, 7, 3, 9, 0, -1, 7, 7, 12], dtype=torch.int32, device="cuda")
    bad, dup = B.check_slot_indices(idx, 10)
    assert (bad, dup) == (1, 3)  # 12 is past the pool; 3 once and 7 twice repeat earlier entries
    assert B.check_slot_indices(idx[:0], 10) == (0, 0)
    big = torch.randperm(4000, dtype=torch.int32, device="cuda")
    assert B.check_slot_indices(big, 4000) == (0, 0)
    assert B.check_slot_indices(big, 3999) == (1, 0)


def test_debug_mode_refuses_repeated_slots(monkeypatch):
    """MAMBA2_CHECK_SLOTS=1 makes every binding call check its index tables first."""
    d = NEMOTRON_H_8B.with_(nheads=16, ngroups=2)
    w = synth.decode_batch(d, seed=55, rows=3, num_slots=4, with_z=False)
    pd = params_dev(w["params"])
    conv = dev(w["conv_pool"], d.state_dtype)
    post = torch.empty(3, d.conv_dim, dtype=torch.bfloat16, device="cuda")
    monkeypatch.setenv("MAMBA2_CHECK_SLOTS", "1")
    with pytest.raises(ValueError, match=r"0 >= num_slots \(4\), 1 repeated"):
        B.mamba2_conv1d_update(d, dev(w["xbc"], BF16), pd["conv_w"], None, post, conv, dev_i32([1, 2, 1]))
    with pytest.raises(ValueError, match=r"1 >= num_slots \(4\), 0 repeated"):
        B.mamba2_conv1d_update(d, dev(w["xbc"], BF16), pd["conv_w"], None, post, conv, dev_i32([1, 2, 4]))
    B.mamba2_conv1d_update(d, dev(w["xbc"], BF16), pd["conv_w"], None, post, conv, dev_i32([1, 2, 0]))
    torch.cuda.synchronize()
