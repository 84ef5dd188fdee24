"""Pins for the fp64 oracle: each check ties it to something other than itself
(hand-worked examples, a library routine, closed forms, the quadratic dual form,
invariants), so a dropped term, wrong sign, wrong index or transposed operand
in the oracle fails at least one of them."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.dual import ssm_dual
from state_space_model_ssm_amd import synth
from state_space_model_ssm_amd.configs import TINY, Dims

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _pack(x, B, C):
    """Post-conv channel layout x || B || C, rows = tokens."""
    T = x.shape[0]
    return np.concatenate([x.reshape(T, -1), B.reshape(T, -1), C.reshape(T, -1)], axis=1)


def _rand_layer(rng, T, H, P, N, G, h0_scale=0.3):
    x = rng.standard_normal((T, H, P))
    B = rng.standard_normal((T, G, N)) / math.sqrt(N)
    C = rng.standard_normal((T, G, N)) / math.sqrt(N)
    dt_raw = rng.standard_normal((T, H)) * 0.7
    A_log = np.log(rng.uniform(1, 16, H))
    dt_bias = np.log(np.expm1(np.exp(rng.uniform(np.log(1e-3), np.log(0.1), H))))
    D = rng.standard_normal(H)
    h0 = rng.standard_normal((H, P, N)) * h0_scale
    return _pack(x, B, C), dt_raw, A_log, dt_bias, D, h0


# ------------------------------------------------------------------ scalars

def test_softplus_closed_forms():
    assert oracle.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    for v in (-30.0, -3.0, -0.5, 0.25, 2.0, 7.5):
        assert oracle.softplus(v) == pytest.approx(math.log(1.0 + math.exp(v)), rel=1e-13)
    assert oracle.softplus(50.0) == pytest.approx(50.0, rel=1e-15)
    assert oracle.softplus(800.0) == 800.0          # must not overflow through exp(v)
    assert oracle.softplus(-50.0) == pytest.approx(math.exp(-50.0), rel=1e-12)


def test_softplus_inverse_roundtrip():
    y = synth._log_uniform(np.random.default_rng(1), 1e-3, 0.1, 64)
    back = np.array([oracle.softplus(v) for v in synth._softplus_inv(y)])
    assert np.max(np.abs(back - y) / y) < 1e-12


def test_silu_closed_form():
    assert oracle.silu(0.0) == 0.0
    for v in (-8.0, -1.0, 0.5, 3.0):
        assert oracle.silu(v) == pytest.approx(v / (1.0 + math.exp(-v)), rel=1e-15)


def test_bf16_rounding_agrees_with_torch_and_generator():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(4000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 4000),
                        np.float32([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 1e-40])]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    ours_gen = synth.round_to_dtype(v, "bf16")
    ours_orc = np.array([oracle.round_bf16(float(a)) for a in v], dtype=np.float32)
    assert np.array_equal(ref.view(np.uint32), ours_gen.view(np.uint32))
    assert np.array_equal(ref.view(np.uint32), ours_orc.view(np.uint32))


# ------------------------------------------------------------------ conv1d

def test_conv_hand_examples():
    cases = json.load(open(os.path.join(GOLDEN, "hand_conv.json")))["cases"]
    for c in cases:
        w = np.array([c["w"]], np.float64)
        u = np.array(c["u"], np.float64)[:, None]
        st = np.array(c["state"], np.float64)[:, None]
        out, ns = oracle.conv1d_seq(u, w, None, st)
        v = np.array(c["pre_activation"], np.float64)
        assert np.allclose(out[:, 0], v / (1.0 + np.exp(-v)), rtol=1e-15, atol=0), c["name"]
        assert np.array_equal(ns[:, 0], np.array(c["new_state"], np.float64)), c["name"]


@pytest.mark.parametrize("W", [1, 2, 4])
@pytest.mark.parametrize("with_bias", [False, True])
def test_conv_matches_torch_conv1d(W, with_bias):
    rng = np.random.default_rng(10 + W)
    T, C = 37, 24
    u = rng.standard_normal((T, C))
    w = rng.standard_normal((C, W))
    b = rng.standard_normal(C) if with_bias else None
    st = rng.standard_normal((W - 1, C))
    out, ns = oracle.conv1d_seq(u, w, b, st)
    full = torch.from_numpy(np.concatenate([st, u], 0).T[None])          # [1, C, W-1+T]
    ref = torch.nn.functional.conv1d(full, torch.from_numpy(w)[:, None, :],
                                     None if b is None else torch.from_numpy(b), groups=C)
    ref = torch.nn.functional.silu(ref)[0].T.numpy()
    assert _rel(out, ref) < 1e-14
    assert np.array_equal(ns, np.concatenate([st, u], 0)[-(W - 1):] if W > 1 else ns)


def test_conv_zero_state_equals_left_zero_padding():
    rng = np.random.default_rng(3)
    T, C, W = 20, 8, 4
    u = rng.standard_normal((T, C))
    w = rng.standard_normal((C, W))
    out, _ = oracle.conv1d_seq(u, w, None, np.zeros((W - 1, C)))
    ref = torch.nn.functional.conv1d(torch.from_numpy(u.T[None]), torch.from_numpy(w)[:, None, :],
                                     padding=W - 1, groups=C)[..., :T]
    assert _rel(out, torch.nn.functional.silu(ref)[0].T.numpy()) < 1e-14


def test_conv_decode_step_equals_last_prefill_row():
    rng = np.random.default_rng(4)
    T, C, W = 9, 16, 4
    u = rng.standard_normal((T, C))
    w = rng.standard_normal((C, W))
    st0 = rng.standard_normal((W - 1, C))
    out_all, st_all = oracle.conv1d_seq(u, w, None, st0)
    st = st0
    for t in range(T):
        o, st = oracle.conv1d_seq(u[t:t + 1], w, None, st)
        assert np.array_equal(o[0], out_all[t])
    assert np.array_equal(st, st_all)


# ------------------------------------------------------------------ recurrence

def test_scan_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_scan.json")))
    x, B, C = (np.array(g[k], np.float64)[:, None] for k in ("x", "B", "C"))
    xbc = _pack(x, B, C)
    dt_bias = np.array([math.log(math.e - 1.0)])
    A_log = np.array([math.log(math.log(2.0))])
    D = np.array([g["D"]])
    h0 = np.array(g["h0"]).reshape(1, 1, 1)
    dt_raw = np.array(g["dt_raw"])[:, None]
    for fn in (oracle.ssm_seq, ssm_dual):
        y, hT = fn(xbc, dt_raw, A_log, dt_bias, D, h0, H=1, P=1, N=1, G=1)
        assert np.allclose(y[:, 0], g["y"], rtol=0, atol=1e-13), fn
        assert hT.reshape(()) == pytest.approx(g["h_final"], abs=1e-13)


@pytest.mark.parametrize("shape", [(64, 4, 16, 16, 1), (23, 4, 3, 5, 2), (17, 6, 2, 3, 3), (9, 2, 4, 8, 2)])
def test_loop_equals_dual_form(shape):
    T, H, P, N, G = shape
    rng = np.random.default_rng(sum(shape))
    xbc, dt_raw, A_log, dt_bias, D, h0 = _rand_layer(rng, T, H, P, N, G)
    z = rng.standard_normal((T, H * P))
    for zz in (None, z):
        y1, h1 = oracle.ssm_seq(xbc, dt_raw, A_log, dt_bias, D, h0, H=H, P=P, N=N, G=G, z=zz)
        y2, h2 = ssm_dual(xbc, dt_raw, A_log, dt_bias, D, h0, H=H, P=P, N=N, G=G, z=zz)
        assert _rel(y1, y2) < 1e-12
        assert _rel(h1, h2) < 1e-12


def test_scalar_closed_form_geometric_series():
    T = 50
    dt_val, x, Bv, Cv, D, h0 = 0.3, 1.7, -0.8, 1.3, 0.4, 2.5
    A_log = math.log(0.9)
    dt_bias = math.log(math.expm1(dt_val))      # softplus(dt_bias) = dt_val
    a = math.exp(-dt_val * 0.9)
    xbc = np.tile([x, Bv, Cv], (T, 1))
    for fn in (oracle.ssm_seq, ssm_dual):
        y, hT = fn(xbc, np.zeros((T, 1)), [A_log], [dt_bias], [D], np.full((1, 1, 1), h0), H=1, P=1, N=1, G=1)
        t = np.arange(1, T + 1)
        h = a ** t * h0 + dt_val * x * Bv * (1 - a ** t) / (1 - a)
        assert _rel(y[:, 0], Cv * h + D * x) < 1e-12
        assert hT.reshape(()) == pytest.approx(h[-1], rel=1e-12)


def test_zero_decay_is_dt_weighted_cumsum():
    rng = np.random.default_rng(5)
    T, H, P, N, G = 30, 4, 3, 5, 2
    xbc, dt_raw, _, dt_bias, D, h0 = _rand_layer(rng, T, H, P, N, G)
    A_log = np.full(H, -np.inf)                    # A = -0, a = 1
    y, hT = oracle.ssm_seq(xbc, dt_raw, A_log, dt_bias, D, h0, H=H, P=P, N=N, G=G)
    x = xbc[:, : H * P].reshape(T, H, P)
    B = xbc[:, H * P: H * P + G * N].reshape(T, G, N)
    C = xbc[:, H * P + G * N:].reshape(T, G, N)
    dt = np.log1p(np.exp(dt_raw + dt_bias))
    gmap = np.arange(H) // (H // G)
    inc = dt[:, :, None, None] * x[:, :, :, None] * B[:, gmap, None, :]    # [T, H, P, N]
    hs = h0[None] + np.cumsum(inc, axis=0)
    yref = np.einsum("thpn,thn->thp", hs, C[:, gmap]) + D[None, :, None] * x
    assert _rel(y, yref.reshape(T, -1)) < 1e-12
    assert _rel(hT, hs[-1]) < 1e-12


def test_vanishing_dt_keeps_initial_state():
    rng = np.random.default_rng(6)
    T, H, P, N, G = 12, 4, 3, 5, 2
    xbc, dt_raw, A_log, _, D, h0 = _rand_layer(rng, T, H, P, N, G, h0_scale=1.0)
    dt_bias = np.full(H, -40.0)                    # dt ~ 4e-18
    y, hT = oracle.ssm_seq(xbc, dt_raw, A_log, dt_bias, D, h0, H=H, P=P, N=N, G=G)
    x = xbc[:, : H * P].reshape(T, H, P)
    C = xbc[:, H * P + G * N:].reshape(T, G, N)
    gmap = np.arange(H) // (H // G)
    yref = np.einsum("hpn,thn->thp", h0, C[:, gmap]) + D[None, :, None] * x
    assert _rel(y, yref.reshape(T, -1)) < 1e-14
    assert _rel(hT, h0) < 1e-14


def test_zero_input_is_pure_decay():
    rng = np.random.default_rng(7)
    T, H, P, N, G = 15, 4, 2, 3, 2
    xbc, dt_raw, A_log, dt_bias, D, h0 = _rand_layer(rng, T, H, P, N, G, h0_scale=1.0)
    xbc[:, : H * P] = 0.0
    _, hT = oracle.ssm_seq(xbc, dt_raw, A_log, dt_bias, D, h0, H=H, P=P, N=N, G=G)
    dt = np.log1p(np.exp(dt_raw + dt_bias))
    decay = np.exp(-np.exp(A_log) * dt.sum(0))
    assert _rel(hT, decay[:, None, None] * h0) < 1e-13


def test_no_input_projection_gives_skip_only():
    rng = np.random.default_rng(8)
    T, H, P, N, G = 10, 4, 3, 4, 2
    xbc, dt_raw, A_log, dt_bias, D, _ = _rand_layer(rng, T, H, P, N, G)
    xbc[:, H * P: H * P + G * N] = 0.0
    y, _ = oracle.ssm_seq(xbc, dt_raw, A_log, dt_bias, D, np.zeros((H, P, N)), H=H, P=P, N=N, G=G)
    x = xbc[:, : H * P].reshape(T, H, P)
    assert np.array_equal(y, (D[None, :, None] * x).reshape(T, -1))


def test_group_map_is_contiguous_blocks():
    """Head h reads group h // (H/G): silencing group 1's B leaves heads 2,3 untouched."""
    rng = np.random.default_rng(9)
    T, H, P, N, G = 6, 4, 2, 3, 2
    xbc, dt_raw, A_log, dt_bias, D, _ = _rand_layer(rng, T, H, P, N, G)
    xbc[:, H * P + N: H * P + 2 * N] = 0.0
    _, hT = oracle.ssm_seq(xbc, dt_raw, A_log, dt_bias, D, np.zeros((H, P, N)), H=H, P=P, N=N, G=G)
    assert np.all(hT[2:] == 0.0) and np.all(np.abs(hT[:2]).sum(axis=(1, 2)) > 0)


def test_grouped_equals_per_head_replicated():
    rng = np.random.default_rng(11)
    T, H, P, N, G = 14, 6, 3, 4, 2
    xbc, dt_raw, A_log, dt_bias, D, h0 = _rand_layer(rng, T, H, P, N, G)
    x = xbc[:, : H * P]
    B = xbc[:, H * P: H * P + G * N].reshape(T, G, N)
    C = xbc[:, H * P + G * N:].reshape(T, G, N)
    rep = np.arange(H) // (H // G)
    xbc_h = np.concatenate([x, B[:, rep].reshape(T, -1), C[:, rep].reshape(T, -1)], 1)
    y1, h1 = oracle.ssm_seq(xbc, dt_raw, A_log, dt_bias, D, h0, H=H, P=P, N=N, G=G)
    y2, h2 = oracle.ssm_seq(xbc_h, dt_raw, A_log, dt_bias, D, h0, H=H, P=P, N=N, G=H)
    assert np.array_equal(y1, y2) and np.array_equal(h1, h2)


def test_split_and_resume_is_bit_identical():
    d = TINY
    w = synth.tiny(d, seed=0)
    pr = w["params"]
    tok = w["prefill"]
    T = tok["xbc"].shape[0]
    kw = dict(H=d.nheads, P=d.headdim, N=d.dstate, G=d.ngroups)
    cs0 = np.zeros((d.conv_width - 1, d.conv_dim))
    h0 = np.zeros((d.nheads, d.headdim, d.dstate))
    y_all, _, cs_all, hs_all = oracle.layer_seq(tok["xbc"], tok["dt_raw"], pr, cs0, h0, z=tok["z"], **kw)
    for k in range(1, T):
        ya, _, csa, hsa = oracle.layer_seq(tok["xbc"][:k], tok["dt_raw"][:k], pr, cs0, h0, z=tok["z"][:k], **kw)
        yb, _, csb, hsb = oracle.layer_seq(tok["xbc"][k:], tok["dt_raw"][k:], pr, csa, hsa, z=tok["z"][k:], **kw)
        assert np.array_equal(np.concatenate([ya, yb]), y_all)
        assert np.array_equal(csb, cs_all) and np.array_equal(hsb, hs_all)


def test_decode_rows_are_permutation_invariant_and_in_place():
    d = Dims(4, 8, 8, 2, 4, 16, "f32", "f32", "f32")
    w = synth.decode_batch(d, seed=3, rows=6, num_slots=10)
    kw = dict(H=d.nheads, P=d.headdim, N=d.dstate, G=d.ngroups)
    cp, sp = w["conv_pool"].astype(np.float64), w["ssm_pool"].astype(np.float64)
    y, _ = oracle.decode(w["xbc"], w["dt_raw"], w["params"], w["slots"], cp, sp, z=w["z"], **kw)
    perm = np.random.default_rng(0).permutation(6)
    cp2, sp2 = w["conv_pool"].astype(np.float64), w["ssm_pool"].astype(np.float64)
    y2, _ = oracle.decode(w["xbc"][perm], w["dt_raw"][perm], w["params"], w["slots"][perm], cp2, sp2,
                          z=w["z"][perm], **kw)
    assert np.array_equal(y2, y[perm]) and np.array_equal(cp, cp2) and np.array_equal(sp, sp2)
    untouched = np.setdiff1d(np.arange(10), w["slots"])
    assert np.all(sp[untouched] == synth.SENTINEL) and np.all(cp[untouched] == synth.SENTINEL)


def test_decode_padding_rows_touch_nothing():
    d = Dims(4, 8, 8, 2, 4, 16, "f32", "f32", "f32")
    w = synth.decode_batch(d, seed=4, rows=4, num_slots=6)
    slots = w["slots"].copy()
    slots[1] = -1
    cp, sp = w["conv_pool"].astype(np.float64), w["ssm_pool"].astype(np.float64)
    y, _ = oracle.decode(w["xbc"], w["dt_raw"], w["params"], slots, cp, sp,
                         H=4, P=8, N=8, G=2)
    assert np.all(y[1] == 0.0)
    assert np.array_equal(sp[w["slots"][1]], w["ssm_pool"][w["slots"][1]])


def test_prefill_then_decode_equals_one_long_sequence():
    """The equivalence contract on the oracle side: a T-token prefill followed by
    single-token steps equals processing all tokens as one sequence."""
    d = TINY
    w = synth.tiny(d, seed=0)
    kw = dict(H=d.nheads, P=d.headdim, N=d.dstate, G=d.ngroups)
    cp, sp = w["conv_pool"].astype(np.float64), w["ssm_pool"].astype(np.float64)
    y_pre, _ = oracle.prefill(w["prefill"]["xbc"], w["prefill"]["dt_raw"], w["params"], w["cu_seqlens"],
                              w["slots"], w["has_initial_state"], cp, sp, z=w["prefill"]["z"], **kw)
    ys = [y_pre]
    for st in w["decode"]:
        yd, _ = oracle.decode(st["xbc"], st["dt_raw"], w["params"], w["slots"], cp, sp, z=st["z"], **kw)
        ys.append(yd)
    allx = np.concatenate([w["prefill"]["xbc"]] + [s["xbc"] for s in w["decode"]])
    alldt = np.concatenate([w["prefill"]["dt_raw"]] + [s["dt_raw"] for s in w["decode"]])
    allz = np.concatenate([w["prefill"]["z"]] + [s["z"] for s in w["decode"]])
    y_one, _, cs, hs = oracle.layer_seq(allx, alldt, w["params"], np.zeros((3, d.conv_dim)),
                                        np.zeros((d.nheads, d.headdim, d.dstate)), z=allz, **kw)
    assert np.array_equal(np.concatenate(ys), y_one)
    assert np.array_equal(sp[w["slots"][0]], hs) and np.array_equal(cp[w["slots"][0]], cs)


def test_bf16_state_emulation_rounds_every_step():
    rng = np.random.default_rng(12)
    T, H, P, N, G = 5, 2, 2, 3, 1
    xbc, dt_raw, A_log, dt_bias, D, h0 = _rand_layer(rng, T, H, P, N, G)
    h0 = synth.round_to_dtype(h0, "bf16").astype(np.float64)
    h = h0.copy()
    for t in range(T):
        _, h = oracle.ssm_seq(xbc[t:t + 1], dt_raw[t:t + 1], A_log, dt_bias, D, h, H=H, P=P, N=N, G=G)
        h = np.vectorize(oracle.round_bf16)(h)
    _, hb = oracle.ssm_seq(xbc, dt_raw, A_log, dt_bias, D, h0, H=H, P=P, N=N, G=G, round_state_bf16=True)
    assert np.array_equal(h, hb)


# ---------------------------------------------------------------- gated RMSNorm
# The "norm" mixer tensor of the record page; the formula is this build's reading
# (see oracle/norm.py). Pins: hand example, unit RMS per group, per-group scale
# and sign behaviour, group independence, the two limits of the SiLU gate.

def _norm_inputs(rows=3, width=64, seed=0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((rows, width)), rng.standard_normal((rows, width))


def test_norm_hand_example():
    # group of 4: y = (3, 4, 0, 0) -> rms = sqrt(25/4) = 2.5 -> (1.2, 1.6, 0, 0)
    y = np.array([[3.0, 4.0, 0.0, 0.0, 1.0, 1.0, 1.0, 1.0]])
    out = oracle.gated_rmsnorm(y, None, np.ones(8), 0.0, 4)
    assert np.allclose(out, [[1.2, 1.6, 0.0, 0.0, 1.0, 1.0, 1.0, 1.0]], rtol=0, atol=1e-15)


def test_norm_unit_rms_per_group_and_group_independence():
    y, z = _norm_inputs()
    out = oracle.gated_rmsnorm(y, z, np.ones(64), 0.0, 16)
    ms = (out.reshape(3, 4, 16) ** 2).mean(axis=2)
    assert np.allclose(ms, 1.0, rtol=0, atol=1e-12)
    y2 = y.copy()
    y2[:, :16] *= 7.0
    y2[:, 3] = -2.0
    out2 = oracle.gated_rmsnorm(y2, z, np.ones(64), 0.0, 16)
    assert np.array_equal(out2[:, 16:], out[:, 16:])


def test_norm_scale_and_sign_per_group():
    y, _ = _norm_inputs(seed=1)
    base = oracle.gated_rmsnorm(y, None, np.ones(64), 0.0, 32)
    c = np.repeat(np.array([[0.25, 3.0]]), 32, axis=1)
    assert np.allclose(oracle.gated_rmsnorm(y * c, None, np.ones(64), 0.0, 32), base, rtol=0, atol=1e-12)
    assert np.allclose(oracle.gated_rmsnorm(-y, None, np.ones(64), 0.0, 32), -base, rtol=0, atol=1e-15)


def test_norm_weight_is_per_channel():
    y, z = _norm_inputs(seed=2)
    w = np.linspace(-2.0, 2.0, 64)
    assert np.allclose(oracle.gated_rmsnorm(y, z, w, 1e-5, 16), w * oracle.gated_rmsnorm(y, z, np.ones(64), 1e-5, 16),
                       rtol=0, atol=1e-14)


def test_norm_gate_limits():
    """SiLU(z) -> z for large z and -> 0 from below for very negative z: a gate of
    +40 * s acts as the multiplier s, a gate of -40 flips the sign."""
    y, _ = _norm_inputs(seed=3)
    plain = oracle.gated_rmsnorm(y, None, np.ones(64), 0.0, 16)
    s = np.random.default_rng(4).uniform(1.0, 2.0, size=y.shape)  # z >= 40: SiLU(z) = z in fp64
    assert np.allclose(oracle.gated_rmsnorm(y, np.full(y.shape, 40.0), np.ones(64), 0.0, 16), plain, rtol=0,
                       atol=1e-12)
    assert np.allclose(oracle.gated_rmsnorm(y, 40.0 * s, np.ones(64), 0.0, 16),
                       oracle.gated_rmsnorm(y * s, None, np.ones(64), 0.0, 16), rtol=0, atol=1e-12)
    assert np.allclose(oracle.gated_rmsnorm(y, np.full(y.shape, -40.0), np.ones(64), 0.0, 16), -plain, rtol=0,
                       atol=1e-12)


def test_norm_zero_group_with_eps_is_zero():
    y = np.zeros((2, 8))
    y[1, 4:] = 1.0
    out = oracle.gated_rmsnorm(y, None, np.ones(8), 1e-5, 4)
    assert np.all(out[0] == 0.0) and np.all(out[1, :4] == 0.0)
    assert np.allclose(out[1, 4:], 1.0 / math.sqrt(1.0 + 1e-5), rtol=0, atol=1e-15)


def test_multi_token_decode_equals_single_steps_and_snapshots():
    """T tokens per row through decode_multi equal T one-token decode calls (the same C
    loop, so bit-identical), and each per-step snapshot is the state after that step."""
    d = TINY
    rng = np.random.default_rng(31)
    w = synth.prefill_batch(d, seed=31, seqlens=[1], num_slots=8, initial_state=False)
    params = w["params"]
    kw = dict(H=d.nheads, P=d.headdim, N=d.dstate, G=d.ngroups)
    Bd, T = 3, 4
    x = rng.standard_normal((Bd, T, d.conv_dim))
    dt = rng.standard_normal((Bd, T, d.nheads)) * 0.7
    z = rng.standard_normal((Bd, T, d.d_inner))
    cp = rng.standard_normal((8, d.conv_width - 1, d.conv_dim))
    sp = rng.standard_normal((8, d.nheads, d.headdim, d.dstate)) * 0.3
    src = np.array([5, -1, 2])
    dst = np.array([[0, 1, -1, 5], [3, 3, 3, 3], [4, -1, 6, 7]])
    cp1, sp1 = cp.copy(), sp.copy()
    y, _ = oracle.decode_multi(x, dt, params, src, dst, cp1, sp1, z=z, **kw)
    cp2, sp2 = cp.copy(), sp.copy()
    for t in range(T):
        yt, _ = oracle.decode(x[:, t], dt[:, t], params, src, cp2, sp2, z=z[:, t], **kw)
        assert np.array_equal(yt, y[:, t])
        for i in (0, 2):
            if dst[i][t] >= 0:
                assert np.array_equal(sp1[dst[i][t]], sp2[src[i]]) and np.array_equal(cp1[dst[i][t]], cp2[src[i]])
    assert np.all(y[1] == 0) and np.array_equal(sp1[3], sp[3]) and np.array_equal(cp1[3], cp[3])
    # without destinations the final state lands in the source slot
    cp3, sp3 = cp.copy(), sp.copy()
    oracle.decode_multi(x, dt, params, src, None, cp3, sp3, z=z, **kw)
    assert np.array_equal(sp3[5], sp2[5]) and np.array_equal(sp3[2], sp2[2]) and np.array_equal(cp3[2], cp2[2])


# ---------------------------------------------------------------- Mamba-1 selective scan
# The "selective_scan_fwd" kernel named on the trace page; the recurrence of the Mamba
# paper (diagonal A per channel and state). Pins: reduction to the (separately pinned)
# scalar-A recurrence, a closed form, A = 0, and the unrolled quadratic form.

def _sel_inputs(T, Dc, N, G, seed):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((T, Dc))
    dr = rng.standard_normal((T, Dc)) * 0.7
    A = -np.exp(rng.uniform(-1.0, 1.5, size=(Dc, N)))
    Bm = rng.standard_normal((T, G, N)) / math.sqrt(N)
    Cm = rng.standard_normal((T, G, N)) / math.sqrt(N)
    return rng, u, dr, A, Bm, Cm


def test_selective_scan_reduces_to_scalar_decay_recurrence():
    """With A constant over a head's channels and states and delta shared by the head, the
    selective scan is the scalar-A recurrence (x = u)."""
    H, P, N, G, T = 4, 3, 5, 2, 9
    rng = np.random.default_rng(40)
    A_log = rng.uniform(-1.0, 1.0, H)
    dt_bias = rng.standard_normal(H) * 0.3
    D = rng.standard_normal(H)
    x = rng.standard_normal((T, H * P))
    Bm = rng.standard_normal((T, G, N))
    Cm = rng.standard_normal((T, G, N))
    dt_raw = rng.standard_normal((T, H))
    h0 = rng.standard_normal((H, P, N)) * 0.3
    z = rng.standard_normal((T, H * P))
    xbc = np.concatenate([x, Bm.reshape(T, G * N), Cm.reshape(T, G * N)], axis=1)
    y2, h2 = oracle.ssm_seq(xbc, dt_raw, A_log, dt_bias, D, h0, H=H, P=P, N=N, G=G, z=z)
    rep = lambda v: np.repeat(v, P, axis=-1)
    A1 = np.repeat(-np.exp(A_log), P)[:, None] * np.ones((1, N))
    y1, h1 = oracle.selective_scan_seq(x, rep(dt_raw), A1, Bm, Cm, h0.reshape(H * P, N), D=rep(D), z=z,
                                       delta_bias=rep(dt_bias))
    assert np.allclose(y1, y2, rtol=1e-12, atol=1e-12)
    assert np.allclose(h1.reshape(H, P, N), h2, rtol=1e-12, atol=1e-13)


def test_selective_scan_scalar_closed_form():
    """Dc = N = 1, constant delta, u, B: h_t = a^t h0 + delta u B (1 - a^t) / (1 - a)."""
    T, dl, uu, bb, cc, A, h0 = 12, 0.3, 1.7, -0.6, 1.3, -0.8, 0.45
    a = math.exp(dl * A)
    y, h = oracle.selective_scan_seq(np.full((T, 1), uu), np.full((T, 1), dl), np.array([[A]]),
                                     np.full((T, 1, 1), bb), np.full((T, 1, 1), cc), np.array([[h0]]),
                                     delta_softplus=False)
    ht = [a ** (t + 1) * h0 + dl * uu * bb * (1 - a ** (t + 1)) / (1 - a) for t in range(T)]
    assert np.allclose(y[:, 0], cc * np.array(ht), rtol=1e-13, atol=1e-14)
    assert math.isclose(h[0, 0], ht[-1], rel_tol=1e-13)


def test_selective_scan_zero_decay_is_cumsum():
    T, Dc, N, G = 7, 4, 3, 1
    rng, u, dr, A, Bm, Cm = _sel_inputs(T, Dc, N, G, 41)
    dl = np.abs(dr) + 0.1
    h0 = rng.standard_normal((Dc, N))
    y, h = oracle.selective_scan_seq(u, dl, np.zeros((Dc, N)), Bm, Cm, h0, delta_softplus=False)
    hs = h0[None] + np.cumsum(dl[:, :, None] * Bm[:, 0][:, None, :] * u[:, :, None], axis=0)
    assert np.allclose(h, hs[-1], rtol=1e-13, atol=1e-13)
    assert np.allclose(y, np.einsum("tn,tdn->td", Cm[:, 0], hs), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("G", [1, 2])
def test_selective_scan_equals_unrolled_quadratic_form(G):
    """y_t[d] = sum_{s<=t} sum_n C_t[n] exp(A[d,n] sum_{s<r<=t} delta_r) delta_s B_s[n] u_s
    + sum_n C_t[n] exp(A[d,n] sum_{r<=t} delta_r) h0[d,n] + D u_t, computed term by term."""
    T, Dc, N = 6, 4, 3
    rng, u, dr, A, Bm, Cm = _sel_inputs(T, Dc, N, G, 42 + G)
    Dv = rng.standard_normal(Dc)
    bias = rng.standard_normal(Dc) * 0.2
    h0 = rng.standard_normal((Dc, N))
    y, _ = oracle.selective_scan_seq(u, dr, A, Bm, Cm, h0, D=Dv, delta_bias=bias)
    dl = np.log1p(np.exp(dr + bias))  # softplus
    ref = np.zeros((T, Dc))
    for t in range(T):
        for d in range(Dc):
            g = d // (Dc // G)
            acc = Dv[d] * u[t, d]
            for n in range(N):
                acc += Cm[t, g, n] * math.exp(A[d, n] * dl[:t + 1, d].sum()) * h0[d, n]
                for s in range(t + 1):
                    acc += Cm[t, g, n] * math.exp(A[d, n] * dl[s + 1:t + 1, d].sum()) * dl[s, d] * Bm[s, g, n] * u[s, d]
            ref[t, d] = acc
    assert np.allclose(y, ref, rtol=1e-11, atol=1e-12)


def test_selective_scan_channels_are_independent():
    T, Dc, N, G = 5, 6, 4, 1
    rng, u, dr, A, Bm, Cm = _sel_inputs(T, Dc, N, G, 44)
    h0 = np.zeros((Dc, N))
    y, h = oracle.selective_scan_seq(u, dr, A, Bm, Cm, h0)
    A2 = A.copy()
    A2[2, 1] *= 3.0
    u2 = u.copy()
    u2[:, 4] += 1.0
    y2, h2 = oracle.selective_scan_seq(u2, dr, A2, Bm, Cm, h0)
    keep = [0, 1, 3, 5]
    assert np.array_equal(y2[:, keep], y[:, keep]) and np.array_equal(h2[keep], h[keep])
    assert not np.allclose(y2[:, 2], y[:, 2]) and not np.allclose(y2[:, 4], y[:, 4])
