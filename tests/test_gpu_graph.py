"""The entry points are HIP-graph capturable (no allocation, memset or host sync
inside): a captured multi-layer decode step, and a captured mixed prefill + decode
call followed by a multi-token step, replay bit-identically to eager execution,
replay after replay."""
import numpy as np
import pytest
import torch

from _helpers import dev
from state_space_model_ssm_amd import binding as B
from state_space_model_ssm_amd import synth
from state_space_model_ssm_amd.configs import NEMOTRON_H_8B

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager_every_time():
    d = NEMOTRON_H_8B
    c, nl, steps = 4, 3, 3
    layers = []
    for l in range(nl):
        w = synth.stack_layer(d, seed=4, layer=l, concurrency=c, steps=steps)
        layers.append({k: dev(v, "bf16") for k, v in (("xbc", w["xbc"]), ("dt", w["dt_raw"]))})
        layers[-1].update({k: dev(w["params"][k], "f32") for k in ("conv_w", "A_log", "dt_bias", "D")})
    rng = np.random.default_rng(5)
    init = [(dev(rng.standard_normal((c, d.nheads, d.headdim, d.dstate)) * 0.3, "bf16"),
             dev(rng.standard_normal((c, d.conv_width - 1, d.conv_dim)), "bf16")) for _ in range(nl)]
    pools = [(s.clone(), v.clone()) for s, v in init]
    idx = torch.arange(c, dtype=torch.int32, device="cuda").flip(0).contiguous()
    post = torch.empty(c, d.conv_dim, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(nl, c, d.d_inner, dtype=torch.bfloat16, device="cuda")

    def run():
        for s_ in range(steps):
            for l, (L, (ssm, conv)) in enumerate(zip(layers, pools)):
                B.mamba2_conv1d_update(d, L["xbc"][s_:s_ + c], L["conv_w"], None, post, conv, idx)
                B.mamba2_state_update(d, post, L["dt"][s_:s_ + c], L["A_log"], L["dt_bias"], L["D"], None, y[l],
                                      ssm, idx)

    def reset():
        for (s, v), (s0, v0) in zip(pools, init):
            s.copy_(s0)
            v.copy_(v0)

    run()
    torch.cuda.synchronize()
    ref_y = y.clone()
    ref_pools = [(s.clone(), v.clone()) for s, v in pools]

    reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        graph.capture_begin()
        run()
        graph.capture_end()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for rep in range(4):
        reset()
        y.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref_y), f"replay {rep}: y differs"
        for (s, v), (rs, rv) in zip(pools, ref_pools):
            assert torch.equal(s, rs) and torch.equal(v, rv), f"replay {rep}: pools differ"
        # some eager work on the same pools between replays
        run()
        torch.cuda.synchronize()


def test_graph_replay_mixed_batch_and_multi_token():
    """A mixed prefill + decode call (the prefill through the fused kernels and their workspace)
    followed by a 3-token decode step of other rows, captured as one graph: every replay equals
    the eager result, with eager work on the same pools between replays."""
    from state_space_model_ssm_amd.configs import BF16, F32
    d = NEMOTRON_H_8B.with_(nheads=16, ngroups=2, state_dtype=F32, out_dtype=BF16)
    w = synth.mixed_batch(d, seed=31, num_prefill=3, len_lo=20, len_hi=150, decode_rows=5, num_slots=16,
                          with_z=True)
    T = int(w["cu_seqlens"][-1])
    rows = T + 5
    f = lambda a: dev(a, "bf16")
    xbc = f(np.concatenate([w["prefill"]["xbc"], w["decode"]["xbc"]]))
    dt = f(np.concatenate([w["prefill"]["dt_raw"], w["decode"]["dt_raw"]]))
    z = f(np.concatenate([w["prefill"]["z"], w["decode"]["z"]]))
    P_ = {k: dev(w["params"][k], "f32") for k in ("conv_w", "A_log", "dt_bias", "D")}
    ssm0, conv0 = dev(w["ssm_pool"], "f32"), dev(w["conv_pool"], "f32")
    cu = torch.from_numpy(w["cu_seqlens"]).cuda()
    pidx = torch.from_numpy(w["prefill_slots"]).cuda()
    didx = torch.from_numpy(w["decode_slots"]).cuda()
    hi = torch.from_numpy(w["has_initial_state"]).cuda()
    ws = B.prefill_workspace(d, T)
    post = torch.empty(rows, d.conv_dim, dtype=torch.float32, device="cuda")
    y = torch.empty(rows, d.d_inner, dtype=torch.bfloat16, device="cuda")
    # multi-token rows: 2 rows x 3 tokens on slots the mixed call does not touch
    used = set(int(v) for v in np.concatenate([w["prefill_slots"], w["decode_slots"]]))
    free = [s for s in range(16) if s not in used][:2]
    rng = np.random.default_rng(32)
    mx = f(rng.standard_normal((2, 3, d.conv_dim)))
    mdt = f(rng.standard_normal((2, 3, d.nheads)) * 0.5)
    msrc = torch.tensor(free, dtype=torch.int32, device="cuda")
    mpost = torch.empty(2, 3, d.conv_dim, dtype=torch.float32, device="cuda")
    my = torch.empty(2, 3, d.d_inner, dtype=torch.bfloat16, device="cuda")
    ssm, conv = ssm0.clone(), conv0.clone()

    def run():
        B.mamba2_mixed_fwd(d, xbc, dt, z, P_["conv_w"], None, P_["A_log"], P_["dt_bias"], P_["D"], post, y, ssm, conv,
                           cu, pidx, hi, didx, ws)
        B.mamba2_conv1d_update_multi(d, mx, P_["conv_w"], None, mpost, conv, msrc)
        B.mamba2_state_update_multi(d, mpost, mdt, P_["A_log"], P_["dt_bias"], P_["D"], None, my, ssm, msrc)

    def reset():
        ssm.copy_(ssm0)
        conv.copy_(conv0)

    run()
    torch.cuda.synchronize()
    ref = (y.clone(), my.clone(), ssm.clone(), conv.clone())
    reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        graph.capture_begin()
        run()
        graph.capture_end()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for rep in range(4):
        reset()
        y.zero_()
        my.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (y, my, ssm, conv)
        for name, a, b in zip(("y", "multi y", "ssm pool", "conv pool"), got, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs"
        reset()
        run()  # eager work on the same buffers between replays
        torch.cuda.synchronize()


def test_native_decode_graph_replays_match_eager():
    """mamba2_decode_graph_*: 3 layers x 2 steps captured once (each step an entry of its own,
    with its own input rows), replayed 4 times with the inputs refilled in place and eager work
    on the same pools between replays; every replay equals the eager calls bit for bit."""
    d = NEMOTRON_H_8B
    c, nl, steps = 5, 3, 2
    rng = np.random.default_rng(8)
    layers = []
    for l in range(nl):
        w = synth.stack_layer(d, seed=4, layer=l, concurrency=c, steps=steps)
        layers.append({"xbc": dev(w["xbc"], "bf16"), "dt": dev(w["dt_raw"], "bf16"),
                       **{k: dev(w["params"][k], "f32") for k in ("conv_w", "A_log", "dt_bias", "D")}})
    init = [(dev(rng.standard_normal((c + 2, d.nheads, d.headdim, d.dstate)) * 0.3, "bf16"),
             dev(rng.standard_normal((c + 2, d.conv_width - 1, d.conv_dim)), "bf16")) for _ in range(nl)]
    pools = [(s_.clone(), v.clone()) for s_, v in init]
    idx = torch.tensor([4, 0, 6, 2, 1], dtype=torch.int32, device="cuda")
    # static input buffers the graph reads (refilled before each replay) and per-entry outputs
    xin = torch.empty(steps, nl, c, d.conv_dim, dtype=torch.bfloat16, device="cuda")
    dtin = torch.empty(steps, nl, c, d.nheads, dtype=torch.bfloat16, device="cuda")
    post = torch.empty(c, d.conv_dim, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(steps, nl, c, d.d_inner, dtype=torch.bfloat16, device="cuda")

    def fill():
        for s_ in range(steps):
            for l, L in enumerate(layers):
                xin[s_, l].copy_(L["xbc"][s_:s_ + c])
                dtin[s_, l].copy_(L["dt"][s_:s_ + c])

    def eager():
        for s_ in range(steps):
            for l, (L, (ssm, conv)) in enumerate(zip(layers, pools)):
                B.mamba2_conv1d_update(d, xin[s_, l], L["conv_w"], None, post, conv, idx)
                B.mamba2_state_update(d, post, dtin[s_, l], L["A_log"], L["dt_bias"], L["D"], None, y[s_, l], ssm,
                                      idx)

    def reset():
        for (s_, v), (s0, v0) in zip(pools, init):
            s_.copy_(s0)
            v.copy_(v0)

    fill()
    eager()
    torch.cuda.synchronize()
    ref_y = y.clone()
    ref_pools = [(s_.clone(), v.clone()) for s_, v in pools]
    entries = [{"xbc": xin[s_, l], "conv_w": L["conv_w"], "conv_b": None, "xbc_post": post,
                "conv_pool": pools[l][1], "dt_raw": dtin[s_, l], "A_log": L["A_log"], "dt_bias": L["dt_bias"],
                "D": L["D"], "z": None, "y": y[s_, l], "ssm_pool": pools[l][0], "state_indices": idx}
               for s_ in range(steps) for l, L in enumerate(layers)]
    graph = B.DecodeGraph(d, entries)
    assert graph.layers == steps * nl and graph.batch == c
    for rep in range(4):
        reset()
        xin.zero_()
        fill()  # the inputs are refilled in place: the graph reads the same buffers
        y.zero_()
        graph.launch()
        torch.cuda.synchronize()
        assert torch.equal(y, ref_y), f"replay {rep}: y differs"
        for (s_, v), (rs, rv) in zip(pools, ref_pools):
            assert torch.equal(s_, rs) and torch.equal(v, rv), f"replay {rep}: pools differ"
        eager()  # eager work on the same pools between replays
        torch.cuda.synchronize()
    graph.close()


def test_native_decode_graph_rejects_bad_setup():
    d = NEMOTRON_H_8B
    with pytest.raises(ValueError, match="no layers"):
        B.DecodeGraph(d, [])
    ssm = torch.zeros(2, d.nheads, d.headdim, d.dstate, dtype=torch.bfloat16, device="cuda")
    conv = torch.zeros(3, d.conv_width - 1, d.conv_dim, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros(1, d.conv_dim, dtype=torch.bfloat16, device="cuda")
    f = lambda *s: torch.zeros(*s, device="cuda")
    entry = {"xbc": x, "conv_w": f(d.conv_dim, d.conv_width), "conv_b": None, "xbc_post": x.clone(),
             "conv_pool": conv, "dt_raw": torch.zeros(1, d.nheads, dtype=torch.bfloat16, device="cuda"),
             "A_log": f(d.nheads), "dt_bias": f(d.nheads), "D": f(d.nheads), "z": None,
             "y": torch.zeros(1, d.d_inner, dtype=torch.bfloat16, device="cuda"), "ssm_pool": ssm,
             "state_indices": torch.zeros(1, dtype=torch.int32, device="cuda")}
    with pytest.raises(ValueError, match="same number of slots"):
        B.DecodeGraph(d, [entry])
