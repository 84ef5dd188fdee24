"""The decode entry points are HIP-graph capturable (no allocation, memset or host
sync inside), and a captured multi-layer decode step replays bit-identically to
eager execution, replay after replay."""
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
