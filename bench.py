#!/usr/bin/env python3
"""Benchmark of the Mamba-2 SSM core at one Nemotron-H-8B layer on one MI355X.

Primary line (the metric's decode half): decode tokens/s of one layer step
(conv1d_update + state_update) for 256 sequences drawn from a 512-slot bf16
state pool (128 heads x headdim 64 x d_state 128, 8 groups). The prefill half
(mamba2_prefill_fwd over 4 x 8192 tokens, bf16 inputs, fp32 state; the layer's
chunk_size is 128, the fused path cuts 32-token blocks; the unfused conv1d_fwd +
chunk_scan_fwd pair and the prefill with the gated RMSNorm alongside) is
reported in the same JSON line under "prefill".

Inputs are seeded synthetic tensors already resident in HBM when timing
starts. Per-kernel durations come from HIP events on the stream the kernels
are launched on (torch's current stream, which the binding passes down).

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16
FP32_VECTOR_PEAK_TFLOPS = 157.3  # published fp32 vector peak, which counts packed (two-per-lane) fp32 instructions
# Without packed fp32 instructions (this build disables them) one FMA per lane and cycle:
# 256 CUs x 4 SIMDs x 16 lanes x 2 flops x 2.4 GHz = 78.6 TFLOP/s.
FP32_VECTOR_UNPACKED_TFLOPS = 78.6
# A transcendental (v_exp_f32) issues at a quarter of the FMA rate (measured 0.28x on this chip), so it
# occupies the issue slots of 4 FMAs: 8 flop-equivalents against the peak above.
EXP_FLOP_EQUIV = 8


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_bytes_per_row(d, state_bytes):
    """Algorithmic HBM bytes of one decode row-layer, split by kernel."""
    H, P, N, G, W = d.nheads, d.headdim, d.dstate, d.ngroups, d.conv_width
    cdim = H * P + 2 * G * N
    act = 2
    su = 2 * H * P * N * state_bytes + cdim * act + H * act + H * P * act   # state r+w, x|B|C in, dt in, y out
    cu = 2 * (W - 1) * cdim * state_bytes + cdim * act + cdim * act          # conv cache r+w, raw in, post out
    minimum = 2 * H * P * N * state_bytes + 2 * (W - 1) * cdim * state_bytes + cdim * act + H * act + H * P * act
    return su, cu, minimum


def scan_algorithmic(d, tokens, nseq, xbc_bytes, y_bytes, state_bytes, chunk=None):
    """Bytes and flops the chunk scan must move/compute (causal SSD, per token) with chunks of
    `chunk` tokens (the layer's chunk_size by default; the fused and block forms run 32)."""
    H, P, N, G = d.nheads, d.headdim, d.dstate, d.ngroups
    Q = d.chunk_size if chunk is None else chunk
    cdim = H * P + 2 * G * N
    nbytes = tokens * (cdim * xbc_bytes + H * 2 + H * P * y_bytes) + nseq * H * P * N * state_bytes
    # C.B^T (per group, causal) + intra-chunk output (causal) + chunk state + inter-chunk output
    flops_per_tok = G * Q * N + H * Q * P + 2 * H * P * N + 2 * H * P * N
    return nbytes, flops_per_tok * tokens


def profiled_record(kernel):
    """The `traffic-json` record of `kernel` under profiles/ (written by profile_report.py from
    rocprofv3 runs: calibrated FETCH_SIZE + WRITE_SIZE bytes per launch, and the kernel-trace
    average duration), or None when there is none or the kernel's sources changed since."""
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            if not line.startswith("traffic-json:"):
                continue
            rec = json.loads(line.split(":", 1)[1])
            if rec.get("kernel") != kernel:
                continue
            h = hashlib.sha256()
            for f in rec["sources"]:
                path_f = os.path.join(ROOT, "state_space_model_ssm_amd", "csrc", f)
                if not os.path.exists(path_f):
                    return None
                h.update(open(path_f, "rb").read())
            return rec if h.hexdigest()[:16] == rec["src_sha"] else None
    return None


def profiled_traffic(kernel):
    rec = profiled_record(kernel)
    return None if rec is None else rec["bytes_per_launch"]


def rocprof_check(kernel, nbytes):
    """Cross-check of a roofline from the profiled record: the kernel-trace average duration
    and the fraction of HBM peak it gives for the same algorithmic bytes."""
    rec = profiled_record(kernel)
    if rec is None or not rec.get("avg_us"):
        return None
    gbs = nbytes / (rec["avg_us"] * 1e-6) / 1e9
    return {"rocprof_avg_us": rec["avg_us"], "frac": round(gbs / HBM_PEAK_GBS, 4)}


def time_region(fn, iters, torch):
    """Average ms of fn() over iters, HIP events on the current stream."""
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


def settle(fn, torch, ms=50.0):
    """Run fn() untimed for about ms of wall time. The GPU's clocks ramp up under load: a
    decode step timed right after a handful of warmup steps measured 4 % slower than after
    this (198.7 against 191.2 us)."""
    import time
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()


def bench_stack(args, torch, np, B, synth, d, dev, bf, time_region):
    """48 Mamba-2 layers x 32 decode steps at several concurrencies, eager and as one
    captured HIP graph per run. Layer l has its own seeded parameters and an input
    buffer of c + 31 rows (step s reads rows [s, s + c)); each layer has its own
    bf16 state and conv pools of c slots, read and written in place every step."""
    from state_space_model_ssm_amd.configs import NEMOTRON_H_8B_MAMBA_LAYERS as NL
    conc = [int(c) for c in args.stack_concurrency.split(",") if c]
    steps = 32
    cmax = max(conc)
    log(f"stack workload: {NL} layers x {steps} steps, concurrency {conc}; generating per-layer inputs")
    layers = []
    for l in range(NL):
        w = synth.stack_layer(d, seed=4, layer=l, concurrency=cmax, steps=steps)
        layers.append({"xbc": dev(w["xbc"], bf), "dt": dev(w["dt_raw"], bf),
                       "conv_w": dev(w["params"]["conv_w"], torch.float32),
                       "A_log": dev(w["params"]["A_log"], torch.float32),
                       "dt_bias": dev(w["params"]["dt_bias"], torch.float32),
                       "D": dev(w["params"]["D"], torch.float32)})
    gen = torch.Generator(device="cuda")
    row_b = decode_bytes_per_row(d, 2)[2]
    out = {"workload": f"{NL}-layer Mamba-2 decode stack at Nemotron-H-8B dims, bf16 state (96 MiB per sequence), "
                       f"{steps} steps of one token; per-layer seeded parameters and inputs; state pools filled "
                       "on the device from a seeded normal generator (std sqrt(0.1))",
           "layers": NL, "steps": steps, "points": []}
    for c in conc:
        gen.manual_seed(1000 + c)
        pools = []
        for l in range(NL):
            ssm = torch.empty(c, d.nheads, d.headdim, d.dstate, dtype=bf, device="cuda")
            ssm.normal_(0.0, 0.1 ** 0.5, generator=gen)
            conv = torch.empty(c, d.conv_width - 1, d.conv_dim, dtype=bf, device="cuda")
            conv.normal_(0.0, 1.0, generator=gen)
            pools.append((ssm, conv))
        idx = torch.arange(c, dtype=torch.int32, device="cuda")
        post = torch.empty(c, d.conv_dim, dtype=bf, device="cuda")
        y = torch.empty(c, d.d_inner, dtype=bf, device="cuda")

        def run(steps_=steps):
            for s_ in range(steps_):
                for L, (ssm, conv) in zip(layers, pools):
                    xb = L["xbc"][s_:s_ + c]
                    B.mamba2_conv1d_update(d, xb, L["conv_w"], None, post, conv, idx)
                    B.mamba2_state_update(d, post, L["dt"][s_:s_ + c], L["A_log"], L["dt_bias"], L["D"], None, y,
                                          ssm, idx)

        run(1)
        torch.cuda.synchronize()
        ms_eager = time_region(run, 1, torch)
        # the same 32 steps x 48 layers as one captured decode graph (mamba2_decode_graph_*)
        graph = B.DecodeGraph(d, [{"xbc": L["xbc"][s_:s_ + c], "conv_w": L["conv_w"], "conv_b": None,
                                   "xbc_post": post, "conv_pool": conv, "dt_raw": L["dt"][s_:s_ + c],
                                   "A_log": L["A_log"], "dt_bias": L["dt_bias"], "D": L["D"], "z": None, "y": y,
                                   "ssm_pool": ssm, "state_indices": idx}
                                  for s_ in range(steps) for L, (ssm, conv) in zip(layers, pools)])
        graph.launch()
        torch.cuda.synchronize()
        ms_graph = time_region(graph.launch, 1, torch)
        tok = c * steps
        bytes_ = row_b * c * NL * steps
        pt = {"concurrency": c,
              "eager": {"tok_s": round(tok / (ms_eager * 1e-3), 1), "ms_per_step": round(ms_eager / steps, 4),
                        "hbm_frac": round(bytes_ / (ms_eager * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
              "graph": {"tok_s": round(tok / (ms_graph * 1e-3), 1), "ms_per_step": round(ms_graph / steps, 4),
                        "hbm_frac": round(bytes_ / (ms_graph * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
        state_mib = c * NL * 2 * d.nheads * d.headdim * d.dstate / 2 ** 20
        if state_mib <= 256:
            pt["note"] = (f"the stack's state ({state_mib:.0f} MiB) fits the 256 MB memory-side cache; "
                          "launch-bound (two short kernels per layer and step)")
        elif c <= 16:
            pt["note"] = (f"state of {state_mib:.0f} MiB streamed from HBM every step; each layer's grid "
                          f"({c} rows x 128 heads) is short, so launch gaps and the tail of each kernel "
                          "dominate")
        graph.close()
        out["points"].append(pt)
        log(f"stack c={c}: eager {ms_eager / steps * 1e3:.0f} us/step, graph {ms_graph / steps * 1e3:.0f} us/step")
        del pools, post, y
        torch.cuda.empty_cache()
    return out


def t1_ab(args, result, torch, B, d, rows, xbc, conv_w, post, conv, idx, dt, A_log, dtb, D, y, ssm, decode_step):
    """The vllm.cpp page's A/B at T = 1: the decode workload's rows, slots and pools through the
    chunk-scan arm, each row a one-token sequence of conv1d_fwd + chunk_scan_fwd
    (has_initial_state = 1, final states written back in place), without and with the scan's
    optional workspace, against conv1d_update + state_update."""
    cu1 = torch.arange(rows + 1, dtype=torch.int32, device="cuda")
    hi1 = torch.ones(rows, dtype=torch.uint8, device="cuda")
    ws1 = torch.empty(max(16, B.mamba2_chunk_scan_workspace_bytes(d, rows, rows)), dtype=torch.uint8, device="cuda")

    def chunk_arm(ws=None):
        B.mamba2_conv1d_fwd(d, xbc, conv_w, None, post, conv, cu1, idx, hi1)
        B.mamba2_chunk_scan_fwd(d, post, dt, A_log, dtb, D, None, y, ssm, cu1, idx, hi1, ws)

    for _ in range(3):
        chunk_arm()
        chunk_arm(ws1)
    ms_chunk = time_region(chunk_arm, args.steps, torch)
    ms_chunk_ws = time_region(lambda: chunk_arm(ws1), args.steps, torch)
    ms_upd = time_region(decode_step, args.steps, torch)
    post_b = rows * d.conv_dim * 2
    moved = lambda a, b: round(abs(a - b) / b * 100.0, 1)
    result["t1_ab"] = {
        "workload": f"{rows} decode rows of one token on the decode workload's slots and pools: the chunk-scan "
                    "arm (conv1d_fwd + chunk_scan_fwd, each row a one-token sequence, chunk 128) against "
                    "conv1d_update + state_update",
        "update_arm": {"us_per_token": round(ms_upd * 1e3 / rows, 4), "us_per_step": round(ms_upd * 1e3, 2),
                       "kernel_launches": 2, "allocations": 0, "memsets": 0,
                       "scratch_bytes": post_b, "scratch": "post-conv xBC rows (caller buffer)"},
        "chunk_arm": {"us_per_token": round(ms_chunk * 1e3 / rows, 4), "us_per_step": round(ms_chunk * 1e3, 2),
                      "kernel_launches": 3, "allocations": 0, "memsets": 0, "scratch_bytes": post_b,
                      "scratch": "post-conv xBC rows (caller buffer)"},
        "chunk_arm_with_workspace": {"us_per_token": round(ms_chunk_ws * 1e3 / rows, 4),
                                     "us_per_step": round(ms_chunk_ws * 1e3, 2), "kernel_launches": 4,
                                     "allocations": 0, "memsets": 0, "scratch_bytes": post_b + ws1.numel(),
                                     "scratch": "post-conv xBC rows + the B/C operand planes (caller buffers)"},
        "per_token_time_moved_pct": moved(ms_chunk, ms_upd),
        "refuted_if_below_pct": 3.0,
        "verdict": "confirmed: the update arm is faster" if moved(ms_chunk, ms_upd) >= 3.0 and ms_upd < ms_chunk
                   else "refuted (under 3 %)"}
    log(f"T=1 A/B: update arm {ms_upd * 1e3:.1f} us, chunk arm {ms_chunk * 1e3:.1f} us "
        f"(with workspace {ms_chunk_ws * 1e3:.1f} us)")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def single_thread_oracle(seconds):
    """The decode sample of the CPU baseline on one thread: a child process with OMP_NUM_THREADS=1
    (the oracle's OpenMP runtime in this process has already fixed its thread count)."""
    import subprocess
    code = ("import os, sys, time, numpy as np; sys.path.insert(0, %r); import oracle; "
            "from state_space_model_ssm_amd import synth; from state_space_model_ssm_amd.configs import NEMOTRON_H_8B as d; "
            "w = synth.decode_batch(d, seed=1, rows=16, num_slots=32, with_z=False); "
            "kw = dict(H=d.nheads, P=d.headdim, N=d.dstate, G=d.ngroups); "
            "cp = w['conv_pool'][w['slots']].astype(np.float64); sp = w['ssm_pool'][w['slots']].astype(np.float64); "
            "t0 = time.perf_counter(); n = 0\n"
            "while time.perf_counter() - t0 < %f:\n"
            "    i = n %% 16; oracle.decode(w['xbc'][i:i+1], w['dt_raw'][i:i+1], w['params'], [0], cp[i:i+1], "
            "sp[i:i+1], **kw); n += 1\n"
            "print(n, time.perf_counter() - t0)") % (ROOT, seconds)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=600)
    if r.returncode != 0:
        return {"error": r.stderr[-400:]}
    n, el = r.stdout.split()
    n, el = int(n), float(el)
    return {"value": round(n / el, 2), "unit": "tok/s", "cores": 1,
            "sample": f"{n} decode row-steps (16 rows of the decode workload, all 128 heads) in {el:.1f} s"}


def cpu_mixed_sample(oracle, synth, seconds):
    """The oracle on a bounded sample of the mixed batch (fp32 state): its first prefill sequence's
    tokens in 64-token pieces, then decode rows, until `seconds` pass; rate in tokens/s."""
    import numpy as np
    from state_space_model_ssm_amd.configs import F32, NEMOTRON_H_8B
    d = NEMOTRON_H_8B.with_(state_dtype=F32)
    kw = dict(H=d.nheads, P=d.headdim, N=d.dstate, G=d.ngroups)
    w = synth.mixed_batch(d, seed=3, num_prefill=8, len_lo=256, len_hi=4096, decode_rows=16, num_slots=32)
    L0 = int(w["cu_seqlens"][1])
    cs = np.zeros((d.conv_width - 1, d.conv_dim))
    hs = np.zeros((d.nheads, d.headdim, d.dstate))
    t0 = time.perf_counter()
    n = 0
    while n < L0 and time.perf_counter() - t0 < seconds / 2:
        _, _, cs, hs = oracle.layer_seq(w["prefill"]["xbc"][n:n + 64], w["prefill"]["dt_raw"][n:n + 64], w["params"],
                                        cs, hs, **kw)
        n += min(64, L0 - n)
    t_pre = time.perf_counter() - t0
    sl = w["decode_slots"]
    cp = w["conv_pool"][sl].astype(np.float64)
    sp = w["ssm_pool"][sl].astype(np.float64)
    t1 = time.perf_counter()
    r = 0
    while time.perf_counter() - t1 < seconds / 2:
        i = r % len(sl)
        oracle.decode(w["decode"]["xbc"][i:i + 1], w["decode"]["dt_raw"][i:i + 1], w["params"], [0], cp[i:i + 1],
                      sp[i:i + 1], **kw)
        r += 1
    t_dec = time.perf_counter() - t1
    T3 = int(w["cu_seqlens"][-1])
    est = T3 / (n / t_pre) + 384 / (r / t_dec)  # seconds the oracle would need for the whole mixed step
    return {"value": round((T3 + 384) / est, 2), "unit": "tok/s", "kind": "oracle",
            "sample": f"{n} prefill tokens of the first sequence in {t_pre:.1f} s and {r} decode row-steps in "
                      f"{t_dec:.1f} s (fp32 state), scaled to the whole step ({T3} prefill tokens + 384 rows)"}


def cpu_stack_sample(oracle, synth, seconds):
    """The oracle on sampled rows of the 48-layer decode stack: one row of each of the first 8 layers
    (their own seeded parameters, inputs and initial slot), one decode step per call, cycled until
    `seconds` pass; the rate is scaled to tokens/s of the whole 48-layer stack."""
    import numpy as np
    from state_space_model_ssm_amd.configs import NEMOTRON_H_8B as d, NEMOTRON_H_8B_MAMBA_LAYERS as NL
    kw = dict(H=d.nheads, P=d.headdim, N=d.dstate, G=d.ngroups)
    layers = []
    for l in range(8):
        w = synth.stack_layer(d, seed=4, layer=l, concurrency=1, steps=1)
        s_, c_ = synth.stack_slot(d, seed=4, layer=l, slot=0)
        layers.append((w, c_[None].astype(np.float64), s_[None].astype(np.float64)))
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        w, cp, sp = layers[n % len(layers)]
        oracle.decode(w["xbc"][:1], w["dt_raw"][:1], w["params"], [0], cp, sp, **kw)
        n += 1
    el = time.perf_counter() - t0
    return {"value": round(n / el / NL, 3), "unit": "tok/s", "kind": "oracle",
            "sample": f"{n} row-layer decode steps (one row of each of 8 stack layers, cycled) in {el:.1f} s; "
                      f"tokens/s of the stack = row-layer steps/s / {NL} layers"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prefill-steps", type=int, default=50)
    ap.add_argument("--prefill-warmup", type=int, default=10)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-fewer-seqs", action="store_true",
                    help="skip the 1- and 2-sequence prefill timings (keeps per-kernel profiles to one workload)")
    ap.add_argument("--no-multi", action="store_true", help="skip the multi-token decode section")
    ap.add_argument("--no-t1ab", action="store_true", help="skip the chunk-scan vs state-update A/B at T = 1")
    ap.add_argument("--no-mamba1", action="store_true", help="skip the Mamba-1 selective scan section")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-mixed", action="store_true", help="skip the mixed prefill+decode batch")
    ap.add_argument("--no-stack", action="store_true", help="skip the 48-layer decode stack sweep")
    ap.add_argument("--stack-concurrency", default="1,16,64,256,1024")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device-to-device copy (known bytes) for counter calibration")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the hot path runs on a single MI355X "
              f"(asked for --gpus {args.gpus}); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from state_space_model_ssm_amd import binding as B
    from state_space_model_ssm_amd import synth
    from state_space_model_ssm_amd.configs import F32, NEMOTRON_H_8B

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    B.lib()

    def dev(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dt).cuda()

    # ------------------------------------------------------------ decode workload
    d = NEMOTRON_H_8B
    rows, nslots = 256, 512
    log(f"decode workload: {rows} rows, {nslots}-slot bf16 pool; generating inputs")
    w = synth.decode_batch(d, seed=1, rows=rows, num_slots=nslots, with_z=False)
    bf = torch.bfloat16
    ssm = dev(w["ssm_pool"], bf)
    conv = dev(w["conv_pool"], bf)
    xbc, dt = dev(w["xbc"], bf), dev(w["dt_raw"], bf)
    conv_w = dev(w["params"]["conv_w"], torch.float32)
    A_log, dtb, D = (dev(w["params"][k], torch.float32) for k in ("A_log", "dt_bias", "D"))
    idx = torch.from_numpy(w["slots"]).cuda()
    post = torch.empty(rows, d.conv_dim, dtype=bf, device="cuda")
    y = torch.empty(rows, d.d_inner, dtype=bf, device="cuda")
    host_params = w["params"]
    host_tok = {"xbc": w["xbc"][:64].copy(), "dt_raw": w["dt_raw"][:64].copy()}
    host_slots = w["ssm_pool"][w["slots"][:64]].copy(), w["conv_pool"][w["slots"][:64]].copy()
    del w

    def conv_step():
        B.mamba2_conv1d_update(d, xbc, conv_w, None, post, conv, idx)

    def su_step():
        B.mamba2_state_update(d, post, dt, A_log, dtb, D, None, y, ssm, idx)

    def decode_step():
        conv_step()
        su_step()

    settle(decode_step, torch)  # the first GPU work of the run: brings the clocks up
    for _ in range(args.warmup):
        decode_step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} decode steps")
    ms_step = time_region(decode_step, args.steps, torch)
    ms_su = time_region(su_step, args.steps, torch)
    ms_conv = time_region(conv_step, args.steps, torch)
    su_b, cu_b, min_b = decode_bytes_per_row(d, 2)
    su_gbs = su_b * rows / (ms_su * 1e-3) / 1e9
    tok_s = rows / (ms_step * 1e-3)
    log(f"decode: {ms_step * 1e3:.1f} us/step ({tok_s / 1e6:.3f} M tok/s); state_update {ms_su * 1e3:.1f} us "
        f"= {su_gbs:.0f} GB/s; conv_update {ms_conv * 1e3:.1f} us")

    result = {
        "metric": "SSM decode tok/s + % HBM peak; chunk-scan prefill tok/s (Nemotron-H-8B layer)",
        "value": round(tok_s, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded NumPy PCG64; random-init layer parameters)",
        "config": {"workload": "Nemotron-H-8B Mamba-2 layer decode, T=1: 256 sequences from a 512-slot bf16 "
                               "state pool (random-permutation slots), 128 heads x headdim 64 x d_state 128, "
                               "8 groups, conv width 4; step = conv1d_update + state_update",
                   "rows": rows, "pool_slots": nslots, "state_dtype": "bf16", "act_dtype": "bf16"},
        "roofline": {"bound": "hbm", "kernel": "state_update_kernel", "achieved": round(su_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(su_gbs / HBM_PEAK_GBS, 4),
                     "traffic": profiled_traffic("state_update_kernel"), "algorithmic_bytes_per_launch": su_b * rows,
                     "avg_launch_us": round(ms_su * 1e3, 2),
                     "rocprof_check": rocprof_check("state_update_kernel", su_b * rows)},
        "decode_detail": {"us_per_step": round(ms_step * 1e3, 2), "state_update_us": round(ms_su * 1e3, 2),
                          "conv_update_us": round(ms_conv * 1e3, 2),
                          "step_algorithmic_bytes": min_b * rows,
                          "step_hbm_frac": round(min_b * rows / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    # ------------------------------------------------------------ the vllm.cpp page's A/B at T = 1
    # The same 256 rows, slots and pools through the chunk-scan arm: each row a one-token
    # sequence of conv1d_fwd + chunk_scan_fwd (has_initial_state = 1, final states written
    # back in place), without and with the scan's optional workspace.
    if not args.no_t1ab:
        t1_ab(args, result, torch, B, d, rows, xbc, conv_w, post, conv, idx, dt, A_log, dtb, D, y, ssm, decode_step)
    del ssm, conv, xbc, dt, post, y
    torch.cuda.empty_cache()

    # ------------------------------------------------------------ multi-token decode (drafted tokens)
    if not args.no_multi:
        Tm, rows_m = 4, 256
        nsl = rows_m * (Tm + 1)
        log(f"multi-token decode workload: {rows_m} rows x {Tm} tokens, bf16 pool of {nsl} slots")
        rng = np.random.Generator(np.random.PCG64(5))
        pm = synth.layer_params(d, rng)
        tm = synth.tokens(d, rng, rows_m * Tm, with_z=False)
        ssm_m = torch.empty(nsl, d.nheads, d.headdim, d.dstate, dtype=bf, device="cuda").normal_(0.0, 0.1 ** 0.5)
        conv_m = torch.empty(nsl, d.conv_width - 1, d.conv_dim, dtype=bf, device="cuda").normal_()
        xm = dev(tm["xbc"].reshape(rows_m, Tm, d.conv_dim), bf)
        dtm = dev(tm["dt_raw"].reshape(rows_m, Tm, d.nheads), bf)
        cwm = dev(pm["conv_w"], torch.float32)
        Am, dtbm, Dm = (dev(pm[k], torch.float32) for k in ("A_log", "dt_bias", "D"))
        srcm = torch.from_numpy(rng.permutation(nsl)[:rows_m].astype(np.int32)).cuda()
        rest = np.setdiff1d(np.arange(nsl), srcm.cpu().numpy())
        dstm = torch.from_numpy(rng.permutation(rest)[:rows_m * Tm].reshape(rows_m, Tm).astype(np.int32)).cuda()
        postm = torch.empty(rows_m, Tm, d.conv_dim, dtype=bf, device="cuda")
        ym = torch.empty(rows_m, Tm, d.d_inner, dtype=bf, device="cuda")
        del tm

        def multi_step(dst):
            B.mamba2_conv1d_update_multi(d, xm, cwm, None, postm, conv_m, srcm, dst)
            B.mamba2_state_update_multi(d, postm, dtm, Am, dtbm, Dm, None, ym, ssm_m, srcm, dst)

        for _ in range(2):
            multi_step(dstm)
            multi_step(None)
        settle(lambda: multi_step(dstm), torch)  # untimed, as for decode: clocks to their sustained state
        ms_snap = time_region(lambda: multi_step(dstm), args.steps, torch)
        settle(lambda: multi_step(None), torch)
        ms_fin = time_region(lambda: multi_step(None), args.steps, torch)
        H, P, N, G, W = d.nheads, d.headdim, d.dstate, d.ngroups, d.conv_width
        cdim = d.conv_dim
        tok_in = cdim * 2 + H * 2 + H * P * 2 + cdim * 2          # raw xBC, dt, y out, post-conv round trip
        state, cstate = H * P * N * 2, (W - 1) * cdim * 2
        b_snap = rows_m * (state + cstate + Tm * (state + cstate) + Tm * tok_in)
        b_fin = rows_m * (2 * (state + cstate) + Tm * tok_in)
        g_snap = b_snap / (ms_snap * 1e-3) / 1e9
        g_fin = b_fin / (ms_fin * 1e-3) / 1e9
        log(f"multi-token decode: every step snapshotted {ms_snap * 1e3:.1f} us ({g_snap:.0f} GB/s), final state "
            f"only {ms_fin * 1e3:.1f} us ({rows_m * Tm / (ms_fin * 1e-3) / 1e6:.2f} M tok/s, {g_fin:.0f} GB/s)")
        result["decode_multi"] = {
            "workload": f"Nemotron-H-8B layer, {rows_m} rows x {Tm} tokens per row (a step verifying drafted "
                        f"tokens), bf16 pools of {nsl} slots; step = conv1d_update_multi + state_update_multi",
            "tokens_per_step": rows_m * Tm,
            "snapshots_every_step": {"ms_per_step": round(ms_snap, 4),
                                     "tok_s": round(rows_m * Tm / (ms_snap * 1e-3), 1),
                                     "roofline": {"bound": "hbm", "achieved": round(g_snap, 1), "peak": HBM_PEAK_GBS,
                                                  "unit": "GB/s", "frac": round(g_snap / HBM_PEAK_GBS, 4),
                                                  "algorithmic_bytes": b_snap}},
            "final_state_only": {"ms_per_step": round(ms_fin, 4), "tok_s": round(rows_m * Tm / (ms_fin * 1e-3), 1),
                                 "roofline": {"bound": "hbm", "achieved": round(g_fin, 1), "peak": HBM_PEAK_GBS,
                                              "unit": "GB/s", "frac": round(g_fin / HBM_PEAK_GBS, 4),
                                              "algorithmic_bytes": b_fin}},
        }
        del ssm_m, conv_m, xm, dtm, postm, ym
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ prefill workload
    if not args.no_prefill:
        d2 = NEMOTRON_H_8B.with_(state_dtype=F32)
        log("prefill workload: 4 x 8192 tokens, chunk 128; generating inputs")
        w2 = synth.prefill_batch(d2, seed=2, seqlens=[8192] * 4, num_slots=8, with_z=False)
        T = int(w2["cu_seqlens"][-1])
        xbc2, dt2 = dev(w2["xbc"], bf), dev(w2["dt_raw"], bf)
        pool2 = torch.zeros(8, d2.nheads, d2.headdim, d2.dstate, device="cuda")
        convp2 = torch.zeros(8, d2.conv_width - 1, d2.conv_dim, device="cuda")
        cw2 = dev(w2["params"]["conv_w"], torch.float32)
        A2, dtb2, D2 = (dev(w2["params"][k], torch.float32) for k in ("A_log", "dt_bias", "D"))
        cu2 = torch.from_numpy(w2["cu_seqlens"]).cuda()
        idx2 = torch.from_numpy(w2["slots"]).cuda()
        hi2 = torch.zeros(4, dtype=torch.uint8, device="cuda")
        post2 = torch.empty(T, d2.conv_dim, dtype=torch.float32, device="cuda")
        y2 = torch.empty(T, d2.d_inner, dtype=bf, device="cuda")
        host_pre = {"xbc": w2["xbc"][:8192].copy(), "dt_raw": w2["dt_raw"][:8192].copy(), "params": w2["params"]}
        del w2

        ws2 = B.prefill_workspace(d2, T)
        # chunk_scan_fwd's workspace has the prefill's layout and size; the calls below never overlap
        assert B.mamba2_chunk_scan_workspace_bytes(d2, T, 4) == ws2.numel()

        def conv_fwd():
            B.mamba2_conv1d_fwd(d2, xbc2, cw2, None, post2, convp2, cu2, idx2, hi2)

        def scan():  # with a workspace: 32-token blocks, B/C planes formed once per group
            B.mamba2_chunk_scan_fwd(d2, post2, dt2, A2, dtb2, D2, None, y2, pool2, cu2, idx2, hi2, ws2)

        def scan_chunks():  # without one: chunks of 128 on chip
            B.mamba2_chunk_scan_fwd(d2, post2, dt2, A2, dtb2, D2, None, y2, pool2, cu2, idx2, hi2)

        def unfused_step():
            conv_fwd()
            scan()

        def prefill_step():  # per-group B/C prep, fused conv(x) + scan, conv cache update
            B.mamba2_prefill_fwd(d2, xbc2, dt2, None, cw2, None, A2, dtb2, D2, y2, pool2, convp2, cu2, idx2, hi2,
                                 ws2)

        for _ in range(args.prefill_warmup):  # untimed
            prefill_step()
        # about 100 ms more untimed: right after 10 warmup steps the clocks are still ramping (the first
        # 20 timed steps measured 7-9 % slower than the next 40 on the same box)
        settle(prefill_step, torch, ms=100.0)
        for _ in range(max(2, args.prefill_warmup // 2)):
            unfused_step()
        torch.cuda.synchronize()
        log(f"timing {args.prefill_steps} prefill steps")
        ms_pre = time_region(prefill_step, args.prefill_steps, torch)
        ms_unf = time_region(unfused_step, args.prefill_steps, torch)
        ms_scan = time_region(scan, args.prefill_steps, torch)
        for _ in range(2):
            scan_chunks()
        ms_chunks = time_region(scan_chunks, args.prefill_steps, torch)
        ms_cf = time_region(conv_fwd, args.prefill_steps, torch)
        # the same call on the first 1 and 2 of the sequences: too few (sequence, head) workgroups to
        # fill the GPU, so each sequence is cut into segments scanned in parallel (segment mode)
        few = {}
        for nb in (() if args.no_fewer_seqs else (1, 2)):
            Tb = 8192 * nb

            def few_step(Tb=Tb, nb=nb):
                B.mamba2_prefill_fwd(d2, xbc2[:Tb], dt2[:Tb], None, cw2, None, A2, dtb2, D2, y2[:Tb], pool2, convp2,
                                     cu2[:nb + 1], idx2[:nb], hi2[:nb], ws2)
            for _ in range(3):
                few_step()
            ms_b = time_region(few_step, args.prefill_steps, torch)
            few[f"{nb}x8192"] = {"ms_per_step": round(ms_b, 4), "tok_s": round(Tb / (ms_b * 1e-3), 1)}
            log(f"prefill {nb} x 8192: {ms_b * 1e3:.1f} us/step ({Tb / (ms_b * 1e-3) / 1e6:.2f} M tok/s)")
        # the layer's gated RMSNorm (y * SiLU(z), normalised over groups of H*P/G channels): the prefill
        # with z and the norm weight, and the norm pass alone on its output
        zgen = torch.Generator(device="cuda")
        zgen.manual_seed(25)
        z2 = torch.empty(T, d2.d_inner, dtype=bf, device="cuda").normal_(0.0, 1.0, generator=zgen)
        nw2 = dev(synth.norm_weight(d2, 25), torch.float32)

        def prefill_norm_step():
            B.mamba2_prefill_fwd(d2, xbc2, dt2, z2, cw2, None, A2, dtb2, D2, y2, pool2, convp2, cu2, idx2, hi2, ws2,
                                 norm_w=nw2)

        def norm_step():  # in place, as mamba2_prefill_fwd applies it
            B.mamba2_gated_rmsnorm(d2, y2, z2, nw2, y2)

        for _ in range(3):
            prefill_norm_step()
        ms_pn = time_region(prefill_norm_step, args.prefill_steps, torch)
        ms_norm = time_region(norm_step, args.prefill_steps, torch)
        norm_bytes = T * d2.d_inner * (2 + 2 + 2) + d2.d_inner * 4  # y and z in, out; the weights once
        norm_gbs = norm_bytes / (ms_norm * 1e-3) / 1e9
        log(f"prefill with the gated norm: {ms_pn * 1e3:.1f} us/step; the norm pass {ms_norm * 1e3:.1f} us "
            f"({norm_gbs:.0f} GB/s)")
        with_norm = {
            "step": "mamba2_prefill_fwd with z and the norm weight (ungated scan, then the gated RMSNorm over "
                    "groups of H*P/G = 1024 channels, in place)",
            "ms_per_step": round(ms_pn, 4), "tok_s": round(T / (ms_pn * 1e-3), 1),
            "norm_us": round(ms_norm * 1e3, 2),
            "norm_roofline": {"bound": "hbm", "kernel": "gated_norm_kernel", "achieved": round(norm_gbs, 1),
                              "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(norm_gbs / HBM_PEAK_GBS, 4),
                              "algorithmic_bytes_per_launch": norm_bytes},
        }
        del z2
        # algorithmic minimum of the whole prefill: raw bf16 xBC + dt in, bf16 y out, final fp32 states;
        # flops of the chunk length each form runs (32-token blocks fused and with a workspace, 128 without)
        pb, pf = scan_algorithmic(d2, T, 4, 2, 2, 4, chunk=32)
        pre_gbs = pb / (ms_pre * 1e-3) / 1e9
        pre_tfs = pf / (ms_pre * 1e-3) / 1e12
        sb, sf = scan_algorithmic(d2, T, 4, 4, 2, 4, chunk=32)
        scan_gbs = sb / (ms_scan * 1e-3) / 1e9
        scan_tfs = sf / (ms_scan * 1e-3) / 1e12
        _, sf128 = scan_algorithmic(d2, T, 4, 4, 2, 4, chunk=128)
        chunks_gbs = sb / (ms_chunks * 1e-3) / 1e9
        chunks_tfs = sf128 / (ms_chunks * 1e-3) / 1e12
        pre_tok_s = T / (ms_pre * 1e-3)
        log(f"prefill (fused): {ms_pre * 1e3:.1f} us/step ({pre_tok_s / 1e6:.2f} M tok/s, {pre_gbs:.0f} GB/s, "
            f"{pre_tfs:.1f} TFLOP/s); unfused {ms_unf * 1e3:.1f} us = conv1d_fwd {ms_cf * 1e3:.1f} + chunk_scan "
            f"{ms_scan * 1e3:.1f} (without a workspace {ms_chunks * 1e3:.1f})")
        result["prefill"] = {
            "value": round(pre_tok_s, 1), "unit": "tok/s", "ms_per_step": round(ms_pre, 4),
            "steps": args.prefill_steps,
            "workload": "Nemotron-H-8B layer prefill: 4 x 8192 tokens (cu_seqlens), bf16 inputs, fp32 state, "
                        "bf16 y, zero initial state, final conv/SSM states to pool slots; layer chunk_size 128; "
                        "step = mamba2_prefill_fwd, whose fused path cuts chunks at 32-token blocks (per-group "
                        "B/C prep kernel + fused conv/scan kernel + conv cache update; flops counted at 32); "
                        "the unfused detail runs conv1d_fwd and chunk_scan_fwd, with a workspace (32-token "
                        "blocks) and without (chunks of 128, flops counted at 128)",
            "roofline": {"bound": "hbm", "kernel": "mamba2_prefill_fwd (whole call)", "achieved": round(pre_gbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(pre_gbs / HBM_PEAK_GBS, 4),
                         "traffic": profiled_traffic("mamba2_prefill_fwd"),
                         "algorithmic_bytes_per_launch": pb, "algorithmic_flops_per_launch": pf,
                         "flops_chunk_length": 32,
                         "mfma_achieved_tflops": round(pre_tfs, 2),
                         "mfma_frac": round(pre_tfs / MFMA_BF16_PEAK_TFLOPS, 4)},
            "fewer_sequences": few,
            "with_gated_norm": with_norm,
            "unfused": {
                "ms_per_step": round(ms_unf, 4), "tok_s": round(T / (ms_unf * 1e-3), 1),
                "step": "conv1d_fwd (fp32 post-conv xBC) + chunk_scan_fwd with a workspace",
                "chunk_scan_us": round(ms_scan * 1e3, 2), "conv1d_fwd_us": round(ms_cf * 1e3, 2),
                "chunk_scan_roofline": {"bound": "mfma", "kernel": "chunk_scan_fwd (whole call: prep + block scan)",
                                        "achieved": round(scan_tfs, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                                        "unit": "TFLOP/s", "frac": round(scan_tfs / MFMA_BF16_PEAK_TFLOPS, 4),
                                        "traffic": profiled_traffic("chunk_scan_fwd"),
                                        "algorithmic_flops_per_launch": sf, "algorithmic_bytes_per_launch": sb,
                                        "hbm_achieved_gbs": round(scan_gbs, 1),
                                        "hbm_frac": round(scan_gbs / HBM_PEAK_GBS, 4)},
                "chunk_scan_no_workspace_us": round(ms_chunks * 1e3, 2),
                "chunk_scan_no_workspace_roofline": {
                    "bound": "mfma", "kernel": "chunk_scan_fast_kernel", "achieved": round(chunks_tfs, 2),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(chunks_tfs / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": profiled_traffic("chunk_scan_fast_kernel"),
                    "algorithmic_flops_per_launch": sf128, "algorithmic_bytes_per_launch": sb,
                    "hbm_achieved_gbs": round(chunks_gbs, 1), "hbm_frac": round(chunks_gbs / HBM_PEAK_GBS, 4)},
            },
        }
        del xbc2, dt2, pool2, convp2, post2, y2, ws2
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ Mamba-1 selective scan
    if not args.no_mamba1:
        from state_space_model_ssm_amd.configs import MAMBA1_8K
        d1 = MAMBA1_8K
        log("mamba-1 selective scan workload: 4 x 8192 tokens, 8192 channels x 16 states; generating inputs")
        w1 = synth.mamba1_batch(d1, seed=6, seqlens=[8192] * 4, num_slots=4, with_z=False)
        T1 = int(w1["cu_seqlens"][-1])
        u1, dl1 = dev(w1["u"], bf), dev(w1["delta_raw"], bf)
        B1, C1 = dev(w1["B"], bf), dev(w1["C"], bf)
        A1, D1, db1 = dev(w1["A"], torch.float32), dev(w1["D"], torch.float32), dev(w1["delta_bias"], torch.float32)
        pool1 = torch.zeros(4, d1.dim, d1.dstate, device="cuda")
        cu1 = torch.from_numpy(w1["cu_seqlens"]).cuda()
        idx1 = torch.from_numpy(w1["slots"]).cuda()
        y1 = torch.empty(T1, d1.dim, dtype=bf, device="cuda")
        del w1

        def sel_step():
            B.mamba1_selective_scan_fwd(d1, u1, dl1, A1, B1, C1, D1, None, db1, y1, pool1, cu1, idx1, None, True)

        for _ in range(args.prefill_warmup):  # untimed, as for the prefill
            sel_step()
        ms_sel = time_region(sel_step, max(3, args.prefill_steps), torch)
        elems = T1 * d1.dim * d1.dstate
        sel_flops = 6 * elems  # per state element: delta*A, a*h + (delta*u)*B, C.h accumulate
        sel_equiv = sel_flops + EXP_FLOP_EQUIV * elems  # plus the exp2 per state element, in FMA issue slots
        sel_bytes = T1 * (3 * d1.dim * 2 + 2 * d1.ngroups * d1.dstate * 2) + 4 * d1.dim * d1.dstate * 4
        sel_tfs = sel_flops / (ms_sel * 1e-3) / 1e12
        sel_eq_tfs = sel_equiv / (ms_sel * 1e-3) / 1e12
        log(f"mamba-1 selective scan: {ms_sel * 1e3:.1f} us ({T1 / (ms_sel * 1e-3) / 1e6:.2f} M tok/s, "
            f"{sel_tfs:.1f} TFLOP/s, {elems / (ms_sel * 1e-3) / 1e12:.2f} T state updates/s)")
        result["mamba1_scan"] = {
            "workload": "Mamba-1 selective scan: 4 x 8192 tokens (cu_seqlens), 8192 channels x 16 states, 1 B/C "
                        "group, bf16 u/delta/B/C and y, fp32 state, softplus(delta + bias), D skip, zero initial "
                        "state, final states to pool slots",
            "value": round(T1 / (ms_sel * 1e-3), 1), "unit": "tok/s", "ms_per_step": round(ms_sel, 4),
            "roofline": {"bound": "alu", "kernel": "selective_scan_kernel", "achieved": round(sel_eq_tfs, 2),
                         "peak": FP32_VECTOR_UNPACKED_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(sel_eq_tfs / FP32_VECTOR_UNPACKED_TFLOPS, 4),
                         "counting": "6 flops per state update plus its exp2 as 8 flop-equivalents (the issue "
                                     "slots of 4 FMAs), against the fp32 vector peak without packed instructions",
                         "flops_only_tflops": round(sel_tfs, 2),
                         "flops_only_frac_of_published_packed_peak": round(sel_tfs / FP32_VECTOR_PEAK_TFLOPS, 4),
                         "traffic": profiled_traffic("selective_scan_kernel"),
                         "algorithmic_flops_per_launch": sel_flops, "exp_per_launch": elems,
                         "algorithmic_bytes_per_launch": sel_bytes,
                         "hbm_achieved_gbs": round(sel_bytes / (ms_sel * 1e-3) / 1e9, 1)},
        }
        del u1, dl1, B1, C1, y1, pool1
        # one-token update: 256 rows from a 512-slot fp32 pool, in place
        rows1, nsl1 = 256, 512
        wd = synth.mamba1_batch(d1, seed=7, seqlens=[1] * rows1, num_slots=nsl1, with_z=False, initial_state=True)
        ud, dld, Bd1, Cd1 = (dev(wd[k], bf) for k in ("u", "delta_raw", "B", "C"))
        poold = dev(wd["ssm_pool"], torch.float32)
        idxd = torch.from_numpy(wd["slots"]).cuda()
        yd1 = torch.empty(rows1, d1.dim, dtype=bf, device="cuda")
        del wd

        def sel_dec():
            B.mamba1_selective_state_update(d1, ud, dld, A1, Bd1, Cd1, D1, None, db1, yd1, poold, idxd)

        for _ in range(3):
            sel_dec()
        ms_dec = time_region(sel_dec, args.steps, torch)
        dec_bytes = rows1 * (2 * d1.dim * d1.dstate * 4 + 3 * d1.dim * 2 + 2 * d1.ngroups * d1.dstate * 2)
        dec_gbs = dec_bytes / (ms_dec * 1e-3) / 1e9
        log(f"mamba-1 decode: {ms_dec * 1e3:.1f} us for {rows1} rows ({rows1 / (ms_dec * 1e-3) / 1e6:.2f} M tok/s, "
            f"{dec_gbs:.0f} GB/s)")
        result["mamba1_scan"]["decode"] = {
            "workload": f"one token for each of {rows1} rows from a {nsl1}-slot fp32 state pool (8192 x 16 per "
                        "slot), in place; step = mamba1_selective_state_update",
            "us_per_step": round(ms_dec * 1e3, 2), "tok_s": round(rows1 / (ms_dec * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": dec_bytes}}
        del ud, dld, Bd1, Cd1, poold, yd1
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ mixed prefill + decode batch
    if not args.no_mixed:
        d3 = NEMOTRON_H_8B.with_(state_dtype=F32)
        log("mixed workload: 8 prefill sequences U[256,4096] + 384 decode rows, 1024-slot fp32 pool")
        w3 = synth.mixed_batch(d3, seed=3, num_prefill=8, len_lo=256, len_hi=4096, decode_rows=384, num_slots=1024)
        T3 = int(w3["cu_seqlens"][-1])
        rows3 = T3 + 384
        xbc3 = dev(np.concatenate([w3["prefill"]["xbc"], w3["decode"]["xbc"]]), bf)
        dt3 = dev(np.concatenate([w3["prefill"]["dt_raw"], w3["decode"]["dt_raw"]]), bf)
        ssm3 = dev(w3["ssm_pool"], torch.float32)
        conv3 = dev(w3["conv_pool"], torch.float32)
        cw3 = dev(w3["params"]["conv_w"], torch.float32)
        A3, dtb3, D3 = (dev(w3["params"][k], torch.float32) for k in ("A_log", "dt_bias", "D"))
        cu3 = torch.from_numpy(w3["cu_seqlens"]).cuda()
        pidx3 = torch.from_numpy(w3["prefill_slots"]).cuda()
        didx3 = torch.from_numpy(w3["decode_slots"]).cuda()
        hi3 = torch.from_numpy(w3["has_initial_state"]).cuda()
        post3 = torch.empty(rows3, d3.conv_dim, dtype=torch.float32, device="cuda")
        y3 = torch.empty(rows3, d3.d_inner, dtype=bf, device="cuda")
        ws3 = B.prefill_workspace(d3, T3)  # prefill segment through mamba2_prefill_fwd
        del w3

        def mixed_step():
            B.mamba2_mixed_fwd(d3, xbc3, dt3, None, cw3, None, A3, dtb3, D3, post3, y3, ssm3, conv3, cu3, pidx3, hi3,
                               didx3, ws3)

        # the split iteration: the prefill segment eagerly, the 384 decode rows as one replay of a
        # captured decode graph over the same buffers
        graph3 = B.DecodeGraph(d3, [{"xbc": xbc3[T3:], "conv_w": cw3, "conv_b": None, "xbc_post": post3[T3:],
                                     "conv_pool": conv3, "dt_raw": dt3[T3:], "A_log": A3, "dt_bias": dtb3, "D": D3,
                                     "z": None, "y": y3[T3:], "ssm_pool": ssm3, "state_indices": didx3}])

        def split_step():
            B.mamba2_prefill_fwd(d3, xbc3[:T3], dt3[:T3], None, cw3, None, A3, dtb3, D3, y3[:T3], ssm3, conv3, cu3,
                                 pidx3, hi3, ws3)
            graph3.launch()

        def prefill_part():
            B.mamba2_prefill_fwd(d3, xbc3[:T3], dt3[:T3], None, cw3, None, A3, dtb3, D3, y3[:T3], ssm3, conv3, cu3,
                                 pidx3, hi3, ws3)

        for _ in range(args.prefill_warmup):  # untimed, as for the prefill
            mixed_step()
            split_step()
        ms_mix = time_region(mixed_step, max(3, args.prefill_steps), torch)
        ms_split = time_region(split_step, max(3, args.prefill_steps), torch)
        ms_mix_pre = time_region(prefill_part, max(3, args.prefill_steps), torch)
        ms_mix_dec = time_region(graph3.launch, max(3, args.prefill_steps), torch)
        graph3.close()
        dec_b = 384 * decode_bytes_per_row(d3, 4)[2]
        pre_b, _ = scan_algorithmic(d3, T3, 8, 2, 2, 4)
        result["mixed"] = {
            "workload": f"one Nemotron-H-8B layer: 8 prefill sequences ({T3} tokens, lengths U[256,4096], "
                        "cu_seqlens) + 384 decode rows, 1024-slot fp32 state pool; step = mamba2_mixed_fwd "
                        "(prefill segment through the fused mamba2_prefill_fwd)",
            "value": round(rows3 / (ms_mix * 1e-3), 1), "unit": "tok/s", "ms_per_step": round(ms_mix, 4),
            "prefill_tokens": T3, "decode_rows": 384,
            "algorithmic_bytes": int(dec_b + pre_b),
            "hbm_frac": round((dec_b + pre_b) / (ms_mix * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "split": {"step": "mamba2_prefill_fwd on the prefill segment (eager) + one replay of the decode rows' "
                              "captured graph (mamba2_decode_graph_launch)",
                      "ms_per_step": round(ms_split, 4), "tok_s": round(rows3 / (ms_split * 1e-3), 1),
                      "hbm_frac": round((dec_b + pre_b) / (ms_split * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "prefill_part_ms": round(ms_mix_pre, 4), "decode_graph_ms": round(ms_mix_dec, 4),
                      "decode_graph_hbm_frac": round(dec_b / (ms_mix_dec * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
        log(f"mixed: {ms_mix * 1e3:.1f} us/step eager, {ms_split * 1e3:.1f} us split ({rows3} rows; prefill "
            f"{ms_mix_pre * 1e3:.1f} + decode graph {ms_mix_dec * 1e3:.1f})")
        del xbc3, dt3, ssm3, conv3, post3, y3, ws3
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ 48-layer decode stack
    if not args.no_stack:
        result["stack"] = bench_stack(args, torch, np, B, synth, NEMOTRON_H_8B, dev, bf, time_region)

    # ------------------------------------------------------------ CPU baseline (oracle)
    if not args.no_cpu_baseline:
        cores = int(os.environ.get("OMP_NUM_THREADS") or len(os.sched_getaffinity(0)))
        os.environ.setdefault("OMP_NUM_THREADS", str(cores))
        import oracle
        kw = dict(H=d.nheads, P=d.headdim, N=d.dstate, G=d.ngroups)
        ssm_h = host_slots[0].astype(np.float64)
        conv_h = host_slots[1].astype(np.float64)
        nrow = ssm_h.shape[0]
        t0 = time.perf_counter()
        done = 0
        while time.perf_counter() - t0 < args.cpu_seconds:
            i = done % nrow  # cycle over the sampled rows; each call is one full layer step of one row
            oracle.decode(host_tok["xbc"][i:i + 1], host_tok["dt_raw"][i:i + 1], host_params, [0],
                          conv_h[i:i + 1], ssm_h[i:i + 1], **kw)
            done += 1
        el = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(done / el, 2), "unit": "tok/s", "cores": cores, "kind": "oracle",
                                  "sample": f"{done} decode row-steps (cycling over {nrow} of the 256 rows, all 128 "
                                            f"heads each) through the fp64 C oracle in {el:.1f} s",
                                  "cpu_model": cpu_model(), "host_threads_visible": len(os.sched_getaffinity(0))}
        log(f"cpu baseline: {done} rows in {el:.1f} s on {cores} threads")
        result["cpu_baseline"]["single_thread"] = single_thread_oracle(args.cpu_seconds / 3)
        result["cpu_baseline"]["mixed"] = cpu_mixed_sample(oracle, synth, args.cpu_seconds / 2)
        result["cpu_baseline"]["stack"] = cpu_stack_sample(oracle, synth, args.cpu_seconds / 2)
        if not args.no_prefill:
            t0 = time.perf_counter()
            n = 0
            T1 = host_pre["xbc"].shape[0]
            cs = np.zeros((d.conv_width - 1, d.conv_dim))
            hs = np.zeros((d.nheads, d.headdim, d.dstate))
            while n < T1 and time.perf_counter() - t0 < args.cpu_seconds:
                _, _, cs, hs = oracle.layer_seq(host_pre["xbc"][n:n + 64], host_pre["dt_raw"][n:n + 64],
                                                host_pre["params"], cs, hs, **kw)
                n += 64
            el = time.perf_counter() - t0
            result["prefill"]["cpu_baseline"] = {
                "value": round(n / el, 2), "unit": "tok/s", "cores": cores, "kind": "oracle",
                "sample": f"first {n} tokens of one 8192-token sequence (all 128 heads) through the fp64 C oracle "
                          f"in {el:.1f} s"}

    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        src.fill_(1.0)
        torch.cuda.synchronize()
        ms_copy = time_region(lambda: dst.copy_(src), 5, torch)
        result["copy_calibration"] = {"bytes_read": 1 << 30, "bytes_written": 1 << 30, "launches": 5,
                                      "gbs": round(2 * (1 << 30) / (ms_copy * 1e-3) / 1e9, 1)}
        del src, dst

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
