#!/usr/bin/env python3
"""Kernel profiles of bench.py's workloads with rocprofv3, summarised as the Markdown files
under profiles/ that bench.py reads back (per-kernel durations, counter-measured HBM bytes and
the `traffic-json` records behind `roofline.traffic`).

    python profile_report.py run [--out DIR] [--passes ktrace,fetch,write,issue]
        on a machine with the GPU: the rocprofv3 passes, each over one bench.py run, into DIR
        (default gpurun_out/prof, relative to the repository root)
    python profile_report.py render [--out DIR]
        reads the passes' result databases from DIR and writes profiles/*.md

Counter calibration: FETCH_SIZE and WRITE_SIZE are in KiB per dispatch; each is scaled by
(known bytes / counted bytes) of a plain 1 GiB device-to-device copy that bench.py's
--copy-calibration makes in the same run, so the figures are bytes as a plain copy counts them.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sqlite3
import statistics
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "state_space_model_ssm_amd", "csrc")

# bench.py runs that the passes profile: every section whose kernels are distinct instantiations
# (the mixed batch, the stack, the 1- and 2-sequence prefills and the T = 1 A/B reuse the same
# kernels on other shapes and would blend into their averages)
SKIP = ["--no-cpu-baseline", "--no-mixed", "--no-stack", "--no-fewer-seqs", "--no-t1ab"]
LONG = ["--steps", "20", "--warmup", "3", "--prefill-steps", "3"] + SKIP
SHORT = ["--steps", "3", "--warmup", "1", "--prefill-steps", "2"] + SKIP + ["--copy-calibration"]
ISSUE_COUNTERS = ["SQ_WAVES", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_SALU",
                  "SQ_INSTS_LDS", "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_BUSY_CYCLES"]
PASSES = {
    "ktrace": (["--kernel-trace", "--stats"], LONG),
    "fetch": (["--pmc", "FETCH_SIZE"], SHORT),
    "write": (["--pmc", "WRITE_SIZE"], SHORT),
    "issue": (["--pmc"] + ISSUE_COUNTERS, ["--steps", "3", "--warmup", "1", "--prefill-steps", "2"] + SKIP),
}
CALIB_KERNEL = "copyBuffer"
# the instantiations of the fused prefill (raw bf16 input, conv width 4, fp32 state) and of the
# block form of chunk_scan_fwd (post-conv fp32 input, conv width 1), as mangled names and as the
# profiler demangles them
FUSED_SCAN = ("fused_scan_kernelILi32ELi4EfDF16b", "fused_scan_kernel<32, 4, float")
FUSED_PREP = ("fused_prep_kernelIDF16bfLi4ELi32E", "fused_prep_kernel<bool _Accum, 4, 32>")
BLOCK_SCAN = ("fused_scan_kernelILi32ELi1Ef", "fused_scan_kernel<32, 1, float")
BLOCK_PREP = ("fused_prep_kernelIffLi1ELi32E", "fused_prep_kernel<float, float, 1, 32>")
CALIB_BYTES = 1 << 30


def pass_command(name, out):
    prof, bench_args = PASSES[name]
    return ["rocprofv3", *prof, "-d", os.path.join(out, name), "-o", "bench", "--", sys.executable,
            os.path.join(ROOT, "bench.py"), *bench_args]


def shown_command(name):
    """The pass's command as recorded in a profile (paths relative to the repository root R)."""
    prof, bench_args = PASSES[name]
    return (f"cd /tmp && export TMPDIR=/tmp && R=/root/repo  # the repository root\n"
            f"timeout -s KILL 300 rocprofv3 {' '.join(prof)} -d $R/gpurun_out/prof/{name} -o bench -- "
            f"python3 $R/bench.py {' '.join(bench_args)}")


def run(out, passes):
    os.makedirs(out, exist_ok=True)
    env = dict(os.environ, TMPDIR="/tmp")
    for name in passes:
        cmd = pass_command(name, out)
        print(f"[profile] pass {name}: {' '.join(cmd)}", flush=True)
        r = subprocess.run(["timeout", "-s", "KILL", "300", *cmd], cwd="/tmp", env=env)
        # rocprofv3 can end with a segmentation fault after the program has finished and the
        # results are written; the program's own status is in the log, so only a kill stops here
        if r.returncode in (124, 137, -9):
            raise SystemExit(f"pass {name} was killed at its time limit")
        print(f"[profile] pass {name} ended with status {r.returncode}", flush=True)


# ------------------------------------------------------------------ reading the databases

def _db(out, name):
    found = sorted(glob.glob(os.path.join(out, name, "**", "*results.db"), recursive=True))
    if not found:
        raise SystemExit(f"no results database under {os.path.join(out, name)}")
    return found[-1]


def kernel_stats(db):
    con = sqlite3.connect(db)
    agg = {}
    for name, dur in con.execute("select name, end - start from kernels"):
        agg.setdefault(name, []).append(dur)
    out = {}
    for name, d in agg.items():
        d = sorted(d)
        out[name] = {"calls": len(d), "avg_us": statistics.mean(d) / 1e3, "p50_us": d[len(d) // 2] / 1e3,
                     "p99_us": d[min(len(d) - 1, int(0.99 * len(d)))] / 1e3, "min_us": d[0] / 1e3,
                     "max_us": d[-1] / 1e3}
    return out


def counter_avgs(db, counter):
    con = sqlite3.connect(db)
    agg = {}
    for k, v in con.execute("select kernel_name, value from counters_collection where counter_name = ?",
                            (counter,)):
        agg.setdefault(k, []).append(v)
    return {k: (statistics.mean(v), len(v), max(v)) for k, v in agg.items()}


def calibrated(db, counter):
    """{kernel: bytes per dispatch} for FETCH_SIZE or WRITE_SIZE, scaled by the copy calibration."""
    vals = counter_avgs(db, counter)
    calib = [mx for k, (_, _, mx) in vals.items() if CALIB_KERNEL in k]
    if not calib:
        raise SystemExit(f"no {CALIB_KERNEL} dispatch in {db}: run the pass with --copy-calibration")
    factor = CALIB_BYTES / (max(calib) * 1024.0)
    return {k: avg * 1024.0 * factor for k, (avg, _, _) in vals.items()}, factor


def matches(name, frag):
    """A kernel name (mangled, or demangled by the profiler) against a fragment or a tuple of
    alternative fragments."""
    return any(f in name for f in ((frag,) if isinstance(frag, str) else frag))


def pick(table, frag):
    """The one entry of `table` whose kernel name matches `frag` (a distinct instantiation)."""
    hits = [k for k in table if matches(k, frag)]
    if len(hits) != 1:
        raise SystemExit(f"{len(hits)} kernels match {frag!r}: {hits}")
    return hits[0]


def src_sha(sources):
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ what each profile covers

def profiles():
    """Profile files: kernels shown (name fragment, algorithmic bytes per dispatch) and the
    traffic records bench.py reads (record name, kernel fragments summed, sources)."""
    sys.path.insert(0, ROOT)
    import bench
    from state_space_model_ssm_amd.configs import F32, MAMBA1_8K, NEMOTRON_H_8B
    d = NEMOTRON_H_8B
    d2 = d.with_(state_dtype=F32)
    H, P, N, G = d.nheads, d.headdim, d.dstate, d.ngroups
    cdim = d.conv_dim
    su_b, cu_b, _ = bench.decode_bytes_per_row(d, 2)
    T = 4 * 8192
    prep_b = T * (2 * G * N * 2 + G * N * 2 + 2 * G * N * 2 + G * 32 * 4)
    scan_b = T * (H * P * 2 + H * 2 + H * P * 2) + 4 * H * P * N * 4
    pre_b, _ = bench.scan_algorithmic(d2, T, 4, 2, 2, 4)
    blk_b, _ = bench.scan_algorithmic(d2, T, 4, 4, 2, 4)
    rows_m, Tm = 256, 4
    state = H * P * N * 2
    multi_tok = cdim * 2 + H * 2 + H * P * 2
    d1 = MAMBA1_8K
    sel_b = T * (3 * d1.dim * 2 + 2 * d1.ngroups * d1.dstate * 2) + 4 * d1.dim * d1.dstate * 4
    dec = ["decode.hip", "common.hpp"]
    fus = ["fused.hip", "common.hpp", "mfma.hpp"]
    return [
        {"file": "state_update_decode-8b.md",
         "title": "state_update_kernel / conv_update_kernel - decode-8b (256 rows, 512-slot bf16 pool, "
                  "Nemotron-H-8B layer)",
         "kernels": [("state_update_kernel", su_b * 256), ("conv_update_kernel", cu_b * 256)],
         "records": [("state_update_kernel", ["state_update_kernel"], dec)]},
        {"file": "prefill_scan_prefill-8b.md",
         "title": "mamba2_prefill_fwd and the unfused prefill - prefill-8b (4 x 8192 tokens, bf16 inputs "
                  "and y, fp32 state)",
         "note": "mamba2_prefill_fwd = fused_prep_kernel (B/C conv once per group into per-block planes) + "
                 "fused_scan_kernel (conv of x inside the scan) + conv_state_kernel; the unfused detail is "
                 "conv_fwd_kernel + conv_state_kernel, then chunk_scan_fwd with a workspace (the prep and scan "
                 "kernels instantiated with conv width 1) or without (chunk_scan_fast_kernel). "
                 "conv_state_kernel rows include both conv paths' launches. gated_norm_kernel is the layer's "
                 "gated RMSNorm (y * SiLU(z) over groups of 1024 channels) that mamba2_prefill_fwd runs after "
                 "the scan when given the norm weight.",
         "kernels": [(FUSED_SCAN, scan_b), (FUSED_PREP, prep_b), (BLOCK_SCAN, None), (BLOCK_PREP, None),
                     ("chunk_scan_fast_kernel", blk_b), ("conv_fwd_kernel", T * cdim * (2 + 4)),
                     ("conv_state_kernel", None), ("gated_norm_kernel", T * H * P * (2 + 2 + 2) + H * P * 4)],
         "records": [("mamba2_prefill_fwd", [FUSED_SCAN, FUSED_PREP], fus + ["conv.hip"]),
                     ("chunk_scan_fwd", [BLOCK_SCAN, BLOCK_PREP], fus),
                     ("chunk_scan_fast_kernel", ["chunk_scan_fast_kernel"], ["scan.hip", "common.hpp",
                                                                           "mfma.hpp"])],
         "algorithmic": {"mamba2_prefill_fwd": pre_b, "chunk_scan_fwd": blk_b}},
        {"file": "state_update_multi_decode-multi-8b.md",
         "title": "state_update_multi_kernel / conv_update_multi_kernel - decode-multi-8b (256 rows x 4 tokens, "
                  "bf16 pools of 1280 slots)",
         "note": "The snapshot form (a destination slot after every token) and the final-state form are two "
                 "instantiations of the state kernel (the one with consecutive p-rows per lane group, `Lb1E`, "
                 "is the final-state form).",
         "kernels": [("state_update_multi_kernelIDF16bDF16bDF16bLi128ELi4ELb0E",
                      rows_m * (state + Tm * state + Tm * multi_tok)),
                     ("state_update_multi_kernelIDF16bDF16bDF16bLi128ELi4ELb1E",
                      rows_m * (2 * state + Tm * multi_tok)),
                     ("conv_update_multi_kernel", None)],
         "records": []},
        {"file": "selective_scan_mamba1-8k.md",
         "title": "selective_scan_kernel / selective_update_kernel - mamba1-8k (4 x 8192 tokens x 8192 "
                  "channels x 16 states; 256 decode rows)",
         "kernels": [("selective_scan_kernel", sel_b), ("selective_update_kernel", None)],
         "records": [("selective_scan_kernel", ["selective_scan_kernel"], ["selective.hip", "common.hpp"])]},
    ]


def _short(name, n=110):
    name = name.replace("\n", " ")
    return name if len(name) <= n else name[: n - 3] + "..."


def render(out):
    ks = kernel_stats(_db(out, "ktrace"))
    fetch, ff = calibrated(_db(out, "fetch"), "FETCH_SIZE")
    write, wf = calibrated(_db(out, "write"), "WRITE_SIZE")
    for prof in profiles():
        lines = [f"# {prof['title']}", ""]
        if prof.get("note"):
            lines += [prof["note"], ""]
        lines += ["Kernel durations (rocprofv3 kernel trace; the profiler adds per-dispatch overhead, so averages",
                  "here can sit above the HIP-event figures bench.py reports):", "", "```",
                  shown_command("ktrace"), "```", "",
                  "| kernel | calls | avg us | p50 us | p99 us | min us | max us |", "|---|---|---|---|---|---|---|"]
        for frag, _ in prof["kernels"]:
            for k in sorted(k for k in ks if matches(k, frag)):
                r = ks[k]
                lines.append(f"| {_short(k)} | {r['calls']} | {r['avg_us']:.1f} | {r['p50_us']:.1f} | "
                             f"{r['p99_us']:.1f} | {r['min_us']:.1f} | {r['max_us']:.1f} |")
        lines += ["", "HBM bytes per dispatch (FETCH_SIZE and WRITE_SIZE, each scaled by what the same counter reads "
                  "for a 1 GiB device copy in the same run):", "", "```", shown_command("fetch"),
                  shown_command("write").split("\n")[1], "```", "",
                  f"Calibration factors: FETCH_SIZE x {ff:.4f}, WRITE_SIZE x {wf:.4f}.", "",
                  "| kernel | fetch MB | write MB | total MB | algorithmic MB | traffic / algorithmic |",
                  "|---|---|---|---|---|---|"]
        for frag, alg in prof["kernels"]:
            for k in sorted(k for k in fetch if matches(k, frag)):
                f_, w_ = fetch.get(k, 0.0), write.get(k, 0.0)
                ratio = f"{(f_ + w_) / alg:.2f}" if alg else ""
                algs = f"{alg / 1e6:.1f}" if alg else ""
                lines.append(f"| {_short(k)} | {f_ / 1e6:.1f} | {w_ / 1e6:.1f} | {(f_ + w_) / 1e6:.1f} | {algs} | "
                             f"{ratio} |")
        lines.append("")
        for rec, frags, sources in prof["records"]:
            names = [pick(fetch, f) for f in frags]
            tnames = [pick(ks, f) for f in frags]
            fb = sum(fetch[n] for n in names)
            wb = sum(write.get(n, 0.0) for n in names)
            entry = {"kernel": rec, "bytes_per_launch": int(fb + wb), "fetch": int(fb), "write": int(wb),
                     "avg_us": round(sum(ks[n]["avg_us"] for n in tnames), 2),
                     "src_sha": src_sha(sources), "sources": sources}
            alg = prof.get("algorithmic", {}).get(rec)
            if alg:
                lines.append(f"{rec}: {int(fb + wb) / 1e6:.1f} MB moved per call against {alg / 1e6:.1f} MB "
                             f"algorithmic ({(fb + wb) / alg:.2f}x).")
            lines.append(f"traffic-json: {json.dumps(entry)}")
        path = os.path.join(ROOT, "profiles", prof["file"])
        open(path, "w").write("\n".join(lines).rstrip() + "\n")
        print(f"wrote {path}")
    render_issue(out, ks)


def render_issue(out, ks):
    """SQ counters of the fused prefill scan: instruction mix per wave and 32-token block."""
    dbs = glob.glob(os.path.join(out, "issue", "**", "*results.db"), recursive=True)
    if not dbs:
        return
    db = sorted(dbs)[-1]
    frag = FUSED_SCAN
    vals = {c: counter_avgs(db, c) for c in ISSUE_COUNTERS}
    key = pick(vals["SQ_WAVES"], frag)
    waves = vals["SQ_WAVES"][key][0]
    blocks_per_wave = 8192 // 32
    dur = ks[pick(ks, frag)]["avg_us"]
    lines = ["# fused_scan_kernel - instruction mix and pipe use, prefill-8b via mamba2_prefill_fwd (4 x 8192 "
             "tokens)", "", "One rocprofv3 pass with eight SQ counters (the most one pass may hold):", "", "```",
             shown_command("issue"), "```", "",
             "| counter | per dispatch | per wave and 32-token block |", "|---|---|---|"]
    for c in ISSUE_COUNTERS:
        v = vals[c][pick(vals[c], frag)][0]
        per = "" if c in ("SQ_WAVES", "SQ_BUSY_CU_CYCLES") else f"{v / waves / blocks_per_wave:.1f}"
        lines.append(f"| {c} | {v:.0f} | {per} |")
    mfma_busy = vals["SQ_VALU_MFMA_BUSY_CYCLES"][pick(vals["SQ_VALU_MFMA_BUSY_CYCLES"], frag)][0]
    valu = vals["SQ_INSTS_VALU"][pick(vals["SQ_INSTS_VALU"], frag)][0]
    cycles = dur * 1e-6 * 2.4e9
    lines += ["", f"Against the kernel's average duration in the kernel trace ({dur:.1f} us, about "
                  f"{cycles / 1e6:.2f} M cycles at 2.4 GHz) over 1,024 SIMDs: MFMA busy "
                  f"{mfma_busy / 1024 / cycles * 100:.0f} % of the cycles; VALU issue (4 cycles per wave "
                  f"instruction) {valu * 4 / 1024 / cycles * 100:.0f} %.", ""]
    path = os.path.join(ROOT, "profiles", "fused_scan_issue_prefill-8b.md")
    open(path, "w").write("\n".join(lines))
    print(f"wrote {path}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", choices=["run", "render"])
    ap.add_argument("--out", default=os.path.join(ROOT, "gpurun_out", "prof"))
    ap.add_argument("--passes", default="ktrace,fetch,write,issue")
    a = ap.parse_args()
    if a.mode == "run":
        run(a.out, [p for p in a.passes.split(",") if p])
    else:
        render(a.out)


if __name__ == "__main__":
    main()
