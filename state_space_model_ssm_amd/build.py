"""Build libmamba2.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

    python -m state_space_model_ssm_amd.build

Every source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled (`-packed-fp32-ops`), then linked into one shared library
next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmamba2.so")
SOURCES = ["api.cpp", "decode.hip", "conv.hip", "scan.hip", "fused.hip", "norm.hip", "selective.hip",
           "static_scratch.hip", "graph.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the gfx950 library)")


def common_flags() -> list:
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(os.path.dirname(HERE), "include"), "-Wno-unused-command-line-argument"]


def build(verbose: bool = False) -> str:
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="mamba2_build_")
    try:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            cmd = [cc, *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
            if src.endswith(".cpp"):
                cmd[1:1] = ["-x", "hip"]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            text = out.decode(errors="replace")
            # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
            lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
            if p.returncode != 0:
                failed.append(src)
                print("\n".join(lines), file=sys.stderr)
            elif verbose and lines:
                print("\n".join(lines))
        if failed:
            raise RuntimeError(f"hipcc failed for {failed}")
        out_tmp = LIB + f".tmp{os.getpid()}"
        subprocess.run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp], check=True)
        os.replace(out_tmp, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
