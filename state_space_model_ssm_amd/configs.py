"""Layer dimensions and the named synthetic workloads.

Nemotron-H-8B dims come from the "Nemotron-H-8B-Base-8K" record, section
"Recurrent state" (ssm_state_size 128, mamba_head_dim 64, mamba_num_heads 128,
n_groups 8; 2 MiB of bf16 state per layer per sequence, 48 Mamba-2 layers).
Conv width 4 and chunk 128 are the Mamba-2 defaults; chunk_size=128 is also
the setting of the vllm.cpp issue's cost table ("Cost, at T=1,
chunk_size=128, nchunks=1").
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

F32 = "f32"
BF16 = "bf16"
DTYPE_BYTES = {F32: 4, BF16: 2}


@dataclass(frozen=True)
class Dims:
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    conv_width: int = 4
    chunk_size: int = 128
    act_dtype: str = BF16    # xBC, dt_raw, z
    state_dtype: str = BF16  # SSM pool and conv pool
    out_dtype: str = BF16    # y
    xbc_dtype: Optional[str] = None  # post-conv xBC; None -> fp32 if state or y is fp32, else act_dtype

    @property
    def post_dtype(self) -> str:
        """Dtype of the post-conv xBC buffer. Rounding post-conv x/B/C to bf16 costs
        ~3e-3 relative accuracy, so it stays fp32 whenever an fp32 result is stored."""
        if self.xbc_dtype is not None:
            return self.xbc_dtype
        return F32 if F32 in (self.state_dtype, self.out_dtype) else self.act_dtype

    @property
    def d_inner(self) -> int:
        return self.nheads * self.headdim

    @property
    def conv_dim(self) -> int:
        return self.nheads * self.headdim + 2 * self.ngroups * self.dstate

    @property
    def heads_per_group(self) -> int:
        return self.nheads // self.ngroups

    def with_(self, **kw) -> "Dims":
        return replace(self, **kw)


#: Tiny single layer, fp32 everywhere (the small case the oracle finishes in milliseconds).
TINY = Dims(nheads=4, headdim=16, dstate=16, ngroups=1, conv_width=4, chunk_size=16,
            act_dtype=F32, state_dtype=F32, out_dtype=F32)

#: One Nemotron-H-8B Mamba-2 layer.
NEMOTRON_H_8B = Dims(nheads=128, headdim=64, dstate=128, ngroups=8, conv_width=4, chunk_size=128)

#: Mamba-2 layers in Nemotron-H-8B (52 layers, 4 of them attention).
NEMOTRON_H_8B_MAMBA_LAYERS = 48


@dataclass(frozen=True)
class Mamba1Dims:
    """Mamba-1 selective scan: ``dim`` channels, ``dstate`` states per channel,
    ``ngroups`` groups sharing B/C (1 in the Mamba paper's layer)."""
    dim: int
    dstate: int
    ngroups: int = 1
    act_dtype: str = BF16
    state_dtype: str = F32
    out_dtype: str = BF16

    def with_(self, **kw) -> "Mamba1Dims":
        return replace(self, **kw)


#: Selective scan with d_inner equal to the Nemotron-H-8B x width (8192) and
#: 16 states per channel, the Mamba paper's default state size.
MAMBA1_8K = Mamba1Dims(dim=8192, dstate=16)


@dataclass(frozen=True)
class Workload:
    name: str
    dims: Dims
    description: str


WORKLOADS = {
    "tiny": Workload("tiny", TINY,
                     "fp32 layer H4 P16 N16 G1 W4 Q16: one 64-token prefill then 8 decode steps, "
                     "4-slot pool, zero initial state"),
    "decode-8b": Workload("decode-8b", NEMOTRON_H_8B,
                          "Nemotron-H-8B layer decode T=1: 256 rows from a 512-slot bf16 pool "
                          "(random permutation slots), state ~ N(0, 0.1)"),
    "prefill-8b": Workload("prefill-8b", NEMOTRON_H_8B.with_(state_dtype=F32),
                           "Nemotron-H-8B layer prefill via chunked SSD: 4 x 8192 tokens, chunk 128, "
                           "bf16 inputs, fp32 state, zero initial state, final states to pool slots"),
    "mixed-8b": Workload("mixed-8b", NEMOTRON_H_8B.with_(state_dtype=F32),
                         "Nemotron-H-8B layer mixed batch: 8 prefill sequences of U[256, 4096] tokens "
                         "packed by cu_seqlens + 384 decode rows, 1024-slot fp32 pool"),
    "stack-8b": Workload("stack-8b", NEMOTRON_H_8B,
                         "48-layer SSM-only decode stack, bf16 state (96 MiB/sequence), "
                         "concurrency 1/16/64/256/1024, 32 steps"),
}
