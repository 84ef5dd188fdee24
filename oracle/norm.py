"""fp64 gated RMSNorm of the mixer output (TEST INFRASTRUCTURE ONLY).

Source: the "Nemotron-H-8B-Base-8K" record lists ``norm`` among the Mamba-2
mixer tensors (section on the safetensors index). The pages give no formula;
the reading used by the library and by this oracle:

    g = y * SiLU(z)            (g = y when there is no z; SiLU(v) = v / (1 + e^-v))
    out[c] = w[c] * g[c] / sqrt(mean of g^2 over c's group + eps)

with groups of ``group`` consecutive channels of a row (by default H*P/G, the
channels of the H/G heads that share one B/C group).

Written as the definition, one row and one group at a time, in fp64.
"""
from __future__ import annotations

import numpy as np


def gated_rmsnorm(y, z, w, eps: float, group: int):
    """y [rows, width]; z [rows, width] or None; w [width]. Returns fp64 [rows, width]."""
    y = np.asarray(y, dtype=np.float64)
    rows, width = y.shape
    w = np.asarray(w, dtype=np.float64).reshape(width)
    assert group > 0 and width % group == 0
    zz = None if z is None else np.asarray(z, dtype=np.float64).reshape(rows, width)
    out = np.empty((rows, width), dtype=np.float64)
    for r in range(rows):
        g = y[r].copy()
        if zz is not None:
            g = g * (zz[r] / (1.0 + np.exp(-zz[r])))
        for c0 in range(0, width, group):
            seg = g[c0:c0 + group]
            ms = np.sum(seg * seg) / group
            out[r, c0:c0 + group] = w[c0:c0 + group] * seg / np.sqrt(ms + eps)
    return out
