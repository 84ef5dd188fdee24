"""Quadratic ("dual", attention-like) form of the selective recurrence, fp64 NumPy.

TEST INFRASTRUCTURE ONLY -- a second formulation used to pin the sequential
C loop on small inputs. It never loops over time: for each head it builds the
T x T causal matrix

    L[t, s] = exp(A * (cum_t - cum_s)) * dt_s   for s <= t, else 0,
    cum_t   = sum_{r <= t} dt_r,

and writes every output as one matrix expression:

    y  = ((C B^T) * L) x + exp(A cum) * (C h0^T) + D x
    hT = exp(A cum_T) h0 + x^T diag(exp(A (cum_T - cum)) dt) B

Unrolling h_t = a_t h_{t-1} + dt_t x_t B_t^T gives exactly this sum, since the
product of the decays a_{s+1} ... a_t is exp(A (cum_t - cum_s)). It uses
NumPy's logaddexp for softplus, so it shares no scalar routine with the C loop.
"""
from __future__ import annotations

import numpy as np


def ssm_dual(xbc_post, dt_raw, A_log, dt_bias, D, h0, *, H, P, N, G, z=None):
    """Same signature and outputs as ``oracle.ssm_seq`` (y [T, H*P], hT [H, P, N])."""
    xbc_post = np.asarray(xbc_post, dtype=np.float64)
    T = xbc_post.shape[0]
    hpg = H // G
    X = xbc_post[:, : H * P].reshape(T, H, P)
    Bm = xbc_post[:, H * P: H * P + G * N].reshape(T, G, N)
    Cm = xbc_post[:, H * P + G * N:].reshape(T, G, N)
    dt = np.logaddexp(0.0, np.asarray(dt_raw, np.float64).reshape(T, H) + np.asarray(dt_bias, np.float64))
    A = -np.exp(np.asarray(A_log, np.float64))
    h0 = np.asarray(h0, np.float64).reshape(H, P, N)
    y = np.zeros((T, H, P))
    hT = np.zeros((H, P, N))
    causal = np.tril(np.ones((T, T), dtype=bool))
    for h in range(H):
        g = h // hpg
        cum = np.cumsum(dt[:, h])
        diff = cum[:, None] - cum[None, :]
        L = np.where(causal, np.exp(A[h] * np.where(causal, diff, 0.0)), 0.0) * dt[None, :, h]
        CB = Cm[:, g, :] @ Bm[:, g, :].T
        y[:, h, :] = (CB * L) @ X[:, h, :]
        y[:, h, :] += np.exp(A[h] * cum)[:, None] * (Cm[:, g, :] @ h0[h].T)
        y[:, h, :] += np.asarray(D, np.float64)[h] * X[:, h, :]
        w = np.exp(A[h] * (cum[-1] - cum)) * dt[:, h]
        hT[h] = np.exp(A[h] * cum[-1]) * h0[h] + X[:, h, :].T @ (w[:, None] * Bm[:, g, :])
    y = y.reshape(T, H * P)
    if z is not None:
        zz = np.asarray(z, np.float64).reshape(T, H * P)
        y = y * (zz / (1.0 + np.exp(-zz)))
    return y, hT
