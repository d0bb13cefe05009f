"""Closed forms of attention for special inputs (float64, CPU).

These are derived by hand, independently of the oracle, and pin both the
oracle and the GPU path at any size:

* q = 0: every allowed score is 0, so P_ij = 1/n_i over the n_i keys query i
  may see. Then O_i is the mean of those values, lse_i = ln n_i, and
    dK = 0,
    dV_j = sum over queries i that see j of dO_i / n_i,
    dQ_i = scale / n_i * [ (sum_j k_j v_j^T) dO_i - D_i sum_j k_j ],
  sums over the keys i sees, with D_i = dO_i . O_i and scale = 1/sqrt(d).
  For causal attention the sums are prefix sums over the document, so the
  cost is O(N d^2) and the forms reach a million tokens.
* constant v (v_j = c for all j): O_i = c, dQ = dK = 0, dV = P^T dO.
"""

from __future__ import annotations

import math

import numpy as np
import torch


def _cumsum0(x):
    """Prefix sums along axis 0 (float64; torch's CPU kernel is much faster than numpy's here)."""
    return torch.from_numpy(np.array(x, dtype=np.float64, order="C", copy=True)).cumsum(0).numpy()


def _bounds(N, cu):
    if cu is None:
        return [(0, N)]
    cu = [int(x) for x in np.asarray(cu).reshape(-1)]
    return list(zip(cu[:-1], cu[1:]))


def q0_forward(v1, cu=None, causal=True):
    """O [N, d] and lse [N] of one head when q = 0."""
    v = np.asarray(v1, dtype=np.float64)
    N, d = v.shape
    O = np.zeros_like(v)
    lse = np.zeros(N)
    for s, e in _bounds(N, cu):
        L = e - s
        if L == 0:
            continue
        if causal:
            n = np.arange(1, L + 1, dtype=np.float64)
            O[s:e] = _cumsum0(v[s:e]) / n[:, None]
            lse[s:e] = np.log(n)
        else:
            O[s:e] = v[s:e].mean(axis=0)
            lse[s:e] = math.log(L)
    return O, lse


def q0_backward(k1, v1, do1, cu=None, causal=True, block=256):
    """dq, dk, dv [N, d] of one head when q = 0."""
    k = np.asarray(k1, dtype=np.float64)
    v = np.asarray(v1, dtype=np.float64)
    do = np.asarray(do1, dtype=np.float64)
    N, d = k.shape
    scale = 1.0 / math.sqrt(d)
    O, _ = q0_forward(v, cu, causal)
    D = (do * O).sum(axis=1)
    dq = np.zeros_like(k)
    dk = np.zeros_like(k)
    dv = np.zeros_like(k)
    for s, e in _bounds(N, cu):
        L = e - s
        if L == 0:
            continue
        if causal:
            n = np.arange(1, L + 1, dtype=np.float64)
            g = do[s:e] / n[:, None]
            dv[s:e] = _cumsum0(g[::-1])[::-1]
            ksum = _cumsum0(k[s:e])
            M = np.zeros((d, d))  # sum over earlier blocks of k_j v_j^T
            for a in range(0, L, block):
                b = min(L, a + block)
                Kb, Vb, Gb = k[s + a:s + b], v[s + a:s + b], do[s + a:s + b]
                T = np.tril(Gb @ Vb.T)  # T[i, j] = dO_i . v_j for block-local j <= i
                t1 = Gb @ M.T + T @ Kb  # (sum_{j<=i} k_j v_j^T) dO_i
                dq[s + a:s + b] = scale / n[a:b, None] * (t1 - D[s + a:s + b, None] * ksum[a:b])
                M += Kb.T @ Vb
        else:
            dv[s:e] = do[s:e].sum(axis=0) / L
            M = k[s:e].T @ v[s:e]
            t1 = do[s:e] @ M.T
            dq[s:e] = scale / L * (t1 - D[s:e, None] * k[s:e].sum(axis=0)[None])
    return dq, dk, dv
