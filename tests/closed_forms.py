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


# ------------------------------------------------------------------ uniform rows
# When every query is orthogonal to the part of the keys that varies (for
# example q_i = [a_i, 0] and k_j = [c, u_j]), q_i . k_j = q_i . c does not
# depend on j, so each row's scores are equal and P_ij = 1/n_i over the n_i
# keys query i may see, whatever the values. Derived by hand from
# dS_ij = P_ij (dP_ij - D_i), dP_ij = dO_i . v_j, D_i = dO_i . O_i:
#   O_i   = mean of the v_j query i sees      lse_i = scale q_i . c + ln n_i
#   dV_j  = sum_{i sees j} dO_i / n_i
#   dQ_i  = scale / n_i [ (sum_j k_j v_j^T) dO_i - D_i sum_j k_j ]   (the c part cancels)
#   dK_j  = scale sum_{i sees j} (dO_i . v_j - D_i) q_i / n_i
#         = scale [ (sum_i q_i dO_i^T / n_i) v_j - sum_i D_i q_i / n_i ]
# For causal attention the dK sums run over i >= j in the document: suffix
# sums of a d x d matrix and a vector, carried block by block from the end.
# q = 0 is the special case dK = 0.


def _revcumsum0(x):
    return _cumsum0(np.asarray(x)[::-1])[::-1]


def uniform_forward(q1, k1, v1, cu=None, causal=True):
    """O [N, d] and lse [N] of one head whose rows have equal scores (see above)."""
    q = np.asarray(q1, dtype=np.float64)
    k = np.asarray(k1, dtype=np.float64)
    N, d = q.shape
    O, lse = q0_forward(v1, cu, causal)  # uniform P: the same means, lse = ln n_i
    for s, e in _bounds(N, cu):
        if e > s:  # key s is visible to every query of its document
            lse[s:e] += (q[s:e] @ k[s]) / math.sqrt(d)
    return O, lse


def uniform_backward(q1, k1, v1, do1, cu=None, causal=True, block=256):
    """dq, dk, dv [N, d] of one head whose rows have equal scores (see above)."""
    q = np.asarray(q1, dtype=np.float64)
    k = np.asarray(k1, dtype=np.float64)
    v = np.asarray(v1, dtype=np.float64)
    do = np.asarray(do1, dtype=np.float64)
    N, d = q.shape
    scale = 1.0 / math.sqrt(d)
    dq, _, dv = q0_backward(k, v, do, cu, causal, block)  # dQ and dV only depend on P and k
    O, _ = q0_forward(v, cu, causal)
    D = (do * O).sum(axis=1)
    dk = np.zeros_like(q)
    for s, e in _bounds(N, cu):
        L = e - s
        if L == 0:
            continue
        if causal:
            n = np.arange(1, L + 1, dtype=np.float64)
            G = do[s:e] / n[:, None]  # dO_i / n_i
            R = (D[s:e] / n)[:, None] * q[s:e]  # D_i q_i / n_i
            M = np.zeros((d, d))  # sum over later blocks of q_i (dO_i / n_i)^T
            w = np.zeros(d)  # sum over later blocks of D_i q_i / n_i
            for b in range(L, 0, -block):
                a = max(0, b - block)
                Qb, Gb, Vb, Rb = q[s + a:s + b], G[a:b], v[s + a:s + b], R[a:b]
                W = np.tril(Gb @ Vb.T)  # W[i, j] = dO_i . v_j / n_i for block-local i >= j
                t1 = Vb @ M.T + W.T @ Qb  # sum_{i >= j} q_i (dO_i . v_j) / n_i
                t2 = w[None] + _revcumsum0(Rb)  # sum_{i >= j} D_i q_i / n_i
                dk[s + a:s + b] = scale * (t1 - t2)
                M += Qb.T @ Gb
                w += Rb.sum(axis=0)
        else:
            M = q[s:e].T @ do[s:e] / L
            w = (D[s:e, None] * q[s:e]).sum(axis=0) / L
            dk[s:e] = scale * (v[s:e] @ M.T - w[None])
    return dq, dk, dv


def uniform_inputs(N, d, seed, scale=1.0, dtype=torch.float64):
    """q, k, v, dO of one head with equal scores along each row: q_i = [a_i, 0],
    k_j = [c, u_j] (halves of d), everything else N(0, scale^2) from seed."""
    g = torch.Generator().manual_seed(seed)
    h = d // 2
    a = torch.randn(N, h, generator=g, dtype=torch.float64) * scale
    c = torch.randn(h, generator=g, dtype=torch.float64) * scale
    u = torch.randn(N, d - h, generator=g, dtype=torch.float64) * scale
    v = torch.randn(N, d, generator=g, dtype=torch.float64) * scale
    do = torch.randn(N, d, generator=g, dtype=torch.float64) * scale
    q = torch.cat([a, torch.zeros(N, d - h, dtype=torch.float64)], dim=1)
    k = torch.cat([c.expand(N, h), u], dim=1)
    return tuple(x.to(dtype) for x in (q, k, v, do))
