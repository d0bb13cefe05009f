"""Oracle for one rank's Ulysses attention, forward and backward (test infrastructure only).

What is computed (float64 throughout):

  * HF Transformers docs, "Ulysses sequence parallelism" (deepspeed_alst),
    opening paragraph: after the first all-to-all each rank holds the whole
    sequence for a subset of heads and computes attention locally over it.
    The congresoia365 article, section "Cómo Funciona Ulysses", step "Atención
    Local", says this is the standard attention mechanism, and heads are
    independent of one another. So each (rank, batch row, head) is plain
    softmax attention over all N tokens:
        S = Q K^T / sqrt(d),  P = softmax_rows(S + mask),  O = P V.
  * Same guide, "sp_attn_implementation" paragraph (and the jianying88 page's
    notes on it): samples packed into one row must not attend across their
    boundaries. allowed(i, j) <=> doc(i) == doc(j) and (not causal or j <= i),
    with documents given by cu_seqlens (int32, [ndoc+1], cu[0] = 0,
    non-decreasing, cu[ndoc] = N; the same packing for every row).
  * congresoia365 article, section "El Desafío del Entrenamiento de
    Secuencias Largas": memory-efficient attention never stores the N x N
    matrix. The saved state of the forward is therefore the per-row
    log-sum-exp, lse_i = log sum_j exp(S_ij) over allowed j (natural log).
  * The backward is the analytic gradient of O with respect to Q, K, V, in
    the plain Jacobian form of the softmax (not the rowsum(dO*O) shortcut):
        dV = P^T dO,  dP = dO V^T,
        dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik),
        dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d).

Computation notes (none changes the definition):
  * Each row is normalised as a whole: max over the whole allowed row, then
    the log of the sum of exponentials, then P = exp(S - lse).
  * Keys outside the query's document carry weight exactly zero, so each
    query row is evaluated over its own document's keys only.
  * Rows are processed in chunks to bound memory; a chunk holds whole rows.

Layouts: q, k, v, dO are [..., N, H, d] (any leading dims, e.g. [sp, B]);
o, dq, dk, dv have the same shape; lse is [..., H, N].
"""

from __future__ import annotations

import math

import numpy as np

_CHUNK_ELEMS = 1 << 23  # float64 elements of one row chunk of S (64 MiB)


def as_f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor (fp32/bf16) or numpy array to float64."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def doc_bounds(N: int, cu_seqlens=None) -> list[tuple[int, int]]:
    """Documents as (start, end) token ranges; None means one document [0, N)."""
    if cu_seqlens is None:
        return [(0, N)]
    cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    if len(cu) < 2 or cu[0] != 0 or cu[-1] != N or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at N")
    return list(zip(cu[:-1], cu[1:]))


def doc_ids(N: int, cu_seqlens=None) -> np.ndarray:
    """Document index of every token position."""
    ids = np.zeros(N, dtype=np.int64)
    for i, (s, e) in enumerate(doc_bounds(N, cu_seqlens)):
        ids[s:e] = i
    return ids


def _doc_of(pos: int, bounds) -> tuple[int, int]:
    for s, e in bounds:
        if s <= pos < e:
            return s, e
    raise IndexError(pos)


def _scores(Qr, qpos, Kd, kpos, causal, scale):
    """Scaled scores of query rows Qr (positions qpos) against one document's keys."""
    S = scale * (Qr @ Kd.T)
    if causal:
        S = np.where(kpos[None, :] <= qpos[:, None], S, -np.inf)
    return S


def _softmax_rows(S):
    """Whole-row softmax of masked scores; returns P and the natural-log lse."""
    m = S.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(S - m).sum(axis=1))
    P = np.exp(S - lse[:, None])
    return P, lse


def _chunks(s: int, e: int, L: int):
    step = max(1, _CHUNK_ELEMS // max(L, 1))
    for r0 in range(s, e, step):
        yield r0, min(e, r0 + step)


def _flatten(x):
    """[..., N, H, d] -> [lead, N, H, d] float64."""
    x = as_f64(x)
    return x.reshape((-1,) + x.shape[-3:])


def attn_fwd(q, k, v, cu_seqlens=None, causal: bool = True):
    """Forward: returns (o [..., N, H, d], lse [..., H, N]) in float64."""
    lead_shape = tuple(q.shape)[:-3]
    Q, K, V = _flatten(q), _flatten(k), _flatten(v)
    G, N, H, d = Q.shape
    scale = 1.0 / math.sqrt(d)
    O = np.zeros_like(Q)
    LSE = np.zeros((G, H, N))
    pos = np.arange(N)
    for g in range(G):
        for h in range(H):
            for s, e in doc_bounds(N, cu_seqlens):
                if e == s:
                    continue
                Kd, Vd = K[g, s:e, h], V[g, s:e, h]
                for r0, r1 in _chunks(s, e, e - s):
                    S = _scores(Q[g, r0:r1, h], pos[r0:r1], Kd, pos[s:e], causal, scale)
                    P, lse = _softmax_rows(S)
                    O[g, r0:r1, h] = P @ Vd
                    LSE[g, h, r0:r1] = lse
    return O.reshape(lead_shape + (N, H, d)), LSE.reshape(lead_shape + (H, N))


def attn_bwd(q, k, v, do, cu_seqlens=None, causal: bool = True):
    """Backward: returns (dq, dk, dv), each [..., N, H, d] float64."""
    lead_shape = tuple(q.shape)[:-3]
    Q, K, V, DO = _flatten(q), _flatten(k), _flatten(v), _flatten(do)
    G, N, H, d = Q.shape
    scale = 1.0 / math.sqrt(d)
    dQ, dK, dV = np.zeros_like(Q), np.zeros_like(Q), np.zeros_like(Q)
    pos = np.arange(N)
    for g in range(G):
        for h in range(H):
            for s, e in doc_bounds(N, cu_seqlens):
                if e == s:
                    continue
                Kd, Vd = K[g, s:e, h], V[g, s:e, h]
                for r0, r1 in _chunks(s, e, e - s):
                    Qr, DOr = Q[g, r0:r1, h], DO[g, r0:r1, h]
                    P, _ = _softmax_rows(_scores(Qr, pos[r0:r1], Kd, pos[s:e], causal, scale))
                    dP = DOr @ Vd.T
                    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
                    dQ[g, r0:r1, h] = scale * (dS @ Kd)
                    dK[g, s:e, h] += scale * (dS.T @ Qr)
                    dV[g, s:e, h] += P.T @ DOr
    shape = lead_shape + (N, H, d)
    return dQ.reshape(shape), dK.reshape(shape), dV.reshape(shape)


# ---- sampled outputs of one head, for sizes where the full oracle is too slow ----
# q1, k1, v1, do1 are one head's [N, d] slices.


def attn_fwd_rows(q1, k1, v1, rows, cu_seqlens=None, causal: bool = True):
    """O and lse of the given query rows only: ([len(rows), d], [len(rows)])."""
    Q, K, V = as_f64(q1), as_f64(k1), as_f64(v1)
    N, d = Q.shape
    scale = 1.0 / math.sqrt(d)
    bounds = doc_bounds(N, cu_seqlens)
    pos = np.arange(N)
    O = np.zeros((len(rows), d))
    LSE = np.zeros(len(rows))
    for n, i in enumerate(rows):
        s, e = _doc_of(int(i), bounds)
        S = _scores(Q[i:i + 1], pos[i:i + 1], K[s:e], pos[s:e], causal, scale)
        P, lse = _softmax_rows(S)
        O[n] = (P @ V[s:e])[0]
        LSE[n] = lse[0]
    return O, LSE


def attn_bwd_dq_rows(q1, k1, v1, do1, rows, cu_seqlens=None, causal: bool = True):
    """dQ of the given query rows only: [len(rows), d]."""
    Q, K, V, DO = as_f64(q1), as_f64(k1), as_f64(v1), as_f64(do1)
    N, d = Q.shape
    scale = 1.0 / math.sqrt(d)
    bounds = doc_bounds(N, cu_seqlens)
    pos = np.arange(N)
    dQ = np.zeros((len(rows), d))
    for n, i in enumerate(rows):
        s, e = _doc_of(int(i), bounds)
        P, _ = _softmax_rows(_scores(Q[i:i + 1], pos[i:i + 1], K[s:e], pos[s:e], causal, scale))
        dP = DO[i:i + 1] @ V[s:e].T
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        dQ[n] = scale * (dS @ K[s:e])[0]
    return dQ


def attn_bwd_dkdv_cols(q1, k1, v1, do1, cols, cu_seqlens=None, causal: bool = True):
    """dK and dV of the given key positions only: ([len(cols), d], [len(cols), d]).

    A key's gradient needs every query row that sees it, each normalised over
    its whole row, so the cost grows with the number of such rows: sample keys
    late in their document (causal) to keep it small.
    """
    Q, K, V, DO = as_f64(q1), as_f64(k1), as_f64(v1), as_f64(do1)
    N, d = Q.shape
    scale = 1.0 / math.sqrt(d)
    bounds = doc_bounds(N, cu_seqlens)
    pos = np.arange(N)
    cols = np.asarray(cols, dtype=np.int64)
    dK = np.zeros((len(cols), d))
    dV = np.zeros((len(cols), d))
    for s, e in bounds:
        sel = np.nonzero((cols >= s) & (cols < e))[0]
        if len(sel) == 0:
            continue
        first_row = int(cols[sel].min()) if causal else s
        kidx = cols[sel] - s
        for r0, r1 in _chunks(first_row, e, e - s):
            Qr, DOr = Q[r0:r1], DO[r0:r1]
            P, _ = _softmax_rows(_scores(Qr, pos[r0:r1], K[s:e], pos[s:e], causal, scale))
            dP = DOr @ V[s:e].T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dK[sel] += scale * (dS[:, kidx].T @ Qr)
            dV[sel] += P[:, kidx].T @ DOr
    return dK, dV
